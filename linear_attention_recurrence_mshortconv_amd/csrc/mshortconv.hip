// Modality-aware short convolution (mShortConv) on gfx950.
//
// Chimera page 1, section 3.3 Eq. 13 (the conv is applied to q, k and v) and
// section 3.4 (text: causal 1D depthwise along the text segment; visual: depthwise
// 3D over (time, height, width), causal in time and symmetric in space, an image
// being a one-frame video; each segment convolved on its own with zero padding;
// results written back to their packed positions). Eq. 12 gives the raster
// order of a grid inside the stream.
//
// Three kernels:
//  * conv_text_kernel: text segments; a thread slides a 4-token window over 16
//    tokens of 8 channels.
//  * conv_gather_kernel: one thread = 8 channels of one token; every tap is a
//    direct 16-byte (bf16) or 32-byte (fp32) load from the packed stream. Used
//    for grids of fp32 data (and as the plain reference arrangement).
//  * conv_tile_kernel (bf16 grids): a block owns a spatial tile (TR rows x TW
//    columns) x a 64-channel slab, stages each frame's tile plus its one-token
//    halo in LDS, and streams over frames with a 3-frame LDS ring for the
//    causal time taps. A thread keeps its channels' weights in registers and
//    slides a 3-row window down its column, so each staged value is read from
//    LDS once per (kw) and feeds up to three output rows.
#include <algorithm>
#include <atomic>
#include <vector>

#include "dtypes.h"
#include "internal.h"

namespace chm {
namespace {

// ---- generic gather kernel ---------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void conv_gather_kernel(const T* __restrict__ x, T* __restrict__ y,
                                                         const float* __restrict__ w_text,
                                                         const float* __restrict__ w_vis, int64_t Ttot,
                                                         int64_t C, Seg seg) {
  const int64_t C8 = C / 8;
  const int64_t cg = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
  const int64_t local = (int64_t)blockIdx.y * 4 + (threadIdx.x >> 6);
  const int64_t b = blockIdx.z;
  if (cg >= C8 || local >= seg.length) return;
  const int64_t p = seg.start + local;
  const int64_t c0 = cg * 8;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  const T* xb = x + b * Ttot * C;
  if (seg.kind == SEG_TEXT) {
    for (int j = 0; j < kTextTaps; ++j) {
      const int64_t src = text_tap_source(seg, p, j);
      if (src < 0) continue;
      float v[8];
      load8(xb + src * C + c0, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(w_text[(c0 + i) * kTextTaps + j], v[i], acc[i]);
    }
  } else {
    const int64_t hw = (int64_t)seg.height * seg.width;
    const int64_t f = local / hw, h = (local / seg.width) % seg.height, w = local % seg.width;  // Eq. 12
    for (int kt = 0; kt < 3; ++kt)
      for (int kh = 0; kh < 3; ++kh)
        for (int kw = 0; kw < 3; ++kw) {
          const int64_t src = vis_tap_source(seg, f, h, w, kt, kh, kw);
          if (src < 0) continue;
          const int tap = kt * 9 + kh * 3 + kw;
          float v[8];
          load8(xb + src * C + c0, v);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(w_vis[(c0 + i) * kVisTaps + tap], v[i], acc[i]);
        }
  }
  store8(y + b * Ttot * C + p * C + c0, acc);
}

// ---- tiled grid kernel (bf16) ----------------------------------------------------
// NF: 1 for a one-frame grid (only the kt = 2 taps can be non-zero), 3 for video.
// CPT: channels per thread (8 -> 16-byte accesses, 4 -> 8-byte accesses).
// A block = TW columns x (64 / CPT) channel groups = TW*64/CPT threads, each
// computing TR output rows of one column.
// Buffer accesses: offsets past a buffer's end read zero and drop stores. Every
// buffer the conv kernels build spans less than kOutside bytes (the launchers
// check), so kOutside marks a position outside the grid.
constexpr uint32_t kOutside = 0x80000000u;   // past every buffer: the launcher keeps them under 2 GiB
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, gfx9 data format

// Segments of one kind go to one launch, up to kMaxBatch at a time, with a table in the
// kernel arguments: each entry holds the segment, its block decomposition and its first
// block; a block finds its entry by binary search over the first blocks. (Packed rows
// of many samples have many short segments, each far too small to fill the chip alone.)
constexpr int kMaxBatch = 48;
struct RowsEntry {
  Seg seg;
  int32_t n_tw, n_rr, rows_per_range, blk0;
};
struct RowsBatch {
  int n, n_slab, n_logical, pad;
  RowsEntry e[kMaxBatch];
};
struct TextEntry {
  Seg seg;
  int32_t n_run4, blk0, pad0, pad1;   // run groups (4 runs of kTextRun tokens each), first block
};
struct TextBatch {
  int n, n_cg, n_logical, pad;        // n_cg: groups of 64 x 8 channels
  TextEntry e[kMaxBatch];
};
__device__ __forceinline__ int32_t uni(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }
// the last entry whose first block is at most lid
template <typename Batch>
__device__ __forceinline__ int entry_of(const Batch& t, int32_t lid) {
  int lo = 0, hi = t.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (lid >= t.e[mid].blk0) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

template <int NF, int CPT, int TR, int TW>
struct TileCfg {
  static constexpr int kGroups = 64 / CPT;            // channel groups per 64-channel slab
  static constexpr int kThreads = TW * kGroups;
  static constexpr int kSR = TR + 2, kSC = TW + 2;    // staged rows / columns (with halo)
  static constexpr int kSlots = kSR * kSC;            // tokens per staged frame tile
  static constexpr int kItems = kSlots * kGroups;     // CPT-channel items per staged frame tile
};

template <int CPT> struct Vec;
template <> struct Vec<8> { using T = uint4; };
template <> struct Vec<4> { using T = uint2; };

__device__ __forceinline__ void unpack(const uint4& u, float* v) {
  v[0] = bf_lo(u.x); v[1] = bf_hi(u.x); v[2] = bf_lo(u.y); v[3] = bf_hi(u.y);
  v[4] = bf_lo(u.z); v[5] = bf_hi(u.z); v[6] = bf_lo(u.w); v[7] = bf_hi(u.w);
}
__device__ __forceinline__ void unpack(const uint2& u, float* v) {
  v[0] = bf_lo(u.x); v[1] = bf_hi(u.x); v[2] = bf_lo(u.y); v[3] = bf_hi(u.y);
}
__device__ __forceinline__ void pack(uint4& u, const float* v) {
  u.x = pack_bf16x2(v[0], v[1]); u.y = pack_bf16x2(v[2], v[3]);
  u.z = pack_bf16x2(v[4], v[5]); u.w = pack_bf16x2(v[6], v[7]);
}
__device__ __forceinline__ void pack(uint2& u, const float* v) {
  u.x = pack_bf16x2(v[0], v[1]); u.y = pack_bf16x2(v[2], v[3]);
}

// FLIP: the adjoint (dx from dy): the 3x3 spatial taps mirrored and the frames walked from the
// last one back (logical frame f is frame frames - 1 - f of the segment, for reads and writes),
// which turns the causal time taps into the anti-causal ones the adjoint needs.
template <int NF, int CPT, int TR, int TW, bool FLIP = false>
__global__ __launch_bounds__(TW * (64 / CPT)) void conv_tile_kernel(
    const uint16_t* __restrict__ x, uint16_t* __restrict__ y, const float* __restrict__ w_vis, int64_t Ttot,
    int64_t C, Seg seg, int n_slab, int n_tw, int n_th, int n_fr, int frames_per_block, int n_logical) {
  using Cfg = TileCfg<NF, CPT, TR, TW>;
  using V = typename Vec<CPT>::T;
  constexpr int NIT = (Cfg::kItems + Cfg::kThreads - 1) / Cfg::kThreads;
  // staged frames [slot][token][group], plus one spare item per thread for the items
  // past kItems of the last load round (every staging write is unconditional)
  __shared__ V tile[NF * Cfg::kSlots * Cfg::kGroups + Cfg::kThreads];

  const int lid = (int)xcd_contiguous_id(blockIdx.x, gridDim.x);
  if (lid >= n_logical) return;
  int r = lid;
  const int tw = r % n_tw; r /= n_tw;
  const int th = r % n_th; r /= n_th;
  const int slab = r % n_slab; r /= n_slab;
  const int fr = r % n_fr; r /= n_fr;
  const int64_t b = r;

  const int tid = threadIdx.x;
  const int g = tid % Cfg::kGroups;              // channel group inside the slab
  const int col = tid / Cfg::kGroups;            // tile column 0..TW-1
  const int h0 = th * TR, w0 = tw * TW;
  const int frame_bytes = seg.height * seg.width * (int)C * 2;
  const uint16_t* xb = x + (b * Ttot + seg.start) * C;
  uint16_t* yb = y + (b * Ttot + seg.start) * C;

  // weights of this thread's channels: wr[kt'][kh][kw][ch], kt' over the used time taps
  float wr[NF][3][3][CPT];
#pragma unroll
  for (int t = 0; t < NF; ++t)
#pragma unroll
    for (int kh = 0; kh < 3; ++kh)
#pragma unroll
      for (int kw = 0; kw < 3; ++kw)
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
          const int kt = 3 - NF + t;
          const int th_ = FLIP ? 2 - kh : kh, tw_ = FLIP ? 2 - kw : kw;
          wr[t][kh][kw][i] = w_vis[((int64_t)slab * 64 + g * CPT + i) * kVisTaps + kt * 9 + th_ * 3 + tw_];
        }

  const int f_begin = fr * frames_per_block;
  const int f_end = min(seg.frames, f_begin + frames_per_block);

  // byte offset inside a frame of (row hh, column ww, channel group gg), or kOutside
  auto offset = [&](int hh, int ww, int gg) -> uint32_t {
    const bool in = (hh >= 0) & (hh < seg.height) & (ww >= 0) & (ww < seg.width);
    return in ? (uint32_t)(((hh * seg.width + ww) * (int)C + slab * 64 + gg * CPT) * 2) : kOutside;
  };
  // Staging of one frame's tile plus halo: every thread first loads its items
  // into registers (all loads in flight together), then stores them to LDS.
  V pre[NIT];
  auto phys = [&](int ff) { return FLIP ? seg.frames - 1 - ff : ff; };   // the segment frame of logical frame ff
  auto fetch = [&](int ff) {
    const auto xr = __builtin_amdgcn_make_buffer_rsrc((void*)(xb + (int64_t)phys(ff) * seg.height * seg.width * C),
                                                      0, frame_bytes, kRsrcWord3);
#pragma unroll
    for (int j = 0; j < NIT; ++j) {
      const int it = tid + j * Cfg::kThreads;
      const int s = it / Cfg::kGroups, gg = it % Cfg::kGroups;
      const uint32_t off = it < Cfg::kItems ? offset(h0 + s / Cfg::kSC - 1, w0 + s % Cfg::kSC - 1, gg) : kOutside;
      if constexpr (CPT == 8) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)off, 0, 0);
        pre[j] = V{v[0], v[1], v[2], v[3]};
      } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(xr, (int)off, 0, 0);
        pre[j] = V{v[0], v[1]};
      }
    }
  };
  auto commit = [&](int slot) {
#pragma unroll
    for (int j = 0; j < NIT; ++j) {
      const int it = tid + j * Cfg::kThreads;
      tile[it < Cfg::kItems ? slot * Cfg::kSlots * Cfg::kGroups + it : NF * Cfg::kSlots * Cfg::kGroups + tid] = pre[j];
    }
  };

  // One step: stage frame f (loaded during the previous step), start loading the
  // next frame, compute the output tile of frame f.
  auto step = [&](int f) {
    lds_barrier();                                    // previous frame's reads are done
    commit(NF == 3 ? f % 3 : 0);
    lds_barrier();
    if (f + 1 < f_end) fetch(f + 1);                  // next frame's loads overlap this frame's math
    float acc[TR][CPT];
#pragma unroll
    for (int rr = 0; rr < TR; ++rr)
#pragma unroll
      for (int i = 0; i < CPT; ++i) acc[rr][i] = 0.f;
#pragma unroll
    for (int t = 0; t < NF; ++t) {
      const int kt = 3 - NF + t;
      const int fsrc = f + kt - 2;
      if (fsrc < 0) continue;                        // frames before the first read zero
      const int slot = NF == 3 ? fsrc % 3 : 0;
#pragma unroll
      for (int ir = 0; ir < TR + 2; ++ir) {          // staged row ir feeds output rows ir-2..ir
#pragma unroll
        for (int kw = 0; kw < 3; ++kw) {
          float v[CPT];
          unpack(tile[(slot * Cfg::kSlots + ir * Cfg::kSC + col + kw) * Cfg::kGroups + g], v);
#pragma unroll
          for (int kh = 0; kh < 3; ++kh) {
            const int orow = ir - kh;
            if (orow < 0 || orow >= TR) continue;
#pragma unroll
            for (int i = 0; i < CPT; ++i) acc[orow][i] = fmaf(wr[t][kh][kw][i], v[i], acc[orow][i]);
          }
        }
      }
    }
    const auto yr = __builtin_amdgcn_make_buffer_rsrc((void*)(yb + (int64_t)phys(f) * seg.height * seg.width * C),
                                                      0, frame_bytes, kRsrcWord3);
#pragma unroll
    for (int rr = 0; rr < TR; ++rr) {
      V out;
      pack(out, acc[rr]);
      const uint32_t off = offset(h0 + rr, w0 + col, g);
      if constexpr (CPT == 8) {
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(__attribute__((ext_vector_type(4))) uint32_t, out), yr, (int)off, 0, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b64(
            __builtin_bit_cast(__attribute__((ext_vector_type(2))) uint32_t, out), yr, (int)off, 0, 0);
      }
    }
  };

  if (NF == 3) {
    for (int ff = max(0, f_begin - 2); ff < f_begin; ++ff) {
      fetch(ff);
      commit(ff % 3);
    }
  }
  if (f_begin < f_end) {
    fetch(f_begin);
    // the first step runs outside the loop, so that every step in it starts with the
    // same outstanding accesses (staged loads, then stores) and waits for loads only
    step(f_begin);
    for (int f = f_begin + 1; f < f_end; ++f) step(f);
  }
}

// One-frame grids (images): a block owns a column strip of TW columns (plus a
// one-column halo on each side) and a 64-channel slab, and streams down a range
// of rows TR at a time. Staged rows live in an LDS ring of TR + 2 rows, so the
// two halo rows of each step are the last rows of the previous step (every input
// row is read from HBM once per strip); the next TR rows are loaded into
// registers while the current TR output rows are computed.
// Loads and stores are buffer accesses relative to the block's first row, with
// 32-bit offsets: taps outside the grid get an offset past the buffer's end and
// read zero, output positions outside it are dropped the same way, so there is
// no branch around a memory access and every wait counts only what it needs.
// FLIP: the 3x3 taps mirrored in both directions, which makes the kernel the adjoint of
// the image conv (dx from dy for the backward).
template <int TR, int TW, bool FLIP>
__global__ __launch_bounds__(TW * 8) void conv_rows_kernel(const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
                                                         const float* __restrict__ w_vis, int64_t Ttot, int64_t C,
                                                         RowsBatch tb) {
  constexpr int NT = TW * 8, SC = TW + 2, RING = TR + 2;
  constexpr int ITEMS = TR * SC * 8;                 // 16-byte items per TR staged rows
  constexpr int NIT = (ITEMS + NT - 1) / NT;
  // ring[slot][column][group] flat, plus one slot per thread for the items past
  // ITEMS of the last load round (so that every staging write is unconditional)
  __shared__ uint4 ring[RING * SC * 8 + NT];

  const int lid = (int)xcd_contiguous_id(blockIdx.x, gridDim.x);
  if (lid >= tb.n_logical) return;
  const RowsEntry& ent = tb.e[entry_of(tb, lid)];
  const Seg seg = ent.seg;
  const int n_tw = ent.n_tw, n_slab = tb.n_slab, n_rr = ent.n_rr, rows_per_range = ent.rows_per_range;
  int r = lid - ent.blk0;
  const int tw = uni(r % n_tw); r = uni(r / n_tw);
  const int slab = uni(r % n_slab); r = uni(r / n_slab);
  const int rr_ix = uni(r % n_rr); r = uni(r / n_rr);
  const int64_t b = r;

  const int tid = threadIdx.x, g = tid & 7, col = tid >> 3;
  const int w0 = tw * TW;
  const int r_begin = rr_ix * rows_per_range;
  const int r_end = min(seg.height, r_begin + rows_per_range);
  // buffers span grid rows base_row .. last_row - 1 of this batch item's segment
  const int base_row = max(r_begin - 1, 0), last_row = min(seg.height, r_end + 1);
  const int row_bytes = seg.width * (int)C * 2;
  const int64_t base_tok = b * Ttot + seg.start + (int64_t)base_row * seg.width;
  const auto xr = __builtin_amdgcn_make_buffer_rsrc((void*)(x + base_tok * C), 0, (last_row - base_row) * row_bytes,
                                                    kRsrcWord3);
  const auto yr = __builtin_amdgcn_make_buffer_rsrc((void*)(y + base_tok * C), 0, (last_row - base_row) * row_bytes,
                                                    kRsrcWord3);

  float wr[3][3][8];
#pragma unroll
  for (int kh = 0; kh < 3; ++kh)
#pragma unroll
    for (int kw = 0; kw < 3; ++kw)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        wr[kh][kw][i] = w_vis[((int64_t)slab * 64 + g * 8 + i) * kVisTaps + 18 + (FLIP ? 8 - kh * 3 - kw : kh * 3 + kw)];

  // byte offset of (grid row hh, grid column ww, channel group gg), or kOutside
  auto offset = [&](int hh, int ww, int gg) -> uint32_t {
    const bool in = (hh >= 0) & (hh < seg.height) & (ww >= 0) & (ww < seg.width);
    return in ? (uint32_t)((hh - base_row) * row_bytes + ww * (int)C * 2 + slab * 128 + gg * 16) : kOutside;
  };
  // ring slot of grid row hh (hh >= r_begin - 1)
  auto slot_of = [&](int hh) { return (hh - r_begin + 1) % RING; };
  uint4 pre[NIT];
  // load grid rows first_row .. first_row + nrows - 1 (nrows <= TR) into registers
  auto fetch = [&](int first_row, int nrows) {
#pragma unroll
    for (int j = 0; j < NIT; ++j) {
      const int it = tid + j * NT;
      const int rowi = it / (SC * 8), rem = it % (SC * 8);
      const int sc = rem >> 3, gg = rem & 7;
      const uint32_t off = ((it < ITEMS) & (rowi < nrows)) ? offset(first_row + rowi, w0 + sc - 1, gg) : kOutside;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)off, 0, 0);
      pre[j] = uint4{v[0], v[1], v[2], v[3]};
    }
  };
  // stage what fetch loaded; items of rows at or past nrows land in the spare slots
  auto commit = [&](int first_row, int nrows) {
#pragma unroll
    for (int j = 0; j < NIT; ++j) {
      const int it = tid + j * NT;
      const int rowi = it / (SC * 8), rem = it % (SC * 8);
      const bool real = (it < ITEMS) & (rowi < nrows);
      ring[real ? slot_of(first_row + rowi) * (SC * 8) + rem : RING * SC * 8 + tid] = pre[j];
    }
  };

  // One step: stage rows h0 + 1 .. h0 + TR (loaded during the previous step), start
  // loading the next step's rows, and compute output rows h0 .. h0 + TR - 1.
  auto step = [&](int h0) {
    lds_barrier();                                   // the previous step's reads of the ring are done
    commit(h0 + 1, TR);                              // rows h0+1 .. h0+TR
    lds_barrier();
    if (h0 + TR < r_end) fetch(h0 + TR + 1, TR);     // next step's new rows, in flight during the math
    float acc[TR][8];
#pragma unroll
    for (int q = 0; q < TR; ++q)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[q][i] = 0.f;
#pragma unroll
    for (int ir = 0; ir < TR + 2; ++ir) {            // staged row h0 - 1 + ir feeds output rows ir-2..ir
      __builtin_amdgcn_sched_barrier(0);              // keep one staged row's values live at a time
      const int sl = slot_of(h0 - 1 + ir);
#pragma unroll
      for (int kw = 0; kw < 3; ++kw) {
        float v[8];
        unpack(ring[(sl * SC + col + kw) * 8 + g], v);
#pragma unroll
        for (int kh = 0; kh < 3; ++kh) {
          const int orow = ir - kh;
          if (orow < 0 || orow >= TR) continue;
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[orow][i] = fmaf(wr[kh][kw][i], v[i], acc[orow][i]);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < TR; ++q) {
      uint4 out;
      pack(out, acc[q]);
      const uint32_t off = h0 + q < r_end ? offset(h0 + q, w0 + col, g) : kOutside;
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(__attribute__((ext_vector_type(4))) uint32_t, out), yr, (int)off, 0, 0);
    }
  };

  // the first step needs rows r_begin - 1 .. r_begin + TR; rows outside the grid stage as zero
  fetch(r_begin - 1, 2);
  commit(r_begin - 1, 2);
  fetch(r_begin + 1, TR);
  // The first step runs outside the loop: every step then starts with the same
  // outstanding accesses (the staged loads, then the previous stores), so the waits
  // before staging count the loads only and the stores stay in flight.
  step(r_begin);
  for (int h0 = r_begin + TR; h0 < r_end; h0 += TR) step(h0);
}

// Text segments (causal, 4 taps): a thread owns 8 channels and kTextRun
// consecutive tokens and keeps its weights and a 4-token window in registers.
// Short runs give enough blocks for a few hundred text tokens; the three window
// tokens before a run are re-read (from L2) by the run that also owns them.
constexpr int kTextRun = 4;
template <typename T>
__global__ __launch_bounds__(256) void conv_text_kernel(const T* __restrict__ x, T* __restrict__ y,
                                                       const float* __restrict__ w_text, int64_t Ttot, int64_t C,
                                                       TextBatch tb) {
  const int lid = blockIdx.x;
  if (lid >= tb.n_logical) return;
  const TextEntry& ent = tb.e[entry_of(tb, lid)];
  const Seg seg = ent.seg;
  int r = lid - ent.blk0;                     // (batch item, run group, channel group)
  const int bx = uni(r % tb.n_cg); r = uni(r / tb.n_cg);
  const int by = uni(r % ent.n_run4);
  const int64_t b = uni(r / ent.n_run4);
  const int64_t C8 = C / 8;
  const int64_t cg = (int64_t)bx * 64 + (threadIdx.x & 63);
  const int64_t run = (int64_t)by * 4 + (threadIdx.x >> 6);
  const int64_t l0 = run * kTextRun;
  if (cg >= C8 || l0 >= seg.length) return;
  const int64_t c0 = cg * 8;
  float w[8][kTextTaps];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 wv = *reinterpret_cast<const float4*>(w_text + (c0 + i) * kTextTaps);
    w[i][0] = wv.x; w[i][1] = wv.y; w[i][2] = wv.z; w[i][3] = wv.w;
  }
  const T* xb = x + b * Ttot * C;
  T* yb = y + b * Ttot * C;
  float win[kTextTaps][8];                         // win[j] = token p - 3 + j
#pragma unroll
  for (int j = 0; j < kTextTaps - 1; ++j) {
    const int64_t src = text_tap_source(seg, seg.start + l0, j);
    if (src >= 0) load8(xb + src * C + c0, win[j + 1]);
    else
#pragma unroll
      for (int i = 0; i < 8; ++i) win[j + 1][i] = 0.f;
  }
  for (int u = 0; u < kTextRun; ++u) {
    const int64_t local = l0 + u;
    if (local >= seg.length) break;
#pragma unroll
    for (int j = 0; j < kTextTaps - 1; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) win[j][i] = win[j + 1][i];
    load8(xb + (seg.start + local) * C + c0, win[kTextTaps - 1]);
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc[i] = 0.f;
#pragma unroll
      for (int j = 0; j < kTextTaps; ++j) acc[i] = fmaf(w[i][j], win[j][i], acc[i]);
    }
    store8(yb + (seg.start + local) * C + c0, acc);
  }
}

__global__ void index_device_kernel(Seg seg, int32_t* __restrict__ idx) {
  const int64_t local = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (local >= seg.length) return;
  const int64_t p = seg.start + local;
  int32_t* row = idx + p * kVisTaps;
  if (seg.kind == SEG_TEXT) {
    for (int j = 0; j < kVisTaps; ++j) row[j] = j < kTextTaps ? (int32_t)text_tap_source(seg, p, j) : -1;
    return;
  }
  // the tile kernel's path: grid point of the output, then the staged neighbour
  const int64_t hw = (int64_t)seg.height * seg.width;
  const int64_t f = local / hw, h = (local / seg.width) % seg.height, w = local % seg.width;
  for (int kt = 0; kt < 3; ++kt)
    for (int kh = 0; kh < 3; ++kh)
      for (int kw = 0; kw < 3; ++kw) {
        const int64_t ff = f + kt - 2, hh = h + kh - 1, ww = w + kw - 1;
        row[kt * 9 + kh * 3 + kw] = grid_inside(seg, ff, hh, ww) ? (int32_t)raster_index(seg, ff, hh, ww) : -1;
      }
}

// Compute units of the current device (256 on MI355X). The query is cached per device in an
// atomic: concurrent first calls from several host threads store the same value.
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  int c = dev < 64 ? cus[dev].load(std::memory_order_relaxed) : 0;
  if (c == 0) {
    int n = 0;
    c = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) ? n : 256;
    if (dev < 64) cus[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

template <int NF, int CPT, int TR, int TW>
hipError_t launch_tile(const uint16_t* x, uint16_t* y, const float* w_vis, int64_t B, int64_t Ttot, int64_t C,
                       const Seg& seg, hipStream_t stream, Marks* marks, bool flip = false) {
  using Cfg = TileCfg<NF, CPT, TR, TW>;
  const int n_slab = (int)(C / 64);
  const int n_tw = (int)((seg.width + TW - 1) / TW);
  const int n_th = (int)((seg.height + TR - 1) / TR);
  // video: split the frames so that there are enough blocks to fill the chip
  int fpb = seg.frames;
  if (NF == 3) {
    const int64_t per_frame_range = (int64_t)n_slab * n_tw * n_th * B;
    const int64_t want = 12 * (int64_t)device_cus();   // about six rounds of resident blocks
    int64_t nfr = (want + per_frame_range - 1) / per_frame_range;
    if (nfr > seg.frames) nfr = seg.frames;
    if (nfr < 1) nfr = 1;
    fpb = (int)((seg.frames + nfr - 1) / nfr);
    if (fpb < 8) fpb = 8 < seg.frames ? 8 : seg.frames;
  }
  const int n_fr = (seg.frames + fpb - 1) / fpb;
  const int64_t n_logical = (int64_t)n_slab * n_tw * n_th * n_fr * B;
  if (n_logical <= 0) return hipSuccess;
  if (n_logical > (int64_t(1) << 30)) return hipErrorInvalidValue;
  const int64_t grid = (n_logical + 7) / 8 * 8;
  if (flip)
    hipLaunchKernelGGL((conv_tile_kernel<NF, CPT, TR, TW, true>), dim3((unsigned)grid), dim3(Cfg::kThreads), 0, stream,
                       x, y, w_vis, Ttot, C, seg, n_slab, n_tw, n_th, n_fr, fpb, (int)n_logical);
  else
    hipLaunchKernelGGL((conv_tile_kernel<NF, CPT, TR, TW>), dim3((unsigned)grid), dim3(Cfg::kThreads), 0, stream, x, y,
                       w_vis, Ttot, C, seg, n_slab, n_tw, n_th, n_fr, fpb, (int)n_logical);
  const hipError_t e = hipGetLastError();
  return e != hipSuccess ? e : mark_after(marks, flip ? "conv_tile_adjoint_kernel" : "conv_tile_kernel", stream);
}

// Byte span of one rows-kernel buffer: (rows_per_range + 2) grid rows; kept
// below kOutside so that the out-of-grid offset always reads zero.
constexpr int64_t kRowsSpanMax = (int64_t)kOutside - 64;

template <int TR, int TW>
bool rows_fit(const Seg& seg, int64_t C) {
  return (int64_t)(TR + 2) * seg.width * C * 2 <= kRowsSpanMax;
}

// The row split of one image segment: rows in ranges (each re-reads 2 halo rows) so that
// the segment alone would be about six rounds of the blocks that fit on the chip at once
// (two per CU): blocks are long-lived, and a grid of a few whole rounds keeps the last
// round full. Returns false when no range fits a buffer.
template <int TR, int TW>
bool rows_entry(const Seg& seg, int64_t B, int64_t C, RowsEntry& ent, int64_t& blocks) {
  const int n_slab = (int)(C / 64);
  ent.seg = seg;
  ent.n_tw = (int)((seg.width + TW - 1) / TW);
  const int64_t per_range = (int64_t)n_slab * ent.n_tw * B;
  const int64_t want = 12 * (int64_t)device_cus();
  int n_rr = (int)std::max<int64_t>(1, std::min<int64_t>((want + per_range - 1) / per_range, (seg.height + 4 * TR - 1) / (4 * TR)));
  int rows_per_range = (seg.height + n_rr - 1) / n_rr;
  rows_per_range = (rows_per_range + TR - 1) / TR * TR;
  // the buffers of one block span rows_per_range + 2 rows
  const int64_t row_bytes = (int64_t)seg.width * C * 2;
  const int64_t max_rows = (kRowsSpanMax / row_bytes - 2) / TR * TR;
  if (max_rows < TR) return false;
  if (rows_per_range > max_rows) rows_per_range = (int)max_rows;
  ent.n_rr = (seg.height + rows_per_range - 1) / rows_per_range;
  ent.rows_per_range = rows_per_range;
  blocks = per_range * ent.n_rr;
  return true;
}

template <int TR, int TW, bool FLIP = false>
hipError_t launch_rows_batch(const uint16_t* x, uint16_t* y, const float* w_vis, int64_t B, int64_t Ttot, int64_t C,
                             const Seg* segs, int n, hipStream_t stream, Marks* marks) {
  for (int i0 = 0; i0 < n; i0 += kMaxBatch) {
    RowsBatch tb;
    tb.n = std::min(kMaxBatch, n - i0);
    tb.n_slab = (int)(C / 64);
    tb.pad = 0;
    int64_t total = 0;
    for (int i = 0; i < tb.n; ++i) {
      int64_t blocks = 0;
      if (!rows_entry<TR, TW>(segs[i0 + i], B, C, tb.e[i], blocks)) return hipErrorInvalidValue;
      tb.e[i].blk0 = (int32_t)total;
      total += blocks;
      if (total > (int64_t(1) << 30)) return hipErrorInvalidValue;
    }
    if (total == 0) continue;
    tb.n_logical = (int)total;
    const int64_t grid = (total + 7) / 8 * 8;
    hipLaunchKernelGGL((conv_rows_kernel<TR, TW, FLIP>), dim3((unsigned)grid), dim3(TW * 8), 0, stream, x, y, w_vis,
                       Ttot, C, tb);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const hipError_t me = mark_after(marks, FLIP ? "conv_rows_adjoint_kernel" : "conv_rows_kernel", stream);
    if (me != hipSuccess) return me;
  }
  return hipSuccess;
}

template <typename T>
hipError_t launch_text_batch(const T* x, T* y, const float* w_text, int64_t B, int64_t Ttot, int64_t C,
                             const Seg* segs, int n, hipStream_t stream, Marks* marks) {
  for (int i0 = 0; i0 < n; i0 += kMaxBatch) {
    TextBatch tb;
    tb.n = std::min(kMaxBatch, n - i0);
    tb.n_cg = (int)((C / 8 + 63) / 64);
    tb.pad = 0;
    int64_t total = 0;
    for (int i = 0; i < tb.n; ++i) {
      const Seg& sg = segs[i0 + i];
      const int64_t runs = (sg.length + kTextRun - 1) / kTextRun;
      TextEntry& e = tb.e[i];
      e.seg = sg;
      e.n_run4 = (int32_t)((runs + 3) / 4);
      e.blk0 = (int32_t)total;
      e.pad0 = e.pad1 = 0;
      total += (int64_t)tb.n_cg * e.n_run4 * B;
      if (total > 0x7fffff00) return hipErrorInvalidValue;
    }
    if (total == 0) continue;
    tb.n_logical = (int)total;
    hipLaunchKernelGGL(conv_text_kernel<T>, dim3((unsigned)total), dim3(256), 0, stream, x, y, w_text, Ttot, C, tb);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const hipError_t me = mark_after(marks, "conv_text_kernel", stream);
    if (me != hipSuccess) return me;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_conv_segment(const void* x, void* y, int64_t B, int64_t Ttot, int64_t C, bool bf16,
                               const float* w_text, const float* w_vis, const Seg& seg, bool force_gather,
                               hipStream_t stream, Marks* marks) {
  if (seg.length == 0 || B == 0) return hipSuccess;
  const bool tiled = bf16 && seg.kind != SEG_TEXT && C % 64 == 0 && !force_gather;
  if (tiled) {
    const uint16_t* xs = static_cast<const uint16_t*>(x);
    uint16_t* ys = static_cast<uint16_t*>(y);
    if (seg.frames == 1 && rows_fit<4, 32>(seg, C))
      return launch_rows_batch<4, 32>(xs, ys, w_vis, B, Ttot, C, &seg, 1, stream, marks);
    if ((int64_t)seg.height * seg.width * C * 2 <= (int64_t)kOutside - 64)
      return launch_tile<3, 4, 4, 16>(xs, ys, w_vis, B, Ttot, C, seg, stream, marks);
  }
  if (B > 65535) return hipErrorInvalidValue;
  if (seg.kind == SEG_TEXT) {
    if (bf16)
      return launch_text_batch<uint16_t>(static_cast<const uint16_t*>(x), static_cast<uint16_t*>(y), w_text, B, Ttot,
                                         C, &seg, 1, stream, marks);
    return launch_text_batch<float>(static_cast<const float*>(x), static_cast<float*>(y), w_text, B, Ttot, C, &seg, 1,
                                    stream, marks);
  }
  const dim3 grid((unsigned)((C / 8 + 63) / 64), (unsigned)((seg.length + 3) / 4), (unsigned)B);
  if (grid.y > 0x7fffffffu) return hipErrorInvalidValue;
  if (bf16) {
    hipLaunchKernelGGL(conv_gather_kernel<uint16_t>, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(x),
                       static_cast<uint16_t*>(y), w_text, w_vis, Ttot, C, seg);
  } else {
    hipLaunchKernelGGL(conv_gather_kernel<float>, grid, dim3(256), 0, stream, static_cast<const float*>(x),
                       static_cast<float*>(y), w_text, w_vis, Ttot, C, seg);
  }
  const hipError_t e = hipGetLastError();
  return e != hipSuccess ? e : mark_after(marks, "conv_gather_kernel", stream);
}

hipError_t launch_conv(const void* x, void* y, int64_t B, int64_t Ttot, int64_t C, bool bf16, const float* w_text,
                       const float* w_vis, const Seg* segs, int nseg, hipStream_t stream, Marks* marks) {
  if (B == 0) return hipSuccess;
  // text segments: one batched launch; image grids that the rows kernel takes: another;
  // every other segment (video, fp32 or oversized grids) on its own
  std::vector<Seg> text, rows, rest;
  const bool tiled_ok = bf16 && C % 64 == 0;
  for (int i = 0; i < nseg; ++i) {
    const Seg& sg = segs[i];
    if (sg.length == 0) continue;
    if (sg.kind == SEG_TEXT) text.push_back(sg);
    else if (tiled_ok && sg.frames == 1 && rows_fit<4, 32>(sg, C)) rows.push_back(sg);
    else rest.push_back(sg);
  }
  hipError_t e = hipSuccess;
  if (!text.empty()) {
    if (B > 65535) return hipErrorInvalidValue;
    e = bf16 ? launch_text_batch<uint16_t>(static_cast<const uint16_t*>(x), static_cast<uint16_t*>(y), w_text, B,
                                           Ttot, C, text.data(), (int)text.size(), stream, marks)
             : launch_text_batch<float>(static_cast<const float*>(x), static_cast<float*>(y), w_text, B, Ttot, C,
                                        text.data(), (int)text.size(), stream, marks);
    if (e != hipSuccess) return e;
  }
  if (!rows.empty()) {
    e = launch_rows_batch<4, 32>(static_cast<const uint16_t*>(x), static_cast<uint16_t*>(y), w_vis, B, Ttot, C,
                                 rows.data(), (int)rows.size(), stream, marks);
    if (e != hipSuccess) return e;
  }
  for (const Seg& sg : rest) {
    e = launch_conv_segment(x, y, B, Ttot, C, bf16, w_text, w_vis, sg, false, stream, marks);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

bool conv_rows_adjoint_ok(const Seg& seg, int64_t C, bool bf16) {
  return bf16 && seg.kind != SEG_TEXT && seg.frames == 1 && C % 64 == 0 && rows_fit<4, 32>(seg, C);
}

hipError_t launch_conv_rows_adjoint(const void* dy, void* dx, const float* w_vis, int64_t B, int64_t Ttot, int64_t C,
                                    const Seg* segs, int n, hipStream_t stream, Marks* marks) {
  if (B == 0 || n == 0) return hipSuccess;
  return launch_rows_batch<4, 32, true>(static_cast<const uint16_t*>(dy), static_cast<uint16_t*>(dx), w_vis, B, Ttot,
                                        C, segs, n, stream, marks);
}

bool conv_tile_adjoint_ok(const Seg& seg, int64_t C, bool bf16) {
  return bf16 && seg.kind != SEG_TEXT && C % 64 == 0 && (int64_t)seg.height * seg.width * C * 2 <= (int64_t)kOutside - 64;
}

hipError_t launch_conv_tile_adjoint(const void* dy, void* dx, const float* w_vis, int64_t B, int64_t Ttot, int64_t C,
                                    const Seg& seg, hipStream_t stream, Marks* marks) {
  if (B == 0 || seg.length == 0) return hipSuccess;
  return launch_tile<3, 4, 4, 16>(static_cast<const uint16_t*>(dy), static_cast<uint16_t*>(dx), w_vis, B, Ttot, C, seg,
                                  stream, marks, true);
}

hipError_t launch_index_device(const Seg& seg, int64_t T, int32_t* idx, hipStream_t stream) {
  (void)T;
  if (seg.length == 0) return hipSuccess;
  const int64_t blocks = (seg.length + 255) / 256;
  hipLaunchKernelGGL(index_device_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, seg, idx);
  return hipGetLastError();
}

}  // namespace chm
