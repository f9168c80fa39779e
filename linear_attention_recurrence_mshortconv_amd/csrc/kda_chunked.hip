// Chunked KDA forward on gfx950 MFMA (bf16 operands, fp32 state), dk = dv = 128.
//
// The recurrence is Eq. 14 of Chimera page 1, section 3.3 (parentheses as on
// page 2): S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T, read out
// as o_t = S_t^T q_t (Eq. 15, inner term). The pages give no chunked form; the
// one used here follows from Eq. 14 by unrolling it over a chunk of 64 tokens.
// With g_r = sum_{i<=r} log a_i per key channel (restarting every chunk),
// incoming state S and u_r = b_r (v_r - S_{r-1}^T Diag(a_r) k_r):
//
//   S_r = Diag(e^{g_r}) (S + sum_{i<=r} (k_i e^{-g_i}) u_i^T)
//   (I + A) U = diag(b) (V - (K e^g) S),      A_ri = b_r sum_c k_rc k_ic e^{g_rc - g_ic}  (i < r)
//   O = (Q e^g) S + Aqk U,                    Aqk_ri = sum_c q_rc k_ic e^{g_rc - g_ic}  (i <= r)
//   S_next = Diag(e^{g_n}) S + (K e^{g_n - g})^T U
//
// so with T = (I + A)^{-1} the chunk step is U = T diag(b) (V - (K e^g) S): the UT transform
// is applied per state column to the residual, and no W = T diag(b) K e^g is formed. Decays are
// running products of alpha (no log / exp). The per-(token, head) L2 normalisation of q and k
// (page 1, Fig. 2) is folded into the bf16 operands as they are formed (K^, K_ and Q^ carry
// 1 / |k| and 1 / |q|), so no product needs a separate norm scaling.
//
// Work layout. A block of 8 waves runs one segment of chunks of one (sequence, head) and
// fills a CU. Waves 0-3 produce: they load a chunk, form its operands and A / Aqk and invert
// the diagonal blocks of I + A; waves 4-7 consume one chunk behind them, each holding 32 state
// columns in registers for the whole segment. The two roles pass each other per-chunk
// operands through two LDS stages, with three block barriers per chunk. Operands live in LDS
// once, row-major [token][channel]; products that contract over tokens read them with the
// gfx950 transposing LDS read (ds_read_b64_tr_b16) instead of keeping transposed copies.
// Channels are stored in a permuted order inside each group of 32 (cpos) so that one 16-byte
// read returns the K order of a state fragment packed from the MFMA D layout.
//
// The sequence is cut into segments so that the chip has one block per CU:
//   summary pass: per segment but the last, one block runs S from 0 and the transition M
//                 from I over it;
//   combine pass: S_start(p + 1) = M_p S_start(p) + S_p, fp32-accurate MFMA;
//   output pass:  each segment reruns from S_start(p), writing o.
// With one segment only the output pass runs, starting from S0.
#include <cstddef>
#include <algorithm>
#include <atomic>
#include <type_traits>
#include <utility>
#include <vector>

#include "dtypes.h"
#include "internal.h"
#include "mfma.h"

namespace chm {
namespace {

constexpr int D = 128;      // dk = dv
constexpr int CT = 64;      // tokens per chunk
constexpr int SBT = 16;     // tokens per decay block
constexpr int NSB = CT / SBT;
constexpr int kTargetBlocks = 256;   // one block per CU
constexpr int kSub = 1;              // output segments per summary segment
constexpr float kL2Eps = 1e-6f;
constexpr float kFastMin = 1.8e-35f; // ~e^{-80}: the chunk-start factorisation is safe above this

__device__ __forceinline__ float pick(float4 v, int u) { return u == 0 ? v.x : u == 1 ? v.y : u == 2 ? v.z : v.w; }
// v split into bf16 high parts (returned) and low parts v - hi (in lo)
__device__ __forceinline__ uint2 pack_split(const float4& v, uint2& lo) {
  const uint2 hi = pack4(v);
  const float4 back = unpack4(hi);
  lo = pack4(make_float4(v.x - back.x, v.y - back.y, v.z - back.z, v.w - back.w));
  return hi;
}
// the 8 bf16 of a fragment scaled by lo (elements 0-3) and hi (4-7)
__device__ __forceinline__ uint4 scale8(uint4 u, float4 lo, float4 hi) {
  return make_uint4(pack_bf16x2(bf_lo(u.x) * lo.x, bf_hi(u.x) * lo.y), pack_bf16x2(bf_lo(u.y) * lo.z, bf_hi(u.y) * lo.w),
                    pack_bf16x2(bf_lo(u.z) * hi.x, bf_hi(u.z) * hi.y), pack_bf16x2(bf_lo(u.w) * hi.z, bf_hi(u.w) * hi.w));
}

// LDS arrays are flat with padded rows (the padding folds into instruction offsets).
//   rk: [CT][D] row-major (kr, kc), row stride D + 16 elements (288 bytes)
//   rm: [CT][D] row-major (qw), row stride D + 8 elements (272 bytes)
//   tr: [CT][CT], row stride CT + 4 elements (136 bytes)
// (measured: the transposing reads and the 16-byte fragment reads of kr and kc
// conflict least at a 288-byte row.)
constexpr int RKS = D + 16;
constexpr int RMS = D + 8;
constexpr int TRS = CT + 4;
__device__ __forceinline__ constexpr int rk(int row, int col) { return row * RKS + col; }
__device__ __forceinline__ constexpr int rm(int row, int col) { return row * RMS + col; }
__device__ __forceinline__ constexpr int tr(int row, int col) { return row * TRS + col; }

// Small arrays first: LDS instruction offsets reach 64 KB from a base register.
// A run of `count` consecutive sequences of `len` tokens each in the packed row dimension
// (rows start .. start + count * len - 1): a batch of B sequences is one run, and samples
// packed in one row with lengths of their own make one run per stretch of equal lengths.
// Each sequence is cut into P output segments (Ps summary segments) of the launch's Lo
// chunks; its per-head workspace region holds E = kSub * Ps summary states, E transitions
// and P start states.
struct SeqDesc {
  int64_t start;          // first row of the run
  int64_t len;            // tokens per sequence
  int64_t ws0;            // first workspace matrix (D x D fp32) of the run
  int32_t count;          // sequences
  int32_t sidx0;          // S0 / S_final index of the run's first sequence
  int32_t P, Ps;          // output and summary segments per (sequence, head)
  int32_t out0, sum0, comb0;   // the run's first block in each pass's grid
  int32_t pad;
};
constexpr int kMaxRuns = 48;   // runs per launch (the kernel arguments stay under 4 KiB)

struct ChunkArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t stride;
  const uint16_t* alpha;
  const uint16_t* beta;
  const float* S0;        // [sequences][H][D][D] or null
  float* ws;              // workspace: D x D fp32 matrices in per-(sequence, head) regions
  uint16_t* o;
  float* S_final;
  const uint16_t* gate;   // output gate [rows][H][D] (token stride gate_stride), or null
  int64_t gate_stride;
  const float* norm_w;    // [D] or null
  float norm_eps;
  int64_t H;
  int dk, dv;             // head sizes (multiples of 8 up to D; the kernels run at D, zero-padded)
  int Lo;                 // chunks per output segment
  int nblk;               // logical blocks of this pass
  int grid;               // launched blocks
  int l2norm;
  int nruns;
  int xcd_ranges;         // give each XCD a contiguous range of logical blocks (one run only)
  // fused conv (the CONV kernels only): q, k, v computed from x [rows][xC] bf16 (the q, k and v
  // channel blocks, head-major inside each) with the weights wT [31][xC] fp32 and the segments
  // of every sequence; conv_back = the farthest any tap reaches back (tokens)
  const uint16_t* x;
  int64_t xC;
  const float* wT;
  const Seg* conv_seg;
  int64_t conv_back;
  int conv_nseg;
  SeqDesc run[kMaxRuns];
};

// The run that logical block `lid` of a pass belongs to: the last run whose first block is
// at most lid (runs without a block in this pass share the next run's first block), by
// binary search over the nondecreasing first blocks.
template <int PASS>   // 0 output, 1 summary, 2 combine
__device__ __forceinline__ int32_t first_block(const SeqDesc& d) {
  return PASS == 0 ? d.out0 : PASS == 1 ? d.sum0 : d.comb0;
}
template <int PASS>
__device__ __forceinline__ int run_of(const ChunkArgs& a, uint32_t lid) {
  int lo = 0, hi = a.nruns - 1;   // the answer lies in [lo, hi]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)lid >= first_block<PASS>(a.run[mid])) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}
// One (sequence, head) of a run: its first row, length, S0 / S_final index and workspace
// region ([E] summary states, [E] transitions, [P] start states, each D x D fp32).
struct SeqView {
  int64_t row0, T, sidx;
  int P, Ps, E;
  float* ws;
};
// (bhl = sequence within the run * H + head; grids stay below 2^31 blocks, so 32-bit
// index arithmetic is enough up to here). Quotients and remainders of block indices pass
// through readfirstlane: the division expands into vector instructions, and a buffer
// descriptor built from a value the compiler cannot see is wave-uniform gets a loop
// around every load that uses it.
__device__ __forceinline__ SeqView seq_view(const ChunkArgs& a, const SeqDesc& d, int32_t bhl) {
  SeqView v;
  const int32_t H = (int32_t)a.H;
  const int32_t seq = uni(bhl / H);
  v.row0 = d.start + (int64_t)seq * d.len;
  v.T = d.len;
  v.sidx = (int64_t)(d.sidx0 + seq) * H + uni(bhl % H);
  v.P = d.P;
  v.Ps = d.Ps;
  v.E = d.Ps * kSub;
  v.ws = a.ws + (d.ws0 + bhl * (int64_t)(2 * v.E + v.P)) * (int64_t)(D * D);
  return v;
}



// the 32 state columns of this wave -> m ([D][D] fp32); svo = lane part of the offset
// the state's rows < dk of its columns < dv (lane rows 16 rt + 4 q4 + r, columns col0 + 16 ct + l16) ->
// m ([dk][dv] fp32)
__device__ __forceinline__ void store_state(const f32x4 (&S)[8][2], float* m, int dk, int dv, int col0, int l16,
                                            int q4) {
#pragma unroll
  for (int rt = 0; rt < 8; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * rt + 4 * q4 + r, col = col0 + 16 * ct + l16;
        if (row < dk && col < dv) m[row * dv + col] = S[rt][ct][r];
      }
}
// Workspace matrices ([D][D] fp32 states and transitions) are kept tile-major: the
// 16 x 16 tile (rt, column block cb, ct) is 256 contiguous floats, lane l = 16 q4 + l16
// holding rows 16 rt + 4 q4 .. + 3 of column 32 cb + 16 ct + l16 (the MFMA D layout),
// so that states move as 16-byte pieces.
__device__ __forceinline__ int tile_off(int cb, int rt, int ct, int lane) {
  return (((cb * 8 + rt) * 2 + ct) * 64 + lane) * 4;
}
__device__ __forceinline__ void store_tiles(const f32x4 (&S)[8][2], float* m, int cb, int lane) {
#pragma unroll
  for (int rt = 0; rt < 8; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) *reinterpret_cast<f32x4*>(m + tile_off(cb, rt, ct, lane)) = S[rt][ct];
}
__device__ __forceinline__ f32x4 load_tile4(const float* m, int cb, int rt, int ct, int lane) {
  return *reinterpret_cast<const f32x4*>(m + tile_off(cb, rt, ct, lane));
}

// Transitions M_e are kept as MFMA A operands, already split into bf16 high and
// low parts: fragment (row tile rt, k slot s) of lane l = 16 q4 + l16 holds row
// 16 rt + l16, columns 32 s + 4 q4 + 0..3 (slots 0-3) and 32 s + 16 + 4 q4 + 0..3
// (slots 4-7); the high uint4 is followed by the low uint4 (64 KiB per matrix).
__device__ __forceinline__ int mfrag_off(int rt, int s, int lane) { return ((rt * 4 + s) * 64 + lane) * 2; }
// Store the 32 columns 32 cb .. 32 cb + 31 held by this wave (D layout) in that form:
// they make up the k slot s = cb of every row tile. Each row tile is transposed
// through this wave's LDS scratch `scr` (two 32 x 40 bf16 arrays, high and low
// parts, laid out like kc: [k][cpos(row)]) and read back with the transposing
// read, so that every global store is a 16-byte piece.
constexpr int kMsP = 40;                            // scratch row pitch (elements)
constexpr int kMsWave = 2 * 32 * kMsP;              // scratch elements per wave
__device__ __forceinline__ void store_mfrag(const f32x4 (&S)[8][2], uint4* m, int cb, int lane, uint16_t* scr) {
  uint16_t* hiB = scr;
  uint16_t* loB = scr + 32 * kMsP;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int kbase = (4 * q4 + (l16 >> 2)) * kMsP + 8 * (l16 & 3);
#pragma unroll
  for (int rt = 0; rt < 8; ++rt) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      uint2 lo;
      const uint2 hi = pack_split(make_float4(S[rt][ct][0], S[rt][ct][1], S[rt][ct][2], S[rt][ct][3]), lo);
      *reinterpret_cast<uint2*>(&hiB[(16 * ct + l16) * kMsP + 8 * q4]) = hi;   // rows 4 q4 .. + 3 at cpos
      *reinterpret_cast<uint2*>(&loB[(16 * ct + l16) * kMsP + 8 * q4]) = lo;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    const uint4 h = cat(ld_tr(&hiB[kbase]), ld_tr(&hiB[kbase + 16 * kMsP]));
    const uint4 l = cat(ld_tr(&loB[kbase]), ld_tr(&loB[kbase + 16 * kMsP]));
    m[mfrag_off(rt, cb, lane)] = h;
    m[mfrag_off(rt, cb, lane) + 1] = l;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
  }
}

// ---- LDS of the pipelined passes ------------------------------------------------------
// A stage holds what the producers form for one chunk and the consumers use one tick later;
// two stages alternate by chunk parity. Arrays are flat with padded rows (the padding folds
// into instruction offsets):
//   kr, kc: [CT][D] row-major, row stride D + 16 elements (288 bytes)
//   qw:     [CT][D] row-major, row stride D + 8 elements (272 bytes)
//   at, aqk: [CT][CT] column-major, stride CT + 4 elements
struct PcStage {
  uint16_t kr[CT * RKS];  // -K^, K^ = k e^{g} / |k| (fast) or k e^{g - m_I} / |k| (blocked), negated so that
                          // the consumers' K^ S products accumulate V - K^ S directly
  uint16_t kc[CT * RKS];  // K_ = k e^{-g} / |k| (fast) or k e^{m_I - g} / |k| (blocked)
  float beta[CT];
  float egn[D];           // e^{g_n}: decay of each key channel over the whole chunk
  float pb[NSB][D];       // per block and channel: product of alpha over block tokens 0..7
  float pf[NSB][D];       //                        ... over block tokens 8..15
  int fast;               // the chunk-start factorisation holds (block-wide vote)
  int pad[3];
};
struct PcLdsOut {         // output pass
  PcStage st[2];
  uint16_t qw[2][CT * RMS];   // Q^ = q e^{g} / |q| (fast) or q e^{g - m_I} / |q| (blocked), per stage;
                              // once a stage's Q^ is used, its qw holds v of the next chunk
  uint16_t at[CT * TRS];      // at[tr(j, i)] = -(K^ K_^T)(i, j) (no b) below the diagonal blocks,
                              // T_II diag(b_I) on them
  uint16_t aqk[CT * TRS];     // aqk[tr(j, i)] = Aqk(i, j), lower triangle with the diagonal
  float adiag[NSB * 272];     // strictly lower A_II in fp32: A_II(i, k) at 272 I + 16 i + k
  float rk[CT];               // 1 / |k_t| (1 without normalisation)
  float rq[CT];
  float rowss[CT * 4];        // gated: per token, each consumer wave's part of the sum of squares
};
struct PcLdsSum {         // summary pass
  PcStage st[2];
  uint16_t vs[CT * RMS];      // v of the consumers' next chunk, row-major (stride RMS)
  uint16_t at[CT * TRS];
  float adiag[NSB * 272];
  float rk[CT];
  float rq[CT];
};
static_assert(sizeof(PcLdsOut) <= 160 * 1024 && sizeof(PcLdsSum) <= 160 * 1024, "one block per CU");
constexpr int kPcThreads = 512;   // 4 producer and 4 consumer waves
static_assert(4 * kMsWave * sizeof(uint16_t) <= sizeof(PcLdsSum), "the four M waves' scratch lies in the summary LDS");

// ---- fused conv in the load stage ------------------------------------------------------
// Chimera page 1, section 3.4: mShortConv on packed storage, each segment convolved on its own
// (Eq. 13; neighbours by Eq. 12, zero outside the segment, causal in time). The CONV kernels
// compute q, k and v of a chunk from x as they load it: producers k (and q), consumers v. Per
// token and tap slot (slots 0-3: the text taps; slots 4-30: visual tap (kt, kh, kw) at
// 4 + 9 kt + 3 kh + kw), the producers tabulate the byte offset of the source token's x row
// inside the chunk's window of x (the rows from conv_back tokens before the chunk on), or an
// offset past the window for zero padding. Each lane then sums its tokens' taps slot by slot
// with fmaf from zero, the slots in increasing order, which is the tap order of the conv
// kernels, and rounds once to bf16: q, k and v are what the conv call stores, bit for bit.
constexpr int kConvSlots = 31;
constexpr uint32_t kOffPad = 0x7FFFFFF0u;   // window offsets stay below this; padding reads past it
struct ConvLds {
  uint32_t nb[2][CT][32];   // per chunk parity: [token][slot] window byte offset of the source row
  Seg seg[kMaxFusedSegs];   // the segments of a sequence
  uint32_t gmask[2];        // per chunk parity: the slot groups its tokens use (bit 0: text taps;
                            // bit 1 + 3 kt + kh: visual taps (kt, kh, 0..2))
  uint32_t pad[2];
};
static_assert(sizeof(PcLdsOut) + sizeof(ConvLds) <= 160 * 1024, "the conv tables fit beside the output pass");

// x rows of the window of chunk c: from max(0, c CT - conv_back) to the sequence end
__device__ __forceinline__ int64_t conv_window_start(const ChunkArgs& a, int64_t c) {
  return max<int64_t>(0, c * CT - a.conv_back);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t conv_window(const ChunkArgs& a, int64_t row0, int64_t T, int64_t c) {
  const int64_t wb = conv_window_start(a, c);
  const int64_t bytes = (T - wb) * a.xC * 2;
  return __builtin_amdgcn_make_buffer_rsrc((void*)(a.x + (row0 + wb) * a.xC), 0,
                                           (int)min<int64_t>(bytes, (int64_t)kOffPad), kRsrcW3);
}
// The table of chunk c (n valid tokens) by the 256 producer threads (ptid): token ptid / 4,
// slots ptid % 4 + 4 m. Thread 0 also forms the chunk's slot-group mask.
__device__ __forceinline__ void conv_fill(const ChunkArgs& a, int64_t T, ConvLds& CL, int64_t c, int ptid) {
  const int i = ptid >> 2, part = ptid & 3;
  const int64_t t0 = c * CT, p = t0 + i;
  const int64_t wb = conv_window_start(a, c);
  const uint32_t C2 = (uint32_t)a.xC * 2;
  uint32_t* row = CL.nb[c & 1][i];
  const int nseg = a.conv_nseg;
  if (p < T) {
    int lo = 0, hi = nseg - 1;   // the segment holding p: the last one starting at or before it
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (CL.seg[mid].start <= p) lo = mid;
      else hi = mid - 1;
    }
    const Seg sg = CL.seg[lo];
    const bool text = sg.kind == SEG_TEXT;
    // grid point of p (Eq. 12), 32-bit: positions inside a sequence stay below 2^31
    const uint32_t local = (uint32_t)(p - sg.start), W = (uint32_t)max(sg.width, 1);
    const uint32_t HW = (uint32_t)max(sg.height, 1) * W;
    const uint32_t f = text ? 0u : local / HW, rem = text ? 0u : local - f * HW;
    const uint32_t hh = rem / W, ww = rem - hh * W;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int slot = part + 4 * m;
      int64_t src = -1;
      if (slot < kTextTaps) {
        if (text) src = text_tap_source(sg, p, slot);
      } else if (slot < kConvSlots && !text) {
        const int tap = slot - kTextTaps;
        src = vis_tap_source(sg, f, hh, ww, tap / 9, (tap / 3) % 3, tap % 3);
      }
      row[slot] = src >= 0 ? (uint32_t)(src - wb) * C2 : kOffPad;
    }
  } else {
#pragma unroll
    for (int m = 0; m < 8; ++m) row[part + 4 * m] = kOffPad;   // tokens past the end: q = k = v = 0
  }
  if (ptid == 0) {
    const int64_t t1 = min<int64_t>(T, t0 + CT);
    uint32_t gm = 0;
    for (int k = 0; k < nseg; ++k) {
      const Seg& g = CL.seg[k];
      if (g.start < t1 && g.start + g.length > t0)
        gm |= g.kind == SEG_TEXT ? 1u : g.frames >= 3 ? 0x3FEu : g.frames == 2 ? 0x3F0u : 0x380u;
    }
    CL.gmask[c & 1] = gm;
  }
}
// NTEN tensors (channel ch[e] + 0..3 of the x rows) of NT tokens (table rows tok[i]) of a chunk,
// summed over the slots of the groups in gm, rounded to bf16 into out[e][i].
template <int NT, int NTEN>
__device__ __forceinline__ void conv_tokens(__amdgpu_buffer_rsrc_t rx, const float* wT, int64_t C,
                                            const uint32_t (*nb)[32], const int (&tok)[NT], const int (&ch)[NTEN],
                                            uint32_t gm, uint2 (&out)[NTEN][NT]) {
  float acc[NTEN][NT][4];
#pragma unroll
  for (int e = 0; e < NTEN; ++e)
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[e][i][r] = 0.f;
  // one group of NS slots from s0 on: every load first, then the multiply-adds in slot order
  auto group = [&](auto nsc, int s0) {
    constexpr int NS = decltype(nsc)::value;
    float4 w[NTEN][NS];
    uint2 xv[NTEN][NS][NT];
#pragma unroll
    for (int e = 0; e < NTEN; ++e)
#pragma unroll
      for (int s = 0; s < NS; ++s) w[e][s] = *reinterpret_cast<const float4*>(wT + (s0 + s) * C + ch[e]);
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const uint32_t off = nb[tok[i]][s0 + s];
#pragma unroll
        for (int e = 0; e < NTEN; ++e) xv[e][s][i] = ld_buf64(rx, (int)(off + 2u * (uint32_t)ch[e]), 0);
      }
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int e = 0; e < NTEN; ++e)
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          const float4 xf = unpack4(xv[e][s][i]);
          acc[e][i][0] = fmaf(w[e][s].x, xf.x, acc[e][i][0]);
          acc[e][i][1] = fmaf(w[e][s].y, xf.y, acc[e][i][1]);
          acc[e][i][2] = fmaf(w[e][s].z, xf.z, acc[e][i][2]);
          acc[e][i][3] = fmaf(w[e][s].w, xf.w, acc[e][i][3]);
        }
  };
  if (gm & 1u) group(std::integral_constant<int, kTextTaps>{}, 0);
  for (int g = 1; g < 10; ++g)
    if ((gm >> g) & 1u) group(std::integral_constant<int, 3>{}, kTextTaps + 3 * (g - 1));
#pragma unroll
  for (int e = 0; e < NTEN; ++e)
#pragma unroll
    for (int i = 0; i < NT; ++i)
      out[e][i] = make_uint2(pack_bf16x2(acc[e][i][0], acc[e][i][1]), pack_bf16x2(acc[e][i][2], acc[e][i][3]));
}

// Decay factors of the blocked factorisation for channels c..c+3 (from a stage's pb, pf):
//   em(I)     = e^{m_I}         product of alpha from the chunk start to block I's token 7
//   enm(I)    = e^{g_n - m_I}   ... after block I's token 7 to the chunk end
//   pair(I,J) = e^{m_I - m_J}   ... after block J's token 7 to block I's token 7
__device__ __forceinline__ float4 ldf4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 em_of(const PcStage& st, int I, int c) {
  float4 r = ldf4(&st.pb[I][c]);
#pragma unroll
  for (int J = 0; J < NSB; ++J)
    if (J < I) r = mul4(r, mul4(ldf4(&st.pb[J][c]), ldf4(&st.pf[J][c])));
  return r;
}
__device__ __forceinline__ float4 enm_of(const PcStage& st, int I, int c) {
  float4 r = ldf4(&st.pf[I][c]);
#pragma unroll
  for (int J = 0; J < NSB; ++J)
    if (J > I) r = mul4(r, mul4(ldf4(&st.pb[J][c]), ldf4(&st.pf[J][c])));
  return r;
}
__device__ __forceinline__ float4 pair_of(const PcStage& st, int I, int J, int c) {
  float4 r = mul4(ldf4(&st.pf[J][c]), ldf4(&st.pb[I][c]));
#pragma unroll
  for (int K = 0; K < NSB; ++K)
    if (K > J && K < I) r = mul4(r, mul4(ldf4(&st.pb[K][c]), ldf4(&st.pf[K][c])));
  return r;
}

// ---- MFMA fragment pieces ------------------------------------------------------------
// Fragment conventions (16x16x32 MFMA): lane = 16 q4 + l16; a row fragment of block `blk`
// holds row 16 blk + l16, positions 32 s + 8 q4 .. + 7 for s = 0..3 (channels 32 s + 4 q4 ..
// + 3 and 32 s + 16 + 4 q4 .. + 3 in the cpos order). The A and B operand layouts of this
// instruction are mirror images, so one fragment serves a matrix as A or its transpose as B.
template <int STRIDE = RKS>
__device__ __forceinline__ void tile_frags(const uint16_t* arr, int blk, uint4 (&f)[4], int l16, int q4) {
#pragma unroll
  for (int s = 0; s < 4; ++s) f[s] = ld128(arr, (SBT * blk + l16) * STRIDE + 32 * s + 8 * q4);
}
// column-operand fragments of block J scaled by e^{m_I - m_J} (blocked factorisation)
__device__ __forceinline__ void pair_frags(const PcStage& st, bool fast, int I, int J, const uint4 (&in)[4],
                                           uint4 (&out)[4], int q4) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
    out[s] = fast ? in[s] : scale8(in[s], pair_of(st, I, J, 32 * s + 4 * q4), pair_of(st, I, J, 32 * s + 16 + 4 * q4));
}
__device__ __forceinline__ f32x4 mma4(const uint4 (&ra)[4], const uint4 (&cb)[4]) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = mma32(ra[s], cb[s], acc);
  return acc;
}
// From acc = ((-K^) K_^T)(I, J) (the operands carry 1 / |k|), with A = diag(b) K^ K_^T strictly
// lower: below the diagonal blocks -A'(I, J) = acc without the row factor b -> at (column-major: a
// lane's four rows are one 8-byte write); on the diagonal A_II = diag(b) (K^ K_^T)(I, I) (strictly
// lower part) -> adiag in fp32. The b of each block row goes into T'_II = T_II diag(b_I) instead
// (invert_diag), so that (I + A) U = diag(b) Z is solved block by block as
// U_I = T'_II (Z_I - sum_{J < I} A'(I, J) U_J) with no row scaling of Z.
__device__ __forceinline__ void epi_a(uint16_t* at, float* adiag, const float* beta, int I, int J, f32x4 acc, int l16,
                                      int q4) {
  const int j = SBT * J + l16;
  if (I == J) {
    const float4 b4 = ldf4(&beta[SBT * I + 4 * q4]);
    const float rowf[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) adiag[272 * I + 16 * (4 * q4 + r) + l16] = 4 * q4 + r > l16 ? -rowf[r] * acc[r] : 0.f;
  } else {
    *reinterpret_cast<uint2*>(&at[tr(j, SBT * I + 4 * q4)]) = pack4(acc);
  }
}
// Aqk(I, J) = (Q^ K_^T)(I, J) (the operands carry 1 / |q| and 1 / |k|), lower triangle
// including the diagonal, column-major
__device__ __forceinline__ void epi_q(uint16_t* aqk, int I, int J, f32x4 acc, int l16, int q4) {
  const int j = SBT * J + l16;
  float v[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = (I > J || 4 * q4 + r >= l16) ? acc[r] : 0.f;
  *reinterpret_cast<uint2*>(&aqk[tr(j, SBT * I + 4 * q4)]) = pack4(make_float4(v[0], v[1], v[2], v[3]));
}
// T'_II = (I + A_II)^{-1} diag(b_I): lane j of a 16-lane group forms column j of T_II by forward
// substitution, x_i = [i = j] - sum_{k < i} A_II(i, k) x_k, reading the rows of A_II
// (written by this wave) as broadcasts; the column, times b of token 16 I + j, goes to at as
// four 8-byte writes.
__device__ __forceinline__ void invert_diag(const float* adiag, const float* beta, uint16_t* at, int I, int jj,
                                            bool write) {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  float x[SBT];
#pragma unroll
  for (int i = 0; i < SBT; ++i) {
    float acc0 = i == jj ? 1.f : 0.f, acc1 = 0.f;
#pragma unroll
    for (int k4 = 0; k4 < (i + 3) / 4; ++k4) {
      const float4 a4 = ldf4(&adiag[272 * I + 16 * i + 4 * k4]);
      const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = 4 * k4 + e;
        if (k < i) {
          if (e & 1) acc1 -= av[e] * x[k];
          else acc0 -= av[e] * x[k];
        }
      }
    }
    x[i] = acc0 + acc1;
  }
  if (write) {
    const float bj = beta[SBT * I + jj];
#pragma unroll
    for (int m = 0; m < 4; ++m)
      *reinterpret_cast<uint2*>(&at[tr(SBT * I + jj, SBT * I + 4 * m)]) =
          make_uint2(pack_bf16x2(bj * x[4 * m], bj * x[4 * m + 1]), pack_bf16x2(bj * x[4 * m + 2], bj * x[4 * m + 3]));
  }
}
// mma16 A fragments of at (transposed reads): block (I, J), J <= I, at I (I + 1) / 2 + J
__device__ __forceinline__ void load_t_frags(const uint16_t* at, uint2 (&af)[10], int l16, int q4) {
#pragma unroll
  for (int I = 0; I < 4; ++I)
#pragma unroll
    for (int J = 0; J <= I; ++J)
      af[I * (I + 1) / 2 + J] = ld_tr(&at[tr(SBT * J + 4 * q4 + (l16 >> 2), SBT * I + 4 * (l16 & 3))]);
}
// X = (I + A)^{-1} diag(b) Z by block forward substitution, X_I = T'_II (Z_I - sum_{J < I} A'(I, J) X_J)
// (af: -A' below the diagonal, T' on it), Z and X in the D layout
__device__ __forceinline__ void block_solve(const uint2 (&af)[10], const f32x4 (&y0)[4], f32x4 (&X)[4]) {
  uint2 Xb[4];
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    f32x4 y = y0[I];
#pragma unroll
    for (int J = 0; J < I; ++J) y = mma16(af[I * (I + 1) / 2 + J], Xb[J], y);
    X[I] = mma16(af[I * (I + 1) / 2 + I], pack4(y), f32x4{0.f, 0.f, 0.f, 0.f});
    Xb[I] = pack4(X[I]);
  }
}

// ---- producer waves ------------------------------------------------------------------
// Producer wave w handles decay block w (tokens 16 w .. 16 w + 15): half-wave hf = tokens
// 8 hf .. 8 hf + 7 of the block, lane cg = 32-lane index = channels 4 cg .. 4 cg + 3.
struct PLoad {
  uint2 k[8], q[8], a[8];   // tokens tk0 .. tk0 + 7, channels c0 .. c0 + 3
  uint16_t bt;              // beta of token `lane` (wave 0)
};
// Buffer loads of chunk c: block-uniform base and bounds (the chunk's first n tokens); reads
// past the bound return zero, which is k = q = beta = 0 for tokens past the end (alpha is set
// to 1 for them when it is used).
// alpha and beta of chunk c (needed first, in phase 1; issued as soon as phase 1 has used the
// previous chunk's)
__device__ __forceinline__ void p_issue_a(const ChunkArgs& a, const SeqView& sv, int64_t h, int64_t c, int wave,
                                          int lane, PLoad& R) {
  const int hf = lane >> 5, c0 = 4 * (lane & 31);
  const int64_t t0 = c * CT;
  const int n = (int)min<int64_t>(CT, sv.T - t0);
  const int64_t row0 = sv.row0 + t0;
  const int sa2 = (int)(a.H * a.dk) * 2;
  const auto ra_ = __builtin_amdgcn_make_buffer_rsrc((void*)(a.alpha + (row0 * a.H + h) * a.dk), 0, n * sa2, kRsrcW3);
  const int va = c0 < a.dk ? (8 * hf) * sa2 + 2 * c0 : kOffOut;   // padded channels: alpha = 1 (p_phase1)
  const int tb = SBT * wave;
#pragma unroll
  for (int i = 0; i < 8; ++i) R.a[i] = ld_buf64(ra_, va, (tb + i) * sa2);
  if (wave == 0) {
    const auto rb_ = __builtin_amdgcn_make_buffer_rsrc((void*)(a.beta + row0 * a.H + h), 0, n * (int)a.H * 2, kRsrcW3);
    R.bt = __builtin_amdgcn_raw_buffer_load_b16(rb_, lane * (int)a.H * 2, 0, 0);
  }
}
// k (and q) of chunk c (issued once phase 2 has used the previous chunk's)
template <bool HASQ>
__device__ __forceinline__ void p_issue_kq(const ChunkArgs& a, const SeqView& sv, int64_t h, int64_t c, int wave,
                                           int lane, PLoad& R) {
  const int hf = lane >> 5, c0 = 4 * (lane & 31);
  const int64_t t0 = c * CT;
  const int n = (int)min<int64_t>(CT, sv.T - t0);
  const int64_t row0 = sv.row0 + t0;
  const int st2 = (int)a.stride * 2;
  const auto rk_ = __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + row0 * a.stride + h * a.dk), 0, n * st2, kRsrcW3);
  const int vk = c0 < a.dk ? (8 * hf) * st2 + 2 * c0 : kOffOut;   // padded channels: k = q = 0
  const int tb = SBT * wave;
#pragma unroll
  for (int i = 0; i < 8; ++i) R.k[i] = ld_buf64(rk_, vk, (tb + i) * st2);
  if (HASQ) {
    const auto rq_ = __builtin_amdgcn_make_buffer_rsrc((void*)(a.q + row0 * a.stride + h * a.dk), 0, n * st2, kRsrcW3);
#pragma unroll
    for (int i = 0; i < 8; ++i) R.q[i] = ld_buf64(rq_, vk, (tb + i) * st2);
  }
}

// CONV: k (and q) of chunk c by the conv of x in the layout of p_issue_kq (the chunk's table
// ready in CL)
template <bool HASQ>
__device__ __forceinline__ void p_conv_kq(const ChunkArgs& a, const SeqView& sv, const ConvLds& CL, int64_t h,
                                          int64_t c, int wave, int lane, PLoad& R) {
  const int hf = lane >> 5, c0 = 4 * (lane & 31);
  int tok[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) tok[i] = SBT * wave + 8 * hf + i;
  const auto rx = conv_window(a, sv.row0, sv.T, c);
  const uint32_t gm = __builtin_amdgcn_readfirstlane(CL.gmask[c & 1]);
  const int kch = (int)((a.H + h) * D) + c0;
  {
    const int ch[1] = {kch};
    uint2 out[1][8];
    conv_tokens<8, 1>(rx, a.wT, a.xC, CL.nb[c & 1], tok, ch, gm, out);
#pragma unroll
    for (int i = 0; i < 8; ++i) R.k[i] = out[0][i];
  }
  if (HASQ) {
    const int ch[1] = {(int)(h * D) + c0};
    uint2 out[1][8];
    conv_tokens<8, 1>(rx, a.wT, a.xC, CL.nb[c & 1], tok, ch, gm, out);
#pragma unroll
    for (int i = 0; i < 8; ++i) R.q[i] = out[0][i];
  }
}

// Phase 1: beta, per-token norms, block decay products of chunk c (n valid tokens) into stage st.
template <bool HASQ>
__device__ __forceinline__ void p_phase1(const ChunkArgs& a, PcStage& st, float* rkn, float* rqn, const PLoad& R, int n,
                                         int wave, int lane, float4 (&al)[8]) {
  const int hf = lane >> 5, cg = lane & 31, c0 = 4 * cg;
  const int tk0 = SBT * wave + 8 * hf;
  if (wave == 0) st.beta[lane] = bf2f(R.bt);
  if (a.l2norm) {
    float ss[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ss[i] = dot4(R.k[i]);
      ss[i + 8] = HASQ ? dot4(R.q[i]) : 0.f;
    }
    const float tot = half_sum16(ss, lane);
    if ((lane & 1) == 0) {
      const int vv = (lane >> 1) & 15;          // 0..7: k of token vv; 8..15: q of token vv - 8
      const float rn = __builtin_amdgcn_rsqf(tot + kL2Eps);
      if (vv < 8) rkn[tk0 + vv] = rn;
      else if (HASQ) rqn[tk0 + vv - 8] = rn;
    }
  } else if (cg < 8) {
    rkn[tk0 + cg] = 1.f;
    rqn[tk0 + cg] = 1.f;
  }
  const uint32_t one2 = 0x3F803F80u;   // alpha = 1 past the end
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool in = tk0 + i < n;
    const bool use = in && c0 < a.dk;
    al[i] = unpack4(make_uint2(use ? clamp_alpha2(R.a[i].x) : one2, use ? clamp_alpha2(R.a[i].y) : one2));
  }
  float4 hp = al[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) hp = mul4(hp, al[i]);
  *reinterpret_cast<float4*>(hf ? &st.pf[wave][c0] : &st.pb[wave][c0]) = hp;
}

// Phase 2: decay factors and the MFMA operands K^, K_ (and Q^) of the chunk into stage st.
// Returns the factorisation vote (the same in every wave: each holds all 128 channels).
template <bool HASQ>
__device__ __forceinline__ bool p_phase2(PcStage& st, uint16_t* qw, const float* rkn, const float* rqn, const PLoad& R,
                                         const float4 (&al)[8], int wave, int lane) {
  const int hf = lane >> 5, cg = lane & 31, c0 = 4 * cg, p0 = cpos(c0);
  const int tk0 = SBT * wave + 8 * hf;
  // per channel: before = decay over the blocks before this one, after = over the blocks after
  // it; the lane's half adds its block's other half on one side
  float4 full[NSB], h0w = make_float4(1.f, 1.f, 1.f, 1.f), h1w = h0w;
#pragma unroll
  for (int J = 0; J < NSB; ++J) {
    const float4 h0 = ldf4(&st.pb[J][c0]), h1 = ldf4(&st.pf[J][c0]);
    full[J] = mul4(h0, h1);
    if (J == wave) { h0w = h0; h1w = h1; }
  }
  float4 egn4 = full[0], before = make_float4(1.f, 1.f, 1.f, 1.f), after = before;
#pragma unroll
  for (int J = 1; J < NSB; ++J) egn4 = mul4(egn4, full[J]);
#pragma unroll
  for (int J = 0; J < NSB; ++J) {
    if (J < wave) before = mul4(before, full[J]);
    if (J > wave) after = mul4(after, full[J]);
  }
  const bool fast = __all(fminf(fminf(egn4.x, egn4.y), fminf(egn4.z, egn4.w)) >= kFastMin) != 0;
  if (wave == 0 && hf == 0) *reinterpret_cast<float4*>(&st.egn[c0]) = egn4;
  if (wave == 0 && lane == 0) st.fast = fast ? 1 : 0;
  // 1 / |k| and 1 / |q| of the lane's tokens go into the operands, so that no product
  // downstream needs a norm scaling
  const float4 rk0 = ldf4(&rkn[tk0]), rk1 = ldf4(&rkn[tk0 + 4]);
  float rkt[8] = {rk0.x, rk0.y, rk0.z, rk0.w, rk1.x, rk1.y, rk1.z, rk1.w};
  float rqt[8];
  if (HASQ) {
    const float4 rq0 = ldf4(&rqn[tk0]), rq1 = ldf4(&rqn[tk0 + 4]);
    rqt[0] = rq0.x; rqt[1] = rq0.y; rqt[2] = rq0.z; rqt[3] = rq0.w;
    rqt[4] = rq1.x; rqt[5] = rq1.y; rqt[6] = rq1.z; rqt[7] = rq1.w;
  }
  auto put = [&](int i, float4 fr, float4 fc) {
    const int tk = tk0 + i;
    const float4 ks = mul4(unpack4(R.k[i]), make_float4(rkt[i], rkt[i], rkt[i], rkt[i]));
    *reinterpret_cast<uint2*>(&st.kr[rk(tk, p0)]) = pack4(mul4(ks, make_float4(-fr.x, -fr.y, -fr.z, -fr.w)));
    *reinterpret_cast<uint2*>(&st.kc[rk(tk, p0)]) = pack4(mul4(ks, fc));
    if (HASQ) {
      const float4 qs = mul4(unpack4(R.q[i]), make_float4(rqt[i], rqt[i], rqt[i], rqt[i]));
      *reinterpret_cast<uint2*>(&qw[rm(tk, p0)]) = pack4(mul4(qs, fr));
    }
  };
  if (fast) {
    // e^{g_t} as a prefix product from the chunk start and e^{g_n - g_t} / e^{g_n} as a suffix
    // product towards the chunk end: no per-element reciprocal
    float4 fw = hf ? mul4(before, h0w) : before;
    float4 bw = mul4(hf ? after : mul4(after, h1w), rcp4(egn4));
    float4 fr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      fw = mul4(fw, al[i]);
      fr[i] = fw;
    }
#pragma unroll
    for (int i = 7; i >= 0; --i) {
      put(i, fr[i], bw);
      if (i > 0) bw = mul4(bw, al[i]);
    }
  } else {
    // blocked: reference m_I = g at the block's token 7; half 1 runs forward (e^{g - m_I} =
    // product over tokens 8..t), half 0 backward (e^{m_I - g} = product over tokens t+1..7)
    if (hf == 1) {
      float4 run = make_float4(1.f, 1.f, 1.f, 1.f);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        run = mul4(run, al[i]);
        put(i, run, rcp4(run));
      }
    } else {
      float4 run = make_float4(1.f, 1.f, 1.f, 1.f);
#pragma unroll
      for (int i = 7; i >= 0; --i) {
        put(i, rcp4(run), run);
        run = mul4(run, al[i]);
      }
    }
  }
  return fast;
}

// Phase 3 of the output pass: the A and Aqk blocks of the chunk and the diagonal inverses.
//   wave 0: the four diagonal A blocks and their inverses (the chunk's longest chain);
//   wave 1: Aqk00 A10 Aqk10 A20 Aqk20 A30;  wave 2: Aqk11 A21 Aqk21 A31 Aqk31;
//   wave 3: Aqk22 A32 Aqk32 Aqk33 Aqk30
__device__ __forceinline__ void p_phase3_out(const PcStage& st, const uint16_t* qw, uint16_t* at, uint16_t* aqk,
                                             float* adiag, bool fast, int wave, int lane) {
  const int l16 = lane & 15, q4 = lane >> 4;
  uint4 cA[4], cB[4], rA[4], sc[4];
  if (wave == 0) {
    __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int I = 0; I < NSB; ++I) {
      tile_frags(st.kc, I, cA, l16, q4);
      tile_frags(st.kr, I, rA, l16, q4);
      epi_a(at, adiag, st.beta, I, I, mma4(rA, cA), l16, q4);
    }
    invert_diag(adiag, st.beta, at, lane >> 4, lane & 15, true);
    __builtin_amdgcn_s_setprio(0);
  } else if (wave == 1) {
    tile_frags(st.kc, 0, cA, l16, q4);
    tile_frags<RMS>(qw, 0, rA, l16, q4);
    epi_q(aqk, 0, 0, mma4(rA, cA), l16, q4);
#pragma unroll
    for (int I = 1; I < NSB; ++I) {
      pair_frags(st, fast, I, 0, cA, sc, q4);
      tile_frags(st.kr, I, rA, l16, q4);
      epi_a(at, adiag, st.beta, I, 0, mma4(rA, sc), l16, q4);
      if (I < 3) {
        tile_frags<RMS>(qw, I, rA, l16, q4);
        epi_q(aqk, I, 0, mma4(rA, sc), l16, q4);
      }
    }
  } else if (wave == 2) {
    tile_frags(st.kc, 1, cA, l16, q4);
    tile_frags<RMS>(qw, 1, rA, l16, q4);
    epi_q(aqk, 1, 1, mma4(rA, cA), l16, q4);
#pragma unroll
    for (int I = 2; I < NSB; ++I) {
      pair_frags(st, fast, I, 1, cA, sc, q4);
      tile_frags(st.kr, I, rA, l16, q4);
      epi_a(at, adiag, st.beta, I, 1, mma4(rA, sc), l16, q4);
      tile_frags<RMS>(qw, I, rA, l16, q4);
      epi_q(aqk, I, 1, mma4(rA, sc), l16, q4);
    }
  } else {
    tile_frags(st.kc, 2, cA, l16, q4);
    tile_frags<RMS>(qw, 2, rA, l16, q4);
    epi_q(aqk, 2, 2, mma4(rA, cA), l16, q4);
    pair_frags(st, fast, 3, 2, cA, sc, q4);
    tile_frags(st.kr, 3, rA, l16, q4);
    epi_a(at, adiag, st.beta, 3, 2, mma4(rA, sc), l16, q4);
    tile_frags<RMS>(qw, 3, rA, l16, q4);
    epi_q(aqk, 3, 2, mma4(rA, sc), l16, q4);
    tile_frags(st.kc, 3, cB, l16, q4);
    epi_q(aqk, 3, 3, mma4(rA, cB), l16, q4);
    tile_frags(st.kc, 0, cB, l16, q4);
    pair_frags(st, fast, 3, 0, cB, sc, q4);
    epi_q(aqk, 3, 0, mma4(rA, sc), l16, q4);
  }
}

// Phase 3 of the summary pass: the A blocks; wave w forms diagonal block w and its inverse (all
// four lane groups compute it, the first writes it) and the blocks below the diagonal
// (wave 0: A10 A32, wave 1: A20, wave 2: A30 A21, wave 3: A31).
__device__ __forceinline__ void p_phase3_sum(const PcStage& st, uint16_t* at, float* adiag, bool fast, int wave,
                                             int lane) {
  const int l16 = lane & 15, q4 = lane >> 4;
  uint4 cA[4], rA[4], sc[4];
  tile_frags(st.kc, wave, cA, l16, q4);
  tile_frags(st.kr, wave, rA, l16, q4);
  __builtin_amdgcn_s_setprio(3);
  epi_a(at, adiag, st.beta, wave, wave, mma4(rA, cA), l16, q4);
  invert_diag(adiag, st.beta, at, wave, l16, q4 == 0);
  __builtin_amdgcn_s_setprio(0);
  auto below = [&](int I, int J) {
    tile_frags(st.kc, J, cA, l16, q4);
    pair_frags(st, fast, I, J, cA, sc, q4);
    tile_frags(st.kr, I, rA, l16, q4);
    epi_a(at, adiag, st.beta, I, J, mma4(rA, sc), l16, q4);
  };
  if (wave == 0) {
    below(1, 0);
    below(3, 2);
  } else if (wave == 1) {
    below(2, 0);
  } else if (wave == 2) {
    below(3, 0);
    below(2, 1);
  } else {
    below(3, 1);
  }
}

// ---- consumer waves ------------------------------------------------------------------
// Consumer wave j owns state columns 32 j .. 32 j + 31 in registers for the whole segment:
// X[rt][ct] holds rows 16 rt + 4 q4 + r, columns 32 j + 16 ct + l16 (the MFMA D layout).

// v of chunk c, rows 16 cw .. 16 cw + 15, loaded whole: half-wave hf takes row 16 cw + 2 i + hf,
// lane channels 4 (lane & 31) .. + 3 (one 256-byte token row per half-wave and load; tokens past
// the end read 0). The consumers' MFMA layout would touch 16 token rows per load; instead the
// rows go through LDS (c_stage_v) and come back in that layout with the transposing read.
template <int ROWS>   // rows per consumer wave: cw takes rows ROWS cw .. ROWS cw + ROWS - 1
__device__ __forceinline__ void c_issue_v(const ChunkArgs& a, const SeqView& sv, int64_t h, int64_t c, int cw,
                                          int lane, uint2 (&vr)[ROWS / 2]) {
  const int64_t t0 = c * CT;
  const int n = (int)min<int64_t>(CT, sv.T - t0);
  const int st2 = (int)a.stride * 2;
  const auto rv = __builtin_amdgcn_make_buffer_rsrc((void*)(a.v + (sv.row0 + t0) * a.stride + h * a.dv), 0, n * st2,
                                                    kRsrcW3);
  const int vo = 4 * (lane & 31) < a.dv ? (ROWS * cw + (lane >> 5)) * st2 + 8 * (lane & 31) : kOffOut;
#pragma unroll
  for (int i = 0; i < ROWS / 2; ++i) vr[i] = ld_buf64(rv, vo, 2 * i * st2);
}
// the rows of c_issue_v -> vbuf ([CT][D], row stride RMS, natural channel order)
template <int ROWS>
__device__ __forceinline__ void c_stage_v(uint16_t* vbuf, const uint2 (&vr)[ROWS / 2], int cw, int lane) {
  const int r0 = ROWS * cw + (lane >> 5), c0 = 4 * (lane & 31);
#pragma unroll
  for (int i = 0; i < ROWS / 2; ++i) *reinterpret_cast<uint2*>(&vbuf[rm(r0 + 2 * i, c0)]) = vr[i];
}

// CONV: the rows of c_issue_v computed by the conv of x (the chunk's table ready in CL)
template <int ROWS>
__device__ __forceinline__ void c_conv_v(const ChunkArgs& a, const SeqView& sv, const ConvLds& CL, int64_t h,
                                         int64_t c, int cw, int lane, uint2 (&vr)[ROWS / 2]) {
  int tok[ROWS / 2];
#pragma unroll
  for (int i = 0; i < ROWS / 2; ++i) tok[i] = ROWS * cw + 2 * i + (lane >> 5);
  const auto rx = conv_window(a, sv.row0, sv.T, c);
  const uint32_t gm = __builtin_amdgcn_readfirstlane(CL.gmask[c & 1]);
  const int ch[1] = {(int)((2 * a.H + h) * D) + 4 * (lane & 31)};
  uint2 out[1][ROWS / 2];
  conv_tokens<ROWS / 2, 1>(rx, a.wT, a.xC, CL.nb[c & 1], tok, ch, gm, out);
#pragma unroll
  for (int i = 0; i < ROWS / 2; ++i) vr[i] = out[0][i];
}

// U = (I + A)^{-1} diag(beta) (V - K^ X) for the wave's column tiles (the block solve with T' and
// A', which carry diag(beta)): the first VCT tiles take V
// (columns col0 + 16 ct of v), the others V = 0 (the transition's columns). V comes from its LDS
// staging in the D layout through the transposing read; (-K^) X accumulates on top (kr holds
// -K^), one k slot of X packed at a time.
// MODE: 0 the factorisation chosen per fragment from `fast`; 1 fast; 2 blocked
template <int NCT, int VCT, int MODE>   // column tiles of 16 (col0 + 16 ct)
__device__ __forceinline__ void c_solve_f(const PcStage& st, const uint16_t* at, const uint16_t* vbuf, bool fast,
                                          const f32x4 (&X)[8][NCT], int col0, f32x4 (&U)[4][NCT], int l16, int q4) {
  const bool blocked = MODE == 0 ? !fast : MODE == 2;
  f32x4 acc[4][NCT];
#pragma unroll
  for (int I = 0; I < 4; ++I)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      if (vbuf != nullptr && ct < VCT) {
        // lane (l16, q4) receives rows 16 I + 4 q4 + 0..3 of column col0 + 16 ct + l16
        const float4 vv = unpack4(ld_tr(&vbuf[rm(SBT * I + 4 * q4 + (l16 >> 2), col0 + 16 * ct + 4 * (l16 & 3))]));
        acc[I][ct] = f32x4{vv.x, vv.y, vv.z, vv.w};
      } else {
        acc[I][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint4 xs[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) xs[ct] = pack8(X[2 * s][ct], X[2 * s + 1][ct]);
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      uint4 kf = ld128(st.kr, (SBT * I + l16) * RKS + 32 * s + 8 * q4);
      if (blocked) kf = scale8(kf, em_of(st, I, 32 * s + 4 * q4), em_of(st, I, 32 * s + 16 + 4 * q4));
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) acc[I][ct] = mma32(kf, xs[ct], acc[I][ct]);
    }
  }
  uint2 af[10];   // T' on the diagonal blocks carries diag(b)
  load_t_frags(at, af, l16, q4);
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const f32x4 y0[4] = {acc[0][ct], acc[1][ct], acc[2][ct], acc[3][ct]};
    f32x4 Xo[4];
    block_solve(af, y0, Xo);
#pragma unroll
    for (int I = 0; I < 4; ++I) U[I][ct] = Xo[I];
  }
}
// SPLIT: each factorisation compiled on its own, so that the fast path is straight-line code whose
// LDS loads the compiler can move ahead of the MFMAs (where the registers allow it)
template <int NCT, int VCT = NCT, bool SPLIT = false>
__device__ __forceinline__ void c_solve(const PcStage& st, const uint16_t* at, const uint16_t* vbuf, bool fast,
                                        const f32x4 (&X)[8][NCT], int col0, f32x4 (&U)[4][NCT], int l16, int q4) {
  if (!SPLIT) c_solve_f<NCT, VCT, 0>(st, at, vbuf, fast, X, col0, U, l16, q4);
  else if (fast) c_solve_f<NCT, VCT, 1>(st, at, vbuf, fast, X, col0, U, l16, q4);
  else c_solve_f<NCT, VCT, 2>(st, at, vbuf, fast, X, col0, U, l16, q4);
}

// X <- Diag(e^{g_n}) X + K~^T U, K~ = (K / |k|) e^{g_n - g} read transposed from kc
template <int NCT, int MODE>   // MODE as for c_solve_f
__device__ __forceinline__ void c_update_f(const PcStage& st, bool fast_rt, f32x4 (&X)[8][NCT],
                                           const f32x4 (&U)[4][NCT], int l16, int q4) {
  const bool fast = MODE == 0 ? fast_rt : MODE == 1;
  uint4 Upf[2][NCT];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) Upf[s][ct] = pack8(U[2 * s][ct], U[2 * s + 1][ct]);
  // A operand K~^T: lane (l16, q4) = channel 16 rt + l16, tokens 32 s + 4 q4 + 0..3 and
  // 32 s + 16 + 4 q4 + 0..3
  const int kbase = rk(4 * q4 + (l16 >> 2), 8 * (l16 & 3));
#pragma unroll
  for (int rt = 0; rt < 8; ++rt) {
    const int cp = 32 * (rt >> 1) + 4 * (rt & 1);   // cpos(16 rt)
    uint4 kt[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
      kt[s] = cat(ld_tr(&st.kc[kbase + rk(32 * s, cp)]), ld_tr(&st.kc[kbase + rk(32 * s + 16, cp)]));
    const float4 eg = ldf4(&st.egn[16 * rt + 4 * q4]);
    if (fast) {   // K~ = K_ e^{g_n}: the factor is a row scaling of the product
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 acc = X[rt][ct];
        acc = mma32(kt[0], Upf[0][ct], acc);
        acc = mma32(kt[1], Upf[1][ct], acc);
        acc[0] *= eg.x; acc[1] *= eg.y; acc[2] *= eg.z; acc[3] *= eg.w;
        X[rt][ct] = acc;
      }
    } else {      // blocked: K~ = K_ e^{g_n - m_I} for the tokens of block I
      const int cl = 16 * rt + (l16 & ~3), u = l16 & 3;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const float f0 = pick(enm_of(st, 2 * s, cl), u), f1 = pick(enm_of(st, 2 * s + 1, cl), u);
        kt[s] = scale8(kt[s], make_float4(f0, f0, f0, f0), make_float4(f1, f1, f1, f1));
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 acc = X[rt][ct];
        acc[0] *= eg.x; acc[1] *= eg.y; acc[2] *= eg.z; acc[3] *= eg.w;
        acc = mma32(kt[0], Upf[0][ct], acc);
        acc = mma32(kt[1], Upf[1][ct], acc);
        X[rt][ct] = acc;
      }
    }
  }
}
template <int NCT, bool SPLIT = false>
__device__ __forceinline__ void c_update(const PcStage& st, bool fast, f32x4 (&X)[8][NCT], const f32x4 (&U)[4][NCT],
                                         int l16, int q4) {
  if (!SPLIT) c_update_f<NCT, 0>(st, fast, X, U, l16, q4);
  else if (fast) c_update_f<NCT, 1>(st, fast, X, U, l16, q4);
  else c_update_f<NCT, 2>(st, fast, X, U, l16, q4);
}

// The output of the chunk, transposed: O^T = S^T Q^T + U^T Aqk^T. With the mirror-image
// operand layouts the packed state serves as the A operand of S^T and the Q^ row fragments
// as the B operand of Q^T, and likewise U and Aqk; the result's D layout gives lane
// (l16, q4) of OT[ct][I] token 16 I + l16 at channels col0 + 16 ct + 4 q4 .. + 3, which go
// out as one 8-byte store.
template <int MODE>   // MODE as for c_solve_f
__device__ __forceinline__ void c_output_f(const PcStage& st, const uint16_t* qw, const uint16_t* aqk, bool fast,
                                           const f32x4 (&S)[8][2], const f32x4 (&U)[4][2], f32x4 (&OT)[2][4], int l16,
                                           int q4) {
  const bool blocked = MODE == 0 ? !fast : MODE == 2;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int I = 0; I < 4; ++I) OT[ct][I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint4 xs[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) xs[ct] = pack8(S[2 * s][ct], S[2 * s + 1][ct]);
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      uint4 qf = ld128(qw, (SBT * I + l16) * RMS + 32 * s + 8 * q4);
      if (blocked) qf = scale8(qf, em_of(st, I, 32 * s + 4 * q4), em_of(st, I, 32 * s + 16 + 4 * q4));
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) OT[ct][I] = mma32(xs[ct], qf, OT[ct][I]);
    }
  }
  uint4 Uf[2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) Uf[s][ct] = pack8(U[2 * s][ct], U[2 * s + 1][ct]);
  // Aqk rows 16 I + l16 at tokens 32 s + 4 q4 + 0..3 and 32 s + 16 + 4 q4 + 0..3 (blocks above
  // the diagonal read as zeros)
  auto qfrag = [&](int I, int s) {
    const int base = tr(32 * s + 4 * q4 + (l16 >> 2), SBT * I + 4 * (l16 & 3));
    return cat(ld_tr(&aqk[base]), ld_tr(&aqk[base + tr(16, 0)]));
  };
  const uint4 qa0 = qfrag(0, 0), qa1 = qfrag(1, 0), qa2 = qfrag(2, 0), qa3 = qfrag(2, 1), qa4 = qfrag(3, 0),
              qa5 = qfrag(3, 1);
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    OT[ct][0] = mma32(Uf[0][ct], qa0, OT[ct][0]);
    OT[ct][1] = mma32(Uf[0][ct], qa1, OT[ct][1]);
    OT[ct][2] = mma32(Uf[0][ct], qa2, OT[ct][2]);
    OT[ct][2] = mma32(Uf[1][ct], qa3, OT[ct][2]);
    OT[ct][3] = mma32(Uf[0][ct], qa4, OT[ct][3]);
    OT[ct][3] = mma32(Uf[1][ct], qa5, OT[ct][3]);
  }
}
template <bool SPLIT = false>
__device__ __forceinline__ void c_output(const PcStage& st, const uint16_t* qw, const uint16_t* aqk, bool fast,
                                         const f32x4 (&S)[8][2], const f32x4 (&U)[4][2], f32x4 (&OT)[2][4], int l16,
                                         int q4) {
  if (!SPLIT) c_output_f<0>(st, qw, aqk, fast, S, U, OT, l16, q4);
  else if (fast) c_output_f<1>(st, qw, aqk, fast, S, U, OT, l16, q4);
  else c_output_f<2>(st, qw, aqk, fast, S, U, OT, l16, q4);
}

// OT (one token per lane, 4 channels) rounded to bf16 -> the stage's kr, used as o staging:
// row 16 I + l16, channels col0 + 16 ct + 4 q4 .. + 3 in natural order (row stride RKS)
__device__ __forceinline__ void c_stage_o(uint16_t* ob, const f32x4 (&OT)[2][4], int col0, int l16, int q4) {
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int I = 0; I < 4; ++I)
      *reinterpret_cast<uint2*>(&ob[rk(SBT * I + l16, col0 + 16 * ct + 4 * q4)]) = pack4(OT[ct][I]);
}
// staged rows 16 cw .. 16 cw + 15 of chunk c -> o: each lane 16 bytes, a 16-lane group one whole
// 256-byte token row; rows past the chunk's n tokens fall outside the buffer bound and are dropped
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void c_store_rows(const ChunkArgs& a, const SeqView& sv, int64_t h, int64_t c,
                                             const uint16_t* ob, int cw, int lane) {
  const int64_t t0 = c * CT;
  const int n = (int)min<int64_t>(CT, sv.T - t0);
  const int so2 = (int)(a.H * a.dv) * 2;
  const auto ro = __builtin_amdgcn_make_buffer_rsrc((void*)(a.o + ((sv.row0 + t0) * a.H + h) * a.dv), 0, n * so2,
                                                    kRsrcW3);
  const int r0 = SBT * cw + (lane >> 4), cc8 = 8 * (lane & 15);
  const int oc = cc8 < a.dv ? 2 * cc8 : kOffOut;   // padded channels are not stored
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint4 u = ld128(ob, rk(r0 + 4 * j, cc8));
    __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{u.x, u.y, u.z, u.w}, ro, (r0 + 4 * j) * so2 + oc, 0, 0);
  }
}

// the gate of the chunk in the layout of OT: gx[ct][I] = 4 bf16 of token 16 I + l16, channels
// col0 + 16 ct + 4 q4 .. + 3
__device__ __forceinline__ void c_issue_gate(const ChunkArgs& a, const SeqView& sv, int64_t h, int64_t c, int col0,
                                             int lane, uint2 (&gx)[2][4]) {
  const int l16 = lane & 15, q4 = lane >> 4;
  const int64_t t0 = c * CT;
  const int n = (int)min<int64_t>(CT, sv.T - t0);
  const int sg2 = (int)a.gate_stride * 2;
  const auto rg = __builtin_amdgcn_make_buffer_rsrc((void*)(a.gate + (sv.row0 + t0) * a.gate_stride + h * D), 0,
                                                    n * sg2, kRsrcW3);
  const int go = l16 * sg2 + 2 * (col0 + 4 * q4);
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int I = 0; I < 4; ++I) gx[ct][I] = ld_buf64(rg, go + 32 * ct, SBT * I * sg2);
}

// ---- output pass ---------------------------------------------------------------------
// One block per (sequence, head, output segment) and CU: waves 0-3 produce, waves 4-7 consume
// (wave 4 + j owns state columns 32 j ..). Per tick t, producers work on chunk c_begin + t and
// consumers on the chunk before it:
//   phase 1  P: loads of c arrive; norms, block products      C: U = T diag(b) (V - K^ S)
//   phase 2  P: K^, K_, Q^ of c; loads of c + 1 issued         C: O^T = S^T Q^T + U^T Aqk^T
//   phase 3  P: A, Aqk of c, diagonal inverses (at, aqk)       C: S update; gated: norm, gate
// with one block barrier after each phase. at and aqk have one copy: consumers read them in
// phases 1 and 2 and producers overwrite them in phase 3; the other per-chunk arrays
// alternate between two stages. The two roles run separate loops with the same number of
// ticks and barriers, so that neither role's registers are held through the other's code.
//
// GATED adds the rest of Eq. 15 short of W_o to the output: o <- Sigmoid(gate) * o / sqrt(mean
// over the head's channels of o^2 + eps) * w. Each consumer wave sums its 32 channels' squares
// per token in phase 2 (rowss); phase 3 reads the four parts and writes o once.
template <bool GATED, bool CONV>
__global__ __launch_bounds__(kPcThreads) void kda_out_kernel(ChunkArgs a) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  PcLdsOut& L = *reinterpret_cast<PcLdsOut*>(lds_raw);
  ConvLds& CL = *reinterpret_cast<ConvLds*>(lds_raw + sizeof(PcLdsOut));   // CONV only

  const uint32_t lid = (a.xcd_ranges && a.grid % 8 == 0) ? xcd_contiguous_id(blockIdx.x, (uint32_t)a.grid)
                                                         : blockIdx.x;
  if (lid >= (uint32_t)a.nblk) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform
  const int cw = wave & 3, col0 = 32 * cw;
  const int l16 = lane & 15, q4 = lane >> 4;
  const SeqDesc& rd = a.run[run_of<0>(a, lid)];
  const int32_t local = (int32_t)lid - rd.out0;
  const int p = uni(local % rd.P);
  const int32_t bhl = uni(local / rd.P);
  const SeqView sv = seq_view(a, rd, bhl);
  const int64_t h = uni(bhl % (int32_t)a.H);
  const int64_t NC = (sv.T + CT - 1) / CT;
  const int64_t c_begin = (int64_t)p * a.Lo;
  const int64_t c_end = min<int64_t>(NC, c_begin + a.Lo);
  const int64_t nch = c_end - c_begin;

  // the Aqk blocks (0,1) and (2,3) above the diagonal are read as zeros (ordered before their
  // first read by the barriers of tick 0)
  for (int e = tid; e < 2 * SBT * SBT; e += kPcThreads) {
    const int I = (e >> 8) * 2, i = (e >> 4) & 15, j = e & 15;
    L.aqk[tr(SBT * (I + 1) + j, SBT * I + i)] = 0;
  }

  if (wave < 4) {
    // ---------------- producers ----------------
    // the next chunk's alpha and beta go out once phase 1 has used this chunk's, its k and q once
    // phase 2 has
    PLoad R;
    float4 al[8];
    bool fast = true;
    if (CONV) {   // the segment table, then the first chunk's tap table (both roles wait for each)
      for (int i = tid; i < a.conv_nseg; i += 256) CL.seg[i] = a.conv_seg[i];
      lds_barrier();
      if (nch > 0) conv_fill(a, sv.T, CL, c_begin, tid);
      lds_barrier();
    }
    if (nch > 0) {
      p_issue_a(a, sv, h, c_begin, wave, lane, R);
      if (CONV) p_conv_kq<true>(a, sv, CL, h, c_begin, wave, lane, R);
      else p_issue_kq<true>(a, sv, h, c_begin, wave, lane, R);
    }
    for (int64_t t = 0; t <= nch; ++t) {
      const int64_t cp = c_begin + t;
      PcStage& sp = L.st[cp & 1];
      if (t < nch) {
        p_phase1<true>(a, sp, L.rk, L.rq, R, (int)min<int64_t>(CT, sv.T - cp * CT), wave, lane, al);
        if (t + 1 < nch) {
          p_issue_a(a, sv, h, cp + 1, wave, lane, R);
          if (CONV) conv_fill(a, sv.T, CL, cp + 1, tid);   // read from phase 2 on
        }
      }
      lds_barrier();
      if (t < nch) {
        fast = p_phase2<true>(sp, L.qw[cp & 1], L.rk, L.rq, R, al, wave, lane);
        if (t + 1 < nch) {
          if (CONV) p_conv_kq<true>(a, sv, CL, h, cp + 1, wave, lane, R);
          else p_issue_kq<true>(a, sv, h, cp + 1, wave, lane, R);
        }
      }
      lds_barrier();
      if (t < nch) p_phase3_out(sp, L.qw[cp & 1], L.at, L.aqk, L.adiag, fast, wave, lane);
      lds_barrier();
    }
  } else {
    // ---------------- consumers ----------------
    f32x4 S[8][2];
    if (sv.P > 1) {   // the segment's start state, chained by the combine pass (tile-major)
      const float* src = sv.ws + (2 * sv.E + p) * D * D;
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) S[rt][ct] = load_tile4(src, cw, rt, ct, lane);
    } else {          // S0 ([dk][dv] row-major, zero-padded to D x D) or zero
      const float* src = a.S0 ? a.S0 + sv.sidx * a.dk * a.dv : nullptr;
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 16 * rt + 4 * q4 + r, col = col0 + 16 * ct + l16;
            S[rt][ct][r] = src != nullptr && row < a.dk && col < a.dv ? src[row * a.dv + col] : 0.f;
          }
    }
    float4 gw[2];   // gated: the norm gain of the lane's channels col0 + 16 ct + 4 q4 .. + 3
    if (GATED) {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        gw[ct] = a.norm_w != nullptr ? ldf4(a.norm_w + col0 + 16 * ct + 4 * q4) : make_float4(1.f, 1.f, 1.f, 1.f);
    }
    uint2 gx[2][4], vr[8];
    f32x4 U[4][2], OT[2][4];
    if (CONV) {   // (the producers' segment and first tap tables)
      lds_barrier();
      lds_barrier();
    }
    for (int64_t t = 0; t <= nch; ++t) {
      const int64_t cc = c_begin + t - 1;
      const PcStage& sc = L.st[cc & 1];
      // the stage's vote, read from LDS: made wave-uniform so that the factorisation choice stays a
      // branch (a value the compiler takes as divergent would run both paths)
      const bool cf = t > 0 && __builtin_amdgcn_readfirstlane(sc.fast) != 0;
      // ---- phase 1: gated, the previous chunk's staged rows go out; U of this chunk
      if (GATED && t > 1) c_store_rows(a, sv, h, cc - 1, L.st[(cc - 1) & 1].kr, cw, lane);
      if (t > 0) {
        if (GATED) c_issue_gate(a, sv, h, cc, col0, lane, gx);
        c_solve<2, 2, !GATED && !CONV>(sc, L.at, L.qw[(cc + 1) & 1], cf, S, col0, U, l16, q4);
      }
      if (t < nch) {   // staged in phase 3
        if (CONV) c_conv_v<16>(a, sv, CL, h, cc + 1, cw, lane, vr);
        else c_issue_v<16>(a, sv, h, cc + 1, cw, lane, vr);
      }
      lds_barrier();
      // ---- phase 2: the output
      if (t > 0) {
        c_output<!GATED && !CONV>(sc, L.qw[cc & 1], L.aqk, cf, S, U, OT, l16, q4);
        if (!GATED) {
          c_stage_o(L.st[cc & 1].kr, OT, col0, l16, q4);   // K^ of this chunk is used up
        } else {
          // this wave's part of each token's sum of squares: over the lane's 8 channels, then
          // over the four lane groups that hold the same token
#pragma unroll
          for (int I = 0; I < 4; ++I) {
            float v = 0.f;
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
              for (int r = 0; r < 4; ++r) v += OT[ct][I][r] * OT[ct][I][r];
            v = halve32(v, v);
            v = halve16(v, v);
            if (q4 == 0) L.rowss[(SBT * I + l16) * 4 + cw] = v;
          }
        }
      }
      lds_barrier();
      // ---- phase 3: the state update; the output rows go out (gated: normalised, staged)
      if (t > 0) {
        if (!GATED) c_store_rows(a, sv, h, cc, L.st[cc & 1].kr, cw, lane);
        c_update<2, !GATED && !CONV>(sc, cf, S, U, l16, q4);
        if (GATED) {
          auto sig = [](float g) { return __builtin_amdgcn_rcpf(1.f + __expf(-g)); };
#pragma unroll
          for (int I = 0; I < 4; ++I) {
            const float4 p4 = ldf4(&L.rowss[(SBT * I + l16) * 4]);
            const float rinv = __builtin_amdgcn_rsqf((p4.x + p4.y + p4.z + p4.w) * (1.f / D) + a.norm_eps);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
              const float4 g = unpack4(gx[ct][I]);
              const float4 w = gw[ct];
              OT[ct][I][0] *= rinv * w.x * sig(g.x);
              OT[ct][I][1] *= rinv * w.y * sig(g.y);
              OT[ct][I][2] *= rinv * w.z * sig(g.z);
              OT[ct][I][3] *= rinv * w.w * sig(g.w);
            }
          }
          c_stage_o(L.st[cc & 1].kr, OT, col0, l16, q4);   // stored in the next tick's phase 1
        }
      }
      // v of the next chunk into this chunk's qw (its Q^ was used in phase 2): read in the next
      // tick's phase 1, before the producers' Q^ of the chunk after goes there
      if (t < nch) c_stage_v<16>(L.qw[cc & 1], vr, cw, lane);
      lds_barrier();
    }
    if (GATED && nch > 0) c_store_rows(a, sv, h, c_end - 1, L.st[(c_end - 1) & 1].kr, cw, lane);
    if (a.S_final != nullptr && p == sv.P - 1)
      store_state(S, a.S_final + sv.sidx * a.dk * a.dv, a.dk, a.dv, col0, l16, q4);
  }
}

// ---- summary pass --------------------------------------------------------------------
// One block of 12 waves per (sequence, head, summary segment): waves 0-3 produce as in the output
// pass (no q); waves 4-11 consume, wave 4 + j holding columns 16 j .. 16 j + 15 both of the state
// S (from 0) and of the transition M (from I). Phase 1 solves for U of the S tile and updates it,
// phase 2 solves for U of the M tile, phase 3 updates M (the stage's kc and egn stay until the
// next tick) and stages the next chunk's v, so that each SIMD's two consumer waves interleave
// their chains with the producer's work. At the segment end S goes to the workspace tile-major and M, through
// LDS, as split bf16 A fragments.
constexpr int kPcSumThreads = 768;
template <bool CONV>
__global__ __launch_bounds__(kPcSumThreads) void kda_sum_kernel(ChunkArgs a) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  PcLdsSum& L = *reinterpret_cast<PcLdsSum*>(lds_raw);
  ConvLds& CL = *reinterpret_cast<ConvLds*>(lds_raw + sizeof(PcLdsSum));   // CONV only

  const uint32_t lid = (a.xcd_ranges && a.grid % 8 == 0) ? xcd_contiguous_id(blockIdx.x, (uint32_t)a.grid)
                                                         : blockIdx.x;
  if (lid >= (uint32_t)a.nblk) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform
  const int l16 = lane & 15, q4 = lane >> 4;
  const SeqDesc& rd = a.run[run_of<1>(a, lid)];
  const int32_t local = (int32_t)lid - rd.sum0;
  const int p = uni(local % rd.Ps);
  const int32_t bhl = uni(local / rd.Ps);
  const SeqView sv = seq_view(a, rd, bhl);
  const int64_t h = uni(bhl % (int32_t)a.H);
  const int64_t NC = (sv.T + CT - 1) / CT;
  const int64_t c_begin = (int64_t)p * a.Lo;
  const int64_t c_end = min<int64_t>(NC, c_begin + a.Lo);   // summary segments are output segments 0 .. P - 2
  const int64_t nch = c_end - c_begin;
  // M staging for the fragment store at the end: bf16 high and low parts, [D][D + 8] each
  constexpr int kMP = D + 8;
  uint16_t* mhi = reinterpret_cast<uint16_t*>(lds_raw);
  uint16_t* mlo = mhi + D * kMP;
  static_assert(2 * D * kMP * sizeof(uint16_t) <= sizeof(PcLdsSum), "M staging fits the summary LDS");

  if (wave < 4) {
    // ---------------- producers ----------------
    PLoad R;   // loads issued as in the output pass
    float4 al[8];
    bool fast = true;
    if (CONV) {   // the segment table, then the first chunk's tap table (both roles wait for each)
      for (int i = tid; i < a.conv_nseg; i += 256) CL.seg[i] = a.conv_seg[i];
      lds_barrier();
      if (nch > 0) conv_fill(a, sv.T, CL, c_begin, tid);
      lds_barrier();
    }
    if (nch > 0) {
      p_issue_a(a, sv, h, c_begin, wave, lane, R);
      if (CONV) p_conv_kq<false>(a, sv, CL, h, c_begin, wave, lane, R);
      else p_issue_kq<false>(a, sv, h, c_begin, wave, lane, R);
    }
    for (int64_t t = 0; t <= nch; ++t) {
      const int64_t cp = c_begin + t;
      PcStage& sp = L.st[cp & 1];
      if (t < nch) {
        p_phase1<false>(a, sp, L.rk, L.rq, R, (int)min<int64_t>(CT, sv.T - cp * CT), wave, lane, al);
        if (t + 1 < nch) {
          p_issue_a(a, sv, h, cp + 1, wave, lane, R);
          if (CONV) conv_fill(a, sv.T, CL, cp + 1, tid);   // read from phase 2 on
        }
      }
      lds_barrier();
      if (t < nch) {
        fast = p_phase2<false>(sp, nullptr, L.rk, L.rq, R, al, wave, lane);
        if (t + 1 < nch) {
          if (CONV) p_conv_kq<false>(a, sv, CL, h, cp + 1, wave, lane, R);
          else p_issue_kq<false>(a, sv, h, cp + 1, wave, lane, R);
        }
      }
      lds_barrier();
      if (t < nch) p_phase3_sum(sp, L.at, L.adiag, fast, wave, lane);
      lds_barrier();
    }
    lds_barrier();   // (the consumers' M staging below)
    lds_barrier();
  } else {
    // ---------------- consumers ----------------
    const int j = wave - 4, col0 = 16 * j;
    // X[rt][0]: the state S (from 0), X[rt][1]: the transition M (from I), both columns 16 j ..
    f32x4 X[8][2];
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        X[rt][0][r] = 0.f;
        X[rt][1][r] = 16 * rt + 4 * q4 + r == col0 + l16 ? 1.f : 0.f;
      }
    uint2 vr[4];
    f32x4 U[4][2];
    if (CONV) {   // (the producers' segment and first tap tables)
      lds_barrier();
      lds_barrier();
    }
    for (int64_t t = 0; t <= nch; ++t) {
      const int64_t cc = c_begin + t - 1;
      const PcStage& sc = L.st[cc & 1];
      // the stage's vote, read from LDS: made wave-uniform so that the factorisation choice stays a
      // branch (a value the compiler takes as divergent would run both paths)
      const bool cf = t > 0 && __builtin_amdgcn_readfirstlane(sc.fast) != 0;
      // phase 1 (the producers' lightest): U of the S and M tiles in one pass over K^ and T
      if (t > 0) c_solve<2, 1>(sc, L.at, L.vs, cf, X, col0, U, l16, q4);
      lds_barrier();
      // phase 2: v of the next chunk into vs (read in the next tick's phase 1; this tick's reads are done)
      if (t < nch) {
        if (CONV) c_conv_v<8>(a, sv, CL, h, cc + 1, j, lane, vr);
        else c_issue_v<8>(a, sv, h, cc + 1, j, lane, vr);
        c_stage_v<8>(L.vs, vr, j, lane);
      }
      lds_barrier();
      // phase 3 (the producers' heaviest): both updates (kc and egn of the stage stay until the next tick)
      if (t > 0) c_update<2>(sc, cf, X, U, l16, q4);
      lds_barrier();
    }
    lds_barrier();   // every wave is past its last LDS read: the LDS is scratch now
    if (nch > 0) {
      // S: the tile (rows, columns 16 j ..) goes out tile-major
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
        *reinterpret_cast<f32x4*>(sv.ws + p * D * D + tile_off(j >> 1, rt, j & 1, lane)) = X[rt][0];
      // M: split into bf16 high and low parts, staged row-major
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = X[rt][1][r];
          const uint16_t hb = f2bf(x);
          const int o = (16 * rt + 4 * q4 + r) * kMP + col0 + l16;
          mhi[o] = hb;
          mlo[o] = f2bf(x - bf2f(hb));
        }
    }
    lds_barrier();
    if (nch > 0) {
      // M as A fragments: wave j forms row tile j of every k slot (row 16 j + l16, columns
      // 32 s + 4 q4 .. + 3 and 32 s + 16 + 4 q4 .. + 3, the high part then the low part)
      uint4* m = reinterpret_cast<uint4*>(sv.ws + (sv.E + p) * D * D);
      const int row = (SBT * j + l16) * kMP;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int c0 = 32 * s4 + 4 * q4;
        const uint2 h0 = *reinterpret_cast<const uint2*>(&mhi[row + c0]);
        const uint2 h1 = *reinterpret_cast<const uint2*>(&mhi[row + c0 + 16]);
        const uint2 l0 = *reinterpret_cast<const uint2*>(&mlo[row + c0]);
        const uint2 l1 = *reinterpret_cast<const uint2*>(&mlo[row + c0 + 16]);
        m[mfrag_off(j, s4, lane)] = cat(h0, h1);
        m[mfrag_off(j, s4, lane) + 1] = cat(l0, l1);
      }
    }
  }
}

// The chain of segment starts, S_start(0) = S0 (or 0) and
//   S_start(kSub (j + 1)) = M_e S_start(kSub j) + S_e,  e = kSub j + kSub - 1,
// the transition and zero-start state of summary segment j over its full length.
// (Starts inside a summary segment are formed by the output pass itself.)
// Column-parallel: block (bh, slice) owns state columns 16 slice .. 16 slice + 15;
// wave w owns rows 16 w .. 16 w + 15 of them in fp32. The base of each step is
// exchanged through LDS split into bf16 high and low parts; products are three
// bf16 MFMAs (hi*hi + hi*lo + lo*hi) with fp32 accumulation, about 16
// significant bits per product. Rows of M for the next kAhead steps are in
// flight while a step computes.
constexpr int CB_T = 512;       // 8 waves
constexpr int BTS = D + 8;      // padded row of the transposed base state
constexpr int kAhead = 3;


__global__ __launch_bounds__(CB_T) void kda_combine_kernel(ChunkArgs a) {
  __shared__ __align__(16) uint16_t bhi[2][16 * BTS];   // [column][cpos(row)], double-buffered
  __shared__ __align__(16) uint16_t blo[2][16 * BTS];
  const uint32_t lid = blockIdx.x;
  if (lid >= (uint32_t)a.nblk) return;
  const SeqDesc& rd = a.run[run_of<2>(a, lid)];
  const int32_t local = (int32_t)lid - rd.comb0;
  const int slice = local % 8;
  const SeqView sv = seq_view(a, rd, local / 8);
  const int P = sv.P;
  const float* WS = sv.ws;                  // [E] summary states
  const float* WM = sv.ws + sv.E * D * D;   // [E] transitions
  float* Sst = sv.ws + 2 * sv.E * D * D;    // [P] start states
  const float* S0 = a.S0 ? a.S0 + sv.sidx * a.dk * a.dv : nullptr;   // [dk][dv], zero-padded to D x D
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, q4 = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = 16 * slice + l16;
  const int row0 = 16 * wave + 4 * q4;       // D-layout rows of this lane: row0 .. row0 + 3

  f32x4 cur;
#pragma unroll
  for (int r = 0; r < 4; ++r) cur[r] = S0 != nullptr && row0 + r < a.dk && col < a.dv ? S0[(row0 + r) * a.dv + col] : 0.f;
  auto store = [&](int po, const f32x4& v) {   // tile-major
    *reinterpret_cast<f32x4*>(Sst + po * D * D + tile_off(slice >> 1, wave, slice & 1, lane)) = v;
  };
  store(0, cur);
  const int nsteps = (P - 1) / kSub;   // chain starts kSub, 2 kSub, .. below P
  // A fragments of M_e for this wave's rows (split bf16, slot s: high 2 s, low 2 s + 1)
  uint4 mq[kAhead][8];
  f32x4 sq[kAhead];
  auto fetch = [&](int step, uint4(&m)[8], f32x4& s_e) {
    if (step < nsteps) {
      const int e = step * kSub + kSub - 1;
      const uint4* mp = reinterpret_cast<const uint4*>(WM + e * D * D);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        m[2 * s] = mp[mfrag_off(wave, s, lane)];
        m[2 * s + 1] = mp[mfrag_off(wave, s, lane) + 1];
      }
      s_e = load_tile4(WS + e * D * D, slice >> 1, wave, slice & 1, lane);
    }
  };
#pragma unroll
  for (int j = 0; j < kAhead; ++j) fetch(j, mq[j], sq[j]);
  // one step of the chain with the operands in slot j; the slot is refilled for the step
  // kAhead later. The loop is unrolled by kAhead so that the slots stay in place: moving a
  // register that a load still targets would wait for that load.
  auto chain_step = [&](int step, int j) {
    const int buf = step & 1;
    {   // base rows row0 .. row0 + 3 of column l16 -> LDS, transposed, split
      uint2 lo;
      const uint2 hi = pack_split(make_float4(cur[0], cur[1], cur[2], cur[3]), lo);
      const int pos = cpos(row0);
      *reinterpret_cast<uint2*>(&bhi[buf][l16 * BTS + pos]) = hi;
      *reinterpret_cast<uint2*>(&blo[buf][l16 * BTS + pos]) = lo;
    }
    lds_barrier();
    uint4 bH[4], bL[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bH[s] = *reinterpret_cast<const uint4*>(&bhi[buf][l16 * BTS + 32 * s + 8 * q4]);
      bL[s] = *reinterpret_cast<const uint4*>(&blo[buf][l16 * BTS + 32 * s + 8 * q4]);
    }
    f32x4 acc0 = sq[j], acc1 = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 ah = mq[j][2 * s], al = mq[j][2 * s + 1];
      acc1 = mma32(al, bH[s], acc1);
      acc2 = mma32(ah, bL[s], acc2);
      acc0 = mma32(ah, bH[s], acc0);
    }
    cur = acc0 + (acc1 + acc2);
    store(kSub * (step + 1), cur);
    fetch(step + kAhead, mq[j], sq[j]);
  };
  for (int step = 0; step < nsteps; step += kAhead) {
#pragma unroll
    for (int j = 0; j < kAhead; ++j)
      if (step + j < nsteps) chain_step(step + j, j);
  }
}

// Host-side plan of a launch: one chunks-per-segment value Lo for all runs (so that no block
// has more than Lo chunks), then per run its segment counts and workspace region, and the runs
// in the order their blocks are handed out (longest blocks first).
struct Plan {
  int Lo = 1;
  std::vector<SeqDesc> desc;   // per run; the first-block fields are filled per launch set
  int64_t ws_mats = 0;         // workspace matrices (D x D fp32)
};

// Estimated time of the two passes for a segment length Lo, in chunk steps of an output block
// (one per CU, about kTargetBlocks at once): the longest block or the total work spread over
// the chip, whichever is larger; a summary block (also one per CU) moves about 0.6 of an output
// block's bytes per chunk and covers up to kSub * Lo chunks. For a batch of equal sequences the
// smallest Lo that gives about kTargetBlocks output blocks is always best; for packed samples
// of mixed lengths a shorter Lo can spread the few long samples' summaries over more blocks.
double plan_cost(const KdaRun* runs, int64_t nruns, int64_t H, int64_t Lo) {
  double w_out = 0, w_sum = 0, max_out = 0, max_sum = 0;
  for (int64_t r = 0; r < nruns; ++r) {
    const int64_t NC = (runs[r].len + CT - 1) / CT;
    const int64_t P = NC <= 1 ? 1 : (NC + Lo - 1) / Lo;
    w_out += (double)runs[r].count * H * NC;
    max_out = std::max(max_out, (double)std::min(NC, Lo));
    if (P > 1) {
      w_sum += (double)runs[r].count * H * (P - 1) * Lo;
      max_sum = std::max(max_sum, (double)std::min((P - 1) * Lo, (int64_t)kSub * Lo));
    }
  }
  return std::max(max_out, w_out / kTargetBlocks) + 0.6 * std::max(max_sum, w_sum / kTargetBlocks);
}

Plan make_plan(const KdaRun* runs, int64_t nruns, int64_t H, bool no_split) {
  Plan pl;
  int64_t chunks = 0;
  for (int64_t r = 0; r < nruns; ++r) chunks += runs[r].count * ((runs[r].len + CT - 1) / CT);
  const int64_t work = H * chunks;
  int64_t Lo = no_split ? (int64_t(1) << 30) : (work + kTargetBlocks - 1) / kTargetBlocks;
  if (Lo < 1) Lo = 1;
  if (Lo > (int64_t(1) << 30)) Lo = int64_t(1) << 30;
  if (!no_split && nruns > 1) {   // mixed lengths: a shorter segment if it is clearly cheaper
    const int64_t L0 = Lo;
    double best = plan_cost(runs, nruns, H, L0);
    for (const int div : {2, 3, 4, 6, 8}) {
      const int64_t cand = std::max<int64_t>(1, (L0 + div - 1) / div);
      const double c = plan_cost(runs, nruns, H, cand);
      if (c < 0.97 * best) {
        best = c;
        Lo = cand;
      }
    }
  }
  pl.Lo = (int)Lo;
  // longest blocks first: the run order is only the order in which blocks are handed out
  std::vector<int64_t> order((size_t)nruns);
  for (int64_t r = 0; r < nruns; ++r) order[(size_t)r] = r;
  auto longest = [&](int64_t r) { return std::min((runs[r].len + CT - 1) / CT, Lo); };
  std::stable_sort(order.begin(), order.end(), [&](int64_t x, int64_t y) { return longest(x) > longest(y); });
  pl.desc.resize((size_t)nruns);
  for (int64_t i = 0; i < nruns; ++i) {
    const KdaRun& run = runs[order[(size_t)i]];
    const int64_t NC = (run.len + CT - 1) / CT;
    const int64_t P = NC <= 1 ? 1 : (NC + Lo - 1) / Lo;
    const int64_t Ps = P > 1 ? (P - 1 + kSub - 1) / kSub : 0;   // summaries up to the last needed boundary
    SeqDesc& d = pl.desc[(size_t)i];
    d.start = run.start;
    d.len = run.len;
    d.ws0 = pl.ws_mats;
    d.count = (int32_t)run.count;
    d.sidx0 = (int32_t)run.sidx0;
    d.P = (int32_t)P;
    d.Ps = (int32_t)Ps;
    d.out0 = d.sum0 = d.comb0 = d.pad = 0;
    if (P > 1) pl.ws_mats += run.count * H * (2 * kSub * Ps + P);
  }
  return pl;
}

// blocks of each pass for the runs [r0, r1) of a plan
struct SetBlocks {
  int64_t out = 0, sum = 0, comb = 0;
};
SetBlocks set_blocks(const Plan& pl, size_t r0, size_t r1, int64_t H) {
  SetBlocks b;
  for (size_t r = r0; r < r1; ++r) {
    const SeqDesc& d = pl.desc[r];
    b.out += (int64_t)d.count * H * d.P;
    b.sum += (int64_t)d.count * H * d.Ps;
    if (d.P > 1) b.comb += (int64_t)d.count * H * 8;
  }
  return b;
}

// The fused conv's weights transposed to wT [31][C] (the text taps, then the visual taps; a
// missing weight array reads as zeros) and the segment table, into the workspace.
__global__ __launch_bounds__(256) void conv_prep_kernel(ConvSrc cs, float* wT, Seg* seg) {
  const int64_t n = (int64_t)kConvSlots * cs.C;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int slot = (int)(e / cs.C);
    const int64_t c = e - slot * cs.C;
    wT[e] = slot < kTextTaps ? (cs.w_text != nullptr ? cs.w_text[c * kTextTaps + slot] : 0.f)
                             : (cs.w_vis != nullptr ? cs.w_vis[c * kVisTaps + slot - kTextTaps] : 0.f);
  }
  if (blockIdx.x == 0 && (int)threadIdx.x < cs.nseg) seg[threadIdx.x] = cs.seg[threadIdx.x];
}

// how far back any tap of the layout reaches (tokens)
int64_t conv_reach_back(const ConvSrc& cs) {
  int64_t back = 0;
  for (int i = 0; i < cs.nseg; ++i) {
    const Seg& g = cs.seg[i];
    const int64_t b = g.kind == SEG_TEXT ? kTextTaps - 1
                                         : std::min<int64_t>(std::max(g.frames - 1, 0), 2) * g.height * g.width +
                                               g.width + 1;
    back = std::max(back, b);
  }
  return back;
}
size_t conv_wT_bytes(int64_t C) { return ((size_t)kConvSlots * C * sizeof(float) + 255) / 256 * 256; }

}  // namespace

bool kda_chunked_conv_supported(const KdaArgs& a) {
  if (a.conv == nullptr || !a.bf16 || a.dk != D || a.dv != D) return false;
  const ConvSrc& cs = *a.conv;
  if (cs.C != a.H * 3 * D || cs.nseg < 1 || cs.nseg > kMaxFusedSegs) return false;
  if ((reinterpret_cast<uintptr_t>(cs.x) & 7) != 0) return false;
  // every offset into a chunk's window stays below the padding offset
  const int64_t back = conv_reach_back(cs);
  return (double)(CT + 1 + 2 * back) * (double)cs.C * 2.0 < (double)kOffPad;
}

bool kda_chunked_supported(const KdaArgs& a) {
  // 8-byte loads of q, k and alpha: token stride a multiple of 4 elements, 8-byte aligned bases
  const uintptr_t al = reinterpret_cast<uintptr_t>(a.q) | reinterpret_cast<uintptr_t>(a.k) |
                       reinterpret_cast<uintptr_t>(a.alpha);
  // head sizes up to D in steps of 8: the kernels run at D with the extra channels zero (k, q, v)
  // or one (alpha), and store only the real ones
  return a.bf16 && a.dk >= 8 && a.dk <= D && a.dk % 8 == 0 && a.dv >= 8 && a.dv <= D && a.dv % 8 == 0 &&
         a.qkv_stride % 4 == 0 && a.qkv_stride <= (int64_t(1) << 24) && (al & 7) == 0;
}

bool kda_chunked_plan_ok(const KdaRun* runs, int64_t nruns, int64_t H, bool no_split) {
  const Plan pl = make_plan(runs, nruns, H, no_split);
  for (size_t r0 = 0; r0 < pl.desc.size(); r0 += kMaxRuns) {
    const SetBlocks b = set_blocks(pl, r0, std::min(pl.desc.size(), r0 + (size_t)kMaxRuns), H);
    if (b.out > 0x7fffff00 || b.sum > 0x7fffff00 || b.comb > 0x7fffff00) return false;
  }
  return true;
}

size_t kda_chunked_workspace(const KdaRun* runs, int64_t nruns, int64_t H, bool no_split, const ConvSrc* conv) {
  const size_t states = (size_t)make_plan(runs, nruns, H, no_split).ws_mats * D * D * sizeof(float);
  return conv == nullptr ? states : states + conv_wT_bytes(conv->C) + (size_t)conv->nseg * sizeof(Seg);
}

hipError_t launch_kda_chunked(const KdaArgs& x, const KdaRun* runs, int64_t nruns, bool no_split, void* workspace,
                              hipStream_t stream, Marks* marks) {
  const Plan pl = make_plan(runs, nruns, x.H, no_split);
  ChunkArgs a;
  a.q = static_cast<const uint16_t*>(x.q);
  a.k = static_cast<const uint16_t*>(x.k);
  a.v = static_cast<const uint16_t*>(x.v);
  a.stride = x.qkv_stride;
  a.alpha = static_cast<const uint16_t*>(x.alpha);
  a.beta = static_cast<const uint16_t*>(x.beta);
  a.S0 = x.S0;
  a.ws = static_cast<float*>(workspace);
  a.o = static_cast<uint16_t*>(x.o);
  a.S_final = x.S_final;
  // the gate is fused into the output pass when its rows and the gain are read as 16-byte
  // pieces; otherwise the separate in-place gate/norm pass runs after it
  const bool gated = x.gate != nullptr;
  const bool fuse_gate = gated && x.dv == D && x.gate_stride % 8 == 0 && (reinterpret_cast<uintptr_t>(x.gate) & 15) == 0 &&
                         (reinterpret_cast<uintptr_t>(x.norm_w) & 15) == 0 && x.gate_stride <= (int64_t(1) << 24);
  a.gate = static_cast<const uint16_t*>(x.gate);
  a.gate_stride = x.gate_stride;
  a.norm_w = x.norm_w;
  a.norm_eps = x.norm_eps;
  a.H = x.H;
  a.dk = (int)x.dk;
  a.dv = (int)x.dv;
  a.Lo = pl.Lo;
  a.l2norm = x.l2norm ? 1 : 0;
  a.xcd_ranges = pl.desc.size() == 1 ? 1 : 0;   // blocks of unequal length: the hardware's round robin
  const bool conv = x.conv != nullptr;
  a.x = nullptr;
  a.xC = 0;
  a.wT = nullptr;
  a.conv_seg = nullptr;
  a.conv_back = 0;
  a.conv_nseg = 0;
  if (conv) {
    if (!kda_chunked_conv_supported(x) || nruns != 1) return hipErrorInvalidValue;
    float* wT = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.ws_mats * D * D * sizeof(float));
    Seg* segs = reinterpret_cast<Seg*>(reinterpret_cast<char*>(wT) + conv_wT_bytes(x.conv->C));
    const int64_t n = (int64_t)kConvSlots * x.conv->C;
    const unsigned blocks = (unsigned)std::min<int64_t>((n + 255) / 256, 1024);
    hipLaunchKernelGGL(conv_prep_kernel, dim3(blocks), dim3(256), 0, stream, *x.conv, wT, segs);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = mark_after(marks, "conv_prep_kernel", stream);
    if (e != hipSuccess) return e;
    a.x = static_cast<const uint16_t*>(x.conv->x);
    a.xC = x.conv->C;
    a.wT = wT;
    a.conv_seg = segs;
    a.conv_back = conv_reach_back(*x.conv);
    a.conv_nseg = x.conv->nseg;
  }
  const size_t lds = sizeof(PcLdsOut) + (conv ? sizeof(ConvLds) : 0);
  const size_t lds_sum = sizeof(PcLdsSum) + (conv ? sizeof(ConvLds) : 0);
  int dev = 0;
  hipError_t de = hipGetDevice(&dev);
  if (de != hipSuccess) return de;
  // The LDS attribute is set once per device; the flag is atomic so that host threads calling
  // at once on one device race on nothing (setting it twice is harmless).
  static std::atomic<bool> attr_done[64];
  if (dev < 0 || dev >= 64 || !attr_done[dev].load(std::memory_order_acquire)) {
    const int lo = (int)sizeof(PcLdsOut), ls = (int)sizeof(PcLdsSum), lc = (int)sizeof(ConvLds);
    const std::pair<const void*, int> fns[] = {
        {reinterpret_cast<const void*>(&kda_out_kernel<false, false>), lo},
        {reinterpret_cast<const void*>(&kda_out_kernel<true, false>), lo},
        {reinterpret_cast<const void*>(&kda_out_kernel<false, true>), lo + lc},
        {reinterpret_cast<const void*>(&kda_sum_kernel<false>), ls},
        {reinterpret_cast<const void*>(&kda_sum_kernel<true>), ls + lc}};
    for (const auto& f : fns) {
      const hipError_t e = hipFuncSetAttribute(f.first, hipFuncAttributeMaxDynamicSharedMemorySize, f.second);
      if (e != hipSuccess) return e;
    }
    if (dev >= 0 && dev < 64) attr_done[dev].store(true, std::memory_order_release);
  }
  auto round8 = [](int64_t n) { return (int)((n + 7) / 8 * 8); };
  // runs go to the kernels kMaxRuns at a time (the table travels in the kernel arguments)
  for (size_t r0 = 0; r0 < pl.desc.size(); r0 += kMaxRuns) {
    const size_t r1 = std::min(pl.desc.size(), r0 + (size_t)kMaxRuns);
    a.nruns = (int)(r1 - r0);
    int64_t out0 = 0, sum0 = 0, comb0 = 0;
    for (size_t r = r0; r < r1; ++r) {
      SeqDesc d = pl.desc[r];
      d.out0 = (int32_t)out0;
      d.sum0 = (int32_t)sum0;
      d.comb0 = (int32_t)comb0;
      a.run[r - r0] = d;
      out0 += (int64_t)d.count * x.H * d.P;
      sum0 += (int64_t)d.count * x.H * d.Ps;
      if (d.P > 1) comb0 += (int64_t)d.count * x.H * 8;
    }
    if (out0 > 0x7fffff00 || sum0 > 0x7fffff00 || comb0 > 0x7fffff00) return hipErrorInvalidValue;
    if (sum0 > 0) {
      ChunkArgs s = a;
      s.nblk = (int)sum0;
      s.grid = round8(sum0);
      if (conv) hipLaunchKernelGGL(kda_sum_kernel<true>, dim3((unsigned)s.grid), dim3(kPcSumThreads), lds_sum, stream, s);
      else hipLaunchKernelGGL(kda_sum_kernel<false>, dim3((unsigned)s.grid), dim3(kPcSumThreads), lds_sum, stream, s);
      hipError_t e = hipGetLastError();
      if (e == hipSuccess) e = mark_after(marks, conv ? "kda_sum_conv_kernel" : "kda_sum_kernel", stream);
      if (e != hipSuccess) return e;
      s.nblk = (int)comb0;
      s.grid = (int)comb0;
      hipLaunchKernelGGL(kda_combine_kernel, dim3((unsigned)comb0), dim3(CB_T), 0, stream, s);
      e = hipGetLastError();
      if (e == hipSuccess) e = mark_after(marks, "kda_combine_kernel", stream);
      if (e != hipSuccess) return e;
    }
    if (out0 == 0) continue;
    a.nblk = (int)out0;
    a.grid = round8(out0);
    if (conv)
      hipLaunchKernelGGL((kda_out_kernel<false, true>), dim3((unsigned)a.grid), dim3(kPcThreads), lds, stream, a);
    else if (fuse_gate)
      hipLaunchKernelGGL((kda_out_kernel<true, false>), dim3((unsigned)a.grid), dim3(kPcThreads), lds, stream, a);
    else
      hipLaunchKernelGGL((kda_out_kernel<false, false>), dim3((unsigned)a.grid), dim3(kPcThreads), lds, stream, a);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess)
      e = mark_after(marks, conv ? "kda_out_conv_kernel" : fuse_gate ? "kda_out_gated_kernel" : "kda_out_kernel", stream);
    if (e != hipSuccess) return e;
  }
  return gated && !fuse_gate ? launch_kda_gate_norm(x, stream, marks) : hipSuccess;
}

}  // namespace chm
