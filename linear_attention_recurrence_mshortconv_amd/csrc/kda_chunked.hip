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
//   (I + A) U = diag(b) V - diag(b) (K e^g) S,  A_ri = b_r sum_c k_rc k_ic e^{g_rc - g_ic}  (i < r)
//   O = (Q e^g) S + Aqk U,                      Aqk_ri = sum_c q_rc k_ic e^{g_rc - g_ic}  (i <= r)
//   S_next = Diag(e^{g_n}) S + (K e^{g_n - g})^T U
//
// so with T = (I + A)^{-1}, W = T diag(b) K e^g and U~ = T diag(b) V, the chunk
// step is U = U~ - W S. Decays are running products of alpha (no log / exp).
// The per-(token, head) L2 normalisation of q and k (page 1, Fig. 2) enters as
// row / column scalings of A, Aqk, W, U and O rather than through the operands.
//
// Work layout. A block of 4 waves runs one segment of chunks of one (batch,
// head); wave w owns state columns 32w..32w+31 in registers, and under 80 KB of
// LDS lets two blocks share a CU. Operands live in LDS once, row-major
// [token][channel]; products that contract over tokens read them with the
// gfx950 transposing LDS read (ds_read_b64_tr_b16) instead of keeping
// transposed copies. Channels are stored in a permuted order inside each group
// of 32 (cpos) so that one 16-byte read returns the K order of a state fragment
// packed from the MFMA D layout.
//
// The sequence is cut into segments so that the chip has enough blocks:
//   summary pass: per summary segment, one block runs S from 0 and one runs the
//                 transition M from I (a summary segment spans kSub output
//                 segments; the state at each output-segment boundary is kept);
//   combine pass: S_start(e + 1) = M_e S_start(base) + S_e, fp32-accurate MFMA;
//   output pass:  each output segment reruns from S_start(p), writing o.
// With one output segment only the output pass runs, starting from S0.
#include "dtypes.h"
#include "internal.h"

namespace chm {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int D = 128;      // dk = dv
constexpr int CT = 64;      // tokens per chunk
constexpr int SBT = 16;     // tokens per decay block
constexpr int NSB = CT / SBT;
constexpr int NTHR = 256;   // 4 waves
constexpr int kTargetBlocks = 512;   // two blocks per CU
constexpr int kSub = 2;              // output segments per summary segment
constexpr float kL2Eps = 1e-6f;
constexpr float kFastMin = 1.8e-35f; // ~e^{-80}: the chunk-start factorisation is safe above this

__device__ __forceinline__ f32x4 mma32(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(uint2 a, uint2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b), c,
                                                   0, 0, 0);
}
__device__ __forceinline__ uint2 pack4(const f32x4& v) {
  return make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}
__device__ __forceinline__ uint2 pack4(const float4& v) {
  return make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
}
__device__ __forceinline__ uint4 pack8(const f32x4& lo, const f32x4& hi) {
  return make_uint4(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[0], hi[1]),
                    pack_bf16x2(hi[2], hi[3]));
}
__device__ __forceinline__ uint4 cat(uint2 a, uint2 b) { return make_uint4(a.x, a.y, b.x, b.y); }
__device__ __forceinline__ float4 unpack4(uint2 u) {
  return make_float4(bf_lo(u.x), bf_hi(u.x), bf_lo(u.y), bf_hi(u.y));
}
__device__ __forceinline__ float4 mul4(float4 a, float4 b) {
  return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w);
}
__device__ __forceinline__ float4 rcp4(float4 a) {
  return make_float4(__builtin_amdgcn_rcpf(a.x), __builtin_amdgcn_rcpf(a.y), __builtin_amdgcn_rcpf(a.z),
                     __builtin_amdgcn_rcpf(a.w));
}
__device__ __forceinline__ float dot4(uint2 u) {
  const float4 f = unpack4(u);
  return f.x * f.x + f.y * f.y + f.z * f.z + f.w * f.w;
}
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
//   rm: [CT][D] row-major, row stride D + 8 elements (272 bytes)
//   tr: [CT][CT], row stride CT + 8 elements (144 bytes: 16-byte reads stay aligned)
constexpr int RMS = D + 8;
constexpr int TRS = CT + 8;
__device__ __forceinline__ constexpr int rm(int row, int col) { return row * RMS + col; }
__device__ __forceinline__ constexpr int tr(int row, int col) { return row * TRS + col; }
// Position of channel (or token) c inside its row: within each group of 32 the
// order is 0-3, 16-19, 4-7, 20-23, 8-11, 24-27, 12-15, 28-31.
__device__ __forceinline__ constexpr int cpos(int c) {
  return (c & ~31) | ((c & 12) << 1) | ((c & 16) >> 2) | (c & 3);
}

// Small arrays first: LDS instruction offsets reach 64 KB from a base register.
struct Lds {
  float beta[CT];
  float rk[CT];           // 1/|k_t| (1 without normalisation)
  float rq[CT];
  float egn[D];           // e^{g_n}
  float pb[NSB][D];       // per block and channel: product of alpha over block tokens 0..8
  float pf[NSB][D];       //                        ... over block tokens 9..15
  float adiag[NSB][SBT][20];   // strictly lower A_II in fp32, column k at 4*(k&3) + (k>>2)
  uint16_t at[CT * TRS];  // -A in the blocks below the diagonal, T_II on it (natural order)
  uint16_t aqk[CT * TRS]; // Aqk (rows scaled 1/|q|, columns 1/|k|), token columns at cpos
  uint16_t kr[CT * RMS];  // K^ = k e^{g} (fast) or k e^{g - m_I} (blocked); output staging at the end
  uint16_t kc[CT * RMS];  // K_ = k e^{-g} (fast) or k e^{m_I - g} (blocked)
  uint16_t qw[CT * RMS];  // Q^ = q e^{g} / q e^{g - m_I} (output pass); then -W
};
static_assert(sizeof(Lds) <= 81920, "two blocks per CU");

struct ChunkArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t stride;
  const uint16_t* alpha;
  const uint16_t* beta;
  const float* S0;        // output pass without split: [BH][D][D] or null
  const float* Sstart;    // output pass with split: [BH][P][D][D]
  float* WS;              // summary: S at output-segment boundaries [BH][E][D][D]
  float* WM;              // summary: transitions to those boundaries [BH][E][D][D]
  uint16_t* o;
  float* S_final;
  int64_t T;
  int64_t H;
  int64_t c_stop;         // summary: chunks from here on are not needed
  int P;                  // segments per (batch, head)
  int L;                  // chunks per segment
  int Lo;                 // chunks per output segment
  int E;                  // entries per (batch, head) in WS / WM
  int nblk;               // logical blocks
  int grid;               // launched blocks
  int l2norm;
};

// Register-level lane exchanges.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_xor1(float v) { return dpp_f<0xB1>(v); }              // quad_perm 1,0,3,2
__device__ __forceinline__ float lane_xor2(float v) { return dpp_f<0x4E>(v); }              // quad_perm 2,3,0,1
__device__ __forceinline__ float lane_xor4(float v) { return dpp_f<0x1B>(dpp_f<0x141>(v)); } // half mirror, quad reverse
__device__ __forceinline__ float lane_xor8(float v) { return dpp_f<0x128>(v); }             // row_ror 8
// lanes < 32 get lo + (lane + 32)'s lo, lanes >= 32 get (lane - 32)'s hi + hi
__device__ __forceinline__ float halve32(float lo, float hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(lo), __float_as_int(hi), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}
// the same across 16-lane rows: lanes with bit 4 clear get lo + lo', set get hi' + hi
__device__ __forceinline__ float halve16(float lo, float hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(lo), __float_as_int(hi), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// Sum 16 per-lane values over the 32 lanes of each half-wave by recursive
// halving; every lane returns the half-wave total of value (lane >> 1) & 15.
__device__ __forceinline__ float half_sum16(const float (&a)[16], int lane) {
  float b8[8], b4[4], b2[2];
#pragma unroll
  for (int j = 0; j < 8; ++j) b8[j] = halve16(a[j], a[j + 8]);
  const bool u3 = (lane >> 3) & 1, u2 = (lane >> 2) & 1, u1 = (lane >> 1) & 1;
#pragma unroll
  for (int j = 0; j < 4; ++j) b4[j] = (u3 ? b8[j + 4] : b8[j]) + lane_xor8(u3 ? b8[j] : b8[j + 4]);
#pragma unroll
  for (int j = 0; j < 2; ++j) b2[j] = (u2 ? b4[j + 2] : b4[j]) + lane_xor4(u2 ? b4[j] : b4[j + 2]);
  float b1 = (u1 ? b2[1] : b2[0]) + lane_xor2(u1 ? b2[0] : b2[1]);
  b1 += lane_xor1(b1);
  return b1;
}

// third descriptor word of a raw buffer resource on gfx9
constexpr int kRsrcW3 = 0x00020000;
__device__ __forceinline__ uint2 ld_buf64(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  return make_uint2(v[0], v[1]);
}

// Block barrier that orders LDS only: global loads in flight stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ uint4 ld128(const uint16_t* base, int idx) {
  return *reinterpret_cast<const uint4*>(base + idx);
}
// Transposing LDS read: within each 16-lane group, lane i receives element i%4
// of the 8-byte reads of lanes 4j + i/4 (j = 0..3) as its element j.
__device__ __forceinline__ uint2 ld_tr(const uint16_t* p) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Decay factors of the blocked factorisation for channels c..c+3 (from pb, pf):
//   em(I)     = e^{m_I}         product of alpha from the chunk start to block I's token 8
//   enm(I)    = e^{g_n - m_I}   ... after block I's token 8 to the chunk end
//   pair(I,J) = e^{m_I - m_J}   ... after block J's token 8 to block I's token 8
__device__ __forceinline__ float4 ldf4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 em_of(const Lds& L, int I, int c) {
  float4 r = ldf4(&L.pb[I][c]);
#pragma unroll
  for (int J = 0; J < NSB; ++J)
    if (J < I) r = mul4(r, mul4(ldf4(&L.pb[J][c]), ldf4(&L.pf[J][c])));
  return r;
}
__device__ __forceinline__ float4 enm_of(const Lds& L, int I, int c) {
  float4 r = ldf4(&L.pf[I][c]);
#pragma unroll
  for (int J = 0; J < NSB; ++J)
    if (J > I) r = mul4(r, mul4(ldf4(&L.pb[J][c]), ldf4(&L.pf[J][c])));
  return r;
}
__device__ __forceinline__ float4 pair_of(const Lds& L, int I, int J, int c) {
  float4 r = mul4(ldf4(&L.pf[J][c]), ldf4(&L.pb[I][c]));
#pragma unroll
  for (int K = 0; K < NSB; ++K)
    if (K > J && K < I) r = mul4(r, mul4(ldf4(&L.pb[K][c]), ldf4(&L.pf[K][c])));
  return r;
}

// One pass over the chunks of one segment of one (batch, head).
// OUT = true: output pass, state S, writes o (and S_final from the last segment).
// OUT = false: summary pass; even logical blocks run S from 0, odd ones the
// transition M from I (no v); both write their state at output-segment boundaries.
//
// Per chunk, phases and the barriers after them:
//   loads; E1: norms and block decay products           | B
//   E2/E3: decay factors, operands kr kc qw; v loads     | C
//   M1T: A / Aqk tiles, diagonal inverses, Q^ S          | D
//   X: block substitution for U~ (registers) and W       | E
//   S: U = U~ - W S, O += Aqk U, state update            | F   (then the o store)
//
// Two factorisations of the pairwise decay e^{g_i - g_j} are used:
//  * fast: one reference at the chunk start (K^ = K e^{g}, K_ = K e^{-g}); valid
//    while every channel decays by less than e^{-80} over the chunk, chosen per
//    chunk by a block-wide vote;
//  * blocked: references at token 8 of each 16-token block, with the factors
//    e^{m_I - m_J}, e^{m_I}, e^{g_n - m_I} applied to fragments as they are
//    read; valid while log(alpha) >= -11 per token.
template <bool OUT>
__global__ __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(2))) void kda_chunk_kernel(ChunkArgs a) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  Lds& L = *reinterpret_cast<Lds*>(lds_raw);

  const uint32_t lid = (a.grid % 8 == 0) ? xcd_contiguous_id(blockIdx.x, (uint32_t)a.grid) : blockIdx.x;
  if (lid >= (uint32_t)a.nblk) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform
  const int l16 = lane & 15, q4 = lane >> 4;
  int64_t bh;
  int p;
  bool mkind = false;
  if (OUT) {
    bh = lid / a.P;
    p = lid % a.P;
  } else {
    mkind = lid & 1;
    bh = (lid >> 1) / a.P;
    p = (lid >> 1) % a.P;
  }
  const bool has_v = OUT || !mkind;
  const int64_t b = bh / a.H, h = bh % a.H;
  const int64_t NC = (a.T + CT - 1) / CT;
  const int64_t c_begin = (int64_t)p * a.L;
  int64_t c_end = min<int64_t>(NC, c_begin + a.L);
  if (!OUT) c_end = min<int64_t>(c_end, a.c_stop);

  // ---- state: rows 16 rt + 4 q4 + r, columns col0 + 16 ct + l16 -----------------
  const int col0 = 32 * wave;
  const int svo = ((4 * q4) * D + col0 + l16) * 4;   // lane part of a state element's byte offset
  f32x4 S[8][2];
  {
    const float* src = nullptr;
    if (OUT) src = a.P > 1 ? a.Sstart + (bh * a.P + p) * D * D : (a.S0 ? a.S0 + bh * D * D : nullptr);
    if (src) {
      const auto rs = __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, D * D * 4, kRsrcW3);
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            S[rt][ct][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, svo, ((16 * rt + r) * D + 16 * ct) * 4, 0));
    } else {
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 16 * rt + 4 * q4 + r, col = col0 + 16 * ct + l16;
            S[rt][ct][r] = (!OUT && mkind && row == col) ? 1.f : 0.f;
          }
    }
  }
  if (OUT && a.P > 1 && p % kSub != 0) {
    // a start inside a summary segment: S_start(p) = M_e S_start(p - p % kSub) + S_e with
    // e = p - 1, in fp32-accurate MFMA (bf16 high and low parts, three products)
    const int e = p - 1;
    const float* Mp = a.WM + (bh * a.E + e) * D * D;
    const float* Sp = a.WS + (bh * a.E + e) * D * D;
    const float* base = a.Sstart + (bh * a.P + (p - p % kSub)) * D * D;
    uint4 bH[4][2], bL[4][2];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int col = col0 + 16 * ct + l16;
        float4 v0, v1;
        v0.x = base[(32 * s + 4 * q4 + 0) * D + col]; v0.y = base[(32 * s + 4 * q4 + 1) * D + col];
        v0.z = base[(32 * s + 4 * q4 + 2) * D + col]; v0.w = base[(32 * s + 4 * q4 + 3) * D + col];
        v1.x = base[(32 * s + 16 + 4 * q4 + 0) * D + col]; v1.y = base[(32 * s + 16 + 4 * q4 + 1) * D + col];
        v1.z = base[(32 * s + 16 + 4 * q4 + 2) * D + col]; v1.w = base[(32 * s + 16 + 4 * q4 + 3) * D + col];
        uint2 l0, l1;
        const uint2 h0 = pack_split(v0, l0), h1 = pack_split(v1, l1);
        bH[s][ct] = cat(h0, h1);
        bL[s][ct] = cat(l0, l1);
      }
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) {
      uint4 aH[4], aL[4];
      const float* mrow = Mp + (16 * rt + l16) * D;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint2 l0, l1;
        const uint2 h0 = pack_split(ldf4(mrow + 32 * s + 4 * q4), l0);
        const uint2 h1 = pack_split(ldf4(mrow + 32 * s + 16 + 4 * q4), l1);
        aH[s] = cat(h0, h1);
        aL[s] = cat(l0, l1);
      }
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        f32x4 acc0, acc1 = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) acc0[r] = Sp[(16 * rt + 4 * q4 + r) * D + col0 + 16 * ct + l16];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          acc1 = mma32(aL[s], bH[s][ct], acc1);
          acc2 = mma32(aH[s], bL[s][ct], acc2);
          acc0 = mma32(aH[s], bH[s][ct], acc0);
        }
        S[rt][ct] = acc0 + (acc1 + acc2);
      }
    }
  }
  auto store_state = [&](float* m) {
    float* dst = m + svo / 4;
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(16 * rt + r) * D + 16 * ct] = S[rt][ct][r];
  };
  if (OUT) {   // the Aqk blocks (0,1) and (2,3) above the diagonal are read as zeros
    for (int e = tid; e < 2 * SBT * SBT; e += NTHR) {
      const int I = (e >> 8) * 2, i = (e >> 4) & 15, j = e & 15;
      L.aqk[tr(SBT * I + i, cpos(SBT * (I + 1) + j))] = 0;
    }
  }

  const uint2 kOnes = make_uint2(0x3F803F80u, 0x3F803F80u);   // alpha = 1 past the end

  for (int64_t c = c_begin; c < c_end; ++c) {
    // Lane-derived addresses are recomputed every chunk (cheap) rather than kept live
    // across the loop: the lane_c id passes through an empty asm so that they cannot be
    // hoisted out of it.
    int lane_c = lane;
    asm volatile("" : "+v"(lane_c));
    const int l16 = lane_c & 15, q4 = lane_c >> 4;
    // elementwise mapping: wave = decay block; half-wave hf = tokens 8 hf .. 8 hf + 7
    // of the block; lane_c cg = channels 4 cg .. 4 cg + 3
    const int hf = lane_c >> 5, cg = lane_c & 31, c0 = 4 * cg, p0 = cpos(c0);
    const int tk0 = SBT * wave + 8 * hf;
    const int64_t t0 = c * CT;
    const int n = (int)min<int64_t>(CT, a.T - t0);

    // ---- loads ----------------------------------------------------------------------
    // Buffer loads: block-uniform base and bounds (the chunk's first n tokens), byte
    // offsets split into a lane_c part and a uniform part. Reads past the bound return
    // zero, which is k = q = v = beta = 0 for tokens past the end; alpha is set to 1.
    uint2 kx[8], qx[8], ax[8], a8;
    uint4 vx[4];
    float bt;
    {
      const int64_t row0 = b * a.T + t0;
      const int st2 = (int)a.stride * 2, sa2 = (int)(a.H * D) * 2;
      const auto rk_ = __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + row0 * a.stride + h * D), 0, n * st2, kRsrcW3);
      const auto rq_ = __builtin_amdgcn_make_buffer_rsrc((void*)(a.q + row0 * a.stride + h * D), 0, n * st2, kRsrcW3);
      const auto ra_ = __builtin_amdgcn_make_buffer_rsrc((void*)(a.alpha + (row0 * a.H + h) * D), 0, n * sa2, kRsrcW3);
      const auto rb_ = __builtin_amdgcn_make_buffer_rsrc((void*)(a.beta + row0 * a.H + h), 0, n * (int)a.H * 2, kRsrcW3);
      const int vk = (8 * hf) * st2 + 2 * c0, va = (8 * hf) * sa2 + 2 * c0;
      const int tb = SBT * wave;   // first token of this wave's block
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        kx[i] = ld_buf64(rk_, vk, (tb + i) * st2);
        qx[i] = OUT ? ld_buf64(rq_, vk, (tb + i) * st2) : make_uint2(0u, 0u);
        const uint2 av = ld_buf64(ra_, va, (tb + i) * sa2);
        ax[i] = tk0 + i < n ? av : kOnes;
      }
      const uint2 av8 = ld_buf64(ra_, va, (tb + 8) * sa2);
      a8 = (hf == 0 && tk0 + 8 < n) ? av8 : kOnes;
      bt = bf2f(__builtin_amdgcn_raw_buffer_load_b16(rb_, tid * (int)a.H * 2, 0, 0));
    }

    // ---- E1: norms, block decay products -------------------------------------------
    if (tid < CT) L.beta[tid] = bt;
    if (a.l2norm) {
      float ss[16];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ss[i] = dot4(kx[i]);
        ss[i + 8] = OUT ? dot4(qx[i]) : 0.f;
      }
      const float tot = half_sum16(ss, lane_c);
      if ((lane_c & 1) == 0) {
        const int vv = (lane_c >> 1) & 15;          // 0..7: k of token vv; 8..15: q of token vv - 8
        const float rn = __builtin_amdgcn_rsqf(tot + kL2Eps);
        if (vv < 8) L.rk[tk0 + vv] = rn; else L.rq[tk0 + vv - 8] = rn;
      }
    } else if (cg < 8) {
      L.rk[tk0 + cg] = 1.f;
      L.rq[tk0 + cg] = 1.f;
    }
    if (hf == 1) {
      float4 run = unpack4(ax[1]);
#pragma unroll
      for (int i = 2; i < 8; ++i) run = mul4(run, unpack4(ax[i]));
      *reinterpret_cast<float4*>(&L.pf[wave][c0]) = run;
    } else {
      float4 run = unpack4(a8);
#pragma unroll
      for (int i = 0; i < 8; ++i) run = mul4(run, unpack4(ax[i]));
      *reinterpret_cast<float4*>(&L.pb[wave][c0]) = run;
    }
    lds_barrier();   // B

    // ---- E2 / E3: decay factors and MFMA operands --------------------------------------
    bool fast;
    {
      float4 full[NSB], pbw = make_float4(1.f, 1.f, 1.f, 1.f);
#pragma unroll
      for (int J = 0; J < NSB; ++J) {
        const float4 pbJ = ldf4(&L.pb[J][c0]);
        full[J] = mul4(pbJ, ldf4(&L.pf[J][c0]));
        if (J == wave) pbw = pbJ;
      }
      float4 egn4 = full[0], em4 = pbw;
#pragma unroll
      for (int J = 1; J < NSB; ++J) egn4 = mul4(egn4, full[J]);
#pragma unroll
      for (int J = 0; J < NSB - 1; ++J)
        if (J < wave) em4 = mul4(em4, full[J]);
      // every wave holds all 128 channels, so every wave reaches the same vote
      fast = __all(fminf(fminf(egn4.x, egn4.y), fminf(egn4.z, egn4.w)) >= kFastMin) != 0;
      if (wave == 0 && hf == 0) *reinterpret_cast<float4*>(&L.egn[c0]) = egn4;
      const float4 iem4 = rcp4(em4);
      // er = e^{g - m_I}, ec = e^{m_I - g}: running products from the block's token 8
      const float4 one4 = make_float4(1.f, 1.f, 1.f, 1.f);
      const float4 mr = fast ? em4 : one4, mc = fast ? iem4 : one4;
      auto put = [&](int i, float4 er, float4 ec) {
        const float4 fr = mul4(er, mr), fc = mul4(ec, mc);
        const int tk = tk0 + i;
        *reinterpret_cast<uint2*>(&L.kr[rm(tk, p0)]) = pack4(mul4(unpack4(kx[i]), fr));
        *reinterpret_cast<uint2*>(&L.kc[rm(tk, p0)]) = pack4(mul4(unpack4(kx[i]), fc));
        if (OUT) *reinterpret_cast<uint2*>(&L.qw[rm(tk, p0)]) = pack4(mul4(unpack4(qx[i]), fr));
      };
      if (hf == 1) {
        float4 run = make_float4(1.f, 1.f, 1.f, 1.f);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (i > 0) run = mul4(run, unpack4(ax[i]));
          put(i, run, rcp4(run));
        }
      } else {
        float4 run = unpack4(a8);
#pragma unroll
        for (int i = 7; i >= 0; --i) {
          if (i < 7) run = mul4(run, unpack4(ax[i + 1]));
          put(i, rcp4(run), run);
        }
      }
    }
    lds_barrier();   // C
    // ---- M1T: A and Aqk blocks, diagonal inverses, Q^ S ---------------------------------
    // state as bf16 B operand: slots 0-3 rows 32s+4q+r, 4-7 rows 32s+16+4q+r
    auto pack_state = [&](uint4(&Sf)[4][2]) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) Sf[s][ct] = pack8(S[2 * s][ct], S[2 * s + 1][ct]);
    };
    f32x4 O[4][2];
    {
      auto frags = [&](const uint16_t* arr, int blk, uint4(&f)[4]) {
#pragma unroll
        for (int s = 0; s < 4; ++s) f[s] = ld128(arr, rm(SBT * blk + l16, 32 * s + 8 * q4));
      };
      auto paired = [&](int I, int J, const uint4(&in)[4], uint4(&out)[4]) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if (fast) {
            out[s] = in[s];
          } else {
            out[s] = scale8(in[s], pair_of(L, I, J, 32 * s + 4 * q4), pair_of(L, I, J, 32 * s + 16 + 4 * q4));
          }
        }
      };
      auto mma4 = [&](const uint4(&ra)[4], const uint4(&cb)[4]) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mma32(ra[s], cb[s], acc);
        return acc;
      };
      // A(I, J) below the diagonal -> at (negated); A(I, I) -> adiag (fp32)
      auto epi_a = [&](int I, int J, f32x4 acc) {
        const int j = SBT * J + l16;
        const float rkj = L.rk[j];
        const float4 b4 = ldf4(&L.beta[SBT * I + 4 * q4]), k4 = ldf4(&L.rk[SBT * I + 4 * q4]);
        const float rowf[4] = {b4.x * k4.x, b4.y * k4.y, b4.z * k4.z, b4.w * k4.w};
        if (I == J) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            L.adiag[I][4 * q4 + r][4 * (l16 & 3) + (l16 >> 2)] = 4 * q4 + r > l16 ? rowf[r] * rkj * acc[r] : 0.f;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) L.at[tr(SBT * I + 4 * q4 + r, j)] = f2bf(-rowf[r] * rkj * acc[r]);
        }
      };
      auto epi_q = [&](int I, int J, f32x4 acc) {
        const int j = SBT * J + l16;
        const float rkj = L.rk[j];
        const float4 rq4 = ldf4(&L.rq[SBT * I + 4 * q4]);
        const float rowf[4] = {rq4.x, rq4.y, rq4.z, rq4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool keep = I > J || 4 * q4 + r >= l16;
          L.aqk[tr(SBT * I + 4 * q4 + r, cpos(j))] = f2bf(keep ? rowf[r] * rkj * acc[r] : 0.f);
        }
      };
      uint4 cA[4], cB[4], rA[4], sc[4];
      if (OUT) {
        // wave 0: A00 Aqk00 A10 A30 Aqk30;  wave 1: A11 Aqk11 Aqk10 A31 Aqk31;
        // wave 2: A22 A20 Aqk22 A32 Aqk32;  wave 3: A33 Aqk33 A21 Aqk21 Aqk20
        if (wave == 0) {
          frags(L.kc, 0, cA);
          frags(L.kr, 0, rA); epi_a(0, 0, mma4(rA, cA));
          frags(L.qw, 0, rA); epi_q(0, 0, mma4(rA, cA));
          frags(L.kr, 1, rA); paired(1, 0, cA, sc); epi_a(1, 0, mma4(rA, sc));
          paired(3, 0, cA, sc);
          frags(L.kr, 3, rA); epi_a(3, 0, mma4(rA, sc));
          frags(L.qw, 3, rA); epi_q(3, 0, mma4(rA, sc));
        } else if (wave == 1) {
          frags(L.kc, 1, cA);
          frags(L.kr, 1, rA); epi_a(1, 1, mma4(rA, cA));
          frags(L.qw, 1, rA); epi_q(1, 1, mma4(rA, cA));
          frags(L.kc, 0, cB); paired(1, 0, cB, sc); epi_q(1, 0, mma4(rA, sc));
          paired(3, 1, cA, sc);
          frags(L.kr, 3, rA); epi_a(3, 1, mma4(rA, sc));
          frags(L.qw, 3, rA); epi_q(3, 1, mma4(rA, sc));
        } else if (wave == 2) {
          frags(L.kc, 2, cA);
          frags(L.kr, 2, rA); epi_a(2, 2, mma4(rA, cA));
          frags(L.kc, 0, cB); paired(2, 0, cB, sc); epi_a(2, 0, mma4(rA, sc));
          frags(L.qw, 2, rA); epi_q(2, 2, mma4(rA, cA));
          paired(3, 2, cA, sc);
          frags(L.kr, 3, rA); epi_a(3, 2, mma4(rA, sc));
          frags(L.qw, 3, rA); epi_q(3, 2, mma4(rA, sc));
        } else {
          frags(L.kc, 3, cA);
          frags(L.kr, 3, rA); epi_a(3, 3, mma4(rA, cA));
          frags(L.qw, 3, rA); epi_q(3, 3, mma4(rA, cA));
          frags(L.kc, 1, cB); paired(2, 1, cB, sc);
          frags(L.kr, 2, rA); epi_a(2, 1, mma4(rA, sc));
          frags(L.qw, 2, rA); epi_q(2, 1, mma4(rA, sc));
          frags(L.kc, 0, cB); paired(2, 0, cB, sc); epi_q(2, 0, mma4(rA, sc));
        }
      } else {
        // wave 0: A00 A10 A20;  wave 1: A11 A21 A31;  wave 2: A22 A32;  wave 3: A33 A30
        if (wave == 0) {
          frags(L.kc, 0, cA);
          frags(L.kr, 0, rA); epi_a(0, 0, mma4(rA, cA));
          frags(L.kr, 1, rA); paired(1, 0, cA, sc); epi_a(1, 0, mma4(rA, sc));
          frags(L.kr, 2, rA); paired(2, 0, cA, sc); epi_a(2, 0, mma4(rA, sc));
        } else if (wave == 1) {
          frags(L.kc, 1, cA);
          frags(L.kr, 1, rA); epi_a(1, 1, mma4(rA, cA));
          frags(L.kr, 2, rA); paired(2, 1, cA, sc); epi_a(2, 1, mma4(rA, sc));
          frags(L.kr, 3, rA); paired(3, 1, cA, sc); epi_a(3, 1, mma4(rA, sc));
        } else if (wave == 2) {
          frags(L.kc, 2, cA);
          frags(L.kr, 2, rA); epi_a(2, 2, mma4(rA, cA));
          frags(L.kr, 3, rA); paired(3, 2, cA, sc); epi_a(3, 2, mma4(rA, sc));
        } else {
          frags(L.kc, 3, cA);
          frags(L.kr, 3, rA); epi_a(3, 3, mma4(rA, cA));
          frags(L.kc, 0, cB); paired(3, 0, cB, sc); epi_a(3, 0, mma4(rA, sc));
        }
      }
      // A_II was written by this wave: order its LDS writes before the reads below
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      {
        // T_II = (I + A_II)^{-1}, I = wave, by forward substitution: lane_c = 16 part + j
        // owns column j and the terms k = part + 4m of every row's sum; the four parts
        // are summed with lane_c swaps
        const int I = wave;
        const int part = lane_c >> 4, jj = lane_c & 15;
        float xs[4] = {0.f, 0.f, 0.f, 0.f};   // x[part + 4m] of column jj
        constexpr int AH = 4;                  // rows of A_II read ahead
        float4 arow[AH];
#pragma unroll
        for (int i = 0; i < AH; ++i) arow[i] = ldf4(&L.adiag[I][i][4 * part]);
#pragma unroll
        for (int i = 0; i < SBT; ++i) {
          const float4 ar = arow[i % AH];
          if (i + AH < SBT) arow[i % AH] = ldf4(&L.adiag[I][i + AH][4 * part]);
          float ps = ar.x * xs[0] + ar.y * xs[1] + ar.z * xs[2] + ar.w * xs[3];
          ps = halve16(ps, ps);
          ps = halve32(ps, ps);
          const float xi = (i == jj ? 1.f : 0.f) - ps;
          if (part == (i & 3)) xs[i >> 2] = xi;
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) L.at[tr(SBT * I + part + 4 * m, SBT * I + jj)] = f2bf(xs[m]);
      }
      if (OUT) {
        // O = diag(1/|q|) Q^ S; the blocked factorisation scales Q^'s channels by e^{m_I}
        uint4 Sf[4][2];
        pack_state(Sf);
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          uint4 qf[4];
          frags(L.qw, I, qf);
          if (!fast) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
              qf[s] = scale8(qf[s], em_of(L, I, 32 * s + 4 * q4), em_of(L, I, 32 * s + 16 + 4 * q4));
          }
          const float4 rq4 = ldf4(&L.rq[SBT * I + 4 * q4]);
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) acc = mma32(qf[s], Sf[s][ct], acc);
            acc[0] *= rq4.x; acc[1] *= rq4.y; acc[2] *= rq4.z; acc[3] *= rq4.w;
            O[I][ct] = acc;
          }
        }
      }
    }
    {
      const int st2 = (int)a.stride * 2;
      if (has_v) {
        // this wave's v columns col0 .. col0 + 31: lane_c = tokens 4 (l >> 2) + j, channels col0 + 8 (l & 3) ..
        const auto rv_ = __builtin_amdgcn_make_buffer_rsrc((void*)(a.v + (b * a.T + t0) * a.stride + h * D), 0, n * st2, kRsrcW3);
        const int vo = (4 * (lane_c >> 2)) * st2 + 2 * (col0 + 8 * (lane_c & 3));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const auto v4 = __builtin_amdgcn_raw_buffer_load_b128(rv_, vo, j * st2, 0);
          vx[j] = make_uint4(v4[0], v4[1], v4[2], v4[3]);
        }
      }
    }
    lds_barrier();   // D

    // ---- X: block substitution X = (I + A)^{-1} diag(sigma) R --------------------------
    // right-hand sides: this wave's v columns (U~, kept in registers) and the K^
    // channel tiles 2 wave, 2 wave + 1 (W, negated, written over those kr channels:
    // no other wave reads them in this phase)
    f32x4 Ut[4][2];
    {
      uint2 af[10];   // block (I, J) at I (I + 1) / 2 + J
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int J = 0; J <= I; ++J)
          af[I * (I + 1) / 2 + J] = *reinterpret_cast<const uint2*>(&L.at[tr(SBT * I + l16, SBT * J + 4 * q4)]);
      auto solve = [&](const f32x4(&y0)[4], f32x4(&X)[4]) {
        uint2 Xb[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          f32x4 y = y0[I];
#pragma unroll
          for (int J = 0; J < I; ++J) y = mma16(af[I * (I + 1) / 2 + J], Xb[J], y);
          X[I] = mma16(af[I * (I + 1) / 2 + I], pack4(y), f32x4{0.f, 0.f, 0.f, 0.f});
          Xb[I] = pack4(X[I]);
        }
      };
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int t = 2 * wave + tt;                       // channels 16 t .. 16 t + 15
        const int tpos = 32 * (t >> 1) + 4 * (t & 1);      // cpos(16 t)
        f32x4 y[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          // lane_c (l16, q4) receives channel 16 t + l16 of tokens 16 I + 4 q4 + 0..3
          const float4 kv = unpack4(ld_tr(&L.kr[rm(SBT * I + 4 * q4 + (l16 >> 2), tpos + 8 * (l16 & 3))]));
          float sc = 1.f;
          if (!fast) sc = pick(em_of(L, I, 16 * t + (l16 & ~3)), l16 & 3);
          const float4 kr4 = mul4(ldf4(&L.beta[SBT * I + 4 * q4]), ldf4(&L.rk[SBT * I + 4 * q4]));
          y[I][0] = kv.x * kr4.x * sc; y[I][1] = kv.y * kr4.y * sc;
          y[I][2] = kv.z * kr4.z * sc; y[I][3] = kv.w * kr4.w * sc;
        }
        f32x4 X[4];
        solve(y, X);
        const int wcol = tpos + 8 * (l16 >> 2) + (l16 & 3);   // cpos(16 t + l16)
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
          for (int r = 0; r < 4; ++r) L.kr[rm(SBT * I + 4 * q4 + r, wcol)] = f2bf(-X[I][r]);
      }
      if (has_v) {
        // v -> channels col0 .. col0 + 31 of qw (Q^ is no longer read; no other wave
        // touches these channels in this phase), then read back transposed
        {
          const int vp = col0 + 16 * (lane_c & 1) + 4 * ((lane_c >> 1) & 1);   // cpos(col0 + 8 (l & 3))
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int row = 4 * (lane_c >> 2) + j;
            *reinterpret_cast<uint2*>(&L.qw[rm(row, vp)]) = make_uint2(vx[j].x, vx[j].y);
            *reinterpret_cast<uint2*>(&L.qw[rm(row, vp + 8)]) = make_uint2(vx[j].z, vx[j].w);
          }
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
          __builtin_amdgcn_wave_barrier();
        }
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const int t = 2 * wave + ct;
          const int tpos = 32 * (t >> 1) + 4 * (t & 1);      // cpos(16 t)
          f32x4 y[4];
#pragma unroll
          for (int I = 0; I < 4; ++I) {
            const float4 vv = unpack4(ld_tr(&L.qw[rm(SBT * I + 4 * q4 + (l16 >> 2), tpos + 8 * (l16 & 3))]));
            const float4 br = ldf4(&L.beta[SBT * I + 4 * q4]);
            y[I][0] = vv.x * br.x; y[I][1] = vv.y * br.y;
            y[I][2] = vv.z * br.z; y[I][3] = vv.w * br.w;
          }
          f32x4 X[4];
          solve(y, X);
#pragma unroll
          for (int I = 0; I < 4; ++I) Ut[I][ct] = X[I];
        }
      } else {
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) Ut[I][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    lds_barrier();   // E

    // ---- S: U = U~ - W S;  O = diag(1/|q|) Q^ S + Aqk U;  S <- Diag(e^{g_n}) S + K~^T diag(1/|k|) U
    {
      uint4 Sf[4][2];
      pack_state(Sf);
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        uint4 wf[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) wf[s] = ld128(L.kr, rm(SBT * I + l16, 32 * s + 8 * q4));
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int s = 0; s < 4; ++s) Ut[I][ct] = mma32(wf[s], Sf[s][ct], Ut[I][ct]);
      }
      if (OUT) {
        uint4 Uf[2][2], qa[6];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) Uf[s][ct] = pack8(Ut[2 * s][ct], Ut[2 * s + 1][ct]);
        qa[0] = ld128(L.aqk, tr(l16, 8 * q4));
        qa[1] = ld128(L.aqk, tr(SBT + l16, 8 * q4));
        qa[2] = ld128(L.aqk, tr(2 * SBT + l16, 8 * q4));
        qa[3] = ld128(L.aqk, tr(2 * SBT + l16, 32 + 8 * q4));
        qa[4] = ld128(L.aqk, tr(3 * SBT + l16, 8 * q4));
        qa[5] = ld128(L.aqk, tr(3 * SBT + l16, 32 + 8 * q4));
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          O[0][ct] = mma32(qa[0], Uf[0][ct], O[0][ct]);
          O[1][ct] = mma32(qa[1], Uf[0][ct], O[1][ct]);
          O[2][ct] = mma32(qa[2], Uf[0][ct], O[2][ct]);
          O[2][ct] = mma32(qa[3], Uf[1][ct], O[2][ct]);
          O[3][ct] = mma32(qa[4], Uf[0][ct], O[3][ct]);
          O[3][ct] = mma32(qa[5], Uf[1][ct], O[3][ct]);
        }
        // output tile -> this wave's channels of qw (natural order) -> o rows, 16 bytes per lane_c;
        // rows past the end fall outside the buffer bound and are dropped
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
          for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) L.qw[rm(SBT * I + 4 * q4 + r, col0 + 16 * ct + l16)] = f2bf(O[I][ct][r]);
      }
    }
    {
      uint4 Upf[2][2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const float4 ka = ldf4(&L.rk[32 * s + 4 * q4]), kb = ldf4(&L.rk[32 * s + 16 + 4 * q4]);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          f32x4 lo = Ut[2 * s][ct], hi = Ut[2 * s + 1][ct];
          lo[0] *= ka.x; lo[1] *= ka.y; lo[2] *= ka.z; lo[3] *= ka.w;
          hi[0] *= kb.x; hi[1] *= kb.y; hi[2] *= kb.z; hi[3] *= kb.w;
          Upf[s][ct] = pack8(lo, hi);
        }
      }
      // A operand K~^T: lane_c (l16, q4) = channel 16 rt + l16, tokens 32 s + 4 q4 + 0..3
      // and 32 s + 16 + 4 q4 + 0..3, read transposed from kc
      const int kbase = rm(4 * q4 + (l16 >> 2), 8 * (l16 & 3));
#pragma unroll
      for (int rt = 0; rt < 8; ++rt) {
        const int cp = 32 * (rt >> 1) + 4 * (rt & 1);   // cpos(16 rt)
        uint4 kt[2];
#pragma unroll
        for (int s = 0; s < 2; ++s)
          kt[s] = cat(ld_tr(&L.kc[kbase + rm(32 * s, cp)]), ld_tr(&L.kc[kbase + rm(32 * s + 16, cp)]));
        const float4 eg = ldf4(&L.egn[16 * rt + 4 * q4]);
        if (fast) {
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            f32x4 acc = S[rt][ct];
            acc = mma32(kt[0], Upf[0][ct], acc);
            acc = mma32(kt[1], Upf[1][ct], acc);
            acc[0] *= eg.x; acc[1] *= eg.y; acc[2] *= eg.z; acc[3] *= eg.w;
            S[rt][ct] = acc;
          }
        } else {
          // blocked: K~ = K_ e^{g_n - m_I} for the tokens of block I
          const int cl = 16 * rt + (l16 & ~3), u = l16 & 3;
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const float f0 = pick(enm_of(L, 2 * s, cl), u), f1 = pick(enm_of(L, 2 * s + 1, cl), u);
            kt[s] = scale8(kt[s], make_float4(f0, f0, f0, f0), make_float4(f1, f1, f1, f1));
          }
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            f32x4 acc = S[rt][ct];
            acc[0] *= eg.x; acc[1] *= eg.y; acc[2] *= eg.z; acc[3] *= eg.w;
            acc = mma32(kt[0], Upf[0][ct], acc);
            acc = mma32(kt[1], Upf[1][ct], acc);
            S[rt][ct] = acc;
          }
        }
      }
    }
    if (OUT) {
      // staged output rows -> o, 16 bytes per lane; rows past the end fall outside the
      // buffer bound and are dropped
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      const int so2 = (int)(a.H * D) * 2;
      const auto ro = __builtin_amdgcn_make_buffer_rsrc((void*)(a.o + ((b * a.T + t0) * a.H + h) * D), 0, n * so2,
                                                        kRsrcW3);
      const int oc = col0 + 8 * (lane_c & 3);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 4 * (lane_c >> 2) + j;
        const uint4 u = *reinterpret_cast<const uint4*>(&L.qw[rm(row, oc)]);
        typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
        const u32x4_t w4 = {u.x, u.y, u.z, u.w};
        __builtin_amdgcn_raw_buffer_store_b128(w4, ro, row * so2 + 2 * oc, 0, 0);
      }
    }
    lds_barrier();   // F

    if (!OUT) {
      const int64_t rel = c - c_begin;
      if ((rel + 1) % a.Lo == 0) {
        const int e = p * kSub + (int)(rel / a.Lo);
        store_state((mkind ? a.WM : a.WS) + (bh * a.E + e) * D * D);
      }
    }
  }

  if (OUT && a.S_final != nullptr && p == a.P - 1) store_state(a.S_final + bh * D * D);
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


__global__ __launch_bounds__(CB_T) void kda_combine_kernel(const float* __restrict__ WS, const float* __restrict__ WM,
                                                           const float* __restrict__ S0, float* __restrict__ Sst,
                                                           int P, int E) {
  __shared__ __align__(16) uint16_t bhi[2][16 * BTS];   // [column][cpos(row)], double-buffered
  __shared__ __align__(16) uint16_t blo[2][16 * BTS];
  const int64_t bh = blockIdx.x / 8;
  const int slice = blockIdx.x % 8;
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, q4 = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = 16 * slice + l16;
  const int row0 = 16 * wave + 4 * q4;       // D-layout rows of this lane: row0 .. row0 + 3
  const int arow = 16 * wave + l16;          // A-operand row of this lane

  f32x4 cur;
#pragma unroll
  for (int r = 0; r < 4; ++r) cur[r] = S0 ? S0[(bh * D + row0 + r) * D + col] : 0.f;
  auto store = [&](int po, const f32x4& v) {
    float* dst = Sst + (bh * P + po) * D * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[(row0 + r) * D + col] = v[r];
  };
  store(0, cur);
  const int nsteps = (P - 1) / kSub;   // chain starts kSub, 2 kSub, .. below P
  // rows of M_e of a step: slots 0-3 columns 32 s + 4 q4 .., 4-7 columns 32 s + 16 + 4 q4 ..
  float4 mq[kAhead][8];
  f32x4 sq[kAhead];
  auto fetch = [&](int step, float4(&m)[8], f32x4& sv) {
    if (step < nsteps) {
      const int e = step * kSub + kSub - 1;
      const float* mp = WM + ((bh * E + e) * D + arow) * D;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        m[2 * s] = ldf4(mp + 32 * s + 4 * q4);
        m[2 * s + 1] = ldf4(mp + 32 * s + 16 + 4 * q4);
      }
      const float* sp = WS + (bh * E + e) * D * D;
#pragma unroll
      for (int k = 0; k < 4; ++k) sv[k] = sp[(row0 + k) * D + col];
    }
  };
#pragma unroll
  for (int j = 0; j < kAhead; ++j) fetch(j, mq[j], sq[j]);
  for (int step = 0; step < nsteps; ++step) {
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
    f32x4 acc0 = sq[0], acc1 = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint2 l0, l1;
      const uint2 h0 = pack_split(mq[0][2 * s], l0), h1 = pack_split(mq[0][2 * s + 1], l1);
      const uint4 ah = cat(h0, h1), al = cat(l0, l1);
      acc1 = mma32(al, bH[s], acc1);
      acc2 = mma32(ah, bL[s], acc2);
      acc0 = mma32(ah, bH[s], acc0);
    }
    cur = acc0 + (acc1 + acc2);
    store(kSub * (step + 1), cur);
#pragma unroll
    for (int j = 0; j + 1 < kAhead; ++j) {
      sq[j] = sq[j + 1];
#pragma unroll
      for (int i = 0; i < 8; ++i) mq[j][i] = mq[j + 1][i];
    }
    fetch(step + kAhead, mq[kAhead - 1], sq[kAhead - 1]);
  }
}

struct Split {
  int Po, Lo;   // output segments, chunks per output segment
  int Ps, Ls;   // summary segments, chunks per summary segment
};

Split choose_split(int64_t B, int64_t T, int64_t H, bool no_split) {
  const int64_t NC = (T + CT - 1) / CT;
  const int64_t BH = B * H;
  if (no_split || NC <= 1 || BH >= kTargetBlocks) return Split{1, (int)NC, 0, 0};
  int64_t P = (kTargetBlocks + BH - 1) / BH;
  if (P > NC) P = NC;
  const int64_t Lo = (NC + P - 1) / P;
  P = (NC + Lo - 1) / Lo;
  if (P <= 1) return Split{1, (int)NC, 0, 0};
  const int64_t Ps = (P - 1 + kSub - 1) / kSub;   // summaries up to the last needed boundary
  return Split{(int)P, (int)Lo, (int)Ps, (int)(kSub * Lo)};
}

}  // namespace

bool kda_chunked_supported(const KdaArgs& a) {
  // 8-byte loads of q, k and alpha: token stride a multiple of 4 elements, 8-byte aligned bases
  const uintptr_t al = reinterpret_cast<uintptr_t>(a.q) | reinterpret_cast<uintptr_t>(a.k) |
                       reinterpret_cast<uintptr_t>(a.alpha);
  return a.bf16 && a.dk == D && a.dv == D && a.qkv_stride % 4 == 0 && a.qkv_stride <= (int64_t(1) << 24) &&
         (al & 7) == 0;
}

int64_t kda_chunked_segments(int64_t B, int64_t T, int64_t H, bool no_split) {
  return choose_split(B, T, H, no_split).Po;
}

size_t kda_chunked_workspace(int64_t B, int64_t T, int64_t H, bool no_split) {
  const Split sp = choose_split(B, T, H, no_split);
  if (sp.Po <= 1) return 0;
  const size_t mat = (size_t)D * D * sizeof(float);
  const size_t E = (size_t)sp.Ps * kSub;
  return (size_t)(B * H) * (2 * E + sp.Po) * mat;
}

hipError_t launch_kda_chunked(const KdaArgs& x, bool no_split, void* workspace, hipStream_t stream) {
  const Split sp = choose_split(x.B, x.T, x.H, no_split);
  const int64_t BH = x.B * x.H;
  if (BH * sp.Po * 2 > 0x7fffff00) return hipErrorInvalidValue;
  ChunkArgs a;
  a.q = static_cast<const uint16_t*>(x.q);
  a.k = static_cast<const uint16_t*>(x.k);
  a.v = static_cast<const uint16_t*>(x.v);
  a.stride = x.qkv_stride;
  a.alpha = static_cast<const uint16_t*>(x.alpha);
  a.beta = static_cast<const uint16_t*>(x.beta);
  a.S0 = x.S0;
  a.Sstart = nullptr;
  a.WS = nullptr;
  a.WM = nullptr;
  a.E = 0;
  a.o = static_cast<uint16_t*>(x.o);
  a.S_final = x.S_final;
  a.T = x.T;
  a.H = x.H;
  a.l2norm = x.l2norm ? 1 : 0;
  const size_t lds = sizeof(Lds);
  int dev = 0;
  hipError_t de = hipGetDevice(&dev);
  if (de != hipSuccess) return de;
  static bool attr_done[64] = {};
  if (dev < 0 || dev >= 64 || !attr_done[dev]) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kda_chunk_kernel<true>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kda_chunk_kernel<false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) attr_done[dev] = true;
  }
  auto round8 = [](int64_t n) { return (int)((n + 7) / 8 * 8); };
  if (sp.Po > 1) {
    const int64_t E = (int64_t)sp.Ps * kSub;
    float* WS = static_cast<float*>(workspace);
    float* WM = WS + BH * E * D * D;
    float* Sst = WM + BH * E * D * D;
    ChunkArgs s = a;
    s.WS = WS;
    s.WM = WM;
    s.P = sp.Ps;
    s.L = sp.Ls;
    s.Lo = sp.Lo;
    s.E = (int)E;
    s.c_stop = (int64_t)(sp.Po - 1) * sp.Lo;
    s.nblk = (int)(2 * BH * sp.Ps);
    s.grid = round8(s.nblk);
    hipLaunchKernelGGL(kda_chunk_kernel<false>, dim3((unsigned)s.grid), dim3(NTHR), lds, stream, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kda_combine_kernel, dim3((unsigned)(BH * 8)), dim3(CB_T), 0, stream, WS, WM, x.S0, Sst, sp.Po,
                       (int)E);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.Sstart = Sst;
    a.WS = WS;
    a.WM = WM;
    a.E = (int)E;
  }
  a.P = sp.Po;
  a.L = sp.Lo;
  a.Lo = sp.Lo;
  a.c_stop = 0;
  a.nblk = (int)(BH * sp.Po);
  a.grid = round8(a.nblk);
  hipLaunchKernelGGL(kda_chunk_kernel<true>, dim3((unsigned)a.grid), dim3(NTHR), lds, stream, a);
  return hipGetLastError();
}

}  // namespace chm
