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
// The per-(token, head) L2 normalisation of q and k (page 1, Fig. 2) is folded
// into the bf16 operands as they are formed (K^, K_ and Q^ carry 1 / |k| and
// 1 / |q|), so no product needs a separate norm scaling.
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
#include <cstddef>
#include <algorithm>
#include <atomic>
#include <vector>

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
// alpha is raised to at least e^{-7.5} (bf16 0x3A11) as it is loaded. The blocked
// factorisation scales k by products of up to 8 alphas and their reciprocals, so its
// bf16 operands then stay within e^{+-60} of k: both factors of every product keep full
// precision (far from the bf16 denormal range), and the reciprocals stay finite. A token
// with a smaller alpha (alpha = 0 included) then keeps 5.5e-4 of each decayed channel
// instead of less, which is below the bf16 resolution of the result.
constexpr uint32_t kAlphaMin2 = 0x3A113A11u;
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t clamp_alpha2(uint32_t u) {   // both bf16 halves (positive)
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, u),
                                                                 __builtin_bit_cast(u16x2_t, kAlphaMin2)));
}

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
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// sum of squares of the bf16 pair(s) in u (v_dot2_f32_bf16)
__device__ __forceinline__ float sq2(uint32_t u, float c) {
  const bf16x2_t v = __builtin_bit_cast(bf16x2_t, u);
  return __builtin_amdgcn_fdot2_f32_bf16(v, v, c, false);
}
__device__ __forceinline__ float dot4(uint2 u) { return sq2(u.y, sq2(u.x, 0.f)); }
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
  float pb[NSB][D];       // per block and channel: product of alpha over block tokens 0..7
  float pf[NSB][D];       //                        ... over block tokens 8..15
  float adiag[NSB * 272];  // strictly lower A_II in fp32: A_II(i, k) at 272 I + 16 i + k
  uint16_t at[CT * TRS];  // column-major: at[tr(j, i)] = -A(i, j) below the diagonal blocks, T_II on them
  uint16_t aqk[CT * TRS]; // column-major: aqk[tr(j, i)] = Aqk(i, j) (rows scaled 1/|q|, columns 1/|k|)
  uint16_t kr[CT * RKS];  // K^ = k e^{g} (fast) or k e^{g - m_I} (blocked); output staging at the end
  uint16_t kc[CT * RKS];  // K_ = k e^{-g} (fast) or k e^{m_I - g} (blocked)
  uint16_t qw[CT * RMS];  // Q^ = q e^{g} / q e^{g - m_I} (output pass); then -W
};
static_assert(sizeof(Lds) <= 81920, "two blocks per CU");

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
  int Lo;                 // chunks per output segment
  int nblk;               // logical blocks of this pass
  int grid;               // launched blocks
  int l2norm;
  int nruns;
  int xcd_ranges;         // give each XCD a contiguous range of logical blocks (one run only)
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
__device__ __forceinline__ int32_t uni(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }
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

// Sum 16 per-lane values over the 16 lanes of each DPP row by recursive halving; lane
// l16 of the row returns the row total of value l16.
__device__ __forceinline__ float row_sum16(const float (&a)[16], int l16) {
  float b8[8], b4[4], b2[2];
  const bool u3 = (l16 >> 3) & 1, u2 = (l16 >> 2) & 1, u1 = (l16 >> 1) & 1, u0 = l16 & 1;
#pragma unroll
  for (int j = 0; j < 8; ++j) b8[j] = (u3 ? a[j + 8] : a[j]) + lane_xor8(u3 ? a[j] : a[j + 8]);
#pragma unroll
  for (int j = 0; j < 4; ++j) b4[j] = (u2 ? b8[j + 4] : b8[j]) + lane_xor4(u2 ? b8[j] : b8[j + 4]);
#pragma unroll
  for (int j = 0; j < 2; ++j) b2[j] = (u1 ? b4[j + 2] : b4[j]) + lane_xor2(u1 ? b4[j] : b4[j + 2]);
  return (u0 ? b2[1] : b2[0]) + lane_xor1(u0 ? b2[0] : b2[1]);
}

// third descriptor word of a raw buffer resource on gfx9
constexpr int kRsrcW3 = 0x00020000;
__device__ __forceinline__ uint2 ld_buf64(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  return make_uint2(v[0], v[1]);
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
//   em(I)     = e^{m_I}         product of alpha from the chunk start to block I's token 7
//   enm(I)    = e^{g_n - m_I}   ... after block I's token 7 to the chunk end
//   pair(I,J) = e^{m_I - m_J}   ... after block J's token 7 to block I's token 7
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

// ---- pieces shared by the output and summary kernels ----------------------------------
// Fragment conventions (16x16x32 MFMA): lane = 16 q4 + l16; a row fragment of block
// `blk` holds row 16 blk + l16, positions 32 s + 8 q4 .. + 7 for s = 0..3.

template <int STRIDE = RKS>
__device__ __forceinline__ void tile_frags(const uint16_t* arr, int blk, uint4 (&f)[4], int l16, int q4) {
#pragma unroll
  for (int s = 0; s < 4; ++s) f[s] = ld128(arr, (SBT * blk + l16) * STRIDE + 32 * s + 8 * q4);
}
// column-operand fragments of block J scaled by e^{m_I - m_J} (blocked factorisation)
__device__ __forceinline__ void pair_frags(const Lds& L, bool fast, int I, int J, const uint4 (&in)[4],
                                           uint4 (&out)[4], int q4) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
    out[s] = fast ? in[s] : scale8(in[s], pair_of(L, I, J, 32 * s + 4 * q4), pair_of(L, I, J, 32 * s + 16 + 4 * q4));
}
__device__ __forceinline__ f32x4 mma4(const uint4 (&ra)[4], const uint4 (&cb)[4]) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = mma32(ra[s], cb[s], acc);
  return acc;
}
// A(I, J) = diag(b) (K^ K_^T)(I, J) (the operands carry 1 / |k|): below the diagonal -> at
// (negated, column-major: a lane's four rows are one 8-byte write), on it (strictly lower
// part) -> adiag in fp32
__device__ __forceinline__ void epi_a(Lds& L, int I, int J, f32x4 acc, int l16, int q4) {
  const int j = SBT * J + l16;
  const float4 b4 = ldf4(&L.beta[SBT * I + 4 * q4]);
  const float rowf[4] = {b4.x, b4.y, b4.z, b4.w};
  if (I == J) {
#pragma unroll
    for (int r = 0; r < 4; ++r) L.adiag[272 * I + 16 * (4 * q4 + r) + l16] = 4 * q4 + r > l16 ? rowf[r] * acc[r] : 0.f;
  } else {
    *reinterpret_cast<uint2*>(&L.at[tr(j, SBT * I + 4 * q4)]) = pack4(
        make_float4(-rowf[0] * acc[0], -rowf[1] * acc[1], -rowf[2] * acc[2], -rowf[3] * acc[3]));
  }
}
// Aqk(I, J) = (Q^ K_^T)(I, J) (the operands carry 1 / |q| and 1 / |k|), lower triangle
// including the diagonal, column-major
__device__ __forceinline__ void epi_q(Lds& L, int I, int J, f32x4 acc, int l16, int q4) {
  const int j = SBT * J + l16;
  float v[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const bool keep = I > J || 4 * q4 + r >= l16;
    v[r] = keep ? acc[r] : 0.f;
  }
  *reinterpret_cast<uint2*>(&L.aqk[tr(j, SBT * I + 4 * q4)]) = pack4(make_float4(v[0], v[1], v[2], v[3]));
}
// T_II = (I + A_II)^{-1}: lane j of a 16-lane group forms column j of T_II by forward
// substitution, x_i = [i = j] - sum_{k < i} A_II(i, k) x_k, reading the rows of A_II
// (written by this wave) as broadcasts; the column goes to at as four 8-byte writes.
__device__ __forceinline__ void invert_diag(Lds& L, int I, int jj, bool write) {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  float x[SBT];
#pragma unroll
  for (int i = 0; i < SBT; ++i) {
    float acc0 = i == jj ? 1.f : 0.f, acc1 = 0.f;
#pragma unroll
    for (int k4 = 0; k4 < (i + 3) / 4; ++k4) {
      const float4 a4 = ldf4(&L.adiag[272 * I + 16 * i + 4 * k4]);
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
#pragma unroll
    for (int m = 0; m < 4; ++m)
      *reinterpret_cast<uint2*>(&L.at[tr(SBT * I + jj, SBT * I + 4 * m)]) =
          make_uint2(pack_bf16x2(x[4 * m], x[4 * m + 1]), pack_bf16x2(x[4 * m + 2], x[4 * m + 3]));
  }
}
// the four diagonal blocks at once, lane = 16 I + j
__device__ __forceinline__ void invert_diag4(Lds& L, int lane) { invert_diag(L, lane >> 4, lane & 15, true); }
// mma16 A fragments of at (transposed reads): block (I, J), J <= I, at I (I + 1) / 2 + J
__device__ __forceinline__ void load_t_frags(const Lds& L, uint2 (&af)[10], int l16, int q4) {
#pragma unroll
  for (int I = 0; I < 4; ++I)
#pragma unroll
    for (int J = 0; J <= I; ++J)
      af[I * (I + 1) / 2 + J] = ld_tr(&L.at[tr(SBT * J + 4 * q4 + (l16 >> 2), SBT * I + 4 * (l16 & 3))]);
}
// X = (I + A)^{-1} Y by block forward substitution, Y and X in the D layout
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
// W = (I + A)^{-1} diag(b) K^ (K^ carries 1 / |k|) for channels 16 t .. 16 t + 15, negated and written
// over the same kr channels (read transposed first; only this wave touches them)
__device__ __forceinline__ void w_tile(Lds& L, bool fast, int t, const uint2 (&af)[10], int l16, int q4) {
  const int tpos = 32 * (t >> 1) + 4 * (t & 1);      // cpos(16 t)
  f32x4 y[4];
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    // lane (l16, q4) receives channel 16 t + l16 of tokens 16 I + 4 q4 + 0..3
    const float4 kv = unpack4(ld_tr(&L.kr[rk(SBT * I + 4 * q4 + (l16 >> 2), tpos + 8 * (l16 & 3))]));
    float sc = 1.f;
    if (!fast) sc = pick(em_of(L, I, 16 * t + (l16 & ~3)), l16 & 3);
    const float4 kr4 = ldf4(&L.beta[SBT * I + 4 * q4]);
    y[I][0] = kv.x * kr4.x * sc; y[I][1] = kv.y * kr4.y * sc;
    y[I][2] = kv.z * kr4.z * sc; y[I][3] = kv.w * kr4.w * sc;
  }
  f32x4 X[4];
  block_solve(af, y, X);
  const int wcol = tpos + 8 * (l16 >> 2) + (l16 & 3);   // cpos(16 t + l16)
#pragma unroll
  for (int I = 0; I < 4; ++I)
#pragma unroll
    for (int r = 0; r < 4; ++r) L.kr[rk(SBT * I + 4 * q4 + r, wcol)] = f2bf(-X[I][r]);
}
// v of channels col0 .. col0 + 31 (vx: lane = tokens 4 (lane >> 2) + j, channels
// col0 + 8 (lane & 3) ..) -> the same channels of qw, which only this wave uses now
__device__ __forceinline__ void stage_v(Lds& L, int col0, const uint4 (&vx)[4], int lane) {
  const int vp = col0 + 16 * (lane & 1) + 4 * ((lane >> 1) & 1);   // cpos(col0 + 8 (lane & 3))
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 4 * (lane >> 2) + j;
    *reinterpret_cast<uint2*>(&L.qw[rm(row, vp)]) = make_uint2(vx[j].x, vx[j].y);
    *reinterpret_cast<uint2*>(&L.qw[rm(row, vp + 8)]) = make_uint2(vx[j].z, vx[j].w);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
}
// U~ = (I + A)^{-1} diag(b) V for the state columns col0 .. col0 + 31 (staged in qw)
__device__ __forceinline__ void u_tiles(const Lds& L, int col0, const uint2 (&af)[10], f32x4 (&Ut)[4][2], int l16,
                                        int q4) {
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int t = col0 / 16 + ct;
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
    block_solve(af, y, X);
#pragma unroll
    for (int I = 0; I < 4; ++I) Ut[I][ct] = X[I];
  }
}
// state as bf16 B operand: slots 0-3 rows 32 s + 4 q4 + r, 4-7 rows 32 s + 16 + 4 q4 + r
__device__ __forceinline__ void pack_state(const f32x4 (&S)[8][2], uint4 (&Sf)[4][2]) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) Sf[s][ct] = pack8(S[2 * s][ct], S[2 * s + 1][ct]);
}
// U += (-W) S (-W in kr)
__device__ __forceinline__ void minus_ws(const Lds& L, const uint4 (&Sf)[4][2], f32x4 (&U)[4][2], int l16, int q4) {
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    uint4 wf[4];
    tile_frags(L.kr, I, wf, l16, q4);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int s = 0; s < 4; ++s) U[I][ct] = mma32(wf[s], Sf[s][ct], U[I][ct]);
  }
}
// S <- Diag(e^{g_n}) S + K~^T U, K~ = (K / |k|) e^{g_n - g} read transposed from kc
__device__ __forceinline__ void update_state(const Lds& L, bool fast, f32x4 (&S)[8][2], const f32x4 (&U)[4][2],
                                             int l16, int q4) {
  uint4 Upf[2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) Upf[s][ct] = pack8(U[2 * s][ct], U[2 * s + 1][ct]);
  // A operand K~^T: lane (l16, q4) = channel 16 rt + l16, tokens 32 s + 4 q4 + 0..3 and
  // 32 s + 16 + 4 q4 + 0..3
  const int kbase = rk(4 * q4 + (l16 >> 2), 8 * (l16 & 3));
#pragma unroll
  for (int rt = 0; rt < 8; ++rt) {
    const int cp = 32 * (rt >> 1) + 4 * (rt & 1);   // cpos(16 rt)
    uint4 kt[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
      kt[s] = cat(ld_tr(&L.kc[kbase + rk(32 * s, cp)]), ld_tr(&L.kc[kbase + rk(32 * s + 16, cp)]));
    const float4 eg = ldf4(&L.egn[16 * rt + 4 * q4]);
    if (fast) {   // K~ = K_ e^{g_n}: the factor is a row scaling of the product
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        f32x4 acc = S[rt][ct];
        acc = mma32(kt[0], Upf[0][ct], acc);
        acc = mma32(kt[1], Upf[1][ct], acc);
        acc[0] *= eg.x; acc[1] *= eg.y; acc[2] *= eg.z; acc[3] *= eg.w;
        S[rt][ct] = acc;
      }
    } else {      // blocked: K~ = K_ e^{g_n - m_I} for the tokens of block I
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
// the 32 state columns of this wave -> m ([D][D] fp32); svo = lane part of the offset
__device__ __forceinline__ void store_state(const f32x4 (&S)[8][2], float* m, int svo) {
  float* dst = m + svo;
#pragma unroll
  for (int rt = 0; rt < 8; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(16 * rt + r) * D + 16 * ct] = S[rt][ct][r];
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
static_assert(offsetof(Lds, kc) == offsetof(Lds, kr) + sizeof(Lds::kr) && 4 * kMsWave <= 2 * CT * RKS,
              "the four M waves' scratch lies in kr and kc");
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

// v of the state columns col0 .. col0 + 31 of the chunk: lane = tokens 4 (lane >> 2) + j,
// channels col0 + 8 (lane & 3) .. + 7; tokens past the end read as zero
__device__ __forceinline__ void load_v(const ChunkArgs& a, int64_t row, int64_t h, int n, int col0, int lane,
                                       uint4 (&vx)[4]) {
  const int st2 = (int)a.stride * 2;
  const auto rv = __builtin_amdgcn_make_buffer_rsrc((void*)(a.v + row * a.stride + h * D), 0, n * st2, kRsrcW3);
  const int vo = (4 * (lane >> 2)) * st2 + 2 * (col0 + 8 * (lane & 3));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const auto v4 = __builtin_amdgcn_raw_buffer_load_b128(rv, vo, j * st2, 0);
    vx[j] = make_uint4(v4[0], v4[1], v4[2], v4[3]);
  }
}

// Output pass over the chunks of one segment of one (batch, head): 4 waves, wave w
// owns state columns 32 w .. 32 w + 31; writes o, and S_final from the last segment.
//
// Per chunk, phases and the barriers after them:
//   loads; E1: norms and block decay products              | B
//   E2/E3: decay factors, operands kr kc qw                 | C
//   M1T: A / Aqk tiles, diagonal inverses, Q^ S; v loads    | D
//   X: block substitution for W (into kr) and U~            | E
//   S: U = U~ - W S, O += Aqk U, state update, o store      | F
//
// Two factorisations of the pairwise decay e^{g_i - g_j} are used:
//  * fast: one reference at the chunk start (K^ = K e^{g}, K_ = K e^{-g}, formed from
//    prefix and suffix products of alpha); valid
//    while every channel decays by less than e^{-80} over the chunk, chosen per
//    chunk by a block-wide vote;
//  * blocked: references at token 7 of each 16-token block, with the factors
//    e^{m_I - m_J}, e^{m_I}, e^{g_n - m_I} applied to fragments as they are
//    read; accurate for every alpha once alpha is raised to e^{-7.5} (kAlphaMin2).
//
// GATED adds the rest of Eq. 15 short of W_o to the output: o <- Sigmoid(gate) *
// o / sqrt(mean over the head's channels of o^2 + eps) * w. Each wave holds 32 of the
// 128 channels of the fp32 output; their per-row sums of squares meet in LDS (adiag)
// behind the chunk's last barrier (F). The output of chunk c is then normalised,
// staged in fp32 over kr and kc (free until the next chunk's operands are formed,
// barrier B) and stored with the gate applied, rounded once, while the loads of chunk
// c + 1 are in flight; the last chunk's after the loop.
constexpr int kStP = 36;   // fp32 output staging pitch (floats per row)
static_assert(offsetof(Lds, kc) == offsetof(Lds, kr) + sizeof(Lds::kr) &&
                  4 * CT * kStP * sizeof(float) <= sizeof(Lds::kr) + sizeof(Lds::kc) &&
                  4 * CT * sizeof(float) <= sizeof(Lds::adiag),
              "gated output staging in kr and kc, row partial sums in adiag");
template <bool GATED>
__global__ __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(2))) void kda_out_kernel(ChunkArgs a) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  Lds& L = *reinterpret_cast<Lds*>(lds_raw);

  const uint32_t lid = (a.xcd_ranges && a.grid % 8 == 0) ? xcd_contiguous_id(blockIdx.x, (uint32_t)a.grid)
                                                         : blockIdx.x;
  if (lid >= (uint32_t)a.nblk) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform
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

  // ---- state: rows 16 rt + 4 q4 + r, columns col0 + 16 ct + l16 -----------------
  const int col0 = 32 * wave;
  const int svo = (4 * q4) * D + col0 + l16;   // lane part of a state element's offset
  f32x4 S[8][2];
  if (sv.P > 1) {
    if (p % kSub == 0) {   // a chain start (tile-major)
      const float* src = sv.ws + (2 * sv.E + p) * D * D;
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) S[rt][ct] = load_tile4(src, wave, rt, ct, lane);
    }
  } else {                 // S0 ([D][D] row-major) or zero
    const float* src = a.S0 ? a.S0 + sv.sidx * D * D : nullptr;
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[rt][ct][r] = src ? src[svo + (16 * rt + r) * D + 16 * ct] : 0.f;
  }
  if (sv.P > 1 && p % kSub != 0) {
    // a start inside a summary segment: S_start(p) = M_e S_start(p - p % kSub) + S_e with
    // e = p - 1, in fp32-accurate MFMA (bf16 high and low parts, three products)
    const int e = p - 1;
    const float* Mp = sv.ws + (sv.E + e) * D * D;
    const float* Sp = sv.ws + e * D * D;
    const float* base = sv.ws + (2 * sv.E + p - p % kSub) * D * D;
    uint4 bH[4][2], bL[4][2];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const f32x4 v0 = load_tile4(base, wave, 2 * s, ct, lane), v1 = load_tile4(base, wave, 2 * s + 1, ct, lane);
        uint2 l0, l1;
        const uint2 h0 = pack_split(make_float4(v0[0], v0[1], v0[2], v0[3]), l0);
        const uint2 h1 = pack_split(make_float4(v1[0], v1[1], v1[2], v1[3]), l1);
        bH[s][ct] = cat(h0, h1);
        bL[s][ct] = cat(l0, l1);
      }
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) {
      uint4 aH[4], aL[4];
      const uint4* Mf = reinterpret_cast<const uint4*>(Mp);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        aH[s] = Mf[mfrag_off(rt, s, lane)];
        aL[s] = Mf[mfrag_off(rt, s, lane) + 1];
      }
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        f32x4 acc0 = load_tile4(Sp, wave, rt, ct, lane), acc1 = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
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
  // the Aqk blocks (0,1) and (2,3) above the diagonal are read as zeros
  for (int e = tid; e < 2 * SBT * SBT; e += NTHR) {
    const int I = (e >> 8) * 2, i = (e >> 4) & 15, j = e & 15;
    L.aqk[tr(SBT * (I + 1) + j, SBT * I + i)] = 0;
  }

  const uint2 kOnes = make_uint2(0x3F803F80u, 0x3F803F80u);   // alpha = 1 past the end
  // GATED: the previous chunk's fp32 output (D layout) and its gate (rows 4 (lane >> 2) + j,
  // channels col0 + 8 (lane & 3) .. + 7), carried into the next chunk step
  f32x4 Og[4][2];
  uint4 gx[4];
  auto gate_epilogue = [&](int64_t cp) {
    int lane_e = lane;
    asm volatile("" : "+v"(lane_e));
    const int e16 = lane_e & 15, e4 = lane_e >> 4;
    const int64_t tp = cp * CT;
    const int np = (int)min<int64_t>(CT, sv.T - tp);
    const int oc = 8 * (lane_e & 3);
    float4 w0 = make_float4(1.f, 1.f, 1.f, 1.f), w1 = w0;   // gain of the lane's output channels
    if (a.norm_w != nullptr) {
      w0 = ldf4(a.norm_w + col0 + oc);
      w1 = ldf4(a.norm_w + col0 + oc + 4);
    }
    float* st = reinterpret_cast<float*>(L.kr) + wave * CT * kStP;
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) st[(16 * I + 4 * e4 + r) * kStP + 16 * ct + e16] = Og[I][ct][r];
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    // rows -> o, scaled by 1 / rms and the gain, with the gate; 16 bytes per lane; rows
    // past the end are dropped
    const int so2 = (int)(a.H * D) * 2;
    const auto ro = __builtin_amdgcn_make_buffer_rsrc((void*)(a.o + ((sv.row0 + tp) * a.H + h) * D), 0, np * so2,
                                                      kRsrcW3);
    auto sig = [](float g) { return __builtin_amdgcn_rcpf(1.f + __expf(-g)); };
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 4 * (lane_e >> 2) + j;
      const float4 p4 = ldf4(&L.adiag[row * 4]);
      const float rinv = __builtin_amdgcn_rsqf((p4.x + p4.y + p4.z + p4.w) * (1.f / D) + a.norm_eps);
      const float4 y0 = mul4(ldf4(&st[row * kStP + oc]), w0), y1 = mul4(ldf4(&st[row * kStP + oc + 4]), w1);
      const float4 g0 = unpack4(make_uint2(gx[j].x, gx[j].y)), g1 = unpack4(make_uint2(gx[j].z, gx[j].w));
      typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
      const u32x4_t w4 = {pack_bf16x2(y0.x * rinv * sig(g0.x), y0.y * rinv * sig(g0.y)),
                          pack_bf16x2(y0.z * rinv * sig(g0.z), y0.w * rinv * sig(g0.w)),
                          pack_bf16x2(y1.x * rinv * sig(g1.x), y1.y * rinv * sig(g1.y)),
                          pack_bf16x2(y1.z * rinv * sig(g1.z), y1.w * rinv * sig(g1.w))};
      __builtin_amdgcn_raw_buffer_store_b128(w4, ro, row * so2 + 2 * (col0 + oc), 0, 0);
    }
  };

  for (int64_t c = c_begin; c < c_end; ++c) {
    // Lane-derived addresses are recomputed every chunk (cheap) rather than kept live
    // across the loop: the lane id passes through an empty asm so that they cannot be
    // hoisted out of it.
    int lane_c = lane;
    asm volatile("" : "+v"(lane_c));
    const int l16 = lane_c & 15, q4 = lane_c >> 4;
    // elementwise mapping: wave = decay block; half-wave hf = tokens 8 hf .. 8 hf + 7
    // of the block; lane cg = channels 4 cg .. 4 cg + 3
    const int hf = lane_c >> 5, cg = lane_c & 31, c0 = 4 * cg, p0 = cpos(c0);
    const int tk0 = SBT * wave + 8 * hf;
    const int64_t t0 = c * CT;
    const int n = (int)min<int64_t>(CT, sv.T - t0);

    // ---- loads ----------------------------------------------------------------------
    // Buffer loads: block-uniform base and bounds (the chunk's first n tokens), byte
    // offsets split into a lane part and a uniform part. Reads past the bound return
    // zero, which is k = q = v = beta = 0 for tokens past the end; alpha is set to 1.
    uint2 kx[8], qx[8], ax[8];
    float bt;
    {
      const int64_t row0 = sv.row0 + t0;
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
        qx[i] = ld_buf64(rq_, vk, (tb + i) * st2);
        const uint2 av = ld_buf64(ra_, va, (tb + i) * sa2);
        ax[i] = tk0 + i < n ? av : kOnes;
      }
      bt = bf2f(__builtin_amdgcn_raw_buffer_load_b16(rb_, tid * (int)a.H * 2, 0, 0));
    }
    if (GATED && c > c_begin) gate_epilogue(c - 1);   // the previous chunk's output, while the loads fly

    // ---- E1: norms, block decay products -------------------------------------------
    if (tid < CT) L.beta[tid] = bt;
    if (a.l2norm) {
      float ss[16];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ss[i] = dot4(kx[i]);
        ss[i + 8] = dot4(qx[i]);
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
    float4 al[8];   // alpha of the lane's tokens
#pragma unroll
    for (int i = 0; i < 8; ++i) al[i] = unpack4(make_uint2(clamp_alpha2(ax[i].x), clamp_alpha2(ax[i].y)));
    {
      float4 hp = al[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) hp = mul4(hp, al[i]);
      *reinterpret_cast<float4*>(hf ? &L.pf[wave][c0] : &L.pb[wave][c0]) = hp;
    }
    lds_barrier();   // B

    // ---- E2 / E3: decay factors and MFMA operands --------------------------------------
    bool fast;
    {
      // per channel: before = decay over the blocks before this one, after = over the
      // blocks after it; the lane's half adds its block's other half on one side
      float4 full[NSB], h0w = make_float4(1.f, 1.f, 1.f, 1.f), h1w = h0w;
#pragma unroll
      for (int J = 0; J < NSB; ++J) {
        const float4 h0 = ldf4(&L.pb[J][c0]), h1 = ldf4(&L.pf[J][c0]);
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
      // every wave holds all 128 channels, so every wave reaches the same vote
      fast = __all(fminf(fminf(egn4.x, egn4.y), fminf(egn4.z, egn4.w)) >= kFastMin) != 0;
      if (wave == 0 && hf == 0) *reinterpret_cast<float4*>(&L.egn[c0]) = egn4;
      // 1 / |k| and 1 / |q| of the lane's tokens (from E1) go into the operands, so that
      // no product downstream needs a norm scaling
      const float4 rk0 = ldf4(&L.rk[tk0]), rk1 = ldf4(&L.rk[tk0 + 4]);
      const float4 rq0 = ldf4(&L.rq[tk0]), rq1 = ldf4(&L.rq[tk0 + 4]);
      const float rkt[8] = {rk0.x, rk0.y, rk0.z, rk0.w, rk1.x, rk1.y, rk1.z, rk1.w};
      const float rqt[8] = {rq0.x, rq0.y, rq0.z, rq0.w, rq1.x, rq1.y, rq1.z, rq1.w};
      auto put = [&](int i, float4 fr, float4 fc) {
        const int tk = tk0 + i;
        const float4 ks = mul4(unpack4(kx[i]), make_float4(rkt[i], rkt[i], rkt[i], rkt[i]));
        const float4 qs = mul4(unpack4(qx[i]), make_float4(rqt[i], rqt[i], rqt[i], rqt[i]));
        *reinterpret_cast<uint2*>(&L.kr[rk(tk, p0)]) = pack4(mul4(ks, fr));
        *reinterpret_cast<uint2*>(&L.kc[rk(tk, p0)]) = pack4(mul4(ks, fc));
        *reinterpret_cast<uint2*>(&L.qw[rm(tk, p0)]) = pack4(mul4(qs, fr));
      };
      if (fast) {
        // e^{g_t} as a prefix product from the chunk start and e^{g_n - g_t} / e^{g_n} as a
        // suffix product towards the chunk end: no per-element reciprocal, and the same
        // instruction stream in both half-waves
        const float4 one4 = make_float4(1.f, 1.f, 1.f, 1.f);
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
        (void)one4;
      } else {
        // blocked: reference m_I = g at the block's token 7; half 1 runs forward
        // (e^{g - m_I} = product over tokens 8..t), half 0 backward (e^{m_I - g} =
        // product over tokens t+1..7)
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
    }
    lds_barrier();   // C

    // ---- M1T: A and Aqk blocks, diagonal inverses, Q^ S ---------------------------------
    f32x4 O[4][2];
    uint4 vx[4];
    {
      uint4 cA[4], cB[4], rA[4], sc[4];
      // wave 0: the four diagonal A blocks and their inverses;
      // wave 1: Aqk00 A10 Aqk10 A20 Aqk20 A30;  wave 2: Aqk11 A21 Aqk21 A31 Aqk31;
      // wave 3: Aqk22 A32 Aqk32 Aqk33 Aqk30
      if (wave == 0) {
        __builtin_amdgcn_s_setprio(3);   // the chunk's critical path
#pragma unroll
        for (int I = 0; I < NSB; ++I) {
          tile_frags(L.kc, I, cA, l16, q4);
          tile_frags(L.kr, I, rA, l16, q4);
          epi_a(L, I, I, mma4(rA, cA), l16, q4);
        }
        invert_diag4(L, lane_c);
        __builtin_amdgcn_s_setprio(0);
      } else if (wave == 1) {
        tile_frags(L.kc, 0, cA, l16, q4);
        tile_frags<RMS>(L.qw, 0, rA, l16, q4); epi_q(L, 0, 0, mma4(rA, cA), l16, q4);
#pragma unroll
        for (int I = 1; I < NSB; ++I) {
          pair_frags(L, fast, I, 0, cA, sc, q4);
          tile_frags(L.kr, I, rA, l16, q4); epi_a(L, I, 0, mma4(rA, sc), l16, q4);
          if (I < 3) { tile_frags<RMS>(L.qw, I, rA, l16, q4); epi_q(L, I, 0, mma4(rA, sc), l16, q4); }
        }
      } else if (wave == 2) {
        tile_frags(L.kc, 1, cA, l16, q4);
        tile_frags<RMS>(L.qw, 1, rA, l16, q4); epi_q(L, 1, 1, mma4(rA, cA), l16, q4);
#pragma unroll
        for (int I = 2; I < NSB; ++I) {
          pair_frags(L, fast, I, 1, cA, sc, q4);
          tile_frags(L.kr, I, rA, l16, q4); epi_a(L, I, 1, mma4(rA, sc), l16, q4);
          tile_frags<RMS>(L.qw, I, rA, l16, q4); epi_q(L, I, 1, mma4(rA, sc), l16, q4);
        }
      } else {
        tile_frags(L.kc, 2, cA, l16, q4);
        tile_frags<RMS>(L.qw, 2, rA, l16, q4); epi_q(L, 2, 2, mma4(rA, cA), l16, q4);
        pair_frags(L, fast, 3, 2, cA, sc, q4);
        tile_frags(L.kr, 3, rA, l16, q4); epi_a(L, 3, 2, mma4(rA, sc), l16, q4);
        tile_frags<RMS>(L.qw, 3, rA, l16, q4); epi_q(L, 3, 2, mma4(rA, sc), l16, q4);
        tile_frags(L.kc, 3, cB, l16, q4); epi_q(L, 3, 3, mma4(rA, cB), l16, q4);
        tile_frags(L.kc, 0, cB, l16, q4); pair_frags(L, fast, 3, 0, cB, sc, q4);
        epi_q(L, 3, 0, mma4(rA, sc), l16, q4);
      }
      // O = Q^ S (Q^ carries 1 / |q|); the blocked factorisation scales Q^'s channels by e^{m_I}
      uint4 Sf[4][2];
      pack_state(S, Sf);
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        uint4 qf[4];
        tile_frags<RMS>(L.qw, I, qf, l16, q4);
        if (!fast) {
#pragma unroll
          for (int s = 0; s < 4; ++s)
            qf[s] = scale8(qf[s], em_of(L, I, 32 * s + 4 * q4), em_of(L, I, 32 * s + 16 + 4 * q4));
        }
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 4; ++s) acc = mma32(qf[s], Sf[s][ct], acc);
          O[I][ct] = acc;
        }
      }
      load_v(a, sv.row0 + t0, h, n, col0, lane_c, vx);
    }
    lds_barrier();   // D

    // ---- X: block substitution X = (I + A)^{-1} diag(sigma) R --------------------------
    // right-hand sides: K^ channel tiles 2 wave, 2 wave + 1 (W, negated, into kr) and
    // this wave's v columns (U~, kept in registers)
    f32x4 Ut[4][2];
    {
      stage_v(L, col0, vx, lane_c);   // first: v (loaded during M1T) leaves the registers
      uint2 af[10];
      load_t_frags(L, af, l16, q4);
      w_tile(L, fast, 2 * wave, af, l16, q4);
      w_tile(L, fast, 2 * wave + 1, af, l16, q4);
      u_tiles(L, col0, af, Ut, l16, q4);
    }
    lds_barrier();   // E

    // ---- S: U = U~ - W S;  O += Aqk U;  S <- Diag(e^{g_n}) S + K~^T diag(1/|k|) U ----------
    {
      uint4 Sf[4][2];
      pack_state(S, Sf);
      minus_ws(L, Sf, Ut, l16, q4);
    }
    {
      uint4 Uf[2][2], qa[6];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) Uf[s][ct] = pack8(Ut[2 * s][ct], Ut[2 * s + 1][ct]);
      // A operand rows 16 I + l16, tokens 32 s + 4 q4 + 0..3 and 32 s + 16 + 4 q4 + 0..3
      auto qfrag = [&](int I, int s) {
        const int base = tr(32 * s + 4 * q4 + (l16 >> 2), SBT * I + 4 * (l16 & 3));
        return cat(ld_tr(&L.aqk[base]), ld_tr(&L.aqk[base + tr(16, 0)]));
      };
      qa[0] = qfrag(0, 0);
      qa[1] = qfrag(1, 0);
      qa[2] = qfrag(2, 0);
      qa[3] = qfrag(2, 1);
      qa[4] = qfrag(3, 0);
      qa[5] = qfrag(3, 1);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        O[0][ct] = mma32(qa[0], Uf[0][ct], O[0][ct]);
        O[1][ct] = mma32(qa[1], Uf[0][ct], O[1][ct]);
        O[2][ct] = mma32(qa[2], Uf[0][ct], O[2][ct]);
        O[2][ct] = mma32(qa[3], Uf[1][ct], O[2][ct]);
        O[3][ct] = mma32(qa[4], Uf[0][ct], O[3][ct]);
        O[3][ct] = mma32(qa[5], Uf[1][ct], O[3][ct]);
      }
      if (!GATED) {
        // output tile -> this wave's channels of qw (natural order; v is consumed)
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
          for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) L.qw[rm(SBT * I + 4 * q4 + r, col0 + 16 * ct + l16)] = f2bf(O[I][ct][r]);
      }
    }
    if (GATED) {
      const int sg2 = (int)a.gate_stride * 2;
      const auto rg = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.gate + (sv.row0 + t0) * a.gate_stride + h * D), 0, n * sg2, kRsrcW3);
      const int gc = col0 + 8 * (lane_c & 3);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const auto g4 = __builtin_amdgcn_raw_buffer_load_b128(rg, (4 * (lane_c >> 2) + j) * sg2 + 2 * gc, 0, 0);
        gx[j] = make_uint4(g4[0], g4[1], g4[2], g4[3]);
      }
      // this wave's part of each row's sum of squares: lane l16 of a DPP row ends with row
      // 16 (l16 >> 2) + 4 q4 + (l16 & 3); adiag is free after the inverses
      float ss[16];
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int r = 0; r < 4; ++r) ss[4 * I + r] = O[I][0][r] * O[I][0][r] + O[I][1][r] * O[I][1][r];
      const float part = row_sum16(ss, l16);
      L.adiag[(16 * (l16 >> 2) + 4 * q4 + (l16 & 3)) * 4 + wave] = part;
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) Og[I][ct] = O[I][ct];
    }
    update_state(L, fast, S, Ut, l16, q4);
    if (!GATED) {
      // staged output rows -> o, 16 bytes per lane; rows past the end fall outside the
      // buffer bound and are dropped
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      const int so2 = (int)(a.H * D) * 2;
      const auto ro = __builtin_amdgcn_make_buffer_rsrc((void*)(a.o + ((sv.row0 + t0) * a.H + h) * D), 0, n * so2,
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
  }
  if (GATED && c_end > c_begin) gate_epilogue(c_end - 1);

  if (a.S_final != nullptr && p == sv.P - 1) store_state(S, a.S_final + sv.sidx * D * D, svo);
}

// Summary pass: one block of 8 waves per (batch, head, summary segment). Waves 0-3 run
// S from 0 (state columns 32 w ..), waves 4-7 the transition M from I (columns
// 32 (w - 4) ..); the chunk operands, A, T and W are formed once for both. The state
// is written at every output-segment boundary (every Lo chunks).
//
// Per chunk, phases and the barriers after them:
//   loads; E1: partial norms, block decay products            | B
//   E2/E3: norms, decay factors, operands kr kc; v loads       | C
//   M1T: A blocks, diagonal inverses                           | D
//   X: W (channel tile w, into kr); U~ (waves 0-3)             | E
//   S: U = U~ - W S (or -W M), state update                    | F
__global__ __launch_bounds__(2 * NTHR) __attribute__((amdgpu_waves_per_eu(2))) void kda_sum_kernel(ChunkArgs a) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  Lds& L = *reinterpret_cast<Lds*>(lds_raw);
  float (&nk)[2][CT] = *reinterpret_cast<float(*)[2][CT]>(lds_raw + sizeof(Lds));   // partial |k|^2

  const uint32_t lid = (a.xcd_ranges && a.grid % 8 == 0) ? xcd_contiguous_id(blockIdx.x, (uint32_t)a.grid)
                                                         : blockIdx.x;
  if (lid >= (uint32_t)a.nblk) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform
  const bool mkind = wave >= 4;
  const int l16 = lane & 15, q4 = lane >> 4;
  const SeqDesc& rd = a.run[run_of<1>(a, lid)];
  const int32_t local = (int32_t)lid - rd.sum0;
  const int p = uni(local % rd.Ps);
  const int32_t bhl = uni(local / rd.Ps);
  const SeqView sv = seq_view(a, rd, bhl);
  const int64_t h = uni(bhl % (int32_t)a.H);
  const int64_t NC = (sv.T + CT - 1) / CT;
  const int64_t Ls = (int64_t)kSub * a.Lo;            // chunks per summary segment
  const int64_t c_stop = (int64_t)(sv.P - 1) * a.Lo;  // the last output segment needs no summary
  const int64_t c_begin = (int64_t)p * Ls;
  const int64_t c_end = min<int64_t>(min<int64_t>(NC, c_begin + Ls), c_stop);

  const int col0 = 32 * (wave & 3);
  f32x4 S[8][2];
#pragma unroll
  for (int rt = 0; rt < 8; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * rt + 4 * q4 + r, col = col0 + 16 * ct + l16;
        S[rt][ct][r] = (mkind && row == col) ? 1.f : 0.f;
      }

  const uint32_t kOne = 0x3F803F80u;   // alpha = 1 past the end
  // Raw inputs of one chunk for this lane: k and alpha of tokens tk0 .. tk0 + 7 at
  // channels c0, c0 + 1, beta of token (tid & 63).
  // Buffer loads bounded by the chunk's valid tokens (zero past the end). The next
  // chunk's loads are issued during the state update of the current one.
  struct Raw {
    uint32_t k[8], a[8];
    uint16_t bt;
  };
  auto issue = [&](int64_t c, Raw& R, int lane_c) {
    const int I = wave & 3, hc = wave >> 2;
    const int hf = lane_c >> 5, c0 = 64 * hc + 2 * (lane_c & 31);
    const int64_t t0 = c * CT;
    const int n = (int)min<int64_t>(CT, sv.T - t0);
    const int64_t row0 = sv.row0 + t0;
    const int st2 = (int)a.stride * 2, sa2 = (int)(a.H * D) * 2;
    const auto rk_ = __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + row0 * a.stride + h * D), 0, n * st2, kRsrcW3);
    const auto ra_ = __builtin_amdgcn_make_buffer_rsrc((void*)(a.alpha + (row0 * a.H + h) * D), 0, n * sa2, kRsrcW3);
    const auto rb_ = __builtin_amdgcn_make_buffer_rsrc((void*)(a.beta + row0 * a.H + h), 0, n * (int)a.H * 2, kRsrcW3);
    const int vk = (8 * hf) * st2 + 2 * c0, va = (8 * hf) * sa2 + 2 * c0;
    const int tb = SBT * I;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      R.k[i] = __builtin_amdgcn_raw_buffer_load_b32(rk_, vk, (tb + i) * st2, 0);
      R.a[i] = __builtin_amdgcn_raw_buffer_load_b32(ra_, va, (tb + i) * sa2, 0);
    }
    R.bt = __builtin_amdgcn_raw_buffer_load_b16(rb_, (lane_c & 63) * (int)a.H * 2, 0, 0);
  };
  Raw nxt;
  if (c_begin < c_end) issue(c_begin, nxt, lane);
  int to_boundary = a.Lo;    // chunks left to the next output-segment boundary
  int e_next = p * kSub;     // its workspace entry

  for (int64_t c = c_begin; c < c_end; ++c) {
    int lane_c = lane;
    asm volatile("" : "+v"(lane_c));
    const int l16 = lane_c & 15, q4 = lane_c >> 4;
    // elementwise mapping: wave -> decay block I = wave & 3 and channel half hc;
    // half-wave hf = tokens 8 hf .. 8 hf + 7 of the block; lane cg = channels c0, c0 + 1
    const int I = wave & 3, hc = wave >> 2;
    const int hf = lane_c >> 5, cg = lane_c & 31, c0 = 64 * hc + 2 * cg, p0 = cpos(c0);
    const int tk0 = SBT * I + 8 * hf;
    const int64_t t0 = c * CT;
    const int n = (int)min<int64_t>(CT, sv.T - t0);

    const Raw cur = nxt;
    uint32_t kx[8], ax[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      kx[i] = cur.k[i];
      ax[i] = tk0 + i < n ? cur.a[i] : kOne;
    }
    const float bt = bf2f(cur.bt);

    // ---- E1: partial norms, block decay products ---------------------------------------
    if (tid < CT) L.beta[tid] = bt;
    if (a.l2norm) {
      float ss[16];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ss[i] = sq2(kx[i], 0.f);
        ss[i + 8] = 0.f;
      }
      const float tot = half_sum16(ss, lane_c);
      const int vv = (lane_c >> 1) & 15;
      if ((lane_c & 1) == 0 && vv < 8) nk[hc][tk0 + vv] = tot;
    }
    float2 al[8];   // alpha of the lane's tokens
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t ac = clamp_alpha2(ax[i]);
      al[i] = make_float2(bf_lo(ac), bf_hi(ac));
    }
    {
      float2 hp = al[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) { hp.x *= al[i].x; hp.y *= al[i].y; }
      *reinterpret_cast<float2*>(hf ? &L.pf[I][c0] : &L.pb[I][c0]) = hp;
    }
    lds_barrier();   // B

    // ---- E2 / E3: norms, decay factors, MFMA operands ---------------------------------
    bool fast;
    {
      float2 full[NSB];
      float2 h0w = make_float2(1.f, 1.f), h1w = h0w, eo = h0w;
#pragma unroll
      for (int J = 0; J < NSB; ++J) {
        const float2 h0 = *reinterpret_cast<const float2*>(&L.pb[J][c0]);
        const float2 h1 = *reinterpret_cast<const float2*>(&L.pf[J][c0]);
        full[J] = make_float2(h0.x * h1.x, h0.y * h1.y);
        if (J == I) { h0w = h0; h1w = h1; }
        // the other channel half, formed the same way, so that every wave votes alike
        const float2 h0o = *reinterpret_cast<const float2*>(&L.pb[J][c0 ^ 64]);
        const float2 h1o = *reinterpret_cast<const float2*>(&L.pf[J][c0 ^ 64]);
        const float2 fo = make_float2(h0o.x * h1o.x, h0o.y * h1o.y);
        eo = J == 0 ? fo : make_float2(eo.x * fo.x, eo.y * fo.y);
      }
      float2 egn2 = full[0], before = make_float2(1.f, 1.f), after = before;
#pragma unroll
      for (int J = 1; J < NSB; ++J) { egn2.x *= full[J].x; egn2.y *= full[J].y; }
#pragma unroll
      for (int J = 0; J < NSB; ++J) {
        if (J < I) { before.x *= full[J].x; before.y *= full[J].y; }
        if (J > I) { after.x *= full[J].x; after.y *= full[J].y; }
      }
      fast = __all(fminf(fminf(egn2.x, egn2.y), fminf(eo.x, eo.y)) >= kFastMin) != 0;
      if (I == 0 && hf == 0) *reinterpret_cast<float2*>(&L.egn[c0]) = egn2;
      // 1 / |k| of the lane's tokens from the two channel halves' partial sums (E1),
      // folded into the operands
      float rkt[8];
      if (a.l2norm) {
        const float4 a0 = ldf4(&nk[0][tk0]), a1 = ldf4(&nk[0][tk0 + 4]);
        const float4 b0 = ldf4(&nk[1][tk0]), b1 = ldf4(&nk[1][tk0 + 4]);
        const float ss[8] = {a0.x + b0.x, a0.y + b0.y, a0.z + b0.z, a0.w + b0.w,
                             a1.x + b1.x, a1.y + b1.y, a1.z + b1.z, a1.w + b1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) rkt[i] = __builtin_amdgcn_rsqf(ss[i] + kL2Eps);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) rkt[i] = 1.f;
      }
      auto put = [&](int i, float fr0, float fr1, float fc0, float fc1) {
        const int tk = tk0 + i;
        const float k0 = bf_lo(kx[i]) * rkt[i], k1 = bf_hi(kx[i]) * rkt[i];
        *reinterpret_cast<uint32_t*>(&L.kr[rk(tk, p0)]) = pack_bf16x2(k0 * fr0, k1 * fr1);
        *reinterpret_cast<uint32_t*>(&L.kc[rk(tk, p0)]) = pack_bf16x2(k0 * fc0, k1 * fc1);
      };
      if (fast) {
        // prefix products e^{g_t}, suffix products e^{g_n - g_t} / e^{g_n}
        float f0 = before.x * (hf ? h0w.x : 1.f), f1 = before.y * (hf ? h0w.y : 1.f);
        float b0 = (after.x * (hf ? 1.f : h1w.x)) * __builtin_amdgcn_rcpf(egn2.x);
        float b1 = (after.y * (hf ? 1.f : h1w.y)) * __builtin_amdgcn_rcpf(egn2.y);
        float fr0[8], fr1[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          f0 *= al[i].x; f1 *= al[i].y;
          fr0[i] = f0; fr1[i] = f1;
        }
#pragma unroll
        for (int i = 7; i >= 0; --i) {
          put(i, fr0[i], fr1[i], b0, b1);
          if (i > 0) { b0 *= al[i].x; b1 *= al[i].y; }
        }
      } else {
        // blocked: reference m_I = g at the block's token 7
        float r0 = 1.f, r1 = 1.f;
        if (hf == 1) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            r0 *= al[i].x; r1 *= al[i].y;
            put(i, r0, r1, __builtin_amdgcn_rcpf(r0), __builtin_amdgcn_rcpf(r1));
          }
        } else {
#pragma unroll
          for (int i = 7; i >= 0; --i) {
            put(i, __builtin_amdgcn_rcpf(r0), __builtin_amdgcn_rcpf(r1), r0, r1);
            r0 *= al[i].x; r1 *= al[i].y;
          }
        }
      }
    }
    uint4 vx[4];
    if (!mkind) load_v(a, sv.row0 + t0, h, n, col0, lane_c, vx);
    lds_barrier();   // C

    // ---- M1T: A blocks, diagonal inverses ------------------------------------------------
    {
      uint4 cA[4], rA[4], sc[4];
      // waves 4-7: diagonal block I = wave - 4 and its inverse; waves 0-3: the blocks below
      // the diagonal (wave 0: A10 A32, wave 1: A20, wave 2: A30 A21, wave 3: A31)
      if (wave >= 4) {
        const int I = wave - 4;
        tile_frags(L.kc, I, cA, l16, q4);
        tile_frags(L.kr, I, rA, l16, q4);
        __builtin_amdgcn_s_setprio(3);
        epi_a(L, I, I, mma4(rA, cA), l16, q4);
        invert_diag(L, I, l16, q4 == 0);
        __builtin_amdgcn_s_setprio(0);
      } else {
        auto below = [&](int I, int J) {
          tile_frags(L.kc, J, cA, l16, q4);
          pair_frags(L, fast, I, J, cA, sc, q4);
          tile_frags(L.kr, I, rA, l16, q4);
          epi_a(L, I, J, mma4(rA, sc), l16, q4);
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
    }
    lds_barrier();   // D

    // ---- X: W channel tile w (into kr); U~ for the S columns ----------------------------
    f32x4 Ut[4][2];
    {
      uint2 af[10];
      load_t_frags(L, af, l16, q4);
      w_tile(L, fast, wave, af, l16, q4);
      if (!mkind) {
        stage_v(L, col0, vx, lane_c);
        u_tiles(L, col0, af, Ut, l16, q4);
      } else {
#pragma unroll
        for (int I2 = 0; I2 < 4; ++I2)
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) Ut[I2][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    lds_barrier();   // E

    // ---- S: U = U~ - W S (M: U = -W M), state update ------------------------------------
    if (c + 1 < c_end) issue(c + 1, nxt, lane_c);
    {
      uint4 Sf[4][2];
      pack_state(S, Sf);
      minus_ws(L, Sf, Ut, l16, q4);
    }
    update_state(L, fast, S, Ut, l16, q4);
    lds_barrier();   // F

    if (--to_boundary == 0) {
      to_boundary = a.Lo;
      const int e = e_next++;   // the entry of this output-segment boundary
      // M: the chunk's kr and kc are free until the next chunk's barrier B
      if (mkind)
        store_mfrag(S, reinterpret_cast<uint4*>(sv.ws + (sv.E + e) * D * D), wave & 3, lane_c,
                    L.kr + (wave - 4) * kMsWave);
      else
        store_tiles(S, sv.ws + e * D * D, wave & 3, lane_c);
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
  const float* S0 = a.S0 ? a.S0 + sv.sidx * D * D : nullptr;
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, q4 = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = 16 * slice + l16;
  const int row0 = 16 * wave + 4 * q4;       // D-layout rows of this lane: row0 .. row0 + 3

  f32x4 cur;
#pragma unroll
  for (int r = 0; r < 4; ++r) cur[r] = S0 ? S0[(row0 + r) * D + col] : 0.f;
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
// (two per CU, about kTargetBlocks at once): the longest block or the total work spread over
// the chip, whichever is larger; a summary block (one per CU, about 0.55 of an output block's
// time per chunk) covers up to kSub * Lo chunks. For a batch of equal sequences the smallest
// Lo that gives about kTargetBlocks output blocks is always best; for packed samples of mixed
// lengths a shorter Lo can spread the few long samples' summaries over more blocks.
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
  return std::max(max_out, w_out / kTargetBlocks) + 0.55 * std::max(max_sum, w_sum / (kTargetBlocks / 2));
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

}  // namespace

bool kda_chunked_supported(const KdaArgs& a) {
  // 8-byte loads of q, k and alpha: token stride a multiple of 4 elements, 8-byte aligned bases
  const uintptr_t al = reinterpret_cast<uintptr_t>(a.q) | reinterpret_cast<uintptr_t>(a.k) |
                       reinterpret_cast<uintptr_t>(a.alpha);
  return a.bf16 && a.dk == D && a.dv == D && a.qkv_stride % 4 == 0 && a.qkv_stride <= (int64_t(1) << 24) &&
         (al & 7) == 0;
}

bool kda_chunked_plan_ok(const KdaRun* runs, int64_t nruns, int64_t H, bool no_split) {
  const Plan pl = make_plan(runs, nruns, H, no_split);
  for (size_t r0 = 0; r0 < pl.desc.size(); r0 += kMaxRuns) {
    const SetBlocks b = set_blocks(pl, r0, std::min(pl.desc.size(), r0 + (size_t)kMaxRuns), H);
    if (b.out > 0x7fffff00 || b.sum > 0x7fffff00 || b.comb > 0x7fffff00) return false;
  }
  return true;
}

size_t kda_chunked_workspace(const KdaRun* runs, int64_t nruns, int64_t H, bool no_split) {
  return (size_t)make_plan(runs, nruns, H, no_split).ws_mats * D * D * sizeof(float);
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
  const bool fuse_gate = gated && x.gate_stride % 8 == 0 && (reinterpret_cast<uintptr_t>(x.gate) & 15) == 0 &&
                         (reinterpret_cast<uintptr_t>(x.norm_w) & 15) == 0 && x.gate_stride <= (int64_t(1) << 24);
  a.gate = static_cast<const uint16_t*>(x.gate);
  a.gate_stride = x.gate_stride;
  a.norm_w = x.norm_w;
  a.norm_eps = x.norm_eps;
  a.H = x.H;
  a.Lo = pl.Lo;
  a.l2norm = x.l2norm ? 1 : 0;
  a.xcd_ranges = pl.desc.size() == 1 ? 1 : 0;   // blocks of unequal length: the hardware's round robin
  const size_t lds = sizeof(Lds), lds_sum = sizeof(Lds) + 2 * CT * sizeof(float);
  int dev = 0;
  hipError_t de = hipGetDevice(&dev);
  if (de != hipSuccess) return de;
  // The LDS attribute is set once per device; the flag is atomic so that host threads calling
  // at once on one device race on nothing (setting it twice is harmless).
  static std::atomic<bool> attr_done[64];
  if (dev < 0 || dev >= 64 || !attr_done[dev].load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kda_out_kernel<false>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kda_out_kernel<true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kda_sum_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds_sum);
    if (e != hipSuccess) return e;
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
      hipLaunchKernelGGL(kda_sum_kernel, dim3((unsigned)s.grid), dim3(2 * NTHR), lds_sum, stream, s);
      hipError_t e = hipGetLastError();
      if (e == hipSuccess) e = mark_after(marks, "kda_sum_kernel", stream);
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
    if (fuse_gate)
      hipLaunchKernelGGL(kda_out_kernel<true>, dim3((unsigned)a.grid), dim3(NTHR), lds, stream, a);
    else
      hipLaunchKernelGGL(kda_out_kernel<false>, dim3((unsigned)a.grid), dim3(NTHR), lds, stream, a);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = mark_after(marks, fuse_gate ? "kda_out_gated_kernel" : "kda_out_kernel", stream);
    if (e != hipSuccess) return e;
  }
  return gated && !fuse_gate ? launch_kda_gate_norm(x, stream, marks) : hipSuccess;
}

}  // namespace chm
