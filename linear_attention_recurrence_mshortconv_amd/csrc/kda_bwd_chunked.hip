// Chunked KDA backward on gfx950 MFMA (bf16 operands, fp32 states and accumulation),
// dk = dv = 128.
//
// The recurrence is Eq. 14 of Chimera page 1, section 3.3 (page 2's parentheses),
// S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T, read out as o_t = S_t^T q_t
// (Eq. 15, inner term), on the L2-normalised q and k (page 1, Fig. 2). Over a chunk of 16
// tokens, with g_t = sum_{s<=t} log a_s per key channel (restarting every chunk), m = g_7,
// the incoming state S and the chunk's operands
//   K^ = k e^{g}, Q^ = q e^{g}, K_ = k e^{g_n - g}, Kr = k e^{g - m}, Kc = k e^{m - g}, Qr = q e^{g - m}
// (rows = tokens; the normalisations folded in), A = strict_lower(Kr Kc^T),
// Aq = lower(Qr Kc^T) (diagonal included) and T = (I + diag(b) A)^{-1}, the forward step is
//   R = V - K^ S,  U = T diag(b) R,  O = Q^ S + Aq U,  S' = Diag(e^{g_n}) S + K_^T U.
// Its reverse, from dO and dS' (the gradient at the chunk's end), is
//   dU = Aq^T dO + K_ dS',  Y = T^T dU,  dR = diag(b) Y = dV,
//   dS = Q^^T dO + Diag(e^{g_n}) dS' - K^^T dR                (carried to the chunk before)
//   dQ^ = dO S^T,  dK^ = -dR S^T,  dK_ = U dS'^T,  dAq = lower(dO U^T),
//   H = strict_lower(Y U^T),  dA = -diag(b) H,  db = rowsum(Y o R) - rowsum(A o H),
//   dQr = dAq Kc,  dKr = dA Kc,  dKc = dAq^T Qr + dA^T Kr,
// and per element, each operand X = x e^{f} giving dx += dX e^{f} and df += dX o X:
//   dq = dQ^ e^{g} + dQr e^{g-m},  dk = dK^ e^{g} + dK_ e^{g_n-g} + dKr e^{g-m} + dKc e^{m-g},
//   dg = dQ^ o Q^ + dQr o Qr + dK^ o K^ - dK_ o K_ + dKr o Kr - dKc o Kc, and at the chunk's
//   last token also sum_t dK_ o K_ + e^{g_n} rowsum(S o dS'); then dlog a_s = sum_{t>=s} dg_t,
//   da = dlog a / a. (m cancels from every product, so the reference point carries no
//   gradient.) The L2 normalisation's backward closes it: dx = (dx^ - x^ (x^ . dx^)) / |x|.
// With a >= e^{-7.5} (the clamp of the forward kernels), every factor over the 8 tokens on
// either side of m stays within e^{+-60}; e^{g} and e^{g_n - g} only shrink, and where they
// underflow the true terms are below fp32 range as well.
//
// Work layout. A block of 8 waves runs one segment of 16-token chunks of one (sequence,
// head); wave w holds state columns 16 w .. 16 w + 15 in registers (the MFMA D layout:
// rows 16 rt + 4 q4 + r, column 16 w + l16) and, for the per-channel gradients, the 16
// channels at row positions 16 w .. 16 w + 15. Operands live in LDS once, rows = tokens,
// channels in the cpos order, so that a 16-byte read returns the K order of a state
// fragment packed from the D layout; products over tokens read them with the transposing
// LDS read. Passes (each sequence cut into segments that run at once):
//   kda_bwd_fwd_kernel<kSum>:  per segment, the end state from zero (L) and from the
//                              identity with v = 0 (the transition product M);
//   chain (fp32):              the start state of every segment, S_{p+1} = M_p S_p + L_p;
//   kda_bwd_fwd_kernel<kCkpt>: per segment from its start state, the state before every
//                              chunk, stored as bf16 MFMA fragments;
//   kda_bwd_grad_kernel<true>: per segment, dS at its start from dS' = 0 at its end (E);
//   chain (fp32):              dS at every segment end, G_{p-1} = M_p^T G_p + E_p;
//   kda_bwd_grad_kernel<false>: the gradients, each segment walked backwards from its G.
#include <algorithm>
#include <atomic>
#include <type_traits>
#include <utility>

#include "dtypes.h"
#include "internal.h"
#include "mfma.h"

namespace chm {
namespace {

constexpr int D = 128;
constexpr int BC = 16;                  // tokens per chunk
constexpr int NWAVE = 8;
constexpr int kThreads = 64 * NWAVE;
constexpr int OP = D + 8;               // [BC][OP] bf16 operand rows (channels at cpos)
constexpr int SP = D + 8;               // [D][SP] bf16 transposed state copies
constexpr int TP = BC + 4;              // [BC][TP] bf16 16 x 16 matrices
constexpr float kL2Eps = 1e-6f;
constexpr int kWaitVm0 = 0x0F70;        // s_waitcnt vmcnt(0) (expcnt and lgkmcnt left alone)
constexpr int kTargetBlocks = 256;      // one block per CU
constexpr int64_t kMinSeg = 256;        // tokens per segment at least

// position of channel p's inverse: the channel stored at row position p
__device__ __forceinline__ constexpr int cinv(int p) {
  return (p & ~31) | ((p & 24) >> 1) | ((p & 4) << 2) | (p & 3);
}
static_assert(cinv(cpos(5)) == 5 && cinv(cpos(22)) == 22 && cinv(cpos(127)) == 127, "cpos inverse");

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t stride;          // elements between consecutive tokens of q, k, v (and dq, dk, dv)
  const uint16_t* alpha;   // [B][T][H][D]
  const uint16_t* beta;    // [B][T][H]
  const uint16_t* dout;    // [B][T][H][D]
  int64_t T, H;
  int64_t seg_len;         // tokens per segment (a multiple of BC)
  int nseg;
  int l2norm;
  // Segments split in two parts (split = 1, with segments): the checkpoint and gradient passes run
  // per part (part 1, the second, first), so the checkpoints of one part at a time are kept
  int split;
  int part;
  int64_t hmax;            // split: checkpoint slots per segment (chunks of its longer part)
  // state passes
  const float* Sin;        // start states: [bh][nseg][D][D] (nseg > 1) or S0 [bh][D][D]; null = zero
  int64_t sin_stride;      // matrices between consecutive (bh, segment) entries of Sin (segments)
  float* Hout;             // split: the summary pass's state at each part boundary, L slots then M
                           // slots, [2][bh][nseg][2 slots][D][D] (the first slot of each pair)
  float* Sout;             // summary end states [bh][nseg][D][D]: L (blocks < BHP), M (blocks >= BHP)
  uint4* ckpt;             // [bh][ceil(T / BC)][8 waves][4][64 lanes] bf16 fragments
  uint2* tfrag;            // [bh][ceil(T / BC)][2][64 lanes]: each chunk's T and T^T mma16 A fragments
  // gradient passes
  const float* Gin;        // dS at segment ends: [bh][nseg][D][D] or dS_final [bh][D][D]; null = zero
  float* Eout;             // local pass: dS at each segment's start [bh][nseg][D][D]
  float* Gmid;             // split: dS at each part boundary [bh][nseg][D][D] (part 1 writes, part 0 reads)
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  uint16_t* dalpha;
  uint16_t* dbeta;
  float* dS0;              // [bh][D][D] or null
};

// The token range of a segment that a split pass runs: part 0 its first ceil(nc / 2) chunks, part 1
// the rest (empty for a one-chunk segment).
__device__ __forceinline__ int64_t part_mid(int64_t t_beg, int64_t t_end) {
  const int64_t nc = (t_end - t_beg + BC - 1) / BC;
  return min<int64_t>(t_end, t_beg + (nc + 1) / 2 * BC);
}
// the checkpoint of the chunk at token t0: per (bh, chunk), or split per (bh, segment, chunk of the
// part that starts at token tp)
__device__ __forceinline__ uint4* ckpt_at(const BwdArgs& a, int64_t bh, int p, int64_t nck, int64_t tp,
                                          int64_t t0) {
  const int64_t slot = a.split ? (bh * a.nseg + p) * a.hmax + (t0 - tp) / BC : bh * nck + t0 / BC;
  return a.ckpt + slot * NWAVE * 4 * 64;
}

// ---- small helpers ----------------------------------------------------------------------
// sum over the 16 lanes of a DPP row, in every lane
__device__ __forceinline__ float rowsum(float x) {
  x += lane_xor1(x);
  x += lane_xor2(x);
  x += lane_xor4(x);
  x += lane_xor8(x);
  return x;
}
// A-operand fragments (16 rows of 8 channels per k slot) of an operand array, plain reads
__device__ __forceinline__ uint4 opfrag(const uint16_t* arr, int s, int l16, int q4) {
  return ld128(arr, l16 * OP + 32 * s + 8 * q4);
}
// A fragment of X^T (rows = channels 16 rt .. 16 rt + 15, k = tokens 4 q4 .. + 3) for mma16:
// the transposing read at token 4 q4 + l16 / 4, position cpos(16 rt + 4 (l16 % 4)) =
// 32 (rt / 2) + 4 (rt % 2) + 8 (l16 % 4), written as the lane's base plus a constant
__device__ __forceinline__ int opT_base(int l16, int q4) { return (4 * q4 + (l16 >> 2)) * OP + 8 * (l16 & 3); }
__device__ __forceinline__ uint2 opT16(const uint16_t* arr, int rt, int base) {
  return ld_tr(&arr[base + 32 * (rt >> 1) + 4 * (rt & 1)]);
}
// B fragment (k = tokens 4 q4 .. + 3, n = channel or v at row position p0 + l16) for mma16
__device__ __forceinline__ uint2 posB16(const uint16_t* arr, int p0, int l16, int q4) {
  return ld_tr(&arr[(4 * q4 + (l16 >> 2)) * OP + p0 + 4 * (l16 & 3)]);
}
// B fragment (k = natural columns 16 w + 4 q4 .. + 3 of a cpos-ordered row set, n = l16)
// used for dout / v columns of a wave's slice: k = tokens, n = v = 16 w + l16
__device__ __forceinline__ uint2 colB16(const uint16_t* arr, int w, int l16, int q4) {
  return ld_tr(&arr[(4 * q4 + (l16 >> 2)) * OP + cpos(16 * w + 4 * (l16 & 3))]);
}
// B fragment of a transposed [D][SP] state copy: k = v in {32 s + 4 q4 + 0..3, 32 s + 16 + 4 q4 + 0..3},
// n = channel at row position 16 w + l16
__device__ __forceinline__ uint4 stB(const uint16_t* st, int s, int w, int l16, int q4) {
  const int col = 16 * w + 4 * (l16 & 3);
  return cat(ld_tr(&st[(32 * s + 4 * q4 + (l16 >> 2)) * SP + col]),
             ld_tr(&st[(32 * s + 16 + 4 * q4 + (l16 >> 2)) * SP + col]));
}
// state fragment for slot s from the D layout (k order of a plain operand read)
__device__ __forceinline__ uint4 sfrag(const f32x4 (&S)[8], int s) { return cat(pack4(S[2 * s]), pack4(S[2 * s + 1])); }

// Decay factors of tokens 4 TQ .. 4 TQ + 3 of one channel, from that channel's clamped alphas
// a[0..15] of the chunk: e^{g} (prefix products), e^{g_n - g} (suffix products), e^{g - m} and
// e^{m - g} (m = g_7: products between token 7 and the token, and their reciprocals), e^{g_n}.
struct Fac4 {
  float g[4], bar[4], fw[4], bw[4], gn;
};
template <int TQ>
__device__ __forceinline__ void factors_q(const float (&a)[BC], Fac4& f) {
  float p = 1.f;
#pragma unroll
  for (int s = 0; s < 4 * TQ; ++s) p *= a[s];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    p *= a[4 * TQ + j];
    f.g[j] = p;
  }
  float q = 1.f;
#pragma unroll
  for (int s = BC - 1; s >= 4 * TQ + 4; --s) q *= a[s];
#pragma unroll
  for (int j = 3; j >= 0; --j) {
    f.bar[j] = q;
    q *= a[4 * TQ + j];
  }
  f.gn = p;
#pragma unroll
  for (int s = 4 * TQ + 4; s < BC; ++s) f.gn *= a[s];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = 4 * TQ + j;
    float r = 1.f;
    if (t <= 7) {
#pragma unroll
      for (int s = t + 1; s <= 7; ++s) r *= a[s];
      f.bw[j] = r;
      f.fw[j] = __builtin_amdgcn_rcpf(r);
    } else {
#pragma unroll
      for (int s = 8; s <= t; ++s) r *= a[s];
      f.fw[j] = r;
      f.bw[j] = __builtin_amdgcn_rcpf(r);
    }
  }
}
// Operands of tokens 4 TQ .. 4 TQ + 3 of channel c into the operand arrays (bf16, channels at
// cpos): -K^, K_, Kr, Kc and (with q) Q^, Qr; with fac also the fp32 factors e^{g}, e^{g_n - g},
// e^{g - m} ([BC][D]); e^{g_n} of the channel when TQ = 0.
struct OpOut {
  uint16_t *kn, *kb, *kr, *kc, *qh, *qr;
  float *fg, *fb, *ff, *gn;
};
// Operand sets: kOpState (-K^, K_), kOpLocal (also Kc, Q^, Qr), kOpAll (also Kr)
constexpr int kOpState = 0, kOpLocal = 1, kOpAll = 2;
template <int TQ, int OPS, bool FAC>
__device__ __forceinline__ void form_ops_q(const uint16_t* al, const uint16_t* kraw, const uint16_t* qraw, const float* rk,
                                           const float* rq, const OpOut& o, int c) {
  float a[BC];
#pragma unroll
  for (int s = 0; s < BC; ++s) a[s] = bf2f(al[s * D + c]);
  Fac4 f;
  factors_q<TQ>(a, f);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = 4 * TQ + j, x = t * OP + cpos(c), e = t * D + c;
    const float kn = bf2f(kraw[e]) * rk[t];
    o.kn[x] = f2bf(-kn * f.g[j]);
    o.kb[x] = f2bf(kn * f.bar[j]);
    if (OPS == kOpAll) o.kr[x] = f2bf(kn * f.fw[j]);
    if (OPS != kOpState) {
      o.kc[x] = f2bf(kn * f.bw[j]);
      const float qn = bf2f(qraw[e]) * rq[t];
      o.qh[x] = f2bf(qn * f.g[j]);
      o.qr[x] = f2bf(qn * f.fw[j]);
    }
    if (FAC) {
      o.fg[e] = f.g[j];
      o.fb[e] = f.bar[j];
      o.ff[e] = f.fw[j];
    }
  }
  if (TQ == 0) o.gn[c] = f.gn;
}
// thread = channel c of tokens 4 tq .. + 3 (tq wave-uniform)
template <int OPS, bool FAC>
__device__ __forceinline__ void form_ops(const uint16_t* al, const uint16_t* kraw, const uint16_t* qraw, const float* rk,
                                         const float* rq, const OpOut& o, int tq, int c) {
  switch (__builtin_amdgcn_readfirstlane(tq)) {
    case 0: form_ops_q<0, OPS, FAC>(al, kraw, qraw, rk, rq, o, c); break;
    case 1: form_ops_q<1, OPS, FAC>(al, kraw, qraw, rk, rq, o, c); break;
    case 2: form_ops_q<2, OPS, FAC>(al, kraw, qraw, rk, rq, o, c); break;
    default: form_ops_q<3, OPS, FAC>(al, kraw, qraw, rk, rq, o, c); break;
  }
}

// Loads of one chunk's token tt, channels 4 cg .. + 3 (tokens past n read q = k = v = dout = 0,
// alpha = 1, beta = 0)
struct RowLoad {
  uint2 q, k, a, v, d;
  uint16_t beta;   // of token `tid` (threads below 16), as loaded: converted where it is used, so
                   // that no wait for the load lands inside the branch that issues it
};
// Buffer descriptors over one chunk's rows: reads past `bytes` return zero and writes there are
// dropped, so no load or store of a chunk sits in a branch (a wait for one that might not have
// been issued would otherwise have to wait for everything).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, kRsrcW3);
}
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void st_buf64(__amdgpu_buffer_rsrc_t r, int voff, uint2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{v.x, v.y}, r, voff, 0, 0);
}
// Row loads of the chunk at t0 (n tokens): token tt, channels c0 .. c0 + 3; beta of token tid
template <bool Q, bool V, bool DO>
__device__ __forceinline__ void load_rows(const BwdArgs& a, int64_t b, int64_t h, int64_t t0, int n, int tt, int c0,
                                          int tid, RowLoad& r) {
  const int64_t row0 = b * a.T + t0;
  const int st2 = (int)a.stride * 2, sa2 = (int)a.H * D * 2;
  const int vq = tt * st2 + 2 * c0, va = tt * sa2 + 2 * c0;
  r.k = ld_buf64(rsrc(a.k + row0 * a.stride + h * D, n * st2), vq, 0);
  r.q = Q ? ld_buf64(rsrc(a.q + row0 * a.stride + h * D, n * st2), vq, 0) : make_uint2(0, 0);
  r.v = V ? ld_buf64(rsrc(a.v + row0 * a.stride + h * D, n * st2), vq, 0) : make_uint2(0, 0);
  r.a = ld_buf64(rsrc(a.alpha + (row0 * a.H + h) * D, n * sa2), va, 0);   // 0 past n: made 1 where used
  r.d = DO ? ld_buf64(rsrc(a.dout + (row0 * a.H + h) * D, n * sa2), va, 0) : make_uint2(0, 0);
  r.beta = __builtin_amdgcn_raw_buffer_load_b16(rsrc(a.beta + row0 * a.H + h, n * (int)a.H * 2),
                                                (tid & (BC - 1)) * (int)a.H * 2 + (tid < BC ? 0 : n * (int)a.H * 2), 0, 0);
}
__device__ __forceinline__ uint2 alpha2(uint2 a) { return make_uint2(clamp_alpha2(a.x), clamp_alpha2(a.y)); }
constexpr uint2 ones2 = {0x3F803F80u, 0x3F803F80u};

// The inversion T = (I + diag(b) A)^{-1} from adiag = -b_r A_ri (i < r): lane j of the first
// 16 forms column j by forward substitution and writes it to tcm (column-major).
__device__ __forceinline__ void invert16(const float* adiag, uint16_t* tcm, int lane) {
  if (lane >= 16) return;
  int j = lane;
  asm volatile("" : "+v"(j));   // formed here: 16 hoisted (i == j) selects would stay live across the chunk loop
  float x[BC];
#pragma unroll
  for (int i = 0; i < BC; ++i) {
    float acc0 = i == j ? 1.f : 0.f, acc1 = 0.f;
#pragma unroll
    for (int k4 = 0; k4 < (i + 3) / 4; ++k4) {
      const float4 a4 = *reinterpret_cast<const float4*>(&adiag[16 * i + 4 * k4]);
      const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kk = 4 * k4 + e;
        if (kk < i) {
          if (e & 1) acc1 += av[e] * x[kk];
          else acc0 += av[e] * x[kk];
        }
      }
    }
    x[i] = acc0 + acc1;
  }
#pragma unroll
  for (int m = 0; m < 4; ++m)
    *reinterpret_cast<uint2*>(&tcm[j * TP + 4 * m]) = pack4(make_float4(x[4 * m], x[4 * m + 1], x[4 * m + 2], x[4 * m + 3]));
}

// ---- the chunk factorisation pass ---------------------------------------------------------
// T = (I + diag(b) A)^{-1}, A = strict_lower(Kr Kc^T), of every chunk once, for all the passes
// after it: one wave per chunk forms Kr, Kc (channels of the pair 2 l, 2 l + 1 per lane over the
// 16 tokens), A on MFMA, and T by forward substitution, and stores the two mma16 A fragments
// the passes use, of T (U = T diag(b) R) and of T^T (Y = T^T dU): [bh][chunk][2][64 lanes] x 8 bytes.
struct TfacLds {          // per wave
  uint16_t kr[BC * OP];
  uint16_t kc[BC * OP];
  uint16_t kraw[BC * D];
  uint16_t al[BC * D];
  uint16_t tcm[BC * TP];  // T column-major
  float adiag[BC * BC];   // -b_r A_ri (i < r)
  float rk[BC];
  float beta[BC];
};
constexpr int kTfacWaves = 4;
__global__ __launch_bounds__(64 * kTfacWaves) void kda_bwd_tfac_kernel(BwdArgs a, int64_t total) {
  extern __shared__ __align__(16) char smem[];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l16 = lane & 15, q4 = lane >> 4;
  TfacLds& L = reinterpret_cast<TfacLds*>(smem)[w];
  const int64_t gc = (int64_t)blockIdx.x * kTfacWaves + w;   // chunk of all sequences and heads
  if (gc >= total) return;                                   // (no block barriers below)
  const int64_t nck = (a.T + BC - 1) / BC;
  const int64_t bh = gc / nck, c = gc % nck;
  const int64_t b = bh / a.H, h = bh % a.H, t0 = c * BC, row0 = b * a.T + t0;
  const int n = (int)min<int64_t>(BC, a.T - t0);
  // loads: lane = token tq, channels 32 cq .. + 31
  const int tq = lane >> 2, cq = lane & 3;
  const int st2 = (int)a.stride * 2, sa2 = (int)a.H * D * 2;
  const auto rk_ = rsrc(a.k + row0 * a.stride + h * D, n * st2);
  const auto ra_ = rsrc(a.alpha + (row0 * a.H + h) * D, n * sa2);
  uint4 kv[4], av[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const auto k4 = __builtin_amdgcn_raw_buffer_load_b128(rk_, tq * st2 + 64 * cq + 16 * j, 0, 0);
    const auto a4 = __builtin_amdgcn_raw_buffer_load_b128(ra_, tq * sa2 + 64 * cq + 16 * j, 0, 0);
    kv[j] = make_uint4(k4[0], k4[1], k4[2], k4[3]);
    av[j] = make_uint4(a4[0], a4[1], a4[2], a4[3]);
  }
  const uint16_t braw = __builtin_amdgcn_raw_buffer_load_b16(rsrc(a.beta + row0 * a.H + h, n * (int)a.H * 2),
                                                             (lane & (BC - 1)) * (int)a.H * 2 + (lane < BC ? 0 : n * (int)a.H * 2), 0, 0);
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) ss = sq2(kv[j].w, sq2(kv[j].z, sq2(kv[j].y, sq2(kv[j].x, ss))));
  ss += lane_xor1(ss);
  ss += lane_xor2(ss);
  const bool in = tq < n;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    *reinterpret_cast<uint4*>(&L.kraw[tq * D + 32 * cq + 8 * j]) = kv[j];
    *reinterpret_cast<uint4*>(&L.al[tq * D + 32 * cq + 8 * j]) =
        in ? make_uint4(clamp_alpha2(av[j].x), clamp_alpha2(av[j].y), clamp_alpha2(av[j].z), clamp_alpha2(av[j].w))
           : make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
  }
  if (cq == 0) L.rk[tq] = a.l2norm ? __builtin_amdgcn_rsqf(ss + kL2Eps) : 1.f;
  if (lane < BC) L.beta[lane] = bf2f(braw);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  // Kr = k e^{g - m} / |k|, Kc = k e^{m - g} / |k| (m = g_7) for channels 2 lane, 2 lane + 1
  {
    float a0[BC], a1[BC];
#pragma unroll
    for (int t = 0; t < BC; ++t) {
      const uint32_t u = *reinterpret_cast<const uint32_t*>(&L.al[t * D + 2 * lane]);
      a0[t] = bf_lo(u);
      a1[t] = bf_hi(u);
    }
    float f0[BC], f1[BC];   // e^{m - g_t} for t <= 7, e^{g_t - m} for t >= 8
    float r0 = 1.f, r1 = 1.f;
#pragma unroll
    for (int t = 7; t >= 0; --t) {
      f0[t] = r0;
      f1[t] = r1;
      r0 *= a0[t];
      r1 *= a1[t];
    }
    r0 = r1 = 1.f;
#pragma unroll
    for (int t = 8; t < BC; ++t) {
      r0 *= a0[t];
      r1 *= a1[t];
      f0[t] = r0;
      f1[t] = r1;
    }
    const int x = cpos(2 * lane);
#pragma unroll
    for (int t = 0; t < BC; ++t) {
      const uint32_t u = *reinterpret_cast<const uint32_t*>(&L.kraw[t * D + 2 * lane]);
      const float rk = L.rk[t], k0 = bf_lo(u) * rk, k1 = bf_hi(u) * rk;
      const float i0 = __builtin_amdgcn_rcpf(f0[t]), i1 = __builtin_amdgcn_rcpf(f1[t]);
      const bool lo = t <= 7;   // f holds e^{m - g} there, e^{g - m} after
      *reinterpret_cast<uint32_t*>(&L.kr[t * OP + x]) = pack_bf16x2(k0 * (lo ? i0 : f0[t]), k1 * (lo ? i1 : f1[t]));
      *reinterpret_cast<uint32_t*>(&L.kc[t * OP + x]) = pack_bf16x2(k0 * (lo ? f0[t] : i0), k1 * (lo ? f1[t] : i1));
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = mma32(opfrag(L.kr, s, l16, q4), opfrag(L.kc, s, l16, q4), acc);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int rr = 4 * q4 + r;
    L.adiag[16 * rr + l16] = rr > l16 ? -L.beta[rr] * acc[r] : 0.f;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  invert16(L.adiag, L.tcm, lane);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  uint2* out = a.tfrag + gc * 2 * 64 + lane;
  out[0] = ld_tr(&L.tcm[(4 * q4 + (l16 >> 2)) * TP + 4 * (l16 & 3)]);
  out[64] = *reinterpret_cast<const uint2*>(&L.tcm[l16 * TP + 4 * q4]);
}
// the T (which = 0) or T^T (which = 1) fragment of chunk `c` of sequence-head bh
__device__ __forceinline__ uint2 tfrag(const BwdArgs& a, int64_t bh, int64_t nck, int64_t c, int which, int lane) {
  return a.tfrag[((bh * nck + c) * 2 + which) * 64 + lane];
}

// ---- forward state passes ----------------------------------------------------------------
constexpr int kCkpt = 0, kSum = 1;
// Two barriers per chunk: the arrays phase 1 writes alternate by chunk parity (phases 2 and 3
// read them), the operands are written in phase 2 once every wave has passed the chunk
// before's phases 3 and 4.
struct FwdIn {
  uint16_t vv[BC * OP];   // v (cpos order)
  uint16_t kraw[BC * D];  // k as loaded (natural order)
  uint16_t al[BC * D];    // alpha raised to the floor (natural order)
  float beta[BC];
  float rk[BC];
};
struct FwdLds {
  uint16_t kn[BC * OP];   // -K^
  uint16_t kb[BC * OP];   // K_
  float gn[D];
  FwdIn in[2];
};

// block bid of a pass over BHP (sequence, head, segment) blocks (the summary pass has 2 BHP: L, then M)
template <int MODE>
__device__ __forceinline__ void fwd_body(const BwdArgs& a, char* smem, int64_t bid, int64_t BHP) {
  FwdLds& L = *reinterpret_cast<FwdLds*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, q4 = lane >> 4;
  const int tt = tid >> 5, cg = tid & 31, c0 = 4 * cg;
  const int tb = opT_base(l16, q4);
  const bool mpart = MODE == kSum && bid >= BHP;   // transition product: from I with v = 0
  const int64_t lb = mpart ? bid - BHP : bid;
  const int p = (int)(lb % a.nseg);
  const int64_t bh = lb / a.nseg;
  const int64_t b = bh / a.H, h = bh % a.H;
  const int64_t s_beg = (int64_t)p * a.seg_len;
  const int64_t s_end = min<int64_t>(a.T, s_beg + a.seg_len);
  const int64_t s_mid = part_mid(s_beg, s_end);
  // split: one part of the segment (the summary pass's part 0 ends at the boundary's state, its part
  // 1 starts there)
  const int64_t t_beg = a.split && a.part == 1 ? s_mid : s_beg;
  const int64_t t_end = a.split && a.part == 0 ? s_mid : s_end;
  const int64_t nck = (a.T + BC - 1) / BC;
  // the summary pass's part-boundary state of this block (L or M, the first slot of its pair)
  float* hslot = MODE == kSum && a.split ? a.Hout + ((mpart ? 2 * BHP : 0) + 2 * lb) * (int64_t)(D * D) : nullptr;

  f32x4 S[8];
  {
    const float* src = nullptr;
    if (MODE == kCkpt && a.Sin != nullptr)
      src = a.Sin + (a.nseg > 1 ? (bh * a.nseg + p) * a.sin_stride : bh) * (int64_t)(D * D);
    if (MODE == kSum && a.split && a.part == 1) src = hslot;
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * rt + 4 * q4 + r, col = 16 * w + l16;
        S[rt][r] = src != nullptr ? src[row * D + col] : (mpart && row == col ? 1.f : 0.f);
      }
  }
  float* out = nullptr;   // the summary pass's state at the end of its range
  if (MODE == kSum)
    out = a.split && a.part == 0 ? hslot : a.Sout + (mpart ? BHP : 0) * (int64_t)(D * D) + lb * (int64_t)(D * D);
  auto store_state = [&]() {
    if (out != nullptr) {
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) out[(16 * rt + 4 * q4 + r) * D + 16 * w + l16] = S[rt][r];
    }
  };
  if (t_end <= t_beg) {   // an empty part 1 (a one-chunk segment): the state passes through (block-uniform)
    store_state();
    return;
  }
  // each chunk's rows and T fragment are loaded one chunk ahead
  RowLoad rl;
  auto load_chunk = [&](int64_t tc, uint2& tf) {
    const int nn = (int)min<int64_t>(BC, t_end - tc);
    if (mpart) load_rows<false, false, false>(a, b, h, tc, nn, tt, c0, tid, rl);
    else load_rows<false, true, false>(a, b, h, tc, nn, tt, c0, tid, rl);
    tf = tfrag(a, bh, nck, tc / BC, 0, lane);
  };
  uint2 tfn;
  load_chunk(t_beg, tfn);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);   // as in the gradient kernel: the loop's counts decide its waits
  int par = 0;
  for (int64_t t0 = t_beg; t0 < t_end; t0 += BC, par ^= 1) {
    const int n = (int)min<int64_t>(BC, t_end - t0);
    FwdIn& I = L.in[par];
    // phase 1: the chunk's rows into LDS, norms; the chunk's start state out
    if (MODE == kCkpt) {
      uint4* dst = ckpt_at(a, bh, p, nck, t_beg, t0) + w * 4 * 64 + lane;
#pragma unroll
      for (int s = 0; s < 4; ++s) dst[s * 64] = sfrag(S, s);
    }
    const bool in = tt < n;
    if (tid < BC) I.beta[tid] = bf2f(rl.beta);
    float ss = dot4(rl.k);
    ss = rowsum(ss);
    ss = halve16(ss, ss);
    const float rk = a.l2norm ? __builtin_amdgcn_rsqf(ss + kL2Eps) : 1.f;
    *reinterpret_cast<uint2*>(&I.al[tt * D + c0]) = in ? alpha2(rl.a) : ones2;
    *reinterpret_cast<uint2*>(&I.vv[tt * OP + cpos(c0)]) = rl.v;
    *reinterpret_cast<uint2*>(&I.kraw[tt * D + c0]) = rl.k;
    if (cg == 0) I.rk[tt] = rk;
    const uint2 tf = tfn;
    // the next chunk's (the last chunk's again after it: no load sits in a branch)
    load_chunk(t0 + BC < t_end ? t0 + BC : t0, tfn);
    lds_barrier();
    // phase 2: decay factors and operands, thread = channel c of tokens 4 tq .. + 3
    form_ops<kOpState, false>(I.al, I.kraw, nullptr, I.rk, nullptr,
                              OpOut{L.kn, L.kb, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, L.gn},
                              tid >> 7, tid & (D - 1));
    lds_barrier();
    // phase 3: R = V - K^ S, diag(b) R; U = T diag(b) R; S <- Diag(e^{g_n}) S + K_^T U
    f32x4 R = {0.f, 0.f, 0.f, 0.f};
    if (!mpart) {
      const float4 v4 = unpack4(colB16(I.vv, w, l16, q4));
      R = f32x4{v4.x, v4.y, v4.z, v4.w};
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) R = mma32(opfrag(L.kn, s, l16, q4), sfrag(S, s), R);
#pragma unroll
    for (int r = 0; r < 4; ++r) R[r] *= I.beta[4 * q4 + r];
    const f32x4 U = mma16(tf, pack4(R), f32x4{0.f, 0.f, 0.f, 0.f});
    const uint2 Ub = pack4(U);
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) {
      const float4 g4 = *reinterpret_cast<const float4*>(&L.gn[16 * rt + 4 * q4]);
      f32x4 x = S[rt];
      x[0] *= g4.x; x[1] *= g4.y; x[2] *= g4.z; x[3] *= g4.w;
      S[rt] = mma16(opT16(L.kb, rt, tb), Ub, x);
    }
  }
  store_state();
}

// ---- gradient passes ---------------------------------------------------------------------
// The arrays that the operand pass reads and writes at many constant offsets come first, within
// the 64 KB that LDS instruction offsets reach from one base register (each access pattern on
// an array beyond that needs a register of its own).
struct GradLds {
  uint16_t qraw[BC * D];  // q, k as loaded (natural order)
  uint16_t kraw[BC * D];
  uint16_t al[BC * D];    // alpha raised to the floor (natural order)
  uint16_t kn[BC * OP];   // -K^
  uint16_t kb[BC * OP];   // K_
  uint16_t kr[BC * OP];
  uint16_t kc[BC * OP];
  uint16_t qh[BC * OP];   // Q^
  uint16_t qr[BC * OP];
  float fg[BC * D];       // e^{g}
  float fb[BC * D];       // e^{g_n - g}
  float ff[BC * D];       // e^{g - m}
                          // (fg, fb, ff hold dq^, dk^ and dalpha once the chain rule has run)
  float rq[BC];
  float rk[BC];
  float beta[BC];
  float gn[D];
  uint16_t dob[BC * OP];  // dout (v at cpos)
  uint16_t uc[BC * OP];   // U (v at cpos); v of the chunk before U is formed
  uint16_t yc[BC * OP];   // Y
  uint16_t aqt[BC * TP];  // Aq^T row-major
  uint16_t daq[BC * TP];  // dAq column-major
  uint16_t dam[BC * TP];  // dA column-major
  float aw[BC * BC];      // A_ri (i < r)
  float dbp[NWAVE * BC];  // per wave: Y . R per token
  float dba[BC];          // -rowsum(A o H)
  uint16_t st[D * SP];    // S^T: [v][channel position]
  uint16_t dst[D * SP];   // dS'^T
};
struct LocalLds {         // the local pass: operands, dout and Aq^T
  uint16_t kn[BC * OP];
  uint16_t kb[BC * OP];
  uint16_t kc[BC * OP];
  uint16_t qh[BC * OP];
  uint16_t qr[BC * OP];
  uint16_t dob[BC * OP];
  uint16_t aqt[BC * TP];
  uint16_t qraw[BC * D];
  uint16_t kraw[BC * D];
  uint16_t al[BC * D];
  float gn[D];
  float beta[BC];
  float rq[BC];
  float rk[BC];
};
static_assert(sizeof(GradLds) <= 160 * 1024, "one block per CU");
constexpr size_t kCkptLocalLds = sizeof(FwdLds) > sizeof(LocalLds) ? sizeof(FwdLds) : sizeof(LocalLds);
static_assert(2 * kCkptLocalLds <= 160 * 1024, "two blocks per CU");

template <bool LOCAL>
__device__ __forceinline__ void grad_body(const BwdArgs& a, char* smem, int64_t bid) {
  typedef typename std::conditional<LOCAL, LocalLds, GradLds>::type Lds;
  Lds& L = *reinterpret_cast<Lds*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, q4 = lane >> 4;
  const int tt = tid >> 5, cg = tid & 31, c0 = 4 * cg;
  const int tb = opT_base(l16, q4);
  const int p = (int)(bid % a.nseg);
  const int64_t bh = bid / a.nseg;
  const int64_t b = bh / a.H, h = bh % a.H;
  const int64_t s_beg = (int64_t)p * a.seg_len;
  const int64_t s_end = min<int64_t>(a.T, s_beg + a.seg_len);
  const int64_t s_mid = part_mid(s_beg, s_end);
  // the local pass runs the whole segment, a split gradient pass one part of it (part 1 from dS at
  // the segment end to the part boundary, part 0 from there to the segment start)
  const bool split = !LOCAL && a.split;
  const int64_t t_beg = split && a.part == 1 ? s_mid : s_beg;
  const int64_t t_end = split && a.part == 0 ? s_mid : s_end;
  const int64_t nck = (a.T + BC - 1) / BC;
  const int pc = 16 * w + l16;    // this lane's channel position (per-channel gradients)
  const int ch = cinv(pc);        // ... and its channel

  f32x4 dS[8];
  {
    const float* src = nullptr;
    if (split && a.part == 0) src = a.Gmid + (bh * a.nseg + p) * (int64_t)(D * D);
    else if (!LOCAL && a.Gin != nullptr) src = a.Gin + (a.nseg > 1 ? (bh * a.nseg + p) : bh) * (int64_t)(D * D);
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        dS[rt][r] = src != nullptr ? src[(16 * rt + 4 * q4 + r) * D + 16 * w + l16] : 0.f;
  }
  // where dS goes at the end: the local pass's segment start, a split part 1's boundary, or dS0
  float* out = nullptr;
  if (LOCAL) out = a.Eout + (bh * a.nseg + p) * (int64_t)(D * D);
  else if (split && a.part == 1) out = a.Gmid + (bh * a.nseg + p) * (int64_t)(D * D);
  else if (p == 0 && a.dS0 != nullptr) out = a.dS0 + bh * (int64_t)(D * D);
  auto store_out = [&]() {
    if (out != nullptr) {
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) out[(16 * rt + 4 * q4 + r) * D + 16 * w + l16] = dS[rt][r];
    }
  };
  if (t_end <= t_beg) {   // an empty part 1 (a one-chunk segment): dS passes through (block-uniform)
    store_out();
    return;
  }
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const int64_t first = (t_end - 1 - t_beg) / BC;   // the segment's last chunk (t_end > t_beg)
  // each chunk's rows are loaded one chunk ahead, its state fragments once the chunk before
  // it is past its phase 3
  RowLoad rl;
  uint4 Sf[4];
  uint2 tfn = make_uint2(0, 0), ttfn;   // the chunk's T and T^T fragments
  auto load_chunk_rows = [&](int64_t c) {
    const int64_t c0t = t_beg + c * BC;
    load_rows<true, !LOCAL, true>(a, b, h, c0t, (int)min<int64_t>(BC, t_end - c0t), tt, c0, tid, rl);
    if (!LOCAL) tfn = tfrag(a, bh, nck, c0t / BC, 0, lane);
    ttfn = tfrag(a, bh, nck, c0t / BC, 1, lane);
  };
  auto load_frags = [&](int64_t c) {
    const uint4* src = ckpt_at(a, bh, p, nck, t_beg, t_beg + c * BC) + w * 4 * 64 + lane;
#pragma unroll
    for (int s = 0; s < 4; ++s) Sf[s] = src[s * 64];
  };
  load_chunk_rows(first);
  if (!LOCAL) load_frags(first);
  // all of these in before the loop: at its head the loop's own counts then decide every wait
  // (merged with this path's, a wait for a prefetched row would wait for everything)
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  for (int64_t ci = first; ci >= 0; --ci) {
    const int64_t t0 = t_beg + ci * BC;
    const int n = (int)min<int64_t>(BC, t_end - t0);
    const bool in = tt < n;
    lds_barrier();   // the previous chunk's reads of the LDS are done
    // phase 1: the chunk's rows into LDS, norms
    if (tid < BC) L.beta[tid] = bf2f(rl.beta);
    float sq = rowsum(dot4(rl.q)), sk = rowsum(dot4(rl.k));
    sq = halve16(sq, sq);
    sk = halve16(sk, sk);
    const float rq = a.l2norm ? __builtin_amdgcn_rsqf(sq + kL2Eps) : 1.f;
    const float rk = a.l2norm ? __builtin_amdgcn_rsqf(sk + kL2Eps) : 1.f;
    *reinterpret_cast<uint2*>(&L.al[tt * D + c0]) = in ? alpha2(rl.a) : ones2;
    *reinterpret_cast<uint2*>(&L.dob[tt * OP + cpos(c0)]) = rl.d;
    *reinterpret_cast<uint2*>(&L.qraw[tt * D + c0]) = rl.q;
    *reinterpret_cast<uint2*>(&L.kraw[tt * D + c0]) = rl.k;
    if (cg == 0) {
      L.rq[tt] = rq;
      L.rk[tt] = rk;
    }
    if constexpr (!LOCAL) *reinterpret_cast<uint2*>(&L.uc[tt * OP + cpos(c0)]) = rl.v;
    const uint2 tf = tfn, ttf = ttfn;
    load_chunk_rows(ci > 0 ? ci - 1 : 0);   // (chunk 0's again after it: no load sits in a branch)
    lds_barrier();
    // phase 2: factors and operands (thread = channel c of tokens 4 tq .. + 3); the transposed
    // state copies and dS' o S per channel
    if constexpr (LOCAL)
      form_ops<kOpLocal, false>(L.al, L.kraw, L.qraw, L.rk, L.rq,
                            OpOut{L.kn, L.kb, nullptr, L.kc, L.qh, L.qr, nullptr, nullptr, nullptr, L.gn}, tid >> 7,
                            tid & (D - 1));
    else
      form_ops<kOpAll, true>(L.al, L.kraw, L.qraw, L.rk, L.rq,
                           OpOut{L.kn, L.kb, L.kr, L.kc, L.qh, L.qr, L.fg, L.fb, L.ff, L.gn}, tid >> 7, tid & (D - 1));
    if constexpr (!LOCAL) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        *reinterpret_cast<uint4*>(&L.st[(16 * w + l16) * SP + 32 * s + 8 * q4]) = Sf[s];
        *reinterpret_cast<uint4*>(&L.dst[(16 * w + l16) * SP + 32 * s + 8 * q4]) = sfrag(dS, s);
      }
    }
    lds_barrier();
    // phase 3: A (wave 0, for db) and Aq (wave 1); dU = K_ dS' and R = V - K^ S (every wave)
    if (!LOCAL && w == 0) {
      if constexpr (!LOCAL) {
        f32x4 acc = zero4;
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mma32(opfrag(L.kr, s, l16, q4), opfrag(L.kc, s, l16, q4), acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rr = 4 * q4 + r;
          L.aw[16 * rr + l16] = rr > l16 ? acc[r] : 0.f;
        }
      }
    } else if (w == 1) {
      f32x4 acc = zero4;
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = mma32(opfrag(L.qr, s, l16, q4), opfrag(L.kc, s, l16, q4), acc);
      float m[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) m[r] = 4 * q4 + r >= l16 ? acc[r] : 0.f;   // Aq(r, i), i = l16 <= r
      *reinterpret_cast<uint2*>(&L.aqt[l16 * TP + 4 * q4]) = pack4(make_float4(m[0], m[1], m[2], m[3]));
    }
    f32x4 dU = zero4;
#pragma unroll
    for (int s = 0; s < 4; ++s) dU = mma32(opfrag(L.kb, s, l16, q4), sfrag(dS, s), dU);
    f32x4 R = zero4;
    if constexpr (!LOCAL) {
      const float4 v4 = unpack4(colB16(L.uc, w, l16, q4));
      R = f32x4{v4.x, v4.y, v4.z, v4.w};
#pragma unroll
      for (int s = 0; s < 4; ++s) R = mma32(opfrag(L.kn, s, l16, q4), Sf[s], R);
      load_frags(ci > 0 ? ci - 1 : 0);
    }
    lds_barrier();
    // phase 4: U, dU += Aq^T dout, Y = T^T dU, dR = diag(b) Y; dS <- Q^^T dout + e^{g_n} dS' - K^^T dR
    const uint2 dOB = colB16(L.dob, w, l16, q4);
    dU = mma16(*reinterpret_cast<const uint2*>(&L.aqt[l16 * TP + 4 * q4]), dOB, dU);
    const f32x4 Y = mma16(ttf, pack4(dU), zero4);
    f32x4 dR;
#pragma unroll
    for (int r = 0; r < 4; ++r) dR[r] = L.beta[4 * q4 + r] * Y[r];
    f32x4 U = zero4;
    if constexpr (!LOCAL) {
      f32x4 bR;
#pragma unroll
      for (int r = 0; r < 4; ++r) bR[r] = L.beta[4 * q4 + r] * R[r];
      U = mma16(tf, pack4(bR), zero4);
      // dv, and this wave's part of Y . R per token
      const auto rdv = rsrc(a.dv + (b * a.T + t0) * a.stride + h * D, n * (int)a.stride * 2);
      float yr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * q4 + r;
        __builtin_amdgcn_raw_buffer_store_b16(f2bf(dR[r]), rdv, t * (int)a.stride * 2 + 2 * (16 * w + l16), 0, 0);
        yr[r] = rowsum(Y[r] * R[r]);
        L.uc[t * OP + cpos(16 * w + l16)] = f2bf(U[r]);
        L.yc[t * OP + cpos(16 * w + l16)] = f2bf(Y[r]);
      }
      if (l16 == 0) *reinterpret_cast<float4*>(&L.dbp[w * BC + 4 * q4]) = make_float4(yr[0], yr[1], yr[2], yr[3]);
    }
    {
      const uint2 dRb = pack4(dR);
#pragma unroll
      for (int rt = 0; rt < 8; ++rt) {
        const float4 g4 = *reinterpret_cast<const float4*>(&L.gn[16 * rt + 4 * q4]);
        f32x4 x = dS[rt];
        x[0] *= g4.x; x[1] *= g4.y; x[2] *= g4.z; x[3] *= g4.w;
        x = mma16(opT16(L.kn, rt, tb), dRb, x);
        dS[rt] = mma16(opT16(L.qh, rt, tb), dOB, x);
      }
    }
    if constexpr (LOCAL) continue;
    else {
      lds_barrier();
      // phase 5: dAq (wave 0), H, dA and rowsum(A o H) (wave 1); per channel position:
      // dQ^ = dout S^T, dK^ = -diag(b) Y S^T, dK_ = U dS'^T
      if (w == 0) {
        f32x4 acc = zero4;
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mma32(opfrag(L.dob, s, l16, q4), opfrag(L.uc, s, l16, q4), acc);
        float m[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) m[r] = 4 * q4 + r >= l16 ? acc[r] : 0.f;
        *reinterpret_cast<uint2*>(&L.daq[l16 * TP + 4 * q4]) = pack4(make_float4(m[0], m[1], m[2], m[3]));
      } else if (w == 1) {
        f32x4 acc = zero4;
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mma32(opfrag(L.yc, s, l16, q4), opfrag(L.uc, s, l16, q4), acc);
        float m[4], ah[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rr = 4 * q4 + r;
          const float hv = rr > l16 ? acc[r] : 0.f;
          m[r] = -L.beta[rr] * hv;
          ah[r] = rowsum(L.aw[16 * rr + l16] * hv);
        }
        *reinterpret_cast<uint2*>(&L.dam[l16 * TP + 4 * q4]) = pack4(make_float4(m[0], m[1], m[2], m[3]));
        if (l16 == 0) *reinterpret_cast<float4*>(&L.dba[4 * q4]) = make_float4(-ah[0], -ah[1], -ah[2], -ah[3]);
      }
      // (and S dS'^T over this wave's 16 channel positions, whose diagonal is sum_v S o dS' per channel:
      // the transposed copies' fragments serve as A and as B operands alike)
      f32x4 dQh = zero4, dYS = zero4, dKb = zero4, sds = zero4;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 sb = stB(L.st, s, w, l16, q4), db = stB(L.dst, s, w, l16, q4);
        dQh = mma32(opfrag(L.dob, s, l16, q4), sb, dQh);
        dYS = mma32(opfrag(L.yc, s, l16, q4), sb, dYS);
        dKb = mma32(opfrag(L.uc, s, l16, q4), db, dKb);
        sds = mma32(sb, db, sds);
      }
      lds_barrier();
      // phase 6: dQr = dAq Kc, dKr = dA Kc, dKc = dAq^T Qr + dA^T Kr; the per-element chain rule
      const uint2 kcB = posB16(L.kc, 16 * w, l16, q4);
      const f32x4 dQr = mma16(ld_tr(&L.daq[(4 * q4 + (l16 >> 2)) * TP + 4 * (l16 & 3)]), kcB, zero4);
      const f32x4 dKr = mma16(ld_tr(&L.dam[(4 * q4 + (l16 >> 2)) * TP + 4 * (l16 & 3)]), kcB, zero4);
      f32x4 dKc = mma16(*reinterpret_cast<const uint2*>(&L.daq[l16 * TP + 4 * q4]), posB16(L.qr, 16 * w, l16, q4), zero4);
      dKc = mma16(*reinterpret_cast<const uint2*>(&L.dam[l16 * TP + 4 * q4]), posB16(L.kr, 16 * w, l16, q4), dKc);
      // dq^ and dk^ through the fp32 factors. For dlog alpha, the products with each operand use
      // the bf16 operand values the MFMA products used: the terms of a token pair on the same side
      // of a split cancel in the suffix sums below, and they cancel to fp32 rounding only when both
      // sides multiply the same values (the difference left, the part that crosses the split,
      // carries the split token's alpha and can be 1e-4 of the terms).
      float dqn[4], dkn[4], dg[4], kb[4], al4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * q4 + r, e = t * D + ch, o = t * OP + pc;
        const float fg = L.fg[e], fb = L.fb[e], ff = L.ff[e], fw = __builtin_amdgcn_rcpf(ff);
        al4[r] = bf2f(L.al[e]);
        const float dKh = -L.beta[t] * dYS[r];
        dqn[r] = dQh[r] * fg + dQr[r] * ff;
        dkn[r] = dKh * fg + dKb[r] * fb + dKr[r] * ff + dKc[r] * fw;
        dg[r] = dQh[r] * bf2f(L.qh[o]) + dQr[r] * bf2f(L.qr[o]) - dKh * bf2f(L.kn[o]) + dKr[r] * bf2f(L.kr[o]) -
                dKc[r] * bf2f(L.kc[o]);
        kb[r] = dKb[r] * bf2f(L.kb[o]);
      }
      // dlog alpha_s = sum_{t >= s} dg_t + sum_{t < s} dK_t o K_t + e^{g_n} rowsum(S o dS'): the K_
      // terms decay from token t + 1 to the chunk's end, the last over the whole chunk
      const float gsum = dg[0] + dg[1] + dg[2] + dg[3], ksum = kb[0] + kb[1] + kb[2] + kb[3];
      const float gu1 = __shfl(gsum, (lane + 16) & 63), gu2 = __shfl(gsum, (lane + 32) & 63),
                  gu3 = __shfl(gsum, (lane + 48) & 63);
      const float kd1 = __shfl(ksum, (lane + 48) & 63), kd2 = __shfl(ksum, (lane + 32) & 63),
                  kd3 = __shfl(ksum, (lane + 16) & 63);
      float after = (q4 < 3 ? gu1 : 0.f) + (q4 < 2 ? gu2 : 0.f) + (q4 < 1 ? gu3 : 0.f);
      float before = (q4 > 0 ? kd1 : 0.f) + (q4 > 1 ? kd2 : 0.f) + (q4 > 2 ? kd3 : 0.f);
      // the diagonal element of position l16 sits in lane 16 (l16 / 4) + l16, element l16 % 4
      const float dsel = (l16 & 3) == 0 ? sds[0] : (l16 & 3) == 1 ? sds[1] : (l16 & 3) == 2 ? sds[2] : sds[3];
      const float sdS = __shfl(dsel, 16 * (l16 >> 2) + l16);
      const float whole = L.gn[ch] * sdS;
      float dla[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        dla[r] = before;
        before += kb[r];
      }
#pragma unroll
      for (int r = 3; r >= 0; --r) {
        after += dg[r];
        dla[r] += after + whole;
      }
      // dq^, dk^ and dalpha replace the factors this lane alone read (element (t, ch))
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = (4 * q4 + r) * D + ch;
        L.fg[e] = dqn[r];
        L.fb[e] = dkn[r];
        L.ff[e] = dla[r] * __builtin_amdgcn_rcpf(al4[r]);
      }
      lds_barrier();
      // phase 7 (thread = token tt, channels 4 cg .. + 3): the L2 normalisation's backward and
      // the stores
      {
        const int e = tt * D + c0;
        float4 dq = *reinterpret_cast<const float4*>(&L.fg[e]);
        float4 dk = *reinterpret_cast<const float4*>(&L.fb[e]);
        const float4 da = *reinterpret_cast<const float4*>(&L.ff[e]);
        if (a.l2norm) {
          const float rqt = L.rq[tt], rkt = L.rk[tt];
          const float4 qn = mul4(unpack4(*reinterpret_cast<const uint2*>(&L.qraw[e])), make_float4(rqt, rqt, rqt, rqt));
          const float4 kn = mul4(unpack4(*reinterpret_cast<const uint2*>(&L.kraw[e])), make_float4(rkt, rkt, rkt, rkt));
          float sq2 = rowsum(qn.x * dq.x + qn.y * dq.y + qn.z * dq.z + qn.w * dq.w);
          float sk2 = rowsum(kn.x * dk.x + kn.y * dk.y + kn.z * dk.z + kn.w * dk.w);
          sq2 = halve16(sq2, sq2);
          sk2 = halve16(sk2, sk2);
          dq = make_float4(rqt * (dq.x - qn.x * sq2), rqt * (dq.y - qn.y * sq2), rqt * (dq.z - qn.z * sq2),
                           rqt * (dq.w - qn.w * sq2));
          dk = make_float4(rkt * (dk.x - kn.x * sk2), rkt * (dk.y - kn.y * sk2), rkt * (dk.z - kn.z * sk2),
                           rkt * (dk.w - kn.w * sk2));
        }
        const int64_t row0 = b * a.T + t0;
        const int st2 = (int)a.stride * 2, sa2 = (int)a.H * D * 2;
        st_buf64(rsrc(a.dq + row0 * a.stride + h * D, n * st2), tt * st2 + 2 * c0, pack4(dq));
        st_buf64(rsrc(a.dk + row0 * a.stride + h * D, n * st2), tt * st2 + 2 * c0, pack4(dk));
        st_buf64(rsrc(a.dalpha + (row0 * a.H + h) * D, n * sa2), tt * sa2 + 2 * c0, pack4(da));
        const int tb16 = tid & (BC - 1);
        float db = L.dba[tb16];
#pragma unroll
        for (int ww = 0; ww < NWAVE; ++ww) db += L.dbp[ww * BC + tb16];
        __builtin_amdgcn_raw_buffer_store_b16(f2bf(db), rsrc(a.dbeta + row0 * a.H + h, n * (int)a.H * 2),
                                              tb16 * (int)a.H * 2 + (tid < BC ? 0 : n * (int)a.H * 2), 0, 0);
      }
    }
  }
  store_out();
}

// ---- chains of segment states on MFMA -------------------------------------------------------
// Y_0 = init, Y_p = A_p Y_{p-1} + X_{p-1} over the segments of each (bh) (forward: A_p = M_{p-1};
// BACK: from the last segment down, Y_p = M_{p+1}^T Y_{p+1} + X_{p+1}), fp32 d x d row-major
// matrices [bh][nseg][D][D], init [bh][D][D] or null. As the forward pass's combine step: block
// (bh, slice) owns columns 16 slice .. 16 slice + 15 of Y, wave w rows 16 w .. 16 w + 15 of them in
// fp32 (MFMA D layout); each step exchanges the base through LDS split into bf16 high and low parts
// and forms the product with three bf16 MFMAs per k slot (hi*hi + hi*lo + lo*hi, about 16
// significant bits per product), the A fragments split from the fp32 M as they arrive. The next
// step's M rows (M^T: columns) and X are loaded while a step computes.
constexpr int kChThreads = 512;
constexpr int kChP = D + 8;   // LDS pitch of the transposed base (bf16 elements)
// v split into bf16 high parts (returned) and low parts v - hi (in lo), 8 values
__device__ __forceinline__ uint4 split8(const float (&v)[8], uint4& lo) {
  const uint2 h0 = pack4(make_float4(v[0], v[1], v[2], v[3])), h1 = pack4(make_float4(v[4], v[5], v[6], v[7]));
  const float4 b0 = unpack4(h0), b1 = unpack4(h1);
  const uint2 l0 = pack4(make_float4(v[0] - b0.x, v[1] - b0.y, v[2] - b0.z, v[3] - b0.w));
  const uint2 l1 = pack4(make_float4(v[4] - b1.x, v[5] - b1.y, v[6] - b1.z, v[7] - b1.w));
  lo = cat(l0, l1);
  return cat(h0, h1);
}
template <bool BACK>
__global__ __launch_bounds__(kChThreads) void kda_bwd_chain_kernel(const float* __restrict__ M,
                                                                   const float* __restrict__ X,
                                                                   const float* __restrict__ init,
                                                                   float* __restrict__ Y, int nseg) {
  __shared__ __align__(16) uint16_t bhi[2][16 * kChP];   // [column][cpos(row)] of the base, by step parity
  __shared__ __align__(16) uint16_t blo[2][16 * kChP];
  const int slice = blockIdx.x & 7;
  const int64_t bh = blockIdx.x >> 3;
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, q4 = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = 16 * slice + l16;
  const int row0 = 16 * w + 4 * q4;   // D-layout rows of this lane: row0 .. row0 + 3
  const int64_t off0 = bh * nseg * (int64_t)(D * D);   // this (bh)'s first matrix
  auto at = [&](const float* base, int p) { return base + off0 + p * (int64_t)(D * D); };
  auto at_w = [&](float* base, int p) { return base + off0 + p * (int64_t)(D * D); };
  f32x4 cur;
#pragma unroll
  for (int r = 0; r < 4; ++r) cur[r] = init != nullptr ? init[(bh * D + row0 + r) * D + col] : 0.f;
  auto put = [&](int p) {
    float* y = at_w(Y, p);
#pragma unroll
    for (int r = 0; r < 4; ++r) y[(row0 + r) * D + col] = cur[r];
  };
  put(BACK ? nseg - 1 : 0);
  // the operands of step i (1 .. nseg - 1): A's 32 values of this lane (row 16 w + l16, k = the
  // positions 32 s + 4 q4 .. + 3 and 32 s + 16 + 4 q4 .. + 3 of each slot s) and X's 4
  struct Ops {
    float a[4][8];
    f32x4 x;
  };
  auto src_of = [&](int i) {   // the segment whose M and X form step i (clamped: no load in a branch)
    const int ic = min(max(i, 1), max(nseg - 1, 1));
    return min(BACK ? nseg - ic : ic - 1, nseg - 1);
  };
  auto fetch = [&](int i, Ops& o) {
    const int src = src_of(i);
    const float* m = at(M, src);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (!BACK) {
        const float4 u = *reinterpret_cast<const float4*>(&m[(16 * w + l16) * D + 32 * s + 4 * q4]);
        const float4 v = *reinterpret_cast<const float4*>(&m[(16 * w + l16) * D + 32 * s + 16 + 4 * q4]);
        o.a[s][0] = u.x; o.a[s][1] = u.y; o.a[s][2] = u.z; o.a[s][3] = u.w;
        o.a[s][4] = v.x; o.a[s][5] = v.y; o.a[s][6] = v.z; o.a[s][7] = v.w;
      } else {
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          o.a[s][i2] = m[(32 * s + 4 * q4 + i2) * D + 16 * w + l16];
          o.a[s][4 + i2] = m[(32 * s + 16 + 4 * q4 + i2) * D + 16 * w + l16];
        }
      }
    }
    const float* x = at(X, src);
#pragma unroll
    for (int r = 0; r < 4; ++r) o.x[r] = x[(row0 + r) * D + col];
  };
  Ops nxt;
  fetch(1, nxt);
  for (int i = 1; i < nseg; ++i) {
    const Ops op = nxt;
    fetch(i + 1, nxt);
    const int buf = i & 1;
    {   // the base's rows row0 .. row0 + 3 of column l16 -> LDS, transposed and split
      uint2 lo;
      const float4 c4 = make_float4(cur[0], cur[1], cur[2], cur[3]);
      const uint2 hi = pack4(c4);
      const float4 b = unpack4(hi);
      lo = pack4(make_float4(c4.x - b.x, c4.y - b.y, c4.z - b.z, c4.w - b.w));
      const int pos = cpos(row0);
      *reinterpret_cast<uint2*>(&bhi[buf][l16 * kChP + pos]) = hi;
      *reinterpret_cast<uint2*>(&blo[buf][l16 * kChP + pos]) = lo;
    }
    lds_barrier();
    f32x4 acc0 = op.x, acc1 = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 bH = *reinterpret_cast<const uint4*>(&bhi[buf][l16 * kChP + 32 * s + 8 * q4]);
      const uint4 bL = *reinterpret_cast<const uint4*>(&blo[buf][l16 * kChP + 32 * s + 8 * q4]);
      uint4 al;
      const uint4 ah = split8(op.a[s], al);
      acc1 = mma32(al, bH, acc1);
      acc2 = mma32(ah, bL, acc2);
      acc0 = mma32(ah, bH, acc0);
    }
    cur = acc0 + (acc1 + acc2);
    put(BACK ? nseg - 1 - i : i);
  }
}
// The chains of the chunked backward (dk = dv = D) for BH (bh) of nseg segments each; as
// launch_kda_chain, on MFMA.
hipError_t launch_bwd_chain(bool back, const float* M, const float* X, const float* init, float* Y, int64_t BH,
                            int nseg, hipStream_t stream) {
  if (BH * 8 > 0x7fffffff) return hipErrorInvalidValue;
  if (BH == 0) return hipSuccess;
  const dim3 grid((unsigned)(BH * 8)), thr(kChThreads);
  if (back) hipLaunchKernelGGL(kda_bwd_chain_kernel<true>, grid, thr, 0, stream, M, X, init, Y, nseg);
  else hipLaunchKernelGGL(kda_bwd_chain_kernel<false>, grid, thr, 0, stream, M, X, init, Y, nseg);
  return hipGetLastError();
}

// The passes. The checkpoint and local passes are independent of each other and run as one
// launch (two blocks per CU: each pass's latency fills the other's gaps).
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void kda_bwd_sum_kernel(BwdArgs a) {
  extern __shared__ __align__(16) char smem[];
  fwd_body<kSum>(a, smem, blockIdx.x, gridDim.x / 2);
}
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void kda_bwd_ckpt_local_kernel(
    BwdArgs a, int local) {
  extern __shared__ __align__(16) char smem[];
  const int64_t n = local ? gridDim.x / 2 : gridDim.x;   // checkpoint blocks first
  if ((int64_t)blockIdx.x < n) fwd_body<kCkpt>(a, smem, blockIdx.x, n);
  else grad_body<true>(a, smem, blockIdx.x - n);
}
__global__ __launch_bounds__(kThreads) void kda_bwd_grad_kernel(BwdArgs a) {
  extern __shared__ __align__(16) char smem[];
  grad_body<false>(a, smem, blockIdx.x);
}

struct Cut {
  int64_t len;
  int nseg;
};
constexpr int kSegMats = 6 + 7;   // per (bh, segment): L, M, start, E, G, spare; 2 x 2 + 2 + 1 at the part boundary
// checkpoint slots per segment of len tokens when split: the chunks of its longer (first) part
int64_t part_slots(int64_t len) { return ((len + BC - 1) / BC + 1) / 2; }
Cut bwd_chunked_cut(int64_t B, int64_t T, int64_t H) {
  const int64_t bh = std::max<int64_t>(1, B * H);
  int64_t P = (kTargetBlocks + bh - 1) / bh;
  P = std::min<int64_t>(P, std::max<int64_t>(1, T / kMinSeg));
  if (P <= 1) return {std::max<int64_t>(T, 1), 1};
  const int64_t len = ((T + P - 1) / P + BC - 1) / BC * BC;
  P = (T + len - 1) / len;
  return P <= 1 ? Cut{T, 1} : Cut{len, (int)P};
}

}  // namespace

bool kda_bwd_chunked_shape(int64_t dk, int64_t dv, bool bf16) { return bf16 && dk == D && dv == D; }

bool kda_bwd_chunked_layout_ok(const KdaArgs& a, const KdaGrads& g) {
  const uintptr_t al = reinterpret_cast<uintptr_t>(a.q) | reinterpret_cast<uintptr_t>(a.k) |
                       reinterpret_cast<uintptr_t>(a.v) | reinterpret_cast<uintptr_t>(a.alpha) |
                       reinterpret_cast<uintptr_t>(g.dout);
  return a.qkv_stride % 4 == 0 && (al & 7) == 0;
}

size_t kda_bwd_chunked_workspace(int64_t B, int64_t T, int64_t H) {
  const Cut c = bwd_chunked_cut(B, T, H);
  const size_t nck = (size_t)((T + BC - 1) / BC);
  const size_t slots = c.nseg > 1 ? (size_t)c.nseg * (size_t)part_slots(c.len) : nck;   // per (b, h)
  const size_t ck = (size_t)(B * H) * slots * D * D * sizeof(uint16_t);
  const size_t tf = (size_t)(B * H) * nck * 2 * 64 * sizeof(uint2);
  const size_t segs = c.nseg > 1 ? (size_t)(B * H) * c.nseg * kSegMats * D * D * sizeof(float) : 0;
  return ck + tf + segs;
}

// Workspace: the bf16 chunk states (with segments: of one part of every segment at a time), the
// chunks' T fragments, then (segments only) per (bh, segment) fp32 D x D matrices: L and M of every
// segment (the summary pass writes [L of all (bh, p)][M of all (bh, p)]), the start states, E, G
// and a spare, then the part-boundary states of the summary pass (L, M: two slots each), the chain's
// part-boundary starts (two slots) and dS at the part boundaries.
hipError_t launch_kda_backward_chunked(const KdaArgs& x, const KdaGrads& g, void* workspace, hipStream_t stream,
                                       Marks* marks) {
  if (x.B * x.H == 0 || x.T == 0) return hipSuccess;
  const Cut c = bwd_chunked_cut(x.B, x.T, x.H);
  const int64_t BH = x.B * x.H;
  if (BH * c.nseg * 2 > 0x7fffffff) return hipErrorInvalidValue;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::atomic<bool> attr_done[64];
  if (dev < 0 || dev >= 64 || !attr_done[dev].load(std::memory_order_acquire)) {
    const std::pair<const void*, int> fns[] = {
        {reinterpret_cast<const void*>(&kda_bwd_sum_kernel), (int)sizeof(FwdLds)},
        {reinterpret_cast<const void*>(&kda_bwd_ckpt_local_kernel), (int)kCkptLocalLds},
        {reinterpret_cast<const void*>(&kda_bwd_grad_kernel), (int)sizeof(GradLds)},
        {reinterpret_cast<const void*>(&kda_bwd_tfac_kernel), (int)(kTfacWaves * sizeof(TfacLds))}};
    for (const auto& f : fns) {
      e = hipFuncSetAttribute(f.first, hipFuncAttributeMaxDynamicSharedMemorySize, f.second);
      if (e != hipSuccess) return e;
    }
    if (dev >= 0 && dev < 64) attr_done[dev].store(true, std::memory_order_release);
  }
  BwdArgs a{};
  a.q = static_cast<const uint16_t*>(x.q);
  a.k = static_cast<const uint16_t*>(x.k);
  a.v = static_cast<const uint16_t*>(x.v);
  a.stride = x.qkv_stride;
  a.alpha = static_cast<const uint16_t*>(x.alpha);
  a.beta = static_cast<const uint16_t*>(x.beta);
  a.dout = static_cast<const uint16_t*>(g.dout);
  a.T = x.T;
  a.H = x.H;
  a.seg_len = c.len;
  a.nseg = c.nseg;
  a.l2norm = x.l2norm ? 1 : 0;
  a.ckpt = static_cast<uint4*>(workspace);
  a.split = c.nseg > 1 ? 1 : 0;
  a.part = 0;
  a.hmax = part_slots(c.len);
  a.sin_stride = 1;
  a.dq = static_cast<uint16_t*>(g.dq);
  a.dk = static_cast<uint16_t*>(g.dk);
  a.dv = static_cast<uint16_t*>(g.dv);
  a.dalpha = static_cast<uint16_t*>(g.dalpha);
  a.dbeta = static_cast<uint16_t*>(g.dbeta);
  a.dS0 = g.dS0;
  const int64_t nck = (x.T + BC - 1) / BC;
  const size_t slots = a.split ? (size_t)c.nseg * (size_t)a.hmax : (size_t)nck;
  const size_t ck = (size_t)BH * slots * D * D * sizeof(uint16_t);
  const size_t tfb = (size_t)BH * (size_t)nck * 2 * 64 * sizeof(uint2);
  a.tfrag = reinterpret_cast<uint2*>(static_cast<char*>(workspace) + ck);
  const int64_t mat = BH * c.nseg * (int64_t)(D * D);
  float* Lw = reinterpret_cast<float*>(static_cast<char*>(workspace) + ck + tfb);
  float* Mw = Lw + mat;
  float* Sst = Mw + mat;
  float* Ew = Sst + mat;
  float* Gw = Ew + mat;
  float* Hw = Lw + 6 * mat;   // part boundary: [L: 2 slots][M: 2 slots] per (bh, segment)
  float* Yw = Hw + 4 * mat;   // the part-boundary starts (slot 1 of each pair)
  float* Gm = Yw + 2 * mat;   // dS at the part boundaries
  const dim3 thr(kThreads);
  const unsigned blocks = (unsigned)(BH * c.nseg);
  {
    const int64_t total = BH * nck;
    hipLaunchKernelGGL(kda_bwd_tfac_kernel, dim3((unsigned)((total + kTfacWaves - 1) / kTfacWaves)),
                       dim3(64 * kTfacWaves), kTfacWaves * sizeof(TfacLds), stream, a, total);
    e = hipGetLastError();
    if (e == hipSuccess) e = mark_after(marks, "kda_bwd_tfac_kernel", stream);
    if (e != hipSuccess) return e;
  }
  if (c.nseg == 1) {   // one segment: the checkpoint pass, then the gradient pass
    a.Sin = x.S0;
    a.Gin = g.dS_final;
    hipLaunchKernelGGL(kda_bwd_ckpt_local_kernel, dim3(blocks), thr, kCkptLocalLds, stream, a, 0);
    e = hipGetLastError();
    if (e == hipSuccess) e = mark_after(marks, "kda_bwd_ckpt_local_kernel", stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kda_bwd_grad_kernel, dim3(blocks), thr, sizeof(GradLds), stream, a);
    e = hipGetLastError();
    return e != hipSuccess ? e : mark_after(marks, "kda_bwd_grad_kernel", stream);
  }
  // Segments, each split in two parts so that the checkpoints of one part at a time are kept: the
  // summary pass in two launches (each segment's L and M at its part boundary, then at its end), the
  // chain of segment starts, the part-boundary starts (S_mid = M_half S_start + L_half, a one-step
  // chain per segment); part 1's checkpoints with the local pass in one launch, the chain of dL/dS at
  // segment ends, part 1's gradients (down to dS at the part boundary), part 0's checkpoints, part 0's
  // gradients.
  {
    BwdArgs s = a;
    s.Sout = Lw;
    s.Hout = Hw;
    for (int part = 0; part < 2 && e == hipSuccess; ++part) {   // part 1 from part 0's boundary state
      s.part = part;
      hipLaunchKernelGGL(kda_bwd_sum_kernel, dim3(2 * blocks), thr, sizeof(FwdLds), stream, s);
      e = hipGetLastError();
      if (e == hipSuccess) e = mark_after(marks, "kda_bwd_sum_kernel", stream);
    }
    if (e == hipSuccess) e = launch_bwd_chain(false, Mw, Lw, x.S0, Sst, BH, c.nseg, stream);
    if (e == hipSuccess) e = mark_after(marks, "kda_bwd_chain_kernel", stream);
    if (e == hipSuccess) e = launch_bwd_chain(false, Hw + 2 * mat, Hw, Sst, Yw, BH * c.nseg, 2, stream);
    if (e == hipSuccess) e = mark_after(marks, "kda_bwd_chain_kernel", stream);
    if (e != hipSuccess) return e;
  }
  {
    BwdArgs l = a;
    l.part = 1;
    l.Sin = Yw + D * D;
    l.sin_stride = 2;
    l.Eout = Ew;
    hipLaunchKernelGGL(kda_bwd_ckpt_local_kernel, dim3(2 * blocks), thr, kCkptLocalLds, stream, l, 1);
    e = hipGetLastError();
    if (e == hipSuccess) e = mark_after(marks, "kda_bwd_ckpt_local_kernel", stream);
    if (e == hipSuccess) e = launch_bwd_chain(true, Mw, Ew, g.dS_final, Gw, BH, c.nseg, stream);
    if (e == hipSuccess) e = mark_after(marks, "kda_bwd_chain_kernel", stream);
    if (e != hipSuccess) return e;
  }
  a.Gin = Gw;
  a.Gmid = Gm;
  for (int part = 1; part >= 0; --part) {
    if (part == 0) {
      BwdArgs c0 = a;
      c0.part = 0;
      c0.Sin = Sst;
      hipLaunchKernelGGL(kda_bwd_ckpt_local_kernel, dim3(blocks), thr, kCkptLocalLds, stream, c0, 0);
      e = hipGetLastError();
      if (e == hipSuccess) e = mark_after(marks, "kda_bwd_ckpt_local_kernel", stream);
      if (e != hipSuccess) return e;
    }
    BwdArgs gp = a;
    gp.part = part;
    hipLaunchKernelGGL(kda_bwd_grad_kernel, dim3(blocks), thr, sizeof(GradLds), stream, gp);
    e = hipGetLastError();
    if (e == hipSuccess) e = mark_after(marks, "kda_bwd_grad_kernel", stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace chm
