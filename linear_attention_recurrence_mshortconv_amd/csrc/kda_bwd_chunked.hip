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
  // state passes
  const float* Sin;        // start states: [bh][nseg][D][D] (nseg > 1) or S0 [bh][D][D]; null = zero
  float* Sout;             // summary end states [bh][nseg][D][D]: L (blocks < BHP), M (blocks >= BHP)
  uint4* ckpt;             // [bh][ceil(T / BC)][8 waves][4][64 lanes] bf16 fragments
  // gradient passes
  const float* Gin;        // dS at segment ends: [bh][nseg][D][D] or dS_final [bh][D][D]; null = zero
  float* Eout;             // local pass: dS at each segment's start [bh][nseg][D][D]
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  uint16_t* dalpha;
  uint16_t* dbeta;
  float* dS0;              // [bh][D][D] or null
};

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
// A fragment of X^T (rows = channels 16 rt .. 16 rt + 15, k = tokens 4 q4 .. + 3) for mma16
__device__ __forceinline__ uint2 opT16(const uint16_t* arr, int rt, int l16, int q4) {
  return ld_tr(&arr[(4 * q4 + (l16 >> 2)) * OP + cpos(16 * rt + 4 * (l16 & 3))]);
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
// tq wave-uniform
__device__ __forceinline__ Fac4 factors4(const float* al, int tq, int c) {
  float a[BC];
#pragma unroll
  for (int s = 0; s < BC; ++s) a[s] = al[s * D + c];
  Fac4 f;
  switch (__builtin_amdgcn_readfirstlane(tq)) {
    case 0: factors_q<0>(a, f); break;
    case 1: factors_q<1>(a, f); break;
    case 2: factors_q<2>(a, f); break;
    default: factors_q<3>(a, f); break;
  }
  return f;
}

// Loads of one chunk's token tt, channels 4 cg .. + 3 (tokens past n read q = k = v = dout = 0,
// alpha = 1, beta = 0)
struct RowLoad {
  uint2 q, k, a, v, d;
};
__device__ __forceinline__ float4 alpha4(uint2 a) { return unpack4(make_uint2(clamp_alpha2(a.x), clamp_alpha2(a.y))); }

// The inversion T = (I + diag(b) A)^{-1} from adiag = -b_r A_ri (i < r): lane j of the first
// 16 forms column j by forward substitution and writes it to tcm (column-major).
__device__ __forceinline__ void invert16(const float* adiag, uint16_t* tcm, int lane) {
  if (lane >= 16) return;
  const int j = lane;
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

// ---- forward state passes ----------------------------------------------------------------
constexpr int kCkpt = 0, kSum = 1;
struct FwdLds {
  uint16_t kn[BC * OP];   // -K^
  uint16_t kb[BC * OP];   // K_
  uint16_t kr[BC * OP];
  uint16_t kc[BC * OP];
  uint16_t vv[BC * OP];   // v (cpos order)
  uint16_t tcm[BC * TP];  // T column-major
  uint16_t kraw[BC * D];  // k as loaded (natural order)
  float al[BC * D];
  float adiag[BC * BC];
  float gn[D];
  float beta[BC];
  float rk[BC];
};

template <int MODE>
__global__ __launch_bounds__(kThreads) void kda_bwd_fwd_kernel(BwdArgs a) {
  extern __shared__ __align__(16) char smem[];
  FwdLds& L = *reinterpret_cast<FwdLds*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, q4 = lane >> 4;
  const int tt = tid >> 5, cg = tid & 31, c0 = 4 * cg;
  const int64_t BHP = (int64_t)gridDim.x / (MODE == kSum ? 2 : 1);
  const int64_t bid = blockIdx.x;
  const bool mpart = MODE == kSum && bid >= BHP;   // transition product: from I with v = 0
  const int64_t lb = mpart ? bid - BHP : bid;
  const int p = (int)(lb % a.nseg);
  const int64_t bh = lb / a.nseg;
  const int64_t b = bh / a.H, h = bh % a.H;
  const int64_t t_beg = (int64_t)p * a.seg_len;
  const int64_t t_end = min<int64_t>(a.T, t_beg + a.seg_len);
  const int64_t nck = (a.T + BC - 1) / BC;

  f32x4 S[8];
  {
    const float* src = nullptr;
    if (MODE == kCkpt && a.Sin != nullptr) src = a.Sin + (a.nseg > 1 ? (bh * a.nseg + p) : bh) * (int64_t)(D * D);
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * rt + 4 * q4 + r, col = 16 * w + l16;
        S[rt][r] = src != nullptr ? src[row * D + col] : (mpart && row == col ? 1.f : 0.f);
      }
  }
  const float4 ones = make_float4(1.f, 1.f, 1.f, 1.f);
  for (int64_t t0 = t_beg; t0 < t_end; t0 += BC) {
    const int n = (int)min<int64_t>(BC, t_end - t0);
    // phase 1: loads, norms; the chunk's start state out
    if (MODE == kCkpt) {
      uint4* dst = a.ckpt + ((bh * nck + t0 / BC) * NWAVE + w) * 4 * 64 + lane;
#pragma unroll
      for (int s = 0; s < 4; ++s) dst[s * 64] = sfrag(S, s);
    }
    const bool in = tt < n;
    const int64_t row = b * a.T + t0 + tt;
    uint2 kr = make_uint2(0, 0), ar = make_uint2(0x3F803F80u, 0x3F803F80u), vr = make_uint2(0, 0);
    if (in) {
      kr = *reinterpret_cast<const uint2*>(a.k + row * a.stride + h * D + c0);
      ar = *reinterpret_cast<const uint2*>(a.alpha + (row * a.H + h) * D + c0);
      if (!mpart) vr = *reinterpret_cast<const uint2*>(a.v + row * a.stride + h * D + c0);
    }
    if (tid < BC) L.beta[tid] = tid < n ? bf2f(a.beta[(b * a.T + t0 + tid) * a.H + h]) : 0.f;
    float ss = dot4(kr);
    ss = rowsum(ss);
    ss = halve16(ss, ss);
    const float rk = a.l2norm ? __builtin_amdgcn_rsqf(ss + kL2Eps) : 1.f;
    *reinterpret_cast<float4*>(&L.al[tt * D + c0]) = in ? alpha4(ar) : ones;
    *reinterpret_cast<uint2*>(&L.vv[tt * OP + cpos(c0)]) = vr;
    *reinterpret_cast<uint2*>(&L.kraw[tt * D + c0]) = kr;
    if (cg == 0) L.rk[tt] = rk;
    lds_barrier();
    // phase 2: decay factors and operands, thread = channel c of tokens 4 tq .. + 3
    {
      const int c = tid & (D - 1), tq = tid >> 7;
      const Fac4 f = factors4(L.al, tq, c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 4 * tq + j, o = t * OP + cpos(c);
        const float kn = bf2f(L.kraw[t * D + c]) * L.rk[t];
        L.kn[o] = f2bf(-kn * f.g[j]);
        L.kb[o] = f2bf(kn * f.bar[j]);
        L.kr[o] = f2bf(kn * f.fw[j]);
        L.kc[o] = f2bf(kn * f.bw[j]);
      }
      if (tq == 0) L.gn[c] = f.gn;
    }
    lds_barrier();
    // phase 3: A and T (wave 0); R = V - K^ S and diag(b) R (every wave)
    if (w == 0) {
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
    }
    f32x4 R = {0.f, 0.f, 0.f, 0.f};
    if (!mpart) {
      const float4 v4 = unpack4(colB16(L.vv, w, l16, q4));
      R = f32x4{v4.x, v4.y, v4.z, v4.w};
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) R = mma32(opfrag(L.kn, s, l16, q4), sfrag(S, s), R);
#pragma unroll
    for (int r = 0; r < 4; ++r) R[r] *= L.beta[4 * q4 + r];
    lds_barrier();
    // phase 4: U = T diag(b) R; S <- Diag(e^{g_n}) S + K_^T U
    const f32x4 U = mma16(ld_tr(&L.tcm[(4 * q4 + (l16 >> 2)) * TP + 4 * (l16 & 3)]), pack4(R), f32x4{0.f, 0.f, 0.f, 0.f});
    const uint2 Ub = pack4(U);
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) {
      const float4 g4 = *reinterpret_cast<const float4*>(&L.gn[16 * rt + 4 * q4]);
      f32x4 x = S[rt];
      x[0] *= g4.x; x[1] *= g4.y; x[2] *= g4.z; x[3] *= g4.w;
      S[rt] = mma16(opT16(L.kb, rt, l16, q4), Ub, x);
    }
    // the next chunk's phase 1 writes al, vv and beta only, which phase 4 does not read
  }
  if (MODE == kSum) {
    float* dst = a.Sout + (mpart ? BHP : 0) * (int64_t)(D * D) + lb * (int64_t)(D * D);
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(16 * rt + 4 * q4 + r) * D + 16 * w + l16] = S[rt][r];
  }
}

// ---- gradient passes ---------------------------------------------------------------------
// Arrays with many per-lane access patterns first: LDS instruction offsets reach 64 KB from a
// base register, and each pattern on an array beyond that needs a register of its own.
struct GradLds {
  uint16_t kn[BC * OP];   // -K^
  uint16_t kb[BC * OP];   // K_
  uint16_t kr[BC * OP];
  uint16_t kc[BC * OP];
  uint16_t qh[BC * OP];   // Q^
  uint16_t qr[BC * OP];
  uint16_t dob[BC * OP];  // dout (v at cpos)
  uint16_t uc[BC * OP];   // U (v at cpos); v of the chunk before U is formed
  uint16_t yc[BC * OP];   // Y
  uint16_t tcm[BC * TP];  // T column-major
  uint16_t aqt[BC * TP];  // Aq^T row-major
  uint16_t daq[BC * TP];  // dAq column-major
  uint16_t dam[BC * TP];  // dA column-major
  float adiag[BC * BC];   // -b_r A_ri (i < r)
  float aw[BC * BC];      // A_ri (i < r)
  float gn[D];
  float dgn[NWAVE * D];   // per wave: sum over its v of S o dS' per channel
  float beta[BC];
  float rq[BC];
  float rk[BC];
  float dbp[NWAVE * BC];  // per wave: Y . R per token
  float dba[BC];          // -rowsum(A o H)
  uint16_t qraw[BC * D];  // q, k as loaded (natural order)
  uint16_t kraw[BC * D];
  float al[BC * D];       // clamped alpha (natural order)
  float fg[BC * D];       // e^{g}
  float fb[BC * D];       // e^{g_n - g}
  float ff[BC * D];       // e^{g - m}
                          // (fg, fb, ff hold dq^, dk^ and dalpha once the chain rule has run)
  uint16_t st[D * SP];    // S^T: [v][channel position]
  uint16_t dst[D * SP];   // dS'^T
};
struct LocalLds {         // the local pass: operands, dout, T and Aq^T
  uint16_t kn[BC * OP];
  uint16_t kb[BC * OP];
  uint16_t kr[BC * OP];
  uint16_t kc[BC * OP];
  uint16_t qh[BC * OP];
  uint16_t qr[BC * OP];
  uint16_t dob[BC * OP];
  uint16_t tcm[BC * TP];
  uint16_t aqt[BC * TP];
  uint16_t qraw[BC * D];
  uint16_t kraw[BC * D];
  float al[BC * D];
  float adiag[BC * BC];
  float gn[D];
  float beta[BC];
  float rq[BC];
  float rk[BC];
};
static_assert(sizeof(GradLds) <= 160 * 1024, "one block per CU");

template <bool LOCAL>
__global__ __launch_bounds__(kThreads) void kda_bwd_grad_kernel(BwdArgs a) {
  extern __shared__ __align__(16) char smem[];
  typedef typename std::conditional<LOCAL, LocalLds, GradLds>::type Lds;
  Lds& L = *reinterpret_cast<Lds*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, q4 = lane >> 4;
  const int tt = tid >> 5, cg = tid & 31, c0 = 4 * cg;
  const int64_t bid = blockIdx.x;
  const int p = (int)(bid % a.nseg);
  const int64_t bh = bid / a.nseg;
  const int64_t b = bh / a.H, h = bh % a.H;
  const int64_t t_beg = (int64_t)p * a.seg_len;
  const int64_t t_end = min<int64_t>(a.T, t_beg + a.seg_len);
  const int64_t nck = (a.T + BC - 1) / BC;
  const int pc = 16 * w + l16;    // this lane's channel position (per-channel gradients)
  const int ch = cinv(pc);        // ... and its channel

  f32x4 dS[8];
  {
    const float* src = nullptr;
    if (!LOCAL && a.Gin != nullptr) src = a.Gin + (a.nseg > 1 ? (bh * a.nseg + p) : bh) * (int64_t)(D * D);
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        dS[rt][r] = src != nullptr ? src[(16 * rt + 4 * q4 + r) * D + 16 * w + l16] : 0.f;
  }
  const float4 ones = make_float4(1.f, 1.f, 1.f, 1.f);
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const int64_t first = (t_end - 1 - t_beg) / BC;   // the segment's last chunk (t_end > t_beg)
  for (int64_t ci = first; ci >= 0; --ci) {
    const int64_t t0 = t_beg + ci * BC;
    const int n = (int)min<int64_t>(BC, t_end - t0);
    lds_barrier();   // the previous chunk's reads of the LDS are done
    // phase 1: loads and norms
    uint4 Sf[4];
    if (!LOCAL) {
      const uint4* src = a.ckpt + ((bh * nck + t0 / BC) * NWAVE + w) * 4 * 64 + lane;
#pragma unroll
      for (int s = 0; s < 4; ++s) Sf[s] = src[s * 64];
    }
    const bool in = tt < n;
    const int64_t row = b * a.T + t0 + tt;
    uint2 qv = make_uint2(0, 0), kv = qv, av = make_uint2(0x3F803F80u, 0x3F803F80u), dv = qv, vv = qv;
    if (in) {
      qv = *reinterpret_cast<const uint2*>(a.q + row * a.stride + h * D + c0);
      kv = *reinterpret_cast<const uint2*>(a.k + row * a.stride + h * D + c0);
      av = *reinterpret_cast<const uint2*>(a.alpha + (row * a.H + h) * D + c0);
      dv = *reinterpret_cast<const uint2*>(a.dout + (row * a.H + h) * D + c0);
      if (!LOCAL) vv = *reinterpret_cast<const uint2*>(a.v + row * a.stride + h * D + c0);
    }
    if (tid < BC) L.beta[tid] = tid < n ? bf2f(a.beta[(b * a.T + t0 + tid) * a.H + h]) : 0.f;
    float sq = rowsum(dot4(qv)), sk = rowsum(dot4(kv));
    sq = halve16(sq, sq);
    sk = halve16(sk, sk);
    const float rq = a.l2norm ? __builtin_amdgcn_rsqf(sq + kL2Eps) : 1.f;
    const float rk = a.l2norm ? __builtin_amdgcn_rsqf(sk + kL2Eps) : 1.f;
    *reinterpret_cast<float4*>(&L.al[tt * D + c0]) = in ? alpha4(av) : ones;
    *reinterpret_cast<uint2*>(&L.dob[tt * OP + cpos(c0)]) = dv;
    *reinterpret_cast<uint2*>(&L.qraw[tt * D + c0]) = qv;
    *reinterpret_cast<uint2*>(&L.kraw[tt * D + c0]) = kv;
    if (cg == 0) {
      L.rq[tt] = rq;
      L.rk[tt] = rk;
    }
    if constexpr (!LOCAL) *reinterpret_cast<uint2*>(&L.uc[tt * OP + cpos(c0)]) = vv;
    lds_barrier();
    // phase 2: factors and operands (thread = channel c of tokens 4 tq .. + 3); the transposed
    // state copies and dS' o S per channel
    {
      const int c = tid & (D - 1), tq = tid >> 7;
      const Fac4 f = factors4(L.al, tq, c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 4 * tq + j, o = t * OP + cpos(c), e = t * D + c;
        const float kn = bf2f(L.kraw[e]) * L.rk[t], qn = bf2f(L.qraw[e]) * L.rq[t];
        L.kn[o] = f2bf(-kn * f.g[j]);
        L.kb[o] = f2bf(kn * f.bar[j]);
        L.kr[o] = f2bf(kn * f.fw[j]);
        L.kc[o] = f2bf(kn * f.bw[j]);
        L.qh[o] = f2bf(qn * f.g[j]);
        L.qr[o] = f2bf(qn * f.fw[j]);
        if constexpr (!LOCAL) {
          L.fg[e] = f.g[j];
          L.fb[e] = f.bar[j];
          L.ff[e] = f.fw[j];
        }
      }
      if (tq == 0) L.gn[c] = f.gn;
    }
    if constexpr (!LOCAL) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        *reinterpret_cast<uint4*>(&L.st[(16 * w + l16) * SP + 32 * s + 8 * q4]) = Sf[s];
        *reinterpret_cast<uint4*>(&L.dst[(16 * w + l16) * SP + 32 * s + 8 * q4]) = sfrag(dS, s);
      }
      // sum over this wave's 16 columns of S o dS' for every row (channel)
      float pa[16], pb[16];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float4 lo = unpack4(make_uint2(Sf[s].x, Sf[s].y)), hi = unpack4(make_uint2(Sf[s].z, Sf[s].w));
        const float sv[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int rt = 2 * s + (e >> 2), r = e & 3;   // row 16 rt + 4 q4 + r
          const float prod = sv[e] * dS[rt][r];
          if (rt < 4) pa[4 * rt + r] = prod;
          else pb[4 * (rt - 4) + r] = prod;
        }
      }
      const float ta = row_sum16(pa, l16), tb = row_sum16(pb, l16);
      // lane l16 holds the total of value l16: row 16 (l16 / 4) + 4 q4 + l16 % 4 (+ 64 for tb)
      const int rrow = 16 * (l16 >> 2) + 4 * q4 + (l16 & 3);
      L.dgn[w * D + rrow] = ta;
      L.dgn[w * D + 64 + rrow] = tb;
    }
    lds_barrier();
    // phase 3: A, T (wave 0) and Aq (wave 1); dU = K_ dS' and R = V - K^ S (every wave)
    if (w == 0) {
      f32x4 acc = zero4;
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = mma32(opfrag(L.kr, s, l16, q4), opfrag(L.kc, s, l16, q4), acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rr = 4 * q4 + r;
        L.adiag[16 * rr + l16] = rr > l16 ? -L.beta[rr] * acc[r] : 0.f;
        if constexpr (!LOCAL) L.aw[16 * rr + l16] = rr > l16 ? acc[r] : 0.f;
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      invert16(L.adiag, L.tcm, lane);
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
    }
    lds_barrier();
    // phase 4: U, dU += Aq^T dout, Y = T^T dU, dR = diag(b) Y; dS <- Q^^T dout + e^{g_n} dS' - K^^T dR
    const uint2 dOB = colB16(L.dob, w, l16, q4);
    dU = mma16(*reinterpret_cast<const uint2*>(&L.aqt[l16 * TP + 4 * q4]), dOB, dU);
    const f32x4 Y = mma16(*reinterpret_cast<const uint2*>(&L.tcm[l16 * TP + 4 * q4]), pack4(dU), zero4);
    f32x4 dR;
#pragma unroll
    for (int r = 0; r < 4; ++r) dR[r] = L.beta[4 * q4 + r] * Y[r];
    f32x4 U = zero4;
    if constexpr (!LOCAL) {
      f32x4 bR;
#pragma unroll
      for (int r = 0; r < 4; ++r) bR[r] = L.beta[4 * q4 + r] * R[r];
      U = mma16(ld_tr(&L.tcm[(4 * q4 + (l16 >> 2)) * TP + 4 * (l16 & 3)]), pack4(bR), zero4);
      // dv, and this wave's part of Y . R per token
      float yr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * q4 + r;
        if (t < n) a.dv[(b * a.T + t0 + t) * a.stride + h * D + 16 * w + l16] = f2bf(dR[r]);
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
        x = mma16(opT16(L.kn, rt, l16, q4), dRb, x);
        dS[rt] = mma16(opT16(L.qh, rt, l16, q4), dOB, x);
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
      f32x4 dQh = zero4, dYS = zero4, dKb = zero4;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 sb = stB(L.st, s, w, l16, q4);
        dQh = mma32(opfrag(L.dob, s, l16, q4), sb, dQh);
        dYS = mma32(opfrag(L.yc, s, l16, q4), sb, dYS);
        dKb = mma32(opfrag(L.uc, s, l16, q4), stB(L.dst, s, w, l16, q4), dKb);
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
        al4[r] = L.al[e];
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
      float sdS = 0.f;
#pragma unroll
      for (int ww = 0; ww < NWAVE; ++ww) sdS += L.dgn[ww * D + ch];
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
      if (in) {
        const int e = tt * D + c0;
        float4 dq = *reinterpret_cast<const float4*>(&L.fg[e]);
        float4 dk = *reinterpret_cast<const float4*>(&L.fb[e]);
        const float4 da = *reinterpret_cast<const float4*>(&L.ff[e]);
        if (a.l2norm) {
          const float4 qn = mul4(unpack4(qv), make_float4(rq, rq, rq, rq));
          const float4 kn = mul4(unpack4(kv), make_float4(rk, rk, rk, rk));
          float sq2 = rowsum(qn.x * dq.x + qn.y * dq.y + qn.z * dq.z + qn.w * dq.w);
          float sk2 = rowsum(kn.x * dk.x + kn.y * dk.y + kn.z * dk.z + kn.w * dk.w);
          sq2 = halve16(sq2, sq2);
          sk2 = halve16(sk2, sk2);
          dq = make_float4(rq * (dq.x - qn.x * sq2), rq * (dq.y - qn.y * sq2), rq * (dq.z - qn.z * sq2),
                           rq * (dq.w - qn.w * sq2));
          dk = make_float4(rk * (dk.x - kn.x * sk2), rk * (dk.y - kn.y * sk2), rk * (dk.z - kn.z * sk2),
                           rk * (dk.w - kn.w * sk2));
        }
        *reinterpret_cast<uint2*>(a.dq + row * a.stride + h * D + c0) = pack4(dq);
        *reinterpret_cast<uint2*>(a.dk + row * a.stride + h * D + c0) = pack4(dk);
        *reinterpret_cast<uint2*>(a.dalpha + (row * a.H + h) * D + c0) = pack4(da);
      }
      if (tid < BC && tid < n) {
        float db = L.dba[tid];
#pragma unroll
        for (int ww = 0; ww < NWAVE; ++ww) db += L.dbp[ww * BC + tid];
        a.dbeta[(b * a.T + t0 + tid) * a.H + h] = f2bf(db);
      }
    }
  }
  float* out = nullptr;
  if (LOCAL) out = a.Eout + (bh * a.nseg + p) * (int64_t)(D * D);
  else if (p == 0 && a.dS0 != nullptr) out = a.dS0 + bh * (int64_t)(D * D);
  if (out != nullptr) {
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) out[(16 * rt + 4 * q4 + r) * D + 16 * w + l16] = dS[rt][r];
  }
}

struct Cut {
  int64_t len;
  int nseg;
};
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
  const size_t ck = (size_t)(B * H) * (size_t)((T + BC - 1) / BC) * D * D * sizeof(uint16_t);
  const size_t segs = c.nseg > 1 ? (size_t)(B * H) * c.nseg * 6 * D * D * sizeof(float) : 0;
  return ck + segs;
}

// Workspace: the bf16 chunk states, then (segments only) L and M of every segment (the
// summary pass writes [L of all (bh, p)][M of all (bh, p)]), the start states, E and G.
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
        {reinterpret_cast<const void*>(&kda_bwd_fwd_kernel<kCkpt>), (int)sizeof(FwdLds)},
        {reinterpret_cast<const void*>(&kda_bwd_fwd_kernel<kSum>), (int)sizeof(FwdLds)},
        {reinterpret_cast<const void*>(&kda_bwd_grad_kernel<true>), (int)sizeof(LocalLds)},
        {reinterpret_cast<const void*>(&kda_bwd_grad_kernel<false>), (int)sizeof(GradLds)}};
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
  a.dq = static_cast<uint16_t*>(g.dq);
  a.dk = static_cast<uint16_t*>(g.dk);
  a.dv = static_cast<uint16_t*>(g.dv);
  a.dalpha = static_cast<uint16_t*>(g.dalpha);
  a.dbeta = static_cast<uint16_t*>(g.dbeta);
  a.dS0 = g.dS0;
  const size_t ck = (size_t)BH * (size_t)((x.T + BC - 1) / BC) * D * D * sizeof(uint16_t);
  const int64_t mat = BH * c.nseg * (int64_t)(D * D);
  float* Lw = reinterpret_cast<float*>(static_cast<char*>(workspace) + ck);
  float* Mw = Lw + mat;
  float* Sst = Mw + mat;
  float* Ew = Sst + mat;
  float* Gw = Ew + mat;
  const dim3 thr(kThreads);
  const unsigned blocks = (unsigned)(BH * c.nseg);
  if (c.nseg > 1) {
    BwdArgs s = a;
    s.Sout = Lw;
    hipLaunchKernelGGL(kda_bwd_fwd_kernel<kSum>, dim3(2 * blocks), thr, sizeof(FwdLds), stream, s);
    e = hipGetLastError();
    if (e == hipSuccess) e = mark_after(marks, "kda_bwd_fwd_kernel", stream);
    if (e == hipSuccess) e = launch_kda_chain(false, Mw, Lw, x.S0, Sst, BH, c.nseg, D, D, stream);
    if (e == hipSuccess) e = mark_after(marks, "kda_chain_kernel", stream);
    if (e != hipSuccess) return e;
    a.Sin = Sst;
  } else {
    a.Sin = x.S0;
  }
  hipLaunchKernelGGL(kda_bwd_fwd_kernel<kCkpt>, dim3(blocks), thr, sizeof(FwdLds), stream, a);
  e = hipGetLastError();
  if (e == hipSuccess) e = mark_after(marks, "kda_bwd_fwd_kernel", stream);
  if (e != hipSuccess) return e;
  if (c.nseg > 1) {
    BwdArgs l = a;
    l.Eout = Ew;
    hipLaunchKernelGGL(kda_bwd_grad_kernel<true>, dim3(blocks), thr, sizeof(LocalLds), stream, l);
    e = hipGetLastError();
    if (e == hipSuccess) e = mark_after(marks, "kda_bwd_local_kernel", stream);
    if (e == hipSuccess) e = launch_kda_chain(true, Mw, Ew, g.dS_final, Gw, BH, c.nseg, D, D, stream);
    if (e == hipSuccess) e = mark_after(marks, "kda_chain_kernel", stream);
    if (e != hipSuccess) return e;
    a.Gin = Gw;
  } else {
    a.Gin = g.dS_final;
  }
  hipLaunchKernelGGL(kda_bwd_grad_kernel<false>, dim3(blocks), thr, sizeof(GradLds), stream, a);
  e = hipGetLastError();
  return e != hipSuccess ? e : mark_after(marks, "kda_bwd_grad_kernel", stream);
}

}  // namespace chm
