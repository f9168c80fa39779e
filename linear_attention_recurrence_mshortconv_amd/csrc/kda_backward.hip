// Backward of the KDA recurrence and of mShortConv (fp32 state and accumulation).
//
// KDA: the recurrence of Chimera page 1, section 3.3, Eq. 14 (page 2's
// parentheses) with the readout o_t = S_t^T q_t (Eq. 15, inner term), per token
//   P = Diag(alpha_t) S_{t-1},  w = v_t - P^T k_t,  S_t = P + beta_t k_t w^T,
// on the L2-normalised q and k (page 1, Fig. 2). Reverse mode, with G = dL/dS_t
// (dS_final at the end, carried back token by token):
//   G += q_t do_t^T;  dq_t = S_t do_t;  r = G^T k_t;  dv_t = beta_t r;
//   dbeta_t = r . w;  dk_t = beta_t (G w - P r);  dP = G - beta_t k_t r^T;
//   dalpha_t = rowsum(dP o S_{t-1});  G <- Diag(alpha_t) dP;  dS0 = G at the start.
// The states S_{t-1} come from a forward pass that keeps the state before every
// 16th token (kda_seq_kernel with a checkpoint buffer); each 16-token block is
// recomputed from its checkpoint, four states at a time in registers.
//
// Both directions run on segments of each sequence at once. The map from a
// segment's start state to its end state is S_end = M S_start + L, with M the
// product of the segment's transitions (I - beta k k^T) Diag(alpha), so the start
// states follow from every segment's (M, L) by a short chain, and dL/dS at the
// segment ends from G_start = M^T G_end + E, E being the segment's own part (its
// reverse recurrence from G = 0).
//
// One block per (batch, head, segment, 16-column slice of d_v), 256 threads = 16
// columns x 16 row-threads as in the forward kernel: the column-wise quantities
// (dv) are complete in a block, the row-wise ones (dq, dk, dalpha, dbeta) are sums
// over all columns: each wave sums its 4 columns (permlane swaps) into its own LDS
// slots, the four waves' slots are added as they are written out every four tokens
// to a per-slice partial, and a second kernel adds the slices and applies the L2
// normalisation's backward. Gradients of q, k and v are written at the inputs'
// token stride, so that they can fill one fused q|k|v gradient for the conv.
//
// mShortConv (page 1, section 3.4; Eq. 13): y[p, c] = sum_taps w[c, tap] x[src(p, tap), c]
// gives dx[s, c] = sum over (p, tap) with src(p, tap) = s of w[c, tap] dy[p, c] (the
// adjoint gather: p is s moved back by the tap's offset, inside the same segment; for an
// image grid, the same 3x3 conv with the taps mirrored in both directions) and
// dw[c, tap] = sum_p x[src(p, tap), c] dy[p, c] (summed over tokens and batch items).
#include <atomic>
#include <vector>

#include "dtypes.h"
#include "internal.h"
#include "lanes.h"

namespace chm {
namespace {

constexpr int kCk = 16;   // tokens per checkpoint (the forward kernel's token batch)
constexpr int kHalf = 4;  // states recomputed and kept at a time



// Stages tokens tok0 .. tok0 + nt - 1 (rows of the [B*T] token axis) of one head in LDS: thread
// (colid, rt) loads token colid, rows RPT rt .. RPT rt + RPT - 1 of q and k (L2-normalised)
// and alpha, and column vs * 16 + rt of v (when sv is given) and of dout; tokens past nt
// read as q = k = 0, alpha = 1, beta = 0.
template <typename T, int RPT>
__device__ __forceinline__ void stage_tokens(const T* __restrict__ q, const T* __restrict__ k,
                                             const T* __restrict__ v, int64_t stride, const T* __restrict__ alpha,
                                             const T* __restrict__ beta, const T* __restrict__ dout, int64_t tok0,
                                             int nt, int64_t h, int64_t H, int dk, int dv, int vs, int l2norm,
                                             float (&sq)[kCk][16 * RPT], float (&sk)[kCk][16 * RPT],
                                             float (&sa)[kCk][16 * RPT], float (*sv)[16], float (&sdo)[kCk][16],
                                             float (&sb)[kCk]) {
  const int colid = threadIdx.x >> 4, rt = threadIdx.x & 15;
  const bool tok_ok = colid < nt;
  const int64_t tok = tok0 + colid;
  float rq[RPT], rk[RPT], ssq = 0.f, ssk = 0.f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = RPT * rt + i;
    const bool ok = tok_ok && row < dk;
    rq[i] = ok ? to_f32(q[tok * stride + h * dk + row]) : 0.f;
    rk[i] = ok ? to_f32(k[tok * stride + h * dk + row]) : 0.f;
    sa[colid][row] = ok ? to_f32(alpha[(tok * H + h) * dk + row]) : 1.f;
    ssq = fmaf(rq[i], rq[i], ssq);
    ssk = fmaf(rk[i], rk[i], ssk);
  }
  const float nq = l2norm ? 1.f / sqrtf(sum16(ssq) + 1e-6f) : 1.f;
  const float nk = l2norm ? 1.f / sqrtf(sum16(ssk) + 1e-6f) : 1.f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    sq[colid][RPT * rt + i] = rq[i] * nq;
    sk[colid][RPT * rt + i] = rk[i] * nk;
  }
  const int vc = vs * 16 + rt;   // token colid, column rt of the slice
  if (sv != nullptr) sv[colid][rt] = (tok_ok && vc < dv) ? to_f32(v[tok * stride + h * dv + vc]) : 0.f;
  sdo[colid][rt] = (tok_ok && vc < dv) ? to_f32(dout[(tok * H + h) * dv + vc]) : 0.f;
  if (rt == 0) sb[colid] = tok_ok ? to_f32(beta[tok * H + h]) : 0.f;
}

template <typename T, int RPT>
__global__ __launch_bounds__(256) void kda_bwd_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, int64_t stride,
    const T* __restrict__ alpha, const T* __restrict__ beta, const T* __restrict__ dout,
    const float* __restrict__ G_end, T* __restrict__ dv_out, float* __restrict__ dS0,
    const float* __restrict__ ckpt, float* __restrict__ part, int64_t Tn, int64_t H, int dk, int dv, int l2norm,
    int64_t seg_len, int nseg) {
  constexpr int DKP = 16 * RPT;
  __shared__ float sq[kCk][DKP], sk[kCk][DKP], sa[kCk][DKP];
  __shared__ float sv[kCk][16], sdo[kCk][16], sb[kCk];
  // per wave: sums of dq, dk, dalpha (and dbeta) over its 4 columns; the 4 waves' slots are
  // added as they are written out
  __shared__ float red[kHalf][4][3][DKP];
  __shared__ float redb[kHalf][4];

  const int n_vs = (dv + 15) / 16;
  const int vs = blockIdx.x % n_vs;
  const int p = (int)((blockIdx.x / n_vs) % nseg);      // segment of the sequence
  const int64_t bh = blockIdx.x / n_vs / nseg;
  const int64_t b = bh / H, h = bh % H;
  const int tid = threadIdx.x, colid = tid >> 4, rt = tid & 15, cw = colid & 3, wave = tid >> 6;
  const int col = vs * 16 + colid;
  const bool col_ok = col < dv;
  const int64_t nb = (Tn + kCk - 1) / kCk;
  constexpr int kNV = (3 * RPT + 3) / 4 * 4;
  const int64_t t_beg = nseg > 1 ? p * seg_len : 0;
  const int64_t t_end = nseg > 1 ? min<int64_t>(Tn, t_beg + seg_len) : Tn;
  const int64_t BTH = (int64_t)gridDim.x / n_vs / nseg * Tn;   // B * H * T: one partial array's rows
  float* pq = part + (int64_t)vs * 3 * BTH * dk;        // this slice's partials
  float* pk = pq + BTH * dk;
  float* pa = pk + BTH * dk;
  float* pb = part + (int64_t)n_vs * 3 * BTH * dk + (int64_t)vs * BTH;

  float G[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = RPT * rt + i;
    G[i] = (G_end != nullptr && col_ok && row < dk) ? G_end[((bh * nseg + p) * dk + row) * dv + col] : 0.f;
  }

  // forward step on the staged token tt: S <- S + k (beta w)^T after the decay; returns w
  auto step = [&](float (&S)[RPT], int tt) {
    float pred = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      S[i] *= sa[tt][RPT * rt + i];
      pred = fmaf(S[i], sk[tt][RPT * rt + i], pred);
    }
    const float w = sv[tt][colid] - sum16(pred);
    const float bw = sb[tt] * w;
#pragma unroll
    for (int i = 0; i < RPT; ++i) S[i] = fmaf(sk[tt][RPT * rt + i], bw, S[i]);
    return w;
  };

  for (int64_t kb = (t_end + kCk - 1) / kCk - 1; kb >= t_beg / kCk; --kb) {
    const int64_t t0 = kb * kCk;
    const int nt = (int)min<int64_t>(kCk, t_end - t0);
    __syncthreads();   // the previous block's reads of the staging arrays are done
    stage_tokens<T, RPT>(q, k, v, stride, alpha, beta, dout, b * Tn + t0, nt, h, H, dk, dv, vs, l2norm, sq, sk, sa,
                         sv, sdo, sb);
    __syncthreads();
    float S0c[RPT];   // the state before token t0
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = RPT * rt + i;
      S0c[i] = (col_ok && row < dk) ? ckpt[((bh * nb + kb) * dk + row) * dv + col] : 0.f;
    }
    for (int part = kCk / kHalf - 1; part >= 0; --part) {
      const int h0 = part * kHalf;
      const int hn = min(kHalf, nt - h0);
      if (hn <= 0) continue;
      float S[RPT];
#pragma unroll
      for (int i = 0; i < RPT; ++i) S[i] = S0c[i];
      for (int tt = 0; tt < h0; ++tt) step(S, tt);   // to the part's first token
      float Sp[kHalf][RPT], wv[kHalf];
#pragma unroll
      for (int j = 0; j < kHalf; ++j) {
        if (j < hn) {
#pragma unroll
          for (int i = 0; i < RPT; ++i) Sp[j][i] = S[i];
          wv[j] = step(S, h0 + j);
        }
      }
      // backward over the part; S is the state after its last token
#pragma unroll
      for (int j = kHalf - 1; j >= 0; --j) {
        if (j >= hn) continue;
        const int tt = h0 + j;
        float St[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) St[i] = (j == hn - 1) ? S[i] : Sp[j + 1][i];
        const float doc = sdo[tt][colid], bt = sb[tt], w = wv[j];
        float r = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          G[i] = fmaf(sq[tt][RPT * rt + i], doc, G[i]);
          r = fmaf(G[i], sk[tt][RPT * rt + i], r);
        }
        r = sum16(r);
        if (rt == 0 && col_ok) from_f32(dv_out + (b * Tn + t0 + tt) * stride + h * dv + col, bt * r);
        const float dbr = sum_cols4(r * w);
        if ((tid & 63) == 0) redb[j][wave] = dbr;
        float vals[kNV];   // dq, dk, dalpha of the lane's rows (then zero padding)
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          const int row = RPT * rt + i;
          const float a = sa[tt][row];
          const float dP = G[i] - bt * sk[tt][row] * r;
          vals[i] = St[i] * doc;
          vals[RPT + i] = bt * (G[i] * w - a * Sp[j][i] * r);
          vals[2 * RPT + i] = dP * Sp[j][i];
          G[i] = a * dP;
        }
#pragma unroll
        for (int f = 3 * RPT; f < kNV; ++f) vals[f] = 0.f;
        float sums[kNV / 4];
        sum_cols4_many<kNV>(vals, sums);
#pragma unroll
        for (int n = 0; n < kNV / 4; ++n) {   // lane of wave row cw holds value 4 n + cw
          const int f = 4 * n + cw;
          if (f < 3 * RPT) red[j][wave][f / RPT][RPT * rt + f % RPT] = sums[n];
        }
      }
      __syncthreads();
      // this slice's sums over its 16 columns -> the partial arrays
      for (int e = tid; e < hn * DKP; e += 256) {
        const int j = e / DKP, row = e % DKP;
        if (row >= dk) continue;
        const int64_t o = ((b * Tn + t0 + h0 + j) * H + h) * dk + row;
        pq[o] = red[j][0][0][row] + red[j][1][0][row] + red[j][2][0][row] + red[j][3][0][row];
        pk[o] = red[j][0][1][row] + red[j][1][1][row] + red[j][2][1][row] + red[j][3][1][row];
        pa[o] = red[j][0][2][row] + red[j][1][2][row] + red[j][2][2][row] + red[j][3][2][row];
      }
      if (tid < hn) pb[(b * Tn + t0 + h0 + tid) * H + h] = redb[tid][0] + redb[tid][1] + redb[tid][2] + redb[tid][3];
      __syncthreads();
    }
  }
  if (dS0 != nullptr && col_ok && p == 0) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = RPT * rt + i;
      if (row < dk) dS0[(bh * dk + row) * dv + col] = G[i];
    }
  }
}

// The reverse recurrence alone over one segment, from G = 0 at its end and without the
// states: G += q^_t do_t^T; r = G^T k^_t; G <- Diag(alpha_t) (G - beta_t k^_t r^T). Writes G
// at the segment's start: the segment's own part of dL/dS before it.
template <typename T, int RPT>
__global__ __launch_bounds__(256) void kda_bwd_local_kernel(
    const T* __restrict__ q, const T* __restrict__ k, int64_t stride, const T* __restrict__ alpha,
    const T* __restrict__ beta, const T* __restrict__ dout, float* __restrict__ E, int64_t Tn, int64_t H, int dk,
    int dv, int l2norm, int64_t seg_len, int nseg) {
  constexpr int DKP = 16 * RPT;
  __shared__ float sq[kCk][DKP], sk[kCk][DKP], sa[kCk][DKP];
  __shared__ float sdo[kCk][16], sb[kCk];
  const int n_vs = (dv + 15) / 16;
  const int vs = blockIdx.x % n_vs;
  const int p = (int)((blockIdx.x / n_vs) % nseg);
  const int64_t bh = blockIdx.x / n_vs / nseg;
  const int64_t b = bh / H, h = bh % H;
  const int tid = threadIdx.x, colid = tid >> 4, rt = tid & 15;
  const int col = vs * 16 + colid;
  const int64_t t_beg = p * seg_len, t_end = min<int64_t>(Tn, t_beg + seg_len);
  float G[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) G[i] = 0.f;
  for (int64_t kb = (t_end + kCk - 1) / kCk - 1; kb >= t_beg / kCk; --kb) {
    const int64_t t0 = kb * kCk;
    const int nt = (int)min<int64_t>(kCk, t_end - t0);
    __syncthreads();
    stage_tokens<T, RPT>(q, k, nullptr, stride, alpha, beta, dout, b * Tn + t0, nt, h, H, dk, dv, vs, l2norm, sq, sk,
                         sa, nullptr, sdo, sb);
    __syncthreads();
    for (int tt = nt - 1; tt >= 0; --tt) {
      const float doc = sdo[tt][colid];
      float r = 0.f;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        G[i] = fmaf(sq[tt][RPT * rt + i], doc, G[i]);
        r = fmaf(G[i], sk[tt][RPT * rt + i], r);
      }
      const float br = sb[tt] * sum16(r);
#pragma unroll
      for (int i = 0; i < RPT; ++i) G[i] = sa[tt][RPT * rt + i] * fmaf(-sk[tt][RPT * rt + i], br, G[i]);
    }
  }
  if (col < dv) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = RPT * rt + i;
      if (row < dk) E[((bh * nseg + p) * dk + row) * dv + col] = G[i];
    }
  }
}

// Chains the segments of one (batch, head, 16-column slice of d_v), given each segment's
// transition product M_p (dk x dk: its end state is M_p times its start state plus its own
// term) and a term X_p per segment:
//   forward (BACK false): Y_0 = init, Y_p = M_{p-1} Y_{p-1} + X_{p-1}: the state at each segment's start;
//   backward (BACK true): Y_{P-1} = init, Y_p = M_{p+1}^T Y_{p+1} + X_{p+1}: dL/dS at each segment's end.
// init may be null (zero). dk <= 128. Each step's matrix goes to LDS whole (mt[j][r] = the factor
// of entry j in row r of the product), and the next step's is loaded into registers meanwhile, so
// a step waits for one load only at the start of the chain.
constexpr int kChainPitch = 132;   // mt rows: 16-byte aligned, 4 banks apart
constexpr int kChainLds = (128 * kChainPitch + 128 * 16) * (int)sizeof(float);
template <bool BACK, bool FULL>   // FULL: dk = 128 (16-byte loads of M)
__global__ __launch_bounds__(256) void kda_chain_kernel(const float* __restrict__ M, const float* __restrict__ X,
                                                        const float* __restrict__ init, float* __restrict__ Y,
                                                        int nseg, int dk, int dv) {
  extern __shared__ float chain_lds[];
  float (*mt)[kChainPitch] = reinterpret_cast<float (*)[kChainPitch]>(chain_lds);
  float (*cur)[16] = reinterpret_cast<float (*)[16]>(chain_lds + 128 * kChainPitch);
  const int n_vs = (dv + 15) / 16;
  const int vs = blockIdx.x % n_vs;
  const int64_t bh = blockIdx.x / n_vs;
  const int tid = threadIdx.x, colid = tid >> 4, rt = tid & 15;
  const int col = vs * 16 + colid;
  const bool col_ok = col < dv;
  auto yat = [&](int p, int row) { return ((bh * nseg + p) * dk + row) * dv + col; };
  // M entries e = 4 (tid + 256 m) + u (FULL) or tid + 256 m (row e / dk, column e % dk)
  const int nm = dk * dk;
  constexpr int NP = FULL ? 16 : 64;
  float4 pre4[FULL ? NP : 1];
  float pre[FULL ? 1 : NP];
  float xv[8];
  auto load = [&](int src) {   // M and X of segment src
    const float* Mp = M + (bh * nseg + src) * (int64_t)nm;
    if constexpr (FULL) {
#pragma unroll
      for (int m = 0; m < NP; ++m) pre4[m] = reinterpret_cast<const float4*>(Mp)[tid + 256 * m];
    } else {
#pragma unroll
      for (int m = 0; m < NP; ++m) {
        const int e = tid + 256 * m;
        pre[m] = e < nm ? Mp[e] : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 8 * rt + i;
      xv[i] = col_ok && row < dk ? X[yat(src, row)] : 0.f;
    }
  };
  auto put = [&](int i, int j, float x) {   // M[i][j]
    if (BACK) mt[i][j] = x;                 // row j of M^T takes M[i][j] at entry i
    else mt[j][i] = x;                      // row i of M takes M[i][j] at entry j
  };
  auto stage = [&]() {
    if constexpr (FULL) {
#pragma unroll
      for (int m = 0; m < NP; ++m) {
        const int e = 4 * (tid + 256 * m), i = e >> 7, j = e & 127;
        put(i, j, pre4[m].x);
        put(i, j + 1, pre4[m].y);
        put(i, j + 2, pre4[m].z);
        put(i, j + 3, pre4[m].w);
      }
    } else {
#pragma unroll
      for (int m = 0; m < NP; ++m) {
        const int e = tid + 256 * m;
        if (e < nm) put(e / dk, e % dk, pre[m]);
      }
    }
  };
  {
    const int p0 = BACK ? nseg - 1 : 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 8 * rt + i;
      const bool ok = col_ok && row < dk;
      const float val = (ok && init != nullptr) ? init[(bh * dk + row) * dv + col] : 0.f;
      cur[row][colid] = val;
      if (ok) Y[yat(p0, row)] = val;
    }
  }
  if (nseg > 1) load(BACK ? nseg - 1 : 0);
  for (int step = 1; step < nseg; ++step) {
    const int p = BACK ? nseg - 1 - step : step;   // the entry formed
    const int src = BACK ? p + 1 : p - 1;          // the segment whose M and X form it
    lds_barrier();   // the previous step's reads of mt are done (the next matrix's loads stay in flight)
    stage();
    float xs[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) xs[i] = xv[i];
    lds_barrier();
    if (step + 1 < nseg) load(BACK ? src - 1 : src + 1);
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    // thread rows 8 rt .. 8 rt + 7: two 16-byte reads of mt per entry j
#pragma unroll 4
    for (int j = 0; j < dk; ++j) {
      const float cj = cur[j][colid];
      const float4 m0 = *reinterpret_cast<const float4*>(&mt[j][8 * rt]);
      const float4 m1 = *reinterpret_cast<const float4*>(&mt[j][8 * rt + 4]);
      acc[0] = fmaf(m0.x, cj, acc[0]);
      acc[1] = fmaf(m0.y, cj, acc[1]);
      acc[2] = fmaf(m0.z, cj, acc[2]);
      acc[3] = fmaf(m0.w, cj, acc[3]);
      acc[4] = fmaf(m1.x, cj, acc[4]);
      acc[5] = fmaf(m1.y, cj, acc[5]);
      acc[6] = fmaf(m1.z, cj, acc[6]);
      acc[7] = fmaf(m1.w, cj, acc[7]);
    }
    lds_barrier();   // every read of cur is done
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 8 * rt + i;
      const bool ok = col_ok && row < dk;
      const float val = ok ? acc[i] + xs[i] : 0.f;
      cur[row][colid] = val;
      if (ok) Y[yat(p, row)] = val;
    }
  }
}

// The chain kernels' LDS (above 64 KB) is allowed once per device; the flag is atomic so that
// host threads calling at once race on nothing (setting it twice is harmless).
hipError_t chain_attr() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::atomic<bool> done[64];
  if (dev >= 0 && dev < 64 && done[dev].load(std::memory_order_acquire)) return hipSuccess;
  const void* fns[] = {reinterpret_cast<const void*>(&kda_chain_kernel<false, false>),
                       reinterpret_cast<const void*>(&kda_chain_kernel<true, false>),
                       reinterpret_cast<const void*>(&kda_chain_kernel<false, true>),
                       reinterpret_cast<const void*>(&kda_chain_kernel<true, true>)};
  for (const void* f : fns) {
    e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kChainLds);
    if (e != hipSuccess) return e;
  }
  if (dev >= 0 && dev < 64) done[dev].store(true, std::memory_order_release);
  return hipSuccess;
}
// one chain launch (see kda_chain_kernel)
hipError_t chain_launch(bool back, const float* M, const float* X, const float* init, float* Y, int64_t chains,
                        int nseg, int dk, int dv, hipStream_t stream) {
  const hipError_t e = chain_attr();
  if (e != hipSuccess) return e;
  const dim3 g((unsigned)chains), t(256);
  if (dk == 128) {
    if (back) hipLaunchKernelGGL((kda_chain_kernel<true, true>), g, t, kChainLds, stream, M, X, init, Y, nseg, dk, dv);
    else hipLaunchKernelGGL((kda_chain_kernel<false, true>), g, t, kChainLds, stream, M, X, init, Y, nseg, dk, dv);
  } else {
    if (back) hipLaunchKernelGGL((kda_chain_kernel<true, false>), g, t, kChainLds, stream, M, X, init, Y, nseg, dk, dv);
    else hipLaunchKernelGGL((kda_chain_kernel<false, false>), g, t, kChainLds, stream, M, X, init, Y, nseg, dk, dv);
  }
  return hipGetLastError();
}

// Adds the slices' partials of one (token, head) row and applies the L2 normalisation's
// backward (x^ = x / n, n = sqrt(|x|^2 + eps): dx = dx^ / n - x (x . dx^) / n^3). One wave
// per row; lane l holds channels l, l + 64, ...
template <typename T>
__global__ __launch_bounds__(256) void kda_bwd_reduce_kernel(
    const T* __restrict__ q, const T* __restrict__ k, int64_t stride, const float* __restrict__ part, int n_vs,
    T* __restrict__ dq, T* __restrict__ dk_out, T* __restrict__ dalpha, T* __restrict__ dbeta, int64_t rows,
    int64_t H, int dk, int l2norm) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int64_t tok = row / H, h = row % H;
  const int64_t BTH = rows;
  float gq[4], gk[4], ga[4], xq[4], xk[4];
  float sqq = 0.f, skk = 0.f, dotq = 0.f, dotk = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = lane + 64 * i;
    gq[i] = gk[i] = ga[i] = xq[i] = xk[i] = 0.f;
    if (c >= dk) continue;
    for (int s = 0; s < n_vs; ++s) {
      const float* base = part + (int64_t)s * 3 * BTH * dk + row * dk + c;
      gq[i] += base[0];
      gk[i] += base[BTH * dk];
      ga[i] += base[2 * BTH * dk];
    }
    xq[i] = to_f32(q[tok * stride + h * dk + c]);
    xk[i] = to_f32(k[tok * stride + h * dk + c]);
    sqq = fmaf(xq[i], xq[i], sqq);
    skk = fmaf(xk[i], xk[i], skk);
    dotq = fmaf(xq[i], gq[i], dotq);
    dotk = fmaf(xk[i], gk[i], dotk);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    sqq += __shfl_xor(sqq, m, 64);
    skk += __shfl_xor(skk, m, 64);
    dotq += __shfl_xor(dotq, m, 64);
    dotk += __shfl_xor(dotk, m, 64);
  }
  const float nq = sqrtf(sqq + 1e-6f), nk = sqrtf(skk + 1e-6f);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = lane + 64 * i;
    if (c >= dk) continue;
    const float vq = l2norm ? gq[i] / nq - xq[i] * dotq / (nq * nq * nq) : gq[i];
    const float vk = l2norm ? gk[i] / nk - xk[i] * dotk / (nk * nk * nk) : gk[i];
    from_f32(dq + tok * stride + h * dk + c, vq);
    from_f32(dk_out + tok * stride + h * dk + c, vk);
    from_f32(dalpha + row * dk + c, ga[i]);
  }
  if (lane == 0) {
    float sb = 0.f;
    for (int s = 0; s < n_vs; ++s) sb += part[(int64_t)n_vs * 3 * BTH * dk + (int64_t)s * BTH + row];
    from_f32(dbeta + row, sb);
  }
}

// The reverse pass over every (batch, head, segment, column slice) from G_end ([B][H][nseg]
// [dk][dv]; the sequence's dS_final when nseg = 1), then the sum over slices with the L2
// backward.
template <typename T>
hipError_t launch_bwd_t(const KdaArgs& a, const KdaGrads& g, const float* G_end, int64_t seg_len, int nseg,
                        float* ckpt, float* part, hipStream_t stream, Marks* marks) {
  const int n_vs = (int)((a.dv + 15) / 16);
  const int64_t blocks = a.B * a.H * n_vs * nseg;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), thr(256);
  const int dk = (int)a.dk, dv = (int)a.dv, nrm = a.l2norm ? 1 : 0;
  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  const T* al = static_cast<const T*>(a.alpha);
  const T* be = static_cast<const T*>(a.beta);
  const T* dout = static_cast<const T*>(g.dout);
  T* dvo = static_cast<T*>(g.dv);
#define CHM_BWD(R)                                                                                                   \
  hipLaunchKernelGGL((kda_bwd_kernel<T, R>), grid, thr, 0, stream, q, k, v, a.qkv_stride, al, be, dout, G_end,     \
                     dvo, g.dS0, ckpt, part, a.T, a.H, dk, dv, nrm, seg_len, nseg)
  if (dk <= 16) CHM_BWD(1);
  else if (dk <= 32) CHM_BWD(2);
  else if (dk <= 64) CHM_BWD(4);
  else if (dk <= 128) CHM_BWD(8);
  else return hipErrorInvalidValue;   // the entry point admits dk <= 128 only
#undef CHM_BWD
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = mark_after(marks, "kda_bwd_kernel", stream);
  if (e != hipSuccess) return e;
  const int64_t rows = a.B * a.T * a.H;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(kda_bwd_reduce_kernel<T>, dim3((unsigned)((rows + 3) / 4)), thr, 0, stream, q, k, a.qkv_stride,
                     part, n_vs, static_cast<T*>(g.dq), static_cast<T*>(g.dk), static_cast<T*>(g.dalpha),
                     static_cast<T*>(g.dbeta), rows, a.H, dk, nrm);
  e = hipGetLastError();
  return e != hipSuccess ? e : mark_after(marks, "kda_bwd_reduce_kernel", stream);
}

// ---- mShortConv backward ---------------------------------------------------------------

// dx: one thread = 8 channels of one token s; every (p, tap) whose tap reads s adds w dy[p]
template <typename T>
__global__ __launch_bounds__(256) void conv_bwd_dx_kernel(const T* __restrict__ dy, T* __restrict__ dx,
                                                          const float* __restrict__ w_text,
                                                          const float* __restrict__ w_vis, int64_t Ttot, int64_t C,
                                                          Seg seg) {
  const int64_t C8 = C / 8;
  const int64_t cg = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
  const int64_t local = (int64_t)blockIdx.y * 4 + (threadIdx.x >> 6);
  const int64_t b = blockIdx.z;
  if (cg >= C8 || local >= seg.length) return;
  const int64_t c0 = cg * 8, s = seg.start + local;
  const T* dyb = dy + b * Ttot * C;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](int64_t p, const float* w, int taps, int tap) {
    float g[8];
    load8(dyb + p * C + c0, g);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = fmaf(w[(c0 + i) * taps + tap], g[i], acc[i]);
  };
  if (seg.kind == SEG_TEXT) {
    for (int j = 0; j < kTextTaps; ++j) {   // tap j of token p reads p + j - 3
      const int64_t p = s + (kTextTaps - 1) - j;
      if (p < seg.start + seg.length) add(p, w_text, kTextTaps, j);
    }
  } else {
    const int64_t hw = (int64_t)seg.height * seg.width;
    const int64_t f = local / hw, hh = (local / seg.width) % seg.height, ww = local % seg.width;
    for (int kt = 0; kt < 3; ++kt)
      for (int kh = 0; kh < 3; ++kh)
        for (int kw = 0; kw < 3; ++kw) {   // tap (kt, kh, kw) of p reads p + (kt - 2, kh - 1, kw - 1)
          const int64_t pf = f + 2 - kt, ph = hh + 1 - kh, pw = ww + 1 - kw;
          if (grid_inside(seg, pf, ph, pw)) add(raster_index(seg, pf, ph, pw), w_vis, kVisTaps, kt * 9 + kh * 3 + kw);
        }
  }
  store8(dx + (b * Ttot + s) * C + c0, acc);
}

// dw: a thread owns 4 channels and a range of tokens of one segment, walks the range in
// raster order (grid coordinates advanced token by token, no divisions in the loop),
// accumulates every tap's sum of x[src] dy in registers, then adds it to dw with one atomic
// per value. KIND: text (4 taps), one-frame grid (the 9 taps of the current frame, dw_vis
// taps 18..26: earlier frames do not exist), video (27 taps).
template <typename T, int KIND>
__global__ __launch_bounds__(256) void conv_bwd_dw_kernel(const T* __restrict__ x, const T* __restrict__ dy,
                                                          float* __restrict__ dw, int64_t Ttot, int64_t C, Seg seg,
                                                          int64_t tokens_per_range) {
  constexpr int TAPS = KIND == SEG_TEXT ? kTextTaps : KIND == SEG_IMAGE ? 9 : kVisTaps;
  constexpr int TAP0 = KIND == SEG_IMAGE ? 18 : 0;
  constexpr int NW = KIND == SEG_TEXT ? kTextTaps : kVisTaps;
  const int64_t C4 = C / 4;
  const int64_t cg = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t p0 = (int64_t)blockIdx.y * tokens_per_range;
  const int64_t b = blockIdx.z;
  if (cg >= C4 || p0 >= seg.length) return;
  const int64_t c0 = cg * 4;
  const int64_t p1 = min<int64_t>(seg.length, p0 + tokens_per_range);
  const T* xb = x + b * Ttot * C;
  const T* dyb = dy + b * Ttot * C;
  float acc[TAPS][4];
#pragma unroll
  for (int t = 0; t < TAPS; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[t][i] = 0.f;
  auto ld4 = [&](const T* p, float (&o)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = to_f32(p[i]);
  };
  int f = 0, hh = 0, ww = 0;   // grid point of token p0
  if (KIND != SEG_TEXT) {
    const int64_t hw = (int64_t)seg.height * seg.width;
    f = (int)(p0 / hw);
    hh = (int)((p0 / seg.width) % seg.height);
    ww = (int)(p0 % seg.width);
  }
  for (int64_t local = p0; local < p1; ++local) {
    const int64_t p = seg.start + local;
    float g[4];
    ld4(dyb + p * C + c0, g);
    if (KIND == SEG_TEXT) {
#pragma unroll
      for (int j = 0; j < TAPS; ++j) {
        const int64_t src = text_tap_source(seg, p, j);
        if (src < 0) continue;
        float xv[4];
        ld4(xb + src * C + c0, xv);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] = fmaf(xv[i], g[i], acc[j][i]);
      }
    } else {
#pragma unroll
      for (int t = 0; t < TAPS; ++t) {
        const int tap = TAP0 + t;
        const int ff = f + tap / 9 - 2, h2 = hh + (tap / 3) % 3 - 1, w2 = ww + tap % 3 - 1;
        if (ff < 0 || h2 < 0 || h2 >= seg.height || w2 < 0 || w2 >= seg.width) continue;
        float xv[4];
        ld4(xb + raster_index(seg, ff, h2, w2) * C + c0, xv);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][i] = fmaf(xv[i], g[i], acc[t][i]);
      }
      if (++ww == seg.width) {
        ww = 0;
        if (++hh == seg.height) {
          hh = 0;
          ++f;
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TAPS; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) atomicAdd(dw + (c0 + i) * NW + TAP0 + t, acc[t][i]);
}

// dw of a grid segment. A wave owns 64 x CPT channels and a range of tokens, and walks it along
// the grid rows keeping the 3 x 3 (x frames) window of x around the current token in registers:
// per token it loads the window's new column only (3 or 9 rows instead of 9 or 27 taps), four
// tokens' loads at a time. Each window row is a buffer descriptor over one grid row of x (empty
// for rows outside the grid), addressed by the column through the wave-uniform offset, so
// columns past the edge read zero with no branch or select. The block's four waves walk four
// consecutive ranges of the same channels and add their sums in LDS before one atomic per value.
// Frames: one (an image: dw_vis taps 18..26) or three (video: all 27).
template <typename T, int CPT>
__device__ __forceinline__ void ld_cpt(__amdgpu_buffer_rsrc_t r, int voff, int soff, float (&o)[CPT]) {
  if constexpr (sizeof(T) == 2 && CPT == 4) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    o[0] = bf_lo(v[0]); o[1] = bf_hi(v[0]); o[2] = bf_lo(v[1]); o[3] = bf_hi(v[1]);
  } else if constexpr (sizeof(T) == 2) {
    const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
    o[0] = bf_lo(v); o[1] = bf_hi(v);
  } else if constexpr (CPT == 4) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    o[0] = __uint_as_float(v[0]); o[1] = __uint_as_float(v[1]); o[2] = __uint_as_float(v[2]); o[3] = __uint_as_float(v[3]);
  } else {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    o[0] = __uint_as_float(v[0]); o[1] = __uint_as_float(v[1]);
  }
}
constexpr int kDwWaves = 4;
template <typename T, int KIND, int CPT>
__global__ __launch_bounds__(64 * kDwWaves) void conv_bwd_dw_grid_kernel(const T* __restrict__ x,
                                                                         const T* __restrict__ dy,
                                                                         float* __restrict__ dw, int64_t Ttot, int64_t C,
                                                                         Seg seg, int64_t tokens_per_range) {
  constexpr int KT = KIND == SEG_IMAGE ? 1 : 3;
  constexpr int TAP0 = KIND == SEG_IMAGE ? 18 : 0;
  constexpr int NV = KT * 9 * CPT;
  constexpr int U = 4;   // tokens whose loads are issued together
  __shared__ float red[kDwWaves - 1][NV][64];
  // the wave index through readfirstlane: everything the buffer descriptors are built from is then
  // visibly wave-uniform (a descriptor in vector registers would loop over lanes at every load)
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t cg = (int64_t)blockIdx.x * 64 + lane;
  const int64_t p0 = ((int64_t)blockIdx.y * kDwWaves + w) * tokens_per_range;
  const int64_t b = blockIdx.z;
  const bool cok = cg < C / CPT;
  const int64_t c0 = cok ? cg * CPT : 0;
  const int voff = (int)(c0 * (int64_t)sizeof(T));
  const int rowb = (int)(seg.width * C * (int64_t)sizeof(T));   // bytes per grid row (below 2^31: checked by the host)
  const int colb = (int)(C * (int64_t)sizeof(T));
  const T* xb = x + b * Ttot * C;
  const T* dyb = dy + b * Ttot * C;
  const int H = seg.height, W = seg.width;
  const int64_t hw = (int64_t)H * W;
  float acc[KT][3][3][CPT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
#pragma unroll
    for (int kh = 0; kh < 3; ++kh)
#pragma unroll
      for (int kw = 0; kw < 3; ++kw)
#pragma unroll
        for (int i = 0; i < CPT; ++i) acc[kt][kh][kw][i] = 0.f;
  if (p0 < seg.length) {   // wave-uniform
    const int64_t p1 = min<int64_t>(seg.length, p0 + tokens_per_range);
    int f = (int)(p0 / hw), hh = (int)((p0 / W) % H), ww = (int)(p0 % W);
    float win[KT][3][3][CPT];
    int64_t local = p0;
    while (local < p1) {
      const int run = (int)min<int64_t>(W - ww, p1 - local);   // tokens left on this grid row
      __amdgpu_buffer_rsrc_t xr[KT][3];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int kh = 0; kh < 3; ++kh) {
          const int ff = f + kt - (KT - 1), h2 = hh + kh - 1;
          const bool rok = ff >= 0 && h2 >= 0 && h2 < H;
          xr[kt][kh] = __builtin_amdgcn_make_buffer_rsrc(
              (void*)(xb + (rok ? seg.start + (int64_t)ff * hw + (int64_t)h2 * W : 0) * C), 0, rok ? rowb : 0,
              0x00020000);
          if (ww > 0) ld_cpt<T, CPT>(xr[kt][kh], voff, (ww - 1) * colb, win[kt][kh][0]);
          else {
#pragma unroll
            for (int i = 0; i < CPT; ++i) win[kt][kh][0][i] = 0.f;
          }
          ld_cpt<T, CPT>(xr[kt][kh], voff, ww * colb, win[kt][kh][1]);
        }
      const auto dr = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(dyb + (seg.start + (int64_t)f * hw + (int64_t)hh * W) * C), 0, rowb, 0x00020000);
      // two groups of U tokens in flight: the next group's loads go out before this group's sums
      // (loads past the row's end read zero; tokens past the range's end add nothing)
      float colA[U][KT][3][CPT], gA[U][CPT], colB[U][KT][3][CPT], gB[U][CPT];
      auto issue = [&](int r, float (&col)[U][KT][3][CPT], float (&g)[U][CPT]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int kh = 0; kh < 3; ++kh) ld_cpt<T, CPT>(xr[kt][kh], voff, (ww + r + u + 1) * colb, col[u][kt][kh]);
          ld_cpt<T, CPT>(dr, voff, (ww + r + u) * colb, g[u]);
        }
      };
      auto sums = [&](int r, const float (&col)[U][KT][3][CPT], const float (&g)[U][CPT]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float keep = r + u < run ? 1.f : 0.f;   // wave-uniform
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int kh = 0; kh < 3; ++kh) {
#pragma unroll
              for (int i = 0; i < CPT; ++i) win[kt][kh][2][i] = col[u][kt][kh][i];
#pragma unroll
              for (int kw = 0; kw < 3; ++kw)
#pragma unroll
                for (int i = 0; i < CPT; ++i)
                  acc[kt][kh][kw][i] = fmaf(win[kt][kh][kw][i], g[u][i] * keep, acc[kt][kh][kw][i]);
#pragma unroll
              for (int i = 0; i < CPT; ++i) {
                win[kt][kh][0][i] = win[kt][kh][1][i];
                win[kt][kh][1][i] = win[kt][kh][2][i];
              }
            }
        }
      };
      issue(0, colA, gA);
      for (int r = 0; r < run; r += 2 * U) {
        issue(r + U, colB, gB);
        sums(r, colA, gA);
        issue(r + 2 * U, colA, gA);
        sums(r + U, colB, gB);
      }
      local += run;
      ww += run;
      if (ww == W) {
        ww = 0;
        if (++hh == H) {
          hh = 0;
          ++f;
        }
      }
    }
  }
  // the four waves' sums, then one atomic per value
  if (w > 0) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int kh = 0; kh < 3; ++kh)
#pragma unroll
        for (int kw = 0; kw < 3; ++kw)
#pragma unroll
          for (int i = 0; i < CPT; ++i) red[w - 1][((kt * 3 + kh) * 3 + kw) * CPT + i][lane] = acc[kt][kh][kw][i];
  }
  __syncthreads();
  if (w == 0 && cok) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int kh = 0; kh < 3; ++kh)
#pragma unroll
        for (int kw = 0; kw < 3; ++kw)
#pragma unroll
          for (int i = 0; i < CPT; ++i) {
            const int v = ((kt * 3 + kh) * 3 + kw) * CPT + i;
            float t = acc[kt][kh][kw][i];
#pragma unroll
            for (int ww2 = 0; ww2 < kDwWaves - 1; ++ww2) t += red[ww2][v][lane];
            atomicAdd(dw + (c0 + i) * kVisTaps + TAP0 + 9 * kt + 3 * kh + kw, t);
          }
  }
}

// Backward of Eq. 15's gate and norm (page 1, section 3.3), y = Sigmoid(g) * o r * w per
// (token, head) row of dv channels, r = 1 / sqrt(mean(o^2) + eps): with n = o r, s = Sigmoid(g)
// and dn = dy s w,
//   dg = dy n w s (1 - s),   do = r (dn - n mean(dn n)),   dw = sum over rows of dy s n.
// Waves walk the rows with a grid stride (lane l holds channels l, l + 64, ...), keep their dw
// sums in registers and add them to dw with one atomic per channel at the end.
template <typename T>
__global__ __launch_bounds__(256) void gate_norm_bwd_kernel(const T* __restrict__ o, const T* __restrict__ gate,
                                                            int64_t gate_stride, const float* __restrict__ w,
                                                            float eps, const T* __restrict__ dy, T* __restrict__ dout,
                                                            T* __restrict__ dgate, float* __restrict__ dw,
                                                            int64_t rows, int64_t H, int dv) {
  const int lane = threadIdx.x & 63;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  float wc[4], wsum[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = lane + 64 * i;
    wc[i] = c < dv ? (w != nullptr ? w[c] : 1.f) : 0.f;
    wsum[i] = 0.f;
  }
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < rows; row += nwaves) {
    const int64_t tok = row / H, h = row % H;
    const T* grow = gate + tok * gate_stride + h * dv;
    float x[4], sg[4], d[4], ss = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = lane + 64 * i;
      const bool ok = c < dv;
      x[i] = ok ? to_f32(o[row * dv + c]) : 0.f;
      sg[i] = ok ? 1.f / (1.f + expf(-to_f32(grow[c]))) : 0.f;
      d[i] = ok ? to_f32(dy[row * dv + c]) : 0.f;
      ss = fmaf(x[i], x[i], ss);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    const float r = 1.f / sqrtf(ss / (float)dv + eps);
    float n[4], dn[4], dot = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      n[i] = x[i] * r;
      dn[i] = d[i] * sg[i] * wc[i];
      dot = fmaf(dn[i], n[i], dot);
      wsum[i] = fmaf(d[i] * sg[i], n[i], wsum[i]);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) dot += __shfl_xor(dot, m, 64);
    const float mean_dn_n = dot / (float)dv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = lane + 64 * i;
      if (c < dv) {
        from_f32(dout + row * dv + c, r * (dn[i] - n[i] * mean_dn_n));
        from_f32(dgate + tok * gate_stride + h * dv + c, d[i] * n[i] * wc[i] * sg[i] * (1.f - sg[i]));
      }
    }
  }
  if (dw != nullptr) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + 64 * i < dv) atomicAdd(dw + lane + 64 * i, wsum[i]);
  }
}

__global__ void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

hipError_t zero(float* p, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

template <typename T>
hipError_t conv_bwd_t(const void* x, const void* dy, void* dx, float* dw_text, float* dw_vis, int64_t B, int64_t Ttot,
                      int64_t C, const float* w_text, const float* w_vis, const Seg* segs, int nseg,
                      hipStream_t stream, Marks* marks) {
  if (B > 65535) return hipErrorInvalidValue;   // grid z of the per-segment kernels; checked before any write
  hipError_t e = zero(dw_text, C * kTextTaps, stream);
  if (e == hipSuccess) e = zero(dw_vis, C * kVisTaps, stream);
  if (e != hipSuccess) return e;
  // dx of the image grids that the rows kernel takes: that kernel with mirrored taps, in one launch
  std::vector<Seg> rows;
  const bool bf16 = sizeof(T) == 2;
  for (int i = 0; i < nseg; ++i)
    if (segs[i].length > 0 && conv_rows_adjoint_ok(segs[i], C, bf16)) rows.push_back(segs[i]);
  e = launch_conv_rows_adjoint(dy, dx, w_vis, B, Ttot, C, rows.data(), (int)rows.size(), stream, nullptr);
  if (e != hipSuccess) return e;
  for (int i = 0; i < nseg; ++i) {
    const Seg& sg = segs[i];
    if (sg.length == 0) continue;
    if (!conv_rows_adjoint_ok(sg, C, bf16) && conv_tile_adjoint_ok(sg, C, bf16)) {   // video grids
      e = launch_conv_tile_adjoint(dy, dx, w_vis, B, Ttot, C, sg, stream, nullptr);
      if (e != hipSuccess) return e;
    } else if (!conv_rows_adjoint_ok(sg, C, bf16)) {   // text, fp32
      const dim3 gx((unsigned)((C / 8 + 63) / 64), (unsigned)((sg.length + 3) / 4), (unsigned)B);
      hipLaunchKernelGGL(conv_bwd_dx_kernel<T>, gx, dim3(256), 0, stream, static_cast<const T*>(dy),
                         static_cast<T*>(dx), w_text, w_vis, Ttot, C, sg);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    // dw: about 512 token ranges per segment and batch item
    const int64_t per = std::max<int64_t>(16, (sg.length + 511) / 512);
    const int64_t ranges = (sg.length + per - 1) / per;
    const bool grid_rows = (int64_t)sg.width * C * (int64_t)sizeof(T) < (int64_t(1) << 31);
    if (sg.kind == SEG_TEXT || !grid_rows) {
      const dim3 gw((unsigned)((C / 4 + 255) / 256), (unsigned)ranges, (unsigned)B);
      if (sg.kind == SEG_TEXT)
        hipLaunchKernelGGL((conv_bwd_dw_kernel<T, SEG_TEXT>), gw, dim3(256), 0, stream, static_cast<const T*>(x),
                           static_cast<const T*>(dy), dw_text, Ttot, C, sg, per);
      else if (sg.frames == 1)
        hipLaunchKernelGGL((conv_bwd_dw_kernel<T, SEG_IMAGE>), gw, dim3(256), 0, stream, static_cast<const T*>(x),
                           static_cast<const T*>(dy), dw_vis, Ttot, C, sg, per);
      else
        hipLaunchKernelGGL((conv_bwd_dw_kernel<T, SEG_VIDEO>), gw, dim3(256), 0, stream, static_cast<const T*>(x),
                           static_cast<const T*>(dy), dw_vis, Ttot, C, sg, per);
    } else {
      const unsigned ry = (unsigned)((ranges + kDwWaves - 1) / kDwWaves);
      if (sg.frames == 1)
        hipLaunchKernelGGL((conv_bwd_dw_grid_kernel<T, SEG_IMAGE, 4>), dim3((unsigned)((C / 4 + 63) / 64), ry, (unsigned)B),
                           dim3(64 * kDwWaves), 0, stream, static_cast<const T*>(x), static_cast<const T*>(dy), dw_vis,
                           Ttot, C, sg, per);
      else
        hipLaunchKernelGGL((conv_bwd_dw_grid_kernel<T, SEG_VIDEO, 2>), dim3((unsigned)((C / 2 + 63) / 64), ry, (unsigned)B),
                           dim3(64 * kDwWaves), 0, stream, static_cast<const T*>(x), static_cast<const T*>(dy), dw_vis,
                           Ttot, C, sg, per);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return mark_after(marks, "conv_bwd_kernels", stream);
}


template <typename T>
hipError_t launch_local_t(const KdaArgs& a, const KdaGrads& g, float* E, int64_t seg_len, int nseg,
                          hipStream_t stream) {
  const int n_vs = (int)((a.dv + 15) / 16);
  const dim3 grid((unsigned)(a.B * a.H * n_vs * nseg)), thr(256);
  const int dk = (int)a.dk, dv = (int)a.dv, nrm = a.l2norm ? 1 : 0;
  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* al = static_cast<const T*>(a.alpha);
  const T* be = static_cast<const T*>(a.beta);
  const T* dout = static_cast<const T*>(g.dout);
#define CHM_LOC(R)                                                                                            \
  hipLaunchKernelGGL((kda_bwd_local_kernel<T, R>), grid, thr, 0, stream, q, k, a.qkv_stride, al, be, dout, E, \
                     a.T, a.H, dk, dv, nrm, seg_len, nseg)
  if (dk <= 16) CHM_LOC(1);
  else if (dk <= 32) CHM_LOC(2);
  else if (dk <= 64) CHM_LOC(4);
  else if (dk <= 128) CHM_LOC(8);
  else return hipErrorInvalidValue;
#undef CHM_LOC
  return hipGetLastError();
}

// How a sequence is cut for the backward: enough segments that the blocks of one pass fill
// the chip about eight times over, each at least kMinSeg tokens, the length a multiple of
// the 16-token checkpoint spacing.
constexpr int64_t kBwdBlocks = 2048, kMinSeg = 64;
struct BwdCut {
  int64_t len;
  int nseg;
};
BwdCut bwd_cut(int64_t B, int64_t T, int64_t H, int64_t dv) {
  const int64_t base = B * H * ((dv + 15) / 16);
  int64_t P = base > 0 ? (kBwdBlocks + base - 1) / base : 1;
  P = std::min<int64_t>(P, std::max<int64_t>(1, T / kMinSeg));
  if (P <= 1) return {T, 1};
  const int64_t len = ((T + P - 1) / P + kCk - 1) / kCk * kCk;
  P = (T + len - 1) / len;
  return P <= 1 ? BwdCut{T, 1} : BwdCut{len, (int)P};
}

}  // namespace

size_t kda_bwd_workspace(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv) {
  const int64_t n_vs = (dv + 15) / 16;
  const int64_t ck = B * H * ((T + kCk - 1) / kCk) * dk * dv;
  const int64_t parts = n_vs * B * T * H * (3 * dk + 1);
  const BwdCut c = bwd_cut(B, T, H, dv);
  const int64_t segs = c.nseg > 1 ? B * H * c.nseg * (4 * dk * dv + dk * dk) : 0;
  return (size_t)(ck + parts + segs) * sizeof(float);
}

// Cut into segments, the reverse recurrence runs on all of them at once. Per segment p, on the
// token-by-token kernels: its own end state from a zero start (L_p) and its transition product
// (M_p, from the identity with v = 0); the chain gives every segment's start state, from which
// the checkpoints are taken; the reverse recurrence from zero gives the segment's own part of
// dL/dS at its start (E_p); the backward chain gives dL/dS at every segment's end; then the
// reverse pass proper runs per segment from there.
hipError_t launch_kda_backward(const KdaArgs& a, const KdaGrads& g, void* workspace, hipStream_t stream,
                               Marks* marks) {
  if (a.B * a.H == 0) return hipSuccess;
  const BwdCut c = bwd_cut(a.B, a.T, a.H, a.dv);
  // every pass's grid must fit before the first launch
  const int64_t slices = std::max((a.dv + 15) / 16, (a.dk + 15) / 16);
  if (a.B * a.H * slices * c.nseg > 0x7fffffff) return hipErrorInvalidValue;
  const int64_t sz = a.B * a.H * c.nseg * a.dk * a.dv;
  float* ckpt = static_cast<float*>(workspace);
  float* part = ckpt + a.B * a.H * ((a.T + kCk - 1) / kCk) * a.dk * a.dv;
  float* Lw = part + ((a.dv + 15) / 16) * a.B * a.T * a.H * (3 * a.dk + 1);
  float* Sst = Lw + sz;
  float* Ew = Sst + sz;
  float* Gend = Ew + sz;
  float* Mw = Gend + sz;
  // forward passes without o, S_final or gate
  KdaArgs f = a;
  f.o = nullptr;
  f.S_final = nullptr;
  f.gate = nullptr;
  f.q = nullptr;
  hipError_t e = hipSuccess;
  const float* G_end = g.dS_final;
  if (c.nseg > 1) {
    const int64_t chains = a.B * a.H * ((a.dv + 15) / 16);
    SeqSegs sl;
    sl.len = c.len;
    sl.nseg = c.nseg;
    sl.Send = Lw;
    sl.zero_start = 1;
    e = launch_kda_sequential(f, stream, marks, nullptr, &sl);
    if (e != hipSuccess) return e;
    KdaArgs fm = f;
    fm.v = nullptr;
    fm.dv = a.dk;
    SeqSegs sm = sl;
    sm.Send = Mw;
    sm.zero_start = 0;
    sm.identity = 1;
    e = launch_kda_sequential(fm, stream, marks, nullptr, &sm);
    if (e != hipSuccess) return e;
    e = chain_launch(false, Mw, Lw, a.S0, Sst, chains, c.nseg, (int)a.dk, (int)a.dv, stream);
    if (e != hipSuccess) return e;
    SeqSegs sc;
    sc.len = c.len;
    sc.nseg = c.nseg;
    sc.Sseg = Sst;
    e = launch_kda_sequential(f, stream, marks, ckpt, &sc);
    if (e != hipSuccess) return e;
    e = a.bf16 ? launch_local_t<uint16_t>(a, g, Ew, c.len, c.nseg, stream)
               : launch_local_t<float>(a, g, Ew, c.len, c.nseg, stream);
    if (e == hipSuccess) e = mark_after(marks, "kda_bwd_local_kernel", stream);
    if (e != hipSuccess) return e;
    e = chain_launch(true, Mw, Ew, g.dS_final, Gend, chains, c.nseg, (int)a.dk, (int)a.dv, stream);
    if (e == hipSuccess) e = mark_after(marks, "kda_chain_kernel", stream);
    if (e != hipSuccess) return e;
    G_end = Gend;
  } else {
    e = launch_kda_sequential(f, stream, marks, ckpt);
    if (e != hipSuccess) return e;
  }
  return a.bf16 ? launch_bwd_t<uint16_t>(a, g, G_end, c.len, c.nseg, ckpt, part, stream, marks)
                : launch_bwd_t<float>(a, g, G_end, c.len, c.nseg, ckpt, part, stream, marks);
}

hipError_t launch_kda_chain(bool back, const float* M, const float* X, const float* init, float* Y, int64_t BH,
                            int nseg, int dk, int dv, hipStream_t stream) {
  const int64_t chains = BH * ((dv + 15) / 16);
  if (chains == 0) return hipSuccess;
  if (chains > 0x7fffffff || dk > 128) return hipErrorInvalidValue;
  return chain_launch(back, M, X, init, Y, chains, nseg, dk, dv, stream);
}

hipError_t launch_gate_norm_backward(const void* o, const void* gate, int64_t gate_stride, const float* norm_w,
                                     float eps, const void* dy, void* dout, void* dgate, float* dnorm_w, int64_t rows,
                                     int64_t H, int64_t dv, bool bf16, hipStream_t stream) {
  if (dnorm_w != nullptr) {
    const hipError_t e = zero(dnorm_w, dv, stream);
    if (e != hipSuccess) return e;
  }
  if (rows == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((rows + 3) / 4, 4096);
  const dim3 g((unsigned)blocks), t(256);
  if (bf16)
    hipLaunchKernelGGL(gate_norm_bwd_kernel<uint16_t>, g, t, 0, stream, static_cast<const uint16_t*>(o),
                       static_cast<const uint16_t*>(gate), gate_stride, norm_w, eps, static_cast<const uint16_t*>(dy),
                       static_cast<uint16_t*>(dout), static_cast<uint16_t*>(dgate), dnorm_w, rows, H, (int)dv);
  else
    hipLaunchKernelGGL(gate_norm_bwd_kernel<float>, g, t, 0, stream, static_cast<const float*>(o),
                       static_cast<const float*>(gate), gate_stride, norm_w, eps, static_cast<const float*>(dy),
                       static_cast<float*>(dout), static_cast<float*>(dgate), dnorm_w, rows, H, (int)dv);
  return hipGetLastError();
}

hipError_t launch_conv_backward(const void* x, const void* dy, void* dx, float* dw_text, float* dw_vis, int64_t B,
                                int64_t T, int64_t C, bool bf16, const float* w_text, const float* w_vis,
                                const Seg* segs, int nseg, hipStream_t stream, Marks* marks) {
  return bf16 ? conv_bwd_t<uint16_t>(x, dy, dx, dw_text, dw_vis, B, T, C, w_text, w_vis, segs, nseg, stream, marks)
              : conv_bwd_t<float>(x, dy, dx, dw_text, dw_vis, B, T, C, w_text, w_vis, segs, nseg, stream, marks);
}

}  // namespace chm
