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
// recomputed from its checkpoint, eight states at a time in registers.
//
// One block per (batch, head, 16-column slice of d_v), 256 threads = 16 columns x
// 16 row-threads as in the forward kernel: the column-wise quantities (dv) are
// complete in a block, the row-wise ones (dq, dk, dalpha, dbeta) are sums over all
// columns: each block sums its 16 columns (permlane swaps inside a wave, LDS atomic
// adds across the four waves, written out once per eight tokens) and writes a
// per-slice partial; a second kernel adds the slices and applies the L2
// normalisation's backward. Gradients of q, k and v are written at the inputs'
// token stride, so that they can fill one fused q|k|v gradient for the conv.
//
// mShortConv (page 1, section 3.4; Eq. 13): y[p, c] = sum_taps w[c, tap] x[src(p, tap), c]
// gives dx[s, c] = sum over (p, tap) with src(p, tap) = s of w[c, tap] dy[p, c] (the
// adjoint gather: p is s moved back by the tap's offset, inside the same segment) and
// dw[c, tap] = sum_p x[src(p, tap), c] dy[p, c] (summed over tokens and batch items).
#include "dtypes.h"
#include "internal.h"

namespace chm {
namespace {

constexpr int kCk = 16;   // tokens per checkpoint (the forward kernel's token batch)
constexpr int kHalf = 8;  // states recomputed and kept at a time

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// sum over the 16 lanes of a DPP row (the row-threads of one column), in every lane
__device__ __forceinline__ float sum16(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}
// sum over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four columns of one wave), in every lane
__device__ __forceinline__ float sum_cols4(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = __int_as_float(r[0]) + __int_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

template <typename T, int RPT>
__global__ __launch_bounds__(256) void kda_bwd_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, int64_t stride,
    const T* __restrict__ alpha, const T* __restrict__ beta, const T* __restrict__ dout,
    const float* __restrict__ dS_final, T* __restrict__ dv_out, float* __restrict__ dS0,
    const float* __restrict__ ckpt, float* __restrict__ part, int64_t Tn, int64_t H, int dk, int dv, int l2norm) {
  constexpr int DKP = 16 * RPT;
  __shared__ float sq[kCk][DKP], sk[kCk][DKP], sa[kCk][DKP];
  __shared__ float sv[kCk][16], sdo[kCk][16], sb[kCk];
  __shared__ float red[kHalf][3][DKP];   // sums of dq, dk, dalpha over the block's 16 columns
  __shared__ float redb[kHalf];

  const int n_vs = (dv + 15) / 16;
  const int64_t bh = blockIdx.x / n_vs;
  const int vs = blockIdx.x % n_vs;
  const int64_t b = bh / H, h = bh % H;
  const int tid = threadIdx.x, colid = tid >> 4, rt = tid & 15;
  const int col = vs * 16 + colid;
  const bool col_ok = col < dv;
  const int64_t nb = (Tn + kCk - 1) / kCk;
  const int64_t BTH = (int64_t)gridDim.x / n_vs * Tn;   // B * H * T: one partial array's rows
  float* pq = part + (int64_t)vs * 3 * BTH * dk;        // this slice's partials
  float* pk = pq + BTH * dk;
  float* pa = pk + BTH * dk;
  float* pb = part + (int64_t)n_vs * 3 * BTH * dk + (int64_t)vs * BTH;

  float G[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rt + 16 * i;
    G[i] = (dS_final != nullptr && col_ok && row < dk) ? dS_final[(bh * dk + row) * dv + col] : 0.f;
  }
  for (int e = tid; e < kHalf * 3 * DKP; e += 256) (&red[0][0][0])[e] = 0.f;
  if (tid < kHalf) redb[tid] = 0.f;

  // forward step on the staged token tt: S <- S + k (beta w)^T after the decay; returns w
  auto step = [&](float (&S)[RPT], int tt) {
    float pred = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      S[i] *= sa[tt][rt + 16 * i];
      pred = fmaf(S[i], sk[tt][rt + 16 * i], pred);
    }
    const float w = sv[tt][colid] - sum16(pred);
    const float bw = sb[tt] * w;
#pragma unroll
    for (int i = 0; i < RPT; ++i) S[i] = fmaf(sk[tt][rt + 16 * i], bw, S[i]);
    return w;
  };

  for (int64_t kb = nb - 1; kb >= 0; --kb) {
    const int64_t t0 = kb * kCk;
    const int nt = (int)min<int64_t>(kCk, Tn - t0);
    __syncthreads();   // the previous block's reads of the staging arrays are done
    {  // stage: thread (colid, rt) loads token colid, rows rt + 16 i; q and k normalised
      const bool tok_ok = colid < nt;
      const int64_t tok = b * Tn + t0 + colid;
      float rq[RPT], rk[RPT], ssq = 0.f, ssk = 0.f;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int row = rt + 16 * i;
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
        sq[colid][rt + 16 * i] = rq[i] * nq;
        sk[colid][rt + 16 * i] = rk[i] * nk;
      }
      const int vc = vs * 16 + rt;   // token colid, column rt of the slice
      sv[colid][rt] = (tok_ok && vc < dv) ? to_f32(v[tok * stride + h * dv + vc]) : 0.f;
      sdo[colid][rt] = (tok_ok && vc < dv) ? to_f32(dout[(tok * H + h) * dv + vc]) : 0.f;
      if (rt == 0) sb[colid] = tok_ok ? to_f32(beta[tok * H + h]) : 0.f;
    }
    __syncthreads();
    float S0c[RPT];   // the state before token t0
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = rt + 16 * i;
      S0c[i] = (col_ok && row < dk) ? ckpt[((bh * nb + kb) * dk + row) * dv + col] : 0.f;
    }
    for (int half = 1; half >= 0; --half) {
      const int h0 = half * kHalf;
      const int hn = min(kHalf, nt - h0);
      if (hn <= 0) continue;
      float S[RPT];
#pragma unroll
      for (int i = 0; i < RPT; ++i) S[i] = S0c[i];
      for (int tt = 0; tt < h0; ++tt) step(S, tt);   // to the half's first token
      float Sp[kHalf][RPT], wv[kHalf];
#pragma unroll
      for (int j = 0; j < kHalf; ++j) {
        if (j < hn) {
#pragma unroll
          for (int i = 0; i < RPT; ++i) Sp[j][i] = S[i];
          wv[j] = step(S, h0 + j);
        }
      }
      // backward over the half; S is the state after its last token
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
          G[i] = fmaf(sq[tt][rt + 16 * i], doc, G[i]);
          r = fmaf(G[i], sk[tt][rt + 16 * i], r);
        }
        r = sum16(r);
        if (rt == 0 && col_ok) from_f32(dv_out + (b * Tn + t0 + tt) * stride + h * dv + col, bt * r);
        const float dbr = sum_cols4(r * w);
        if ((tid & 63) == 0) atomicAdd(&redb[j], dbr);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          const int row = rt + 16 * i;
          const float a = sa[tt][row];
          const float dqv = St[i] * doc;
          const float dkv = bt * (G[i] * w - a * Sp[j][i] * r);
          const float dP = G[i] - bt * sk[tt][row] * r;
          const float dav = dP * Sp[j][i];
          G[i] = a * dP;
          const float s0 = sum_cols4(dqv), s1 = sum_cols4(dkv), s2 = sum_cols4(dav);
          if ((tid & 63) < 16) {
            atomicAdd(&red[j][0][row], s0);
            atomicAdd(&red[j][1][row], s1);
            atomicAdd(&red[j][2][row], s2);
          }
        }
      }
      __syncthreads();
      // this slice's sums over its 16 columns -> the partial arrays
      for (int e = tid; e < hn * DKP; e += 256) {
        const int j = e / DKP, row = e % DKP;
        if (row >= dk) continue;
        const int64_t o = ((b * Tn + t0 + h0 + j) * H + h) * dk + row;
        pq[o] = red[j][0][row];
        pk[o] = red[j][1][row];
        pa[o] = red[j][2][row];
      }
      if (tid < hn) pb[(b * Tn + t0 + h0 + tid) * H + h] = redb[tid];
      __syncthreads();
      for (int e = tid; e < kHalf * 3 * DKP; e += 256) (&red[0][0][0])[e] = 0.f;
      if (tid < kHalf) redb[tid] = 0.f;
    }
  }
  if (dS0 != nullptr && col_ok) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = rt + 16 * i;
      if (row < dk) dS0[(bh * dk + row) * dv + col] = G[i];
    }
  }
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

template <typename T>
hipError_t launch_bwd_t(const KdaArgs& a, const KdaGrads& g, float* ckpt, float* part, hipStream_t stream,
                        Marks* marks) {
  const int n_vs = (int)((a.dv + 15) / 16);
  const int64_t blocks = a.B * a.H * n_vs;
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
  hipLaunchKernelGGL((kda_bwd_kernel<T, R>), grid, thr, 0, stream, q, k, v, a.qkv_stride, al, be, dout, g.dS_final, \
                     dvo, g.dS0, ckpt, part, a.T, a.H, dk, dv, nrm)
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

// dw: a thread owns 4 channels and a range of tokens of one segment, accumulates every
// tap's sum of x[src] dy in registers, then adds it to dw with one atomic per value
template <typename T, int TAPS>
__global__ __launch_bounds__(256) void conv_bwd_dw_kernel(const T* __restrict__ x, const T* __restrict__ dy,
                                                          float* __restrict__ dw, int64_t Ttot, int64_t C, Seg seg,
                                                          int64_t tokens_per_range) {
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
  for (int64_t local = p0; local < p1; ++local) {
    const int64_t p = seg.start + local;
    float g[4];
    ld4(dyb + p * C + c0, g);
    if (TAPS == kTextTaps) {
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
      const int64_t hw = (int64_t)seg.height * seg.width;
      const int64_t f = local / hw, hh = (local / seg.width) % seg.height, ww = local % seg.width;
#pragma unroll
      for (int t = 0; t < TAPS; ++t) {
        const int64_t src = vis_tap_source(seg, f, hh, ww, t / 9, (t / 3) % 3, t % 3);
        if (src < 0) continue;
        float xv[4];
        ld4(xb + src * C + c0, xv);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][i] = fmaf(xv[i], g[i], acc[t][i]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TAPS; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) atomicAdd(dw + (c0 + i) * TAPS + t, acc[t][i]);
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
  hipError_t e = zero(dw_text, C * kTextTaps, stream);
  if (e == hipSuccess) e = zero(dw_vis, C * kVisTaps, stream);
  if (e != hipSuccess) return e;
  if (B > 65535) return hipErrorInvalidValue;
  for (int i = 0; i < nseg; ++i) {
    const Seg& sg = segs[i];
    if (sg.length == 0) continue;
    const dim3 gx((unsigned)((C / 8 + 63) / 64), (unsigned)((sg.length + 3) / 4), (unsigned)B);
    hipLaunchKernelGGL(conv_bwd_dx_kernel<T>, gx, dim3(256), 0, stream, static_cast<const T*>(dy),
                       static_cast<T*>(dx), w_text, w_vis, Ttot, C, sg);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // dw: about 64 token ranges per segment and batch item
    const int64_t per = std::max<int64_t>(16, (sg.length + 63) / 64);
    const dim3 gw((unsigned)((C / 4 + 255) / 256), (unsigned)((sg.length + per - 1) / per), (unsigned)B);
    if (sg.kind == SEG_TEXT)
      hipLaunchKernelGGL((conv_bwd_dw_kernel<T, kTextTaps>), gw, dim3(256), 0, stream, static_cast<const T*>(x),
                         static_cast<const T*>(dy), dw_text, Ttot, C, sg, per);
    else
      hipLaunchKernelGGL((conv_bwd_dw_kernel<T, kVisTaps>), gw, dim3(256), 0, stream, static_cast<const T*>(x),
                         static_cast<const T*>(dy), dw_vis, Ttot, C, sg, per);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return mark_after(marks, "conv_bwd_kernels", stream);
}

}  // namespace

size_t kda_bwd_workspace(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv) {
  const int64_t n_vs = (dv + 15) / 16;
  const int64_t ck = B * H * ((T + kCk - 1) / kCk) * dk * dv;
  const int64_t parts = n_vs * B * T * H * (3 * dk + 1);
  return (size_t)(ck + parts) * sizeof(float);
}

hipError_t launch_kda_backward(const KdaArgs& a, const KdaGrads& g, void* workspace, hipStream_t stream,
                               Marks* marks) {
  if (a.B * a.H == 0) return hipSuccess;
  float* ckpt = static_cast<float*>(workspace);
  float* part = ckpt + a.B * a.H * ((a.T + kCk - 1) / kCk) * a.dk * a.dv;
  // forward pass keeping the checkpoints (no o, no S_final, no gate)
  KdaArgs f = a;
  f.o = nullptr;
  f.S_final = nullptr;
  f.gate = nullptr;
  hipError_t e = launch_kda_sequential(f, stream, marks, ckpt);
  if (e != hipSuccess) return e;
  return a.bf16 ? launch_bwd_t<uint16_t>(a, g, ckpt, part, stream, marks)
                : launch_bwd_t<float>(a, g, ckpt, part, stream, marks);
}

hipError_t launch_conv_backward(const void* x, const void* dy, void* dx, float* dw_text, float* dw_vis, int64_t B,
                                int64_t T, int64_t C, bool bf16, const float* w_text, const float* w_vis,
                                const Seg* segs, int nseg, hipStream_t stream, Marks* marks) {
  return bf16 ? conv_bwd_t<uint16_t>(x, dy, dx, dw_text, dw_vis, B, T, C, w_text, w_vis, segs, nseg, stream, marks)
              : conv_bwd_t<float>(x, dy, dx, dw_text, dw_vis, B, T, C, w_text, w_vis, segs, nseg, stream, marks);
}

}  // namespace chm
