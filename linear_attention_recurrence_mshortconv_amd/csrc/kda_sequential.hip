// Token-by-token KDA forward in fp32 (any dk, dv <= 256; fp32 or bf16 storage).
//
// Chimera page 1, section 3.3: Eq. 14 with page 2's parenthesisation,
//   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
// computed as S <- Diag(alpha_t) S; u = beta_t (v_t - S^T k_t); S <- S + k_t u^T;
// and the readout o_t = S_t^T q_t (inner term of Eq. 15). The state is fp32
// (page 1, section 5.6: FP32 KDA state).
//
// One block per (batch, head, 16-column slice of d_v); 256 threads = 16 columns
// x 16 row-threads. A row-thread holds rows rt, rt+16, ... of its column in
// registers; the two reductions over d_k per token are 16-lane shuffles. Tokens
// are staged in LDS 16 at a time.
#include "dtypes.h"
#include "internal.h"

namespace chm {
namespace {

constexpr int kTokBatch = 16;
constexpr int kMaxRowsPerThread = 16;   // dk <= 256

template <typename T>
__global__ __launch_bounds__(256) void kda_seq_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                      const T* __restrict__ v, int64_t stride,
                                                      const T* __restrict__ alpha, const T* __restrict__ beta,
                                                      const float* __restrict__ S0, T* __restrict__ o,
                                                      float* __restrict__ S_final, int64_t Tn, int64_t H, int dk,
                                                      int dv, int l2norm) {
  __shared__ float sk[kTokBatch][256];
  __shared__ float sq[kTokBatch][256];
  __shared__ float sa[kTokBatch][256];
  __shared__ float sv[kTokBatch][16];
  __shared__ float sb[kTokBatch];

  const int n_vs = (dv + 15) / 16;
  const int64_t bh = blockIdx.x / n_vs;
  const int vs = blockIdx.x % n_vs;
  const int64_t b = bh / H, h = bh % H;
  const int tid = threadIdx.x;
  const int colid = tid >> 4, rt = tid & 15;
  const int col = vs * 16 + colid;
  const bool col_ok = col < dv;

  float s[kMaxRowsPerThread];
#pragma unroll
  for (int i = 0; i < kMaxRowsPerThread; ++i) {
    const int row = rt + 16 * i;
    s[i] = (S0 != nullptr && col_ok && row < dk) ? S0[(bh * dk + row) * dv + col] : 0.f;
  }

  for (int64_t t0 = 0; t0 < Tn; t0 += kTokBatch) {
    const int nt = (int)min<int64_t>(kTokBatch, Tn - t0);
    __syncthreads();
    for (int e = tid; e < kTokBatch * 256; e += 256) {
      const int tt = e / 256, i = e % 256;
      float kv = 0.f, qv = 0.f, av = 1.f;
      if (tt < nt && i < dk) {
        const int64_t tok = b * Tn + t0 + tt;
        kv = to_f32(k[tok * stride + h * dk + i]);
        qv = to_f32(q[tok * stride + h * dk + i]);
        av = to_f32(alpha[(tok * H + h) * dk + i]);
      }
      sk[tt][i] = kv; sq[tt][i] = qv; sa[tt][i] = av;
    }
    for (int e = tid; e < kTokBatch * 16; e += 256) {
      const int tt = e / 16, c = vs * 16 + e % 16;
      const int64_t tok = b * Tn + t0 + tt;
      sv[tt][e % 16] = (tt < nt && c < dv) ? to_f32(v[tok * stride + h * dv + c]) : 0.f;
    }
    for (int e = tid; e < kTokBatch; e += 256) {
      const int64_t tok = b * Tn + t0 + e;
      sb[e] = e < nt ? to_f32(beta[tok * H + h]) : 0.f;
    }
    __syncthreads();
    if (l2norm) {
      // one wave per 4 tokens: x / sqrt(sum x^2 + 1e-6) over d_k, for q and k
      const int wave = tid >> 6, lane = tid & 63;
      for (int tt = wave; tt < nt; tt += 4) {
        float ssk = 0.f, ssq = 0.f;
        for (int i = lane; i < dk; i += 64) { ssk += sk[tt][i] * sk[tt][i]; ssq += sq[tt][i] * sq[tt][i]; }
        for (int off = 32; off > 0; off >>= 1) { ssk += __shfl_xor(ssk, off); ssq += __shfl_xor(ssq, off); }
        const float rk = 1.f / sqrtf(ssk + 1e-6f), rq = 1.f / sqrtf(ssq + 1e-6f);
        for (int i = lane; i < dk; i += 64) { sk[tt][i] *= rk; sq[tt][i] *= rq; }
      }
      __syncthreads();
    }
    for (int tt = 0; tt < nt; ++tt) {
      float pred = 0.f;
#pragma unroll
      for (int i = 0; i < kMaxRowsPerThread; ++i) {
        const int row = rt + 16 * i;
        if (row < dk) {
          s[i] *= sa[tt][row];
          pred = fmaf(s[i], sk[tt][row], pred);
        }
      }
      pred += __shfl_xor(pred, 1, 16);
      pred += __shfl_xor(pred, 2, 16);
      pred += __shfl_xor(pred, 4, 16);
      pred += __shfl_xor(pred, 8, 16);
      const float u = sb[tt] * (sv[tt][colid] - pred);
      float out = 0.f;
#pragma unroll
      for (int i = 0; i < kMaxRowsPerThread; ++i) {
        const int row = rt + 16 * i;
        if (row < dk) {
          s[i] = fmaf(sk[tt][row], u, s[i]);
          out = fmaf(s[i], sq[tt][row], out);
        }
      }
      out += __shfl_xor(out, 1, 16);
      out += __shfl_xor(out, 2, 16);
      out += __shfl_xor(out, 4, 16);
      out += __shfl_xor(out, 8, 16);
      if (rt == 0 && col_ok) from_f32(o + ((b * Tn + t0 + tt) * H + h) * dv + col, out);
    }
  }
  if (S_final != nullptr && col_ok) {
#pragma unroll
    for (int i = 0; i < kMaxRowsPerThread; ++i) {
      const int row = rt + 16 * i;
      if (row < dk) S_final[(bh * dk + row) * dv + col] = s[i];
    }
  }
}

}  // namespace

hipError_t launch_kda_sequential(const KdaArgs& a, hipStream_t stream, Marks* marks) {
  if (a.B * a.H == 0) return hipSuccess;
  const int n_vs = (int)((a.dv + 15) / 16);
  const int64_t blocks = a.B * a.H * n_vs;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (a.T == 0 && a.S_final == nullptr) return hipSuccess;
  if (a.bf16) {
    hipLaunchKernelGGL(kda_seq_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), a.qkv_stride, static_cast<const uint16_t*>(a.alpha),
                       static_cast<const uint16_t*>(a.beta), a.S0, static_cast<uint16_t*>(a.o), a.S_final, a.T, a.H,
                       (int)a.dk, (int)a.dv, (int)a.l2norm);
  } else {
    hipLaunchKernelGGL(kda_seq_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const float*>(a.q), static_cast<const float*>(a.k), static_cast<const float*>(a.v),
                       a.qkv_stride, static_cast<const float*>(a.alpha), static_cast<const float*>(a.beta), a.S0,
                       static_cast<float*>(a.o), a.S_final, a.T, a.H, (int)a.dk, (int)a.dv, (int)a.l2norm);
  }
  const hipError_t e = hipGetLastError();
  return e != hipSuccess ? e : mark_after(marks, "kda_seq_kernel", stream);
}

}  // namespace chm
