// Token-by-token KDA forward in fp32 (any dk, dv <= 256; fp32 or bf16 storage), and the
// output gate and norm of Eq. 15 as a separate in-place pass over o.
//
// Chimera page 1, section 3.3: Eq. 14 with page 2's parenthesisation,
//   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
// computed as S <- Diag(alpha_t) S; u = beta_t (v_t - S^T k_t); S <- S + k_t u^T;
// and the readout o_t = S_t^T q_t (inner term of Eq. 15). The state is fp32
// (page 1, section 5.6: FP32 KDA state).
//
// One block per (batch, head, 16-column slice of d_v); 256 threads = 16 columns
// x 16 row-threads. A row-thread holds rows RPT rt .. RPT rt + RPT - 1 of its
// column in registers; the 16 row-threads of a column are one DPP row, so the two
// reductions over d_k per token are four DPP adds each. Tokens are staged in LDS
// 16 at a time, double-buffered: the next batch's loads are in flight while the
// current batch runs.
#include <algorithm>

#include "dtypes.h"
#include "internal.h"
#include "lanes.h"

namespace chm {
namespace {

constexpr int kTokBatch = 16;

// A value as the conv call would store it: rounded to bf16 for bf16 storage.
__device__ __forceinline__ float stored(float v, const uint16_t*) { return bf2f(f2bf(v)); }
__device__ __forceinline__ float stored(float v, const float*) { return v; }

// OUT false: no readout (o is not written; the state passes of the backward).
// CONV: q, k, v computed in the load stage from the conv source cs (page 1, section 3.4:
// each segment convolved on its own, zero outside it; Eq. 13), not read from q, k, v.
template <typename T, int RPT, bool OUT, bool CONV>
__global__ __launch_bounds__(256) void kda_seq_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                      const T* __restrict__ v, int64_t stride,
                                                      const T* __restrict__ alpha, const T* __restrict__ beta,
                                                      const float* __restrict__ S0, T* __restrict__ o,
                                                      float* __restrict__ S_final, int64_t Tn, int64_t H, int dk,
                                                      int dv, int l2norm, float* __restrict__ ckpt, SeqSegs sg,
                                                      ConvSrc cs) {
  constexpr int DKP = 16 * RPT;   // staged rows; rows past dk hold k = q = 0, alpha = 1
  __shared__ float sk[2][kTokBatch][DKP];
  __shared__ float sq[2][OUT ? kTokBatch : 1][OUT ? DKP : 1];   // q only for the readout
  __shared__ float sa[2][kTokBatch][DKP];
  __shared__ float sv[2][kTokBatch][16];
  __shared__ float sb[2][kTokBatch];
  // CONV: the weights of this block's q and k rows and v columns, [tap][channel] with the 4
  // text taps first and the 27 visual taps after them, and the segment table
  constexpr int kTaps = kTextTaps + kVisTaps;
  __shared__ float wq[CONV ? kTaps : 1][CONV ? DKP : 1], wk[CONV ? kTaps : 1][CONV ? DKP : 1];
  __shared__ float wv[CONV ? kTaps : 1][16];
  __shared__ Seg sseg[CONV ? kMaxFusedSegs : 1];

  const int n_vs = (dv + 15) / 16;
  const int vs = blockIdx.x % n_vs;
  const int p = (int)((blockIdx.x / n_vs) % sg.nseg);          // segment of the sequence
  const int64_t bh = blockIdx.x / n_vs / sg.nseg;
  const int64_t b = bh / H, h = bh % H;
  const int64_t t_beg = sg.nseg > 1 ? p * sg.len : 0;
  const int64_t t_end = sg.nseg > 1 ? min<int64_t>(Tn, t_beg + sg.len) : Tn;
  const int64_t seg_ix = bh * sg.nseg + p;
  const int tid = threadIdx.x;
  const int colid = tid >> 4, rt = tid & 15;
  const int col = vs * 16 + colid;
  const bool col_ok = col < dv;

  const float* init = sg.zero_start || sg.identity ? nullptr
                      : p == 0                     ? (S0 != nullptr ? S0 + bh * dk * dv : nullptr)
                      : (sg.Sseg != nullptr ? sg.Sseg + seg_ix * dk * dv : nullptr);
  float s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = RPT * rt + i;
    s[i] = sg.identity ? (col_ok && row == col ? 1.f : 0.f)
                       : (init != nullptr && col_ok && row < dk) ? init[row * dv + col] : 0.f;
  }

  if constexpr (CONV) {
    const int64_t qc = h * dk, kc = H * dk + h * dk, vch = 2 * H * dk + h * dv;
    auto wgt = [&](int64_t c, int tap) {
      return tap < kTextTaps ? (cs.w_text != nullptr ? cs.w_text[c * kTextTaps + tap] : 0.f)
                             : (cs.w_vis != nullptr ? cs.w_vis[c * kVisTaps + tap - kTextTaps] : 0.f);
    };
    for (int e = tid; e < kTaps * DKP; e += 256) {
      const int tap = e / DKP, row = e % DKP;
      wq[tap][row] = row < dk ? wgt(qc + row, tap) : 0.f;
      wk[tap][row] = row < dk ? wgt(kc + row, tap) : 0.f;
    }
    for (int e = tid; e < kTaps * 16; e += 256) {
      const int tap = e / 16, c = vs * 16 + e % 16;
      wv[tap][e % 16] = c < dv ? wgt(vch + c, tap) : 0.f;
    }
    if (tid == 0)
      for (int i = 0; i < cs.nseg; ++i) sseg[i] = cs.seg[i];
    __syncthreads();
  }

  // one batch of tokens: thread (colid, rt) loads token colid, rows RPT rt .. RPT rt + RPT - 1
  float rk[RPT], rq[RPT], ra[RPT], rv, rb;
  // CONV: q (rows), k (rows) and v (column vs * 16 + rt) of token t by the segment's taps
  auto conv_token = [&](int64_t t) {
    const T* xs = static_cast<const T*>(cs.x) + b * Tn * cs.C;
    const int64_t qc = h * dk, kc = H * dk + h * dk, vc = 2 * H * dk + h * dv + vs * 16 + rt;
    const bool v_ok = vs * 16 + rt < dv;
    float aq[RPT], ak[RPT], av = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) aq[i] = ak[i] = 0.f;
    // N taps at once: all their loads are issued before the first multiply (src < 0: zero padding)
    auto add = [&](const int64_t (&src)[3], const int (&tap)[3], int N) {
      float xq[3][RPT], xk[3][RPT], xv[3];
#pragma unroll
      for (int n = 0; n < 3; ++n) {
        const bool in = n < N && src[n] >= 0;
        const T* xr = xs + (in ? src[n] : 0) * cs.C;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          const int row = RPT * rt + i;
          xq[n][i] = in && row < dk ? to_f32(xr[qc + row]) : 0.f;
          xk[n][i] = in && row < dk ? to_f32(xr[kc + row]) : 0.f;
        }
        xv[n] = in && v_ok ? to_f32(xr[vc]) : 0.f;
      }
#pragma unroll
      for (int n = 0; n < 3; ++n) {
        if (n >= N) break;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          const int row = RPT * rt + i;
          aq[i] = fmaf(wq[tap[n]][row], xq[n][i], aq[i]);
          ak[i] = fmaf(wk[tap[n]][row], xk[n][i], ak[i]);
        }
        av = fmaf(wv[tap[n]][rt], xv[n], av);
      }
    };
    int lo = 0, hi = cs.nseg - 1;   // the segment holding t: the last one starting at or before it
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sseg[mid].start <= t) lo = mid; else hi = mid - 1;
    }
    const Seg sgt = sseg[lo];
    if (sgt.kind == SEG_TEXT) {
      for (int j0 = 0; j0 < kTextTaps; j0 += 3) {
        int64_t src[3];
        int tap[3];
#pragma unroll
        for (int n = 0; n < 3; ++n) {
          tap[n] = min(j0 + n, kTextTaps - 1);
          src[n] = text_tap_source(sgt, t, tap[n]);
        }
        add(src, tap, min(3, kTextTaps - j0));
      }
    } else {
      const int64_t local = t - sgt.start, hw = (int64_t)sgt.height * sgt.width;
      const int64_t f = local / hw, hh = (local / sgt.width) % sgt.height, ww = local % sgt.width;
      for (int kt = 3 - min(sgt.frames, 3); kt < 3; ++kt)
        for (int kh = 0; kh < 3; ++kh) {
          int64_t src[3];
          int tap[3];
#pragma unroll
          for (int kw = 0; kw < 3; ++kw) {
            src[kw] = vis_tap_source(sgt, f, hh, ww, kt, kh, kw);
            tap[kw] = kTextTaps + kt * 9 + kh * 3 + kw;
          }
          add(src, tap, 3);
        }
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      rq[i] = stored(aq[i], xs);
      rk[i] = stored(ak[i], xs);
    }
    rv = stored(av, xs);
  };
  auto load = [&](int64_t t0) {
    const int nt = (int)min<int64_t>(kTokBatch, t_end - t0);
    const bool tok_ok = colid < nt;
    const int64_t tok = b * Tn + t0 + colid;
    if constexpr (CONV) {
      if (tok_ok) {
        conv_token(t0 + colid);
      } else {
#pragma unroll
        for (int i = 0; i < RPT; ++i) rq[i] = rk[i] = 0.f;
        rv = 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = RPT * rt + i;
      const bool ok = tok_ok && row < dk;
      if constexpr (!CONV) {
        rk[i] = ok ? to_f32(k[tok * stride + h * dk + row]) : 0.f;
        rq[i] = ok && q != nullptr ? to_f32(q[tok * stride + h * dk + row]) : 0.f;
      }
      ra[i] = ok ? to_f32(alpha[(tok * H + h) * dk + row]) : 1.f;
    }
    // v: token colid, column vs * 16 + rt; beta: token colid
    const int vc = vs * 16 + rt;
    if constexpr (!CONV) rv = (tok_ok && vc < dv && v != nullptr) ? to_f32(v[tok * stride + h * dv + vc]) : 0.f;
    rb = tok_ok ? to_f32(beta[tok * H + h]) : 0.f;
  };
  // store a loaded batch to buffer `buf` and normalise its q and k rows
  auto stage = [&](int buf) {
    if (l2norm) {
      float ssk = 0.f, ssq = 0.f;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        ssk = fmaf(rk[i], rk[i], ssk);
        ssq = fmaf(rq[i], rq[i], ssq);
      }
      const float nk = 1.f / sqrtf(sum16(ssk) + 1e-6f), nq = 1.f / sqrtf(sum16(ssq) + 1e-6f);
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        rk[i] *= nk;
        rq[i] *= nq;
      }
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      sk[buf][colid][RPT * rt + i] = rk[i];
      if (OUT) sq[buf][colid][RPT * rt + i] = rq[i];
      sa[buf][colid][RPT * rt + i] = ra[i];
    }
    sv[buf][colid][rt] = rv;
    if (rt == 0) sb[buf][colid] = rb;
  };

  if (t_beg < t_end) {
    load(t_beg);
    stage(0);
  }
  __syncthreads();
  int buf = 0;
  for (int64_t t0 = t_beg; t0 < t_end; t0 += kTokBatch) {
    const int nt = (int)min<int64_t>(kTokBatch, t_end - t0);
    const bool more = t0 + kTokBatch < t_end;
    if (more) load(t0 + kTokBatch);                  // in flight during this batch
    if (ckpt != nullptr && col_ok) {                 // the state before this batch (for the backward)
      float* dst = ckpt + ((bh * ((Tn + kTokBatch - 1) / kTokBatch) + t0 / kTokBatch) * dk) * dv + col;
#pragma unroll
      for (int i = 0; i < RPT; ++i)
        if (RPT * rt + i < dk) dst[(int64_t)(RPT * rt + i) * dv] = s[i];
    }
    for (int tt = 0; tt < nt; ++tt) {
      float pred = 0.f;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int row = RPT * rt + i;
        s[i] *= sa[buf][tt][row];
        pred = fmaf(s[i], sk[buf][tt][row], pred);
      }
      pred = sum16(pred);
      const float u = sb[buf][tt] * (sv[buf][tt][colid] - pred);
      float out = 0.f;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int row = RPT * rt + i;
        s[i] = fmaf(sk[buf][tt][row], u, s[i]);
        if (OUT) out = fmaf(s[i], sq[buf][tt][row], out);
      }
      if (OUT) {
        out = sum16(out);
        if (rt == 0 && col_ok) from_f32(o + ((b * Tn + t0 + tt) * H + h) * dv + col, out);
      }
    }
    if (more) stage(buf ^ 1);                        // the other buffer was last read a batch ago
    __syncthreads();
    buf ^= 1;
  }
  if (S_final != nullptr && col_ok && p == sg.nseg - 1) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = RPT * rt + i;
      if (row < dk) S_final[(bh * dk + row) * dv + col] = s[i];
    }
  }
  if (sg.Send != nullptr && col_ok) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = RPT * rt + i;
      if (row < dk) sg.Send[(seg_ix * dk + row) * dv + col] = s[i];
    }
  }
}

// Output gate and norm of Eq. 15 (page 1, section 3.3) short of W_o, in place on o:
//   o <- Sigmoid(gate) * o / sqrt(mean_c o_c^2 + eps) * w_c   over the dv channels of one head.
// One wave per (token, head) row; lane l holds channels l, l + 64, ... (dv <= 256).
template <typename T>
__global__ __launch_bounds__(256) void kda_gate_norm_kernel(T* __restrict__ o, const T* __restrict__ gate,
                                                            int64_t gate_stride, const float* __restrict__ w,
                                                            float eps, int64_t rows, int64_t H, int dv) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int64_t tok = row / H, h = row % H;
  T* orow = o + row * dv;
  const T* grow = gate + tok * gate_stride + h * dv;
  float x[4], ss = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = lane + 64 * i;
    x[i] = c < dv ? to_f32(orow[c]) : 0.f;
    ss = fmaf(x[i], x[i], ss);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
  const float r = 1.f / sqrtf(ss / (float)dv + eps);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = lane + 64 * i;
    if (c < dv) {
      const float sg = 1.f / (1.f + expf(-to_f32(grow[c])));
      from_f32(orow + c, x[i] * r * (w != nullptr ? w[c] : 1.f) * sg);
    }
  }
}

template <typename T, int R>
hipError_t launch_seq_r(const KdaArgs& a, int64_t blocks, hipStream_t stream, float* ckpt, const SeqSegs& sg) {
  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  const T* al = static_cast<const T*>(a.alpha);
  const T* be = static_cast<const T*>(a.beta);
  T* o = static_cast<T*>(a.o);
  const dim3 g((unsigned)blocks), t(256);
  const int dk = (int)a.dk, dv = (int)a.dv, nrm = (int)a.l2norm;
  const ConvSrc cs = a.conv != nullptr ? *a.conv : ConvSrc{};
  if (a.conv != nullptr) {
    if constexpr (R <= 8)   // the conv weights of wider heads do not fit the LDS
      hipLaunchKernelGGL((kda_seq_kernel<T, R, true, true>), g, t, 0, stream, q, k, v, a.qkv_stride, al, be, a.S0, o,
                         a.S_final, a.T, a.H, dk, dv, nrm, ckpt, sg, cs);
    else
      return hipErrorInvalidValue;
  } else if (o != nullptr) {
    hipLaunchKernelGGL((kda_seq_kernel<T, R, true, false>), g, t, 0, stream, q, k, v, a.qkv_stride, al, be, a.S0, o,
                       a.S_final, a.T, a.H, dk, dv, nrm, ckpt, sg, cs);
  } else {
    hipLaunchKernelGGL((kda_seq_kernel<T, R, false, false>), g, t, 0, stream, q, k, v, a.qkv_stride, al, be, a.S0, o,
                       a.S_final, a.T, a.H, dk, dv, nrm, ckpt, sg, cs);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_seq(const KdaArgs& a, int64_t blocks, hipStream_t stream, float* ckpt, const SeqSegs& sg) {
  if (a.dk <= 16) return launch_seq_r<T, 1>(a, blocks, stream, ckpt, sg);
  if (a.dk <= 32) return launch_seq_r<T, 2>(a, blocks, stream, ckpt, sg);
  if (a.dk <= 64) return launch_seq_r<T, 4>(a, blocks, stream, ckpt, sg);
  if (a.dk <= 128) return launch_seq_r<T, 8>(a, blocks, stream, ckpt, sg);
  return launch_seq_r<T, 16>(a, blocks, stream, ckpt, sg);
}

}  // namespace

hipError_t launch_kda_gate_norm(const KdaArgs& a, hipStream_t stream, Marks* marks) {
  const int64_t rows = a.B * a.T * a.H;
  if (rows == 0) return hipSuccess;
  const int64_t blocks = (rows + 3) / 4;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 g((unsigned)blocks), t(256);
  if (a.bf16)
    hipLaunchKernelGGL(kda_gate_norm_kernel<uint16_t>, g, t, 0, stream, static_cast<uint16_t*>(a.o),
                       static_cast<const uint16_t*>(a.gate), a.gate_stride, a.norm_w, a.norm_eps, rows, a.H, (int)a.dv);
  else
    hipLaunchKernelGGL(kda_gate_norm_kernel<float>, g, t, 0, stream, static_cast<float*>(a.o),
                       static_cast<const float*>(a.gate), a.gate_stride, a.norm_w, a.norm_eps, rows, a.H, (int)a.dv);
  const hipError_t e = hipGetLastError();
  return e != hipSuccess ? e : mark_after(marks, "kda_gate_norm_kernel", stream);
}

hipError_t launch_kda_sequential(const KdaArgs& a, hipStream_t stream, Marks* marks, float* ckpt,
                                 const SeqSegs* segs) {
  if (a.B * a.H == 0) return hipSuccess;
  const SeqSegs sg = segs != nullptr ? *segs : SeqSegs{};
  if (sg.nseg < 1 || (sg.nseg > 1 && (sg.len <= 0 || sg.len % kTokBatch != 0))) return hipErrorInvalidValue;
  const int n_vs = (int)((a.dv + 15) / 16);
  const int64_t blocks = a.B * a.H * n_vs * sg.nseg;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (a.T == 0 && a.S_final == nullptr && sg.Send == nullptr) return hipSuccess;
  hipError_t e = a.bf16 ? launch_seq<uint16_t>(a, blocks, stream, ckpt, sg)
                        : launch_seq<float>(a, blocks, stream, ckpt, sg);
  if (e == hipSuccess) e = mark_after(marks, "kda_seq_kernel", stream);
  if (e == hipSuccess && a.gate != nullptr) e = launch_kda_gate_norm(a, stream, marks);
  return e;
}

// Sequence cut of the token-by-token forward. One (batch, head) scans its tokens in order, so a
// batch of few heads leaves most of the chip idle; cut into P segments, every segment runs at
// once in three passes of the same kernel: its end state from a zero start (L_p), its transition
// product M_p (Eq. 14 with v = 0 from the identity: the state after the segment is M_p S + L_p
// for a start state S), and, after the chain S_start(p + 1) = M_p S_start(p) + L_p, its readout
// from the true start state. P targets about eight blocks per CU, segments of at least 256 tokens
// (below that the chain and the two extra launches cost more than the shorter scan saves)
// and a whole number of token batches; the chain takes d_k <= 128.
constexpr int64_t kSplitBlocks = 2048, kSplitMinSeg = 256;

SeqCut seq_fwd_cut(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv) {
  if (dk > 128 || B * H == 0) return {T, 1};
  const int64_t base = B * H * std::max((dv + 15) / 16, (dk + 15) / 16);
  int64_t P = (kSplitBlocks + base - 1) / base;
  P = std::min<int64_t>(P, std::max<int64_t>(1, T / kSplitMinSeg));
  if (P <= 1) return {T, 1};
  const int64_t len = ((T + P - 1) / P + kTokBatch - 1) / kTokBatch * kTokBatch;
  P = (T + len - 1) / len;
  return P <= 1 ? SeqCut{T, 1} : SeqCut{len, (int)P};
}

size_t kda_seq_split_workspace(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv) {
  const SeqCut c = seq_fwd_cut(B, T, H, dk, dv);
  if (c.nseg <= 1) return 0;
  return (size_t)(B * H * c.nseg * (2 * dk * dv + dk * dk)) * sizeof(float);   // L, start states, M
}

hipError_t launch_kda_sequential_split(const KdaArgs& a, void* workspace, hipStream_t stream, Marks* marks) {
  const SeqCut c = seq_fwd_cut(a.B, a.T, a.H, a.dk, a.dv);
  if (c.nseg <= 1) return launch_kda_sequential(a, stream, marks);
  if (workspace == nullptr) return hipErrorInvalidValue;
  const int64_t sz = a.B * a.H * c.nseg * a.dk * a.dv;
  float* L = static_cast<float*>(workspace);
  float* Sst = L + sz;
  float* M = Sst + sz;
  KdaArgs f = a;   // state passes: no readout, S_final or gate
  f.q = nullptr;
  f.o = nullptr;
  f.S_final = nullptr;
  f.gate = nullptr;
  SeqSegs sl;
  sl.len = c.len;
  sl.nseg = c.nseg;
  sl.Send = L;
  sl.zero_start = 1;
  hipError_t e = launch_kda_sequential(f, stream, marks, nullptr, &sl);
  if (e != hipSuccess) return e;
  KdaArgs fm = f;
  fm.v = nullptr;
  fm.dv = a.dk;
  SeqSegs sm = sl;
  sm.Send = M;
  sm.zero_start = 0;
  sm.identity = 1;
  e = launch_kda_sequential(fm, stream, marks, nullptr, &sm);
  if (e != hipSuccess) return e;
  e = launch_kda_chain(false, M, L, a.S0, Sst, a.B * a.H, c.nseg, (int)a.dk, (int)a.dv, stream);
  if (e == hipSuccess) e = mark_after(marks, "kda_chain_kernel", stream);
  if (e != hipSuccess) return e;
  SeqSegs so;
  so.len = c.len;
  so.nseg = c.nseg;
  so.Sseg = Sst;
  return launch_kda_sequential(a, stream, marks, nullptr, &so);
}

}  // namespace chm
