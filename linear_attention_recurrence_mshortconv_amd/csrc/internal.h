// Internal declarations shared by the C ABI layer and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "grid.h"

namespace chm {

// ---- Per-kernel timing marks ----------------------------------------------------
// Optional. When a launcher gets a non-null Marks, it records ev[n] on the launch
// stream after each kernel it launches and names that kernel in names[n - 1]; the
// entry point records ev[0] before the first launch. The caller checks `cap`
// against the launch count before any launch, so these never run out.
struct Marks {
  hipEvent_t* ev;
  const char** names;
  int32_t cap;
  int32_t n;
};
inline hipError_t mark_begin(Marks* m, hipStream_t s) {
  if (m == nullptr) return hipSuccess;
  m->n = 1;
  return hipEventRecord(m->ev[0], s);
}
inline hipError_t mark_after(Marks* m, const char* kernel, hipStream_t s) {
  if (m == nullptr || m->n >= m->cap) return hipSuccess;
  m->names[m->n - 1] = kernel;
  return hipEventRecord(m->ev[m->n++], s);
}

// ---- mShortConv -------------------------------------------------------------
// y = mShortConv(x) for one segment, x/y [B][T][C] with C % 8 == 0.
hipError_t launch_conv_segment(const void* x, void* y, int64_t B, int64_t T, int64_t C, bool bf16,
                               const float* w_text, const float* w_vis, const Seg& seg,
                               bool force_gather, hipStream_t stream, Marks* marks = nullptr);

// y = mShortConv(x) for all segments of a layout: the text segments in one batched launch,
// the image grids of the rows kernel in another, every other segment on its own.
hipError_t launch_conv(const void* x, void* y, int64_t B, int64_t T, int64_t C, bool bf16, const float* w_text,
                       const float* w_vis, const Seg* segs, int nseg, hipStream_t stream, Marks* marks = nullptr);

// The image conv's adjoint (dx from dy) on the rows kernel with mirrored taps, for the image
// segments that conv_rows_adjoint_ok accepts (bf16, one frame, C a multiple of 64).
bool conv_rows_adjoint_ok(const Seg& seg, int64_t C, bool bf16);
hipError_t launch_conv_rows_adjoint(const void* dy, void* dx, const float* w_vis, int64_t B, int64_t Ttot, int64_t C,
                                    const Seg* segs, int n, hipStream_t stream, Marks* marks = nullptr);

// The conv's adjoint on the tile kernel (mirrored spatial taps, frames walked from the last one back),
// for the grid segments that conv_tile_adjoint_ok accepts (bf16, C a multiple of 64, a frame within
// 32-bit buffer offsets).
bool conv_tile_adjoint_ok(const Seg& seg, int64_t C, bool bf16);
hipError_t launch_conv_tile_adjoint(const void* dy, void* dx, const float* w_vis, int64_t B, int64_t Ttot, int64_t C,
                                    const Seg& seg, hipStream_t stream, Marks* marks = nullptr);

// Device-side neighbour table [T][27] for one segment (the conv kernels' arithmetic).
hipError_t launch_index_device(const Seg& seg, int64_t T, int32_t* idx, hipStream_t stream);

// ---- KDA ----------------------------------------------------------------------
// Conv source of the fused conv + recurrence: q|k|v of every token
// are computed from x [B][T][C] (C = H (2 dk + dv); the q, k and v channels in that order)
// by the mShortConv of the segment layout, rounded to the storage type as the conv call
// would store them, and never written out.
constexpr int kMaxFusedSegs = 32;
struct ConvSrc {
  const void* x = nullptr;
  int64_t C = 0;
  const float* w_text = nullptr;   // [C][4], or null when no segment is text
  const float* w_vis = nullptr;    // [C][27], or null when no segment is visual
  int nseg = 0;
  Seg seg[kMaxFusedSegs];
};

struct KdaArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t qkv_stride;   // elements between consecutive tokens of q, k, v
  const void* alpha;    // [B][T][H][dk]
  const void* beta;     // [B][T][H]
  const float* S0;      // [B][H][dk][dv] or null
  void* o;              // [B][T][H][dv]
  float* S_final;       // [B][H][dk][dv] or null
  int64_t B, T, H, dk, dv;
  bool bf16;
  bool l2norm;
  // Output gate and norm (Eq. 15 short of W_o), applied to o when gate != null:
  // o <- Sigmoid(gate) * o / sqrt(mean over the head's dv channels of o^2 + norm_eps) * norm_w
  const void* gate = nullptr;   // [B][T][H][dv], consecutive tokens gate_stride elements apart
  int64_t gate_stride = 0;
  const float* norm_w = nullptr;  // [dv] or null (ones)
  float norm_eps = 0.f;
  // Fused conv: q, k, v are ignored and computed from conv->x (the token-by-token kernel, or
  // the chunked kernels when kda_chunked_conv_supported).
  const ConvSrc* conv = nullptr;
};

// Optional cut of every sequence into nseg segments of len tokens (a multiple of 16; the last
// one shorter), run by separate blocks, for the backward's passes. Segment p starts from S0
// (p = 0) or from Sseg[b][h][p] (p > 0; null = zero), or from zero (zero_start), or from the
// identity (identity: dv == dk, v taken as zero, so the end state is the segment's transition
// product); Send[b][h][p] receives each segment's end state when not null.
struct SeqSegs {
  int64_t len = 0;
  int nseg = 1;
  const float* Sseg = nullptr;
  float* Send = nullptr;
  int zero_start = 0;
  int identity = 0;
};
// Token-by-token fp32 kernel: any dk, dv in 1..256 (with a gate: then the gate/norm kernel on o).
// With ckpt: also the state before every 16th token, [B][H][ceil(T/16)][dk][dv] fp32 (o may be null).
// q, v and o may be null when no output is wanted (v null = zero values).
hipError_t launch_kda_sequential(const KdaArgs& a, hipStream_t stream, Marks* marks = nullptr, float* ckpt = nullptr,
                                 const SeqSegs* segs = nullptr);
// o <- Sigmoid(gate) * RMSNorm(o) in place, one wave per (token, head): a.o, a.gate, a.norm_w.
hipError_t launch_kda_gate_norm(const KdaArgs& a, hipStream_t stream, Marks* marks = nullptr);

// ---- Backward ---------------------------------------------------------------------
// Gradients of one KDA call (the inputs in KdaArgs): dout [B][T][H][dv] in; dq, dk, dv out
// at the inputs' token stride, dalpha [B][T][H][dk], dbeta [B][T][H] (dtype), dS0 fp32.
struct KdaGrads {
  const void* dout;
  const float* dS_final;   // or null (zero)
  void* dq;
  void* dk;
  void* dv;
  void* dalpha;
  void* dbeta;
  float* dS0;              // or null
};
// The token-by-token forward over a sequence cut into segments (end states, transition products,
// the chain of start states, then the readout per segment); one unsplit launch when the cut has
// one segment (d_k > 128, short sequences, enough heads). Workspace: kda_seq_split_workspace bytes.
struct SeqCut {
  int64_t len;
  int nseg;
};
SeqCut seq_fwd_cut(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv);
size_t kda_seq_split_workspace(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv);
hipError_t launch_kda_sequential_split(const KdaArgs& a, void* workspace, hipStream_t stream, Marks* marks = nullptr);
size_t kda_bwd_workspace(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv);
hipError_t launch_kda_backward(const KdaArgs& a, const KdaGrads& g, void* workspace, hipStream_t stream,
                               Marks* marks = nullptr);
// The same gradients on MFMA (bf16, dk = dv = 128; the inputs and dout 8-byte aligned with a
// token stride that is a multiple of 4): 16-token chunks, each sequence cut into segments
// joined by fp32 chains; the workspace holds the bf16 state before every chunk.
bool kda_bwd_chunked_shape(int64_t dk, int64_t dv, bool bf16);
bool kda_bwd_chunked_layout_ok(const KdaArgs& a, const KdaGrads& g);
size_t kda_bwd_chunked_workspace(int64_t B, int64_t T, int64_t H);
hipError_t launch_kda_backward_chunked(const KdaArgs& a, const KdaGrads& g, void* workspace, hipStream_t stream,
                                       Marks* marks = nullptr);
// The segment chains of the backward passes for BH (sequence, head) pairs of nseg segments each,
// M [BH][nseg][dk][dk], X, Y [BH][nseg][dk][dv], init [BH][dk][dv] or null (fp32, row-major):
// forward (back false) Y_0 = init, Y_p = M_{p-1} Y_{p-1} + X_{p-1}; backward (back true)
// Y_{nseg-1} = init, Y_p = M_{p+1}^T Y_{p+1} + X_{p+1}.
hipError_t launch_kda_chain(bool back, const float* M, const float* X, const float* init, float* Y, int64_t BH,
                            int nseg, int dk, int dv, hipStream_t stream);
// Backward of the gate and norm: do [rows][dv] and dgate (gate layout) in the dtype, dnorm_w [dv]
// fp32 written (summed over rows) when not null; rows = B * T * H.
hipError_t launch_gate_norm_backward(const void* o, const void* gate, int64_t gate_stride, const float* norm_w,
                                     float eps, const void* dy, void* dout, void* dgate, float* dnorm_w, int64_t rows,
                                     int64_t H, int64_t dv, bool bf16, hipStream_t stream);
// dx (dtype, [B][T][C]) and dw_text [C][4], dw_vis [C][27] (fp32, written) of y = mShortConv(x) against dy.
hipError_t launch_conv_backward(const void* x, const void* dy, void* dx, float* dw_text, float* dw_vis, int64_t B,
                                int64_t T, int64_t C, bool bf16, const float* w_text, const float* w_vis,
                                const Seg* segs, int nseg, hipStream_t stream, Marks* marks = nullptr);

// Chunked MFMA path (bf16, dk = dv = 128). The sequences come as runs: `count` consecutive
// sequences of `len` tokens from row `start` on, whose S0 / S_final entries start at `sidx0`.
// A batch of B sequences of T tokens is the single run {0, T, B, 0}; samples packed in one
// row are one run per stretch of equal lengths.
struct KdaRun {
  int64_t start, len, count, sidx0;
};
bool kda_chunked_supported(const KdaArgs& a);
// With a.conv: the fused conv in the chunked kernels' load stage (bf16 x, one run, the window
// of x that a chunk's taps reach addressable with 32-bit offsets).
bool kda_chunked_conv_supported(const KdaArgs& a);
bool kda_chunked_plan_ok(const KdaRun* runs, int64_t nruns, int64_t H, bool no_split);   // grid sizes fit
// bytes; with conv, the transposed weights and the segment table after the states
size_t kda_chunked_workspace(const KdaRun* runs, int64_t nruns, int64_t H, bool no_split,
                             const ConvSrc* conv = nullptr);
hipError_t launch_kda_chunked(const KdaArgs& a, const KdaRun* runs, int64_t nruns, bool no_split, void* workspace,
                              hipStream_t stream, Marks* marks = nullptr);

}  // namespace chm
