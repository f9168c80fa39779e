/*
 * chimera_mshortconv.h -- C ABI of the KDA + mShortConv forward for AMD MI355X (gfx950).
 *
 * The method is the sequence mixer of the Chimera visual diffusion backbone
 * ("Chimera: Designing and Chinchilla-Scaling Hybrid Visual Diffusion
 * Transformers", arXiv 2607.28611; page 1, section 3.3, Eq. 12-15, and
 * section 3.4):
 *
 *   (Q, K, V) = mShortConv(W_qkv x)                                   Eq. 13
 *   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T   Eq. 14
 *   o_t = S_t^T q_t                       (inner term of Eq. 15)
 *   y_t = Sigmoid(g_t) * RMSNorm(o_t)     (Eq. 15 short of the output projection)
 *
 * over one packed token stream: text tokens first, then visual tokens in
 * time-first raster order (Eq. 12). This library computes the mShortConv and
 * the recurrence with its readout; the projections around them are not part
 * of it.
 *
 * Conventions for every entry point:
 *  - Pointers marked "device" are HIP device memory; "host" is ordinary host
 *    memory. The caller allocates and frees every buffer and owns the stream.
 *    No *_fwd call allocates memory or synchronises the device. The library
 *    keeps no state between calls beyond per-device facts it looks up once
 *    (the compute-unit count, a kernel's LDS attribute), kept in atomics, so
 *    calls from several host threads are safe; calls that share a workspace
 *    or outputs on one device must not overlap.
 *  - Errors are returned as status codes; nothing aborts or throws across the
 *    ABI. All arguments are checked before any launch; on an error nothing is
 *    written. A failed kernel launch returns CHIMERA_ERR_HIP. A fault inside a
 *    kernel surfaces at the caller's next synchronisation.
 *  - Values are not checked on the device: NaN and Inf propagate.
 *  - All tensors are dense, row-major, with the innermost index last.
 */
#ifndef CHIMERA_MSHORTCONV_H
#define CHIMERA_MSHORTCONV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum chimera_status {
  CHIMERA_OK = 0,
  CHIMERA_ERR_NULL = 1,         /* a required pointer is NULL */
  CHIMERA_ERR_SHAPE = 2,        /* a size is negative, zero where it may not be, or too large */
  CHIMERA_ERR_DTYPE = 3,        /* unknown dtype */
  CHIMERA_ERR_SEGMENTS = 4,     /* the segment table does not tile [0, T) or a grid is malformed */
  CHIMERA_ERR_UNSUPPORTED = 5,  /* a valid request this library does not implement */
  CHIMERA_ERR_WORKSPACE = 6,    /* workspace missing or smaller than chimera_kda_workspace_size() */
  CHIMERA_ERR_HIP = 7           /* a HIP runtime call or kernel launch failed */
} chimera_status;

typedef enum chimera_dtype {
  CHIMERA_F32 = 0,              /* IEEE binary32 */
  CHIMERA_BF16 = 1              /* bfloat16: the upper half of binary32 */
} chimera_dtype;

typedef enum chimera_seg_kind {
  CHIMERA_SEG_TEXT = 0,         /* causal 1D segment */
  CHIMERA_SEG_IMAGE = 1,        /* one-frame grid: frames == 1 */
  CHIMERA_SEG_VIDEO = 2         /* frames x height x width grid, time-first raster order */
} chimera_seg_kind;

/*
 * One modality segment of the packed stream, covering tokens
 * [start, start + length). Text: frames = height = width = 0. Image and video:
 * length == frames * height * width, and grid point (i, j, k) (time, height,
 * width) is token start + i*height*width + j*width + k (Eq. 12). Segments
 * must be listed in increasing start order and tile [0, T) with no gap or
 * overlap (Chimera page 1, section 3.2: text first, then the visual tokens).
 */
typedef struct chimera_segment {
  int32_t kind;                 /* chimera_seg_kind */
  int32_t frames;
  int32_t height;
  int32_t width;
  int64_t start;
  int64_t length;
} chimera_segment;

/* Taps of the short convolution (Chimera page 1, section 3.4; sizes are this
 * library's reading of "short"): text uses CHIMERA_TEXT_TAPS taps, tap j
 * reading the token j - 3 places earlier in the text segment; visual grids use
 * a 3x3x3 kernel, tap kt*9 + kh*3 + kw reading grid offset (kt-2, kh-1, kw-1):
 * causal in time (current and two earlier frames), symmetric in space. Taps
 * outside the segment read zero. An image uses only the kt = 2 slice. */
#define CHIMERA_TEXT_TAPS 4
#define CHIMERA_VIS_TAPS 27

/*
 * chimera_mshortconv_index -- the neighbour table of a segment layout.
 * Chimera page 1, section 3.3 Eq. 12 (raster order) and section 3.4
 * (per-segment views, causal in time, zero padding at segment edges).
 *
 *   segs  host, nseg entries (see chimera_segment)
 *   T     total tokens; the segments must tile [0, T)
 *   idx   host int32 [T][27], written: source token of tap j for token p, or
 *         -1 where the tap reads zero padding. Text rows fill taps 0..3 and
 *         hold -1 in taps 4..26.
 *
 * Host only and synchronous. Returns CHIMERA_ERR_NULL, CHIMERA_ERR_SHAPE or
 * CHIMERA_ERR_SEGMENTS on bad input (idx untouched).
 */
chimera_status chimera_mshortconv_index(const chimera_segment* segs, int32_t nseg, int64_t T,
                                        int32_t* idx);

/*
 * chimera_mshortconv_index_device -- the same table, computed on the device
 * from the segment descriptors with the device-side grid helpers (raster index
 * and bounds of Eq. 12) that the convolution kernels are written with. The
 * kernels' own gathers (staged tiles, buffer offsets, text windows) do not run
 * here; their taps are checked through chimera_mshortconv_fwd itself, with
 * one-hot weights and inputs that encode each token's position.
 *
 *   idx_dev  device int32 [T][27], written asynchronously on `stream`.
 */
chimera_status chimera_mshortconv_index_device(const chimera_segment* segs, int32_t nseg, int64_t T,
                                               int32_t* idx_dev, hipStream_t stream);

/*
 * chimera_mshortconv_fwd -- modality-aware short convolution (Eq. 13;
 * Chimera page 1, section 3.4; page 2, mShortConv paragraph).
 *
 *   x       device [B][T][C], dtype dt: the projected q|k|v of every token
 *           (any channel count; the conv is depthwise)
 *   y       device [B][T][C], dtype dt, written: y[b,p,c] = sum over taps of
 *           w[c,tap] * x[b, neighbour(p,tap), c], accumulated in fp32 and
 *           rounded once to dt. Must not alias x.
 *   w_text  device fp32 [C][4]
 *   w_vis   device fp32 [C][27], (kt, kh, kw) row-major
 *   segs    host, nseg entries; the same layout for every batch item
 *
 * No bias, no activation. Asynchronous on `stream`. Requires C % 8 == 0.
 */
chimera_status chimera_mshortconv_fwd(const void* x, void* y, int64_t B, int64_t T, int64_t C,
                                      chimera_dtype dt, const float* w_text, const float* w_vis,
                                      const chimera_segment* segs, int32_t nseg, hipStream_t stream);

/* Flags of chimera_kda_fwd. */
#define CHIMERA_KDA_L2NORM_QK 1u   /* divide q and k by sqrt(sum of squares over d_k + 1e-6) per
                                      (token, head) before the recurrence (Chimera page 1, Fig. 2:
                                      the "L2" boxes between mShortConv and the recurrence) */
#define CHIMERA_KDA_SEQUENTIAL 2u  /* use the token-by-token fp32 kernel for every shape */
#define CHIMERA_KDA_NO_SPLIT 4u    /* either kernel without splitting the sequence into segments */

/*
 * chimera_kda_workspace_size -- bytes of device workspace chimera_kda_fwd
 * needs for these sizes and flags (0 when it needs none). Returns 0 for
 * invalid sizes as well; chimera_kda_fwd reports those.
 */
size_t chimera_kda_workspace_size(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                  chimera_dtype dt, uint32_t flags);

/*
 * chimera_kda_fwd -- KDA forward: Eq. 14 and the readout o_t = S_t^T q_t
 * (Chimera page 1, section 3.3; Eq. 14's parentheses as printed on page 2).
 * The decay Diag(alpha_t) acts first; the erase and the write then use the
 * decayed state; the readout uses the state after token t.
 *
 *   q, k    device [B][T][H][dk], dtype dt, consecutive tokens qkv_stride
 *           elements apart (the [H][dk] block of one token is contiguous);
 *           element (b, t, h, i) at base + (b*T + t)*qkv_stride + h*dk + i
 *   v       device [B][T][H][dv], same token stride
 *   qkv_stride  elements between tokens: H*dk for separate tensors, or the
 *           channel count of a fused q|k|v tensor such as mshortconv's output
 *   alpha   device [B][T][H][dk], dtype dt, values in (0, 1]: per-channel decay
 *   beta    device [B][T][H], dtype dt, values in (0, 1): erase/write strength
 *   S0      device fp32 [B][H][dk][dv], or NULL for a zero initial state
 *   o       device [B][T][H][dv], dtype dt, written (fp32 accumulation, one rounding)
 *   S_final device fp32 [B][H][dk][dv], written, or NULL
 *   flags   CHIMERA_KDA_* bits
 *   workspace  device, at least chimera_kda_workspace_size(...) bytes, or
 *           NULL when that size is 0; contents on entry do not matter
 *
 * Supported: dk, dv in 1..256 for the token-by-token kernel (fp32 and bf16).
 * Unless CHIMERA_KDA_NO_SPLIT, that kernel cuts each sequence into segments
 * (dk <= 128, when the batch's heads leave the chip idle) and runs them at
 * once: each segment's end state from zero and its transition product (Eq. 14
 * with v = 0 from the identity), a chain for the start states, then the
 * readout from them; the result equals the unsplit scan up to fp32 rounding,
 * and chimera_kda_workspace_size then counts 4 (2 dk dv + dk dk) bytes per
 * (batch item, head, segment). The rest of this paragraph is the chunked path:
 * the chunked MFMA kernel runs for bf16 with dk and dv multiples of 8 up to 128
 * (qkv_stride a multiple of 4, q, k and alpha 8-byte aligned). It works at 128
 * channels: smaller heads are zero-padded inside the kernels (their extra k, q,
 * v channels read as 0 and alpha as 1, and only the real channels of o and
 * S_final are written), so a head costs the same at any size up to 128. alpha < 0
 * is undefined.
 *
 * Small alpha on the chunked kernel: it factors the decay inside 16-token
 * blocks and raises every alpha below e^-7.5 (about 5.5e-4) to e^-7.5 as it
 * loads it, which keeps every factor within bf16 range and precision. The result
 * then departs from Eq. 14 only where an alpha is below that value: such a token
 * keeps e^-7.5 of each decayed state channel instead of alpha of it, an absolute
 * error of at most 5.5e-4 times that channel's magnitude (alpha = 0, complete
 * forgetting, leaves 5.5e-4 of the old channel), under one bf16 rounding step of
 * the channel (2^-8 relative). CHIMERA_KDA_SEQUENTIAL (the token-by-token
 * kernel) uses alpha exactly as given, for callers that need hard resets to be
 * exact.
 * Asynchronous on `stream`; o and S_final must not alias any input.
 */
chimera_status chimera_kda_fwd(const void* q, const void* k, const void* v, int64_t qkv_stride,
                               const void* alpha, const void* beta, const float* S0,
                               void* o, float* S_final,
                               int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                               chimera_dtype dt, uint32_t flags,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * chimera_kda_fwd_noalloc -- chimera_kda_fwd for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. The same
 * computation, kernels, results and errors as chimera_kda_fwd with the same arguments, except
 * that the workspace is not an argument: it is a device array of
 * CHIMERA_KDA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on (from the
 * first use there until the process ends).
 *
 *   q .. flags, stream   as for chimera_kda_fwd
 *
 * Returns CHIMERA_ERR_WORKSPACE, before any launch and any HIP call, when
 * chimera_kda_workspace_size() for these sizes and flags exceeds
 * CHIMERA_KDA_NOALLOC_SCRATCH_BYTES (the batched workloads of this library need at most 96 MiB).
 * Calls no hipMalloc or hipFree. Every call on one GPU uses that GPU's one array: calls that
 * overlap on one device (on two streams, or from two host threads) race and must not be issued.
 */
#define CHIMERA_KDA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
chimera_status chimera_kda_fwd_noalloc(const void* q, const void* k, const void* v, int64_t qkv_stride,
                                       const void* alpha, const void* beta, const float* S0, void* o,
                                       float* S_final, int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                       chimera_dtype dt, uint32_t flags, hipStream_t stream);

/*
 * chimera_kda_fwd_conv -- mShortConv and KDA in one pass (Chimera page 1, section 3.4:
 * the conv on packed storage fused with the recurrence; Eq. 13 then Eq. 14): q, k and v of
 * every token are computed from x in the recurrence's load stage, rounded to dt as
 * chimera_mshortconv_fwd would store them, and never written to memory.
 *
 *   x         device [B][T][C], dt, C = H * (2 * dk + dv): the q, k, v channels in that
 *             order, head-major inside each
 *   w_text, w_vis, segs, nseg   as for chimera_mshortconv_fwd (nseg <= 32 here); every
 *             sequence of the batch has the layout segs
 *   alpha, beta, S0, o, S_final, B, T, H, dk, dv, dt   as for chimera_kda_fwd
 *   flags     CHIMERA_KDA_L2NORM_QK, CHIMERA_KDA_SEQUENTIAL, CHIMERA_KDA_NO_SPLIT
 *   workspace device, at least chimera_kda_conv_workspace_size(...) bytes, owned by the
 *             caller (may be NULL when that size is 0)
 *
 * Two paths, chosen as for chimera_kda_fwd:
 *   - bf16 with dk = dv = 128 (and a layout whose farthest tap, 2 frames + 1 row + 1 token
 *     back for video, keeps a chunk's window of x below 2 GiB): the chunked MFMA kernels with
 *     the conv in their load stage. The conv sums its taps in the order of the conv kernels
 *     and rounds once, so q, k and v equal chimera_mshortconv_fwd's output bit for bit and
 *     the result equals chimera_mshortconv_fwd followed by chimera_kda_fwd (same flags) on
 *     the views q, k, v = y[..., 0:H*dk], y[..., H*dk:2*H*dk], y[..., 2*H*dk:] (alpha clamped
 *     as there).
 *   - otherwise, and with CHIMERA_KDA_SEQUENTIAL: the token-by-token fp32 kernel (dk <= 128,
 *     else CHIMERA_ERR_UNSUPPORTED), equal to the two calls with CHIMERA_KDA_SEQUENTIAL up to
 *     the order of the conv's fp32 sums; no workspace.
 * More than 32 segments: CHIMERA_ERR_UNSUPPORTED. A workspace below the size:
 * CHIMERA_ERR_WORKSPACE before any launch. o must not alias x. Asynchronous on `stream`.
 */
size_t chimera_kda_conv_workspace_size(const chimera_segment* segs, int32_t nseg, int64_t B, int64_t T,
                                       int64_t H, int64_t dk, int64_t dv, chimera_dtype dt, uint32_t flags);
chimera_status chimera_kda_fwd_conv(const void* x, const float* w_text, const float* w_vis,
                                    const chimera_segment* segs, int32_t nseg, const void* alpha,
                                    const void* beta, const float* S0, void* o, float* S_final,
                                    int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                    chimera_dtype dt, uint32_t flags, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/*
 * Per-kernel timing variants. Each runs exactly the launches of the call it is
 * named after, with the same arguments and results, and additionally records
 * HIP events on `stream`: marks[0] before the first kernel, then marks[i] right
 * after the i-th kernel is enqueued, with names[i-1] set to a static,
 * NUL-terminated name of that kernel. The elapsed time between marks[i-1] and
 * marks[i] is then the device time of kernel i (plus the gap between
 * launches). *used receives the number of marks recorded (0 when nothing was
 * launched).
 *
 *   marks     host array of `capacity` events, created by the caller with
 *             timing enabled (hipEventCreate), owned by the caller
 *   names     host array of `capacity` pointers, written
 *   capacity  at least nseg + 1 for the conv, CHIMERA_KDA_MAX_KERNELS + 1 for
 *             KDA, CHIMERA_KDA_CONV_MAX_KERNELS + 1 for the fused conv + KDA;
 *             otherwise CHIMERA_ERR_SHAPE before any launch
 *
 * Errors as for the untimed call; a failed event record is CHIMERA_ERR_HIP.
 * The marks serve measurement: they add a few microseconds of event overhead
 * per kernel.
 */
#define CHIMERA_KDA_MAX_KERNELS 4
#define CHIMERA_KDA_CONV_MAX_KERNELS 4   /* chimera_kda_fwd_conv_timed: capacity at least this + 1 */
chimera_status chimera_mshortconv_fwd_timed(const void* x, void* y, int64_t B, int64_t T, int64_t C,
                                            chimera_dtype dt, const float* w_text, const float* w_vis,
                                            const chimera_segment* segs, int32_t nseg, hipStream_t stream,
                                            hipEvent_t* marks, const char** names, int32_t capacity,
                                            int32_t* used);
chimera_status chimera_kda_fwd_timed(const void* q, const void* k, const void* v, int64_t qkv_stride,
                                     const void* alpha, const void* beta, const float* S0, void* o, float* S_final,
                                     int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, chimera_dtype dt,
                                     uint32_t flags, void* workspace, size_t workspace_bytes, hipStream_t stream,
                                     hipEvent_t* marks, const char** names, int32_t capacity, int32_t* used);
chimera_status chimera_kda_fwd_conv_timed(const void* x, const float* w_text, const float* w_vis,
                                          const chimera_segment* segs, int32_t nseg, const void* alpha,
                                          const void* beta, const float* S0, void* o, float* S_final, int64_t B,
                                          int64_t T, int64_t H, int64_t dk, int64_t dv, chimera_dtype dt,
                                          uint32_t flags, void* workspace, size_t workspace_bytes,
                                          hipStream_t stream, hipEvent_t* marks, const char** names,
                                          int32_t capacity, int32_t* used);

/*
 * chimera_kda_fwd_gated -- chimera_kda_fwd followed by the output gate and norm of
 * Eq. 15 (Chimera page 1, section 3.3) short of the output projection W_o:
 *
 *   y_t = Sigmoid(gate_t) * RMSNorm(S_t^T q_t),
 *   RMSNorm(x)_c = x_c / sqrt(mean over the head's dv channels of x^2 + norm_eps) * w_c
 *
 * per (token, head). gate_t is the layer's W_gate projection, given as an input
 * (the projection itself is not part of this library). Eq. 15 does not fix the norm's
 * extent, gain or epsilon: here it runs over each head's dv channels on their own,
 * with one gain vector shared by the heads and epsilon inside the square root.
 *
 *   gate         device [B][T][H][dv], dtype dt, consecutive tokens gate_stride
 *                elements apart (gate_stride >= H*dv; a view into a wider
 *                projection output is accepted)
 *   norm_weight  device fp32 [dv], or NULL for a gain of 1
 *   norm_eps     >= 0 and finite, else CHIMERA_ERR_SHAPE
 *   o            receives y, dtype dt
 *
 * All other arguments, the workspace (chimera_kda_workspace_size with the same
 * flags), S_final and the errors are those of chimera_kda_fwd; a NULL gate with
 * T > 0 is CHIMERA_ERR_NULL. The chunked kernel applies the gate and norm to its fp32
 * output before the one rounding to dt when gate is 16-byte aligned and gate_stride
 * is a multiple of 8; otherwise, and on the token-by-token kernel, a separate pass
 * applies them to o in place after the recurrence (o is then rounded to dt twice).
 */
chimera_status chimera_kda_fwd_gated(const void* q, const void* k, const void* v, int64_t qkv_stride,
                                     const void* alpha, const void* beta, const float* S0, const void* gate,
                                     int64_t gate_stride, const float* norm_weight, float norm_eps, void* o,
                                     float* S_final, int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                     chimera_dtype dt, uint32_t flags, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* Timing variant of chimera_kda_fwd_gated, as the ones above; capacity at least
 * CHIMERA_KDA_GATED_MAX_KERNELS + 1. */
#define CHIMERA_KDA_GATED_MAX_KERNELS 5
chimera_status chimera_kda_fwd_gated_timed(const void* q, const void* k, const void* v, int64_t qkv_stride,
                                           const void* alpha, const void* beta, const float* S0, const void* gate,
                                           int64_t gate_stride, const float* norm_weight, float norm_eps, void* o,
                                           float* S_final, int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                           chimera_dtype dt, uint32_t flags, void* workspace, size_t workspace_bytes,
                                           hipStream_t stream, hipEvent_t* marks, const char** names,
                                           int32_t capacity, int32_t* used);

/*
 * chimera_kda_fwd_varlen -- KDA forward over samples packed in one token row, with the
 * state restarting at every packed sample boundary (Chimera page 1, section 3.3: S0 = 0
 * at each sample boundary; section 5.1: mixed-resolution samples of different lengths
 * packed together), and optionally the output gate and norm of chimera_kda_fwd_gated.
 *
 *   q, k, v, alpha, beta, o, gate
 *               as for chimera_kda_fwd(_gated) with B = 1 and T = cu_seqlens[nseq]
 *               (row-major [T][H][d], [T][H] for beta; token strides qkv_stride and
 *               gate_stride)
 *   cu_seqlens  host int64 [nseq + 1]: sample n is rows cu_seqlens[n] .. cu_seqlens[n+1]-1;
 *               cu_seqlens[0] = 0 and the offsets never decrease (empty samples are
 *               allowed: their S_final is their S0), else CHIMERA_ERR_SHAPE
 *   S0          device fp32 [nseq][H][dk][dv], or NULL for zero initial states
 *   S_final     device fp32 [nseq][H][dk][dv], written, or NULL
 *   gate        NULL for the plain readout; otherwise as in chimera_kda_fwd_gated (then
 *               norm_weight and norm_eps are used, and checked likewise)
 *   workspace   at least chimera_kda_varlen_workspace_size(...) bytes with the same
 *               cu_seqlens, sizes, dtype and flags
 *
 * A packed row of equal-length samples gives the same result as chimera_kda_fwd with
 * B = nseq. The chunked kernel launches once for up to 48 stretches of equal-length
 * consecutive samples; the token-by-token kernel once per such stretch. The chunked
 * kernel raises alpha below e^-7.5 to that value, with the bound stated at
 * chimera_kda_fwd (CHIMERA_KDA_SEQUENTIAL is exact). Errors as for chimera_kda_fwd;
 * host only until the launches, asynchronous on `stream`.
 */
size_t chimera_kda_varlen_workspace_size(const int64_t* cu_seqlens, int32_t nseq, int64_t H, int64_t dk,
                                         int64_t dv, chimera_dtype dt, uint32_t flags);
chimera_status chimera_kda_fwd_varlen(const void* q, const void* k, const void* v, int64_t qkv_stride,
                                      const void* alpha, const void* beta, const float* S0, const void* gate,
                                      int64_t gate_stride, const float* norm_weight, float norm_eps, void* o,
                                      float* S_final, const int64_t* cu_seqlens, int32_t nseq, int64_t H, int64_t dk,
                                      int64_t dv, chimera_dtype dt, uint32_t flags, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);
/* Timing variant, as the ones above; capacity at least 2 * nseq + 4. */
chimera_status chimera_kda_fwd_varlen_timed(const void* q, const void* k, const void* v, int64_t qkv_stride,
                                            const void* alpha, const void* beta, const float* S0, const void* gate,
                                            int64_t gate_stride, const float* norm_weight, float norm_eps, void* o,
                                            float* S_final, const int64_t* cu_seqlens, int32_t nseq, int64_t H,
                                            int64_t dk, int64_t dv, chimera_dtype dt, uint32_t flags, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream, hipEvent_t* marks,
                                            const char** names, int32_t capacity, int32_t* used);

/*
 * Backward pass (the gradients of the two forward calls), fp32 state and accumulation.
 *
 * chimera_kda_bwd -- gradients of (o, S_final) = chimera_kda_fwd(q, k, v, alpha, beta, S0)
 * (Eq. 14 and the readout o_t = S_t^T q_t, with the per-head L2 normalisation of q and k
 * when CHIMERA_KDA_L2NORM_QK is set) against dout = dL/do and dS_final = dL/dS_final:
 *
 *   q, k, v, qkv_stride, alpha, beta, S0   the forward's inputs, as for chimera_kda_fwd
 *   dout      device [B][T][H][dv], dtype dt
 *   dS_final  device fp32 [B][H][dk][dv], or NULL for zero
 *   dq, dk    device, written, dtype dt, at the layout of q and k (token stride qkv_stride:
 *             views into one fused q|k|v gradient are accepted)
 *   dv        device, written, at the layout of v
 *   dalpha    device [B][T][H][dk], written, dtype dt
 *   dbeta     device [B][T][H], written, dtype dt
 *   dS0       device fp32 [B][H][dk][dv], written, or NULL
 *   workspace at least chimera_kda_bwd_workspace_size(...) bytes (same flags)
 *
 * dk <= 128 (CHIMERA_ERR_UNSUPPORTED above). Long sequences are cut into segments that run
 * at once, joined through each segment's transition product (the cut depends only on B, T,
 * H, dk, dv, the dtype and the flags). Two paths:
 *   - bf16 with dk = dv = 128 and T > 0, unless CHIMERA_KDA_SEQUENTIAL: the chunked form on
 *     MFMA (16-token chunks; the reverse of the chunk step of Eq. 14 per chunk, the states
 *     at chunk starts recomputed from forward passes inside the call and kept in the
 *     workspace as bf16, 32 KiB each: with segments, each segment's two halves run one
 *     after the other and only one half's states are kept, about B H ceil(T/32) of them,
 *     plus 13 fp32 d x d matrices per segment; one segment keeps all B H ceil(T/16)).
 *     q, k, v, alpha and dout must be 8-byte aligned with qkv_stride a multiple of 4, else
 *     CHIMERA_ERR_UNSUPPORTED before any launch. Like the chunked forward, it raises alpha
 *     below e^-7.5 to e^-7.5 (dalpha is then the gradient at the raised value);
 *   - otherwise token by token in fp32 (a checkpointed reverse pass: the fp32 state before
 *     every 16th token and per-slice partial sums in the workspace).
 * CHIMERA_KDA_NO_SPLIT is ignored. Asynchronous on `stream`; the outputs must not alias the
 * inputs.
 */
size_t chimera_kda_bwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, chimera_dtype dt,
                                      uint32_t flags);
chimera_status chimera_kda_bwd(const void* q, const void* k, const void* v, int64_t qkv_stride, const void* alpha,
                               const void* beta, const float* S0, const void* dout, const float* dS_final, void* dq,
                               void* dk_out, void* dv_out, void* dalpha, void* dbeta, float* dS0, int64_t B,
                               int64_t T, int64_t H, int64_t dk, int64_t dv, chimera_dtype dt, uint32_t flags,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * chimera_gate_norm_bwd -- gradients of Eq. 15's gate and norm (page 1, section 3.3; the
 * epilogue of chimera_kda_fwd_gated), y = Sigmoid(gate) * o / sqrt(mean(o^2) + norm_eps) *
 * norm_weight per (token, head) row of dv channels, against dy:
 *
 *   o             device [B][T][H][dv], dt: the KDA output before the gate (as chimera_kda_fwd
 *                 writes it)
 *   gate          device, dt, [B*T][H][dv] with consecutive tokens gate_stride elements apart
 *   norm_weight   device fp32 [dv], or NULL for ones
 *   dy            device [B][T][H][dv], dt
 *   dout          device [B][T][H][dv], written, dt: dL/do, the dout of chimera_kda_bwd
 *   dgate         device, written, dt, at the gate's layout
 *   dnorm_weight  device fp32 [dv], written (summed over every row), or NULL
 *
 * dv <= 256. The outputs must not alias the inputs. Asynchronous on `stream`.
 */
chimera_status chimera_gate_norm_bwd(const void* o, const void* gate, int64_t gate_stride, const float* norm_weight,
                                     float norm_eps, const void* dy, void* dout, void* dgate, float* dnorm_weight,
                                     int64_t B, int64_t T, int64_t H, int64_t dv, chimera_dtype dt,
                                     hipStream_t stream);

/*
 * chimera_kda_bwd_varlen -- gradients of chimera_kda_fwd_varlen (samples packed in one row,
 * the state restarting at every sample; page 1, section 3.3) without a gate: the arguments
 * of chimera_kda_bwd with B = 1 and T = cu_seqlens[nseq], and per sample its S0, dS_final
 * and dS0 ([nseq][H][dk][dv] each; S0 and dS_final may be NULL for zero). Each run of
 * consecutive samples of equal length is one batched backward on views of the packed
 * tensors; the runs share the workspace (chimera_kda_bwd_varlen_workspace_size: the
 * largest run's need). An empty sample gives dS0 = dS_final. Paths, flags and layout rules
 * as for chimera_kda_bwd (a misaligned layout is refused before the first run launches).
 */
size_t chimera_kda_bwd_varlen_workspace_size(const int64_t* cu_seqlens, int32_t nseq, int64_t H, int64_t dk,
                                             int64_t dv, chimera_dtype dt, uint32_t flags);
chimera_status chimera_kda_bwd_varlen(const void* q, const void* k, const void* v, int64_t qkv_stride,
                                      const void* alpha, const void* beta, const float* S0, const void* dout,
                                      const float* dS_final, void* dq, void* dk_out, void* dv_out, void* dalpha,
                                      void* dbeta, float* dS0, const int64_t* cu_seqlens, int32_t nseq, int64_t H,
                                      int64_t dk, int64_t dv, chimera_dtype dt, uint32_t flags, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/*
 * chimera_mshortconv_bwd -- gradients of y = chimera_mshortconv_fwd(x) against dy:
 *
 *   x, dy     device [B][T][C], dtype dt
 *   dx        device [B][T][C], written, dtype dt: dx[s, c] = sum of w[c, tap] dy[p, c] over
 *             the (p, tap) whose tap reads token s (fp32 accumulation, one rounding)
 *   dw_text   device fp32 [C][4], written: sum over batch items and text tokens p of
 *             x[src(p, tap), c] dy[p, c]
 *   dw_vis    device fp32 [C][27], written, likewise over the visual tokens
 *   w_text, w_vis, segs, nseg   as for the forward
 *
 * The weight gradients are summed with atomic adds (the order, and so the last bits, may
 * differ from run to run). Asynchronous on `stream`; dx must not alias x or dy.
 */
chimera_status chimera_mshortconv_bwd(const void* x, const void* dy, void* dx, float* dw_text, float* dw_vis,
                                      int64_t B, int64_t T, int64_t C, chimera_dtype dt, const float* w_text,
                                      const float* w_vis, const chimera_segment* segs, int32_t nseg,
                                      hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char* chimera_status_string(chimera_status s);

#ifdef __cplusplus
}
#endif
#endif /* CHIMERA_MSHORTCONV_H */
