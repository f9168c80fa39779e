// C ABI of the library: argument checks, the host neighbour table, dispatch.
// Nothing here throws; every error becomes a chimera_status before any launch.
#include "chimera_mshortconv.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include "internal.h"

using chm::Seg;

namespace {

constexpr int64_t kMaxTokens = int64_t(1) << 40;

chimera_status hip_status(hipError_t e) { return e == hipSuccess ? CHIMERA_OK : CHIMERA_ERR_HIP; }

// The segments must tile [0, T) in order (Chimera page 1, section 3.2: one
// packed stream, text first then the visual tokens; section 3.4: each segment
// is a separate view). Grids must match their lengths (Eq. 12).
chimera_status check_segments(const chimera_segment* segs, int32_t nseg, int64_t T, bool* any_text,
                              bool* any_vis) {
  if (T < 0 || T > kMaxTokens || nseg < 0) return CHIMERA_ERR_SHAPE;
  if (nseg > 0 && segs == nullptr) return CHIMERA_ERR_NULL;
  if (T > 0 && nseg == 0) return CHIMERA_ERR_SEGMENTS;
  int64_t next = 0;
  *any_text = *any_vis = false;
  for (int32_t i = 0; i < nseg; ++i) {
    const chimera_segment& s = segs[i];
    if (s.start != next || s.length < 1 || s.length > kMaxTokens) return CHIMERA_ERR_SEGMENTS;
    if (s.kind == CHIMERA_SEG_TEXT) {
      if (s.frames != 0 || s.height != 0 || s.width != 0) return CHIMERA_ERR_SEGMENTS;
      *any_text = true;
    } else if (s.kind == CHIMERA_SEG_IMAGE || s.kind == CHIMERA_SEG_VIDEO) {
      if (s.frames < 1 || s.height < 1 || s.width < 1) return CHIMERA_ERR_SEGMENTS;
      if (s.kind == CHIMERA_SEG_IMAGE && s.frames != 1) return CHIMERA_ERR_SEGMENTS;
      const int64_t n = int64_t(s.frames) * s.height * s.width;   // each factor < 2^31
      if (n != s.length) return CHIMERA_ERR_SEGMENTS;
      *any_vis = true;
    } else {
      return CHIMERA_ERR_SEGMENTS;
    }
    next = s.start + s.length;
  }
  if (next != T) return CHIMERA_ERR_SEGMENTS;
  return CHIMERA_OK;
}

Seg to_seg(const chimera_segment& s) {
  Seg g;
  g.start = s.start;
  g.length = s.length;
  g.kind = s.kind;
  g.frames = s.frames;
  g.height = s.height;
  g.width = s.width;
  return g;
}

}  // namespace

extern "C" {

const char* chimera_status_string(chimera_status s) {
  switch (s) {
    case CHIMERA_OK: return "ok";
    case CHIMERA_ERR_NULL: return "a required pointer is NULL";
    case CHIMERA_ERR_SHAPE: return "invalid size";
    case CHIMERA_ERR_DTYPE: return "unknown dtype";
    case CHIMERA_ERR_SEGMENTS: return "segment table does not tile [0, T) or a grid is malformed";
    case CHIMERA_ERR_UNSUPPORTED: return "request not supported by this library";
    case CHIMERA_ERR_WORKSPACE: return "workspace missing or too small";
    case CHIMERA_ERR_HIP: return "HIP runtime or launch failure";
  }
  return "unknown status";
}

chimera_status chimera_mshortconv_index(const chimera_segment* segs, int32_t nseg, int64_t T, int32_t* idx) {
  bool any_text, any_vis;
  const chimera_status st = check_segments(segs, nseg, T, &any_text, &any_vis);
  if (st != CHIMERA_OK) return st;
  if (T > 0 && idx == nullptr) return CHIMERA_ERR_NULL;
  if (T > (int64_t(1) << 31) / chm::kVisTaps) return CHIMERA_ERR_SHAPE;   // int32 table entries
  for (int32_t i = 0; i < nseg; ++i) {
    const Seg s = to_seg(segs[i]);
    if (s.kind == chm::SEG_TEXT) {
      for (int64_t p = s.start; p < s.start + s.length; ++p) {
        int32_t* row = idx + p * chm::kVisTaps;
        for (int j = 0; j < chm::kVisTaps; ++j)
          row[j] = j < chm::kTextTaps ? (int32_t)chm::text_tap_source(s, p, j) : -1;
      }
      continue;
    }
    for (int64_t f = 0; f < s.frames; ++f)
      for (int64_t h = 0; h < s.height; ++h)
        for (int64_t w = 0; w < s.width; ++w) {
          int32_t* row = idx + chm::raster_index(s, f, h, w) * chm::kVisTaps;
          for (int kt = 0; kt < 3; ++kt)
            for (int kh = 0; kh < 3; ++kh)
              for (int kw = 0; kw < 3; ++kw)
                row[kt * 9 + kh * 3 + kw] = (int32_t)chm::vis_tap_source(s, f, h, w, kt, kh, kw);
        }
  }
  return CHIMERA_OK;
}

chimera_status chimera_mshortconv_index_device(const chimera_segment* segs, int32_t nseg, int64_t T,
                                               int32_t* idx_dev, hipStream_t stream) {
  bool any_text, any_vis;
  const chimera_status st = check_segments(segs, nseg, T, &any_text, &any_vis);
  if (st != CHIMERA_OK) return st;
  if (T > 0 && idx_dev == nullptr) return CHIMERA_ERR_NULL;
  if (T > (int64_t(1) << 31) / chm::kVisTaps) return CHIMERA_ERR_SHAPE;
  for (int32_t i = 0; i < nseg; ++i) {
    const hipError_t e = chm::launch_index_device(to_seg(segs[i]), T, idx_dev, stream);
    if (e != hipSuccess) return CHIMERA_ERR_HIP;
  }
  return CHIMERA_OK;
}

static chimera_status conv_fwd(const void* x, void* y, int64_t B, int64_t T, int64_t C, chimera_dtype dt,
                               const float* w_text, const float* w_vis, const chimera_segment* segs, int32_t nseg,
                               hipStream_t stream, chm::Marks* marks) {
  if (dt != CHIMERA_F32 && dt != CHIMERA_BF16) return CHIMERA_ERR_DTYPE;
  if (B < 0 || C < 0) return CHIMERA_ERR_SHAPE;
  bool any_text, any_vis;
  const chimera_status st = check_segments(segs, nseg, T, &any_text, &any_vis);
  if (st != CHIMERA_OK) return st;
  if (B == 0 || T == 0 || C == 0) return CHIMERA_OK;
  if (C % 8 != 0 || C > (int64_t(1) << 24)) return CHIMERA_ERR_SHAPE;
  if (x == nullptr || y == nullptr) return CHIMERA_ERR_NULL;
  if ((any_text && w_text == nullptr) || (any_vis && w_vis == nullptr)) return CHIMERA_ERR_NULL;
  if (x == y) return CHIMERA_ERR_UNSUPPORTED;
  if (marks != nullptr && chm::mark_begin(marks, stream) != hipSuccess) return CHIMERA_ERR_HIP;
  std::vector<Seg> sv((size_t)nseg);
  for (int32_t i = 0; i < nseg; ++i) sv[(size_t)i] = to_seg(segs[i]);
  return hip_status(chm::launch_conv(x, y, B, T, C, dt == CHIMERA_BF16, w_text, w_vis, sv.data(), nseg, stream, marks));
}

chimera_status chimera_mshortconv_fwd(const void* x, void* y, int64_t B, int64_t T, int64_t C, chimera_dtype dt,
                                      const float* w_text, const float* w_vis, const chimera_segment* segs,
                                      int32_t nseg, hipStream_t stream) {
  return conv_fwd(x, y, B, T, C, dt, w_text, w_vis, segs, nseg, stream, nullptr);
}

chimera_status chimera_mshortconv_fwd_timed(const void* x, void* y, int64_t B, int64_t T, int64_t C,
                                            chimera_dtype dt, const float* w_text, const float* w_vis,
                                            const chimera_segment* segs, int32_t nseg, hipStream_t stream,
                                            hipEvent_t* marks, const char** names, int32_t capacity,
                                            int32_t* used) {
  if (marks == nullptr || names == nullptr || used == nullptr) return CHIMERA_ERR_NULL;
  *used = 0;
  if (nseg < 0 || capacity < nseg + 1) return CHIMERA_ERR_SHAPE;
  chm::Marks m{marks, names, capacity, 0};
  const chimera_status st = conv_fwd(x, y, B, T, C, dt, w_text, w_vis, segs, nseg, stream, &m);
  *used = m.n;
  return st;
}

static bool kda_sizes_ok(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv) {
  return B >= 0 && T >= 0 && H >= 0 && dk >= 1 && dk <= 256 && dv >= 1 && dv <= 256 && T <= kMaxTokens &&
         B <= (int64_t(1) << 20) && H <= (int64_t(1) << 16);
}

// Packed samples as runs of consecutive samples of equal length (chunked kernels take runs).
// cu_seqlens must already be checked.
static std::vector<chm::KdaRun> varlen_runs(const int64_t* cu, int32_t nseq) {
  std::vector<chm::KdaRun> runs;
  for (int32_t n = 0; n < nseq; ++n) {
    const int64_t len = cu[n + 1] - cu[n];
    if (!runs.empty() && runs.back().len == len) {
      ++runs.back().count;
    } else {
      runs.push_back(chm::KdaRun{cu[n], len, 1, n});
    }
  }
  return runs;
}

// 0 = c_0 <= c_1 <= ... <= c_nseq, the last at most kMaxTokens
static chimera_status check_cu(const int64_t* cu, int32_t nseq) {
  if (nseq < 0) return CHIMERA_ERR_SHAPE;
  if (cu == nullptr) return CHIMERA_ERR_NULL;
  if (cu[0] != 0) return CHIMERA_ERR_SHAPE;
  for (int32_t n = 0; n < nseq; ++n)
    if (cu[n + 1] < cu[n] || cu[n + 1] > kMaxTokens) return CHIMERA_ERR_SHAPE;
  return CHIMERA_OK;
}

// Workspace of one KDA call over `runs`; `uniform`: the one run of a [B][T] batch, whose
// token-by-token path cuts the sequences into segments unless CHIMERA_KDA_NO_SPLIT.
static size_t runs_workspace(const std::vector<chm::KdaRun>& runs, int64_t rows, int64_t H, int64_t dk, int64_t dv,
                             chimera_dtype dt, uint32_t flags, bool uniform) {
  chm::KdaArgs a{};
  a.B = 1; a.T = rows; a.H = H; a.dk = dk; a.dv = dv; a.bf16 = dt == CHIMERA_BF16;
  if (rows * H == 0) return 0;
  const bool no_split = (flags & CHIMERA_KDA_NO_SPLIT) != 0;
  if ((flags & CHIMERA_KDA_SEQUENTIAL) || !chm::kda_chunked_supported(a))
    return uniform && !no_split ? chm::kda_seq_split_workspace(runs[0].count, runs[0].len, H, dk, dv) : 0;
  return chm::kda_chunked_workspace(runs.data(), (int64_t)runs.size(), H, no_split);
}

size_t chimera_kda_workspace_size(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, chimera_dtype dt,
                                  uint32_t flags) {
  if (!kda_sizes_ok(B, T, H, dk, dv) || (dt != CHIMERA_F32 && dt != CHIMERA_BF16)) return 0;
  if (B * T == 0) return 0;
  const std::vector<chm::KdaRun> runs{chm::KdaRun{0, T, B, 0}};
  return runs_workspace(runs, B * T, H, dk, dv, dt, flags, true);
}

size_t chimera_kda_varlen_workspace_size(const int64_t* cu_seqlens, int32_t nseq, int64_t H, int64_t dk,
                                         int64_t dv, chimera_dtype dt, uint32_t flags) {
  if (check_cu(cu_seqlens, nseq) != CHIMERA_OK || (dt != CHIMERA_F32 && dt != CHIMERA_BF16)) return 0;
  const int64_t rows = cu_seqlens[nseq];
  if (!kda_sizes_ok(1, rows, H, dk, dv) || rows == 0) return 0;
  return runs_workspace(varlen_runs(cu_seqlens, nseq), rows, H, dk, dv, dt, flags, false);
}

// Output gate and norm of Eq. 15 (absent when gate == null and gated == false).
struct GateArgs {
  bool gated;
  const void* gate;
  int64_t gate_stride;
  const float* norm_w;
  float norm_eps;
};

// One KDA call over `runs` (see chm::KdaRun) of a [B][T] = [1][rows] or [B][T] token array;
// `varlen` calls come with B = 1 and T = rows.
static chimera_status kda_fwd(const void* q, const void* k, const void* v, int64_t qkv_stride, const void* alpha,
                              const void* beta, const float* S0, void* o, float* S_final, int64_t B, int64_t T,
                              int64_t H, int64_t dk, int64_t dv, chimera_dtype dt, uint32_t flags, void* workspace,
                              size_t workspace_bytes, hipStream_t stream, chm::Marks* marks, const GateArgs& g,
                              const std::vector<chm::KdaRun>* varlen = nullptr) {
  if (dt != CHIMERA_F32 && dt != CHIMERA_BF16) return CHIMERA_ERR_DTYPE;
  if (!kda_sizes_ok(B, T, H, dk, dv)) return CHIMERA_ERR_SHAPE;
  if (flags & ~(CHIMERA_KDA_L2NORM_QK | CHIMERA_KDA_SEQUENTIAL | CHIMERA_KDA_NO_SPLIT)) return CHIMERA_ERR_UNSUPPORTED;
  if (B == 0 || H == 0 || (varlen != nullptr && varlen->empty())) return CHIMERA_OK;
  if (T > 0) {
    if (q == nullptr || k == nullptr || v == nullptr || alpha == nullptr || beta == nullptr || o == nullptr)
      return CHIMERA_ERR_NULL;
    if (qkv_stride < H * dk || qkv_stride < H * dv) return CHIMERA_ERR_SHAPE;
    if (g.gated) {
      if (g.gate == nullptr) return CHIMERA_ERR_NULL;
      if (g.gate_stride < H * dv || g.gate_stride > (int64_t(1) << 40)) return CHIMERA_ERR_SHAPE;
    }
  }
  if (g.gated && !(g.norm_eps >= 0.f && g.norm_eps < 3.0e38f)) return CHIMERA_ERR_SHAPE;   // NaN fails too
  chm::KdaArgs a;
  a.q = q; a.k = k; a.v = v; a.qkv_stride = qkv_stride; a.alpha = alpha; a.beta = beta;
  a.S0 = S0; a.o = o; a.S_final = S_final;
  a.B = B; a.T = T; a.H = H; a.dk = dk; a.dv = dv;
  a.bf16 = dt == CHIMERA_BF16;
  a.l2norm = (flags & CHIMERA_KDA_L2NORM_QK) != 0;
  if (g.gated && T > 0) {
    a.gate = g.gate;
    a.gate_stride = g.gate_stride;
    a.norm_w = g.norm_w;
    a.norm_eps = g.norm_eps;
  }
  const std::vector<chm::KdaRun> uniform{chm::KdaRun{0, T, B, 0}};
  const std::vector<chm::KdaRun>& runs = varlen != nullptr ? *varlen : uniform;
  const bool chunked = !(flags & CHIMERA_KDA_SEQUENTIAL) && chm::kda_chunked_supported(a) && B * T > 0;
  const bool no_split = (flags & CHIMERA_KDA_NO_SPLIT) != 0;
  if (chunked) {
    if (!chm::kda_chunked_plan_ok(runs.data(), (int64_t)runs.size(), H, no_split)) return CHIMERA_ERR_SHAPE;
    const size_t need = chm::kda_chunked_workspace(runs.data(), (int64_t)runs.size(), H, no_split);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return CHIMERA_ERR_WORKSPACE;
  }
  const bool seq_split = !chunked && varlen == nullptr && !no_split && B * T > 0;
  if (seq_split) {
    const size_t need = chm::kda_seq_split_workspace(B, T, H, dk, dv);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return CHIMERA_ERR_WORKSPACE;
  }
  if (marks != nullptr && chm::mark_begin(marks, stream) != hipSuccess) return CHIMERA_ERR_HIP;
  if (chunked) return hip_status(chm::launch_kda_chunked(a, runs.data(), (int64_t)runs.size(), no_split, workspace,
                                                         stream, marks));
  if (seq_split) return hip_status(chm::launch_kda_sequential_split(a, workspace, stream, marks));
  if (varlen == nullptr) return hip_status(chm::launch_kda_sequential(a, stream, marks));
  // token-by-token kernel: one launch per run, on views of the packed tensors
  const int64_t e = dt == CHIMERA_BF16 ? 2 : 4;
  for (const chm::KdaRun& r : runs) {
    chm::KdaArgs s = a;
    auto at = [&](const void* p, int64_t elems) {
      return p == nullptr ? nullptr : static_cast<const void*>(static_cast<const char*>(p) + elems * e);
    };
    s.q = at(q, r.start * qkv_stride);
    s.k = at(k, r.start * qkv_stride);
    s.v = at(v, r.start * qkv_stride);
    s.alpha = at(alpha, r.start * H * dk);
    s.beta = at(beta, r.start * H);
    s.o = const_cast<void*>(at(o, r.start * H * dv));
    s.gate = a.gate == nullptr ? nullptr : at(a.gate, r.start * a.gate_stride);
    s.S0 = S0 == nullptr ? nullptr : S0 + r.sidx0 * H * dk * dv;
    s.S_final = S_final == nullptr ? nullptr : S_final + r.sidx0 * H * dk * dv;
    s.B = r.count;
    s.T = r.len;
    const hipError_t he = chm::launch_kda_sequential(s, stream, marks);
    if (he != hipSuccess) return CHIMERA_ERR_HIP;
  }
  return CHIMERA_OK;
}

// The fused conv + recurrence: argument checks, then the chunked kernels with the conv in their
// load stage (bf16, dk = dv = 128, the window a chunk's taps reach within 32-bit offsets, unless
// CHIMERA_KDA_SEQUENTIAL), else the token-by-token kernel. need = the chunked path's workspace
// bytes (0 for the token-by-token kernel).
struct ConvCall {
  chm::ConvSrc cs;
  chm::KdaArgs a;
  bool chunked = false;
  size_t need = 0;
};
static chimera_status conv_call(const void* x, const float* w_text, const float* w_vis, const chimera_segment* segs,
                                int32_t nseg, const void* alpha, const void* beta, const float* S0, void* o,
                                float* S_final, int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                chimera_dtype dt, uint32_t flags, bool check_ptrs, ConvCall& c) {
  if (dt != CHIMERA_F32 && dt != CHIMERA_BF16) return CHIMERA_ERR_DTYPE;
  if (!kda_sizes_ok(B, T, H, dk, dv)) return CHIMERA_ERR_SHAPE;
  if (dk > 128) return CHIMERA_ERR_UNSUPPORTED;
  if (flags & ~(CHIMERA_KDA_L2NORM_QK | CHIMERA_KDA_SEQUENTIAL | CHIMERA_KDA_NO_SPLIT)) return CHIMERA_ERR_UNSUPPORTED;
  bool any_text, any_vis;
  const chimera_status st = check_segments(segs, nseg, T, &any_text, &any_vis);
  if (st != CHIMERA_OK) return st;
  if (nseg > chm::kMaxFusedSegs) return CHIMERA_ERR_UNSUPPORTED;
  if (check_ptrs && B > 0 && H > 0 && T > 0) {
    if (x == nullptr || alpha == nullptr || beta == nullptr || o == nullptr) return CHIMERA_ERR_NULL;
    if ((any_text && w_text == nullptr) || (any_vis && w_vis == nullptr)) return CHIMERA_ERR_NULL;
    if (x == o) return CHIMERA_ERR_UNSUPPORTED;
  }
  c.cs.x = x;
  c.cs.C = H * (2 * dk + dv);
  c.cs.w_text = w_text;
  c.cs.w_vis = w_vis;
  c.cs.nseg = nseg;
  for (int32_t i = 0; i < nseg; ++i) c.cs.seg[i] = to_seg(segs[i]);
  chm::KdaArgs& a = c.a;
  a.q = a.k = a.v = nullptr;
  a.qkv_stride = c.cs.C;
  a.alpha = alpha; a.beta = beta;
  a.S0 = S0; a.o = o; a.S_final = S_final;
  a.B = B; a.T = T; a.H = H; a.dk = dk; a.dv = dv;
  a.bf16 = dt == CHIMERA_BF16;
  a.l2norm = (flags & CHIMERA_KDA_L2NORM_QK) != 0;
  a.conv = &c.cs;
  c.chunked = !(flags & CHIMERA_KDA_SEQUENTIAL) && B * T * H > 0 && chm::kda_chunked_supported(a) &&
              chm::kda_chunked_conv_supported(a);
  if (c.chunked) {
    const chm::KdaRun run{0, T, B, 0};
    const bool no_split = (flags & CHIMERA_KDA_NO_SPLIT) != 0;
    if (!chm::kda_chunked_plan_ok(&run, 1, H, no_split)) return CHIMERA_ERR_SHAPE;
    c.need = chm::kda_chunked_workspace(&run, 1, H, no_split, &c.cs);
  }
  return CHIMERA_OK;
}

size_t chimera_kda_conv_workspace_size(const chimera_segment* segs, int32_t nseg, int64_t B, int64_t T, int64_t H,
                                       int64_t dk, int64_t dv, chimera_dtype dt, uint32_t flags) {
  ConvCall c;
  if (conv_call(nullptr, nullptr, nullptr, segs, nseg, nullptr, nullptr, nullptr, nullptr, nullptr, B, T, H, dk, dv,
                dt, flags, false, c) != CHIMERA_OK)
    return 0;
  return c.need;
}

static chimera_status kda_fwd_conv(const void* x, const float* w_text, const float* w_vis,
                                   const chimera_segment* segs, int32_t nseg, const void* alpha, const void* beta,
                                   const float* S0, void* o, float* S_final, int64_t B, int64_t T, int64_t H,
                                   int64_t dk, int64_t dv, chimera_dtype dt, uint32_t flags, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream, chm::Marks* marks) {
  ConvCall c;
  const chimera_status st = conv_call(x, w_text, w_vis, segs, nseg, alpha, beta, S0, o, S_final, B, T, H, dk, dv, dt,
                                      flags, true, c);
  if (st != CHIMERA_OK) return st;
  if (B == 0 || H == 0) return CHIMERA_OK;
  if (c.chunked && (workspace == nullptr || workspace_bytes < c.need)) return CHIMERA_ERR_WORKSPACE;
  if (marks != nullptr && chm::mark_begin(marks, stream) != hipSuccess) return CHIMERA_ERR_HIP;
  if (c.chunked) {
    const chm::KdaRun run{0, T, B, 0};
    return hip_status(chm::launch_kda_chunked(c.a, &run, 1, (flags & CHIMERA_KDA_NO_SPLIT) != 0, workspace, stream,
                                              marks));
  }
  return hip_status(chm::launch_kda_sequential(c.a, stream, marks));
}

chimera_status chimera_kda_fwd_conv(const void* x, const float* w_text, const float* w_vis,
                                    const chimera_segment* segs, int32_t nseg, const void* alpha, const void* beta,
                                    const float* S0, void* o, float* S_final, int64_t B, int64_t T, int64_t H,
                                    int64_t dk, int64_t dv, chimera_dtype dt, uint32_t flags, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  return kda_fwd_conv(x, w_text, w_vis, segs, nseg, alpha, beta, S0, o, S_final, B, T, H, dk, dv, dt, flags,
                      workspace, workspace_bytes, stream, nullptr);
}

chimera_status chimera_kda_fwd_conv_timed(const void* x, const float* w_text, const float* w_vis,
                                          const chimera_segment* segs, int32_t nseg, const void* alpha,
                                          const void* beta, const float* S0, void* o, float* S_final, int64_t B,
                                          int64_t T, int64_t H, int64_t dk, int64_t dv, chimera_dtype dt,
                                          uint32_t flags, void* workspace, size_t workspace_bytes, hipStream_t stream,
                                          hipEvent_t* marks, const char** names, int32_t capacity, int32_t* used) {
  if (marks == nullptr || names == nullptr || used == nullptr) return CHIMERA_ERR_NULL;
  *used = 0;
  if (capacity < CHIMERA_KDA_CONV_MAX_KERNELS + 1) return CHIMERA_ERR_SHAPE;
  chm::Marks m{marks, names, capacity, 0};
  const chimera_status st = kda_fwd_conv(x, w_text, w_vis, segs, nseg, alpha, beta, S0, o, S_final, B, T, H, dk, dv,
                                         dt, flags, workspace, workspace_bytes, stream, &m);
  *used = m.n;
  return st;
}

chimera_status chimera_kda_fwd(const void* q, const void* k, const void* v, int64_t qkv_stride, const void* alpha,
                               const void* beta, const float* S0, void* o, float* S_final, int64_t B, int64_t T,
                               int64_t H, int64_t dk, int64_t dv, chimera_dtype dt, uint32_t flags, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  return kda_fwd(q, k, v, qkv_stride, alpha, beta, S0, o, S_final, B, T, H, dk, dv, dt, flags, workspace,
                 workspace_bytes, stream, nullptr, GateArgs{false, nullptr, 0, nullptr, 0.f});
}

chimera_status chimera_kda_fwd_timed(const void* q, const void* k, const void* v, int64_t qkv_stride,
                                     const void* alpha, const void* beta, const float* S0, void* o, float* S_final,
                                     int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, chimera_dtype dt,
                                     uint32_t flags, void* workspace, size_t workspace_bytes, hipStream_t stream,
                                     hipEvent_t* marks, const char** names, int32_t capacity, int32_t* used) {
  if (marks == nullptr || names == nullptr || used == nullptr) return CHIMERA_ERR_NULL;
  *used = 0;
  if (capacity < CHIMERA_KDA_MAX_KERNELS + 1) return CHIMERA_ERR_SHAPE;
  chm::Marks m{marks, names, capacity, 0};
  const chimera_status st = kda_fwd(q, k, v, qkv_stride, alpha, beta, S0, o, S_final, B, T, H, dk, dv, dt, flags,
                                    workspace, workspace_bytes, stream, &m, GateArgs{false, nullptr, 0, nullptr, 0.f});
  *used = m.n;
  return st;
}

chimera_status chimera_kda_fwd_gated(const void* q, const void* k, const void* v, int64_t qkv_stride,
                                     const void* alpha, const void* beta, const float* S0, const void* gate,
                                     int64_t gate_stride, const float* norm_weight, float norm_eps, void* o,
                                     float* S_final, int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                     chimera_dtype dt, uint32_t flags, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  return kda_fwd(q, k, v, qkv_stride, alpha, beta, S0, o, S_final, B, T, H, dk, dv, dt, flags, workspace,
                 workspace_bytes, stream, nullptr, GateArgs{true, gate, gate_stride, norm_weight, norm_eps});
}

chimera_status chimera_kda_fwd_gated_timed(const void* q, const void* k, const void* v, int64_t qkv_stride,
                                           const void* alpha, const void* beta, const float* S0, const void* gate,
                                           int64_t gate_stride, const float* norm_weight, float norm_eps, void* o,
                                           float* S_final, int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                           chimera_dtype dt, uint32_t flags, void* workspace, size_t workspace_bytes,
                                           hipStream_t stream, hipEvent_t* marks, const char** names,
                                           int32_t capacity, int32_t* used) {
  if (marks == nullptr || names == nullptr || used == nullptr) return CHIMERA_ERR_NULL;
  *used = 0;
  if (capacity < CHIMERA_KDA_GATED_MAX_KERNELS + 1) return CHIMERA_ERR_SHAPE;
  chm::Marks m{marks, names, capacity, 0};
  const chimera_status st =
      kda_fwd(q, k, v, qkv_stride, alpha, beta, S0, o, S_final, B, T, H, dk, dv, dt, flags, workspace,
              workspace_bytes, stream, &m, GateArgs{true, gate, gate_stride, norm_weight, norm_eps});
  *used = m.n;
  return st;
}

static chimera_status kda_fwd_varlen(const void* q, const void* k, const void* v, int64_t qkv_stride,
                                     const void* alpha, const void* beta, const float* S0, const void* gate,
                                     int64_t gate_stride, const float* norm_weight, float norm_eps, void* o,
                                     float* S_final, const int64_t* cu_seqlens, int32_t nseq, int64_t H, int64_t dk,
                                     int64_t dv, chimera_dtype dt, uint32_t flags, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream, chm::Marks* marks) {
  const chimera_status cs = check_cu(cu_seqlens, nseq);
  if (cs != CHIMERA_OK) return cs;
  const std::vector<chm::KdaRun> runs = varlen_runs(cu_seqlens, nseq);
  const GateArgs g{gate != nullptr, gate, gate_stride, norm_weight, norm_eps};
  return kda_fwd(q, k, v, qkv_stride, alpha, beta, S0, o, S_final, 1, cu_seqlens[nseq], H, dk, dv, dt, flags,
                 workspace, workspace_bytes, stream, marks, g, &runs);
}

chimera_status chimera_kda_fwd_varlen(const void* q, const void* k, const void* v, int64_t qkv_stride,
                                      const void* alpha, const void* beta, const float* S0, const void* gate,
                                      int64_t gate_stride, const float* norm_weight, float norm_eps, void* o,
                                      float* S_final, const int64_t* cu_seqlens, int32_t nseq, int64_t H, int64_t dk,
                                      int64_t dv, chimera_dtype dt, uint32_t flags, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  return kda_fwd_varlen(q, k, v, qkv_stride, alpha, beta, S0, gate, gate_stride, norm_weight, norm_eps, o, S_final,
                        cu_seqlens, nseq, H, dk, dv, dt, flags, workspace, workspace_bytes, stream, nullptr);
}

chimera_status chimera_kda_fwd_varlen_timed(const void* q, const void* k, const void* v, int64_t qkv_stride,
                                            const void* alpha, const void* beta, const float* S0, const void* gate,
                                            int64_t gate_stride, const float* norm_weight, float norm_eps, void* o,
                                            float* S_final, const int64_t* cu_seqlens, int32_t nseq, int64_t H,
                                            int64_t dk, int64_t dv, chimera_dtype dt, uint32_t flags, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream, hipEvent_t* marks,
                                            const char** names, int32_t capacity, int32_t* used) {
  if (marks == nullptr || names == nullptr || used == nullptr) return CHIMERA_ERR_NULL;
  *used = 0;
  if (nseq < 0 || (int64_t)capacity < 2 * (int64_t)nseq + 4) return CHIMERA_ERR_SHAPE;
  chm::Marks m{marks, names, capacity, 0};
  const chimera_status st =
      kda_fwd_varlen(q, k, v, qkv_stride, alpha, beta, S0, gate, gate_stride, norm_weight, norm_eps, o, S_final,
                     cu_seqlens, nseq, H, dk, dv, dt, flags, workspace, workspace_bytes, stream, &m);
  *used = m.n;
  return st;
}

// The backward runs on the chunked MFMA kernels for bf16 heads of 128 (unless
// CHIMERA_KDA_SEQUENTIAL), on the token-by-token kernels otherwise.
static bool bwd_chunked(int64_t T, int64_t dk, int64_t dv, chimera_dtype dt, uint32_t flags) {
  return T > 0 && (flags & CHIMERA_KDA_SEQUENTIAL) == 0 && chm::kda_bwd_chunked_shape(dk, dv, dt == CHIMERA_BF16);
}
static size_t bwd_workspace(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, chimera_dtype dt,
                            uint32_t flags) {
  return bwd_chunked(T, dk, dv, dt, flags) ? chm::kda_bwd_chunked_workspace(B, T, H)
                                           : chm::kda_bwd_workspace(B, T, H, dk, dv);
}
static hipError_t bwd_launch(const chm::KdaArgs& a, const chm::KdaGrads& g, chimera_dtype dt, uint32_t flags,
                             void* workspace, hipStream_t stream) {
  return bwd_chunked(a.T, a.dk, a.dv, dt, flags) ? chm::launch_kda_backward_chunked(a, g, workspace, stream)
                                                 : chm::launch_kda_backward(a, g, workspace, stream);
}

size_t chimera_kda_bwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, chimera_dtype dt,
                                      uint32_t flags) {
  if (!kda_sizes_ok(B, T, H, dk, dv) || dk > 128 || (dt != CHIMERA_F32 && dt != CHIMERA_BF16)) return 0;
  return bwd_workspace(B, T, H, dk, dv, dt, flags);
}

chimera_status chimera_kda_bwd(const void* q, const void* k, const void* v, int64_t qkv_stride, const void* alpha,
                               const void* beta, const float* S0, const void* dout, const float* dS_final, void* dq,
                               void* dk_out, void* dv_out, void* dalpha, void* dbeta, float* dS0, int64_t B,
                               int64_t T, int64_t H, int64_t dk, int64_t dv, chimera_dtype dt, uint32_t flags,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (dt != CHIMERA_F32 && dt != CHIMERA_BF16) return CHIMERA_ERR_DTYPE;
  if (!kda_sizes_ok(B, T, H, dk, dv)) return CHIMERA_ERR_SHAPE;
  if (dk > 128) return CHIMERA_ERR_UNSUPPORTED;
  if (flags & ~(CHIMERA_KDA_L2NORM_QK | CHIMERA_KDA_SEQUENTIAL | CHIMERA_KDA_NO_SPLIT)) return CHIMERA_ERR_UNSUPPORTED;
  if (B == 0 || H == 0) return CHIMERA_OK;
  if (T > 0) {
    if (q == nullptr || k == nullptr || v == nullptr || alpha == nullptr || beta == nullptr || dout == nullptr ||
        dq == nullptr || dk_out == nullptr || dv_out == nullptr || dalpha == nullptr || dbeta == nullptr)
      return CHIMERA_ERR_NULL;
    if (qkv_stride < H * dk || qkv_stride < H * dv) return CHIMERA_ERR_SHAPE;
  }
  const size_t need = bwd_workspace(B, T, H, dk, dv, dt, flags);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return CHIMERA_ERR_WORKSPACE;
  chm::KdaArgs a{};
  a.q = q; a.k = k; a.v = v; a.qkv_stride = qkv_stride; a.alpha = alpha; a.beta = beta;
  a.S0 = S0; a.o = nullptr; a.S_final = nullptr;
  a.B = B; a.T = T; a.H = H; a.dk = dk; a.dv = dv;
  a.bf16 = dt == CHIMERA_BF16;
  a.l2norm = (flags & CHIMERA_KDA_L2NORM_QK) != 0;
  const chm::KdaGrads g{dout, dS_final, dq, dk_out, dv_out, dalpha, dbeta, dS0};
  if (bwd_chunked(T, dk, dv, dt, flags) && !chm::kda_bwd_chunked_layout_ok(a, g)) return CHIMERA_ERR_UNSUPPORTED;
  return hip_status(bwd_launch(a, g, dt, flags, workspace, stream));
}

chimera_status chimera_gate_norm_bwd(const void* o, const void* gate, int64_t gate_stride, const float* norm_weight,
                                     float norm_eps, const void* dy, void* dout, void* dgate, float* dnorm_weight,
                                     int64_t B, int64_t T, int64_t H, int64_t dv, chimera_dtype dt,
                                     hipStream_t stream) {
  if (dt != CHIMERA_F32 && dt != CHIMERA_BF16) return CHIMERA_ERR_DTYPE;
  if (!kda_sizes_ok(B, T, H, 1, dv)) return CHIMERA_ERR_SHAPE;
  if (!(norm_eps >= 0.f && norm_eps < 3.0e38f)) return CHIMERA_ERR_SHAPE;   // NaN fails too
  const int64_t rows = B * T * H;
  if (rows > 0) {
    if (o == nullptr || gate == nullptr || dy == nullptr || dout == nullptr || dgate == nullptr)
      return CHIMERA_ERR_NULL;
    if (gate_stride < H * dv || gate_stride > (int64_t(1) << 40)) return CHIMERA_ERR_SHAPE;
    if (dout == o || dout == dy || dgate == gate) return CHIMERA_ERR_UNSUPPORTED;
  }
  if (rows == 0 && dnorm_weight == nullptr) return CHIMERA_OK;
  return hip_status(chm::launch_gate_norm_backward(o, gate, gate_stride, norm_weight, norm_eps, dy, dout, dgate,
                                                   dnorm_weight, rows, H, dv, dt == CHIMERA_BF16, stream));
}

size_t chimera_kda_bwd_varlen_workspace_size(const int64_t* cu_seqlens, int32_t nseq, int64_t H, int64_t dk,
                                             int64_t dv, chimera_dtype dt, uint32_t flags) {
  (void)flags;
  if (check_cu(cu_seqlens, nseq) != CHIMERA_OK || (dt != CHIMERA_F32 && dt != CHIMERA_BF16)) return 0;
  if (!kda_sizes_ok(1, cu_seqlens[nseq], H, dk, dv)) return 0;
  size_t need = 0;
  for (const chm::KdaRun& r : varlen_runs(cu_seqlens, nseq))
    need = std::max(need, bwd_workspace(r.count, r.len, H, dk, dv, dt, flags));
  return need;
}

chimera_status chimera_kda_bwd_varlen(const void* q, const void* k, const void* v, int64_t qkv_stride,
                                      const void* alpha, const void* beta, const float* S0, const void* dout,
                                      const float* dS_final, void* dq, void* dk_out, void* dv_out, void* dalpha,
                                      void* dbeta, float* dS0, const int64_t* cu_seqlens, int32_t nseq, int64_t H,
                                      int64_t dk, int64_t dv, chimera_dtype dt, uint32_t flags, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  if (dt != CHIMERA_F32 && dt != CHIMERA_BF16) return CHIMERA_ERR_DTYPE;
  const chimera_status cs = check_cu(cu_seqlens, nseq);
  if (cs != CHIMERA_OK) return cs;
  const int64_t rows = cu_seqlens[nseq];
  if (!kda_sizes_ok(1, rows, H, dk, dv)) return CHIMERA_ERR_SHAPE;
  if (dk > 128) return CHIMERA_ERR_UNSUPPORTED;
  if (flags & ~(CHIMERA_KDA_L2NORM_QK | CHIMERA_KDA_SEQUENTIAL | CHIMERA_KDA_NO_SPLIT)) return CHIMERA_ERR_UNSUPPORTED;
  if (nseq == 0 || H == 0) return CHIMERA_OK;
  if (rows > 0) {
    if (q == nullptr || k == nullptr || v == nullptr || alpha == nullptr || beta == nullptr || dout == nullptr ||
        dq == nullptr || dk_out == nullptr || dv_out == nullptr || dalpha == nullptr || dbeta == nullptr)
      return CHIMERA_ERR_NULL;
    if (qkv_stride < H * dk || qkv_stride < H * dv) return CHIMERA_ERR_SHAPE;
  }
  const std::vector<chm::KdaRun> runs = varlen_runs(cu_seqlens, nseq);
  size_t need = 0;
  for (const chm::KdaRun& r : runs) need = std::max(need, bwd_workspace(r.count, r.len, H, dk, dv, dt, flags));
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return CHIMERA_ERR_WORKSPACE;
  if (rows > 0 && bwd_chunked(rows, dk, dv, dt, flags)) {
    // a run's views start a whole number of rows in, which keeps the base pointers' alignment
    chm::KdaArgs a{};
    a.q = q; a.k = k; a.v = v; a.qkv_stride = qkv_stride; a.alpha = alpha;
    const chm::KdaGrads g{dout, dS_final, dq, dk_out, dv_out, dalpha, dbeta, dS0};
    if (!chm::kda_bwd_chunked_layout_ok(a, g)) return CHIMERA_ERR_UNSUPPORTED;
  }
  // each run of equal lengths is a batch on views of the packed tensors; the runs share the workspace
  const int64_t e = dt == CHIMERA_BF16 ? 2 : 4;
  auto at = [&](const void* p, int64_t elems) {
    return p == nullptr ? nullptr : static_cast<const char*>(p) + elems * e;
  };
  auto mut = [&](void* p, int64_t elems) { return p == nullptr ? nullptr : static_cast<char*>(p) + elems * e; };
  const int64_t state = H * dk * dv;
  for (const chm::KdaRun& r : runs) {
    chm::KdaArgs a{};
    a.q = at(q, r.start * qkv_stride); a.k = at(k, r.start * qkv_stride); a.v = at(v, r.start * qkv_stride);
    a.qkv_stride = qkv_stride;
    a.alpha = at(alpha, r.start * H * dk); a.beta = at(beta, r.start * H);
    a.S0 = S0 == nullptr ? nullptr : S0 + r.sidx0 * state;
    a.o = nullptr; a.S_final = nullptr;
    a.B = r.count; a.T = r.len; a.H = H; a.dk = dk; a.dv = dv;
    a.bf16 = dt == CHIMERA_BF16;
    a.l2norm = (flags & CHIMERA_KDA_L2NORM_QK) != 0;
    const chm::KdaGrads g{at(dout, r.start * H * dv), dS_final == nullptr ? nullptr : dS_final + r.sidx0 * state,
                          mut(dq, r.start * qkv_stride), mut(dk_out, r.start * qkv_stride),
                          mut(dv_out, r.start * qkv_stride), mut(dalpha, r.start * H * dk), mut(dbeta, r.start * H),
                          dS0 == nullptr ? nullptr : dS0 + r.sidx0 * state};
    const hipError_t he = bwd_launch(a, g, dt, flags, workspace, stream);
    if (he != hipSuccess) return CHIMERA_ERR_HIP;
  }
  return CHIMERA_OK;
}

chimera_status chimera_mshortconv_bwd(const void* x, const void* dy, void* dx, float* dw_text, float* dw_vis,
                                      int64_t B, int64_t T, int64_t C, chimera_dtype dt, const float* w_text,
                                      const float* w_vis, const chimera_segment* segs, int32_t nseg,
                                      hipStream_t stream) {
  if (dt != CHIMERA_F32 && dt != CHIMERA_BF16) return CHIMERA_ERR_DTYPE;
  if (B < 0 || C < 0) return CHIMERA_ERR_SHAPE;
  bool any_text, any_vis;
  const chimera_status st = check_segments(segs, nseg, T, &any_text, &any_vis);
  if (st != CHIMERA_OK) return st;
  if (C % 8 != 0 || C > (int64_t(1) << 24)) return CHIMERA_ERR_SHAPE;
  if (dw_text == nullptr || dw_vis == nullptr) return CHIMERA_ERR_NULL;
  if (B > 0 && T > 0) {
    if (x == nullptr || dy == nullptr || dx == nullptr) return CHIMERA_ERR_NULL;
    if ((any_text && w_text == nullptr) || (any_vis && w_vis == nullptr)) return CHIMERA_ERR_NULL;
    if (dx == x || dx == dy) return CHIMERA_ERR_UNSUPPORTED;
  }
  std::vector<Seg> sv((size_t)nseg);
  for (int32_t i = 0; i < nseg; ++i) sv[(size_t)i] = to_seg(segs[i]);
  return hip_status(chm::launch_conv_backward(x, dy, dx, dw_text, dw_vis, B, T, C, dt == CHIMERA_BF16, w_text,
                                              w_vis, sv.data(), nseg, stream));
}

}  // extern "C"
