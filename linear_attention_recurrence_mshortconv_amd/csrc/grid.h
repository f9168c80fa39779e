// Segment geometry shared by the host index builder and the device kernels.
//
// Chimera page 1, section 3.3, Eq. 12: inside a visual segment, grid point
// (i, j, k) = (time, height, width) sits at raster index m = i*H*W + j*W + k;
// section 3.4: each modality segment is convolved on its own (zero outside
// it), causal in time and symmetric in space; text is causal 1D.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define CHM_HD __host__ __device__ __forceinline__
#else
#define CHM_HD inline
#endif

namespace chm {

enum : int32_t { SEG_TEXT = 0, SEG_IMAGE = 1, SEG_VIDEO = 2 };
constexpr int kTextTaps = 4;
constexpr int kVisTaps = 27;

// Kernel-argument copy of one segment (plain data, passed by value).
struct Seg {
  int64_t start;
  int64_t length;
  int32_t kind;
  int32_t frames;
  int32_t height;
  int32_t width;
};

// Eq. 12: raster position of grid point (f, h, w) of a visual segment.
CHM_HD int64_t raster_index(const Seg& s, int64_t f, int64_t h, int64_t w) {
  return s.start + (f * s.height + h) * (int64_t)s.width + w;
}

// True when (f, h, w) lies on the segment's grid.
CHM_HD bool grid_inside(const Seg& s, int64_t f, int64_t h, int64_t w) {
  return f >= 0 && f < s.frames && h >= 0 && h < s.height && w >= 0 && w < s.width;
}

// Source token of visual tap (kt, kh, kw) for the token at grid point
// (f, h, w), or -1 when the tap reads zero padding. Offsets (kt-2, kh-1, kw-1).
CHM_HD int64_t vis_tap_source(const Seg& s, int64_t f, int64_t h, int64_t w, int kt, int kh, int kw) {
  const int64_t ff = f + kt - 2, hh = h + kh - 1, ww = w + kw - 1;
  return grid_inside(s, ff, hh, ww) ? raster_index(s, ff, hh, ww) : -1;
}

// Source token of text tap j (offset j - 3) for token p of a text segment.
CHM_HD int64_t text_tap_source(const Seg& s, int64_t p, int j) {
  const int64_t src = p + j - (kTextTaps - 1);
  return src >= s.start ? src : -1;
}

}  // namespace chm
