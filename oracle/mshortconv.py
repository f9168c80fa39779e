"""Oracle for the modality-aware short convolution (mShortConv), fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix (Chimera, page 1, sections 3.3-3.4; page 2, mShortConv
paragraph):

* Eq. 13: q, k and v are each passed through the short convolution before
  the recurrence; the conv is depthwise (one kernel per channel).
* Text tokens are gathered from their packed positions and mixed by a causal
  1D depthwise conv along the text segment.
* Visual tokens are viewed as their (time, height, width) grid and mixed by a
  depthwise 3D conv; an image is the special case of one frame.
* The conv runs inside each modality segment on its own: no kernel crosses a
  text/visual or sample boundary. Outputs return to their packed positions.
* Along time the 3D conv is causal (current and earlier frames only); in
  space it is symmetric.
* Eq. 12: grid point (i, j, k) (time, height, width) sits at raster index
  m = i*H*W + j*W + k inside its segment.

Readings where the pages leave a step open:

* Kernel sizes: 4 taps for text; 3x3x3 for visual grids.
* Tap j of the text kernel reads offset j - 3 (taps 0..3 read p-3 .. p).
  Visual tap (kt, kh, kw), stored row-major as kt*9 + kh*3 + kw, reads
  offset (kt - 2, kh - 1, kw - 1). This is cross-correlation.
* Taps that fall outside the segment (before the text start, before frame 0,
  outside a frame's rows or columns) read zero; nothing wraps from one row to
  the next.
* One visual kernel per channel; an image uses only its kt = 2 slice.
* No bias and no activation after the conv.
"""
from __future__ import annotations

import numpy as np

TEXT, IMAGE, VIDEO = 0, 1, 2
N_TEXT_TAPS = 4
N_VIS_TAPS = 27


def _seg_fields(seg):
    """Accept a dataclass-like object or a dict describing one segment."""
    if isinstance(seg, dict):
        g = seg.get
        return int(g("kind")), int(g("start")), int(g("length")), int(g("frames", 0)), \
            int(g("height", 0)), int(g("width", 0))
    return int(seg.kind), int(seg.start), int(seg.length), int(seg.frames), \
        int(seg.height), int(seg.width)


def neighbours_ref(segments, T: int) -> np.ndarray:
    """Source position of every conv tap, -1 where the tap reads zero padding.

    Returns int32 [T, 27]. Text rows use taps 0..3 (offsets -3..0 along the
    text segment) and hold -1 in taps 4..26. Visual rows use all 27 taps in
    (kt, kh, kw) row-major order (offsets kt-2, kh-1, kw-1 on the grid).
    Eq. 12 (page 1, section 3.3) maps grid coordinates to raster positions.
    """
    idx = np.full((T, N_VIS_TAPS), -1, dtype=np.int64)
    for seg in segments:
        kind, start, length, F, Hh, Ww = _seg_fields(seg)
        if length == 0:
            continue
        if kind == TEXT:
            pos = np.arange(start, start + length)
            for j in range(N_TEXT_TAPS):
                src = pos + (j - 3)
                ok = src >= start
                idx[pos[ok], j] = src[ok]
            continue
        assert F * Hh * Ww == length, "visual segment length must equal frames*height*width"
        m = np.arange(length)
        # invert Eq. 12: m = i*H*W + j*W + k
        i = m // (Hh * Ww)
        j = (m // Ww) % Hh
        kk = m % Ww
        for kt in range(3):
            for kh in range(3):
                for kw in range(3):
                    ti, hj, wk = i + (kt - 2), j + (kh - 1), kk + (kw - 1)
                    ok = (ti >= 0) & (hj >= 0) & (hj < Hh) & (wk >= 0) & (wk < Ww)
                    src = start + ti * Hh * Ww + hj * Ww + wk      # Eq. 12
                    idx[start + m[ok], kt * 9 + kh * 3 + kw] = src[ok]
    return idx.astype(np.int32)


def conv_ref(x: np.ndarray, w_text: np.ndarray, w_vis: np.ndarray, segments) -> np.ndarray:
    """mShortConv by the segment-view definition (page 1, section 3.4).

    x [B, T, C] (any float dtype, used exactly in fp64), w_text [C, 4],
    w_vis [C, 27]. Returns fp64 [B, T, C].

    Text segments: zero-pad three tokens in front of the segment and sum the
    shifted copies, tap j weighting the copy shifted by j - 3. Visual
    segments: reshape to [B, F, H, W, C], zero-pad (2, 0) in time and (1, 1)
    in height and width, and sum the 27 shifted copies.
    """
    x = np.asarray(x, dtype=np.float64)
    wt = np.asarray(w_text, dtype=np.float64)
    wv = np.asarray(w_vis, dtype=np.float64)
    B, T, C = x.shape
    y = np.zeros_like(x)
    for seg in segments:
        kind, s, L, F, Hh, Ww = _seg_fields(seg)
        if L == 0:
            continue
        xs = x[:, s:s + L, :]
        if kind == TEXT:
            xp = np.concatenate([np.zeros((B, 3, C)), xs], axis=1)
            acc = np.zeros((B, L, C))
            for j in range(N_TEXT_TAPS):
                acc += wt[:, j] * xp[:, j:j + L, :]
            y[:, s:s + L, :] = acc
            continue
        g = xs.reshape(B, F, Hh, Ww, C)
        gp = np.pad(g, ((0, 0), (2, 0), (1, 1), (1, 1), (0, 0)))
        acc = np.zeros((B, F, Hh, Ww, C))
        for kt in range(3):
            for kh in range(3):
                for kw in range(3):
                    acc += wv[:, kt * 9 + kh * 3 + kw] * gp[:, kt:kt + F, kh:kh + Hh, kw:kw + Ww, :]
        y[:, s:s + L, :] = acc.reshape(B, L, C)
    return y


def conv_gather_ref(x: np.ndarray, w_text: np.ndarray, w_vis: np.ndarray, segments,
                    idx: np.ndarray | None = None) -> np.ndarray:
    """The same convolution as a gather: y[p, c] = sum_j w[c, j] * x[idx[p, j], c].

    ``idx`` defaults to ``neighbours_ref``. Rows of text segments take weights
    from w_text (taps 0..3), rows of visual segments from w_vis.
    """
    x = np.asarray(x, dtype=np.float64)
    B, T, C = x.shape
    if idx is None:
        idx = neighbours_ref(segments, T)
    is_text = np.zeros(T, dtype=bool)
    for seg in segments:
        kind, s, L, _, _, _ = _seg_fields(seg)
        if kind == TEXT:
            is_text[s:s + L] = True
    y = np.zeros_like(x)
    wt = np.asarray(w_text, dtype=np.float64)
    wv = np.asarray(w_vis, dtype=np.float64)
    for j in range(N_VIS_TAPS):
        src = idx[:, j]
        ok = src >= 0
        for rows_mask, w_col in ((ok & is_text, wt[:, j] if j < N_TEXT_TAPS else None),
                                 (ok & ~is_text, wv[:, j])):
            rows = np.nonzero(rows_mask)[0]
            if rows.size == 0:
                continue
            assert w_col is not None, "a text row reads a tap beyond the text kernel"
            y[:, rows, :] += w_col * x[:, src[rows], :]
    return y
