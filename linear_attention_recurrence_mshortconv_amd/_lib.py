"""ctypes binding of ``libchimera_mshortconv.so`` (argument marshalling only).

Each function here has the name of the C entry point it calls without the
``chimera_`` prefix. torch tensors supply device memory and the current HIP
stream; every step of the computation runs in the library's kernels. If the
library is not built this raises instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libchimera_mshortconv.so")

F32, BF16 = 0, 1
KDA_L2NORM_QK = 1
KDA_SEQUENTIAL = 2
KDA_NO_SPLIT = 4
KDA_NOALLOC_SCRATCH_BYTES = 128 << 20   # CHIMERA_KDA_NOALLOC_SCRATCH_BYTES
TEXT_TAPS, VIS_TAPS = 4, 27

STATUS = {0: "ok", 1: "null pointer", 2: "bad shape", 3: "bad dtype", 4: "bad segments",
          5: "unsupported", 6: "workspace", 7: "hip error"}


class ChimeraError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} returned {status} ({msg})")
        self.status = status


class SegmentStruct(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("frames", ctypes.c_int32), ("height", ctypes.c_int32),
                ("width", ctypes.c_int32), ("start", ctypes.c_int64), ("length", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m linear_attention_recurrence_mshortconv_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, u32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
    seg_p = ctypes.POINTER(SegmentStruct)
    L.chimera_status_string.restype = ctypes.c_char_p
    L.chimera_status_string.argtypes = [ctypes.c_int]
    L.chimera_mshortconv_index.restype = ctypes.c_int
    L.chimera_mshortconv_index.argtypes = [seg_p, i32, i64, vp]
    L.chimera_mshortconv_index_device.restype = ctypes.c_int
    L.chimera_mshortconv_index_device.argtypes = [seg_p, i32, i64, vp, vp]
    L.chimera_mshortconv_fwd.restype = ctypes.c_int
    L.chimera_mshortconv_fwd.argtypes = [vp, vp, i64, i64, i64, ctypes.c_int, vp, vp, seg_p, i32, vp]
    L.chimera_kda_workspace_size.restype = sz
    L.chimera_kda_workspace_size.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, u32]
    L.chimera_kda_fwd.restype = ctypes.c_int
    L.chimera_kda_fwd.argtypes = [vp, vp, vp, i64, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                  ctypes.c_int, u32, vp, sz, vp]
    pp, cp = ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_char_p)
    L.chimera_mshortconv_fwd_timed.restype = ctypes.c_int
    L.chimera_mshortconv_fwd_timed.argtypes = L.chimera_mshortconv_fwd.argtypes + [pp, cp, i32,
                                                                                     ctypes.POINTER(i32)]
    L.chimera_kda_fwd_timed.restype = ctypes.c_int
    L.chimera_kda_fwd_timed.argtypes = L.chimera_kda_fwd.argtypes + [pp, cp, i32, ctypes.POINTER(i32)]
    L.chimera_kda_fwd_gated.restype = ctypes.c_int
    L.chimera_kda_fwd_gated.argtypes = [vp, vp, vp, i64, vp, vp, vp, vp, i64, vp, ctypes.c_float, vp, vp,
                                        i64, i64, i64, i64, i64, ctypes.c_int, u32, vp, sz, vp]
    L.chimera_kda_fwd_gated_timed.restype = ctypes.c_int
    L.chimera_kda_fwd_gated_timed.argtypes = L.chimera_kda_fwd_gated.argtypes + [pp, cp, i32, ctypes.POINTER(i32)]
    L.chimera_kda_bwd_workspace_size.restype = sz
    L.chimera_kda_bwd_workspace_size.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, u32]
    L.chimera_kda_bwd.restype = ctypes.c_int
    L.chimera_kda_bwd.argtypes = [vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                  i64, i64, i64, i64, i64, ctypes.c_int, u32, vp, sz, vp]
    L.chimera_mshortconv_bwd.restype = ctypes.c_int
    L.chimera_mshortconv_bwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, vp, vp, seg_p, i32, vp]
    L.chimera_kda_varlen_workspace_size.restype = sz
    L.chimera_kda_varlen_workspace_size.argtypes = [vp, i32, i64, i64, i64, ctypes.c_int, u32]
    L.chimera_kda_fwd_varlen.restype = ctypes.c_int
    L.chimera_kda_fwd_varlen.argtypes = [vp, vp, vp, i64, vp, vp, vp, vp, i64, vp, ctypes.c_float, vp, vp,
                                         vp, i32, i64, i64, i64, ctypes.c_int, u32, vp, sz, vp]
    L.chimera_kda_bwd_varlen_workspace_size.restype = sz
    L.chimera_kda_bwd_varlen_workspace_size.argtypes = [vp, i32, i64, i64, i64, ctypes.c_int, u32]
    L.chimera_kda_bwd_varlen.restype = ctypes.c_int
    L.chimera_kda_bwd_varlen.argtypes = [vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                         vp, i32, i64, i64, i64, ctypes.c_int, u32, vp, sz, vp]
    L.chimera_gate_norm_bwd.restype = ctypes.c_int
    L.chimera_gate_norm_bwd.argtypes = [vp, vp, i64, vp, ctypes.c_float, vp, vp, vp, vp, i64, i64, i64, i64,
                                        ctypes.c_int, vp]
    L.chimera_kda_fwd_conv.restype = ctypes.c_int
    L.chimera_kda_fwd_conv.argtypes = [vp, vp, vp, seg_p, i32, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                       ctypes.c_int, u32, vp, sz, vp]
    L.chimera_kda_fwd_conv_timed.restype = ctypes.c_int
    L.chimera_kda_fwd_conv_timed.argtypes = L.chimera_kda_fwd_conv.argtypes + [pp, cp, i32, ctypes.POINTER(i32)]
    L.chimera_kda_conv_workspace_size.restype = sz
    L.chimera_kda_conv_workspace_size.argtypes = [seg_p, i32, i64, i64, i64, i64, i64, ctypes.c_int, u32]
    L.chimera_kda_fwd_noalloc.restype = ctypes.c_int
    L.chimera_kda_fwd_noalloc.argtypes = [vp, vp, vp, i64, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                          ctypes.c_int, u32, vp]
    L.chimera_kda_fwd_varlen_timed.restype = ctypes.c_int
    L.chimera_kda_fwd_varlen_timed.argtypes = L.chimera_kda_fwd_varlen.argtypes + [pp, cp, i32, ctypes.POINTER(i32)]
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().chimera_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise ChimeraError(fn, status, status_string(status))


def segment_array(segments: Sequence) -> "ctypes.Array":
    """Pack segment descriptions (objects with kind/start/length/frames/height/width, or dicts)."""
    arr = (SegmentStruct * max(1, len(segments)))()
    for i, s in enumerate(segments):
        get = (lambda k, d=0: s.get(k, d)) if isinstance(s, dict) else (lambda k, d=0: getattr(s, k, d))
        arr[i].kind = int(get("kind"))
        arr[i].frames = int(get("frames"))
        arr[i].height = int(get("height"))
        arr[i].width = int(get("width"))
        arr[i].start = int(get("start"))
        arr[i].length = int(get("length"))
    return arr


def _stream(t) -> int:
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(cond: bool, msg: str):
    """Argument check of the wrappers: raises before anything reaches the library."""
    if not cond:
        raise ValueError(msg)


def _dense(t, name: str, shape, dtype, device):
    """t must be a dense (contiguous) tensor of this shape and dtype on `device`: the library
    reads it through one pointer with the row-major strides of `shape`."""
    _need(t is not None, f"{name} is required")
    _need(tuple(t.shape) == tuple(shape), f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    _need(t.dtype == dtype, f"{name}: dtype {t.dtype}, expected {dtype}")
    _need(t.device == device, f"{name}: on {t.device}, expected {device}")
    _need(t.is_contiguous(), f"{name} must be contiguous (no expanded or strided views)")


def _opt_dense(t, name: str, shape, dtype, device):
    if t is not None:
        _dense(t, name, shape, dtype, device)


def _on_gpu(t, name: str):
    _need(t.is_cuda, f"{name} must be a GPU tensor: the library runs every step on the device")


def _conv_weights(w_text, w_vis, C: int, device):
    """The conv weights as device fp32 [C][4] and [C][27] (copied when they are not)."""
    import torch
    w_text = w_text.to(device=device, dtype=torch.float32).contiguous()
    w_vis = w_vis.to(device=device, dtype=torch.float32).contiguous()
    _need(tuple(w_text.shape) == (C, TEXT_TAPS), f"w_text: shape {tuple(w_text.shape)}, expected {(C, TEXT_TAPS)}")
    _need(tuple(w_vis.shape) == (C, VIS_TAPS), f"w_vis: shape {tuple(w_vis.shape)}, expected {(C, VIS_TAPS)}")
    return w_text, w_vis


def mshortconv_index(segments: Sequence, T: int) -> np.ndarray:
    """Host neighbour table int32 [T, 27] (chimera_mshortconv_index)."""
    idx = np.empty((max(T, 0), VIS_TAPS), dtype=np.int32)
    segs = segment_array(segments)
    _check("chimera_mshortconv_index",
           lib().chimera_mshortconv_index(segs, len(segments), T, idx.ctypes.data if T > 0 else None))
    return idx


def mshortconv_index_device(segments: Sequence, T: int, device="cuda"):
    """Device neighbour table int32 [T, 27] from the kernels' own arithmetic."""
    import torch
    idx = torch.full((max(T, 0), VIS_TAPS), -7, dtype=torch.int32, device=device)
    segs = segment_array(segments)
    _check("chimera_mshortconv_index_device",
           lib().chimera_mshortconv_index_device(segs, len(segments), T, _ptr(idx) if T > 0 else None, _stream(idx)))
    return idx


class Marks:
    """Timing marks for the *_fwd_timed calls: `capacity` torch.cuda.Events with timing enabled.

    After a call, ``kernels()`` gives (kernel name, milliseconds) for each kernel
    the call launched, read from the events (this synchronises on them).
    """

    def __init__(self, capacity: int, device="cuda"):
        import torch
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(capacity)]
        stream = torch.cuda.current_stream(device)
        for e in self.events:           # torch creates the HIP event on its first record
            e.record(stream)
        self.handles = (ctypes.c_void_p * capacity)(*[e.cuda_event for e in self.events])
        self.names = (ctypes.c_char_p * capacity)()
        self.used = ctypes.c_int32(0)
        self.capacity = capacity

    def kernels(self):
        n = self.used.value
        return [(self.names[i].decode(), self.events[i].elapsed_time(self.events[i + 1])) for i in range(n - 1)]


def mshortconv_fwd(x, w_text, w_vis, segments: Sequence, out=None, marks: Optional[Marks] = None):
    """y = mShortConv(x) for x [B, T, C] (bf16 or fp32) on the GPU (chimera_mshortconv_fwd).

    With `marks`, calls chimera_mshortconv_fwd_timed instead and records them.
    """
    import torch
    _need(x.dim() == 3, "x must be [B, T, C]")
    B, T, C = x.shape
    _dense(x, "x", (B, T, C), x.dtype, x.device)
    _opt_dense(out, "out", (B, T, C), x.dtype, x.device)
    w_text, w_vis = _conv_weights(w_text, w_vis, C, x.device)
    _on_gpu(x, "x")
    y = torch.empty_like(x) if out is None else out
    segs = segment_array(segments)
    args = (_ptr(x), _ptr(y), B, T, C, _dtype_code(x), _ptr(w_text), _ptr(w_vis), segs, len(segments), _stream(x))
    if marks is None:
        _check("chimera_mshortconv_fwd", lib().chimera_mshortconv_fwd(*args))
    else:
        _check("chimera_mshortconv_fwd_timed",
               lib().chimera_mshortconv_fwd_timed(*args, marks.handles, marks.names, marks.capacity,
                                                  ctypes.byref(marks.used)))
    return y


def kda_workspace_size(B, T, H, dk, dv, dtype_code: int, flags: int) -> int:
    return int(lib().chimera_kda_workspace_size(B, T, H, dk, dv, dtype_code, flags))


def _token_view_stride(t, B, T, H, d) -> int:
    """Token stride of a [B, T, H, d] view whose [H, d] block per token is contiguous."""
    _need(tuple(t.shape) == (B, T, H, d), f"shape {tuple(t.shape)}, expected {(B, T, H, d)}")
    s = t.stride()
    if T > 1 or B > 1:
        _need(s[3] == 1 and s[2] == d and (B == 1 or s[0] == T * s[1]) and (T <= 1 or s[1] >= H * d),
              f"strides {s}: each token's [H, d] block must be dense, tokens evenly spaced")
    return s[1] if T > 0 else H * d


def kda_fwd(q, k, v, alpha, beta, S0=None, *, l2norm: bool = True, sequential: bool = False,
            no_split: bool = False, out=None, want_state: bool = True, workspace=None,
            marks: Optional[Marks] = None, state_out=None, gate=None, norm_weight=None,
            norm_eps: float = 1e-6):
    """KDA forward on the GPU (chimera_kda_fwd; chimera_kda_fwd_timed with `marks`).

    q, k [B, T, H, dk], v [B, T, H, dv] with a shared token stride (views into a
    fused q|k|v tensor are accepted), alpha [B, T, H, dk], beta [B, T, H], S0
    fp32 [B, H, dk, dv] or None. Returns (o [B, T, H, dv], S_final or None);
    `out` and `state_out` are written in place when given.

    With `gate` ([B, T, H, dv] in the same dtype, any token stride) the output is
    Sigmoid(gate) * RMSNorm(o) per (token, head), with gain `norm_weight` (fp32
    [dv] or None) and `norm_eps` (chimera_kda_fwd_gated / _gated_timed).
    """
    import torch
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    dev, tdt = k.device, k.dtype
    stride = _token_view_stride(q, B, T, H, dk)
    _need(_token_view_stride(k, B, T, H, dk) == stride and _token_view_stride(v, B, T, H, dv) == stride,
          "q, k, v must share one token stride")
    _need(q.device == dev and v.device == dev and q.dtype == tdt and v.dtype == tdt, "q, k, v: one device and dtype")
    _dense(alpha, "alpha", (B, T, H, dk), tdt, dev)
    _dense(beta, "beta", (B, T, H), tdt, dev)
    _opt_dense(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    _opt_dense(state_out, "state_out", (B, H, dk, dv), torch.float32, dev)
    _opt_dense(out, "out", (B, T, H, dv), tdt, dev)
    _on_gpu(k, "k")
    dt = _dtype_code(k)
    flags = (KDA_L2NORM_QK if l2norm else 0) | (KDA_SEQUENTIAL if sequential else 0) | (KDA_NO_SPLIT if no_split else 0)
    o = torch.empty((B, T, H, dv), dtype=k.dtype, device=k.device) if out is None else out
    Sf = state_out
    if Sf is None and want_state:
        Sf = torch.empty((B, H, dk, dv), dtype=torch.float32, device=k.device)
    need = kda_workspace_size(B, T, H, dk, dv, dt, flags)
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=k.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    tail = (B, T, H, dk, dv, dt, flags, _ptr(workspace), wbytes, _stream(k))
    if gate is not None:
        _need(gate.dtype == tdt and gate.device == dev, "gate: the dtype and device of q, k, v")
        gstride = _token_view_stride(gate, B, T, H, dv)
        _opt_dense(norm_weight, "norm_weight", (dv,), torch.float32, dev)
        args = (_ptr(q), _ptr(k), _ptr(v), stride, _ptr(alpha), _ptr(beta), _ptr(S0), _ptr(gate), gstride,
                _ptr(norm_weight), float(norm_eps), _ptr(o), _ptr(Sf)) + tail
        if marks is None:
            _check("chimera_kda_fwd_gated", lib().chimera_kda_fwd_gated(*args))
        else:
            _check("chimera_kda_fwd_gated_timed",
                   lib().chimera_kda_fwd_gated_timed(*args, marks.handles, marks.names, marks.capacity,
                                                     ctypes.byref(marks.used)))
        return o, Sf
    args = (_ptr(q), _ptr(k), _ptr(v), stride, _ptr(alpha), _ptr(beta), _ptr(S0), _ptr(o), _ptr(Sf)) + tail
    if marks is None:
        _check("chimera_kda_fwd", lib().chimera_kda_fwd(*args))
    else:
        _check("chimera_kda_fwd_timed",
               lib().chimera_kda_fwd_timed(*args, marks.handles, marks.names, marks.capacity,
                                           ctypes.byref(marks.used)))
    return o, Sf


def _cu_array(cu_seqlens) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))


def kda_varlen_workspace_size(cu_seqlens, H, dk, dv, dtype_code: int, flags: int) -> int:
    cu = _cu_array(cu_seqlens)
    return int(lib().chimera_kda_varlen_workspace_size(cu.ctypes.data, len(cu) - 1, H, dk, dv, dtype_code, flags))


def kda_fwd_varlen(q, k, v, alpha, beta, cu_seqlens, S0=None, *, l2norm: bool = True, sequential: bool = False,
                   no_split: bool = False, out=None, want_state: bool = True, workspace=None,
                   marks: Optional[Marks] = None, state_out=None, gate=None, norm_weight=None,
                   norm_eps: float = 1e-6):
    """KDA forward over samples packed in one row (chimera_kda_fwd_varlen; _timed with `marks`).

    q, k [T, H, dk], v [T, H, dv] (a shared token stride; views into a fused q|k|v
    tensor are accepted), alpha [T, H, dk], beta [T, H]; `cu_seqlens` the N + 1 sample
    offsets (host sequence, 0 first, nondecreasing, T last). The state restarts at every
    sample start, from S0[n] (fp32 [N, H, dk, dv]) or zero. Returns (o [T, H, dv],
    S_final [N, H, dk, dv] or None). `gate`, `norm_weight`, `norm_eps` as in kda_fwd.
    """
    import torch
    T, H, dk = k.shape
    dv = v.shape[-1]
    dev, tdt = k.device, k.dtype
    cu = _cu_array(cu_seqlens)
    N = len(cu) - 1
    _need(N >= 0 and cu[0] == 0 and cu[-1] == T and bool(np.all(np.diff(cu) >= 0)),
          "cu_seqlens: 0 first, nondecreasing, T last")
    stride = _token_view_stride(q.unsqueeze(0), 1, T, H, dk)
    _need(_token_view_stride(k.unsqueeze(0), 1, T, H, dk) == stride and
          _token_view_stride(v.unsqueeze(0), 1, T, H, dv) == stride, "q, k, v must share one token stride")
    _need(q.device == dev and v.device == dev and q.dtype == tdt and v.dtype == tdt, "q, k, v: one device and dtype")
    _dense(alpha, "alpha", (T, H, dk), tdt, dev)
    _dense(beta, "beta", (T, H), tdt, dev)
    _opt_dense(S0, "S0", (N, H, dk, dv), torch.float32, dev)
    _opt_dense(state_out, "state_out", (N, H, dk, dv), torch.float32, dev)
    _opt_dense(out, "out", (T, H, dv), tdt, dev)
    _on_gpu(k, "k")
    dt = _dtype_code(k)
    flags = (KDA_L2NORM_QK if l2norm else 0) | (KDA_SEQUENTIAL if sequential else 0) | (KDA_NO_SPLIT if no_split else 0)
    o = torch.empty((T, H, dv), dtype=k.dtype, device=k.device) if out is None else out
    Sf = state_out
    if Sf is None and want_state:
        Sf = torch.empty((N, H, dk, dv), dtype=torch.float32, device=k.device)
    need = kda_varlen_workspace_size(cu, H, dk, dv, dt, flags)
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=k.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    gstride = 0
    if gate is not None:
        _need(gate.dtype == tdt and gate.device == dev, "gate: the dtype and device of q, k, v")
        gstride = _token_view_stride(gate.unsqueeze(0), 1, T, H, dv)
        _opt_dense(norm_weight, "norm_weight", (dv,), torch.float32, dev)
    args = (_ptr(q), _ptr(k), _ptr(v), stride, _ptr(alpha), _ptr(beta), _ptr(S0), _ptr(gate), gstride,
            _ptr(norm_weight), float(norm_eps), _ptr(o), _ptr(Sf), cu.ctypes.data, N, H, dk, dv, dt, flags,
            _ptr(workspace), wbytes, _stream(k))
    if marks is None:
        _check("chimera_kda_fwd_varlen", lib().chimera_kda_fwd_varlen(*args))
    else:
        _check("chimera_kda_fwd_varlen_timed",
               lib().chimera_kda_fwd_varlen_timed(*args, marks.handles, marks.names, marks.capacity,
                                                  ctypes.byref(marks.used)))
    return o, Sf


def kda_bwd(q, k, v, alpha, beta, S0, dout, dS_final=None, *, l2norm: bool = True, grads=None, workspace=None,
            sequential: bool = False):
    """Gradients of kda_fwd (chimera_kda_bwd). Inputs as for kda_fwd; dout [B, T, H, dv]
    (input dtype), dS_final fp32 [B, H, dk, dv] or None. `grads` = (dq, dk, dv) tensors with
    the layout of q, k, v (views into one fused gradient are accepted), else fresh tensors.
    sequential: the token-by-token kernels also for bf16 heads of 128 (CHIMERA_KDA_SEQUENTIAL).
    Returns dict dq, dk, dv, dalpha, dbeta, dS0."""
    import torch
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    dev, tdt = k.device, k.dtype
    stride = _token_view_stride(q, B, T, H, dk)
    _need(_token_view_stride(k, B, T, H, dk) == stride and _token_view_stride(v, B, T, H, dv) == stride,
          "q, k, v must share one token stride")
    _need(q.device == dev and v.device == dev and q.dtype == tdt and v.dtype == tdt, "q, k, v: one device and dtype")
    _dense(alpha, "alpha", (B, T, H, dk), tdt, dev)
    _dense(beta, "beta", (B, T, H), tdt, dev)
    _dense(dout, "dout", (B, T, H, dv), tdt, dev)
    _opt_dense(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    _opt_dense(dS_final, "dS_final", (B, H, dk, dv), torch.float32, dev)
    _on_gpu(k, "k")
    dt = _dtype_code(k)
    if grads is None:
        _need(stride == H * dk and stride == H * dv, "strided (fused) inputs: pass `grads` with their layout")
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dkk, dvv = grads
    for g, t in zip(grads, (q, k, v)):
        _need(g.shape == t.shape and g.stride() == t.stride() and g.dtype == tdt and g.device == dev,
              "grads must have the layout, dtype and device of q, k, v")
    dalpha = torch.empty_like(alpha)
    dbeta = torch.empty_like(beta)
    dS0 = torch.empty((B, H, dk, dv), dtype=torch.float32, device=k.device)
    flags = (KDA_L2NORM_QK if l2norm else 0) | (KDA_SEQUENTIAL if sequential else 0)
    need = int(lib().chimera_kda_bwd_workspace_size(B, T, H, dk, dv, dt, flags))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=k.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("chimera_kda_bwd", lib().chimera_kda_bwd(
        _ptr(q), _ptr(k), _ptr(v), stride, _ptr(alpha), _ptr(beta), _ptr(S0), _ptr(dout), _ptr(dS_final),
        _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dalpha), _ptr(dbeta), _ptr(dS0), B, T, H, dk, dv, dt,
        flags, _ptr(workspace), wbytes, _stream(k)))
    return {"dq": dq, "dk": dkk, "dv": dvv, "dalpha": dalpha, "dbeta": dbeta, "dS0": dS0}


def kda_bwd_varlen(q, k, v, alpha, beta, cu_seqlens, S0, dout, dS_final=None, *, l2norm: bool = True, grads=None,
                   workspace=None, sequential: bool = False):
    """Gradients of kda_fwd_varlen without a gate (chimera_kda_bwd_varlen): q, k, v [T, H, d] (views
    into one packed row), cu_seqlens the sample offsets; S0, dS_final, and the returned dS0 are
    [nseq, H, dk, dv] fp32. Returns dict dq, dk, dv, dalpha, dbeta, dS0."""
    import torch
    T, H, dk = k.shape
    dv = v.shape[-1]
    dev, tdt = k.device, k.dtype
    stride = _token_view_stride(q[None], 1, T, H, dk)
    _need(_token_view_stride(k[None], 1, T, H, dk) == stride and _token_view_stride(v[None], 1, T, H, dv) == stride,
          "q, k, v must share one token stride")
    _need(q.device == dev and v.device == dev and q.dtype == tdt and v.dtype == tdt, "q, k, v: one device and dtype")
    cu = _cu_array(cu_seqlens)
    nseq = len(cu) - 1
    _need(nseq >= 0 and cu[0] == 0 and cu[-1] == T and bool(np.all(np.diff(cu) >= 0)),
          "cu_seqlens: 0 first, nondecreasing, T last")
    _dense(alpha, "alpha", (T, H, dk), tdt, dev)
    _dense(beta, "beta", (T, H), tdt, dev)
    _dense(dout, "dout", (T, H, dv), tdt, dev)
    _opt_dense(S0, "S0", (nseq, H, dk, dv), torch.float32, dev)
    _opt_dense(dS_final, "dS_final", (nseq, H, dk, dv), torch.float32, dev)
    _on_gpu(k, "k")
    dt = _dtype_code(k)
    if grads is None:
        _need(stride == H * dk and stride == H * dv, "strided (fused) inputs: pass `grads` with their layout")
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dkk, dvv = grads
    for g, t in zip(grads, (q, k, v)):
        _need(g.shape == t.shape and g.stride() == t.stride() and g.dtype == tdt and g.device == dev,
              "grads must have the layout, dtype and device of q, k, v")
    dalpha = torch.empty_like(alpha)
    dbeta = torch.empty_like(beta)
    dS0 = torch.empty((nseq, H, dk, dv), dtype=torch.float32, device=k.device)
    flags = (KDA_L2NORM_QK if l2norm else 0) | (KDA_SEQUENTIAL if sequential else 0)
    need = int(lib().chimera_kda_bwd_varlen_workspace_size(cu.ctypes.data, nseq, H, dk, dv, dt, flags))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=k.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("chimera_kda_bwd_varlen", lib().chimera_kda_bwd_varlen(
        _ptr(q), _ptr(k), _ptr(v), stride, _ptr(alpha), _ptr(beta), _ptr(S0), _ptr(dout), _ptr(dS_final),
        _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dalpha), _ptr(dbeta), _ptr(dS0), cu.ctypes.data, nseq, H, dk, dv, dt,
        flags, _ptr(workspace), wbytes, _stream(k)))
    return {"dq": dq, "dk": dkk, "dv": dvv, "dalpha": dalpha, "dbeta": dbeta, "dS0": dS0}


def gate_norm_bwd(o, gate, norm_weight, dy, norm_eps: float = 1e-6, *, want_weight_grad: bool = True):
    """Gradients of Sigmoid(gate) * RMSNorm(o) * norm_weight (chimera_gate_norm_bwd): o, dy
    [B, T, H, dv]; gate [B, T, H, dv] with a token stride of its own. Returns (dout, dgate,
    dnorm_weight or None)."""
    import torch
    _need(o.dim() == 4, "o must be [B, T, H, dv]")
    B, T, H, dv = o.shape
    dev, tdt = o.device, o.dtype
    _dense(o, "o", (B, T, H, dv), tdt, dev)
    _dense(dy, "dy", (B, T, H, dv), tdt, dev)
    _need(gate.dtype == tdt and gate.device == dev, "gate: the dtype and device of o")
    gs = _token_view_stride(gate, B, T, H, dv)
    _opt_dense(norm_weight, "norm_weight", (dv,), torch.float32, dev)
    _on_gpu(o, "o")
    dout = torch.empty_like(o)
    dgate = torch.empty_strided(gate.shape, gate.stride(), dtype=gate.dtype, device=gate.device)
    dw = torch.empty(dv, dtype=torch.float32, device=o.device) if want_weight_grad else None
    _check("chimera_gate_norm_bwd", lib().chimera_gate_norm_bwd(
        _ptr(o), _ptr(gate), gs, _ptr(norm_weight), float(norm_eps), _ptr(dy), _ptr(dout), _ptr(dgate), _ptr(dw),
        B, T, H, dv, _dtype_code(o), _stream(o)))
    return dout, dgate, dw


def mshortconv_bwd(x, dy, w_text, w_vis, segments: Sequence, dx=None):
    """Gradients of mshortconv_fwd (chimera_mshortconv_bwd): returns (dx, dw_text, dw_vis)."""
    import torch
    _need(x.dim() == 3, "x must be [B, T, C]")
    B, T, C = x.shape
    _dense(x, "x", (B, T, C), x.dtype, x.device)
    _dense(dy, "dy", (B, T, C), x.dtype, x.device)
    _opt_dense(dx, "dx", (B, T, C), x.dtype, x.device)
    w_text, w_vis = _conv_weights(w_text, w_vis, C, x.device)
    _on_gpu(x, "x")
    dx = torch.empty_like(x) if dx is None else dx
    dwt = torch.empty((C, TEXT_TAPS), dtype=torch.float32, device=x.device)
    dwv = torch.empty((C, VIS_TAPS), dtype=torch.float32, device=x.device)
    segs = segment_array(segments)
    _check("chimera_mshortconv_bwd", lib().chimera_mshortconv_bwd(
        _ptr(x), _ptr(dy), _ptr(dx), _ptr(dwt), _ptr(dwv), B, T, C, _dtype_code(x), _ptr(w_text), _ptr(w_vis),
        segs, len(segments), _stream(x)))
    return dx, dwt, dwv


def kda_conv_workspace_size(segments: Sequence, B: int, T: int, H: int, dk: int, dv: int, dtype_code: int,
                            flags: int) -> int:
    arr = segment_array(segments)
    return int(lib().chimera_kda_conv_workspace_size(arr, len(segments), B, T, H, dk, dv, dtype_code, flags))


def kda_fwd_conv(x, w_text, w_vis, segments: Sequence, alpha, beta, S0=None, *, H: int, dk: int, dv: int,
                 l2norm: bool = True, sequential: bool = False, no_split: bool = False, out=None,
                 state_out=None, want_state: bool = True, workspace=None, marks: Optional[Marks] = None):
    """mShortConv and KDA in one pass (chimera_kda_fwd_conv; chimera_kda_fwd_conv_timed with
    `marks`): x [B, T, H*(2 dk + dv)] holds the pre-conv q|k|v channels; returns
    (o [B, T, H, dv], S_final or None)."""
    import torch
    _need(x.dim() == 3, "x must be [B, T, C]")
    B, T, C = x.shape
    dev, tdt = x.device, x.dtype
    _need(C == H * (2 * dk + dv), f"x has {C} channels, expected H * (2 dk + dv) = {H * (2 * dk + dv)}")
    _dense(x, "x", (B, T, C), tdt, dev)
    _dense(alpha, "alpha", (B, T, H, dk), tdt, dev)
    _dense(beta, "beta", (B, T, H), tdt, dev)
    _opt_dense(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    _opt_dense(out, "out", (B, T, H, dv), tdt, dev)
    _opt_dense(state_out, "state_out", (B, H, dk, dv), torch.float32, dev)
    w_text, w_vis = _conv_weights(w_text, w_vis, C, dev)
    _on_gpu(x, "x")
    dt = _dtype_code(x)
    flags = (KDA_L2NORM_QK if l2norm else 0) | (KDA_SEQUENTIAL if sequential else 0) | (KDA_NO_SPLIT if no_split else 0)
    o = out if out is not None else torch.empty((B, T, H, dv), dtype=x.dtype, device=x.device)
    Sf = state_out if state_out is not None else (
        torch.empty((B, H, dk, dv), dtype=torch.float32, device=x.device) if want_state else None)
    arr = segment_array(segments)
    need = int(lib().chimera_kda_conv_workspace_size(arr, len(segments), B, T, H, dk, dv, dt, flags))
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(x), _ptr(w_text), _ptr(w_vis), arr, len(segments), _ptr(alpha), _ptr(beta), _ptr(S0), _ptr(o),
            _ptr(Sf), B, T, H, dk, dv, dt, flags, _ptr(workspace), wbytes, _stream(x))
    if marks is None:
        _check("chimera_kda_fwd_conv", lib().chimera_kda_fwd_conv(*args))
    else:
        _check("chimera_kda_fwd_conv_timed",
               lib().chimera_kda_fwd_conv_timed(*args, marks.handles, marks.names, marks.capacity,
                                                ctypes.byref(marks.used)))
    return o, Sf


def split_qkv(y, H: int, d: int):
    """Views q, k, v [B, T, H, d] into a fused [B, T, 3*H*d] conv output (no copy)."""
    B, T, C = y.shape
    _need(C == 3 * H * d, f"y has {C} channels, expected 3 * H * d = {3 * H * d}")
    parts = y.view(B, T, 3, H, d)
    return parts[:, :, 0], parts[:, :, 1], parts[:, :, 2]
