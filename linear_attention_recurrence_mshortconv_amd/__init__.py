"""KDA + mShortConv forward for AMD MI355X (gfx950).

The modality-aware short convolution and the Kimi Delta Attention recurrence
of the Chimera backbone (arXiv 2607.28611, page 1, sections 3.3-3.4), as a
C-ABI HIP library (``include/chimera_mshortconv.h``) with a thin ctypes
binding. Build with ``python -m linear_attention_recurrence_mshortconv_amd.build``.
"""
from ._lib import (  # noqa: F401
    BF16, F32, KDA_L2NORM_QK, KDA_NO_SPLIT, KDA_NOALLOC_SCRATCH_BYTES, KDA_SEQUENTIAL, ChimeraError, LIB_PATH, Marks, SegmentStruct,
    gate_norm_bwd, kda_bwd, kda_bwd_varlen, kda_conv_workspace_size, kda_fwd, kda_fwd_conv, kda_fwd_varlen, kda_varlen_workspace_size, kda_workspace_size, lib,
    mshortconv_bwd, mshortconv_fwd, mshortconv_index, mshortconv_index_device, segment_array, split_qkv,
    status_string,
)
