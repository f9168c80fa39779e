"""CPU oracle for the mShortConv + KDA forward (fp64, numpy).

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here. The
HIP library never does: it shares no code, header, table or helper with this
package, and this package imports nothing from it.

Each function is the plain definition of one step, written from the Chimera
pages (arXiv 2607.28611):

* ``neighbours_ref``  -- which packed position every conv tap reads
  (page 1, section 3.3, Eq. 12 raster order; section 3.4 per-segment views).
* ``conv_ref``        -- the modality-aware short convolution on q, k, v
  (page 1, section 3.3, Eq. 13; section 3.4; page 2, the mShortConv paragraph).
* ``conv_gather_ref`` -- the same convolution written as a gather through
  ``neighbours_ref`` (a second formulation, used to pin the first).
* ``l2norm_ref``      -- per-(token, head) L2 normalisation of q and k after the
  conv (page 1, Fig. 2, the "L2" boxes between mShortConv and the recurrence).
* ``kda_ref``         -- the token-by-token gated delta rule, Eq. 14 with the
  parenthesisation of page 2's LaTeX, and the inner readout S_t^T q_t of
  Eq. 15 (page 1, section 3.3).
* ``kda_varlen_ref``  -- several samples packed in one row, the state restarting at
  every sample boundary (page 1, section 3.3).
* ``gated_rmsnorm_ref`` -- Sigmoid(gate) times the per-head RMSNorm of the
  readout, the rest of Eq. 15 before the output projection (page 1, section 3.3).
* ``backward``        -- gradients of the conv and of the recurrence (with the L2
  normalisation), as torch fp64 autograd of the same definitions
  (``conv_backward_ref``, ``kda_backward_ref``); import ``oracle.backward``.
* ``round_bf16_ref``  -- rounding to the bf16 output dtype (round to nearest,
  ties to even), used where a path stores a bf16 intermediate.

Every function here is pinned by ``-m "not gpu"`` tests against hand-derived
fixtures, closed forms, library routines or brute force; see ``tests/``.
"""
from .mshortconv import neighbours_ref, conv_ref, conv_gather_ref, TEXT, IMAGE, VIDEO
from .kda import l2norm_ref, kda_ref, kda_varlen_ref, gated_rmsnorm_ref
from .rounding import round_bf16_ref

__all__ = [
    "neighbours_ref", "conv_ref", "conv_gather_ref", "l2norm_ref", "kda_ref", "kda_varlen_ref", "gated_rmsnorm_ref",
    "round_bf16_ref", "TEXT", "IMAGE", "VIDEO",
]
