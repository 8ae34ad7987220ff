"""libmuon: the Muon optimizer step's hot path (momentum, batched Newton-Schulz,
apply) as hand-written HIP kernels for AMD Instinct MI355X (gfx950).

The C ABI is include/muon.h; this package is its thin binding.  The shared
library is loaded on first use and its absence raises an error.
"""
from .api import (  # noqa: F401
    Context, MuonError, Plan, minimax_coeffs, newton_schulz_noalloc, ns_params, ns_workspace_bytes,
    workspace_bytes,
)
from .muon_step import MuonStep  # noqa: F401
from . import _lib  # noqa: F401
