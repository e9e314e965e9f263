"""MI355X (gfx950) Muon optimizer step: Python binding of libmuon.

The binding only marshals arguments: every step of the optimizer runs in the
HIP kernels of ``libmuon.so`` (built from ``csrc/`` by ``build.py``).  There
is no fallback: if the library is missing, :func:`load` raises.

Names follow the C ABI in ``include/muon.h``:

* :func:`muon_init` / :func:`muon_destroy`
* :func:`muon_workspace_size`
* :func:`muon_step_batched`
* :func:`adamw_step`

plus helpers that build the C descriptors from PyTorch tensors
(:func:`muon_matrix`, :func:`muon_hparams`, :func:`adamw_tensor`,
:func:`adamw_hparams`).
"""

from ._lib import (  # noqa: F401
    LIB_PATH,
    MUON_BF16,
    MUON_F32,
    SCALE_MODES,
    MuonError,
    AdamwHparams,
    AdamwTensor,
    MuonHparams,
    MuonMatrix,
    adamw_hparams,
    adamw_step,
    adamw_step_clipped,
    adamw_step_clipped_noalloc,
    adamw_workspace_size,
    adamw_tensor,
    exported_symbols,
    load,
    muon_destroy,
    muon_hparams,
    muon_init,
    muon_matrix,
    muon_profile_collect,
    muon_profile_enable,
    PhaseTimes,
    PHASES,
    muon_step_batched,
    muon_test_gram_bf16,
    muon_test_poly_bf16,
    muon_test_update_bf16,
    muon_test_split_matrices,
    muon_workspace_size,
)
from .route import route_parameters  # noqa: F401
