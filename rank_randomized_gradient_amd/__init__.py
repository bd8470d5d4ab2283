"""Randomized low-rank gradient sketching on MI355X (gfx950).

The hot path of a linear layer W (d x k) trained from a rank-r sketch of its
gradient, as hand-written HIP kernels behind the C ABI in include/rgc.h:
projection sampling, XP = X P, C += D^T (X P), and the normalized update
with stochastic rounding to bf16. `rgc` is the thin ctypes binding;
`sketched_linear` wraps a bf16 linear layer whose backward feeds the sketch.
"""
from .rgc import (  # noqa: F401
    RgcError,
    Workspace,
    abi_version,
    load_library,
    rgc_accumulate,
    rgc_accumulate_batch,
    rgc_accumulate_batch_deferred,
    rgc_apply,
    rgc_apply_batch,
    rgc_apply_carried,
    rgc_apply_carried_batch,
    rgc_apply_from_seed,
    rgc_apply_scaled,
    rgc_apply_scaled_batch,
    rgc_project,
    rgc_project_batch,
    rgc_project_shared,
    rgc_linear_forward,
    rgc_linear_forward_batch,
    rgc_linear_backward,
    rgc_sample_projection,
    rgc_sample_projections,
    rgc_test_philox,
    rgc_test_reconstruct,
    rgc_test_stochastic_round,
)
from .sketched_linear import SketchedLinear, SketchedLinearFunction  # noqa: F401,E402
