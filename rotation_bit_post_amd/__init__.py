"""ReSpinQuant's online path on AMD Instinct MI355X (gfx950).

The compute lives in ``librsq.so`` (hand-written HIP kernels behind a C ABI,
``include/rsq.h``); this package holds the ctypes binding (``_binding``), the
build script (``build``), the offline site conversion (``offline``) and the
decoder-layer linear path built from the entry points (``path``).
Importing it fails if the library has not been built.
"""
from ._binding import (  # noqa: F401
    LIB, LIB_PATH, EXPORTS, RsqError,
    RSQ_F32, RSQ_BF16, RSQ_QA_RMSNORM, RSQ_MAX_RANK, RSQ_FP4,
    rsq_version, rsq_packed_row_bytes, rsq_site_bytes, rsq_site_prepare,
    rsq_qgemm_workspace_bytes, rsq_correct_workspace_bytes, rsq_layer_workspace_bytes, rsq_workspace,
    rsq_subspace_correct, rsq_quant_act, rsq_correct_quant, rsq_qgemm, rsq_qgemm_residual, rsq_layer_fused,
    rsq_codes_to_fp4, rsq_qgemm_fp4, rsq_rotate_weight, RSQ_ROTATE_RIGHT, RSQ_ROTATE_LEFT,
)
