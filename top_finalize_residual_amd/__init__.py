"""MI355X-native fused MoE finalize + residual add + RMSNorm.

The op (vLLM pull request #62174, Details): for each token, the weighted sum
of its K routed-expert GEMM2 rows gathered through a permutation map, times
the routed scaling factor, plus the shared-expert output and the residual,
rounded once to bf16 for the new residual stream, then RMSNorm with gamma and
eps. Also the same tail with no routed part (residual_add_rmsnorm), and both
with the normalised output as dynamic per-token FP8 (the _fp8 forms). All are
hand-written HIP kernels for gfx950 behind a C ABI
(include/moe_finalize_rmsnorm.h); this package is the thin Python binding.
"""
from .binding import (  # noqa: F401
    MFRError,
    PATH_PERSIST,
    PATH_STREAM,
    PATH_TOKEN,
    PATH_UNSUPPORTED,
    moe_finalize_rmsnorm,
    moe_finalize_rmsnorm_checked,
    moe_finalize_rmsnorm_checked_raw,
    moe_finalize_rmsnorm_fp8,
    moe_finalize_rmsnorm_fp8_checked,
    moe_finalize_rmsnorm_fp8_checked_raw,
    moe_finalize_rmsnorm_fp8_raw,
    moe_finalize_rmsnorm_path,
    moe_finalize_rmsnorm_raw,
    residual_add_rmsnorm,
    residual_add_rmsnorm_fp8,
    residual_add_rmsnorm_fp8_raw,
    residual_add_rmsnorm_raw,
    strerror,
)
from .deferred import (  # noqa: F401,E402
    MoEOutput,
    UnfinalizedMoEOutput,
    defer_moe_finalize,
    fused_add_rmsnorm,
)
