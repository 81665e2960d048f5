"""timestep_adaptive_bit_amd: the timestep-adaptive-bit quantized linear on MI355X.

The compute lives in libtabit.so (hand-written HIP for gfx950, C ABI in
include/tabit.h); this package is its thin Python binding.  Importing the
package does not load the library; the first Context() or call does, and
raises if the library has not been built.
"""
from ._lib import (  # noqa: F401
    Context, Layer, TabitError, load, version, act_workspace_bytes, gemm_config_info,
    gemm_config_choose, mxfp4_config_info, mxfp4_config_choose, plane_config_info,
    plane_config_choose,
    weight_planes_bytes,
    dmpq_workspace_bytes, noalloc_scratch_bytes,
    header_functions, LIB_PATH,
    OK, EINVAL, ESHAPE, EALIGN, ERANGE, ENOSCHED, EHIP, ENOMEM,
    FMT_INT8, FMT_MXFP4, PATH_MASKED, PATH_BITSERIAL, PATH_PLANES, PATH_HQDM, PATH_MXFP4_GEMM,
    OPT_GEMM_CONFIG, OPT_MXFP4_CONFIG, OPT_PLANE_CONFIG, OPT_HQDM_CONFIG, hqdm_config_info,
    ACT_NONE, ACT_GELU,
)

__all__ = [
    "Context", "TabitError", "load", "version", "act_workspace_bytes", "gemm_config_info",
    "gemm_config_choose", "header_functions", "FMT_INT8", "FMT_MXFP4", "PATH_MASKED",
    "PATH_BITSERIAL", "PATH_PLANES", "OPT_GEMM_CONFIG", "OPT_MXFP4_CONFIG", "OPT_PLANE_CONFIG",
    "plane_config_info", "plane_config_choose", "weight_planes_bytes", "dmpq_workspace_bytes",
    "mxfp4_config_choose",
    "PATH_HQDM", "OPT_HQDM_CONFIG", "hqdm_config_info", "noalloc_scratch_bytes",
    "ACT_NONE", "ACT_GELU",
]
