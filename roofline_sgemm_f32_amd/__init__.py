"""MI355X (gfx950) single-precision dense matrix multiply, C = A * B.

The compute path is a C-ABI shared library of hand-written HIP kernels
(``libsgemm.so``, declared in ``include/sgemm.h``); ``binding`` is a thin
ctypes layer over it.  Importing the package does not load the library; the
first call does, and raises if it is missing.
"""
from .binding import (EXPORTS, MAX_SPLITS, OP_N, OP_T, STATIC_SCRATCH_BYTES, STATUS, VARIANTS,
                      SgemmError, copy_f32, copy_f32_launch, library_path, load, plan_config,
                      probe_mfma, probe_valu, sgemm, sgemm_colmajor, sgemm_ex, sgemm_f32,
                      sgemm_f32_variant, split_plan, status_string, variant_name, VALU_CHAINS)

__all__ = ["EXPORTS", "MAX_SPLITS", "OP_N", "OP_T", "STATIC_SCRATCH_BYTES", "STATUS", "VARIANTS",
           "SgemmError", "copy_f32", "copy_f32_launch", "library_path", "load", "plan_config",
           "probe_mfma", "probe_valu", "sgemm", "sgemm_colmajor", "sgemm_ex", "sgemm_f32",
           "sgemm_f32_variant", "split_plan", "status_string", "variant_name", "VALU_CHAINS"]
