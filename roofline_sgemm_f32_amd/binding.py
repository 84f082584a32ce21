"""ctypes binding over libsgemm.so (declared in include/sgemm.h).

Argument marshalling only: every step of the product runs in the library's
HIP kernels.  PyTorch supplies device memory and the stream.  If the library
has not been built, the first call raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "libsgemm.so")
_lib = None

# sgemm_variant_t
VARIANTS = {
    "auto": 0,
    "k1_coalesced": 1,
    "k2_lds_tiled32": 2,
    "k3_regtile_db": 3,
    "k4_mfma": 4,
    "k2_lds_tiled16": 5,
    "k2_lds_tiled32_pad1": 6,
    "k0_naive": 7,
    "k2_lds_tiled16_pad1": 8,
    "k4_mfma_tile128": 9,
    "k4_mfma_tile64": 10,
    "k4_mfma_tile128x256": 11,
}

# sgemm_status_t
STATUS = {
    0: "SGEMM_OK", 1: "SGEMM_ERR_DIM", 2: "SGEMM_ERR_LD", 3: "SGEMM_ERR_NULLPTR",
    4: "SGEMM_ERR_VARIANT", 5: "SGEMM_ERR_ALIAS", 6: "SGEMM_ERR_LAUNCH",
    7: "SGEMM_ERR_UNSUPPORTED", 8: "SGEMM_ERR_ARG", 9: "SGEMM_ERR_SCRATCH",
}

EXPORTS = ["sgemm_f32", "sgemm_f32_variant", "sgemm_copy_f32", "sgemm_copy_f32_launch",
           "sgemm_status_string", "sgemm_variant_name", "sgemm_auto_variant",
           "sgemm_last_hip_error", "sgemm_abi_version", "sgemm_probe_valu_f32",
           "sgemm_probe_mfma_f32", "sgemm_f32_ex", "sgemm_f32_colmajor", "sgemm_f32_ex_split",
           "sgemm_split_plan", "sgemm_plan_config", "sgemm_f32_ex_split_noalloc"]

MAX_SPLITS = 64
STATIC_SCRATCH_BYTES = 64 * 1024 * 1024  # SGEMM_STATIC_SCRATCH_BYTES

OP_N, OP_T = 0, 1


class SgemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_string(status)})")


def library_path() -> str:
    return _LIB_PATH


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libsgemm.so; raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m roofline_sgemm_f32_amd.build`"
                           " (there is no non-HIP fallback)")
    lib = ctypes.CDLL(p)
    i64, vp, cint = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    gemm = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp]
    lib.sgemm_f32.argtypes = gemm
    lib.sgemm_f32.restype = cint
    lib.sgemm_f32_variant.argtypes = [cint, *gemm]
    lib.sgemm_f32_variant.restype = cint
    f32 = ctypes.c_float
    ex = [cint, cint, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64, vp]
    lib.sgemm_f32_ex.argtypes = ex
    lib.sgemm_f32_ex.restype = cint
    lib.sgemm_f32_colmajor.argtypes = ex
    lib.sgemm_f32_colmajor.restype = cint
    lib.sgemm_f32_ex_split.argtypes = [*ex[:-1], cint, vp]
    lib.sgemm_f32_ex_split.restype = cint
    lib.sgemm_f32_ex_split_noalloc.argtypes = [*ex[:-1], cint, vp]
    lib.sgemm_f32_ex_split_noalloc.restype = cint
    lib.sgemm_split_plan.argtypes = [cint, cint, i64, i64, i64, vp, i64, vp, i64, cint,
                                     ctypes.POINTER(i64)]
    lib.sgemm_split_plan.restype = cint
    ip = ctypes.POINTER(cint)
    lib.sgemm_plan_config.argtypes = [cint, cint, i64, i64, i64, vp, i64, vp, i64, ip, ip, ip, ip,
                                      ip, ctypes.POINTER(i64)]
    lib.sgemm_plan_config.restype = cint
    lib.sgemm_copy_f32.argtypes = [vp, vp, i64, vp]
    lib.sgemm_copy_f32.restype = cint
    lib.sgemm_copy_f32_launch.argtypes = [vp, vp, i64, cint, i64, vp]
    lib.sgemm_copy_f32_launch.restype = cint
    lib.sgemm_status_string.argtypes = [cint]
    lib.sgemm_status_string.restype = ctypes.c_char_p
    lib.sgemm_variant_name.argtypes = [cint]
    lib.sgemm_variant_name.restype = ctypes.c_char_p
    lib.sgemm_auto_variant.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64]
    lib.sgemm_auto_variant.restype = cint
    lib.sgemm_last_hip_error.argtypes = []
    lib.sgemm_last_hip_error.restype = cint
    lib.sgemm_probe_valu_f32.argtypes = [vp, i64, cint, i64, ctypes.c_float, ctypes.c_float, vp]
    lib.sgemm_probe_valu_f32.restype = cint
    lib.sgemm_probe_mfma_f32.argtypes = [vp, vp, vp, i64, i64, vp]
    lib.sgemm_probe_mfma_f32.restype = cint
    lib.sgemm_abi_version.argtypes = []
    lib.sgemm_abi_version.restype = cint
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().sgemm_status_string(int(status)).decode()


def variant_name(variant: int) -> str | None:
    r = load().sgemm_variant_name(int(variant))
    return r.decode() if r is not None else None


def _variant_id(variant) -> int:
    if isinstance(variant, str):
        if variant not in VARIANTS:
            raise ValueError(f"unknown variant {variant!r}; one of {sorted(VARIANTS)}")
        return VARIANTS[variant]
    return int(variant)


def sgemm_f32_variant(variant, M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    """Raw entry point: integer pointers and sizes; returns the status code."""
    return load().sgemm_f32_variant(_variant_id(variant), M, N, K, A, lda, B, ldb, C, ldc, stream)


def sgemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    return load().sgemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream)


def _ld(t, name):
    import torch
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride (row-major)")
    return max(t.stride(0), t.shape[1], 1) if t.shape[0] > 1 else max(t.shape[1], 1)


def _stream_handle(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def sgemm(A, B, out=None, variant="auto"):
    """C = A @ B for float32 CUDA (ROCm) tensors, computed by libsgemm on the
    current stream.  Row-major views with any row stride >= the row length
    are accepted; ``out`` (M x N, written, never read) may be supplied."""
    import torch
    if A.device.type != "cuda" or B.device.type != "cuda":
        raise ValueError("operands must be GPU tensors")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {tuple(A.shape)} x {tuple(B.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    elif out.shape != (M, N):
        raise ValueError("out has the wrong shape")
    lda, ldb, ldc = _ld(A, "A"), _ld(B, "B"), _ld(out, "out")
    st = sgemm_f32_variant(variant, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb,
                           out.data_ptr(), ldc, _stream_handle(A.device))
    if st != 0:
        raise SgemmError(st, "sgemm_f32_variant")
    return out


def sgemm_ex(A, B, out=None, transa=False, transb=False, alpha=1.0, beta=0.0, splits=None,
             noalloc=False):
    """C = alpha op(A) op(B) + beta C (row-major float32 GPU tensors).  A is
    M x K, or K x M with transa (op(A) = A^T); B is K x N, or N x K with
    transb.  ``out`` holds C (read only when beta != 0); it is allocated when
    omitted (then beta must be 0).  ``splits`` (sgemm_f32_ex_split): None or
    0 chooses the K split by shape, 1 never splits, 2..64 asks for at most
    that many K chunks.  ``noalloc`` calls sgemm_f32_ex_split_noalloc, whose
    scratch is the library's static device array (the library then
    allocates nothing)."""
    import torch
    if A.device.type != "cuda" or B.device.type != "cuda":
        raise ValueError("operands must be GPU tensors")
    M, K = (A.shape[1], A.shape[0]) if transa else tuple(A.shape)
    Kb, N = (B.shape[1], B.shape[0]) if transb else tuple(B.shape)
    if Kb != K:
        raise ValueError("inner dimensions differ")
    if out is None:
        if beta != 0:
            raise ValueError("beta != 0 needs out")
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    elif tuple(out.shape) != (M, N):
        raise ValueError("out has the wrong shape")
    args = (int(transa), int(transb), M, N, K, alpha, A.data_ptr(), _ld(A, "A"), B.data_ptr(),
            _ld(B, "B"), beta, out.data_ptr(), _ld(out, "out"))
    if noalloc:
        name = "sgemm_f32_ex_split_noalloc"
        st = load().sgemm_f32_ex_split_noalloc(*args, int(splits or 0), _stream_handle(A.device))
    elif splits is None:
        name = "sgemm_f32_ex"
        st = load().sgemm_f32_ex(*args, _stream_handle(A.device))
    else:
        name = "sgemm_f32_ex_split"
        st = load().sgemm_f32_ex_split(*args, int(splits), _stream_handle(A.device))
    if st != 0:
        raise SgemmError(st, name)
    return out


def split_plan(M, N, K, transa=False, transb=False, lda=None, ldb=None, A_ptr=0, B_ptr=0,
               splits=0):
    """(chunks, kchunk) of the K split sgemm_f32_ex_split would run (host
    only; the pointers enter only through their 16-byte alignment)."""
    lda = (max(M, 1) if transa else max(K, 1)) if lda is None else lda
    ldb = (max(K, 1) if transb else max(N, 1)) if ldb is None else ldb
    kc = ctypes.c_int64(0)
    r = load().sgemm_split_plan(int(transa), int(transb), M, N, K, A_ptr or None, lda,
                                B_ptr or None, ldb, int(splits), ctypes.byref(kc))
    if r < 0:
        raise SgemmError(-r, "sgemm_split_plan")
    return r, kc.value


def plan_config(M, N, K, transa=False, transb=False, lda=None, ldb=None, A_ptr=0, B_ptr=0):
    """The kernel configuration a shape-chosen call runs (host only): dict
    with engine ("mfma", "thin" or None), tile (tile_m, tile_n), k_groups,
    packed, splits, kchunk; splits 0 when neither kernel is launched."""
    lda = (max(M, 1) if transa else max(K, 1)) if lda is None else lda
    ldb = (max(K, 1) if transb else max(N, 1)) if ldb is None else ldb
    en, tm, tn, wk, pk = (ctypes.c_int(0) for _ in range(5))
    kc = ctypes.c_int64(0)
    r = load().sgemm_plan_config(int(transa), int(transb), M, N, K, A_ptr or None, lda,
                                 B_ptr or None, ldb, ctypes.byref(en), ctypes.byref(tm),
                                 ctypes.byref(tn), ctypes.byref(wk), ctypes.byref(pk),
                                 ctypes.byref(kc))
    if r < 0:
        raise SgemmError(-r, "sgemm_plan_config")
    return {"engine": {1: "mfma", 2: "thin"}.get(en.value), "tile": (tm.value, tn.value),
            "k_groups": wk.value, "packed": bool(pk.value), "splits": r, "kchunk": kc.value}


def _ld_col(t, name):
    """Leading dimension of a column-major 2-D view (unit row stride)."""
    import torch
    if t.dtype != torch.float32 or t.dim() != 2:
        raise TypeError(f"{name} must be a 2-D float32 tensor")
    if t.shape[0] > 1 and t.stride(0) != 1:
        raise ValueError(f"{name} must be column-major (unit row stride)")
    return max(t.stride(1), t.shape[0], 1) if t.shape[1] > 1 else max(t.shape[0], 1)


def sgemm_colmajor(A, B, out, transa=False, transb=False, alpha=1.0, beta=0.0):
    """The column-major (BLAS) convention on column-major tensor views
    (stride(0) == 1): out (m x n) = alpha op(A) op(B) + beta out."""
    m, n = out.shape
    k = A.shape[0] if transa else A.shape[1]
    st = load().sgemm_f32_colmajor(int(transa), int(transb), m, n, k, alpha, A.data_ptr(),
                                   _ld_col(A, "A"), B.data_ptr(), _ld_col(B, "B"), beta,
                                   out.data_ptr(), _ld_col(out, "out"), _stream_handle(out.device))
    if st != 0:
        raise SgemmError(st, "sgemm_f32_colmajor")
    return out


def copy_f32(dst, src):
    """dst[:] = src[:] (float32 GPU tensors, contiguous) with the copy probe."""
    n = src.numel()
    if dst.numel() != n or not (dst.is_contiguous() and src.is_contiguous()):
        raise ValueError("copy needs contiguous tensors of equal size")
    st = load().sgemm_copy_f32(dst.data_ptr(), src.data_ptr(), n, _stream_handle(src.device))
    if st != 0:
        raise SgemmError(st, "sgemm_copy_f32")
    return dst


def copy_f32_launch(dst, src, block: int, grid: int):
    """The copy probe with an explicit workgroup size and count."""
    n = src.numel()
    if dst.numel() != n or not (dst.is_contiguous() and src.is_contiguous()):
        raise ValueError("copy needs contiguous tensors of equal size")
    st = load().sgemm_copy_f32_launch(dst.data_ptr(), src.data_ptr(), n, block, grid,
                                      _stream_handle(src.device))
    if st != 0:
        raise SgemmError(st, "sgemm_copy_f32_launch")
    return dst


VALU_CHAINS = 32
MFMA_WAVES_PER_BLOCK = 4
MFMA_ACC_PER_WAVE = 4


def probe_valu(blocks: int, block: int, iters: int, x: float, y: float, out=None):
    """Run the VALU multiply-add probe; returns the (blocks*block, VALU_CHAINS)
    output tensor (final chain values).  Work: blocks*block*iters*VALU_CHAINS*2
    FLOP."""
    import torch
    if out is None:
        out = torch.empty((blocks * block, VALU_CHAINS), dtype=torch.float32, device="cuda")
    elif out.numel() < blocks * block * VALU_CHAINS or not out.is_contiguous():
        raise ValueError("out too small or not contiguous")
    st = load().sgemm_probe_valu_f32(out.data_ptr(), blocks, block, iters, x, y,
                                     _stream_handle(out.device))
    if st != 0:
        raise SgemmError(st, "sgemm_probe_valu_f32")
    return out


def probe_mfma(a_vals, b_vals, blocks: int, iters: int, out=None):
    """Run the matrix-core probe; returns (blocks*4, 4, 32, 32) accumulators.
    Work: blocks*16*iters*4096 FLOP."""
    import torch
    n = blocks * MFMA_WAVES_PER_BLOCK * MFMA_ACC_PER_WAVE
    if out is None:
        out = torch.empty((blocks * MFMA_WAVES_PER_BLOCK, MFMA_ACC_PER_WAVE, 32, 32),
                          dtype=torch.float32, device="cuda")
    elif out.numel() < n * 1024 or not out.is_contiguous():
        raise ValueError("out too small or not contiguous")
    for v in (a_vals, b_vals):
        if v.numel() != 64 or v.dtype != torch.float32 or v.device.type != "cuda" or not v.is_contiguous():
            raise ValueError("a_vals and b_vals must be 64 contiguous float32 GPU values")
    st = load().sgemm_probe_mfma_f32(out.data_ptr(), a_vals.data_ptr(), b_vals.data_ptr(), blocks,
                                     iters, _stream_handle(out.device))
    if st != 0:
        raise SgemmError(st, "sgemm_probe_mfma_f32")
    return out
