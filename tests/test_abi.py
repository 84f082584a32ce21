"""The C ABI on the CPU: the library loads, exports what include/sgemm.h
declares, and rejects bad arguments on the host without any HIP call."""
import ctypes
import os
import re

import pytest

import roofline_sgemm_f32_amd as rs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgemm.h")

OK, DIM, LD, NULLPTR, VARIANT, ALIAS, LAUNCH, UNSUPPORTED, ARG, SCRATCH = range(10)

# Distinct, non-overlapping fake device addresses: validation never
# dereferences them and returns before any HIP call.
PA, PB, PC = 1 << 40, 2 << 40, 3 << 40


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rs.library_path()):
        pytest.skip("libsgemm.so not built (run __graft_entry__.build())")
    return rs.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(sgemm_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(rs.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_and_variant_names(lib):
    assert rs.status_string(OK) == "ok"
    for s in range(1, 10):
        assert rs.status_string(s) not in ("ok", "unknown status")
    assert rs.status_string(1234) == "unknown status"
    for name, vid in rs.VARIANTS.items():
        assert rs.variant_name(vid) == name
    assert rs.variant_name(99) is None
    assert lib.sgemm_abi_version() == 1


def call(variant, M, N, K, A=PA, lda=None, B=PB, ldb=None, C=PC, ldc=None):
    lda = max(K, 1) if lda is None else lda
    ldb = max(N, 1) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    return rs.sgemm_f32_variant(variant, M, N, K, A, lda, B, ldb, C, ldc, None)


@pytest.mark.parametrize("variant", list(rs.VARIANTS.values()))
def test_validation_codes(lib, variant):
    assert call(variant, -1, 4, 4) == DIM
    assert call(variant, 4, -1, 4) == DIM
    assert call(variant, 4, 4, -1) == DIM
    assert call(variant, 4, 4, 8, lda=7) == LD
    assert call(variant, 4, 8, 4, ldb=7) == LD
    assert call(variant, 4, 8, 4, ldc=7) == LD
    assert call(variant, 4, 4, 0, lda=0) == LD  # lda >= max(1, K)
    assert call(variant, 4, 4, 4, C=None) == NULLPTR
    assert call(variant, 4, 4, 4, A=None) == NULLPTR
    assert call(variant, 4, 4, 4, B=None) == NULLPTR
    # Empty outputs are a successful no-op even with null pointers.
    assert call(variant, 0, 4, 4, A=None, B=None, C=None) == OK
    assert call(variant, 4, 0, 4, A=None, B=None, C=None) == OK
    # Output overlapping an input.
    assert call(variant, 4, 4, 4, C=PA + 4) == ALIAS
    assert call(variant, 4, 4, 4, C=PB - 8) == ALIAS


def test_unknown_variant(lib):
    assert call(len(rs.VARIANTS), 4, 4, 4) == VARIANT  # one past the last variant
    assert call(-1, 4, 4, 4) == VARIANT


def test_alias_edges(lib):
    # C's last element is A's first element: overlap by one float.
    M, N, K = 3, 5, 7
    c_bytes = ((M - 1) * N + N) * 4
    assert call(4, M, N, K, C=PA - c_bytes + 4, A=PA) == ALIAS
    # A's last element is C's first.
    a_bytes = ((M - 1) * K + K) * 4
    assert call(4, M, N, K, C=PA + a_bytes - 4, A=PA) == ALIAS


def test_k4_rejects_offsets_beyond_32_bits_and_auto_falls_back(lib):
    M, N, K, lda = 256, 256, 16, 1 << 25  # 127 rows of lda exceed 2 GiB of offset
    assert call(4, M, N, K, lda=lda) == UNSUPPORTED
    auto = lib.sgemm_auto_variant(M, N, K, PA, lda, PB, N, PC, N)
    assert auto == rs.VARIANTS["k3_regtile_db"]
    assert lib.sgemm_auto_variant(4096, 4096, 4096, PA, 4096, PB, 4096, PC, 4096) == rs.VARIANTS["k4_mfma"]
    assert lib.sgemm_auto_variant(-1, 4, 4, PA, 4, PB, 4, PC, 4) == -DIM


def test_copy_validation(lib):
    f = lib.sgemm_copy_f32_launch
    assert f(PB, PA, -1, 256, 16, None) == ARG
    assert f(PB, PA, 100, 100, 16, None) == ARG
    assert f(PB, PA, 100, 2048, 16, None) == ARG
    assert f(PB, PA, 100, 256, 0, None) == ARG
    assert f(PB, PA, 0, 256, 16, None) == OK
    assert f(None, PA, 100, 256, 16, None) == NULLPTR
    assert f(PA + 8, PA, 100, 256, 16, None) == ALIAS
    assert lib.sgemm_copy_f32(PA, PA, -5, None) == ARG
    assert lib.sgemm_copy_f32(PA, PA, 0, None) == OK


def test_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        rs.sgemm(torch.ones(2, 2), torch.ones(2, 2))


def test_probe_validation(lib):
    assert lib.sgemm_probe_valu_f32(PA, 0, 64, 1, 1.0, 1.0, None) == ARG
    assert lib.sgemm_probe_valu_f32(PA, 1, 96, 1, 1.0, 1.0, None) == ARG
    assert lib.sgemm_probe_valu_f32(PA, 1 << 21, 64, 1, 1.0, 1.0, None) == ARG
    assert lib.sgemm_probe_valu_f32(PA, 1, 64, -1, 1.0, 1.0, None) == ARG
    assert lib.sgemm_probe_valu_f32(None, 1, 64, 1, 1.0, 1.0, None) == NULLPTR
    assert lib.sgemm_probe_mfma_f32(PA, None, PB, 1, 1, None) == NULLPTR
    assert lib.sgemm_probe_mfma_f32(PA, PB, PC, 0, 1, None) == ARG
    assert lib.sgemm_probe_mfma_f32(PA, PB, PC, 1, -1, None) == ARG


def ex(ta, tb, M, N, K, alpha=1.0, A=PA, lda=None, B=PB, ldb=None, beta=0.0, C=PC, ldc=None, lib=None):
    lda = (max(M, 1) if ta else max(K, 1)) if lda is None else lda
    ldb = (max(K, 1) if tb else max(N, 1)) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    return rs.load().sgemm_f32_ex(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, None)


def test_ex_validation(lib):
    assert ex(2, 0, 4, 4, 4) == ARG and ex(0, -1, 4, 4, 4) == ARG
    assert ex(0, 0, -1, 4, 4) == DIM
    # Leading dimensions follow the stored shapes.
    assert ex(0, 0, 4, 5, 6, lda=5) == LD      # A M x K needs lda >= K
    assert ex(1, 0, 4, 5, 6, lda=3) == LD      # A K x M needs lda >= M
    assert ex(0, 0, 4, 5, 6, ldb=4) == LD      # B K x N needs ldb >= N
    assert ex(0, 1, 4, 5, 6, ldb=5) == LD      # B N x K needs ldb >= K
    assert ex(0, 0, 4, 5, 6, ldc=4) == LD
    assert ex(0, 0, 4, 5, 6, C=None) == NULLPTR
    assert ex(0, 0, 4, 5, 6, A=None) == NULLPTR
    assert ex(0, 0, 0, 5, 6, A=None, B=None, C=None) == OK
    # Output overlapping a read operand.
    assert ex(0, 0, 4, 5, 6, C=PA + 8) == ALIAS
    assert ex(1, 1, 4, 5, 6, C=PB) == ALIAS


def test_colmajor_maps_to_swapped_rowmajor(lib):
    # Column-major validation is the swapped row-major one: ldc >= m, and
    # op(A) m x k with A stored m x k needs lda >= m.
    f = rs.load().sgemm_f32_colmajor
    assert f(0, 0, 4, 5, 6, 1.0, PA, 3, PB, 6, 0.0, PC, 4, None) == LD   # lda < m
    assert f(0, 0, 4, 5, 6, 1.0, PA, 4, PB, 5, 0.0, PC, 4, None) == LD   # ldb < k
    assert f(0, 0, 4, 5, 6, 1.0, PA, 4, PB, 6, 0.0, PC, 3, None) == LD   # ldc < m
    assert f(1, 0, 4, 5, 6, 1.0, PA, 5, PB, 6, 0.0, PC, 4, None) == LD   # A k x m: lda >= k
    assert f(0, 1, 4, 5, 6, 1.0, PA, 4, PB, 4, 0.0, PC, 4, None) == LD   # B n x k: ldb >= n
    assert f(3, 0, 4, 5, 6, 1.0, PA, 4, PB, 6, 0.0, PC, 4, None) == ARG


def test_ex_split_validation(lib):
    f = rs.load().sgemm_f32_ex_split
    # The split request is checked first; the rest as sgemm_f32_ex.
    assert f(0, 0, 4, 5, 6, 1.0, PA, 6, PB, 5, 0.0, PC, 5, -1, None) == ARG
    assert f(0, 0, 4, 5, 6, 1.0, PA, 6, PB, 5, 0.0, PC, 5, rs.MAX_SPLITS + 1, None) == ARG
    assert f(0, 0, 4, 5, 6, 1.0, PA, 5, PB, 5, 0.0, PC, 5, 2, None) == LD
    assert f(0, 0, -1, 5, 6, 1.0, PA, 6, PB, 5, 0.0, PC, 5, 2, None) == DIM
    assert f(0, 0, 4, 5, 6, 1.0, PA, 6, PB, 5, 0.0, PA + 4, 5, 2, None) == ALIAS
    assert f(2, 0, 4, 5, 6, 1.0, PA, 6, PB, 5, 0.0, PC, 5, 2, None) == ARG
    assert f(0, 0, 0, 5, 6, 1.0, None, 6, None, 5, 0.0, None, 5, rs.MAX_SPLITS, None) == OK


def test_split_plan_errors(lib):
    with pytest.raises(rs.SgemmError):
        rs.split_plan(64, 64, 64, splits=-1)
    with pytest.raises(rs.SgemmError):
        rs.split_plan(64, 64, 64, lda=10)
    with pytest.raises(rs.SgemmError):
        rs.split_plan(-1, 64, 64)


ALIGNED = 1 << 40  # a 16-byte aligned fake address


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (512, 512, 512), (1024, 1024, 1024),
                                   (1024, 1024, 4096), (256, 256, 16384), (128, 128, 4096),
                                   (2048, 2048, 2048), (4096, 4096, 4096), (1, 1, 1),
                                   (300, 17, 129), (3001, 4099, 2047), (64, 64, 1 << 20)])
@pytest.mark.parametrize("trans", [(0, 0), (1, 1)])
def test_split_plan_chunks_cover_k(lib, M, N, K, trans):
    # Whatever is asked, the chunks are whole slabs (32 of K with 16-byte
    # loads, else 16), every chunk is nonempty and together they cover K once.
    for splits in [0, 1, 2, 3, 5, 16, rs.MAX_SPLITS]:
        for ptr in [ALIGNED, ALIGNED + 4]:
            S, kc = rs.split_plan(M, N, K, transa=trans[0], transb=trans[1], A_ptr=ptr,
                                  B_ptr=ALIGNED, splits=splits)
            assert S >= 1
            if S == 1:
                assert kc == K
                continue
            vec = ptr % 16 == 0 and (M if trans[0] else K) % 4 == 0 and (K if trans[1] else N) % 4 == 0
            assert kc % (32 if vec else 16) == 0
            assert (S - 1) * kc < K <= S * kc
            assert S <= (32 if splits == 0 else splits)
            if splits == 1:
                raise AssertionError("splits=1 must not split")


def test_split_plan_choices(lib):
    # Outputs of few 32 x 32 tiles with a long K are split; outputs of fewer
    # than 1024 64 x 64 tiles take the cost model's split when it saves 5 %;
    # larger outputs are not split.
    plan = lambda M, N, K: rs.split_plan(M, N, K, A_ptr=ALIGNED, B_ptr=ALIGNED)[0]
    assert plan(64, 64, 65536) == 32
    assert plan(128, 128, 4096) == 16
    assert plan(256, 256, 16384) == 8
    assert plan(256, 256, 2048) == 8
    assert plan(128, 128, 1024) == 4
    assert plan(256, 256, 768) == 3
    assert plan(512, 512, 4096) == 2
    # Too little K to save: square 256 and 512.
    assert plan(256, 256, 256) == 1
    assert plan(512, 512, 512) == 1
    for n in (1024, 2048, 4096, 8192):
        assert plan(n, n, n) == 1
    assert plan(1024, 1024, 4096) == 1
    assert plan(3001, 4099, 2047) == 1
    # A short K is never cut below one slab.
    assert plan(64, 64, 40) == 1
    # 64 x 64 tiles under 4 per CU with a long K (measured on MI355X against
    # the unsplit choice: 64 x 8192 x 8192 153 -> 80 us, 192 x 8192 x 8192
    # 297 -> 222, 1536^2 x 4096 214 -> 170, 256 x 2048 x 16384 304 -> 148).
    assert plan(64, 8192, 8192) == 8
    assert plan(8192, 64, 8192) == 8
    assert plan(192, 8192, 8192) == 4
    assert plan(1536, 1536, 4096) == 4
    assert plan(256, 2048, 16384) == 8
    assert plan(1536, 1024, 1024) == 2
    # ... and where the model finds no 5 % (measured within noise).
    assert plan(1024, 1024, 2048) == 1
    assert plan(1280, 1280, 1280) == 1
    assert plan(2048, 1024, 8192) == 1
    assert plan(64, 16384, 4096) == 1
    # No chunk below 512 of K from the model.
    assert plan(768, 768, 768) == 1
    for M, N, K in [(64, 8192, 4096), (768, 768, 4096), (512, 1024, 8192)]:
        S, kc = rs.split_plan(M, N, K, A_ptr=ALIGNED, B_ptr=ALIGNED)
        assert S > 1 and kc >= 512 and kc % 32 == 0 and (S - 1) * kc < K <= S * kc
    # Up to 768 tiles of 32 x 32 with K <= 2048 run unsplit on 32 x 32 tiles
    # with K groups (one round of three workgroups per CU).
    for M, N, K in [(64, 8192, 1024), (640, 640, 640), (512, 1024, 1024), (192, 4096, 1024), (64, 8192, 2048),
                    (768, 1024, 1280)]:
        assert rs.split_plan(M, N, K, A_ptr=ALIGNED, B_ptr=ALIGNED) == (1, K)


def test_plan_config_choices(lib):
    # Tile configuration of shape-chosen calls (measured choices on MI355X).
    cfg = lambda M, N, K, **kw: rs.plan_config(M, N, K, A_ptr=ALIGNED, B_ptr=ALIGNED, **kw)
    big = cfg(4096, 4096, 4096)
    assert big == {"engine": "mfma", "tile": (128, 256), "k_groups": 1, "packed": False, "splits": 1,
                   "kchunk": 4096}
    assert cfg(8192, 8192, 8192)["tile"] == (128, 256)
    for ta, tb in [(True, False), (False, True), (True, True)]:      # every storage orientation
        assert cfg(4096, 4096, 4096, transa=ta, transb=tb, lda=4096, ldb=4096)["tile"] == (128, 256)
    assert cfg(6144, 6144, 6144)["tile"] == (128, 128)               # 2.25 rounds of 128 x 256
    assert cfg(3072, 3072, 3072)["tile"] == (64, 64)
    small = cfg(256, 256, 256)
    assert small["tile"] == (32, 32) and small["k_groups"] == 4 and small["splits"] == 1
    # Up to 1024 such tiles with K <= 2048: one round of three (up to 768
    # tiles) or four workgroups per CU.
    for M, N, K in [(640, 640, 640), (896, 896, 896), (1024, 1024, 1024), (1024, 1024, 2048)]:
        mid = cfg(M, N, K)
        assert mid["tile"] == (32, 32) and mid["k_groups"] == 4 and mid["splits"] == 1, (M, N, K, mid)
    assert cfg(1024, 1024, 4096)["tile"] == (64, 64) and cfg(1024, 1024, 4096)["k_groups"] == 4
    assert cfg(1056, 1024, 1024)["tile"] == (64, 64)  # 1056 tiles of 32 x 32
    assert cfg(640, 640, 4096)["tile"] == (64, 64)    # a longer K
    assert cfg(128, 128, 4096)["splits"] == 16
    skinny = cfg(64, 8192, 8192)
    assert skinny["tile"] == (64, 64) and skinny["k_groups"] == 1 and skinny["splits"] == 8
    # Narrow outputs: 128 x 256 and 128 x 128 tiles would be mostly empty.
    for M, N, K in [(65536, 128, 1024), (65536, 64, 4096), (65536, 160, 2048), (65536, 192, 1024),
                    (32768, 320, 2048)]:
        assert cfg(M, N, K)["tile"] == (64, 64), (M, N, K)
    # Unaligned operands of a large output: packed copies, 64 x 64 tiles.
    ragged = cfg(3001, 4099, 2047)
    assert ragged["packed"] and ragged["tile"] == (64, 64) and ragged["splits"] == 1
    # A thin unaligned operand of a large product is copied; a large one of a
    # memory-bound product, or the operands of a mid-size product, are not.
    assert cfg(8192, 13, 8192)["packed"] and cfg(13, 8192, 8191)["packed"]
    assert not cfg(1, 8191, 8192)["packed"]
    assert not cfg(1024, 1027, 1024)["packed"] and not cfg(1023, 1023, 1023)["packed"]
    # 4 GFLOP or more with small copies: copied (and split on the copies).
    assert cfg(767, 769, 4095)["packed"] and cfg(513, 511, 8193)["packed"]
    # 1 GFLOP or more with K >= 1536: copied too; a shorter K is not.
    assert cfg(511, 513, 4095)["packed"] and cfg(800, 801, 2047)["packed"] and cfg(600, 601, 1600)["packed"]
    assert not cfg(700, 701, 1500)["packed"] and not cfg(300, 301, 4095)["packed"]
    assert not cfg(64, 64, 1000001)["packed"]      # copies of 512 MB for an 8 GFLOP product


def test_plan_config_agrees_with_split_plan(lib):
    for M, N, K in [(64, 64, 65536), (256, 256, 768), (512, 512, 4096), (192, 8192, 8192),
                    (1024, 1024, 4096), (4096, 4096, 4096), (1536, 1024, 1024)]:
        c = rs.plan_config(M, N, K, A_ptr=ALIGNED, B_ptr=ALIGNED)
        assert (c["splits"], c["kchunk"]) == rs.split_plan(M, N, K, A_ptr=ALIGNED, B_ptr=ALIGNED)


def test_plan_config_empty_and_errors(lib):
    for M, N, K in [(0, 5, 5), (5, 0, 5), (5, 5, 0)]:
        c = rs.plan_config(M, N, K, A_ptr=ALIGNED, B_ptr=ALIGNED)
        assert c == {"engine": None, "tile": (0, 0), "k_groups": 0, "packed": False, "splits": 0,
                     "kchunk": 0}
    with pytest.raises(rs.SgemmError):
        rs.plan_config(-1, 4, 4)
    with pytest.raises(rs.SgemmError):
        rs.plan_config(64, 64, 64, lda=10)
    assert lib.sgemm_plan_config(0, 0, 64, 64, 64, None, 64, None, 64, None, None, None, None, None,
                                 None) == 1


def test_plan_config_thin(lib):
    # M <= 8 or N <= 8 with a large operand that suits 16-byte loads, of
    # 384 MB or more (256 MB for 2 to 4 columns, 16 MB for a single column):
    # the thin kernels on the vector units.
    cfg = lambda M, N, K, **kw: rs.plan_config(M, N, K, A_ptr=ALIGNED, B_ptr=ALIGNED, **kw)
    for M in (1, 4, 8):
        c = cfg(M, 16384, 16384)
        assert c["engine"] == "thin" and c["tile"] == (M, 256) and c["k_groups"] == 4
        assert c["splits"] > 1 and c["kchunk"] >= 256
        assert cfg(M, 8192, 8192)["engine"] == "mfma"             # 268 MB: measured no faster
    for N in (2, 3, 8):
        c = cfg(16384, N, 16384)
        # 4-wave workgroups (16 rows) for one or two columns with M >= 16384.
        assert c["engine"] == "thin" and c["tile"] == (16 if N <= 2 else 32, N) and c["kchunk"] % 1024 == 0
    assert cfg(16383, 2, 16384)["tile"] == (32, 2) and cfg(65536, 1, 4096)["tile"] == (16, 1)
    for N in (2, 4):
        assert cfg(8192, N, 8192)["engine"] == "thin"             # 268 MB, few columns
        assert cfg(8192, N, 7680)["engine"] == "mfma"             # 252 MB
    for N in (5, 8):
        assert cfg(8192, N, 8192)["engine"] == "mfma"             # 268 MB: measured no faster
    assert cfg(8192, 1, 8192)["engine"] == "thin"                 # one column: from 16 MB
    assert cfg(4096, 1, 1024)["engine"] == "thin"
    assert cfg(4096, 1, 1020)["engine"] == "mfma"
    assert cfg(16384, 8, 16384, transb=True)["engine"] == "thin"  # B is staged, any orientation
    assert cfg(8, 16384, 16384, transa=True)["engine"] == "thin"  # A read by scalar loads
    # A streamed operand stored with K contiguous on the other side: the
    # transposed product on the same kernels, stored transposed.
    c = cfg(16384, 8, 16384, transa=True, lda=16384)
    assert c["engine"] == "thin" and c["tile"] == (256, 8) and c["k_groups"] == 4
    c = cfg(8, 16384, 16384, transb=True, ldb=16384)
    assert c["engine"] == "thin" and c["tile"] == (8, 32)
    assert cfg(1, 16384, 16384, transb=True, ldb=16384)["tile"] == (1, 16)
    assert cfg(1, 8192, 8192, transb=True, ldb=8192)["engine"] == "mfma"   # from 384 MB when transposed
    assert cfg(16384, 8, 16384, transa=True, lda=16385)["engine"] == "thin"  # rows not 16-byte chunks: 4-byte loads
    assert cfg(16, 16384, 16384)["engine"] == "mfma"              # not thin
    assert cfg(1, 16383, 16384)["engine"] == "thin"               # B rows not 16-byte chunks: 4-byte loads
    assert cfg(16384, 1, 16383)["engine"] == "thin"               # A rows not 16-byte chunks: 4-byte loads
    # Unaligned streams with up to 4 rows or columns of C: from 16 MB.
    assert cfg(1, 4095, 4096)["engine"] == "thin" and cfg(4096, 3, 2047)["engine"] == "thin"
    assert cfg(8, 4095, 4096)["engine"] == "mfma" and cfg(8192, 8, 8191)["engine"] == "mfma"
    assert cfg(1 << 27, 1, 4)["engine"] == "thin"                 # rows the thin_n grid can count
    assert cfg((1 << 27) + 4, 1, 4)["engine"] == "mfma"
    # A split request bypasses the thin path.
    assert rs.split_plan(8, 16384, 16384, A_ptr=ALIGNED, B_ptr=ALIGNED, splits=1) == (1, 16384)


def _no_gpu_visible():
    """True when no GPU can run anything here: no KFD device node, and the
    HIP runtime counts no device.  Only then may a valid call with fake
    pointers reach the launch (which must then fail cleanly)."""
    if os.path.exists("/dev/kfd"):
        return False
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return True
    n = ctypes.c_int(0)
    rc = hip.hipGetDeviceCount(ctypes.byref(n))
    return rc != 0 or n.value == 0


def test_launch_failure_without_device(lib):
    """A valid call whose launch fails (here: no GPU in the machine) returns
    SGEMM_ERR_LAUNCH and records the HIP error; the process is not aborted."""
    if not _no_gpu_visible():
        pytest.skip("a GPU is visible: fake device pointers must not be launched on")
    assert lib.sgemm_f32(64, 64, 64, PA, 64, PB, 64, PC, 64, None) == LAUNCH
    err = lib.sgemm_last_hip_error()
    assert err != 0
    # The shape-chosen split path (it would use the workspace) fails the same way.
    assert lib.sgemm_f32_ex_split(0, 0, 64, 64, 8192, 1.0, PA, 8192, PB, 64, 0.0, PC, 64, 0, None) == LAUNCH
    assert lib.sgemm_f32_ex_split_noalloc(0, 0, 64, 64, 8192, 1.0, PA, 8192, PB, 64, 0.0, PC, 64, 0,
                                          None) == LAUNCH
    for v in rs.VARIANTS.values():
        assert call(v, 40, 40, 40) == LAUNCH
    assert lib.sgemm_copy_f32(PB, PA, 1000, None) == LAUNCH
    assert lib.sgemm_last_hip_error() == err


def test_noalloc_validation(lib):
    f = lib.sgemm_f32_ex_split_noalloc
    args = (0, 0, 64, 64, 64, 1.0, PA, 64, PB, 64, 0.0, PC, 64)
    assert f(*args, -1, None) == ARG
    assert f(*args, rs.MAX_SPLITS + 1, None) == ARG
    assert f(2, 0, 64, 64, 64, 1.0, PA, 64, PB, 64, 0.0, PC, 64, 0, None) == ARG
    assert f(0, 0, -1, 64, 64, 1.0, PA, 64, PB, 64, 0.0, PC, 64, 0, None) == DIM
    assert f(0, 0, 64, 64, 64, 1.0, PA, 32, PB, 64, 0.0, PC, 64, 0, None) == LD
    assert f(0, 0, 64, 64, 64, 1.0, PA, 64, PB, 64, 0.0, PA + 4, 64, 0, None) == ALIAS
    assert f(0, 0, 0, 64, 64, 1.0, None, 64, None, 64, 0.0, None, 64, 0, None) == OK
    # Two chunks of 4096 x 4096 partial products: 128 MiB, over the 64 MiB
    # static scratch; refused on the host, before any HIP call.
    assert rs.STATIC_SCRATCH_BYTES == 64 << 20
    big = (0, 0, 4096, 4096, 8192, 1.0, PA, 8192, PB, 4096, 0.0, PC, 4096)
    assert f(*big, 2, None) == SCRATCH
    assert rs.status_string(SCRATCH) != "unknown status"
