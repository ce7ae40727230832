"""The C ABI on the host: the library loads, exports every declared entry
point, and rejects bad arguments before touching the GPU (these calls never
reach a HIP launch, so they run without a device)."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

import w4a16_bit_matmul_amd as wq

HEADER = os.path.join(ROOT, "include", "libwq.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("wq_quantize_groups", "wq_pack_int4", "wq_dequant", "wq_gemm_w4a16"):
        assert required in names
    assert set(names) == set(wq.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = wq.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_version_and_strerror():
    assert wq.wq_version() >= 100
    for st in (0, -1, -2, -3, -4, -5):
        assert len(wq.strerror(st)) > 5
    assert wq.strerror(-99) == "unknown status"


@pytest.mark.parametrize("N,K,g", [(8192, 8192, 128), (37, 96, 32), (1, 32, 32), (28672, 8192, 32)])
def test_layout_bytes(N, K, g):
    q, s, z = wq.wq_layout_bytes(N, K, g)
    Np, Kp, G = (N + 15) // 16 * 16, (K + 127) // 128 * 128, K // g
    assert q == Np * Kp // 2 and s == 2 * N * G and z == N * ((G + 1) // 2)


def test_layout_bytes_rejects():
    for args, st in [((0, 128, 128), wq.WQ_EINVAL), ((16, -128, 128), wq.WQ_EINVAL),
                     ((16, 128, 64), wq.WQ_EUNSUPPORTED), ((16, 96, 128), wq.WQ_EUNSUPPORTED)]:
        with pytest.raises(wq.WQError) as e:
            wq.wq_layout_bytes(*args)
        assert e.value.status == st


P = ctypes.c_void_p
A = P(0x10000)      # aligned fake device address (never dereferenced)
B = P(0x10001)      # misaligned


def call(name, *args):
    return getattr(wq.lib(), name)(*args)


def test_quantize_validation():
    f = "wq_quantize_groups"
    assert call(f, None, 1, 16, 128, 128, None, A, None, None, None, None) == wq.WQ_EINVAL
    assert call(f, A, 1, 16, 128, 128, None, None, None, None, None, None) == wq.WQ_EINVAL
    assert call(f, A, 7, 16, 128, 128, None, A, None, None, None, None) == wq.WQ_EINVAL
    assert call(f, A, 1, 0, 128, 128, None, A, None, None, None, None) == wq.WQ_EINVAL
    assert call(f, A, 1, 16, 128, 64, None, A, None, None, None, None) == wq.WQ_EUNSUPPORTED
    assert call(f, A, 1, 16, 160, 128, None, A, None, None, None, None) == wq.WQ_EUNSUPPORTED
    assert call(f, B, 1, 16, 128, 128, None, A, None, None, None, None) == wq.WQ_EALIGN
    assert call(f, A, 1, 16, 128, 128, None, A, None, B, None, None) == wq.WQ_EALIGN


def test_pack_and_dequant_validation():
    assert call("wq_pack_int4", None, A, 16, 128, 128, A, A, None) == wq.WQ_EINVAL
    assert call("wq_pack_int4", A, A, 16, 100, 32, A, A, None) == wq.WQ_EUNSUPPORTED
    assert call("wq_pack_int4", A, A, 16, 128, 128, B, A, None) == wq.WQ_EALIGN
    assert call("wq_dequant", A, A, A, 16, 128, 128, 5, A, None) == wq.WQ_EINVAL
    assert call("wq_dequant", A, A, A, 16, 128, 128, 0, None, None) == wq.WQ_EINVAL
    assert call("wq_dequant", A, A, A, 16, 128, 48, 0, A, None) == wq.WQ_EUNSUPPORTED
    assert call("wq_dequant", A, A, A, 16, 128, 128, 0, B, None) == wq.WQ_EALIGN


def test_gemm_validation():
    f = "wq_gemm_w4a16_ex"
    ok = (A, A, A, A, A, None, 0)
    assert call(f, 0, 16, 128, 128, *ok, 0, None) == wq.WQ_EINVAL
    assert call(f, 1, 16, 128, 128, None, A, A, A, A, None, 0, 0, None) == wq.WQ_EINVAL
    assert call(f, 1, 16, 128, 128, *ok, 9, None) == wq.WQ_EINVAL
    assert call(f, 1, 16, 128, 32 * 3, *ok, 0, None) == wq.WQ_EUNSUPPORTED
    assert call(f, 1, 16, 100, 32, *ok, 0, None) == wq.WQ_EUNSUPPORTED
    assert call(f, 1, 16, 128, 128, B, A, A, A, A, None, 0, 0, None) == wq.WQ_EALIGN
    assert call("wq_gemm_w4a16", 1, 16, 128, 128, A, A, A, A, B, None, 0, None) == wq.WQ_EALIGN


def test_workspace_query_and_check():
    # host-only: either kernel family asks for a workspace when it splits K
    # across workgroups to fill the GPU (few row or column blocks); the
    # query covers both families (the M=128, N=28672 GEMM splits nothing)
    assert wq.wq_gemm_workspace_bytes(128, 28672, 8192, 128) == 0
    for M, N, K, g in [(1, 1024, 28672, 32), (8, 1024, 8192, 128), (1, 48, 28672, 128), (16, 64, 28672, 32)]:
        for path in (wq.WQ_PATH_GEMV, wq.WQ_PATH_MFMA):
            need = wq.wq_gemm_workspace_bytes(M, N, K, g, path)
            assert 0 < need <= wq.wq_gemm_workspace_bytes(M, N, K, g), (M, N, K, g, path)
            # counter region, then KS fp32 partial-sum planes padded to whole
            # tiles: GEMV MT x 16 per workgroup (1 x 8 for the eight-row
            # one-row kernel), MFMA 16*MB x 128
            plan = wq.wq_gemm_plan(M, N, K, g, path)
            gx, gy, ks = (int(v) for v in plan.split("grid=(", 1)[1].split(")", 1)[0].split(","))
            if path == wq.WQ_PATH_GEMV and "half" in plan:
                rows, cols = 1, 8
            elif path == wq.WQ_PATH_GEMV:
                rows, cols = int(plan.split("MT=", 1)[1].split(",")[0]), 16
            else:
                rows, cols = 16 * int(plan.split("MB=", 1)[1].split(",")[0]), 128
            assert gy * rows >= M and gx * cols >= N
            assert need == wq.WQ_WORKSPACE_COUNTER_BYTES + ks * gy * rows * gx * cols * 4, (M, N, K, g, path, plan)
            st = call("wq_gemm_w4a16_ex", M, N, K, g, A, A, A, A, A, None, 0, path, None)
            assert st == wq.WQ_EWORKSPACE
            st = call("wq_gemm_w4a16_ex", M, N, K, g, A, A, A, A, A, A, need - 1, path, None)
            assert st == wq.WQ_EWORKSPACE
            st = call("wq_gemm_w4a16_ex", M, N, K, g, A, A, A, A, A, B, need, path, None)
            assert st == wq.WQ_EALIGN
    assert wq.wq_gemm_workspace_bytes(0, 16, 128, 128) == 0
    assert wq.wq_gemm_workspace_bytes(1, 16, 128, 128, 9) == 0


def split_k(plan):
    return int(re.search(r"split_k=(\d+)", plan).group(1))


def test_gemm_plan_names_the_dispatched_kernel():
    # host-only description of the kernel each problem runs: the decode GEMV
    # (one row block of 16 outputs per workgroup, no K split) and the M=128 MFMA
    # GEMM (eight 16-row blocks per workgroup)
    d = wq.wq_gemm_plan(1, 8192, 8192, 128)
    assert d.startswith("gemv_mfma_kernel<MT=1, W=16, KQ=4, G=128>") and "grid=(512,1,1)" in d and split_k(d) == 1, d
    # one row of x over few row blocks: eight weight rows per workgroup
    d = wq.wq_gemm_plan(1, 1024, 8192, 32)
    assert d.startswith("gemv_mfma_half_kernel<W=16, KQ=4, G=32>") and "grid=(128,1,1)" in d, d
    d = wq.wq_gemm_plan(128, 28672, 8192, 128)
    assert d.startswith("gemm_kernel<MB=8, NPW=2, G=128>") and "grid=(224,1,1)" in d, d
    # 4-bit GEMV past eight rows: a sixteen-row activation tile when that
    # still leaves 128 workgroups before a K split, two eight-row tiles below
    assert wq.wq_gemm_plan(128, 256, 1024, 32, wq.WQ_PATH_GEMV).startswith("gemv_mfma_kernel<MT=16")
    d = wq.wq_gemm_plan(16, 28672, 8192, 128)
    assert d.startswith("gemv_mfma_kernel<MT=16, W=4, KQ=4, G=128, RB=4>") and "grid=(448,1,1)" in d, d
    d = wq.wq_gemm_plan(8, 28672, 8192, 32)
    assert d.startswith("gemv_mfma_kernel<MT=8, W=8, KQ=4, G=32, RB=2>") and "grid=(896,1,1)" in d, d
    # narrow outputs (N <= 2048) with 9..32 rows: eight-row tiles in
    # sixteen-wave workgroups over all of K where that fills the GPU (at least
    # 64 workgroups and eight K segments, sixteen past 256 workgroups, one pass
    # over K unless the grid has 256); otherwise the plans above
    for M, N, K in ((16, 1024, 8192), (32, 1024, 8192), (16, 2048, 8192), (32, 2048, 8192), (32, 1024, 14336),
                    (24, 512, 4096), (16, 512, 8192), (12, 520, 4224), (32, 1024, 4096)):
        for g in (32, 128):
            d = wq.wq_gemm_plan(M, N, K, g, wq.WQ_PATH_GEMV)
            assert d.startswith(f"gemv_mfma_kernel<MT=8, W=16, KQ=4, G={g}>") and split_k(d) == 1, d
            assert f"grid=({(N + 15) // 16},{(M + 7) // 8},1) block=1024" in d, d
        assert wq.wq_gemm_mxfp4_plan(M, N, K, wq.WQ_PATH_GEMV).startswith("gemv_mfma_kernel<MT=8, W=16, KQ=4, G=32, RB=1, MXFP4>")
        assert wq.wq_gemm_nvfp4_plan(M, N, K, wq.WQ_PATH_GEMV).startswith("gemv_mfma_kernel<MT=8, W=16, KQ=4, G=16, RB=1, NVFP4>")
        # 8-bit codes keep eight-wave workgroups
        assert "W=8" in wq.wq_gemm_w8a16_plan(M, N, K, 32, wq.WQ_PATH_GEMV)
    d = wq.wq_gemm_plan(16, 1024, 14336, 32)  # two passes over K, 128 workgroups: split
    assert d.startswith("gemv_mfma_kernel<MT=8, W=8,") and split_k(d) == 4, d
    # too few K segments (K = 2048: four; K = 4096 past 256 workgroups) or
    # workgroups (N = 64, 160): the plans above
    for M, N, K in ((32, 2048, 2048), (16, 1024, 2048), (32, 2048, 4096), (16, 64, 8192), (24, 160, 8192), (9, 300, 1024)):
        d = wq.wq_gemm_plan(M, N, K, 128, wq.WQ_PATH_GEMV)
        assert "W=16" not in d, (M, N, K, d)
    d = wq.wq_gemm_plan(8, 1024, 8192, 32)
    assert d.startswith("gemv_mfma_kernel<MT=8, W=8,") and split_k(d) == 2, d
    d = wq.wq_gemm_plan(33, 1024, 8192, 32, wq.WQ_PATH_GEMV)
    assert d.startswith("gemv_mfma_kernel<MT=16") and "grid=(64,3," in d, d
    assert wq.wq_gemm_plan(16, 2064, 8192, 32).startswith("gemv_mfma_kernel<MT=16")
    assert wq.wq_gemm_w8a16_plan(16, 28672, 8192, 128, wq.WQ_PATH_GEMV).startswith("gemv_mfma_kernel<MT=16, W=8, KQ=4, G=128, RB=1, BITS=8>")
    assert wq.wq_gemm_plan(1, 256, 1024, 32, wq.WQ_PATH_MFMA).startswith("gemm_kernel<MB=1, NPW=2, G=32>")
    # a small grid splits K across workgroups in whole eight-tile chunks
    d = wq.wq_gemm_plan(128, 8192, 8192, 128)
    assert d.startswith("gemm_kernel<MB=4,") and "grid=(64,2,2)" in d and split_k(d) == 2, d
    d = wq.wq_gemm_plan(32, 1024, 8192, 32, wq.WQ_PATH_MFMA)
    assert "grid=(8,1,8)" in d and "split_k=8" in d, d
    assert split_k(wq.wq_gemm_plan(128, 28672, 8192, 128)) == 1
    assert split_k(wq.wq_gemm_plan(1, 48, 28672, 128)) > 1
    # one pass of the waves covers K = 8192 at one row: no split, which would
    # only leave waves idle and add the hand-off
    assert split_k(wq.wq_gemm_plan(1, 1024, 8192, 32)) == 1
    # the AUTO rule's bounds: the same values in the header and the binding
    m = re.search(r"#define WQ_WORKSPACE_COUNTER_BYTES (\d+)", open(HEADER).read())
    assert m and int(m.group(1)) == wq.WQ_WORKSPACE_COUNTER_BYTES
    for name in ("WQ_AUTO_GEMV_MAX_N", "WQ_AUTO_NARROW_GEMV_MAX_M", "WQ_AUTO_INT4_GEMV_MAX_M",
                 "WQ_AUTO_INT4_G32_LONG_K", "WQ_AUTO_INT4_G32_LONG_K_GEMV_MAX_M", "WQ_AUTO_FP4_GEMV_MAX_M",
                 "WQ_AUTO_INT8_GEMV_MAX_M"):
        m = re.search(r"#define %s (\d+)" % name, open(HEADER).read())
        assert m and int(m.group(1)) == getattr(wq, name), name
    # the binding's restatement of the rule agrees with the plans of every
    # code format, group and K: small N keeps the GEMV for more rows, long K
    # at group 32 fewer
    for K in (4096, 16384, 16512, 28672):
        plans = {("int4", 32): lambda M, N: wq.wq_gemm_plan(M, N, K, 32),
                 ("int4", 128): lambda M, N: wq.wq_gemm_plan(M, N, K, 128),
                 ("int8", 32): lambda M, N: wq.wq_gemm_w8a16_plan(M, N, K, 32),
                 ("mxfp4", 32): lambda M, N: wq.wq_gemm_mxfp4_plan(M, N, K),
                 ("nvfp4", 16): lambda M, N: wq.wq_gemm_nvfp4_plan(M, N, K)}
        for (fmt, group), plan in plans.items():
            for M in (1, 4, 5, 8, 9, 16, 17, 32, 33, 128):
                for N in (256, 1024, 2048, 2064, 8192, 16384, 16400, 28672):
                    mfma = plan(M, N).startswith("gemm_kernel")
                    assert mfma == wq.auto_uses_mfma(M, N, fmt, K, group), (fmt, group, K, M, N)
    with pytest.raises(ValueError):
        wq.auto_uses_mfma(16, 8192)  # the 4-bit rule needs K and the group
    assert not wq.auto_uses_mfma(32, 1024, "int8") and wq.auto_uses_mfma(33, 1024, "int8")
    assert wq.auto_uses_mfma(9, 8192, "int8") and not wq.auto_uses_mfma(8, 28672, "int8")
    assert wq.auto_uses_mfma(16, 28672, "int8") and wq.auto_uses_mfma(9, 2064, "int8")
    for fmt in ("mxfp4", "nvfp4"):
        assert not wq.auto_uses_mfma(16, 28672, fmt) and wq.auto_uses_mfma(17, 28672, fmt)
        assert not wq.auto_uses_mfma(32, 2048, fmt) and wq.auto_uses_mfma(33, 2048, fmt)
        assert wq.auto_uses_mfma(17, 2064, fmt)
    for g in (32, 128):
        assert not wq.auto_uses_mfma(16, 8192, "int4", 8192, g) and wq.auto_uses_mfma(17, 8192, "int4", 8192, g)
        assert not wq.auto_uses_mfma(32, 2048, "int4", 28672, g) and wq.auto_uses_mfma(33, 1024, "int4", 8192, g)
    assert not wq.auto_uses_mfma(16, 8192, "int4", 28672, 128) and wq.auto_uses_mfma(9, 8192, "int4", 28672, 32)
    assert not wq.auto_uses_mfma(8, 8192, "int4", 28672, 32) and not wq.auto_uses_mfma(16, 8192, "int4", 16384, 32)
    hi = wq.WQ_AUTO_INT4_GEMV_MAX_M
    assert wq.wq_gemm_plan(hi, 8192, 8192, 128).startswith("gemv_mfma_kernel"), hi
    assert wq.wq_gemm_plan(hi + 1, 8192, 8192, 128).startswith("gemm_kernel"), hi
    i8 = wq.WQ_AUTO_INT8_GEMV_MAX_M
    assert wq.wq_gemm_w8a16_plan(i8, 8192, 8192, 128).startswith("gemv_mfma_kernel")
    assert wq.wq_gemm_w8a16_plan(i8 + 1, 8192, 8192, 128).startswith("gemm_kernel")
    fp4 = wq.WQ_AUTO_FP4_GEMV_MAX_M
    assert wq.wq_gemm_mxfp4_plan(fp4, 8192, 8192).startswith("gemv_mfma_kernel")
    assert wq.wq_gemm_mxfp4_plan(fp4 + 1, 8192, 8192).startswith("gemm_kernel")
    buf = ctypes.create_string_buffer(8)
    assert wq.lib().wq_gemm_plan(1, 8192, 8192, 128, 0, buf, 8) == wq.WQ_OK and len(buf.value) == 7
    assert wq.lib().wq_gemm_plan(1, 8192, 8192, 128, 0, None, 8) == wq.WQ_EINVAL
    assert wq.lib().wq_gemm_plan(0, 8192, 8192, 128, 0, buf, 8) == wq.WQ_EINVAL
    assert wq.lib().wq_gemm_plan(1, 8192, 8192, 128, 7, buf, 8) == wq.WQ_EINVAL
    assert wq.lib().wq_gemm_plan(1, 8192, 8192, 48, 0, buf, 8) == wq.WQ_EUNSUPPORTED



def test_sequence_call_checks_every_product_first():
    # host-only: an error in any product of the sequence returns before
    # anything is enqueued (no GPU here, so nothing could run anyway)
    P = ctypes.c_void_p
    ok = (P * 2)(A, A)
    bad = (P * 2)(A, None)
    f = wq.lib().wq_gemm_w4a16_seq
    assert f(2, 1, 16, 128, 128, ok, ok, ok, ok, bad, None, 0, None) == wq.WQ_EINVAL
    assert f(2, 1, 16, 128, 128, ok, ok, ok, ok, (P * 2)(A, B), None, 0, None) == wq.WQ_EALIGN
    assert f(-1, 1, 16, 128, 128, ok, ok, ok, ok, ok, None, 0, None) == wq.WQ_EINVAL
    assert f(2, 1, 16, 128, 128, None, ok, ok, ok, ok, None, 0, None) == wq.WQ_EINVAL
    assert f(0, 1, 16, 128, 128, None, None, None, None, None, None, 0, None) == wq.WQ_OK
    assert f(1, 1, 16, 100, 32, ok, ok, ok, ok, ok, None, 0, None) == wq.WQ_EUNSUPPORTED


def test_quantize_scheme_checked_on_host():
    # an unknown scheme, like any other argument error, returns before
    # anything is enqueued
    f = "wq_quantize_groups_ex"
    assert call(f, A, wq.WQ_BF16, 16, 128, 128, 2, None, A, None, A, A, None) == wq.WQ_EINVAL
    assert call(f, A, wq.WQ_BF16, 16, 128, 128, -1, None, A, None, A, A, None) == wq.WQ_EINVAL
    assert call(f, A, wq.WQ_BF16, 16, 100, 32, wq.WQ_SYM, None, A, None, A, A, None) == wq.WQ_EUNSUPPORTED
    assert call(f, B, wq.WQ_BF16, 16, 128, 128, wq.WQ_SYM, None, A, None, A, A, None) == wq.WQ_EALIGN


@pytest.mark.parametrize("N,K,g", [(8192, 8192, 128), (37, 96, 32), (28672, 8192, 32)])
def test_layout_bytes_w8(N, K, g):
    q, s = wq.wq_layout_bytes_w8(N, K, g)
    Np, Kp = (N + 15) // 16 * 16, (K + 127) // 128 * 128
    assert q == Np * Kp and s == 2 * N * (K // g)
    with pytest.raises(wq.WQError):
        wq.wq_layout_bytes_w8(N, K, 64)


def test_w8_entry_points_checked_on_host():
    f = "wq_quantize_w8"
    assert call(f, None, 1, 16, 128, 128, None, A, A, None) == wq.WQ_EINVAL
    assert call(f, A, 1, 16, 128, 128, None, None, A, None) == wq.WQ_EINVAL
    assert call(f, A, 9, 16, 128, 128, None, A, A, None) == wq.WQ_EINVAL
    assert call(f, A, 1, 16, 160, 128, None, A, A, None) == wq.WQ_EUNSUPPORTED
    assert call(f, A, 1, 16, 128, 128, B, A, A, None) == wq.WQ_EALIGN
    assert call(f, A, 1, 16, 128, 128, None, A, B, None) == wq.WQ_EALIGN
    assert call("wq_pack_int8", None, 16, 128, A, None) == wq.WQ_EINVAL
    assert call("wq_pack_int8", A, 0, 128, A, None) == wq.WQ_EINVAL
    assert call("wq_pack_int8", A, 16, 100, A, None) == wq.WQ_EUNSUPPORTED
    assert call("wq_pack_int8", A, 16, 128, B, None) == wq.WQ_EALIGN
    assert call("wq_dequant_w8", A, A, 16, 128, 128, 5, A, None) == wq.WQ_EINVAL
    assert call("wq_dequant_w8", A, A, 16, 128, 48, 0, A, None) == wq.WQ_EUNSUPPORTED
    assert call("wq_dequant_w8", B, A, 16, 128, 128, 0, A, None) == wq.WQ_EALIGN
    g = "wq_gemm_w8a16_ex"
    # no zero-point argument: x, qpacked, s, y, workspace, bytes, path, stream
    assert call(g, 0, 16, 128, 128, A, A, A, A, None, 0, 0, None) == wq.WQ_EINVAL
    assert call(g, 1, 16, 128, 128, A, None, A, A, None, 0, 0, None) == wq.WQ_EINVAL
    assert call(g, 1, 16, 128, 128, A, A, A, A, None, 0, 9, None) == wq.WQ_EINVAL
    assert call(g, 1, 16, 100, 32, A, A, A, A, None, 0, 0, None) == wq.WQ_EUNSUPPORTED
    assert call(g, 1, 16, 128, 128, A, B, A, A, None, 0, 0, None) == wq.WQ_EALIGN
    assert call("wq_gemm_w8a16", 1, 16, 128, 128, B, A, A, A, None, 0, None) == wq.WQ_EALIGN
    # the int8 GEMV runs eight-wave workgroups and may split K further than the
    # 4-bit one: its workspace follows its own launch plan (counter region, then
    # KS fp32 partial-sum planes of MT x 16 per workgroup)
    plan = wq.wq_gemm_w8a16_plan(1, 1024, 8192, 32, wq.WQ_PATH_GEMV)
    gx, gy, ks = (int(v) for v in plan.split("grid=(", 1)[1].split(")", 1)[0].split(","))
    need = wq.WQ_WORKSPACE_COUNTER_BYTES + ks * gy * 1 * gx * 16 * 4
    assert ks > 1 and wq.wq_gemm_w8a16_workspace_bytes(1, 1024, 8192, 32) >= need, plan
    assert call(g, 1, 1024, 8192, 32, A, A, A, A, None, 0, 0, None) == wq.WQ_EWORKSPACE
    assert call(g, 1, 1024, 8192, 32, A, A, A, A, A, need - 1, 0, None) == wq.WQ_EWORKSPACE


def test_w8_plan_names_the_dispatched_kernel():
    d = wq.wq_gemm_w8a16_plan(1, 8192, 8192, 128)
    assert d.startswith("gemv_mfma_kernel<MT=1, W=8, KQ=4, G=128, RB=1, BITS=8>") and "grid=(512,1,1)" in d, d
    d = wq.wq_gemm_w8a16_plan(128, 28672, 8192, 128)
    assert d.startswith("gemm_kernel<MB=8, NPW=2, G=128, BITS=8>") and "grid=(224,1,1)" in d, d
    assert wq.wq_gemm_w8a16_plan(1, 256, 1024, 32, wq.WQ_PATH_MFMA).startswith("gemm_kernel<MB=1, NPW=2, G=32, BITS=8>")


def test_kv_entry_points_checked_on_host():
    c, s, z = wq.wq_kv_layout_bytes(4096, 1024)
    assert (c, s, z) == (4096 * 512, 4096 * 8 * 2, 4096 * 4)
    assert wq.wq_kv_layout_bytes(10, 384)[2] == 10 * 2
    with pytest.raises(wq.WQError) as e:
        wq.wq_kv_layout_bytes(10, 200)
    assert e.value.status == wq.WQ_EUNSUPPORTED
    f = "wq_kv_quantize"
    assert call(f, None, 1, 4, 1024, None, 8, A, A, A, None) == wq.WQ_EINVAL
    assert call(f, A, 1, 4, 1024, None, 8, A, A, None, None) == wq.WQ_EINVAL
    assert call(f, A, 5, 4, 1024, None, 8, A, A, A, None) == wq.WQ_EINVAL
    assert call(f, A, 1, 0, 1024, None, 8, A, A, A, None) == wq.WQ_EINVAL
    assert call(f, A, 1, 4, 1024, None, 0, A, A, A, None) == wq.WQ_EINVAL
    assert call(f, A, 1, 4, 1000, None, 8, A, A, A, None) == wq.WQ_EUNSUPPORTED
    assert call(f, B, 1, 4, 1024, None, 8, A, A, A, None) == wq.WQ_EALIGN
    assert call(f, A, 1, 4, 1024, B, 8, A, A, A, None) == wq.WQ_EALIGN
    g = "wq_kv_dequant"
    assert call(g, A, A, A, 4, 1024, None, 8, 7, A, None) == wq.WQ_EINVAL
    assert call(g, A, A, None, 4, 1024, None, 8, 0, A, None) == wq.WQ_EINVAL
    assert call(g, A, A, A, 4, 96, None, 8, 0, A, None) == wq.WQ_EUNSUPPORTED
    assert call(g, A, A, A, 4, 1024, None, 8, 0, B, None) == wq.WQ_EALIGN


def test_awq_entry_points_checked_on_host():
    f = "wq_quantize_groups_scaled"
    assert call(f, None, 1, 16, 128, 128, 0, A, None, A, None, A, A, None) == wq.WQ_EINVAL
    assert call(f, A, 1, 16, 128, 128, 3, A, None, A, None, A, A, None) == wq.WQ_EINVAL
    assert call(f, A, 1, 16, 100, 32, 0, A, None, A, None, A, A, None) == wq.WQ_EUNSUPPORTED
    assert call(f, A, 1, 16, 128, 128, 0, B, None, A, None, A, A, None) == wq.WQ_EALIGN
    g = "wq_scale_activations"
    assert call(g, None, 4, 128, A, A, None) == wq.WQ_EINVAL
    assert call(g, A, 4, 128, None, A, None) == wq.WQ_EINVAL
    assert call(g, A, 0, 128, A, A, None) == wq.WQ_EINVAL
    assert call(g, A, 4, 100, A, A, None) == wq.WQ_EUNSUPPORTED
    assert call(g, A, 4, 128, B, A, None) == wq.WQ_EALIGN
    h = "wq_channel_absmean"
    assert call(h, None, 4, 128, A, None) == wq.WQ_EINVAL
    assert call(h, A, 4, -1, A, None) == wq.WQ_EINVAL
    assert call(h, A, 4, 128, B, None) == wq.WQ_EALIGN


def test_mxfp4_entry_points_checked_on_host():
    q, e = wq.wq_layout_bytes_mxfp4(8192, 8192)
    assert q == 8192 * 8192 // 2 and e == 8192 * 256
    with pytest.raises(wq.WQError) as err:
        wq.wq_layout_bytes_mxfp4(16, 100)
    assert err.value.status == wq.WQ_EUNSUPPORTED
    f = "wq_quantize_mxfp4"
    assert call(f, None, 1, 16, 128, None, A, A, None) == wq.WQ_EINVAL
    assert call(f, A, 1, 16, 128, None, None, A, None) == wq.WQ_EINVAL
    assert call(f, A, 4, 16, 128, None, A, A, None) == wq.WQ_EINVAL
    assert call(f, A, 1, 16, 100, None, A, A, None) == wq.WQ_EUNSUPPORTED
    assert call(f, B, 1, 16, 128, None, A, A, None) == wq.WQ_EALIGN
    assert call("wq_pack_mxfp4", A, 16, 96 + 4, A, None) == wq.WQ_EUNSUPPORTED
    assert call("wq_pack_mxfp4", A, 16, 128, B, None) == wq.WQ_EALIGN
    assert call("wq_dequant_mxfp4", A, A, 16, 128, 3, A, None) == wq.WQ_EINVAL
    assert call("wq_dequant_mxfp4", A, A, 16, 128, 0, B, None) == wq.WQ_EALIGN
    g = "wq_gemm_mxfp4_ex"
    assert call(g, 1, 16, 128, A, A, None, A, None, 0, 0, None) == wq.WQ_EINVAL  # e8 missing
    assert call(g, 0, 16, 128, A, A, A, A, None, 0, 0, None) == wq.WQ_EINVAL
    assert call(g, 1, 16, 100, A, A, A, A, None, 0, 0, None) == wq.WQ_EUNSUPPORTED
    assert call(g, 1, 16, 128, B, A, A, A, None, 0, 0, None) == wq.WQ_EALIGN
    assert call(g, 1, 16, 128, A, A, A, A, None, 0, 5, None) == wq.WQ_EINVAL
    # a one-row GEMV over K = 28672 splits K, so a missing workspace is refused
    # before anything is launched (the plan is checked first: the call must not
    # reach a launch with these placeholder pointers)
    assert split_k(wq.wq_gemm_mxfp4_plan(1, 1024, 28672)) > 1
    need = wq.wq_gemm_mxfp4_workspace_bytes(1, 1024, 28672)
    assert need > 0 and call(g, 1, 1024, 28672, A, A, A, A, None, 0, 0, None) == wq.WQ_EWORKSPACE
    d = wq.wq_gemm_mxfp4_plan(1, 8192, 8192)
    assert d.startswith("gemv_mfma_kernel<MT=1, W=16, KQ=4, G=32, RB=1, MXFP4>") and "grid=(512,1,1)" in d, d
    d = wq.wq_gemm_mxfp4_plan(128, 28672, 8192)
    assert d.startswith("gemm_kernel<MB=8, NPW=2, G=32, MXFP4>") and "grid=(224,1,1)" in d, d


def test_read_probe_argument_checks():
    # host-only: every rejection happens before a launch, and count == 0
    # enqueues nothing (so fake, aligned pointers are safe here)
    f = wq.lib().wq_read_probe
    A, B = ctypes.c_void_p(1 << 20), ctypes.c_void_p((1 << 20) + 8)
    for nt in (0, 1):
        assert f(A, 1 << 20, 1 << 24, 0, 8, nt, A, None) == wq.WQ_OK
    assert f(None, 1 << 20, 1 << 24, 1, 8, 0, A, None) == wq.WQ_EINVAL
    assert f(A, 1 << 20, 1 << 24, 1, 8, 0, None, None) == wq.WQ_EINVAL
    assert f(A, 0, 1 << 24, 1, 8, 0, A, None) == wq.WQ_EINVAL
    assert f(A, 1000, 1 << 24, 1, 8, 0, A, None) == wq.WQ_EINVAL            # not a multiple of 256
    assert f(A, 1 << 20, (1 << 20) - 256, 1, 8, 0, A, None) == wq.WQ_EINVAL  # span smaller than a window
    assert f(A, 1 << 20, 1 << 24, -1, 8, 0, A, None) == wq.WQ_EINVAL
    for chunks in (0, 3, 5, 32):
        assert f(A, 1 << 20, 1 << 24, 1, chunks, 0, A, None) == wq.WQ_EINVAL
    assert f(A, 1 << 20, 1 << 24, 1, 8, 2, A, None) == wq.WQ_EINVAL
    assert f(B, 1 << 20, 1 << 24, 1, 8, 0, A, None) == wq.WQ_EALIGN
    assert f(A, 1 << 20, 1 << 24, 1, 8, 0, ctypes.c_void_p((1 << 20) + 2), None) == wq.WQ_EALIGN


def test_binding_rejects_bad_activations_and_outputs():
    """The Python binding checks x (contiguous fp16 [M][K] on the weights'
    device) and a caller-given y (contiguous fp16 [M][N]) before any C call:
    a wrong dtype or shape would otherwise be read as fp16 bits or written out
    of bounds."""
    import torch
    N, K, g = 32, 256, 128
    qb, sb, zb = wq.wq_layout_bytes(N, K, g)
    qw = wq.QuantizedWeight(torch.zeros(qb, dtype=torch.uint8), torch.zeros((N, K // g), dtype=torch.float16),
                            torch.zeros((N, zb // N), dtype=torch.uint8), N, K, g)
    x = torch.zeros((3, K), dtype=torch.float16)
    with pytest.raises(ValueError, match="float16"):
        wq.wq_gemm_w4a16(x.float(), qw)
    with pytest.raises(ValueError, match="contiguous"):
        wq.wq_gemm_w4a16(torch.zeros((K, 3), dtype=torch.float16).t(), qw)
    with pytest.raises(ValueError, match="K=128"):
        wq.wq_gemm_w4a16(torch.zeros((3, 128), dtype=torch.float16), qw)
    with pytest.raises(ValueError, match=r"\[3\]\[32\]"):
        wq.wq_gemm_w4a16(x, qw, y=torch.zeros((3, 16), dtype=torch.float16))
    with pytest.raises(ValueError, match=r"\[3\]\[32\]"):
        wq.wq_gemm_w4a16(x, qw, y=torch.zeros((3, 32), dtype=torch.float32))
    q8 = wq.QuantizedWeight8(torch.zeros(N * K * 2, dtype=torch.uint8), torch.zeros((N, K // g), dtype=torch.float16),
                             N, K, g)
    with pytest.raises(ValueError):
        wq.wq_gemm_w8a16(x.to(torch.bfloat16), q8)
    qm = wq.QuantizedWeightMX(torch.zeros(qb, dtype=torch.uint8), torch.zeros((N, K // 32), dtype=torch.uint8), N, K)
    with pytest.raises(ValueError):
        wq.wq_gemm_mxfp4(x, qm, y=torch.zeros((2, 32), dtype=torch.float16))


def test_nvfp4_entry_points_checked_on_host():
    # layout sizes: MXFP4 tiles, one scale byte per 16 values
    qb, sb = wq.wq_layout_bytes_nvfp4(100, 1152)
    assert (qb, sb) == (112 * 1152 // 2, 100 * 72)
    g = "wq_gemm_nvfp4_ex"
    # K a multiple of 32; the tensor scale and the scale bytes are required
    assert call(g, 4, 64, 48, A, A, A, A, A, None, 0, 0, None) == wq.WQ_EUNSUPPORTED
    assert call(g, 4, 64, 256, A, A, A, None, A, None, 0, 0, None) == wq.WQ_EINVAL
    assert call(g, 4, 64, 256, A, A, None, A, A, None, 0, 0, None) == wq.WQ_EINVAL
    assert call(g, 4, 64, 256, A, A, A, B, A, None, 0, 0, None) == wq.WQ_EALIGN
    assert call("wq_quantize_nvfp4", A, wq.WQ_F32, 64, 256, None, A, None, None, None) == wq.WQ_EINVAL
    assert call("wq_quantize_nvfp4", A, wq.WQ_F32, 64, 80, None, A, A, None, None) == wq.WQ_EUNSUPPORTED
    assert call("wq_dequant_nvfp4", A, A, None, 64, 256, wq.WQ_F32, A, None) == wq.WQ_EINVAL
    # plans: the matrix-core GEMV up to WQ_AUTO_FP4_GEMV_MAX_M rows, the GEMM past it
    hi = wq.WQ_AUTO_FP4_GEMV_MAX_M
    assert wq.wq_gemm_nvfp4_plan(1, 8192, 8192).startswith("gemv_mfma_kernel<MT=1, W=16, KQ=4, G=16, RB=1, NVFP4>")
    assert wq.wq_gemm_nvfp4_plan(4, 8192, 8192).startswith("gemv_mfma_kernel<MT=4, W=8, KQ=4, G=16, RB=1, NVFP4>")
    assert wq.wq_gemm_nvfp4_plan(hi, 8192, 8192).startswith("gemv_mfma_kernel<MT=16, W=8, KQ=4, G=16, RB=2, NVFP4>")
    assert wq.wq_gemm_nvfp4_plan(hi + 1, 8192, 8192).startswith("gemm_kernel<MB=2, NPW=2, G=16, NVFP4>")
    # the workspace query covers the format's own plans
    for M, N, K in [(1, 1024, 28672), (8, 1024, 8192), (128, 48, 28672)]:
        need = wq.wq_gemm_nvfp4_workspace_bytes(M, N, K)
        for path in (wq.WQ_PATH_GEMV, wq.WQ_PATH_MFMA):
            plan = wq.wq_gemm_nvfp4_plan(M, N, K, path)
            if split_k(plan) > 1:
                assert need > 0, (M, N, K, plan)

