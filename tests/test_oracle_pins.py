"""Pins of the CPU oracle against what the pages and mathematics fix.

These tests never touch the HIP library.  Each one checks the oracle against
something other than itself: numbers printed on the pages (fixtures under
tests/golden/, each with its citation), exact rational arithmetic, an
independent library conversion, or an invariant that a dropped term, a wrong
sign, a wrong index or a transposed operand would break.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import golden
import workloads


# --------------------------------------------------------------------------
# The 8-weight INT4 worked example (quantization post, "Numerical example")
# --------------------------------------------------------------------------

def _example(orc, pad_to=None):
    w = np.array(workloads.WORKED_EXAMPLE_W, np.float32)
    if pad_to:
        w = np.concatenate([w, np.zeros(pad_to - w.size, np.float32)])
    q, s, z = orc.quantize_groups(w[None, :], w.size)
    return w, q[0], s[0, 0], z[0, 0]


def test_worked_example_codes_scale_zero(orc):
    g = golden("int4_worked_example.json")["printed"]
    w, q, s_bits, z = _example(orc)
    assert list(q) == g["q"] == g["round"]
    assert z == g["z"]
    s = float(np.uint16(s_bits).view(np.float16))
    assert round(s, g["s_decimals"]) == g["s"]
    # the real-valued zero-point printed before rounding: -min/s
    assert abs(-g["min"] / s - g["z_real"]) < 0.005
    assert abs((g["max"] - g["min"]) - g["range"]) < 1e-12


def test_worked_example_dequant_error_mse(orc):
    g = golden("int4_worked_example.json")["printed"]
    w, q, s_bits, z = _example(orc)
    w_hat = orc.dequant(q[None], np.array([[s_bits]], np.uint16), np.array([[z]], np.uint8), 8)[0]
    tol = 10.0 ** -g["decimals"]  # printed to 3 decimals (the page rounds s to 0.1553)
    assert np.all(np.abs(w_hat - np.array(g["w_hat"])) <= tol)
    err = w_hat.astype(np.float64) - w.astype(np.float64)
    assert np.all(np.abs(err - np.array(g["error"])) <= tol)
    mse = float(np.mean(err ** 2))
    assert round(mse, 4) == g["mse_approx"]


def test_worked_example_encode_column(orc):
    """The printed w/s+z column agrees with the oracle's stored scale to the
    printed precision, except the one misprinted entry, which still encodes to 0."""
    g = golden("int4_worked_example.json")["printed"]
    w, q, s_bits, z = _example(orc)
    s = np.float32(np.uint16(s_bits).view(np.float16))
    t = (w / s + np.float32(z)).astype(np.float64)
    printed = np.array(g["w_over_s_plus_z"])
    ok = np.abs(t - printed) <= 0.01
    assert list(np.nonzero(~ok)[0]) == [5]
    assert q[5] == 0 and t[5] > 0


@pytest.mark.parametrize("group", [32, 128])
def test_worked_example_padded_to_real_group(orc, group):
    """Zero padding to a real group size keeps min, max, s and z; pads get code z."""
    _, q8, s8, z8 = _example(orc)
    _, q, s, z = _example(orc, pad_to=group)
    assert s == s8 and z == z8
    assert list(q[:8]) == list(q8)
    assert np.all(q[8:] == z8)


def test_worked_example_storage(orc):
    g = golden("int4_worked_example.json")["printed"]
    parts = g["storage_parts_bytes"]
    n = len(g["q"])
    b = orc.storage_bytes(n, 4, n, scale_bits=16, zero_bits=4)
    assert b == parts["codes"] + parts["scale_bf16"] + parts["zero_int4"] == g["storage_bytes_quantized_approx"]
    assert round(g["storage_bytes_bf16_weights"] / b, 1) == g["reduction_factor_approx"]


# --------------------------------------------------------------------------
# Bits per weight (Cruxly lesson, granularity and memory arithmetic)
# --------------------------------------------------------------------------

def test_bits_per_weight(orc):
    g = golden("bits_per_weight.json")["printed"]
    b128 = orc.bits_per_weight(4, 128, 16, 0)
    b32 = orc.bits_per_weight(4, 32, 16, 0)
    assert b128 == g["g128_bits"] and b32 == g["g32_bits"]
    assert round(g["params_70b"] * b128 / 8 / 1e9, g["gb_decimals"]) == g["g128_gb"]
    assert round(g["params_70b"] * b32 / 8 / 1e9, g["gb_decimals"]) == g["g32_gb"]
    # storage of the 70B model computed by groups agrees with bits/weight
    assert orc.storage_bytes(int(g["params_70b"]), 4, 128, 16, 0) == pytest.approx(g["params_70b"] * b128 / 8)
    # counting the 4-bit zero-point as well (what this library stores)
    assert orc.bits_per_weight(4, 128, 16, 4) == 4.15625
    assert orc.bits_per_weight(4, 32, 16, 4) == 4.625


# --------------------------------------------------------------------------
# Symmetric quantizers (absmax int8 and +-7 INT4)
# --------------------------------------------------------------------------

def test_absmax_int8_example(orc):
    g = golden("int8_absmax_example.json")
    w = np.array(g["w"])
    q, s, w_hat = orc.symmetric(w, 8)
    assert s == pytest.approx(np.max(np.abs(w)) / g["printed"]["qmax"], rel=0, abs=0)
    assert list(q) == [17, -71, 47, 127]
    rel = np.abs(w_hat - w) / np.abs(w)
    assert rel.max() < 0.01  # the page: error below one percent
    w2 = np.concatenate([w, [g["outlier"]]])
    q2, s2, w_hat2 = orc.symmetric(w2, 8)
    assert round(s2, 4) == g["printed"]["s_with_outlier"]
    assert s2 == 20.0 / 127.0
    assert q2[-1] == 127
    rel2 = abs(w_hat2[0] - w2[0]) / abs(w2[0])
    assert round(100 * rel2) == g["printed"]["relative_error_with_outlier_percent"]


def test_symmetric_int4_outlier(orc):
    g = golden("symmetric_int4_outlier.json")
    rng = np.random.default_rng(7)
    for case in g["cases"]:
        M = case["M"]
        w = np.concatenate([rng.uniform(-M, M, 63), [M]])
        q, s, w_hat = orc.symmetric(w, g["bits"])
        assert s == M / g["levels"]
        assert round(s, 2 if M > 2 else 3) == case["s_approx"]
        assert round(s / 2, 2 if M > 2 else 3) == case["half_step_approx"]
        assert round(100 * s / 2) == case["relative_error_of_unit_value_percent"]
        assert np.all(np.abs(q) <= g["levels"])
        assert np.all(np.abs(w - w_hat) <= s / 2 * (1 + 1e-12))


def _sym(orc, w, group, dtype=None):
    w = np.ascontiguousarray(w, np.float32)
    if w.ndim == 1:
        w = w[None, :]
    q, s, z = orc.quantize_groups(w, group, dtype=dtype, scheme=orc.SYM)
    return q, s, z


def test_symmetric_groups_printed_outlier_numbers(orc):
    # The same page's INT4 calculation through the group quantizer with an fp16
    # scale: a group holding the outlier 30.0 and values of magnitude about 1,
    # and the same values with the outlier removed (M = 1).
    g = golden("symmetric_int4_outlier.json")
    rng = np.random.default_rng(11)
    for case, group in [(c, grp) for c in g["cases"] for grp in (32, 128)]:
        M = case["M"]
        w = np.concatenate([[M], rng.uniform(-1.0, 1.0, group - 1)]).astype(np.float32)
        if M < 2:
            w = np.clip(w, -1.0, 1.0)
            w[0] = 1.0
        q, s, z = _sym(orc, w, group)
        sh = float(orc.f16_bits_to_f32(s)[0])
        assert z[0, 0] == 8
        assert round(sh, 2 if M > 2 else 3) == case["s_approx"]
        assert round(sh / 2, 2 if M > 2 else 3) == case["half_step_approx"]
        w_hat = sh * (q[0].astype(np.float64) - 8)
        # the half-step bound, widened by the fp16 rounding of the scale
        s32 = np.float32(np.float32(M) / np.float32(7.0))
        bound = sh / 2 + 7 * abs(float(s32) - sh)
        assert np.all(np.abs(w - w_hat) <= bound * (1 + 1e-7))
        # the outlier itself is the top code
        assert q[0, 0] == 15


def test_symmetric_groups_equal_textbook_when_scale_is_exact(orc):
    # When max|w| = 7 * 2^e the scale 2^e is exact in fp32 and fp16, so the
    # fp32 steps reduce to the fp64 textbook rule q = round(w / s) (its own
    # implementation in orc.symmetric), codes offset by the zero-point 8.
    rng = np.random.default_rng(12)
    for e in (-9, -4, 0, 3):
        for group in (32, 128):
            w = rng.uniform(-7.0, 7.0, (6, group)) * 2.0 ** e
            w[:, 0] = 7.0 * 2.0 ** e * np.where(np.arange(6) % 2, 1, -1)
            w = w.astype(np.float32)
            q, s, z = _sym(orc, w, group)
            for r in range(6):
                qt, st, wt = orc.symmetric(w[r].astype(np.float64), 4)
                assert st == 2.0 ** e
                assert orc.f16_bits_to_f32(s[r])[0] == 2.0 ** e
                assert np.array_equal(q[r].astype(np.int64) - 8, qt)
                assert np.array_equal(st * (q[r].astype(np.float64) - 8), wt)


def test_symmetric_groups_invariants_ties_and_degenerate(orc):
    rng = np.random.default_rng(13)
    W = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    W[:, 5] *= 20  # an outlier channel
    for group in (32, 128):
        q, s, z = _sym(orc, W, group)
        assert np.all(z == 8) and q.min() >= 1 and q.max() <= 15
        sh = orc.f16_bits_to_f32(s.ravel()).reshape(s.shape).astype(np.float64)
        w_hat = np.repeat(sh, group, axis=1) * (q.astype(np.float64) - 8)
        amax = np.abs(W.reshape(8, -1, group)).max(axis=2)
        s32 = (amax.astype(np.float32) / np.float32(7.0)).astype(np.float64)
        bound = np.repeat(sh / 2 + 7 * np.abs(s32 - sh), group, axis=1)
        assert np.all(np.abs(W - w_hat) <= bound * (1 + 1e-7))
        # negating the weights negates the symmetric codes
        qn, sn, _ = _sym(orc, -W, group)
        assert np.array_equal(sn, s) and np.array_equal(qn.astype(int) - 8, -(q.astype(int) - 8))
    # exact halves round to even: s = 1 (max |w| = 7), w = k + 0.5
    w = np.array([7.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5] + [0.0] * 24, np.float32)
    q, s, z = _sym(orc, w, 32)
    assert list(q[0, :8].astype(int) - 8) == [7, 0, 2, 2, 0, -2, -2, 4]
    # an all-zero group: scale 0, zero-point 8, every code 8 (decodes to 0)
    q, s, z = _sym(orc, np.zeros(32, np.float32), 32)
    assert s[0, 0] == 0 and z[0, 0] == 8 and np.all(q == 8)
    # bf16 input is widened exactly: same result as its fp32 value
    Wb = orc.f32_to_bf16_bits(W)
    qb, sb, zb = orc.quantize_groups(Wb, 32, dtype=orc.BF16, scheme=orc.SYM)
    W32 = (Wb.astype(np.uint32) << 16).view(np.float32)
    q2, s2, z2 = _sym(orc, W32, 32)
    assert np.array_equal(qb, q2) and np.array_equal(sb, s2)


# --------------------------------------------------------------------------
# Group absmax int8 (W8A16): the same page's int8 rule with an fp16 scale per
# group of 32 or 128 weights
# --------------------------------------------------------------------------

def _w8(orc, w, group, dtype=None):
    w = np.ascontiguousarray(w, np.float32)
    if w.ndim == 1:
        w = w[None, :]
    return orc.quantize_w8(w, group, dtype=dtype)


@pytest.mark.parametrize("group", [32, 128])
def test_w8_groups_printed_example(orc, group):
    # The four printed weights, and the same with the outlier 20.0 appended,
    # padded with zeros to a whole group (zeros change neither max|w| nor the
    # other codes).
    g = golden("int8_absmax_example.json")
    w = np.zeros(group, np.float32)
    w[:4] = g["w"]
    q, s = _w8(orc, w, group)
    sh = float(orc.f16_bits_to_f32(s)[0])
    assert list(q[0, :4]) == [17, -71, 47, 127] and np.all(q[0, 4:] == 0)
    w_hat = sh * q[0, :4].astype(np.float64)
    assert np.max(np.abs(w_hat - w[:4]) / np.abs(w[:4])) < 0.01  # below one percent
    w[4] = g["outlier"]
    q, s = _w8(orc, w, group)
    sh = float(orc.f16_bits_to_f32(s)[0])
    assert round(sh, 4) == g["printed"]["s_with_outlier"]
    assert list(q[0, :5]) == [1, -3, 2, 6, 127]
    assert round(100 * abs(sh * 1 - w[0]) / w[0]) == g["printed"]["relative_error_with_outlier_percent"]


def test_w8_groups_equal_textbook_when_scale_is_exact(orc):
    # max|w| = 127 * 2^e makes s = 2^e exact in fp32 and fp16: the fp32 steps
    # reduce to the fp64 textbook rule (orc.symmetric at 8 bits).
    rng = np.random.default_rng(21)
    for e in (-12, -7, 0, 2):
        for group in (32, 128):
            w = rng.uniform(-127.0, 127.0, (6, group)) * 2.0 ** e
            w[:, 3] = 127.0 * 2.0 ** e * np.where(np.arange(6) % 2, 1, -1)
            w = w.astype(np.float32)
            q, s = _w8(orc, w, group)
            for r in range(6):
                qt, st, wt = orc.symmetric(w[r].astype(np.float64), 8)
                assert st == 2.0 ** e
                assert orc.f16_bits_to_f32(s[r])[0] == 2.0 ** e
                assert np.array_equal(q[r].astype(np.int64), qt)
                assert np.array_equal(st * q[r].astype(np.float64), wt)


def test_w8_groups_invariants(orc):
    rng = np.random.default_rng(22)
    W = (rng.standard_normal((8, 512)) * 0.02).astype(np.float32)
    W[:, 17] *= 20  # an outlier channel
    for group in (32, 128):
        q, s = _w8(orc, W, group)
        sh = orc.f16_bits_to_f32(s.ravel()).reshape(s.shape).astype(np.float64)
        assert q.min() >= -127 and q.max() <= 127
        # half-step bound, widened by the fp16 rounding of the scale
        amax = np.abs(W.reshape(8, -1, group)).max(axis=2)
        s32 = (amax.astype(np.float32) / np.float32(127.0)).astype(np.float64)
        bound = np.repeat(sh / 2 + 127 * np.abs(s32 - sh), group, axis=1)
        w_hat = np.repeat(sh, group, axis=1) * q.astype(np.float64)
        assert np.all(np.abs(W - w_hat) <= bound * (1 + 1e-7))
        # every group's largest magnitude gets the top code
        Wg, qg = W.reshape(8, -1, group), q.reshape(8, -1, group).astype(int)
        top = np.take_along_axis(qg, np.abs(Wg).argmax(axis=2)[..., None], axis=2)[..., 0]
        assert np.all(np.abs(top) == 127)
        # codes keep the order of the weights inside a group, and the sign
        order = np.argsort(Wg, axis=2, kind="stable")
        assert np.all(np.diff(np.take_along_axis(qg, order, axis=2), axis=2) >= 0)
        assert np.all(np.sign(qg) * np.sign(Wg) >= 0)
        # negating the weights negates the codes; scales unchanged
        qn, sn = _w8(orc, -W, group)
        assert np.array_equal(sn, s) and np.array_equal(qn.astype(int), -q.astype(int))
        # re-quantizing the decoded weights returns the same codes and scales
        q2, s2 = _w8(orc, orc.dequant_w8(q, s, group), group)
        assert np.array_equal(q2, q) and np.array_equal(s2, s)


def test_w8_ties_degenerate_and_input_dtypes(orc):
    # exact halves round to even: s = 1 (max |w| = 127), w = k + 0.5
    w = np.array([127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5] + [0.0] * 24, np.float32)
    q, s = _w8(orc, w, 32)
    assert orc.f16_bits_to_f32(s)[0] == 1.0
    assert list(q[0, :8]) == [127, 0, 2, 2, 0, -2, -2, 126]
    # all-zero group: scale 0, codes 0; a tiny group whose scale underflows fp16
    q, s = _w8(orc, np.zeros(32, np.float32), 32)
    assert s[0, 0] == 0 and np.all(q == 0)
    tiny = np.full(32, 2.0 ** -40, np.float32)
    q, s = _w8(orc, tiny, 32)
    assert s[0, 0] == 0 and np.all(q == 0)
    # a non-finite weight, or a scale past fp16's range, is an error
    with pytest.raises(orc.OracleError):
        _w8(orc, np.array([np.inf] + [0.0] * 31, np.float32), 32)
    with pytest.raises(orc.OracleError):
        _w8(orc, np.array([127.0 * 70000.0] + [0.0] * 31, np.float32), 32)
    # bf16 and fp16 inputs are widened exactly
    rng = np.random.default_rng(23)
    W = (rng.standard_normal((4, 256)) * 0.02).astype(np.float32)
    Wb = orc.f32_to_bf16_bits(W)
    qb, sb = orc.quantize_w8(Wb, 128, dtype=orc.BF16)
    q2, s2 = _w8(orc, (Wb.astype(np.uint32) << 16).view(np.float32), 128)
    assert np.array_equal(qb, q2) and np.array_equal(sb, s2)
    Wh = W.astype(np.float16)
    qh, sh = orc.quantize_w8(Wh.view(np.uint16), 128, dtype=orc.F16)
    q3, s3 = _w8(orc, Wh.astype(np.float32), 128)
    assert np.array_equal(qh, q3) and np.array_equal(sh, s3)


def test_w8_dequant_exact_all_codes(orc):
    rng = np.random.default_rng(24)
    scales = np.concatenate([
        np.array([0x0001, 0x0155, 0x03FF, 0x0400, 0x1F42, 0x3C00, 0x7BFF], np.uint16),
        rng.integers(0x0001, 0x7C00, 25).astype(np.uint16),
    ])
    codes = np.arange(-127, 128, dtype=np.int8)
    q = np.tile(codes, (scales.size, 1))
    s = scales[:, None].copy()
    f32 = orc.dequant_w8(q, s, codes.size, orc.F32)
    f16 = orc.dequant_w8(q, s, codes.size, orc.F16)
    b16 = orc.dequant_w8(q, s, codes.size, orc.BF16)
    exact = np.array([[float(Fraction(float(np.uint16(sv).view(np.float16))) * int(c)) for c in codes]
                      for sv in scales])
    assert np.array_equal(f32.astype(np.float64), exact)  # exact in fp32
    with np.errstate(over="ignore"):  # 65504 * 127 rounds to fp16 infinity
        assert np.array_equal(f16, exact.astype(np.float16).view(np.uint16))
    ref_b = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b16, ref_b)


def test_w8_pack_device_is_a_bijection_and_byte_order(orc):
    for N, K in [(16, 128), (37, 96), (5, 416)]:
        nbytes = orc.device_bytes_w8(N, K)
        assert nbytes == ((N + 15) // 16 * 16) * ((K + 127) // 128 * 128)
        seen = np.zeros(nbytes, np.int64)
        for n in range(N):
            q = np.zeros((N, K), np.int8)
            q[n, :] = 1
            p = orc.pack_device_w8(q)
            assert p.sum() == K
            seen += p
        assert seen.max() == 1 and seen.sum() == N * K
        rng = np.random.default_rng(N + K)
        q = rng.integers(-127, 128, (N, K)).astype(np.int8)
        assert np.array_equal(orc.unpack_device_w8(orc.pack_device_w8(q), N, K), q)
    # hand-placed elements: row 3, columns 40..47 (MFMA step 1 -> half 0, second
    # eight bytes; column block c = 1 -> lane 19); row 0, column 100 (step 3 ->
    # half 1, second eight bytes, c = 0, e = 4); row 17, column 130 (second row
    # block, second K tile: tile 1 * 2 + 1 = 3, step 0, lane 1, e = 2)
    q = np.zeros((32, 256), np.int8)
    q[3, 40:48] = -5
    q[0, 100] = 77
    q[17, 130] = -128 + 1
    p = orc.pack_device_w8(q)
    assert np.all(p[16 * 19 + 8: 16 * 19 + 16] == np.uint8(251))
    assert p[1024 + 8 + 4] == 77
    assert p[3 * 2048 + 16 * 1 + 2] == np.uint8(129)
    assert np.count_nonzero(p) == 10


def test_w8_gemm_rows(orc):
    rng = np.random.default_rng(25)
    M, N, K, g = 3, 40, 256, 32
    W = rng.standard_normal((N, K)).astype(np.float32) * 0.02
    x = workloads.f32_to_f16_bits(rng.standard_normal((M, K)).astype(np.float32))
    q, s = orc.quantize_w8(W, g)
    w_hat = orc.dequant_w8(q, s, g)
    y = orc.gemm_f64(x, w_hat)
    assert np.array_equal(orc.gemm_rows_w8_f64(x, q, s, g, 10, 17), y[:, 10:27])
    # a one-hot activation row selects one decoded weight per output
    xo = np.zeros((1, K), np.float32)
    xo[0, 77] = 1.0
    yo = orc.gemm_rows_w8_f64(workloads.f32_to_f16_bits(xo), q, s, g, 0, N)
    assert np.array_equal(yo[0], w_hat[:, 77].astype(np.float64))


# --------------------------------------------------------------------------
# INT4 KV cache in blocks of 128 (quantization post, "KV cache quantization")
# --------------------------------------------------------------------------

def test_kv_block_holds_the_printed_example():
    # the page's 8 weights padded to one block of 128, placed as block 3 of a
    # token vector of 8 heads x 128: codes, scale and zero-point as printed
    import oracle as orc
    g = golden("int4_worked_example.json")
    X = (np.random.default_rng(40).standard_normal((3, 1024)) * 0.5).astype(np.float32)
    X[1, 384:512] = 0.0
    X[1, 384:392] = workloads.WORKED_EXAMPLE_W
    cache = orc.kv_alloc(3, 1024)
    orc.kv_quantize(X, cache)
    codes, s, z = cache
    assert round(float(orc.f16_bits_to_f32(s[1, 3:4])[0]), g["printed"]["s_decimals"]) == g["printed"]["s"]
    assert (z[1, 1] & 15) == g["printed"]["z"]
    x_hat = orc.kv_dequant(cache, 3, 1024)
    w_hat = x_hat[1, 384:392]
    assert np.allclose(w_hat, g["printed"]["w_hat"], atol=1e-3, rtol=0)
    # the block's codes, read back through the documented nibble positions
    word = int(codes[1, 3 * 64: 3 * 64 + 4].view(np.uint32)[0])
    got = [(word >> (4 * (4 * (e % 2) + e // 2))) & 15 for e in range(8)]
    assert got == g["printed"]["q"]


def test_kv_storage_per_value():
    # half a byte per value plus the per-block scale and zero-point
    import oracle as orc
    hd = 1024
    codes, s, z = orc.kv_alloc(1, hd)
    per_value = (codes.nbytes + s.nbytes + z.nbytes) / hd
    assert per_value == 0.5 + 2.5 / 128
    assert round(2 / per_value, 2) == 3.85  # against a 2-byte fp16/bf16 cache


def test_kv_blocks_invariants_and_bound():
    import oracle as orc
    rng = np.random.default_rng(41)
    T, hd = 16, 1024
    X = (rng.standard_normal((T, hd)) * 2.0).astype(np.float32)
    X[:, 77] *= 30  # an outlier channel in every token
    cache = orc.kv_alloc(T, hd)
    orc.kv_quantize(X, cache)
    codes, s, z = cache
    sh = orc.f16_bits_to_f32(s.ravel()).reshape(s.shape).astype(np.float64)
    x_hat = orc.kv_dequant(cache, T, hd).astype(np.float64)
    Xb = X.reshape(T, hd // 128, 128).astype(np.float64)
    lo = np.minimum(Xb.min(axis=2), 0)
    hi = np.maximum(Xb.max(axis=2), 0)
    s32 = ((hi - lo).astype(np.float32) / np.float32(15)).astype(np.float64)
    bound = sh / 2 + 15 * np.abs(s32 - sh)
    err = np.abs(x_hat.reshape(T, hd // 128, 128) - Xb).max(axis=2)
    assert np.all(err <= bound * (1 + 1e-6))
    # each block's zero-point decodes to exactly zero and lies in [0, 15]
    zz = np.stack([z & 15, z >> 4], axis=2).reshape(T, -1)[:, :hd // 128]
    assert zz.max() <= 15
    # blocks are independent: changing one block leaves every other one alone
    X2 = X.copy()
    X2[5, 300] = 100.0
    c2 = orc.kv_alloc(T, hd)
    orc.kv_quantize(X2, c2)
    diff_s = np.argwhere(c2[1] != s)
    assert all(tuple(d) == (5, 2) for d in diff_s) and len(diff_s) == 1


def test_kv_slots_scatter_skip_and_keep():
    import oracle as orc
    rng = np.random.default_rng(42)
    T, hd, S = 6, 256, 10
    X = rng.standard_normal((T, hd)).astype(np.float32)
    ref = orc.kv_alloc(T, hd)
    orc.kv_quantize(X, ref)
    cache = orc.kv_alloc(S, hd)
    for a in cache:
        a[...] = 0xAB if a.dtype == np.uint8 else 0x1234  # previous contents
    slots = np.array([7, 2, -1, 9, 10, 0], np.int32)  # -1 and 10 are outside the cache
    orc.kv_quantize(X, cache, slot=slots)
    for t, row in enumerate(slots):
        if 0 <= row < S:
            for a, b in zip(cache, ref):
                assert np.array_equal(a[row], b[t])
    for row in (1, 3, 4, 5, 6, 8):  # untouched rows keep their contents
        assert np.all(cache[0][row] == 0xAB) and np.all(cache[1][row] == 0x1234)
    got = orc.kv_dequant(cache, T, hd, slot=slots)
    assert np.all(got[2] == 0) and np.all(got[4] == 0)
    assert np.array_equal(got[0], orc.kv_dequant(ref, T, hd)[0])


def test_kv_odd_block_count_and_grid_exact_values():
    # hd = 384 (three blocks: the third zero-point alone in its byte); values
    # of the form 2^-4 * (c - z0) with codes 0 and 15 in every block decode
    # exactly
    import oracle as orc
    rng = np.random.default_rng(43)
    T, hd = 5, 384
    c = rng.integers(0, 16, (T, hd))
    c[:, ::128] = 0
    c[:, 1::128] = 15
    z0 = rng.integers(1, 15, (T, hd // 128))
    X = (np.ldexp(1.0, -4) * (c - np.repeat(z0, 128, axis=1))).astype(np.float32)
    cache = orc.kv_alloc(T, hd)
    orc.kv_quantize(X, cache)
    assert np.array_equal(orc.kv_dequant(cache, T, hd), X)
    assert np.all((cache[2][:, 1] >> 4) == 0)
    zz = np.stack([cache[2][:, 0] & 15, cache[2][:, 0] >> 4, cache[2][:, 1] & 15], axis=1)
    assert np.array_equal(zz, z0)


# --------------------------------------------------------------------------
# AWQ-style per-input-channel scaling (quantization post "AWQ"; methods page,
# the symmetric int4 example by hand)
# --------------------------------------------------------------------------

def test_awq_toy_example(orc):
    g = golden("awq_toy_example.json")
    w = np.array([g["w"]], np.float32)
    x = np.array(g["x"], np.float64)
    c = g["salient_channel"]
    assert x[c] / np.delete(x, c).max() == g["printed"]["salient_activation_ratio"]

    def run(f):
        a = np.ones(4, np.float32)
        a[c] = f
        q, s, z = orc.quantize_groups(w, 4, scheme=orc.SYM, alpha=a)
        sh = float(orc.f16_bits_to_f32(s)[0])
        w_eff = sh * (q[0].astype(np.float64) - 8) / a  # the layer's effective weights (x / alpha times W' hat)
        return q[0].astype(int) - 8, sh, w_eff

    q1, s1, w1 = run(1.0)
    assert np.all(np.abs(q1) <= g["levels"])
    y_err_plain = abs(x @ w1 - x @ w[0].astype(np.float64))
    for f in (1.5, 2.0, 3.0, 4.0):  # factors that keep f * |w_c| below the group's max |w|
        qf, sf, wf = run(f)
        assert sf == s1  # same scale ...
        assert np.array_equal(np.delete(qf, c), np.delete(q1, c))  # ... so the other channels' rounding is unchanged
        assert np.array_equal(np.delete(wf, c), np.delete(w1, c))
        assert abs(wf[c] - w[0, c]) < abs(w1[c] - w[0, c])  # the salient channel is kept more finely
        assert abs(wf[c] - w[0, c]) <= sf / (2 * f) * (1 + 1e-6)
        assert abs(x @ wf - x @ w[0].astype(np.float64)) < y_err_plain
    # past max|w| / |w_c| the scaled weight raises the group maximum: a larger scale
    # for every channel, so the other channels' rounding changes
    q5, s5, w5 = run(5.0)
    assert s5 > s1 and not np.array_equal(np.delete(w5, c), np.delete(w1, c))


def test_awq_fold_identities(orc):
    rng = np.random.default_rng(50)
    W = (rng.standard_normal((12, 256)) * 0.02).astype(np.float32)
    for group in (32, 128):
        plain = orc.quantize_groups(W, group)
        # alpha = 1 is no fold at all
        assert all(np.array_equal(a, b) for a, b in zip(orc.quantize_groups(W, group, alpha=np.ones(256)), plain))
        # a power of two on every channel commutes with the quantizer: same
        # codes and zero-points, scales times that power (exact in fp16)
        for e in (-3, 2):
            q, s, z = orc.quantize_groups(W, group, alpha=np.full(256, 2.0 ** e, np.float32))
            assert np.array_equal(q, plain[0]) and np.array_equal(z, plain[2])
            assert np.array_equal(orc.f16_bits_to_f32(s.ravel()), orc.f16_bits_to_f32(plain[1].ravel()) * 2.0 ** e)
    # the fold multiplies before quantizing: W diag(alpha) through the plain quantizer
    alpha = rng.uniform(0.5, 3.0, 256).astype(np.float32)
    Wa = (W * alpha[None, :]).astype(np.float32)
    assert all(np.array_equal(a, b) for a, b in zip(orc.quantize_groups(W, 32, alpha=alpha),
                                                     orc.quantize_groups(Wa, 32)))


def test_awq_activation_side_and_statistic(orc):
    rng = np.random.default_rng(51)
    M, K = 9, 384
    x = workloads.f32_to_f16_bits(rng.standard_normal((M, K)).astype(np.float32) * 3)
    alpha = rng.uniform(0.3, 5.0, K).astype(np.float32)
    xf = x.view(np.float16).astype(np.float32)
    want = (xf / alpha[None, :]).astype(np.float32).astype(np.float16).view(np.uint16)
    assert np.array_equal(orc.scale_activations(x, alpha), want)
    p2 = (2.0 ** rng.integers(-2, 3, K)).astype(np.float32)  # powers of two: exact
    assert np.array_equal(orc.scale_activations(x, p2).view(np.float16).astype(np.float64),
                          xf.astype(np.float64) / p2[None, :])
    # the statistic: fp32 sum of |x| in row order, then / M
    acc = np.zeros(K, np.float32)
    for m in range(M):
        acc = (acc + np.abs(xf[m])).astype(np.float32)
    assert np.array_equal(orc.channel_absmean(x), (acc / np.float32(M)).astype(np.float32))
    # the maths cancels: with power-of-two factors, x' (W diag(alpha))^T = x W^T exactly
    W = rng.standard_normal((5, K)).astype(np.float32)
    xs = orc.scale_activations(x, p2)
    y1 = orc.gemm_f64(xs, (W * p2[None, :]).astype(np.float32))
    assert np.array_equal(y1, orc.gemm_f64(x, W))


def test_channel_absmean_exact_means():
    """The per-channel mean |x| on inputs whose fp32 sums are exact (small
    integers and halves in fp16), against exact rational means: with M a power
    of two the mean is exact in fp32; with M = 3 and a constant magnitude per
    channel the correctly rounded division returns that magnitude.  Every
    channel has its own values, so a transposed or shifted index fails."""
    import oracle as orc
    rng = np.random.default_rng(52)
    for M, K in ((8, 40), (16, 24), (1, 9)):
        mag = rng.integers(0, 200, (M, K)) / 2.0          # 0, 0.5, ... 99.5: exact in fp16
        mag[:, 3] = 1000.0 + np.arange(M)                  # a channel of distinct large values
        sign = np.where(rng.integers(0, 2, (M, K)) == 1, -1.0, 1.0)
        x = workloads.f32_to_f16_bits((sign * mag).astype(np.float32))
        got = orc.channel_absmean(x).astype(np.float64)
        for k in range(K):
            want = Fraction(sum(Fraction(v) for v in mag[:, k]), M)
            assert Fraction(float(got[k])) == want, (M, k)
    M, K = 3, 17
    per_channel = (np.arange(K) * 3 + 1) / 4.0  # 0.25, 1.0, 1.75, ...: distinct per channel
    sign = np.where(rng.integers(0, 2, (M, K)) == 1, -1.0, 1.0)
    x = workloads.f32_to_f16_bits((sign * per_channel[None, :]).astype(np.float32))
    assert np.array_equal(orc.channel_absmean(x).astype(np.float64), per_channel)
    # a row permutation does not change exact sums; doubling every value doubles the means
    x8 = workloads.f32_to_f16_bits((rng.integers(-64, 64, (8, 12)) / 4.0).astype(np.float32))
    base = orc.channel_absmean(x8)
    assert np.array_equal(orc.channel_absmean(x8[::-1].copy()), base)
    x8d = workloads.f32_to_f16_bits((x8.view(np.float16).astype(np.float32) * 2))
    assert np.array_equal(orc.channel_absmean(x8d), base * 2)


# --------------------------------------------------------------------------
# MXFP4 (quantization post, "Microscaling: NVFP4 and MXFP4"; element and scale
# formats from the microscaling paper it cites)
# --------------------------------------------------------------------------

def test_mxfp4_storage_matches_printed_bits():
    import oracle as orc
    # the methods page prints NVFP4 as 4.5 bits (one 8-bit scale per 16 values)
    # and 70B x 4.5 / 8 = 39.4 GB; MXFP4 (one 8-bit scale per 32) is 4.25 bits
    assert orc.bits_per_weight(4, 16, 8, 0) == 4.5
    assert round(orc.storage_bytes(70_000_000_000, 4, 16, 8, 0) / 1e9, 1) == 39.4
    assert orc.bits_per_weight(4, 32, 8, 0) == 4.25


def test_mxfp4_grid_and_decoding():
    # 16 codes: sign bit 3, then a 4-point exponent range with one mantissa bit
    # and a subnormal step; the largest magnitude is 6, the smallest nonzero 0.5
    import oracle as orc
    q = np.tile(np.arange(16, dtype=np.uint8), 2).reshape(1, 32)
    v = orc.dequant_mxfp4(q, np.array([[127]], np.uint8))[0, :16].astype(np.float64)
    mags = v[:8]
    assert mags[0] == 0 and np.all(np.diff(mags) > 0)
    assert mags.max() == 6.0 and mags[1] == 0.5
    assert np.array_equal(v[8:], -mags)
    # one mantissa bit: neighbouring magnitudes within a binade differ by half the binade's base
    assert np.array_equal(mags[2:] / np.repeat([1.0, 2.0, 4.0], 2), np.tile([1.0, 1.5], 3))
    # the scale byte is a power of two 2^(e8 - 127), applied exactly, down to
    # e8 = 0 (fp32 subnormals) and up to 252, the largest a finite fp32 block gives
    for e8 in (0, 1, 100, 127, 140, 252):
        w = orc.dequant_mxfp4(q, np.array([[e8]], np.uint8))[0, :16].astype(np.float64)
        assert np.array_equal(w, v * 2.0 ** (e8 - 127))


def test_mxfp4_encoding_is_nearest_with_ties_to_even():
    import oracle as orc
    grid = orc.dequant_mxfp4(np.tile(np.arange(8, dtype=np.uint8), 4).reshape(1, 32),
                             np.array([[127]], np.uint8))[0, :8].astype(np.float64)
    rng = np.random.default_rng(60)
    vals = np.concatenate([rng.uniform(0, 8, 4000), (grid[:-1] + grid[1:]) / 2, grid, [7.0, 7.5, 6.5]])
    vals = vals.astype(np.float32)
    # blocks of 31 test values behind a leading 4.0, which pins each block's
    # scale to 1 (its maximum lies in [4, 8))
    vals = np.concatenate([vals, np.zeros((-vals.size) % 31, np.float32)]).reshape(-1, 31)
    row = np.concatenate([np.full((vals.shape[0], 1), 4.0, np.float32), vals], axis=1).reshape(1, -1)
    q, e8 = orc.quantize_mxfp4(row)
    blocks_max = np.abs(row.reshape(-1, 32)).max(axis=1)
    assert np.all(e8 == 127 + np.floor(np.log2(blocks_max)).astype(int) - 2)
    got = grid[q[0] & 7]
    for v, g in zip(row[0].astype(np.float64), got):
        d = np.abs(grid - v)
        best = np.flatnonzero(d == d.min())
        want = grid[best[0]] if best.size == 1 else grid[[b for b in best if b % 2 == 0][0]]
        assert g == want, (v, g, want)
    # negative values mirror, keeping the sign bit (also when they round to zero)
    qn, e8n = orc.quantize_mxfp4(-row)
    assert np.array_equal(e8n, e8) and np.array_equal(qn & 7, q & 7) and np.all(qn[row != 0] & 8)


def test_mxfp4_scale_commutes_with_powers_of_two_and_grid_is_lossless():
    import oracle as orc
    rng = np.random.default_rng(61)
    W = (rng.standard_normal((6, 256)) * 0.05).astype(np.float32)
    q, e8 = orc.quantize_mxfp4(W)
    for k in (-5, 3):
        qk, e8k = orc.quantize_mxfp4((W * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(qk, q) and np.array_equal(e8k.astype(int), e8.astype(int) + k)
    # every block's largest code is 4 or 6 times the scale (the maximum lands in [4, 8))
    mags = orc.dequant_mxfp4(q, np.full_like(e8, 127))
    top = np.abs(mags.reshape(6, -1, 32)).max(axis=2)
    assert np.all((top == 4) | (top == 6))
    # values on the grid times a block's power of two, with a 4 or 6 in each block, decode exactly
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    c = rng.integers(0, 8, (6, 256))
    c[:, ::32] = rng.choice([6, 7], (6, 8))
    sign = np.where(rng.integers(0, 2, (6, 256)) == 1, -1.0, 1.0)
    e = rng.integers(-20, 5, (6, 8))
    Wg = (sign * grid[c] * np.repeat(2.0 ** e, 32, axis=1)).astype(np.float32)
    qg, e8g = orc.quantize_mxfp4(Wg)
    assert np.array_equal(orc.dequant_mxfp4(qg, e8g), Wg)
    assert np.array_equal(e8g.astype(int), e + 127)
    # all-zero block: scale byte 0, codes 0
    qz, ez = orc.quantize_mxfp4(np.zeros((1, 32), np.float32))
    assert ez[0, 0] == 0 and np.all(qz == 0)


def test_mxfp4_error_bound_and_device_layout():
    import oracle as orc
    rng = np.random.default_rng(62)
    W = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    W[:, 9] *= 20
    q, e8 = orc.quantize_mxfp4(W)
    X = np.repeat(2.0 ** (e8.astype(np.float64) - 127), 32, axis=1)
    err = np.abs(orc.dequant_mxfp4(q, e8).astype(np.float64) - W)
    v = np.abs(W) / X
    half_step = np.where(v < 2, 0.25, np.where(v < 4, 0.5, np.where(v <= 6, 1.0, np.inf)))
    assert np.all(err <= half_step * X)
    assert np.all(err[v > 6] <= (v[v > 6] - 6) * X[v > 6])  # saturation
    # device layout: column e of a word in nibble e; the tile geometry of the INT4 layout
    qq = np.zeros((16, 128), np.uint8)
    qq[0, :8] = np.arange(1, 9)
    p = orc.pack_device_mxfp4(qq)
    word = int(p[:4].view(np.uint32)[0])
    assert [(word >> (4 * i)) & 15 for i in range(8)] == list(range(1, 9))
    qq = np.zeros((16, 128), np.uint8)
    qq[3, 40:48] = 9
    p = orc.pack_device_mxfp4(qq)
    assert np.all(p[19 * 16 + 4: 19 * 16 + 8] == 0x99) and p.sum() == 4 * 0x99


@pytest.mark.parametrize("M,N,K,n0,nrows", [(3, 40, 256, 10, 17), (2, 33, 96, 0, 33), (1, 21, 160, 20, 1),
                                            (4, 50, 64, 0, 1)])
def test_mxfp4_gemm_rows(M, N, K, n0, nrows):
    """The MXFP4 product rows equal the fp64 product of the oracle's decoded
    weights (the same sums in the same order) on ragged shapes, for the first,
    middle and last row ranges; scale bytes differ per row and per block, so a
    wrong scale-row stride or block index changes the result."""
    import oracle as orc
    rng = np.random.default_rng(63 + M * 7 + N)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W *= (2.0 ** rng.integers(-6, 7, (N, K // 32))).repeat(32, axis=1).astype(np.float32)
    x = workloads.f32_to_f16_bits(rng.standard_normal((M, K)).astype(np.float32))
    q, e8 = orc.quantize_mxfp4(W)
    assert len(np.unique(e8)) > 8
    w_hat = orc.dequant_mxfp4(q, e8)
    y = orc.gemm_f64(x, w_hat)
    assert np.array_equal(orc.gemm_rows_mxfp4_f64(x, q, e8, n0, nrows), y[:, n0:n0 + nrows])
    assert np.array_equal(orc.gemm_rows_mxfp4_f64(x, q, e8, 0, N), y)
    # one-hot activations select the decoded weights of one input channel, exactly
    for k in (0, 37, K - 1):
        xo = np.zeros((1, K), np.float32)
        xo[0, k] = 1.0
        yo = orc.gemm_rows_mxfp4_f64(workloads.f32_to_f16_bits(xo), q, e8, 0, N)
        grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
        want = np.where(q[:, k] & 8, -1.0, 1.0) * grid[q[:, k] & 7] * 2.0 ** (e8[:, k // 32].astype(np.float64) - 127)
        assert np.array_equal(yo[0], want)


# --------------------------------------------------------------------------
# NVFP4 (methods page, "Hardware, formats and the roofline" key box: 4-bit
# values, one E4M3 scale per 16 values, a per-tensor fp32 scale, 4.5 bits)
# --------------------------------------------------------------------------

E2M1_GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
             Fraction(6)]


def _e4m3_grid():
    """The 127 finite non-negative E4M3 magnitudes from torch's own float8
    decoder (codes 0..126), as exact fractions."""
    import torch
    v = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return [Fraction(float(x)) for x in v]


def _nearest(a, d, grid):
    """Index of the grid value g minimizing |a - g d| (exact), ties to the even
    index, brute force over the whole grid."""
    dist = [abs(a - g * d) for g in grid]
    best = min(dist)
    idx = [i for i, x in enumerate(dist) if x == best]
    return idx[0] if len(idx) == 1 else [i for i in idx if i % 2 == 0][0]


def test_nvfp4_storage_matches_printed_bits():
    import oracle as orc
    # the key box prints 4.5 bits per value, 70B x 4.5 / 8 = 39.4 GB, and a
    # 3.56x reduction from fp16 (the per-tensor scale adds 32 bits per tensor)
    assert orc.bits_per_weight(4, 16, 8, 0) == 4.5
    assert round(orc.storage_bytes(70_000_000_000, 4, 16, 8, 0) / 1e9, 1) == 39.4
    assert round(16 / orc.bits_per_weight(4, 16, 8, 0), 2) == 3.56


def test_nvfp4_scale_byte_decodes_as_e4m3():
    # code 2 (E2M1 1.0) times scale byte c times S = 1 decodes to E4M3(c):
    # every one of the 127 finite magnitudes, against torch's float8 decoder
    import oracle as orc
    grid = _e4m3_grid()
    s8 = np.arange(127, dtype=np.uint8).reshape(-1, 1)
    q = np.full((127, 16), 2, np.uint8)
    w = orc.dequant_nvfp4(q, s8, 1.0)
    assert [Fraction(float(x)) for x in w[:, 0]] == grid
    assert float(grid[126]) == 448.0 and float(grid[8]) == 2.0 ** -6 and float(grid[1]) == 2.0 ** -9


def test_nvfp4_scales_and_codes_are_nearest_with_ties_to_even():
    import oracle as orc
    e4 = _e4m3_grid()
    rng = np.random.default_rng(70)
    S = 2.0 ** -8  # a first block with max|w| = 2688 * 2^-8 fixes S exactly
    d6 = Fraction(6) * Fraction(S)
    mids = [(e4[k] + e4[k + 1]) / 2 * d6 for k in range(0, 126, 5)]
    maxes = [float(m) for m in mids] + list(rng.uniform(0, 448 * 6 * S, 40)) + [448 * 6 * S, 0.25 * 2 ** -9 * 6 * S]
    rows = [np.full(16, 0.0, np.float32)]
    rows[0][0] = 2688 * S
    for m in maxes:
        blk = (rng.uniform(-1, 1, 16) * m).astype(np.float32)
        blk[3] = np.float32(m)
        rows.append(blk)
    W = np.concatenate(rows).reshape(1, -1).astype(np.float32)
    q, s8, St = orc.quantize_nvfp4(W)
    assert St == S
    for j in range(W.shape[1] // 16):
        blk = W[0, 16 * j:16 * j + 16]
        bmax = Fraction(float(np.abs(blk).max()))
        assert s8[0, j] == _nearest(bmax, d6, e4), j
        sb = e4[s8[0, j]]
        for i in range(16):
            v = Fraction(float(blk[i]))
            m = 0 if sb == 0 else _nearest(abs(v), sb * Fraction(S), E2M1_GRID)
            assert q[0, 16 * j + i] & 7 == m, (j, i)
            assert (q[0, 16 * j + i] >> 3) == (1 if blk[i] < 0 else 0)


def test_nvfp4_tensor_scale_grid_values_and_powers_of_two():
    import oracle as orc
    rng = np.random.default_rng(71)
    # the tensor scale: fp32 of max|w| / 2688, 1 for an all-zero tensor
    W = (rng.standard_normal((5, 64)) * 0.03).astype(np.float32)
    q, s8, S = orc.quantize_nvfp4(W)
    assert S == float(np.float32(float(np.abs(W).max()) / 2688.0))
    qz, sz, Sz = orc.quantize_nvfp4(np.zeros((2, 32), np.float32))
    assert Sz == 1.0 and not sz.any() and not qz.any()
    # scaling the tensor by 2^k scales S by 2^k and keeps every byte
    for k in (-7, 5):
        qk, sk, Sk = orc.quantize_nvfp4((W * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(qk, q) and np.array_equal(sk, s8) and Sk == S * 2.0 ** k
    # weights on the grid (E2M1 times an E4M3 scale times a power-of-two S,
    # each block holding a 6, one block with scale 448) decode exactly
    e4 = np.array([float(x) for x in _e4m3_grid()])
    grid = np.array([float(x) for x in E2M1_GRID])
    Sg = 2.0 ** -12
    sc = rng.integers(40, 127, (4, 8))
    sc[0, 0] = 126
    c = rng.integers(0, 8, (4, 128))
    c[:, ::16] = 7
    sign = np.where(rng.integers(0, 2, (4, 128)) == 1, -1.0, 1.0)
    Wg = (sign * grid[c] * np.repeat(e4[sc], 16, axis=1) * Sg).astype(np.float32)
    qg, sg, Sgot = orc.quantize_nvfp4(Wg)
    assert Sgot == Sg and np.array_equal(sg, sc) and np.array_equal(qg & 7, c)
    assert np.array_equal(orc.dequant_nvfp4(qg, sg, Sgot), Wg)


def test_nvfp4_error_bound():
    import oracle as orc
    rng = np.random.default_rng(72)
    W = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    W[:, 9] *= 30
    q, s8, S = orc.quantize_nvfp4(W)
    e4 = np.array([float(x) for x in _e4m3_grid()])
    X = np.repeat(e4[s8], 16, axis=1) * S  # the step unit of each block
    w_hat = orc.dequant_nvfp4(q, s8, S).astype(np.float64)
    err = np.abs(w_hat - W)
    v = np.abs(W) / np.where(X > 0, X, 1.0)
    half_step = np.where(v < 2, 0.25, np.where(v < 4, 0.5, np.where(v <= 6, 1.0, np.inf)))
    ulp32 = np.abs(W) * 2.0 ** -23  # the final fp32 rounding
    inside = (v <= 6) & (X > 0)
    assert np.all(err[inside] <= half_step[inside] * X[inside] + ulp32[inside])
    # past 6 the code saturates; the block scale rounds to within 1/16 of the
    # block's max / 6, so the saturated part stays below the scale's rounding
    sat = (v > 6) & (X > 0)
    assert np.all(err[sat] <= (v[sat] - 6) * X[sat] + ulp32[sat]) and np.all(v[sat] < 6 * (1 + 1 / 16) + 1e-9)


@pytest.mark.parametrize("M,N,K,n0,nrows", [(3, 40, 256, 10, 17), (2, 33, 96, 0, 33), (1, 21, 160, 20, 1),
                                            (4, 50, 64, 0, 1)])
def test_nvfp4_gemm_rows(M, N, K, n0, nrows):
    """The NVFP4 product rows equal the fp64 product of the exactly decoded
    weights E2M1 * E4M3 * S, decoded here with torch's float8 grid; block
    scales differ per row and per block, so a wrong scale-row stride or block
    index changes the result."""
    import oracle as orc
    rng = np.random.default_rng(73 + M * 7 + N)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W *= (2.0 ** rng.integers(-6, 7, (N, K // 16))).repeat(16, axis=1).astype(np.float32)
    x = workloads.f32_to_f16_bits(rng.standard_normal((M, K)).astype(np.float32))
    q, s8, S = orc.quantize_nvfp4(W)
    assert len(np.unique(s8)) > 8
    e4 = np.array([float(v) for v in _e4m3_grid()])
    grid = np.array([float(v) for v in E2M1_GRID])
    w_exact = np.where(q & 8, -1.0, 1.0) * grid[q & 7] * np.repeat(e4[s8], 16, axis=1) * S
    xf = orc.f16_bits_to_f32(x).reshape(M, K).astype(np.float64)
    y = np.array([[sum(xf[m, k] * w_exact[n, k] for k in range(K)) for n in range(N)] for m in range(M)])
    assert np.allclose(orc.gemm_rows_nvfp4_f64(x, q, s8, S, n0, nrows), y[:, n0:n0 + nrows], rtol=1e-12, atol=1e-12)
    assert np.allclose(orc.gemm_rows_nvfp4_f64(x, q, s8, S, 0, N), y, rtol=1e-12, atol=1e-12)
    # one-hot activations select the exactly decoded weights of one input channel
    for k in (0, 37 % K, K - 1):
        xo = np.zeros((1, K), np.float32)
        xo[0, k] = 1.0
        yo = orc.gemm_rows_nvfp4_f64(workloads.f32_to_f16_bits(xo), q, s8, S, 0, N)
        assert np.array_equal(yo[0], w_exact[:, k])


# --------------------------------------------------------------------------
# Number formats against independent implementations
# --------------------------------------------------------------------------

def test_f32_to_f16_against_numpy_structured(orc):
    """Every sign/exponent/top-mantissa combination with the low 13 bits set to
    the values that decide rounding, plus the whole fp16-subnormal input range."""
    hi = np.arange(1 << 19, dtype=np.uint32) << np.uint32(13)
    lows = np.array([0, 1, 0x7FF, 0xFFF, 0x1000, 0x1001, 0x17FF, 0x1FFF], np.uint32)
    bits = (hi[:, None] | lows[None, :]).ravel()
    sub = np.arange(0x33000000 - 64, 0x38800000 + 64, 3, dtype=np.uint32)
    bits = np.concatenate([bits, sub, sub | np.uint32(0x80000000)])
    f = bits.view(np.float32)
    ours = orc.f32_to_f16_bits(f)
    ref = f.astype(np.float16).view(np.uint16)
    nan = np.isnan(f)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all((ours[nan] & 0x7C00) == 0x7C00) and np.all((ours[nan] & 0x3FF) != 0)


def test_f32_to_f16_random_exhaustive_sample(orc):
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    nan = np.isnan(f)
    assert np.array_equal(orc.f32_to_f16_bits(f)[~nan], f.astype(np.float16).view(np.uint16)[~nan])


def test_f16_to_f32_exhaustive(orc):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = orc.f16_bits_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.all(np.isnan(ours[nan]))


def test_f32_to_bf16_against_torch(orc):
    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x18000 & 0xFFFF], np.uint32)
    bits = (hi[:, None] | lows[None, :]).ravel()
    f = bits.view(np.float32)
    keep = ~np.isnan(f)
    f = f[keep]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.f32_to_bf16_bits(f), ref)


# --------------------------------------------------------------------------
# Quantizer: constructed cases and invariants
# --------------------------------------------------------------------------

def test_ties_round_half_to_even(orc):
    """s = 0.25 and z = 4 exactly (min -1, max 2.75); these weights put w/s + z
    exactly on k + 1/2, where round-half-to-even and round-half-up differ."""
    base = [-1.0, 2.75]
    ties = [0.125, 0.375, -0.875, 2.625, 0.625, -0.125]
    expect = [4, 6, 0, 14, 6, 4]  # 4.5->4, 5.5->6, 0.5->0, 14.5->14, 6.5->6, 3.5->4
    w = np.array([base + ties], np.float32)
    q, s, z = orc.quantize_groups(w, w.shape[1])
    assert s[0, 0] == np.float16(0.25).view(np.uint16) and z[0, 0] == 4
    assert list(q[0, 2:]) == expect
    assert list(q[0, :2]) == [0, 15]


def test_zero_point_tie_rounds_to_even(orc):
    """min -1.125, max 2.625: s = 0.25 exactly and -min/s = 4.5 exactly, so the
    zero-point is 4 under round-half-to-even (5 under round-half-up)."""
    w = np.array([[-1.125, 2.625, 0.0, 1.0]], np.float32)
    q, s, z = orc.quantize_groups(w, 4)
    assert s[0, 0] == np.float16(0.25).view(np.uint16)
    assert z[0, 0] == 4
    # -4.5 + 4 = -0.5 -> 0 and 10.5 + 4 = 14.5 -> 14 (ties again), 1/0.25 + 4 = 8
    assert list(q[0]) == [0, 14, 4, 8]


def test_encode_uses_the_stored_fp16_scale(orc):
    """Range 3.8 gives s32 = 0.25333.. which fp16 rounds up to s_h = 0.25341797.
    A weight between 6.5*s32 and 6.5*s_h encodes to z+6 with the stored scale
    and to z+7 with the unrounded one."""
    s32 = np.float32(3.8) / np.float32(15.0)
    s_h = np.float32(np.float16(s32))
    assert s_h > s32
    w_mid = np.float32(6.5 * (float(s32) + float(s_h)) / 2)
    w = np.array([[-1.0, 2.8, w_mid, 0.0]], np.float32)
    q, s, z = orc.quantize_groups(w, 4)
    assert s[0, 0] == np.float16(s32).view(np.uint16) and z[0, 0] == 4
    assert q[0, 2] == 10


def test_degenerate_and_one_signed_groups(orc):
    g = 32
    zeros = np.zeros(g, np.float32)
    const_pos = np.full(g, 0.3, np.float32)
    const_neg = np.full(g, -0.3, np.float32)
    all_pos = np.linspace(0.1, 0.5, g).astype(np.float32)
    all_neg = -all_pos
    tiny = np.full(g, 1e-9, np.float32)  # range/15 rounds to fp16 zero
    W = np.stack([zeros, const_pos, const_neg, all_pos, all_neg, tiny])
    q, s, z = orc.quantize_groups(W, g)
    assert s[0, 0] == 0 and z[0, 0] == 0 and np.all(q[0] == 0)
    assert s[5, 0] == 0 and z[5, 0] == 0 and np.all(q[5] == 0)
    # constant positive: range [0, 0.3] -> z = 0, every code 15
    assert z[1, 0] == 0 and np.all(q[1] == 15)
    # constant negative: range [-0.3, 0] -> z = 15, every code 0
    assert z[2, 0] == 15 and np.all(q[2] == 0)
    assert z[3, 0] == 0 and q[3, -1] == 15
    assert z[4, 0] == 15 and q[4, -1] == 0
    w_hat = orc.dequant(q, s, z, g)
    assert np.all(w_hat[0] == 0)
    np.testing.assert_allclose(w_hat[1], 0.3, rtol=2e-3)
    np.testing.assert_allclose(w_hat[2], -0.3, rtol=2e-3)


def test_subnormal_scale(orc):
    """A group whose scale is an fp16 subnormal keeps it (no flush to zero)."""
    w = np.array([[-3e-6, 0.0, 2e-6, 5e-6]], np.float32)
    q, s, z = orc.quantize_groups(w, 4)
    assert 0 < s[0, 0] < 0x0400
    sh = float(np.uint16(s[0, 0]).view(np.float16))
    assert abs(sh - np.float16(np.float32(8e-6) / np.float32(15.0))) == 0


def test_nonfinite_scale_is_an_error(orc):
    w = np.array([[-5e5, 5e5, 0.0, 1.0]], np.float32)
    with pytest.raises(orc.OracleError):
        orc.quantize_groups(w, 4)


@pytest.mark.parametrize("group", [32, 128])
def test_quantizer_invariants(orc, group):
    N, K = 24, 1024
    W = workloads.bf16_bits_to_f32(workloads.gen_weights(11, N, K, outlier_frac=0.01))
    q, s, z = orc.quantize_groups(W, group)
    assert q.max() <= 15 and z.max() <= 15
    sh = s.view(np.float16).astype(np.float64)
    w_hat = orc.dequant(q, s, z, group).astype(np.float64)
    # error bound: half a step plus what rounding the scale to fp16 can move
    # the clipped top code (15 steps of |s32 - s_h|), plus fp32 rounding slack
    Wg = W.reshape(N, K // group, group).astype(np.float64)
    lo = np.minimum(Wg.min(-1), 0)
    hi = np.maximum(Wg.max(-1), 0)
    s32 = (hi - lo) / 15
    bound = sh / 2 + 15 * np.abs(s32 - sh) + 1e-6 * sh
    err = np.abs(Wg - w_hat.reshape(Wg.shape)).max(-1)
    assert np.all(err <= bound)
    # the reconstruction reaches both ends of every group's (widened) range
    assert np.all(np.abs(w_hat.reshape(Wg.shape).max(-1) - hi) <= sh)
    assert np.all(np.abs(w_hat.reshape(Wg.shape).min(-1) - lo) <= sh)


@pytest.mark.parametrize("group", [32, 128])
def test_requantize_is_identity(orc, group):
    """Quantizing w_hat again returns the same codes, scales and zero-points in
    every group whose codes reach both 0 and 15 (15*s_h is exact in fp32)."""
    W = workloads.bf16_bits_to_f32(workloads.gen_weights(12, 16, 512, outlier_frac=0.01))
    q, s, z = orc.quantize_groups(W, group)
    w_hat = orc.dequant(q, s, z, group)
    q2, s2, z2 = orc.quantize_groups(w_hat, group)
    G = 512 // group
    full = (q.reshape(16, G, group).min(-1) == 0) & (q.reshape(16, G, group).max(-1) == 15)
    assert full.mean() > 0.5
    assert np.array_equal(s2[full], s[full]) and np.array_equal(z2[full], z[full])
    assert np.array_equal(q2.reshape(16, G, group)[full], q.reshape(16, G, group)[full])


def test_permutation_within_group(orc):
    rng = np.random.default_rng(3)
    W = rng.standard_normal((4, 128)).astype(np.float32)
    perm = rng.permutation(128)
    q, s, z = orc.quantize_groups(W, 128)
    qp, sp, zp = orc.quantize_groups(np.ascontiguousarray(W[:, perm]), 128)
    assert np.array_equal(qp, q[:, perm]) and np.array_equal(sp, s) and np.array_equal(zp, z)


def test_rows_and_groups_are_independent(orc):
    """Changing one group changes only that group's outputs (catches a wrong
    row or group index)."""
    W = workloads.bf16_bits_to_f32(workloads.gen_weights(13, 8, 256, outlier_frac=0.0))
    q, s, z = orc.quantize_groups(W, 32)
    W2 = W.copy()
    W2[5, 64:96] *= 3.0
    q2, s2, z2 = orc.quantize_groups(W2, 32)
    diff_s = s2 != s
    assert diff_s[5, 2] and diff_s.sum() == 1
    mask = np.ones_like(q, bool)
    mask[5, 64:96] = False
    assert np.array_equal(q2[mask], q[mask])


def test_bf16_and_f32_inputs_agree(orc):
    b = workloads.gen_weights(14, 8, 256, outlier_frac=0.01)
    f = workloads.bf16_bits_to_f32(b)
    r1 = orc.quantize_groups(b, 128, dtype=orc.BF16)
    r2 = orc.quantize_groups(f, 128)
    for a, c in zip(r1, r2):
        assert np.array_equal(a, c)


# --------------------------------------------------------------------------
# Dequantization: exact in fp32, one rounding to fp16 / bf16
# --------------------------------------------------------------------------

def test_dequant_exact_all_code_pairs(orc):
    rng = np.random.default_rng(5)
    scales = np.concatenate([
        np.array([0x0001, 0x0155, 0x03FF, 0x0400, 0x30F8, 0x3C00, 0x7BFF], np.uint16),
        rng.integers(0x0001, 0x7C00, 57).astype(np.uint16),
    ])
    qq, zz = np.meshgrid(np.arange(16), np.arange(16), indexing="ij")
    q = np.tile(qq.ravel().astype(np.uint8), (scales.size, 1))
    z = np.tile(zz.ravel().astype(np.uint8), (scales.size, 1))
    s = np.repeat(scales[:, None], 256, axis=1)
    # one group per element: g = 1
    f32 = orc.dequant(q, s, z, 1, orc.F32)
    f16 = orc.dequant(q, s, z, 1, orc.F16)
    b16 = orc.dequant(q, s, z, 1, orc.BF16)
    exact = [[Fraction(float(np.uint16(sv).view(np.float16))) * (int(a) - int(b))
              for a, b in zip(qr, zr)] for sv, qr, zr in zip(scales, q, z)]
    exact_f = np.array([[float(v) for v in row] for row in exact])
    assert np.array_equal(f32.astype(np.float64), exact_f)  # exact in fp32
    assert np.array_equal(f16, exact_f.astype(np.float16).view(np.uint16))
    ref_b = torch.from_numpy(exact_f.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b16, ref_b)


# --------------------------------------------------------------------------
# Packing
# --------------------------------------------------------------------------

def test_pack_device_is_a_bijection(orc):
    """Each element lands in its own nibble; pad nibbles stay zero; unpack
    inverts pack; shapes with ragged rows and columns included."""
    for N, K in [(16, 128), (37, 96), (5, 416)]:
        nbytes = orc.device_bytes(N, K)
        assert nbytes == ((N + 15) // 16 * 16) * ((K + 127) // 128 * 128) // 2
        seen = np.zeros(2 * nbytes, np.int64)
        # mark one element at a time in batches: code 1 at positions (n, k)
        for n in range(N):
            q = np.zeros((N, K), np.uint8)
            q[n, :] = 1
            p = orc.pack_device(q)
            nib = np.stack([p & 15, p >> 4], axis=1).ravel()
            assert nib.sum() == K
            seen += nib
        assert seen.max() == 1 and seen.sum() == N * K
        rng = np.random.default_rng(N * K)
        q = rng.integers(0, 16, (N, K)).astype(np.uint8)
        assert np.array_equal(orc.unpack_device(orc.pack_device(q), N, K), q)


def test_pack_device_word_order(orc):
    """Within one 32-bit word the eight columns 8c..8c+7 sit in nibbles
    0,4,1,5,2,6,3,7 (pairs of neighbouring columns 16 bits apart)."""
    q = np.zeros((16, 128), np.uint8)
    q[0, :8] = np.arange(1, 9)
    p = orc.pack_device(q)
    word = int(p[:4].view(np.uint32)[0])
    nibbles = [(word >> (4 * i)) & 15 for i in range(8)]
    assert nibbles == [1, 3, 5, 7, 2, 4, 6, 8]
    # row 3, columns 40..47 (word j=1 of lane 3 + 16*1)
    q = np.zeros((16, 128), np.uint8)
    q[3, 40:48] = 9
    p = orc.pack_device(q)
    lane = 3 + 16 * 1
    assert np.all(p[lane * 16 + 4: lane * 16 + 8] == 0x99)
    assert p.sum() == 4 * 0x99


def test_pack_canonical_and_zeros(orc):
    q = np.array([[1, 2, 3, 4]], np.uint8)
    assert list(orc.pack_canonical(q)[0]) == [0x21, 0x43]
    z = np.array([[5, 6, 7]], np.uint8)
    assert list(orc.pack_zeros(z)[0]) == [0x65, 0x07]


# --------------------------------------------------------------------------
# The product: brute force against exact rational arithmetic
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1, 3, 8), (3, 5, 16), (2, 7, 64)])
def test_gemm_f64_brute_force_exact(orc, M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    x = workloads.f32_to_f16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = rng.standard_normal((N, K)).astype(np.float32)
    y = orc.gemm_f64(x, w)
    xf = x.view(np.float16)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(xf[m, k])) * Fraction(float(w[n, k])) for k in range(K))
            mag = sum(abs(float(xf[m, k]) * float(w[n, k])) for k in range(K))
            assert abs(float(exact) - y[m, n]) <= K * 2.0 ** -52 * mag


def test_gemm_rows_matches_full(orc):
    rng = np.random.default_rng(9)
    M, N, K, g = 3, 40, 256, 32
    W = rng.standard_normal((N, K)).astype(np.float32) * 0.02
    x = workloads.f32_to_f16_bits(rng.standard_normal((M, K)).astype(np.float32))
    q, s, z = orc.quantize_groups(W, g)
    y = orc.gemm_f64(x, orc.dequant(q, s, z, g))
    assert np.array_equal(orc.gemm_rows_f64(x, q, s, z, g, 10, 17), y[:, 10:27])


def test_one_hot_activation_selects_a_weight(orc):
    rng = np.random.default_rng(10)
    W = rng.standard_normal((6, 128)).astype(np.float32)
    q, s, z = orc.quantize_groups(W, 32)
    w_hat = orc.dequant(q, s, z, 32)
    x = np.zeros((1, 128), np.float32)
    x[0, 77] = 1.0
    y = orc.gemm_f64(workloads.f32_to_f16_bits(x), w_hat)
    assert np.array_equal(y[0], w_hat[:, 77].astype(np.float64))


# --------------------------------------------------------------------------
# Roofline arithmetic (Cruxly lesson, roofline paragraph)
# --------------------------------------------------------------------------

def test_roofline_numbers():
    g = golden("roofline.json")
    ridge = g["assumed"]["tflops"] / g["assumed"]["tbps"]
    assert round(ridge) == g["printed"]["ridge_flop_per_byte"]
    # fp16: 2 FLOP per weight per batch row over 2 bytes -> batch FLOP/byte
    assert round(ridge / 100) * 100 == g["printed"]["fp16_crossover_batch_about"]
    # 4-bit: 2 FLOP per batch row over half a byte -> 4 * batch FLOP/byte
    assert round(ridge / 4) == g["printed"]["int4_crossover_batch"]
