"""INT4 KV cache in blocks of 128 on the HIP path against the oracle: cache
rows (codes, scales, zero-points) bit-exact after scattering tokens into
slots, decoding bit-exact, for decode-sized appends and a long prefill."""
import numpy as np
import pytest
import torch

import oracle
import w4a16_bit_matmul_amd as wq
import workloads
from parity import f16_bits, oracle_dtype, say, to_dev_weights

pytestmark = pytest.mark.gpu


def _tokens(seed, T, hd, x_dtype):
    """Synthetic K/V rows: N(0, 1) with a few large channels (the same
    channels in every token), as bf16 / fp16 bit patterns or fp32."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, hd)).astype(np.float32)
    X[:, rng.choice(hd, max(1, hd // 100), replace=False)] *= 8.0
    if x_dtype == "bf16":
        return workloads.f32_to_bf16_bits(X)
    if x_dtype == "f16":
        return workloads.f32_to_f16_bits(X)
    return X


def _gpu_cache_from(c_host):
    codes, s, z = c_host
    S, hd = codes.shape[0], codes.shape[1] * 2
    cache = wq.kv_cache_alloc(S, hd)
    cache.codes.copy_(torch.from_numpy(codes))
    cache.s.copy_(torch.from_numpy(s.view(np.int16)).view(torch.float16))
    cache.zpacked.copy_(torch.from_numpy(z))
    return cache


def _assert_cache_equal(cache, c_host):
    codes, s, z = c_host
    got_c = cache.codes.cpu().numpy()
    assert np.array_equal(got_c, codes), f"codes differ at rows {np.unique(np.argwhere(got_c != codes)[:, 0])[:5]}"
    assert np.array_equal(f16_bits(cache.s), s), "scales differ"
    assert np.array_equal(cache.zpacked.cpu().numpy(), z), "zero-points differ"


@pytest.mark.parametrize("T,hd", [(1, 128), (3, 384), (64, 1024), (37, 1024), (5, 640)])
@pytest.mark.parametrize("x_dtype", ["bf16", "f16", "f32"])
def test_kv_quantize_rows_bit_exact(T, hd, x_dtype):
    say(f"kv quantize T={T} hd={hd} {x_dtype}")
    X = _tokens(100 + T + hd, T, hd, x_dtype)
    ref = oracle.kv_alloc(T, hd)
    oracle.kv_quantize(X, ref, dtype=oracle_dtype(x_dtype))
    cache = wq.kv_cache_alloc(T, hd)
    wq.wq_kv_quantize(to_dev_weights(X, x_dtype), cache)
    torch.cuda.synchronize()
    _assert_cache_equal(cache, ref)


@pytest.mark.parametrize("hd", [1024, 384])
def test_kv_append_into_slots(hd):
    """Decode-style append: tokens scattered into named rows of a larger cache
    that already holds data; slots outside the cache are skipped and rows not
    named keep their bytes (checked against the oracle on the same start)."""
    say(f"kv append hd={hd}")
    S, T = 300, 64
    rng = np.random.default_rng(7 + hd)
    start = oracle.kv_alloc(S, hd)
    oracle.kv_quantize(_tokens(8, S, hd, "f32"), start)  # previous contents
    slots = rng.choice(S, T, replace=False).astype(np.int32)
    slots[5], slots[17], slots[40] = -3, S, S + 1000
    X = _tokens(9 + hd, T, hd, "bf16")
    ref = tuple(a.copy() for a in start)
    oracle.kv_quantize(X, ref, slot=slots, dtype=oracle.BF16)
    cache = _gpu_cache_from(start)
    wq.wq_kv_quantize(to_dev_weights(X, "bf16"), cache, slot=torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    _assert_cache_equal(cache, ref)


@pytest.mark.parametrize("out_dtype", ["f32", "f16", "bf16"])
def test_kv_dequant_bit_exact(out_dtype):
    say(f"kv dequant -> {out_dtype}")
    S, hd, T = 200, 1024, 50
    rng = np.random.default_rng(11)
    ref = oracle.kv_alloc(S, hd)
    oracle.kv_quantize(_tokens(12, S, hd, "f32"), ref)
    slots = rng.choice(S, T, replace=False).astype(np.int32)
    slots[3], slots[9] = -1, S
    od = {"f32": oracle.F32, "f16": oracle.F16, "bf16": oracle.BF16}[out_dtype]
    td = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[out_dtype]
    want = oracle.kv_dequant(ref, T, hd, slot=slots, out_dtype=od)
    got = wq.wq_kv_dequant(_gpu_cache_from(ref), T, slot=torch.from_numpy(slots).cuda(), out_dtype=td)
    torch.cuda.synchronize()
    got = got.cpu().numpy() if out_dtype == "f32" else got.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_kv_printed_example_and_special_blocks():
    """The quantization post's eight weights padded into a block, plus exact
    ties, an all-zero block, a one-signed block and a subnormal-scale block."""
    say("kv special blocks")
    hd = 768
    X = np.zeros((2, hd), np.float32)
    X[0, 128:136] = workloads.WORKED_EXAMPLE_W
    X[0, 256:264] = [-1.0, 2.75, 0.125, 0.375, -0.875, 2.625, 0.625, -0.125]
    X[0, 512:640] = np.linspace(0.1, 0.5, 128)
    X[1, 0:4] = [-3e-6, 0.0, 2e-6, 5e-6]
    X[1, 128:256] = -np.linspace(0.1, 0.5, 128)
    ref = oracle.kv_alloc(2, hd)
    oracle.kv_quantize(X, ref)
    cache = wq.kv_cache_alloc(2, hd)
    wq.wq_kv_quantize(torch.from_numpy(X).cuda(), cache)
    torch.cuda.synchronize()
    _assert_cache_equal(cache, ref)
    word = int(cache.codes[0, 64:68].cpu().numpy().view(np.uint32)[0])
    assert [(word >> (4 * (4 * (e % 2) + e // 2))) & 15 for e in range(8)] == [8, 5, 11, 6, 15, 0, 7, 10]


def test_kv_prefill_full_size():
    """A 32768-token prefill of one layer's K (8 KV heads x 128, bf16) into a
    cache of the same length: every row bit-exact, and the decoded cache
    exact against the oracle's decoding."""
    T, hd = 32768, 1024
    say(f"kv prefill T={T} hd={hd}")
    X = _tokens(13, T, hd, "bf16")
    ref = oracle.kv_alloc(T, hd)
    oracle.kv_quantize(X, ref, dtype=oracle.BF16)
    cache = wq.kv_cache_alloc(T, hd)
    wq.wq_kv_quantize(to_dev_weights(X, "bf16"), cache)
    torch.cuda.synchronize()
    _assert_cache_equal(cache, ref)
    rows = np.random.default_rng(14).choice(T, 256, replace=False).astype(np.int32)
    got = wq.wq_kv_dequant(cache, 256, slot=torch.from_numpy(rows).cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), oracle.kv_dequant(ref, 256, hd, slot=rows))
