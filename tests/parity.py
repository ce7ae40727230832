"""Shared helpers of the GPU parity tests: move seeded host inputs to the GPU,
run the HIP path through the C ABI, and compare with the oracle."""
from __future__ import annotations

import re
import sys

import numpy as np
import torch

import oracle
import w4a16_bit_matmul_amd as wq

TOL = 1e-2  # max relative error of y, from the workload specification


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev_weights(W: np.ndarray, w_dtype: str) -> torch.Tensor:
    if w_dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(W, np.float32)).cuda()
    t = torch.from_numpy(np.ascontiguousarray(W, np.uint16).view(np.int16)).cuda()
    return t.view(torch.bfloat16 if w_dtype == "bf16" else torch.float16)


def to_dev_f16(x_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x_bits, np.uint16).view(np.int16)).cuda().view(torch.float16)


def f16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def oracle_dtype(w_dtype: str) -> int:
    return {"f32": oracle.F32, "bf16": oracle.BF16, "f16": oracle.F16}[w_dtype]


def gpu_quantize(W_host: np.ndarray, w_dtype: str, group: int, scheme: int = wq.WQ_ASYM):
    Wd = to_dev_weights(W_host, w_dtype)
    out = wq.wq_quantize_groups(Wd, group, codes=True, packed=True, scheme=scheme)
    torch.cuda.synchronize()
    return out


def assert_quantize_matches(W_host: np.ndarray, w_dtype: str, group: int, out=None, scheme: int = wq.WQ_ASYM):
    """Codes, scales, zero-points and both packed layouts bit-exact vs the oracle."""
    if out is None:
        out = gpu_quantize(W_host, w_dtype, group, scheme)
    q, s, z = oracle.quantize_groups(W_host, group, dtype=oracle_dtype(w_dtype),
                                     scheme=oracle.SYM if scheme == wq.WQ_SYM else oracle.ASYM)
    s_gpu = f16_bits(out["s"])
    assert np.array_equal(s_gpu, s), f"scales differ at {np.argwhere(s_gpu != s)[:5]}"
    z_gpu = out["z_codes"].cpu().numpy()
    assert np.array_equal(z_gpu, z), f"zero-points differ at {np.argwhere(z_gpu != z)[:5]}"
    q_gpu = out["q_codes"].cpu().numpy()
    assert np.array_equal(q_gpu, q), f"codes differ at {np.argwhere(q_gpu != q)[:5]}"
    assert np.array_equal(out["qw"].qpacked.cpu().numpy(), oracle.pack_device(q))
    assert np.array_equal(out["qw"].zpacked.cpu().numpy(), oracle.pack_zeros(z))
    return q, s, z, out


# Elementwise floors.  The GEMV multiplies x by the exact code differences
# q - z (small integers, exact in fp16) on the matrix cores, sums the exact
# products in fp32 and applies each group's scale once, so its elementwise
# error against the exact-What product is checked down to 1e-3 of max|y|.  The MFMA path multiplies fp16(What): one rounding per weight, a
# relative error uniform in +-2^-11 (rms 2^-11/sqrt(3) = 2.8e-4).  Over K terms
# the output error then has about 2.8e-4 times the spread of y itself, so an
# output near zero can carry an error of ~3e-4 of max|y|; against the
# exact-What product the MFMA path's elementwise check therefore floors at
# 5e-2 of max|y| (3e-4 / 5e-2 = 6e-3, inside the 1e-2 bound, where a 1e-2
# floor would ask for 1e-4).  The MFMA path is additionally checked element by
# element, with the GEMV's 1e-3 floor, against the fp64 product of the
# oracle's fp16-rounded What, which is exactly what the matrix cores multiply
# (compare_y_path).
FLOOR_GEMV = 1e-3
FLOOR_MFMA = 5e-2


def floor_for(path, M, N, fmt="int4", K=None, group=None):
    return FLOOR_MFMA if uses_mfma(path, M, N, fmt, K, group) else FLOOR_GEMV


def compare_y(y_gpu: torch.Tensor, y_ref: np.ndarray, tol: float = TOL, floor_frac: float = FLOOR_MFMA):
    """Max relative error (normwise: max|y - y_ref| / max|y_ref|, the gate) and
    the elementwise relative error with its denominator floored at
    floor_frac * max|y_ref|; both must be within tol."""
    y = y_gpu.detach().float().cpu().numpy().astype(np.float64)
    assert y.shape == y_ref.shape
    assert np.all(np.isfinite(y))
    err = np.abs(y - y_ref)
    scale = np.abs(y_ref).max()
    normwise = err.max() / scale if scale > 0 else err.max()
    floor = max(floor_frac * scale, 1e-30)
    elementwise = (err / np.maximum(np.abs(y_ref), floor)).max()
    assert normwise <= tol, f"normwise relative error {normwise:.3e}"
    assert elementwise <= tol, f"elementwise relative error {elementwise:.3e}"
    return normwise, elementwise


def uses_mfma(path, M, N, fmt="int4", K=None, group=None) -> bool:
    return path == wq.WQ_PATH_MFMA or (path == wq.WQ_PATH_AUTO and wq.auto_uses_mfma(M, N, fmt, K, group))


def compare_y_path(y_gpu: torch.Tensor, y_ref: np.ndarray, y_ref16: np.ndarray | None, path, M, tol: float = TOL,
                   fmt: str = "int4", K=None, group=None):
    """The gate against the exact-What oracle product (normwise, and
    elementwise with the path's floor); on the MFMA path, also the elementwise
    check at FLOOR_GEMV against y_ref16, the oracle product of fp16(What).
    Returns (normwise, elementwise, elementwise vs y_ref16 or None)."""
    N = y_ref.shape[1]
    nw, ew = compare_y(y_gpu, y_ref, tol=tol, floor_frac=floor_for(path, M, N, fmt, K, group))
    ew16 = None
    if uses_mfma(path, M, N, fmt, K, group) and y_ref16 is not None:
        _, ew16 = compare_y(y_gpu, y_ref16, tol=tol, floor_frac=FLOOR_GEMV)
    return nw, ew, ew16


def ref16(x_bits: np.ndarray, w_hat_f16_bits: np.ndarray) -> np.ndarray:
    """fp64 oracle product of x with fp16 weights given as bit patterns."""
    w = np.ascontiguousarray(w_hat_f16_bits, np.uint16).view(np.float16).astype(np.float32)  # exact widening
    return oracle.gemm_f64(x_bits, w)


def split_k(plan: str) -> int:
    """The K split count a kernel description names."""
    return int(re.search(r"split_k=(\d+)", plan).group(1))
