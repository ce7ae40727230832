"""CPU oracle for group-wise asymmetric INT4 quantization and y = x * What^T.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
CPU-baseline leg of the benchmark, never by the product package.  It wraps the
plain C implementation in ``wq_oracle.c`` (built with gcc, no fast-math, no
contraction) through ctypes and numpy arrays.  It shares no code with the HIP
path.

Every function names the passage it follows; the readings taken where the pages
are silent are listed at the top of ``wq_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wq_oracle.c")
_LIB = os.path.join(_HERE, "_liborc.so")

F32, BF16, F16 = 0, 1, 2
EINVAL, ERANGE = -1, -6

_lib = None


def build(verbose: bool = False, out: str | None = None, sanitize: bool = False) -> str:
    """Compile the oracle with gcc (plain IEEE binary32/64, no FMA contraction).
    sanitize=True adds AddressSanitizer and UndefinedBehaviorSanitizer (every
    report fatal) for the sanitized test run; out names the library file."""
    target = out or _LIB
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
        "-ffp-contract=off", "-fno-fast-math", "-fno-finite-math-only",
    ]
    if sanitize:
        cmd += ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    cmd += ["-o", target + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(target + ".tmp", target)
    return target


def _load():
    global _lib
    if _lib is not None:
        return _lib
    alt = os.environ.get("WQ_ORACLE_LIB")  # a separately built copy (the sanitized test run)
    if alt:
        lib = ctypes.CDLL(alt)
    else:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    sig = {
        "orc_set_threads": (None, [I]),
        "orc_get_threads": (I, []),
        "orc_f16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "orc_f32_to_f16": (ctypes.c_uint16, [ctypes.c_float]),
        "orc_f32_to_bf16": (ctypes.c_uint16, [ctypes.c_float]),
        "orc_f32_to_f16_array": (None, [P, I64, P]),
        "orc_f32_to_bf16_array": (None, [P, I64, P]),
        "orc_quantize_groups": (I, [P, I, I64, I64, I, P, P, P]),
        "orc_quantize_groups_ex": (I, [P, I, I64, I64, I, I, P, P, P]),
        "orc_dequant": (I, [P, P, P, I64, I64, I, I, P]),
        "orc_pack_canonical": (I, [P, I64, I64, P]),
        "orc_device_bytes": (I64, [I64, I64]),
        "orc_pack_device": (I, [P, I64, I64, P]),
        "orc_unpack_device": (I, [P, I64, I64, P]),
        "orc_pack_zeros": (I, [P, I64, I64, P]),
        "orc_gemm_f64": (I, [I64, I64, I64, P, P, P]),
        "orc_gemm_rows_f64": (I, [I64, I64, I64, I, P, P, P, P, I64, I64, P]),
        "orc_symmetric": (I, [P, I64, I, P, P, P]),
        "orc_quantize_w8": (I, [P, I, I64, I64, I, P, P]),
        "orc_dequant_w8": (I, [P, P, I64, I64, I, I, P]),
        "orc_device_bytes_w8": (I64, [I64, I64]),
        "orc_pack_device_w8": (I, [P, I64, I64, P]),
        "orc_unpack_device_w8": (I, [P, I64, I64, P]),
        "orc_gemm_rows_w8_f64": (I, [I64, I64, I64, I, P, P, P, I64, I64, P]),
        "orc_kv_quantize": (I, [P, I, I64, I64, P, I64, P, P, P]),
        "orc_quantize_groups_scaled": (I, [P, I, I64, I64, I, I, P, P, P, P]),
        "orc_quantize_mxfp4": (I, [P, I, I64, I64, P, P]),
        "orc_dequant_mxfp4": (I, [P, P, I64, I64, I, P]),
        "orc_pack_device_mxfp4": (I, [P, I64, I64, P]),
        "orc_gemm_rows_mxfp4_f64": (I, [I64, I64, I64, P, P, P, I64, I64, P]),
        "orc_quantize_nvfp4": (I, [P, I, I64, I64, P, P, P]),
        "orc_dequant_nvfp4": (I, [P, P, ctypes.c_float, I64, I64, I, P]),
        "orc_gemm_rows_nvfp4_f64": (I, [I64, I64, I64, P, P, P, ctypes.c_float, I64, I64, P]),
        "orc_scale_activations": (I, [P, I64, I64, P, P]),
        "orc_channel_absmean": (I, [P, I64, I64, P]),
        "orc_kv_dequant": (I, [P, P, P, I64, I64, P, I64, I, P]),
        "orc_bits_per_weight": (ctypes.c_double, [I, I, I, I]),
        "orc_storage_bytes": (ctypes.c_double, [I64, I, I, I, I]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


class OracleError(RuntimeError):
    pass


def _check(status: int, what: str):
    if status != 0:
        raise OracleError(f"{what} failed with status {status}")


def set_threads(n: int) -> None:
    _load().orc_set_threads(int(n))


def get_threads() -> int:
    return int(_load().orc_get_threads())


# --- number formats ---------------------------------------------------------

def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> fp16 bit patterns, round to nearest even, subnormals kept."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, np.uint16)
    _load().orc_f32_to_f16_array(_ptr(a), a.size, _ptr(out))
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns, round to nearest even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, np.uint16)
    _load().orc_f32_to_bf16_array(_ptr(a), a.size, _ptr(out))
    return out


def f16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    lib = _load()
    h = np.ascontiguousarray(h, np.uint16).ravel()
    return np.array([lib.orc_f16_to_f32(int(v)) for v in h], np.float32)


# --- quantizer ---------------------------------------------------------------

ASYM, SYM = 0, 1


def quantize_groups(W: np.ndarray, group: int, dtype: int | None = None, scheme: int = ASYM, alpha=None):
    """Group-wise INT4 quantization of W[N][K].  ASYM: the pages' "minimum
    maths" (s = (max - min)/15, z = round(-min/s), q = clip(round(w/s + z), 0,
    15)).  SYM: symmetric 4-bit (s = max|w|/7, q = clip(round(w/s), -7, 7),
    stored as q + 8 with zero-point 8).

    ``W`` is float32, or uint16 bit patterns with ``dtype`` BF16 or F16.
    ``alpha`` (float32 [K], optional): the AWQ fold, each weight multiplied
    by its input channel's factor (one fp32 multiplication) before quantizing.
    Returns (q[N][K] uint8, s[N][K/g] uint16 fp16 bits, z[N][K/g] uint8).
    """
    W = np.ascontiguousarray(W)
    if dtype is None:
        if W.dtype == np.float32:
            dtype = F32
        else:
            raise ValueError("give dtype for non-float32 input")
    N, K = W.shape
    G = K // group
    q = np.empty((N, K), np.uint8)
    s = np.empty((N, G), np.uint16)
    z = np.empty((N, G), np.uint8)
    a = None if alpha is None else np.ascontiguousarray(alpha, np.float32)
    assert a is None or a.shape == (K,)
    _check(_load().orc_quantize_groups_scaled(_ptr(W), dtype, N, K, group, scheme, None if a is None else _ptr(a),
                                              _ptr(q), _ptr(s), _ptr(z)), "orc_quantize_groups")
    return q, s, z


def dequant(q: np.ndarray, s: np.ndarray, z: np.ndarray, group: int, out_dtype: int = F32) -> np.ndarray:
    """w_hat = s * (q - z) (the pages' decoding), as fp32 values or fp16/bf16 bits."""
    q = np.ascontiguousarray(q, np.uint8)
    s = np.ascontiguousarray(s, np.uint16)
    z = np.ascontiguousarray(z, np.uint8)
    N, K = q.shape
    out = np.empty((N, K), np.float32 if out_dtype == F32 else np.uint16)
    _check(_load().orc_dequant(_ptr(q), _ptr(s), _ptr(z), N, K, group, out_dtype, _ptr(out)), "orc_dequant")
    return out


# --- packing -----------------------------------------------------------------

def pack_canonical(q: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, np.uint8)
    N, K = q.shape
    out = np.empty((N, K // 2), np.uint8)
    _check(_load().orc_pack_canonical(_ptr(q), N, K, _ptr(out)), "orc_pack_canonical")
    return out


def device_bytes(N: int, K: int) -> int:
    return int(_load().orc_device_bytes(N, K))


def pack_device(q: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, np.uint8)
    N, K = q.shape
    out = np.empty(device_bytes(N, K), np.uint8)
    _check(_load().orc_pack_device(_ptr(q), N, K, _ptr(out)), "orc_pack_device")
    return out


def unpack_device(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, np.uint8)
    q = np.empty((N, K), np.uint8)
    _check(_load().orc_unpack_device(_ptr(packed), N, K, _ptr(q)), "orc_unpack_device")
    return q


def pack_zeros(z: np.ndarray) -> np.ndarray:
    z = np.ascontiguousarray(z, np.uint8)
    N, G = z.shape
    out = np.empty((N, (G + 1) // 2), np.uint8)
    _check(_load().orc_pack_zeros(_ptr(z), N, G, _ptr(out)), "orc_pack_zeros")
    return out


# --- product -------------------------------------------------------------------

def gemm_f64(x_f16_bits: np.ndarray, w_hat: np.ndarray) -> np.ndarray:
    """y[m][n] = sum_k x[m][k] * w_hat[n][k], in fp64, summed in k order."""
    x = np.ascontiguousarray(x_f16_bits, np.uint16)
    w = np.ascontiguousarray(w_hat, np.float32)
    M, K = x.shape
    N, K2 = w.shape
    assert K == K2
    y = np.empty((M, N), np.float64)
    _check(_load().orc_gemm_f64(M, N, K, _ptr(x), _ptr(w), _ptr(y)), "orc_gemm_f64")
    return y


def gemm_rows_f64(x_f16_bits, q, s, z, group: int, n0: int, nrows: int) -> np.ndarray:
    """Columns n0..n0+nrows-1 of y (all M rows), from codes/scales/zeros."""
    x = np.ascontiguousarray(x_f16_bits, np.uint16)
    q = np.ascontiguousarray(q, np.uint8)
    s = np.ascontiguousarray(s, np.uint16)
    z = np.ascontiguousarray(z, np.uint8)
    M, K = x.shape
    N = q.shape[0]
    y = np.empty((M, nrows), np.float64)
    _check(_load().orc_gemm_rows_f64(M, N, K, group, _ptr(x), _ptr(q), _ptr(s), _ptr(z), n0, nrows, _ptr(y)),
           "orc_gemm_rows_f64")
    return y


# --- group absmax int8 (W8A16) ---------------------------------------------

def quantize_w8(W: np.ndarray, group: int, dtype: int | None = None):
    """Group absmax int8 ("Quantization Methods Compared", section "What
    quantisation does": s = max|w| / 127, q = round(w / s)) with an fp16 scale
    per group of ``group`` weights along K: s = fp16(fl32(max|w| / 127)),
    q = clip(rne(fl32(w / s)), -127, 127); a zero scale gives codes 0.
    Returns (q[N][K] int8, s[N][K/g] uint16 fp16 bits)."""
    W = np.ascontiguousarray(W)
    if dtype is None:
        if W.dtype == np.float32:
            dtype = F32
        else:
            raise ValueError("give dtype for non-float32 input")
    N, K = W.shape
    q = np.empty((N, K), np.int8)
    s = np.empty((N, K // group), np.uint16)
    _check(_load().orc_quantize_w8(_ptr(W), dtype, N, K, group, _ptr(q), _ptr(s)), "orc_quantize_w8")
    return q, s


def dequant_w8(q: np.ndarray, s: np.ndarray, group: int, out_dtype: int = F32) -> np.ndarray:
    """w_hat = s * q (exact in fp32), as fp32 values or fp16/bf16 bits."""
    q = np.ascontiguousarray(q, np.int8)
    s = np.ascontiguousarray(s, np.uint16)
    N, K = q.shape
    out = np.empty((N, K), np.float32 if out_dtype == F32 else np.uint16)
    _check(_load().orc_dequant_w8(_ptr(q), _ptr(s), N, K, group, out_dtype, _ptr(out)), "orc_dequant_w8")
    return out


def device_bytes_w8(N: int, K: int) -> int:
    return int(_load().orc_device_bytes_w8(N, K))


def pack_device_w8(q: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, np.int8)
    N, K = q.shape
    out = np.empty(device_bytes_w8(N, K), np.uint8)
    _check(_load().orc_pack_device_w8(_ptr(q), N, K, _ptr(out)), "orc_pack_device_w8")
    return out


def unpack_device_w8(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, np.uint8)
    q = np.empty((N, K), np.int8)
    _check(_load().orc_unpack_device_w8(_ptr(packed), N, K, _ptr(q)), "orc_unpack_device_w8")
    return q


def gemm_rows_w8_f64(x_f16_bits, q, s, group: int, n0: int, nrows: int) -> np.ndarray:
    """Columns n0..n0+nrows-1 of y = x * (s * q)^T (all M rows), in fp64."""
    x = np.ascontiguousarray(x_f16_bits, np.uint16)
    q = np.ascontiguousarray(q, np.int8)
    s = np.ascontiguousarray(s, np.uint16)
    M, K = x.shape
    N = q.shape[0]
    y = np.empty((M, nrows), np.float64)
    _check(_load().orc_gemm_rows_w8_f64(M, N, K, group, _ptr(x), _ptr(q), _ptr(s), n0, nrows, _ptr(y)),
           "orc_gemm_rows_w8_f64")
    return y


# --- MXFP4 (E2M1 elements, blocks of 32, E8M0 scale) ---------------------------

def quantize_mxfp4(W: np.ndarray, dtype: int | None = None):
    """MXFP4 quantization of W[N][K] (K a multiple of 32): per block of 32
    along K an E8M0 scale 2^(floor(log2 max|w|) - 2) and E2M1 codes (nearest,
    ties to even, saturating at 6; sign in bit 3).  Returns (q uint8 [N][K],
    e8 uint8 [N][K/32])."""
    W = np.ascontiguousarray(W)
    if dtype is None:
        if W.dtype == np.float32:
            dtype = F32
        else:
            raise ValueError("give dtype for non-float32 input")
    N, K = W.shape
    q = np.empty((N, K), np.uint8)
    e8 = np.empty((N, K // 32), np.uint8)
    _check(_load().orc_quantize_mxfp4(_ptr(W), dtype, N, K, _ptr(q), _ptr(e8)), "orc_quantize_mxfp4")
    return q, e8


def dequant_mxfp4(q: np.ndarray, e8: np.ndarray, out_dtype: int = F32) -> np.ndarray:
    q = np.ascontiguousarray(q, np.uint8)
    e8 = np.ascontiguousarray(e8, np.uint8)
    N, K = q.shape
    out = np.empty((N, K), np.float32 if out_dtype == F32 else np.uint16)
    _check(_load().orc_dequant_mxfp4(_ptr(q), _ptr(e8), N, K, out_dtype, _ptr(out)), "orc_dequant_mxfp4")
    return out


def pack_device_mxfp4(q: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, np.uint8)
    N, K = q.shape
    out = np.empty(device_bytes(N, K), np.uint8)
    _check(_load().orc_pack_device_mxfp4(_ptr(q), N, K, _ptr(out)), "orc_pack_device_mxfp4")
    return out


def gemm_rows_mxfp4_f64(x_f16_bits, q, e8, n0: int, nrows: int) -> np.ndarray:
    x = np.ascontiguousarray(x_f16_bits, np.uint16)
    q = np.ascontiguousarray(q, np.uint8)
    e8 = np.ascontiguousarray(e8, np.uint8)
    M, K = x.shape
    N = q.shape[0]
    y = np.empty((M, nrows), np.float64)
    _check(_load().orc_gemm_rows_mxfp4_f64(M, N, K, _ptr(x), _ptr(q), _ptr(e8), n0, nrows, _ptr(y)),
           "orc_gemm_rows_mxfp4_f64")
    return y


# --- NVFP4 (E2M1 elements, blocks of 16, E4M3 scale, fp32 tensor scale) -------

def quantize_nvfp4(W: np.ndarray, dtype: int | None = None):
    """NVFP4 quantization of W[N][K] (K a multiple of 16): the per-tensor fp32
    scale S = fp32(max|W| / (6 * 448)); per block of 16 along K the E4M3 scale
    byte nearest to the block's max|w| / (6 S), and E2M1 codes nearest to
    w / (E4M3 * S) (ties to even, saturating; sign in bit 3).  Returns
    (q uint8 [N][K], s8 uint8 [N][K/16], S float)."""
    W = np.ascontiguousarray(W)
    if dtype is None:
        if W.dtype == np.float32:
            dtype = F32
        else:
            raise ValueError("give dtype for non-float32 input")
    N, K = W.shape
    q = np.empty((N, K), np.uint8)
    s8 = np.empty((N, K // 16), np.uint8)
    S = np.zeros(1, np.float32)
    _check(_load().orc_quantize_nvfp4(_ptr(W), dtype, N, K, _ptr(q), _ptr(s8), _ptr(S)), "orc_quantize_nvfp4")
    return q, s8, float(S[0])


def dequant_nvfp4(q: np.ndarray, s8: np.ndarray, tensor_scale: float, out_dtype: int = F32) -> np.ndarray:
    q = np.ascontiguousarray(q, np.uint8)
    s8 = np.ascontiguousarray(s8, np.uint8)
    N, K = q.shape
    out = np.empty((N, K), np.float32 if out_dtype == F32 else np.uint16)
    _check(_load().orc_dequant_nvfp4(_ptr(q), _ptr(s8), tensor_scale, N, K, out_dtype, _ptr(out)),
           "orc_dequant_nvfp4")
    return out


def gemm_rows_nvfp4_f64(x_f16_bits, q, s8, tensor_scale: float, n0: int, nrows: int) -> np.ndarray:
    x = np.ascontiguousarray(x_f16_bits, np.uint16)
    q = np.ascontiguousarray(q, np.uint8)
    s8 = np.ascontiguousarray(s8, np.uint8)
    M, K = x.shape
    N = q.shape[0]
    y = np.empty((M, nrows), np.float64)
    _check(_load().orc_gemm_rows_nvfp4_f64(M, N, K, _ptr(x), _ptr(q), _ptr(s8), tensor_scale, n0, nrows, _ptr(y)),
           "orc_gemm_rows_nvfp4_f64")
    return y


# --- AWQ-style per-input-channel scaling --------------------------------------

def scale_activations(x_f16_bits: np.ndarray, alpha) -> np.ndarray:
    """x' = fp16(fl32(x / alpha[k])) (the activation side of the AWQ fold)."""
    x = np.ascontiguousarray(x_f16_bits, np.uint16)
    a = np.ascontiguousarray(alpha, np.float32)
    M, K = x.shape
    out = np.empty((M, K), np.uint16)
    _check(_load().orc_scale_activations(_ptr(x), M, K, _ptr(a), _ptr(out)), "orc_scale_activations")
    return out


def channel_absmean(x_f16_bits: np.ndarray) -> np.ndarray:
    """Mean |x| of each input channel (fp32 sum in row order, then / M)."""
    x = np.ascontiguousarray(x_f16_bits, np.uint16)
    M, K = x.shape
    out = np.empty(K, np.float32)
    _check(_load().orc_channel_absmean(_ptr(x), M, K, _ptr(out)), "orc_channel_absmean")
    return out


# --- INT4 KV cache in blocks of 128 ------------------------------------------

def kv_alloc(S: int, hd: int):
    """Empty (zero-filled) cache arrays for S rows of hd values."""
    nb = hd // 128
    return (np.zeros((S, hd // 2), np.uint8), np.zeros((S, nb), np.uint16), np.zeros((S, (nb + 1) // 2), np.uint8))


def kv_quantize(X: np.ndarray, cache, slot=None, dtype: int | None = None):
    """Quantizes each token's vector X[t] (hd values, blocks of 128: the
    "KV cache quantization" section's int4 cache) into cache row slot[t]
    (default t), in place; slots outside the cache are skipped."""
    X = np.ascontiguousarray(X)
    if dtype is None:
        if X.dtype == np.float32:
            dtype = F32
        else:
            raise ValueError("give dtype for non-float32 input")
    T, hd = X.shape
    codes, s, z = cache
    sl = None if slot is None else np.ascontiguousarray(slot, np.int32)
    _check(_load().orc_kv_quantize(_ptr(X), dtype, T, hd, None if sl is None else _ptr(sl), codes.shape[0],
                                   _ptr(codes), _ptr(s), _ptr(z)), "orc_kv_quantize")
    return cache


def kv_dequant(cache, T: int, hd: int, slot=None, out_dtype: int = F32) -> np.ndarray:
    codes, s, z = cache
    sl = None if slot is None else np.ascontiguousarray(slot, np.int32)
    out = np.empty((T, hd), np.float32 if out_dtype == F32 else np.uint16)
    _check(_load().orc_kv_dequant(_ptr(codes), _ptr(s), _ptr(z), T, hd, None if sl is None else _ptr(sl),
                                  codes.shape[0], out_dtype, _ptr(out)), "orc_kv_dequant")
    return out


# --- symmetric quantizers and storage ----------------------------------------

def symmetric(w, bits: int):
    """Symmetric absmax quantizer: s = max|w| / (2^(bits-1) - 1), q = round(w/s)."""
    w = np.ascontiguousarray(w, np.float64).ravel()
    q = np.empty(w.shape, np.int32)
    s = ctypes.c_double()
    w_hat = np.empty(w.shape, np.float64)
    _check(_load().orc_symmetric(_ptr(w), w.size, bits, _ptr(q), ctypes.byref(s), _ptr(w_hat)), "orc_symmetric")
    return q, s.value, w_hat


def bits_per_weight(bits: int, group: int, scale_bits: int = 16, zero_bits: int = 0) -> float:
    return float(_load().orc_bits_per_weight(bits, group, scale_bits, zero_bits))


def storage_bytes(n: int, bits: int, group: int, scale_bits: int = 16, zero_bits: int = 0) -> float:
    return float(_load().orc_storage_bytes(n, bits, group, scale_bits, zero_bits))
