"""libwq: group-wise asymmetric INT4 weight quantization and the fused W4A16
matmul for AMD MI355X (gfx950).

This module is the thin Python binding of the C ABI declared in
``include/libwq.h``: it marshals torch device tensors (PyTorch supplies device
memory and streams only) into the C calls of the same names.  Every step of the
computation runs in the HIP kernels of ``libwq.so``; there is no other path.
If the library has not been built, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwq.so")

WQ_OK, WQ_EINVAL, WQ_EUNSUPPORTED, WQ_EALIGN, WQ_EWORKSPACE, WQ_EHIP = 0, -1, -2, -3, -4, -5
WQ_F32, WQ_BF16, WQ_F16 = 0, 1, 2
WQ_PATH_AUTO, WQ_PATH_GEMV, WQ_PATH_MFMA = 0, 1, 2
WQ_ASYM, WQ_SYM = 0, 1
WQ_AUTO_GEMV_MAX_N = 2048  # WQ_PATH_AUTO: every format keeps the GEMV up to
WQ_AUTO_NARROW_GEMV_MAX_M = 32  # this many rows when N <= WQ_AUTO_GEMV_MAX_N; otherwise up to
WQ_AUTO_INT4_GEMV_MAX_M = 16  # this many rows of 4-bit integer codes (at group 32 with
WQ_AUTO_INT4_G32_LONG_K = 16384  # K above this only up to
WQ_AUTO_INT4_G32_LONG_K_GEMV_MAX_M = 8  # this many),
WQ_AUTO_FP4_GEMV_MAX_M = 16  # this many rows of MXFP4 / NVFP4 codes
WQ_AUTO_INT8_GEMV_MAX_M = 8  # and this many rows of int8 codes


def auto_uses_mfma(M: int, N: int, fmt: str = "int4", K: int | None = None, group: int | None = None) -> bool:
    """Whether WQ_PATH_AUTO runs the MFMA GEMM kernel for M rows, N outputs and
    K inputs of code format fmt ("int4", "int8", "mxfp4" or "nvfp4"): the
    library's rule, restated.  4-bit integer codes need K and group."""
    if fmt not in ("int4", "int8", "mxfp4", "nvfp4"):
        raise ValueError(f"unknown code format {fmt!r}")
    if M <= WQ_AUTO_NARROW_GEMV_MAX_M and N <= WQ_AUTO_GEMV_MAX_N:
        return False
    if fmt == "int4":
        if K is None or group is None:
            raise ValueError("the 4-bit rule depends on K and group")
        long_k = group == 32 and K > WQ_AUTO_INT4_G32_LONG_K
        return M > (WQ_AUTO_INT4_G32_LONG_K_GEMV_MAX_M if long_k else WQ_AUTO_INT4_GEMV_MAX_M)
    if fmt in ("mxfp4", "nvfp4"):
        return M > WQ_AUTO_FP4_GEMV_MAX_M
    return M > WQ_AUTO_INT8_GEMV_MAX_M


WQ_WORKSPACE_COUNTER_BYTES = 2048  # leading counter bytes of a split-K workspace (zero before first use)
WQ_NOALLOC_SCRATCH_BYTES = WQ_WORKSPACE_COUNTER_BYTES + (16 << 20)  # per-GPU scratch of wq_gemm_w4a16_noalloc

EXPORTED = (
    "wq_version", "wq_strerror", "wq_layout_bytes", "wq_quantize_groups", "wq_quantize_groups_ex", "wq_pack_int4",
    "wq_dequant",
    "wq_gemm_workspace_bytes", "wq_gemm_workspace_bytes_ex", "wq_gemm_plan", "wq_gemm_w4a16", "wq_gemm_w4a16_ex", "wq_gemm_w4a16_seq",
    "wq_gemm_w4a16_noalloc",
    "wq_layout_bytes_w8", "wq_quantize_w8", "wq_pack_int8", "wq_dequant_w8", "wq_gemm_w8a16_workspace_bytes",
    "wq_gemm_w8a16", "wq_gemm_w8a16_ex", "wq_gemm_w8a16_plan",
    "wq_kv_layout_bytes", "wq_kv_quantize", "wq_kv_dequant",
    "wq_quantize_groups_scaled", "wq_scale_activations", "wq_channel_absmean",
    "wq_layout_bytes_mxfp4", "wq_quantize_mxfp4", "wq_pack_mxfp4", "wq_dequant_mxfp4",
    "wq_gemm_mxfp4_workspace_bytes", "wq_gemm_mxfp4", "wq_gemm_mxfp4_ex", "wq_gemm_mxfp4_plan",
    "wq_layout_bytes_nvfp4", "wq_quantize_nvfp4", "wq_dequant_nvfp4",
    "wq_gemm_nvfp4_workspace_bytes", "wq_gemm_nvfp4", "wq_gemm_nvfp4_ex", "wq_gemm_nvfp4_plan",
    "wq_read_probe", "wq_mfma_probe", "wq_clock_probe",
)

_lib = None


class WQError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {strerror(status)} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libwq.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first (python __graft_entry__.py or "
                          f"python w4a16_bit_matmul_amd/_build.py)")
    L = ctypes.CDLL(LIB_PATH)
    P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "wq_version": (I, []),
        "wq_strerror": (ctypes.c_char_p, [I]),
        "wq_layout_bytes": (I, [I64, I64, I, ctypes.POINTER(SZ), ctypes.POINTER(SZ), ctypes.POINTER(SZ)]),
        "wq_quantize_groups": (I, [P, I, I64, I64, I, P, P, P, P, P, P]),
        "wq_quantize_groups_ex": (I, [P, I, I64, I64, I, I, P, P, P, P, P, P]),
        "wq_pack_int4": (I, [P, P, I64, I64, I, P, P, P]),
        "wq_dequant": (I, [P, P, P, I64, I64, I, I, P, P]),
        "wq_gemm_workspace_bytes": (SZ, [I64, I64, I64, I]),
        "wq_gemm_workspace_bytes_ex": (SZ, [I64, I64, I64, I, I]),
        "wq_gemm_plan": (I, [I64, I64, I64, I, I, ctypes.c_char_p, SZ]),
        "wq_gemm_w4a16": (I, [I64, I64, I64, I, P, P, P, P, P, P, SZ, P]),
        "wq_gemm_w4a16_ex": (I, [I64, I64, I64, I, P, P, P, P, P, P, SZ, I, P]),
        "wq_gemm_w4a16_seq": (I, [I, I64, I64, I64, I, P, P, P, P, P, P, SZ, P]),
        "wq_gemm_w4a16_noalloc": (I, [I64, I64, I64, I, P, P, P, P, P, P]),
        "wq_layout_bytes_w8": (I, [I64, I64, I, ctypes.POINTER(SZ), ctypes.POINTER(SZ)]),
        "wq_quantize_w8": (I, [P, I, I64, I64, I, P, P, P, P]),
        "wq_pack_int8": (I, [P, I64, I64, P, P]),
        "wq_dequant_w8": (I, [P, P, I64, I64, I, I, P, P]),
        "wq_gemm_w8a16_workspace_bytes": (SZ, [I64, I64, I64, I]),
        "wq_gemm_w8a16": (I, [I64, I64, I64, I, P, P, P, P, P, SZ, P]),
        "wq_gemm_w8a16_ex": (I, [I64, I64, I64, I, P, P, P, P, P, SZ, I, P]),
        "wq_gemm_w8a16_plan": (I, [I64, I64, I64, I, I, ctypes.c_char_p, SZ]),
        "wq_kv_layout_bytes": (I, [I64, I64, ctypes.POINTER(SZ), ctypes.POINTER(SZ), ctypes.POINTER(SZ)]),
        "wq_kv_quantize": (I, [P, I, I64, I64, P, I64, P, P, P, P]),
        "wq_kv_dequant": (I, [P, P, P, I64, I64, P, I64, I, P, P]),
        "wq_quantize_groups_scaled": (I, [P, I, I64, I64, I, I, P, P, P, P, P, P, P]),
        "wq_scale_activations": (I, [P, I64, I64, P, P, P]),
        "wq_channel_absmean": (I, [P, I64, I64, P, P]),
        "wq_layout_bytes_mxfp4": (I, [I64, I64, ctypes.POINTER(SZ), ctypes.POINTER(SZ)]),
        "wq_quantize_mxfp4": (I, [P, I, I64, I64, P, P, P, P]),
        "wq_pack_mxfp4": (I, [P, I64, I64, P, P]),
        "wq_dequant_mxfp4": (I, [P, P, I64, I64, I, P, P]),
        "wq_gemm_mxfp4_workspace_bytes": (SZ, [I64, I64, I64]),
        "wq_gemm_mxfp4": (I, [I64, I64, I64, P, P, P, P, P, SZ, P]),
        "wq_gemm_mxfp4_ex": (I, [I64, I64, I64, P, P, P, P, P, SZ, I, P]),
        "wq_gemm_mxfp4_plan": (I, [I64, I64, I64, I, ctypes.c_char_p, SZ]),
        "wq_layout_bytes_nvfp4": (I, [I64, I64, ctypes.POINTER(SZ), ctypes.POINTER(SZ)]),
        "wq_quantize_nvfp4": (I, [P, I, I64, I64, P, P, P, P, P]),
        "wq_dequant_nvfp4": (I, [P, P, P, I64, I64, I, P, P]),
        "wq_gemm_nvfp4_workspace_bytes": (SZ, [I64, I64, I64]),
        "wq_gemm_nvfp4": (I, [I64, I64, I64, P, P, P, P, P, P, SZ, P]),
        "wq_gemm_nvfp4_ex": (I, [I64, I64, I64, P, P, P, P, P, P, SZ, I, P]),
        "wq_gemm_nvfp4_plan": (I, [I64, I64, I64, I, ctypes.c_char_p, SZ]),
        "wq_read_probe": (I, [P, SZ, SZ, I, I, I, P, P]),
        "wq_mfma_probe": (I, [I, I, I, P, P]),
        "wq_clock_probe": (I, [I, ctypes.c_uint32, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def strerror(status: int) -> str:
    return lib().wq_strerror(status).decode()


def _check(status: int, what: str) -> None:
    if status != WQ_OK:
        raise WQError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_obj(stream=None):
    return torch.cuda.current_stream() if stream is None else stream


def _stream(stream=None):
    return ctypes.c_void_p(_stream_obj(stream).cuda_stream)


# Workspaces of calls that pass none: one per (device, stream), grown on
# demand.  It is allocated and zero-filled on the stream the products run on,
# so the zeros are in place before the first product reads its counters, and
# products on one stream run in order, so they can share it (each leaves its
# counters zero again).  Concurrent streams get separate workspaces.
_workspaces: dict = {}


def _default_workspace(need: int, device: torch.device, stream=None):
    if not need:
        return None
    s = _stream_obj(stream)
    key = (device.index if device.index is not None else torch.cuda.current_device(), s.cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < need:
        with torch.cuda.stream(s):
            ws = torch.zeros(need, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def _check_x(x: torch.Tensor, K: int, weight: torch.Tensor) -> int:
    """x must be a contiguous fp16 [M][K] tensor on the weights' device."""
    if x.dtype != torch.float16 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError(f"x must be a contiguous 2-D float16 tensor (got {x.dtype}, shape {tuple(x.shape)})")
    if x.shape[1] != K:
        raise ValueError(f"x has K={x.shape[1]}, the weight K={K}")
    if x.device != weight.device:
        raise ValueError(f"x is on {x.device}, the weight on {weight.device}")
    return x.shape[0]


def _out_y(y, M: int, N: int, x: torch.Tensor) -> torch.Tensor:
    """The output tensor: a new fp16 [M][N] tensor, or the caller's, which must
    be exactly that (shape, dtype, contiguous, on x's device)."""
    if y is None:
        return torch.empty((M, N), dtype=torch.float16, device=x.device)
    if y.shape != (M, N) or y.dtype != torch.float16 or not y.is_contiguous() or y.device != x.device:
        raise ValueError(f"y must be a contiguous float16 [{M}][{N}] tensor on {x.device} "
                         f"(got {y.dtype}, shape {tuple(y.shape)}, on {y.device})")
    return y


_DT = {torch.float32: WQ_F32, torch.bfloat16: WQ_BF16, torch.float16: WQ_F16}


@dataclass
class QuantizedWeight:
    """Device buffers of one quantized [N][K] weight matrix."""
    qpacked: torch.Tensor  # uint8, tile layout (wq_layout_bytes)
    s: torch.Tensor        # float16 [N][K/group]
    zpacked: torch.Tensor  # uint8 [N][ceil(G/2)]
    N: int
    K: int
    group: int


def wq_version() -> int:
    return int(lib().wq_version())


def wq_layout_bytes(N: int, K: int, group: int):
    q, s, z = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().wq_layout_bytes(N, K, group, ctypes.byref(q), ctypes.byref(s), ctypes.byref(z)), "wq_layout_bytes")
    return q.value, s.value, z.value


def wq_gemm_workspace_bytes(M: int, N: int, K: int, group: int, path: int | None = None) -> int:
    """Workspace bytes for either kernel family (path None), or for the one
    family `path` selects."""
    if path is None:
        return int(lib().wq_gemm_workspace_bytes(M, N, K, group))
    return int(lib().wq_gemm_workspace_bytes_ex(M, N, K, group, path))


def wq_gemm_plan(M: int, N: int, K: int, group: int, path: int = WQ_PATH_AUTO) -> str:
    """One-line description of the kernel and launch shape wq_gemm_w4a16 uses."""
    buf = ctypes.create_string_buffer(256)
    _check(lib().wq_gemm_plan(M, N, K, group, path, buf, len(buf)), "wq_gemm_plan")
    return buf.value.decode()


def alloc_quantized(N: int, K: int, group: int, device="cuda") -> QuantizedWeight:
    qb, _, zb = wq_layout_bytes(N, K, group)
    return QuantizedWeight(torch.empty(qb, dtype=torch.uint8, device=device),
                           torch.empty((N, K // group), dtype=torch.float16, device=device),
                           torch.empty((N, zb // N), dtype=torch.uint8, device=device), N, K, group)


def wq_quantize_groups(W: torch.Tensor, group: int, *, codes: bool = False, packed: bool = True,
                       out: QuantizedWeight | None = None, scheme: int = WQ_ASYM, alpha: torch.Tensor | None = None,
                       stream=None):
    """Quantize W[N][K] (float32, bfloat16 or float16, on the GPU) with the
    asymmetric (WQ_ASYM) or symmetric (WQ_SYM: codes q + 8, zero-point 8)
    4-bit scheme; with ``alpha`` (float32 [K] on the GPU) the weights are first
    multiplied by the per-input-channel factors (wq_quantize_groups_scaled).

    Returns a dict with ``s`` (fp16 [N][G]) and, as requested, ``q_codes``
    (uint8 [N][K]), ``z_codes`` (uint8 [N][G]) and ``qw`` (QuantizedWeight with
    the packed device layouts)."""
    N, K = W.shape
    G = K // group if group else 0
    dev = W.device
    qw = out
    if packed and qw is None:
        qw = alloc_quantized(N, K, group, dev)
    s = qw.s if packed else torch.empty((N, G), dtype=torch.float16, device=dev)
    q_codes = torch.empty((N, K), dtype=torch.uint8, device=dev) if codes else None
    z_codes = torch.empty((N, G), dtype=torch.uint8, device=dev) if codes else None
    assert alpha is None or (alpha.dtype == torch.float32 and alpha.numel() == K and alpha.is_contiguous())
    _check(lib().wq_quantize_groups_scaled(_ptr(W), _DT.get(W.dtype, -1), N, K, group, scheme, _ptr(alpha),
                                           _ptr(q_codes), _ptr(s), _ptr(z_codes), _ptr(qw.qpacked) if packed else None,
                                           _ptr(qw.zpacked) if packed else None, _stream(stream)),
           "wq_quantize_groups")
    return {"s": s, "q_codes": q_codes, "z_codes": z_codes, "qw": qw if packed else None}


def wq_pack_int4(q_codes: torch.Tensor, z_codes: torch.Tensor, group: int, stream=None) -> QuantizedWeight:
    """Pack codes [N][K] and zero-points [N][G] into the device layouts (the
    returned QuantizedWeight's ``s`` is left uninitialised)."""
    N, K = q_codes.shape
    qw = alloc_quantized(N, K, group, q_codes.device)
    _check(lib().wq_pack_int4(_ptr(q_codes), _ptr(z_codes), N, K, group, _ptr(qw.qpacked), _ptr(qw.zpacked),
                              _stream(stream)), "wq_pack_int4")
    return qw


def wq_dequant(qw: QuantizedWeight, out_dtype=torch.float32, stream=None) -> torch.Tensor:
    out = torch.empty((qw.N, qw.K), dtype=out_dtype, device=qw.qpacked.device)
    _check(lib().wq_dequant(_ptr(qw.qpacked), _ptr(qw.s), _ptr(qw.zpacked), qw.N, qw.K, qw.group,
                            _DT.get(out_dtype, -1), _ptr(out), _stream(stream)), "wq_dequant")
    return out


def wq_gemm_w4a16(x: torch.Tensor, qw: QuantizedWeight, *, y: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, path: int = WQ_PATH_AUTO, stream=None) -> torch.Tensor:
    """y[M][N] = x[M][K] * What^T, What = s * (q - z), fp16 in and out.
    Without a workspace, a split-K shape uses the binding's workspace for this
    stream (allocated once, zero-filled on the stream)."""
    M = _check_x(x, qw.K, qw.qpacked)
    y = _out_y(y, M, qw.N, x)
    if workspace is None:
        workspace = _default_workspace(wq_gemm_workspace_bytes(M, qw.N, qw.K, qw.group), x.device, stream)
    _check(lib().wq_gemm_w4a16_ex(M, qw.N, qw.K, qw.group, _ptr(x), _ptr(qw.qpacked), _ptr(qw.s),
                                  _ptr(qw.zpacked), _ptr(y), _ptr(workspace),
                                  0 if workspace is None else workspace.numel() * workspace.element_size(),
                                  path, _stream(stream)), "wq_gemm_w4a16")
    return y


def wq_gemm_w4a16_noalloc(x: torch.Tensor, qw: QuantizedWeight, *, y: torch.Tensor | None = None,
                          stream=None) -> torch.Tensor:
    """wq_gemm_w4a16 through the allocation-free entry point: its split-K
    scratch is the library's fixed per-GPU array (calls on one GPU must not
    overlap).  With y given, this wrapper allocates nothing either."""
    M = _check_x(x, qw.K, qw.qpacked)
    y = _out_y(y, M, qw.N, x)
    _check(lib().wq_gemm_w4a16_noalloc(M, qw.N, qw.K, qw.group, _ptr(x), _ptr(qw.qpacked), _ptr(qw.s),
                                       _ptr(qw.zpacked), _ptr(y), _stream(stream)), "wq_gemm_w4a16_noalloc")
    return y


def wq_gemm_w4a16_seq_prepared(xs, qws, ys, *, workspace: torch.Tensor | None = None, stream=None):
    """Marshals the arguments of wq_gemm_w4a16_seq once and returns a function
    of no arguments that issues the whole sequence (one C call) on the stream
    current at preparation time.  The buffers stay referenced by the function."""
    count = len(xs)
    assert len(qws) == count and len(ys) == count and count > 0
    q0 = qws[0]
    M = _check_x(xs[0], q0.K, q0.qpacked)
    for x, qw, y in zip(xs, qws, ys):
        assert _check_x(x, q0.K, qw.qpacked) == M and (qw.N, qw.K, qw.group) == (q0.N, q0.K, q0.group)
        _out_y(y, M, q0.N, x)
    if workspace is None:
        workspace = _default_workspace(wq_gemm_workspace_bytes(M, q0.N, q0.K, q0.group), xs[0].device, stream)
    arr = lambda ts: (ctypes.c_void_p * count)(*[t.data_ptr() for t in ts])
    args = (count, M, q0.N, q0.K, q0.group, arr(xs), arr([q.qpacked for q in qws]), arr([q.s for q in qws]),
            arr([q.zpacked for q in qws]), arr(ys), _ptr(workspace),
            0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream))
    fn = lib().wq_gemm_w4a16_seq
    keep = (list(xs), list(qws), list(ys), workspace)

    def call():
        _check(fn(*args), "wq_gemm_w4a16_seq")
        return keep[2]
    return call


def wq_gemm_w4a16_seq(xs, qws, ys, *, workspace: torch.Tensor | None = None, stream=None):
    """ys[i] = xs[i] * What_i^T for every i, issued back to back by one C call
    (wq_gemm_w4a16_seq).  All products have one shape; ys are preallocated
    fp16 [M][N] tensors."""
    if len(xs) == 0:
        return ys
    return wq_gemm_w4a16_seq_prepared(xs, qws, ys, workspace=workspace, stream=stream)()


# ---- group absmax int8 weights (W8A16) --------------------------------------

@dataclass
class QuantizedWeight8:
    """Device buffers of one int8-quantized [N][K] weight matrix."""
    qpacked: torch.Tensor  # uint8, 2048-byte tiles (wq_layout_bytes_w8)
    s: torch.Tensor        # float16 [N][K/group]
    N: int
    K: int
    group: int


def wq_layout_bytes_w8(N: int, K: int, group: int):
    q, s = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().wq_layout_bytes_w8(N, K, group, ctypes.byref(q), ctypes.byref(s)), "wq_layout_bytes_w8")
    return q.value, s.value


def alloc_quantized_w8(N: int, K: int, group: int, device="cuda") -> QuantizedWeight8:
    qb, _ = wq_layout_bytes_w8(N, K, group)
    return QuantizedWeight8(torch.empty(qb, dtype=torch.uint8, device=device),
                            torch.empty((N, K // group), dtype=torch.float16, device=device), N, K, group)


def wq_quantize_w8(W: torch.Tensor, group: int, *, codes: bool = False, packed: bool = True,
                   out: QuantizedWeight8 | None = None, stream=None):
    """Group absmax int8 quantization of W[N][K] (float32, bfloat16 or float16,
    on the GPU).  Returns a dict with ``s`` (fp16 [N][G]) and, as requested,
    ``q_codes`` (int8 [N][K]) and ``qw`` (QuantizedWeight8)."""
    N, K = W.shape
    G = K // group if group else 0
    dev = W.device
    qw = out
    if packed and qw is None:
        qw = alloc_quantized_w8(N, K, group, dev)
    s = qw.s if packed else torch.empty((N, G), dtype=torch.float16, device=dev)
    q_codes = torch.empty((N, K), dtype=torch.int8, device=dev) if codes else None
    _check(lib().wq_quantize_w8(_ptr(W), _DT.get(W.dtype, -1), N, K, group, _ptr(q_codes), _ptr(s),
                                _ptr(qw.qpacked) if packed else None, _stream(stream)), "wq_quantize_w8")
    return {"s": s, "q_codes": q_codes, "qw": qw if packed else None}


def wq_pack_int8(q_codes: torch.Tensor, group: int, stream=None) -> QuantizedWeight8:
    """Pack int8 codes [N][K] into the tile layout (the returned weight's ``s``
    is left uninitialised)."""
    N, K = q_codes.shape
    qw = alloc_quantized_w8(N, K, group, q_codes.device)
    _check(lib().wq_pack_int8(_ptr(q_codes), N, K, _ptr(qw.qpacked), _stream(stream)), "wq_pack_int8")
    return qw


def wq_dequant_w8(qw: QuantizedWeight8, out_dtype=torch.float32, stream=None) -> torch.Tensor:
    out = torch.empty((qw.N, qw.K), dtype=out_dtype, device=qw.qpacked.device)
    _check(lib().wq_dequant_w8(_ptr(qw.qpacked), _ptr(qw.s), qw.N, qw.K, qw.group, _DT.get(out_dtype, -1),
                               _ptr(out), _stream(stream)), "wq_dequant_w8")
    return out


def wq_gemm_w8a16_workspace_bytes(M: int, N: int, K: int, group: int) -> int:
    return int(lib().wq_gemm_w8a16_workspace_bytes(M, N, K, group))


def wq_gemm_w8a16_plan(M: int, N: int, K: int, group: int, path: int = WQ_PATH_AUTO) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(lib().wq_gemm_w8a16_plan(M, N, K, group, path, buf, len(buf)), "wq_gemm_w8a16_plan")
    return buf.value.decode()


def wq_gemm_w8a16(x: torch.Tensor, qw: QuantizedWeight8, *, y: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, path: int = WQ_PATH_AUTO, stream=None) -> torch.Tensor:
    """y[M][N] = x[M][K] * What^T, What = s * q (int8 codes), fp16 in and out
    (workspace as for wq_gemm_w4a16)."""
    M = _check_x(x, qw.K, qw.qpacked)
    y = _out_y(y, M, qw.N, x)
    if workspace is None:
        workspace = _default_workspace(wq_gemm_w8a16_workspace_bytes(M, qw.N, qw.K, qw.group), x.device, stream)
    _check(lib().wq_gemm_w8a16_ex(M, qw.N, qw.K, qw.group, _ptr(x), _ptr(qw.qpacked), _ptr(qw.s), _ptr(y),
                                  _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
                                  path, _stream(stream)), "wq_gemm_w8a16")
    return y


# ---- INT4 KV cache in blocks of 128 -------------------------------------------

@dataclass
class KVCache:
    """Device arrays of an INT4 KV cache of S rows (token slots) of hd values."""
    codes: torch.Tensor  # uint8 [S][hd/2]
    s: torch.Tensor      # float16 [S][hd/128]
    zpacked: torch.Tensor  # uint8 [S][ceil(hd/256)]
    S: int
    hd: int


def wq_kv_layout_bytes(S: int, hd: int):
    c, s, z = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().wq_kv_layout_bytes(S, hd, ctypes.byref(c), ctypes.byref(s), ctypes.byref(z)), "wq_kv_layout_bytes")
    return c.value, s.value, z.value


def kv_cache_alloc(S: int, hd: int, device="cuda") -> KVCache:
    wq_kv_layout_bytes(S, hd)  # validates hd
    nb = hd // 128
    return KVCache(torch.zeros((S, hd // 2), dtype=torch.uint8, device=device),
                   torch.zeros((S, nb), dtype=torch.float16, device=device),
                   torch.zeros((S, (nb + 1) // 2), dtype=torch.uint8, device=device), S, hd)


def wq_kv_quantize(X: torch.Tensor, cache: KVCache, slot: torch.Tensor | None = None, stream=None) -> KVCache:
    """Quantizes X [T][hd] (fp32, bf16 or fp16, on the GPU) into cache rows
    slot[t] (int32 device tensor, or None for rows 0..T-1)."""
    T, hd = X.shape
    assert hd == cache.hd
    assert slot is None or (slot.dtype == torch.int32 and slot.numel() == T and slot.is_contiguous())
    _check(lib().wq_kv_quantize(_ptr(X), _DT.get(X.dtype, -1), T, hd, _ptr(slot), cache.S, _ptr(cache.codes),
                                _ptr(cache.s), _ptr(cache.zpacked), _stream(stream)), "wq_kv_quantize")
    return cache


def wq_kv_dequant(cache: KVCache, T: int, slot: torch.Tensor | None = None, out_dtype=torch.float16,
                  stream=None) -> torch.Tensor:
    assert slot is None or (slot.dtype == torch.int32 and slot.numel() == T and slot.is_contiguous())
    out = torch.empty((T, cache.hd), dtype=out_dtype, device=cache.codes.device)
    _check(lib().wq_kv_dequant(_ptr(cache.codes), _ptr(cache.s), _ptr(cache.zpacked), T, cache.hd, _ptr(slot),
                               cache.S, _DT.get(out_dtype, -1), _ptr(out), _stream(stream)), "wq_kv_dequant")
    return out


# ---- AWQ-style per-input-channel scaling ---------------------------------------

def wq_scale_activations(x: torch.Tensor, alpha: torch.Tensor, out: torch.Tensor | None = None,
                         stream=None) -> torch.Tensor:
    """x' = fp16(x / alpha[k]) for x [M][K] fp16 and alpha float32 [K]."""
    M, K = x.shape
    assert x.dtype == torch.float16 and alpha.dtype == torch.float32 and alpha.numel() == K
    if out is None:
        out = torch.empty_like(x)
    _check(lib().wq_scale_activations(_ptr(x), M, K, _ptr(alpha), _ptr(out), _stream(stream)), "wq_scale_activations")
    return out


def wq_channel_absmean(x: torch.Tensor, stream=None) -> torch.Tensor:
    """Mean |x| per input channel of x [M][K] fp16 (fp32 sum in row order)."""
    M, K = x.shape
    assert x.dtype == torch.float16
    out = torch.empty(K, dtype=torch.float32, device=x.device)
    _check(lib().wq_channel_absmean(_ptr(x), M, K, _ptr(out), _stream(stream)), "wq_channel_absmean")
    return out


# ---- MXFP4 weights (E2M1 codes, blocks of 32, E8M0 scales) ---------------------

@dataclass
class QuantizedWeightMX:
    """Device buffers of one MXFP4-quantized [N][K] weight matrix."""
    qpacked: torch.Tensor  # uint8, 1 KB tiles (natural nibble order)
    e8: torch.Tensor       # uint8 [N][K/32]
    N: int
    K: int


def wq_layout_bytes_mxfp4(N: int, K: int):
    q, e = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().wq_layout_bytes_mxfp4(N, K, ctypes.byref(q), ctypes.byref(e)), "wq_layout_bytes_mxfp4")
    return q.value, e.value


def alloc_quantized_mxfp4(N: int, K: int, device="cuda") -> QuantizedWeightMX:
    qb, _ = wq_layout_bytes_mxfp4(N, K)
    return QuantizedWeightMX(torch.empty(qb, dtype=torch.uint8, device=device),
                             torch.empty((N, K // 32), dtype=torch.uint8, device=device), N, K)


def wq_quantize_mxfp4(W: torch.Tensor, *, codes: bool = False, stream=None):
    """MXFP4 quantization of W[N][K] (float32, bfloat16 or float16, on the GPU).
    Returns a dict with ``qw`` (QuantizedWeightMX) and, if asked, ``q_codes``
    (uint8 [N][K])."""
    N, K = W.shape
    qw = alloc_quantized_mxfp4(N, K, W.device)
    q_codes = torch.empty((N, K), dtype=torch.uint8, device=W.device) if codes else None
    _check(lib().wq_quantize_mxfp4(_ptr(W), _DT.get(W.dtype, -1), N, K, _ptr(q_codes), _ptr(qw.e8), _ptr(qw.qpacked),
                                   _stream(stream)), "wq_quantize_mxfp4")
    return {"qw": qw, "q_codes": q_codes}


def wq_pack_mxfp4(q_codes: torch.Tensor, stream=None) -> QuantizedWeightMX:
    """Pack codes [N][K] into the tile layout (the returned weight's ``e8`` is
    left uninitialised)."""
    N, K = q_codes.shape
    qw = alloc_quantized_mxfp4(N, K, q_codes.device)
    _check(lib().wq_pack_mxfp4(_ptr(q_codes), N, K, _ptr(qw.qpacked), _stream(stream)), "wq_pack_mxfp4")
    return qw


def wq_dequant_mxfp4(qw: QuantizedWeightMX, out_dtype=torch.float32, stream=None) -> torch.Tensor:
    out = torch.empty((qw.N, qw.K), dtype=out_dtype, device=qw.qpacked.device)
    _check(lib().wq_dequant_mxfp4(_ptr(qw.qpacked), _ptr(qw.e8), qw.N, qw.K, _DT.get(out_dtype, -1), _ptr(out),
                                  _stream(stream)), "wq_dequant_mxfp4")
    return out


def wq_gemm_mxfp4_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().wq_gemm_mxfp4_workspace_bytes(M, N, K))


def wq_gemm_mxfp4_plan(M: int, N: int, K: int, path: int = WQ_PATH_AUTO) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(lib().wq_gemm_mxfp4_plan(M, N, K, path, buf, len(buf)), "wq_gemm_mxfp4_plan")
    return buf.value.decode()


def wq_gemm_mxfp4(x: torch.Tensor, qw: QuantizedWeightMX, *, y: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, path: int = WQ_PATH_AUTO, stream=None) -> torch.Tensor:
    """y[M][N] = x[M][K] * What^T with MXFP4 weights, fp16 in and out
    (workspace as for wq_gemm_w4a16)."""
    M = _check_x(x, qw.K, qw.qpacked)
    y = _out_y(y, M, qw.N, x)
    if workspace is None:
        workspace = _default_workspace(wq_gemm_mxfp4_workspace_bytes(M, qw.N, qw.K), x.device, stream)
    _check(lib().wq_gemm_mxfp4_ex(M, qw.N, qw.K, _ptr(x), _ptr(qw.qpacked), _ptr(qw.e8), _ptr(y), _ptr(workspace),
                                  0 if workspace is None else workspace.numel() * workspace.element_size(), path,
                                  _stream(stream)), "wq_gemm_mxfp4")
    return y


# ---- NVFP4 weights (E2M1 codes, blocks of 16, E4M3 scales, fp32 tensor scale) --

@dataclass
class QuantizedWeightNV:
    """Device buffers of one NVFP4-quantized [N][K] weight matrix."""
    qpacked: torch.Tensor       # uint8, 1 KB tiles (the MXFP4 layout)
    s8: torch.Tensor            # uint8 [N][K/16], E4M3 block scales
    tensor_scale: torch.Tensor  # float32 [1]
    N: int
    K: int


def wq_layout_bytes_nvfp4(N: int, K: int):
    q, s = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().wq_layout_bytes_nvfp4(N, K, ctypes.byref(q), ctypes.byref(s)), "wq_layout_bytes_nvfp4")
    return q.value, s.value


def alloc_quantized_nvfp4(N: int, K: int, device="cuda") -> QuantizedWeightNV:
    qb, _ = wq_layout_bytes_nvfp4(N, K)
    return QuantizedWeightNV(torch.empty(qb, dtype=torch.uint8, device=device),
                             torch.empty((N, K // 16), dtype=torch.uint8, device=device),
                             torch.empty(1, dtype=torch.float32, device=device), N, K)


def wq_quantize_nvfp4(W: torch.Tensor, *, codes: bool = False, stream=None):
    """NVFP4 quantization of W[N][K] (float32, bfloat16 or float16, on the GPU).
    Returns a dict with ``qw`` (QuantizedWeightNV) and, if asked, ``q_codes``
    (uint8 [N][K])."""
    N, K = W.shape
    qw = alloc_quantized_nvfp4(N, K, W.device)
    q_codes = torch.empty((N, K), dtype=torch.uint8, device=W.device) if codes else None
    _check(lib().wq_quantize_nvfp4(_ptr(W), _DT.get(W.dtype, -1), N, K, _ptr(q_codes), _ptr(qw.s8),
                                   _ptr(qw.tensor_scale), _ptr(qw.qpacked), _stream(stream)), "wq_quantize_nvfp4")
    return {"qw": qw, "q_codes": q_codes}


def wq_dequant_nvfp4(qw: QuantizedWeightNV, out_dtype=torch.float32, stream=None) -> torch.Tensor:
    out = torch.empty((qw.N, qw.K), dtype=out_dtype, device=qw.qpacked.device)
    _check(lib().wq_dequant_nvfp4(_ptr(qw.qpacked), _ptr(qw.s8), _ptr(qw.tensor_scale), qw.N, qw.K,
                                  _DT.get(out_dtype, -1), _ptr(out), _stream(stream)), "wq_dequant_nvfp4")
    return out


def wq_gemm_nvfp4_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().wq_gemm_nvfp4_workspace_bytes(M, N, K))


def wq_gemm_nvfp4_plan(M: int, N: int, K: int, path: int = WQ_PATH_AUTO) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(lib().wq_gemm_nvfp4_plan(M, N, K, path, buf, len(buf)), "wq_gemm_nvfp4_plan")
    return buf.value.decode()


def wq_gemm_nvfp4(x: torch.Tensor, qw: QuantizedWeightNV, *, y: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, path: int = WQ_PATH_AUTO, stream=None) -> torch.Tensor:
    """y[M][N] = x[M][K] * What^T with NVFP4 weights, fp16 in and out
    (workspace as for wq_gemm_w4a16)."""
    M = _check_x(x, qw.K, qw.qpacked)
    y = _out_y(y, M, qw.N, x)
    if workspace is None:
        workspace = _default_workspace(wq_gemm_nvfp4_workspace_bytes(M, qw.N, qw.K), x.device, stream)
    _check(lib().wq_gemm_nvfp4_ex(M, qw.N, qw.K, _ptr(x), _ptr(qw.qpacked), _ptr(qw.s8), _ptr(qw.tensor_scale),
                                  _ptr(y), _ptr(workspace),
                                  0 if workspace is None else workspace.numel() * workspace.element_size(), path,
                                  _stream(stream)), "wq_gemm_nvfp4")
    return y


def wq_read_probe(src: torch.Tensor, window_bytes: int, count: int, *, chunks: int = 8, nontemporal: bool = False,
                  sink: torch.Tensor | None = None, stream=None) -> None:
    """count streaming reads of window_bytes each, rotating over the bytes of
    the device tensor src (a measurement aid: the read ceiling for a product
    whose time is the reading of its weights)."""
    span = src.numel() * src.element_size()
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=src.device)
    _check(lib().wq_read_probe(_ptr(src), window_bytes, span, count, chunks, int(nontemporal), _ptr(sink),
                               _stream(stream)),
           "wq_read_probe")


MFMA_PROBE_FLOP_PER_WAVE_ITER = 8 * 16384  # eight v_mfma_f32_16x16x32_f16 per wave and iteration


def wq_mfma_probe(workgroups: int, iters: int, count: int, *, sink: torch.Tensor | None = None, stream=None) -> int:
    """count launches of the matrix-core probe; returns the FLOP of one launch
    (workgroups x 4 waves x iters x 8 x 16384)."""
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    _check(lib().wq_mfma_probe(workgroups, iters, count, _ptr(sink), _stream(stream)), "wq_mfma_probe")
    return workgroups * 4 * iters * MFMA_PROBE_FLOP_PER_WAVE_ITER


def wq_clock_probe(workgroups: int = 256, ticks: int = 2000, stream=None):
    """Enqueues the clock probe on the stream and returns the device tensor
    [workgroups][2] (shader clock counter advance, 100 MHz real-time counter
    advance); synchronize before reading it.  Core clock in MHz =
    100 * out[:, 0] / out[:, 1]."""
    out = torch.zeros((workgroups, 2), dtype=torch.int64, device="cuda")
    _check(lib().wq_clock_probe(workgroups, ticks, _ptr(out), _stream(stream)), "wq_clock_probe")
    return out

