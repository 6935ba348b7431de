"""ctypes binding of libnf4moe.so (the C ABI in include/nf4moe.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their pointers and the current HIP stream are passed to the C
entry points, and a non-zero status becomes an exception carrying the
library's message.  PyTorch supplies device memory and streams; every step of
the computation runs in the library's HIP kernels.  If the shared library is
missing, every call raises -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnf4moe.so")

F32, BF16, F16 = 0, 1, 2
NOALLOC_SCRATCH_BYTES = 32 << 20  # NF4MOE_NOALLOC_SCRATCH_BYTES
EPI_NONE, EPI_SWIGLU, EPI_SWIGLU_BWD = 0, 1, 2

STATUS = {
    0: "NF4MOE_OK", -1: "NF4MOE_EINVAL", -2: "NF4MOE_ESHAPE", -3: "NF4MOE_EBLOCK",
    -4: "NF4MOE_ETOPK", -5: "NF4MOE_EDTYPE", -6: "NF4MOE_EWORKSPACE",
    -7: "NF4MOE_EOVERFLOW", -8: "NF4MOE_EHIP",
}


class Nf4MoeError(RuntimeError):
    """A library call returned a negative status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class LoraStruct(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("r", ctypes.c_int),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int)]


_c_i64 = ctypes.c_int64
_c_int = ctypes.c_int
_c_vp = ctypes.c_void_p
_c_size = ctypes.c_size_t

_DGRAD_ARGS = [_c_vp, _c_int, _c_i64, _c_vp, _c_int, _c_vp, _c_vp, _c_vp, _c_int, _c_i64,
               _c_i64, _c_i64, _c_int, _c_vp, _c_int, _c_vp, _c_vp, _c_vp, _c_int, _c_vp]
_BACKWARD_ARGS = [_c_vp, _c_int, _c_vp, _c_vp, _c_int, _c_i64, _c_int, _c_int, _c_int, _c_int,
                  _c_int, _c_vp, _c_vp, _c_vp, _c_vp, ctypes.POINTER(LoraStruct),
                  ctypes.POINTER(LoraStruct), _c_vp, _c_int, _c_vp, _c_vp, _c_vp, _c_vp,
                  _c_vp, _c_size, _c_vp]

_SIGNATURES = {
    "nf4moe_strerror": (ctypes.c_char_p, [_c_int]),
    "nf4moe_last_error": (ctypes.c_char_p, []),
    "nf4moe_version": (ctypes.c_char_p, []),
    "nf4moe_codebook": (_c_int, [ctypes.POINTER(ctypes.c_float)]),
    "nf4moe_packed_bytes": (_c_i64, [_c_i64, _c_i64, _c_i64]),
    "nf4_quantize_experts": (_c_int, [_c_vp, _c_int, _c_i64, _c_i64, _c_i64, _c_int,
                                      _c_vp, _c_vp, _c_vp, _c_vp]),
    "nf4moe_f16_range_check": (_c_int, [_c_vp, _c_int, _c_i64, _c_vp, _c_vp]),
    "moe_route_permute_workspace": (_c_size, [_c_i64, _c_int, _c_int]),
    "moe_route_permute": (_c_int, [_c_vp, _c_i64, _c_int, _c_int, _c_int, _c_vp, _c_vp,
                                   _c_vp, _c_vp, _c_vp, _c_vp, _c_size, _c_vp]),
    "grouped_nf4_gemm": (_c_int, [_c_vp, _c_int, _c_i64, _c_vp, _c_int, _c_vp, _c_vp,
                                  _c_vp, _c_int, _c_i64, _c_i64, _c_i64,
                                  ctypes.POINTER(LoraStruct), _c_int, _c_vp, _c_vp,
                                  _c_vp, _c_int, _c_vp]),
    "moe_expert_forward_workspace": (_c_size, [_c_i64, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "moe_expert_forward": (_c_int, [_c_vp, _c_int, _c_vp, _c_i64, _c_int, _c_int, _c_int,
                                    _c_int, _c_int, _c_vp, _c_vp, _c_vp, _c_vp,
                                    ctypes.POINTER(LoraStruct), ctypes.POINTER(LoraStruct),
                                    _c_vp, _c_int, _c_vp, _c_size, _c_vp]),
    "moe_expert_forward_noalloc": (_c_int, [_c_vp, _c_int, _c_vp, _c_i64, _c_int, _c_int, _c_int,
                                            _c_int, _c_int, _c_vp, _c_vp, _c_vp, _c_vp,
                                            ctypes.POINTER(LoraStruct),
                                            ctypes.POINTER(LoraStruct), _c_vp, _c_int, _c_vp]),
    "moe_expert_forward_routing": (_c_int, [_c_vp, _c_i64, _c_int, _c_int, _c_int, _c_int,
                                            ctypes.POINTER(_c_vp), ctypes.POINTER(_c_vp),
                                            ctypes.POINTER(_c_vp), ctypes.POINTER(_c_vp)]),
    "nbit_codebook": (_c_int, [_c_int, ctypes.POINTER(ctypes.c_float)]),
    "nbit_quantize_experts": (_c_int, [_c_int, _c_vp, _c_int, _c_i64, _c_i64, _c_i64, _c_int,
                                       _c_vp, _c_vp, _c_vp, _c_vp]),
    "grouped_nbit_gemm": (_c_int, [_c_int, _c_vp, _c_int, _c_i64, _c_vp, _c_int, _c_vp, _c_vp,
                                   _c_vp, _c_int, _c_i64, _c_i64, _c_i64,
                                   ctypes.POINTER(LoraStruct), _c_int, _c_vp, _c_vp,
                                   _c_vp, _c_int, _c_vp]),
    "moe_expert_forward_nbit": (_c_int, [_c_int, _c_vp, _c_int, _c_vp, _c_i64, _c_int, _c_int,
                                         _c_int, _c_int, _c_int, _c_vp, _c_vp, _c_vp, _c_vp,
                                         ctypes.POINTER(LoraStruct), ctypes.POINTER(LoraStruct),
                                         _c_vp, _c_int, _c_vp, _c_size, _c_vp]),
    "grouped_nf4_gemm_swiglu_bwd": (_c_int, [_c_vp, _c_i64, _c_vp, _c_int, _c_vp, _c_vp, _c_vp,
                                             _c_int, _c_i64, _c_i64, _c_i64,
                                             ctypes.POINTER(LoraStruct), _c_vp, _c_vp, _c_vp,
                                             _c_vp]),
    "grouped_nf4_gemm_dgrad": (_c_int, _DGRAD_ARGS),
    "grouped_nbit_gemm_dgrad": (_c_int, [_c_int] + _DGRAD_ARGS),
    "moe_expert_backward_workspace": (_c_size, [_c_i64, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "moe_expert_backward": (_c_int, _BACKWARD_ARGS),
    "moe_expert_backward_nbit": (_c_int, [_c_int] + _BACKWARD_ARGS),
    "grouped_mxfp4_gemm": (_c_int, [_c_vp, _c_int, _c_i64, _c_vp, _c_int, _c_vp, _c_vp, _c_vp,
                                    _c_int, _c_i64, _c_i64, _c_i64, _c_int, _c_vp, _c_vp, _c_vp,
                                    _c_int, _c_vp]),
    "moe_expert_forward_mxfp4": (_c_int, [_c_vp, _c_int, _c_vp, _c_i64, _c_int, _c_int, _c_int,
                                          _c_int, _c_int, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                          _c_int, _c_vp, _c_size, _c_vp]),
}

# storage modes of the nbit entry points (NF4MOE_QT_* in include/nf4moe.h)
QUANT_TYPES = {"nf4": 0, "fp4": 1, "int8": 3, "fp8": 4, "bf16": 5, "fp16": 6}
EIGHT_BIT = ("int8", "fp8")  # one byte per element: packed stacks are [E, N, K]
PASSTHROUGH = ("bf16", "fp16")  # the weights themselves, [E, N, K], no absmax
WHOLE = EIGHT_BIT + PASSTHROUGH  # one element per K position


def _qt(quant_type: str) -> int:
    if quant_type not in QUANT_TYPES:
        raise ValueError(f"unknown quant_type {quant_type!r} (one of {sorted(QUANT_TYPES)})")
    return QUANT_TYPES[quant_type]

_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the shared library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m grouped_nf4_gemm_quantize_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        lib = load()
        msg = lib.nf4moe_last_error().decode()
        raise Nf4MoeError(status, msg or lib.nf4moe_strerror(status).decode())


# ------------------------------------------------------------ torch helpers

def _torch():
    import torch

    return torch


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.float32:
        return F32
    if dt == torch.bfloat16:
        return BF16
    if dt == torch.float16:
        return F16
    raise TypeError(f"unsupported dtype {dt}")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(device=None) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def codebook(quant_type: str = "nf4"):
    """The 16 fp32 levels of a storage mode, by code (list of floats)."""
    lib = load()
    buf = (ctypes.c_float * 16)()
    if quant_type == "nf4":
        _check(lib.nf4moe_codebook(buf))
    else:
        _check(lib.nbit_codebook(_qt(quant_type), buf))
    return list(buf)


def packed_bytes(E: int, N: int, K: int) -> int:
    n = load().nf4moe_packed_bytes(E, N, K)
    if n < 0:
        _check(int(n))
    return int(n)


def quantize(w, nonfinite_flag=None, quant_type: str = "nf4"):
    """Quantise w [E, N, K] (fp32 or bf16, GPU) -> (packed u8, absmax f32).

    The passthrough modes return (the [E, N, K] bf16 / fp16 weights, None).
    """
    torch = _torch()
    if w.dim() != 3:
        raise ValueError("w must be [E, N, K]")
    E, N, K = w.shape
    if quant_type in PASSTHROUGH:
        dt = torch.bfloat16 if quant_type == "bf16" else torch.float16
        packed = torch.empty((E, N, K), dtype=dt, device=w.device)
        args = (_ptr(w), _dtype_code(w.dtype), E, N, K, 64, _ptr(packed), None,
                _ptr(nonfinite_flag), _stream(w.device))
        _check(load().nbit_quantize_experts(_qt(quant_type), *args))
        return packed, None
    per_byte = 1 if quant_type in EIGHT_BIT else 2
    packed = torch.empty((E, N, K // per_byte), dtype=torch.uint8, device=w.device)
    absmax = torch.empty((E, N, max(K // 64, 1)), dtype=torch.float32, device=w.device)
    args = (_ptr(w), _dtype_code(w.dtype), E, N, K, 64, _ptr(packed), _ptr(absmax),
            _ptr(nonfinite_flag), _stream(w.device))
    if quant_type == "nf4":
        _check(load().nf4_quantize_experts(*args))
    else:
        _check(load().nbit_quantize_experts(_qt(quant_type), *args))
    return packed, absmax


def f16_range_check(t, flags):
    """OR into ``flags`` (one int32 on the GPU) what an fp16 conversion of the
    bf16 / fp32 tensor ``t`` would lose (see nf4moe_f16_range_check)."""
    if not t.is_contiguous():
        raise ValueError("t must be contiguous")
    _check(load().nf4moe_f16_range_check(_ptr(t), _dtype_code(t.dtype), t.numel(), _ptr(flags),
                                         _stream(t.device)))
    return flags


def route_permute(logits, k: int, renormalize: bool = True):
    """Top-k routing and the expert-grouped pair permutation."""
    torch = _torch()
    T, E = logits.shape
    dev = logits.device
    P = T * k
    out = dict(
        ids=torch.empty((T, k), dtype=torch.int32, device=dev),
        w=torch.empty((T, k), dtype=torch.float32, device=dev),
        sorted_pair=torch.empty(P, dtype=torch.int32, device=dev),
        pair_pos=torch.empty(P, dtype=torch.int32, device=dev),
        offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
    )
    lib = load()
    ws_bytes = lib.moe_route_permute_workspace(T, E, k)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _check(lib.moe_route_permute(_ptr(logits), T, E, k, int(bool(renormalize)),
                                 _ptr(out["ids"]), _ptr(out["w"]), _ptr(out["sorted_pair"]),
                                 _ptr(out["pair_pos"]), _ptr(out["offsets"]), _ptr(ws),
                                 ws_bytes, _stream(dev)))
    return out


def make_lora(A, B, scale: float):
    """LoRA struct for A [E, r, K], B [E, N, r] (bf16 or fp16 GPU tensors).

    The tensors must stay alive until the call that uses the struct returns.
    """
    if A is None:
        return None
    s = LoraStruct(_ptr(A), _ptr(B), int(A.shape[1]), float(scale), _dtype_code(A.dtype))
    return s


def grouped_gemm(a, packed, absmax, offsets, P: int, gather=None, gather_div: int = 1,
                 lora=None, swiglu: bool = False, row_scale=None, scatter=None,
                 out=None, out_dtype=None, out_rows: Optional[int] = None,
                 quant_type: str = "nf4"):
    """Grouped NF4 GEMM (see grouped_nf4_gemm in include/nf4moe.h).

    ``lora`` is ``(A, B, scale)`` or None.  Returns ``out``.
    """
    torch = _torch()
    E, N, K2 = packed.shape
    K = K2 if quant_type in WHOLE else K2 * 2
    n_out = N // 2 if swiglu else N
    if out is None:
        rows = out_rows if out_rows is not None else P
        out = torch.empty((rows, n_out), dtype=out_dtype or torch.float16, device=a.device)
    lib = load()
    ls = make_lora(*lora) if lora is not None else None
    args = (_ptr(a), _dtype_code(a.dtype), a.shape[0], _ptr(gather), gather_div, _ptr(packed),
            _ptr(absmax), _ptr(offsets), E, P, N, K,
            ctypes.byref(ls) if ls is not None else None, EPI_SWIGLU if swiglu else EPI_NONE,
            _ptr(row_scale), _ptr(scatter), _ptr(out), _dtype_code(out.dtype),
            _stream(a.device))
    if quant_type == "nf4":
        _check(lib.grouped_nf4_gemm(*args))
    else:
        _check(lib.grouped_nbit_gemm(_qt(quant_type), *args))
    return out


def grouped_gemm_swiglu_bwd(a, packed, absmax, offsets, P: int, dh, gather=None,
                            gather_div: int = 1, lora=None, out=None, h_out=None):
    """The gate_up GEMM recomputed with the SwiGLU backward as its epilogue
    (see grouped_nf4_gemm_swiglu_bwd in include/nf4moe.h): returns
    ``out`` = [dh * up * silu'(gate) | dh * silu(gate)], fp16 [P, N]; pass an
    fp16 ``h_out`` [P, N/2] to get h = silu(gate) * up as well."""
    torch = _torch()
    E, N, K2 = packed.shape
    if out is None:
        out = torch.empty((P, N), dtype=torch.float16, device=a.device)
    ls = make_lora(*lora) if lora is not None else None
    _check(load().grouped_nf4_gemm_swiglu_bwd(
        _ptr(a), a.shape[0], _ptr(gather), gather_div, _ptr(packed), _ptr(absmax),
        _ptr(offsets), E, P, N, K2 * 2, ctypes.byref(ls) if ls is not None else None, _ptr(dh),
        _ptr(out), _ptr(h_out), _stream(a.device)))
    return out


def forward_workspace_bytes(T: int, H: int, I: int, E: int, k: int, r: int = 0) -> int:
    """Workspace of moe_forward; ``r`` is the larger adapter rank (0: none)."""
    return int(load().moe_expert_forward_workspace(T, H, I, E, k, r))


def moe_forward(x, logits, k: int, gu_packed, gu_absmax, dn_packed, dn_absmax,
                gu_lora=None, dn_lora=None, renormalize: bool = True, y=None,
                y_dtype=None, workspace=None, quant_type: str = "nf4"):
    """Full routed-expert layer (see moe_expert_forward in include/nf4moe.h).

    ``gu_lora`` / ``dn_lora`` are ``(A, B, scale)`` or None.  ``workspace`` is an
    optional preallocated uint8 GPU tensor.  Returns ``y``.
    """
    torch = _torch()
    T, H = x.shape
    E = logits.shape[1]
    I = dn_packed.shape[2] * (1 if quant_type in WHOLE else 2)
    if y is None:
        y = torch.empty((T, H), dtype=y_dtype or torch.bfloat16, device=x.device)
    lib = load()
    r = max([l[0].shape[1] for l in (gu_lora, dn_lora) if l is not None and l[0] is not None],
            default=0)
    ws_bytes = lib.moe_expert_forward_workspace(T, H, I, E, k, r)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    ls_gu = make_lora(*gu_lora) if gu_lora is not None else None
    ls_dn = make_lora(*dn_lora) if dn_lora is not None else None
    args = (_ptr(x), _dtype_code(x.dtype), _ptr(logits), T, H, I, E, k, int(bool(renormalize)),
            _ptr(gu_packed), _ptr(gu_absmax), _ptr(dn_packed), _ptr(dn_absmax),
            ctypes.byref(ls_gu) if ls_gu is not None else None,
            ctypes.byref(ls_dn) if ls_dn is not None else None,
            _ptr(y), _dtype_code(y.dtype), _ptr(workspace), workspace.numel(),
            _stream(x.device))
    if quant_type == "nf4":
        _check(lib.moe_expert_forward(*args))
    else:
        _check(lib.moe_expert_forward_nbit(_qt(quant_type), *args))
    return y


def moe_forward_noalloc(x, logits, k: int, gu_packed, gu_absmax, dn_packed, dn_absmax,
                        gu_lora=None, dn_lora=None, renormalize: bool = True, y=None,
                        y_dtype=None):
    """The layer forward on the library's fixed per-device scratch memory
    (see moe_expert_forward_noalloc): no workspace argument, nothing
    allocated by the library.  Returns ``y``."""
    torch = _torch()
    T, H = x.shape
    E = logits.shape[1]
    I = dn_packed.shape[2] * 2
    if y is None:
        y = torch.empty((T, H), dtype=y_dtype or torch.bfloat16, device=x.device)
    ls_gu = make_lora(*gu_lora) if gu_lora is not None else None
    ls_dn = make_lora(*dn_lora) if dn_lora is not None else None
    _check(load().moe_expert_forward_noalloc(
        _ptr(x), _dtype_code(x.dtype), _ptr(logits), T, H, I, E, k, int(bool(renormalize)),
        _ptr(gu_packed), _ptr(gu_absmax), _ptr(dn_packed), _ptr(dn_absmax),
        ctypes.byref(ls_gu) if ls_gu is not None else None,
        ctypes.byref(ls_dn) if ls_dn is not None else None,
        _ptr(y), _dtype_code(y.dtype), _stream(x.device)))
    return y


def forward_routing(workspace, T: int, H: int, I: int, E: int, k: int):
    """Device pointers (ints) of the routing a forward left in its workspace."""
    ids, w, sp, off = _c_vp(), _c_vp(), _c_vp(), _c_vp()
    _check(load().moe_expert_forward_routing(_ptr(workspace), T, H, I, E, k,
                                             ctypes.byref(ids), ctypes.byref(w),
                                             ctypes.byref(sp), ctypes.byref(off)))
    return dict(ids=ids.value, w=w.value, sorted_pair=sp.value, offsets=off.value)


def grouped_dgrad(a, packed, absmax, offsets, P: int, gather=None, gather_div: int = 1,
                  g_pre=None, row_scale=None, scatter=None, out=None, out_dtype=None,
                  out_rows: Optional[int] = None, quant_type: str = "nf4"):
    """Grouped dgrad through the packed stack (see grouped_nf4_gemm_dgrad).

    ``g_pre`` (the forward's [gate | up] pre-activation rows) selects the
    SwiGLU-backward epilogue.  Returns ``out`` ([rows, K] or [rows, 2K]).
    """
    torch = _torch()
    E, N, K2 = packed.shape
    K = K2 * 2
    n_out = 2 * K if g_pre is not None else K
    if out is None:
        rows = out_rows if out_rows is not None else P
        out = torch.empty((rows, n_out), dtype=out_dtype or torch.float16, device=a.device)
    lib = load()
    args = (_ptr(a), _dtype_code(a.dtype), a.shape[0], _ptr(gather), gather_div, _ptr(packed),
            _ptr(absmax), _ptr(offsets), E, P, N, K,
            EPI_SWIGLU_BWD if g_pre is not None else EPI_NONE, _ptr(g_pre),
            _dtype_code(g_pre.dtype) if g_pre is not None else F16, _ptr(row_scale),
            _ptr(scatter), _ptr(out), _dtype_code(out.dtype), _stream(a.device))
    if quant_type == "nf4":
        _check(lib.grouped_nf4_gemm_dgrad(*args))
    else:
        _check(lib.grouped_nbit_gemm_dgrad(_qt(quant_type), *args))
    return out


def backward_workspace_bytes(T: int, H: int, I: int, E: int, k: int, r: int = 0) -> int:
    return int(load().moe_expert_backward_workspace(T, H, I, E, k, r))


def moe_backward(x, logits, dy, k: int, gu_packed, gu_absmax, dn_packed, dn_absmax,
                 gu_lora=None, dn_lora=None, renormalize: bool = True, dx=None,
                 dx_dtype=None, workspace=None, quant_type: str = "nf4"):
    """Layer backward (see moe_expert_backward in include/nf4moe.h).

    Returns ``(dx, grads)`` where ``grads`` holds ``dA_gu``/``dB_gu`` and
    ``dA_dn``/``dB_dn`` (fp32) for the adapters given.
    """
    torch = _torch()
    T, H = x.shape
    E = logits.shape[1]
    I = dn_packed.shape[2] * 2
    dev = x.device
    if dx is None:
        dx = torch.empty((T, H), dtype=dx_dtype or torch.bfloat16, device=dev)
    r = 0
    grads = {}
    if gu_lora is not None:
        r = int(gu_lora[0].shape[1])
        grads["dA_gu"] = torch.empty((E, r, H), dtype=torch.float32, device=dev)
        grads["dB_gu"] = torch.empty((E, 2 * I, r), dtype=torch.float32, device=dev)
    if dn_lora is not None:
        r = int(dn_lora[0].shape[1])
        grads["dA_dn"] = torch.empty((E, r, I), dtype=torch.float32, device=dev)
        grads["dB_dn"] = torch.empty((E, H, r), dtype=torch.float32, device=dev)
    lib = load()
    ws_bytes = lib.moe_expert_backward_workspace(T, H, I, E, k, r)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    ls_gu = make_lora(*gu_lora) if gu_lora is not None else None
    ls_dn = make_lora(*dn_lora) if dn_lora is not None else None
    args = (_ptr(x), _dtype_code(x.dtype), _ptr(logits), _ptr(dy), _dtype_code(dy.dtype), T, H,
            I, E, k, int(bool(renormalize)), _ptr(gu_packed), _ptr(gu_absmax), _ptr(dn_packed),
            _ptr(dn_absmax), ctypes.byref(ls_gu) if ls_gu is not None else None,
            ctypes.byref(ls_dn) if ls_dn is not None else None, _ptr(dx), _dtype_code(dx.dtype),
            _ptr(grads.get("dA_gu")), _ptr(grads.get("dB_gu")), _ptr(grads.get("dA_dn")),
            _ptr(grads.get("dB_dn")), _ptr(workspace), workspace.numel(), _stream(dev))
    if quant_type == "nf4":
        _check(lib.moe_expert_backward(*args))
    else:
        _check(lib.moe_expert_backward_nbit(_qt(quant_type), *args))
    return dx, grads


def grouped_gemm_mxfp4(a, blocks, scales, offsets, P: int, gather=None, gather_div: int = 1,
                       swiglu: bool = False, row_scale=None, scatter=None, out=None,
                       out_dtype=None, out_rows: Optional[int] = None):
    """Grouped GEMM on MXFP4 stacks (see grouped_mxfp4_gemm in include/nf4moe.h)."""
    torch = _torch()
    E, N, K2 = blocks.shape
    K = K2 * 2
    n_out = N // 2 if swiglu else N
    if out is None:
        rows = out_rows if out_rows is not None else P
        out = torch.empty((rows, n_out), dtype=out_dtype or torch.float16, device=a.device)
    _check(load().grouped_mxfp4_gemm(
        _ptr(a), _dtype_code(a.dtype), a.shape[0], _ptr(gather), gather_div, _ptr(blocks),
        _ptr(scales), _ptr(offsets), E, P, N, K, EPI_SWIGLU if swiglu else EPI_NONE,
        _ptr(row_scale), _ptr(scatter), _ptr(out), _dtype_code(out.dtype), _stream(a.device)))
    return out


def moe_forward_mxfp4(x, logits, k: int, gu_blocks, gu_scales, dn_blocks, dn_scales,
                      renormalize: bool = True, y=None, y_dtype=None, workspace=None):
    """Routed-expert layer on MXFP4 stacks (see moe_expert_forward_mxfp4)."""
    torch = _torch()
    T, H = x.shape
    E = logits.shape[1]
    I = dn_blocks.shape[2] * 2
    if y is None:
        y = torch.empty((T, H), dtype=y_dtype or torch.bfloat16, device=x.device)
    lib = load()
    ws_bytes = lib.moe_expert_forward_workspace(T, H, I, E, k, 0)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    _check(lib.moe_expert_forward_mxfp4(
        _ptr(x), _dtype_code(x.dtype), _ptr(logits), T, H, I, E, k, int(bool(renormalize)),
        _ptr(gu_blocks), _ptr(gu_scales), _ptr(dn_blocks), _ptr(dn_scales), _ptr(y),
        _dtype_code(y.dtype), _ptr(workspace), workspace.numel(), _stream(x.device)))
    return y
