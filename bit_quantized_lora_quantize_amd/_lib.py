"""ctypes binding of libqlora (include/qlora.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libqlora.so.  PyTorch supplies device memory and the current
stream.  The library must have been built (``build_lib.build()``); there is
no fallback of any kind, and calls raise when it is missing.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import re
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# QLORA_LIB names another build of the same library (for instance the
# host-sanitized libqlora_san.so)
LIB_PATH = os.environ.get("QLORA_LIB") or os.path.join(_PKG, "libqlora.so")
SAN_LIB_PATH = os.path.join(_PKG, "libqlora_san.so")
# benchmark build: the same library plus qlora_time_next_weight_kernel
# (include/qlora_timing.h)
TIMED_LIB_PATH = os.path.join(_PKG, "libqlora_timed.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "qlora.h")

QLORA_OP_QUANTIZE, QLORA_OP_FWD, QLORA_OP_BWD = 0, 1, 2
QLORA_OP_FWD_DROPOUT, QLORA_OP_BWD_DROPOUT = 3, 4
QLORA_ERR_SCRATCH = -6
QLORA_STATIC_SCRATCH_BYTES = 32 << 20
QLORA_MAX_GROUP = 8
BLOCK, GROUP = 64, 256

_P = ctypes.c_void_p
_I64 = ctypes.c_int64


class _Nf4(ctypes.Structure):
    _fields_ = [("d_out", _I64), ("d_in", _I64), ("codes", _P), ("scale_codes", _P),
                ("scale2", _P), ("scale_mean", _P)]


class _FwdItem(ctypes.Structure):
    _fields_ = [("w", _Nf4), ("X", _P), ("A", _P), ("B", _P), ("r", _I64),
                ("lora_alpha", ctypes.c_float), ("Y", _P), ("T_save", _P),
                ("workspace", _P), ("workspace_bytes", ctypes.c_size_t)]


class _QuantItem(ctypes.Structure):
    _fields_ = [("W", _P), ("q", _Nf4), ("workspace", _P), ("workspace_bytes", ctypes.c_size_t)]


class _DequantItem(ctypes.Structure):
    _fields_ = [("q", _Nf4), ("W_bf16", _P)]


class _Nf4Blocked(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("block", ctypes.c_int64), ("group", ctypes.c_int64),
                ("codes", ctypes.c_void_p), ("scale_codes", ctypes.c_void_p),
                ("scale2", ctypes.c_void_p), ("scale_mean", ctypes.c_void_p)]


class _Dropout(ctypes.Structure):
    _fields_ = [("p", ctypes.c_float), ("seed", ctypes.c_uint64), ("offset", ctypes.c_uint64),
                ("keep_rows", _P), ("keep_cols", _P)]


class _AdamwParam(ctypes.Structure):
    _fields_ = [("param", _P), ("param_bf16", _P), ("grad", _P), ("m", _P), ("v", _P),
                ("n", _I64)]


class QloraError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {qlora_status_string(status)} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libqlora.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libqlora.so is not built ({LIB_PATH}); run "
                              "python -m bit_quantized_lora_quantize_amd.build_lib")
        L = ctypes.CDLL(LIB_PATH)
        L.qlora_status_string.restype = ctypes.c_char_p
        L.qlora_status_string.argtypes = [ctypes.c_int]
        L.qlora_abi_version.restype = ctypes.c_int
        L.qlora_nf4_sizes.argtypes = [_I64, _I64] + [ctypes.POINTER(ctypes.c_size_t)] * 4
        L.qlora_workspace_bytes.restype = ctypes.c_size_t
        L.qlora_workspace_bytes.argtypes = [ctypes.c_int, _I64, _I64, _I64, _I64]
        L.qlora_quantize_nf4.argtypes = [_P, ctypes.POINTER(_Nf4), _P, ctypes.c_size_t, _P]
        L.qlora_dequant_bf16.argtypes = [ctypes.POINTER(_Nf4), _P, _P]
        L.qlora_sumsq_workspace_bytes.restype = ctypes.c_size_t
        L.qlora_sumsq_workspace_bytes.argtypes = [ctypes.c_int, ctypes.POINTER(_AdamwParam)]
        L.qlora_grad_sumsq.argtypes = [ctypes.c_int, ctypes.POINTER(_AdamwParam), _P, _P,
                                       ctypes.c_size_t, _P]
        L.qlora_adamw_step.argtypes = [ctypes.c_int, ctypes.POINTER(_AdamwParam), ctypes.c_float,
                                       ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                       ctypes.c_float, _I64, _P, ctypes.c_float, _P]
        L.qlora_merge_nf4.argtypes = [ctypes.POINTER(_Nf4), _P, _P, _I64, ctypes.c_float, _P,
                                      ctypes.POINTER(_Nf4), _P, ctypes.c_size_t, _P]
        L.qlora_linear_fwd.argtypes = [ctypes.POINTER(_Nf4), _P, _I64, _P, _P, _I64,
                                       ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P]
        L.qlora_linear_fwd_many.argtypes = [ctypes.c_int, ctypes.POINTER(_FwdItem), _I64, _P]
        L.qlora_quantize_nf4_many.argtypes = [ctypes.c_int, ctypes.POINTER(_QuantItem), _P]
        L.qlora_dequant_bf16_many.argtypes = [ctypes.c_int, ctypes.POINTER(_DequantItem), _P]
        L.qlora_linear_fwd_noalloc.argtypes = [ctypes.POINTER(_Nf4), _P, _I64, _P, _P, _I64,
                                               ctypes.c_float, _P, _P, _P]
        L.qlora_linear_bwd.argtypes = [ctypes.POINTER(_Nf4), _P, _P, _I64, _P, _P, _I64,
                                       ctypes.c_float, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        if hasattr(L, "qlora_time_next_weight_kernel"):     # libqlora_timed.so only
            L.qlora_time_next_weight_kernel.argtypes = [_P, _P]
        L.qlora_nf4_blocked_sizes.argtypes = [_I64, _I64, _I64] + [ctypes.POINTER(ctypes.c_size_t)] * 3
        L.qlora_quantize_blocked_workspace_bytes.restype = ctypes.c_size_t
        L.qlora_quantize_blocked_workspace_bytes.argtypes = [_I64, _I64, _I64]
        L.qlora_quantize_nf4_blocked.argtypes = [_P, ctypes.POINTER(_Nf4Blocked), _P,
                                                 ctypes.c_size_t, _P]
        L.qlora_dequant_bf16_blocked.argtypes = [ctypes.POINTER(_Nf4Blocked), _P, _P]
        L.qlora_dropout_mask.argtypes = [_P, _I64, _I64, ctypes.POINTER(_Dropout), _P, _P, _P]
        L.qlora_linear_fwd_dropout.argtypes = [ctypes.POINTER(_Nf4), _P, _I64, _P, _P, _I64,
                                               ctypes.c_float, ctypes.POINTER(_Dropout), _P, _P,
                                               _P, ctypes.c_size_t, _P]
        L.qlora_linear_bwd_dropout.argtypes = [ctypes.POINTER(_Nf4), _P, _P, _I64, _P, _P, _I64,
                                               ctypes.c_float, ctypes.POINTER(_Dropout), _P, _P,
                                               _P, _P, _P, ctypes.c_size_t, _P]
        _lib = L
    return _lib


@contextlib.contextmanager
def library(path: str):
    """Route the calls made inside the block through another in-tree build of
    the library (libqlora_timed.so for per-kernel timing, or a test build);
    the default library is restored afterwards."""
    global LIB_PATH, _lib
    if not os.path.exists(path):
        raise ImportError(f"{os.path.basename(path)} is not built ({path}); run "
                          "python -m bit_quantized_lora_quantize_amd.build_lib")
    saved = (LIB_PATH, _lib)
    LIB_PATH, _lib = path, None
    try:
        yield lib()
    finally:
        if torch.cuda.is_initialized():
            torch.cuda.synchronize()
        LIB_PATH, _lib = saved


def header_functions() -> list[str]:
    """Names of the functions include/qlora.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qlora_[a-z0-9_]+)\s*\(", text)))


def qlora_status_string(status: int) -> str:
    return lib().qlora_status_string(int(status)).decode()


def qlora_abi_version() -> int:
    return lib().qlora_abi_version()


def _check(status: int, where: str):
    if status != 0:
        raise QloraError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def qlora_time_next_weight_kernel(start, stop) -> None:
    """Bracket the next weight-kernel launch with two recorded events
    (hipEvent_t handles as integers or c_void_p); only inside
    library(TIMED_LIB_PATH)."""
    L = lib()
    if not hasattr(L, "qlora_time_next_weight_kernel"):
        raise RuntimeError("qlora_time_next_weight_kernel is only in libqlora_timed.so; "
                           "use _lib.library(_lib.TIMED_LIB_PATH)")
    _check(L.qlora_time_next_weight_kernel(start, stop), "qlora_time_next_weight_kernel")


def qlora_nf4_sizes(d_out: int, d_in: int) -> tuple[int, int, int, int]:
    out = [ctypes.c_size_t() for _ in range(4)]
    _check(lib().qlora_nf4_sizes(d_out, d_in, *[ctypes.byref(o) for o in out]), "qlora_nf4_sizes")
    return tuple(o.value for o in out)


def qlora_workspace_bytes(op: int, d_out: int, d_in: int, M: int = 0, r: int = 1) -> int:
    return int(lib().qlora_workspace_bytes(op, d_out, d_in, M, r))


# ------------------------------------------------------------- weight state

@dataclass
class NF4Weight:
    """The four device buffers of an NF4 + double-quantized weight."""
    d_out: int
    d_in: int
    codes: torch.Tensor        # uint8 [n/2]
    scale_codes: torch.Tensor  # uint8 [n/64]
    scale2: torch.Tensor       # float32 [ceil(n/64/256)]
    scale_mean: torch.Tensor   # float32 [1]

    @staticmethod
    def empty(d_out: int, d_in: int, device="cuda") -> "NF4Weight":
        cb, sb, s2b, _ = qlora_nf4_sizes(d_out, d_in)
        return NF4Weight(d_out, d_in,
                         torch.empty(cb, dtype=torch.uint8, device=device),
                         torch.empty(sb, dtype=torch.uint8, device=device),
                         torch.empty(s2b // 4, dtype=torch.float32, device=device),
                         torch.empty(1, dtype=torch.float32, device=device))

    def c_struct(self) -> _Nf4:
        return _Nf4(self.d_out, self.d_in, self.codes.data_ptr(), self.scale_codes.data_ptr(),
                    self.scale2.data_ptr(), self.scale_mean.data_ptr())

    @property
    def device(self):
        return self.codes.device

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size()
                   for t in (self.codes, self.scale_codes, self.scale2, self.scale_mean))


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def _need(t: torch.Tensor, dtype, shape, name):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on the GPU, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


# ---------------------------------------------------------------- entry points

def qlora_quantize_nf4(W: torch.Tensor, out: Optional[NF4Weight] = None,
                       workspace: Optional[torch.Tensor] = None) -> NF4Weight:
    d_out, d_in = W.shape
    _need(W, torch.float32, (d_out, d_in), "W")
    q = out if out is not None else NF4Weight.empty(d_out, d_in, W.device)
    need = qlora_workspace_bytes(QLORA_OP_QUANTIZE, d_out, d_in)
    ws = workspace if workspace is not None else _workspace(need, W.device)
    qs = q.c_struct()
    _check(lib().qlora_quantize_nf4(_ptr(W), ctypes.byref(qs), _ptr(ws), ws.numel(),
                                    _stream(W.device)), "qlora_quantize_nf4")
    return q


def qlora_dequant_bf16(q: NF4Weight, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    Wb = out if out is not None else torch.empty((q.d_out, q.d_in), dtype=torch.bfloat16,
                                                 device=q.device)
    _need(Wb, torch.bfloat16, (q.d_out, q.d_in), "W_bf16")
    qs = q.c_struct()
    _check(lib().qlora_dequant_bf16(ctypes.byref(qs), _ptr(Wb), _stream(q.device)),
           "qlora_dequant_bf16")
    return Wb


def qlora_quantize_nf4_many(Ws: Sequence[torch.Tensor],
                            outs: Optional[Sequence[NF4Weight]] = None,
                            workspaces: Optional[Sequence[torch.Tensor]] = None) -> list:
    """qlora_quantize_nf4 for up to QLORA_MAX_GROUP tensors in one call (the
    same results bit for bit)."""
    if not 1 <= len(Ws) <= QLORA_MAX_GROUP:
        raise ValueError(f"1 .. {QLORA_MAX_GROUP} tensors per call")
    arr = (_QuantItem * len(Ws))()
    qs, keep = [], []
    for i, W in enumerate(Ws):
        d_out, d_in = W.shape
        _need(W, torch.float32, (d_out, d_in), "W")
        q = outs[i] if outs is not None else NF4Weight.empty(d_out, d_in, W.device)
        if workspaces is not None:
            ws = workspaces[i]
        else:
            ws = _workspace(qlora_workspace_bytes(QLORA_OP_QUANTIZE, d_out, d_in), W.device)
        keep.append(ws)
        arr[i] = _QuantItem(W.data_ptr(), q.c_struct(), ws.data_ptr(), ws.numel())
        qs.append(q)
    _check(lib().qlora_quantize_nf4_many(len(Ws), arr, _stream(Ws[0].device)),
           "qlora_quantize_nf4_many")
    return qs


def qlora_dequant_bf16_many(qs: Sequence[NF4Weight],
                            outs: Optional[Sequence[torch.Tensor]] = None) -> list:
    """qlora_dequant_bf16 for up to QLORA_MAX_GROUP weights in one call."""
    if not 1 <= len(qs) <= QLORA_MAX_GROUP:
        raise ValueError(f"1 .. {QLORA_MAX_GROUP} weights per call")
    arr = (_DequantItem * len(qs))()
    res = []
    for i, q in enumerate(qs):
        Wb = outs[i] if outs is not None else torch.empty((q.d_out, q.d_in), dtype=torch.bfloat16,
                                                          device=q.device)
        _need(Wb, torch.bfloat16, (q.d_out, q.d_in), "W_bf16")
        arr[i] = _DequantItem(q.c_struct(), Wb.data_ptr())
        res.append(Wb)
    _check(lib().qlora_dequant_bf16_many(len(qs), arr, _stream(qs[0].device)),
           "qlora_dequant_bf16_many")
    return res


@dataclass
class NF4Blocked:
    """NF4 + double quantization of a flat array at general block sizes."""
    n: int
    block: int
    group: int
    codes: torch.Tensor        # uint8 [ceil(n/2)]
    scale_codes: torch.Tensor  # uint8 [ceil(n/block)]
    scale2: torch.Tensor       # float32 [ceil(n1/group)]
    scale_mean: torch.Tensor   # float32 [1]

    @staticmethod
    def empty(n: int, block: int = 64, group: int = 256, device="cuda") -> "NF4Blocked":
        cb, sb, s2b = qlora_nf4_blocked_sizes(n, block, group)
        return NF4Blocked(n, block, group,
                          torch.empty(cb, dtype=torch.uint8, device=device),
                          torch.empty(sb, dtype=torch.uint8, device=device),
                          torch.empty(s2b // 4, dtype=torch.float32, device=device),
                          torch.empty(1, dtype=torch.float32, device=device))

    def c_struct(self) -> _Nf4Blocked:
        return _Nf4Blocked(self.n, self.block, self.group, self.codes.data_ptr(),
                           self.scale_codes.data_ptr(), self.scale2.data_ptr(),
                           self.scale_mean.data_ptr())


def qlora_nf4_blocked_sizes(n: int, block: int, group: int) -> tuple[int, int, int]:
    out = [ctypes.c_size_t() for _ in range(3)]
    _check(lib().qlora_nf4_blocked_sizes(n, block, group, *[ctypes.byref(o) for o in out]),
           "qlora_nf4_blocked_sizes")
    return tuple(o.value for o in out)


def qlora_quantize_blocked_workspace_bytes(n: int, block: int, group: int) -> int:
    return int(lib().qlora_quantize_blocked_workspace_bytes(n, block, group))


def qlora_quantize_nf4_blocked(W: torch.Tensor, block: int = 64, group: int = 256,
                               out: Optional[NF4Blocked] = None,
                               workspace: Optional[torch.Tensor] = None) -> NF4Blocked:
    """Quantize the values of W (FP32, any shape, contiguous) as one flat
    array with first-level blocks of `block` and groups of `group` scales."""
    if W.dtype != torch.float32 or not W.is_contiguous() or not W.is_cuda:
        raise ValueError("W: expected a contiguous float32 tensor on the GPU")
    n = W.numel()
    q = out if out is not None else NF4Blocked.empty(n, block, group, W.device)
    need = qlora_quantize_blocked_workspace_bytes(n, q.block, q.group)
    ws = workspace if workspace is not None else _workspace(need, W.device)
    qs = q.c_struct()
    _check(lib().qlora_quantize_nf4_blocked(_ptr(W), ctypes.byref(qs), _ptr(ws), ws.numel(),
                                            _stream(W.device)), "qlora_quantize_nf4_blocked")
    return q


def qlora_dequant_bf16_blocked(q: NF4Blocked, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    Wb = out if out is not None else torch.empty(q.n, dtype=torch.bfloat16, device=q.codes.device)
    if Wb.dtype != torch.bfloat16 or Wb.numel() != q.n or not Wb.is_contiguous():
        raise ValueError("out: expected a contiguous bfloat16 tensor of n elements")
    qs = q.c_struct()
    _check(lib().qlora_dequant_bf16_blocked(ctypes.byref(qs), _ptr(Wb), _stream(Wb.device)),
           "qlora_dequant_bf16_blocked")
    return Wb


def qlora_merge_nf4(q: NF4Weight, A: torch.Tensor, B: torch.Tensor, lora_alpha: float,
                    W_merged: Optional[torch.Tensor] = None, requantize: bool = True,
                    out: Optional[NF4Weight] = None,
                    workspace: Optional[torch.Tensor] = None):
    """Merged FP32 weight Wh + (lora_alpha / r) B A and, with requantize,
    its NF4 state.  Returns (W_merged, NF4Weight or None)."""
    r = A.shape[0]
    _need(A, torch.bfloat16, (r, q.d_in), "A")
    _need(B, torch.bfloat16, (q.d_out, r), "B")
    Wm = W_merged if W_merged is not None else torch.empty((q.d_out, q.d_in), dtype=torch.float32,
                                                           device=q.device)
    _need(Wm, torch.float32, (q.d_out, q.d_in), "W_merged")
    qs = q.c_struct()
    qo, qos, ws = None, None, None
    if requantize:
        qo = out if out is not None else NF4Weight.empty(q.d_out, q.d_in, q.device)
        qos = qo.c_struct()
        need = qlora_workspace_bytes(QLORA_OP_QUANTIZE, q.d_out, q.d_in)
        ws = workspace if workspace is not None else _workspace(need, q.device)
    _check(lib().qlora_merge_nf4(ctypes.byref(qs), _ptr(A), _ptr(B), r, float(lora_alpha),
                                 _ptr(Wm), ctypes.byref(qos) if qos is not None else None,
                                 _ptr(ws) if ws is not None else None,
                                 ws.numel() if ws is not None else 0, _stream(q.device)),
           "qlora_merge_nf4")
    return Wm, qo


@dataclass
class AdamwParam:
    """One trainable tensor of the optimizer step: FP32 master values,
    gradient and the two moments (all the same shape), and an optional BF16
    compute copy refreshed after the step."""
    param: torch.Tensor
    grad: torch.Tensor
    m: torch.Tensor
    v: torch.Tensor
    param_bf16: Optional[torch.Tensor] = None


def _adamw_array(params: Sequence[AdamwParam]):
    arr = (_AdamwParam * max(1, len(params)))()
    for i, t in enumerate(params):
        n = t.param.numel()
        for name, x in (("grad", t.grad), ("m", t.m), ("v", t.v)):
            _need(x, torch.float32, tuple(t.param.shape), name)
        _need(t.param, torch.float32, tuple(t.param.shape), "param")
        if t.param_bf16 is not None:
            _need(t.param_bf16, torch.bfloat16, tuple(t.param.shape), "param_bf16")
        arr[i] = _AdamwParam(t.param.data_ptr(),
                             t.param_bf16.data_ptr() if t.param_bf16 is not None else None,
                             t.grad.data_ptr(), t.m.data_ptr(), t.v.data_ptr(), n)
    return arr


class AdamwParamSet:
    """A list of AdamwParam checked once, with its C descriptor array (and the
    sum-of-squares workspace) built once, for repeated steps over the same
    tensors.  The tensors must keep their storage while the set is in use."""

    def __init__(self, params: Sequence[AdamwParam]):
        self.params = list(params)
        self.count = len(self.params)
        self.arr = _adamw_array(self.params)
        self.device = self.params[0].param.device if self.params else None
        self._ws = None

    def sumsq_workspace(self) -> torch.Tensor:
        if self._ws is None:
            need = int(lib().qlora_sumsq_workspace_bytes(self.count, self.arr))
            self._ws = _workspace(need, self.device)
        return self._ws


def _as_set(params) -> AdamwParamSet:
    return params if isinstance(params, AdamwParamSet) else AdamwParamSet(params)


def qlora_sumsq_workspace_bytes(params) -> int:
    ps = _as_set(params)
    return int(lib().qlora_sumsq_workspace_bytes(ps.count, ps.arr))


def qlora_grad_sumsq(params, acc: torch.Tensor,
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """acc (FP64 [1], device) += the fixed-order sum of squared gradients of
    `params` (a list of AdamwParam or an AdamwParamSet)."""
    ps = _as_set(params)
    if ps.count == 0:
        return acc
    _need(acc, torch.float64, (1,), "acc")
    ws = workspace if workspace is not None else ps.sumsq_workspace()
    _check(lib().qlora_grad_sumsq(ps.count, ps.arr, _ptr(acc), _ptr(ws), ws.numel(),
                                  _stream(acc.device)), "qlora_grad_sumsq")
    return acc


def qlora_adamw_step(params, lr: float, beta1: float = 0.9, beta2: float = 0.999,
                     eps: float = 1e-8, weight_decay: float = 0.0, step: int = 1,
                     grad_sumsq: Optional[torch.Tensor] = None,
                     max_grad_norm: float = 0.0) -> None:
    """One AdamW step over `params` (a list of AdamwParam or an
    AdamwParamSet), clipped by the global norm when grad_sumsq is given."""
    ps = _as_set(params)
    if ps.count == 0:
        return
    if grad_sumsq is not None:
        _need(grad_sumsq, torch.float64, (1,), "grad_sumsq")
    _check(lib().qlora_adamw_step(ps.count, ps.arr, float(lr), float(beta1), float(beta2),
                                  float(eps), float(weight_decay), int(step), _ptr(grad_sumsq),
                                  float(max_grad_norm), _stream(ps.device)),
           "qlora_adamw_step")


@dataclass
class Dropout:
    """LoRA dropout of the training-mode forward and its backward: drop
    probability p, generator key `seed` and counter words `offset` (a new
    offset per layer and step; the backward passes the same values)."""
    p: float
    seed: int
    offset: int = 0
    # optional saved mask (M > 16): int32 [M, d_in / 32] and [d_in, ceil(M / 32)]
    # device tensors the forward fills and the backward reads (saved_mask())
    keep_rows: Optional[torch.Tensor] = None
    keep_cols: Optional[torch.Tensor] = None

    def c_struct(self) -> _Dropout:
        rows = self.keep_rows.data_ptr() if self.keep_rows is not None else None
        cols = self.keep_cols.data_ptr() if self.keep_cols is not None else None
        return _Dropout(float(self.p), int(self.seed) & (2**64 - 1), int(self.offset) & (2**64 - 1),
                        rows, cols)

    def saved_mask(self, M: int, d_in: int, device="cuda") -> "Dropout":
        """The same dropout with buffers for the forward to save its mask in."""
        rows = torch.empty((M, d_in // 32), dtype=torch.int32, device=device)
        cols = torch.empty((d_in, (M + 31) // 32), dtype=torch.int32, device=device)
        return Dropout(self.p, self.seed, self.offset, rows, cols)


def _fwd(q, X, A, B, lora_alpha, Y, T_save, workspace, dropout):
    M = X.shape[0]
    r = A.shape[0]
    _need(X, torch.bfloat16, (M, q.d_in), "X")
    _need(A, torch.bfloat16, (r, q.d_in), "A")
    _need(B, torch.bfloat16, (q.d_out, r), "B")
    Y = Y if Y is not None else torch.empty((M, q.d_out), dtype=torch.bfloat16, device=X.device)
    _need(Y, torch.bfloat16, (M, q.d_out), "Y")
    if T_save is not None:
        _need(T_save, torch.float32, (M, r), "T_save")
    op = QLORA_OP_FWD if dropout is None else QLORA_OP_FWD_DROPOUT
    need = qlora_workspace_bytes(op, q.d_out, q.d_in, M, r)
    ws = workspace if workspace is not None else _workspace(need, X.device)
    qs = q.c_struct()
    if dropout is None:
        _check(lib().qlora_linear_fwd(ctypes.byref(qs), _ptr(X), M, _ptr(A), _ptr(B), r,
                                      float(lora_alpha), _ptr(Y), _ptr(T_save), _ptr(ws),
                                      ws.numel(), _stream(X.device)), "qlora_linear_fwd")
    else:
        ds = dropout.c_struct()
        _check(lib().qlora_linear_fwd_dropout(ctypes.byref(qs), _ptr(X), M, _ptr(A), _ptr(B), r,
                                              float(lora_alpha), ctypes.byref(ds), _ptr(Y),
                                              _ptr(T_save), _ptr(ws), ws.numel(),
                                              _stream(X.device)), "qlora_linear_fwd_dropout")
    return Y


def qlora_linear_fwd(q: NF4Weight, X: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                     lora_alpha: float, Y: Optional[torch.Tensor] = None,
                     T_save: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    return _fwd(q, X, A, B, lora_alpha, Y, T_save, workspace, None)


def qlora_linear_fwd_noalloc(q: NF4Weight, X: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                             lora_alpha: float, Y: torch.Tensor,
                             T_save: Optional[torch.Tensor] = None) -> torch.Tensor:
    """qlora_linear_fwd with the library's fixed device scratch as its
    workspace: the library allocates nothing (the caller passes Y)."""
    M = X.shape[0]
    r = A.shape[0]
    _need(X, torch.bfloat16, (M, q.d_in), "X")
    _need(A, torch.bfloat16, (r, q.d_in), "A")
    _need(B, torch.bfloat16, (q.d_out, r), "B")
    _need(Y, torch.bfloat16, (M, q.d_out), "Y")
    if T_save is not None:
        _need(T_save, torch.float32, (M, r), "T_save")
    qs = q.c_struct()
    _check(lib().qlora_linear_fwd_noalloc(ctypes.byref(qs), _ptr(X), M, _ptr(A), _ptr(B), r,
                                          float(lora_alpha), _ptr(Y), _ptr(T_save),
                                          _stream(X.device)), "qlora_linear_fwd_noalloc")
    return Y


def qlora_linear_fwd_dropout(q: NF4Weight, X: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                             lora_alpha: float, dropout: Dropout,
                             Y: Optional[torch.Tensor] = None,
                             T_save: Optional[torch.Tensor] = None,
                             workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Training-mode forward: the LoRA branch sees keep * X / (1 - p)."""
    return _fwd(q, X, A, B, lora_alpha, Y, T_save, workspace, dropout)


def qlora_dropout_mask(X: torch.Tensor, dropout: Dropout, X_kept: Optional[torch.Tensor] = None,
                       keep_bits: Optional[torch.Tensor] = None, want_bits: bool = False):
    """(X with dropped elements cleared, keep words [d, ceil(M/32)] or None)."""
    M, d = X.shape
    _need(X, torch.bfloat16, (M, d), "X")
    X_kept = X_kept if X_kept is not None else torch.empty_like(X)
    _need(X_kept, torch.bfloat16, (M, d), "X_kept")
    if want_bits and keep_bits is None:
        keep_bits = torch.empty((d, (M + 31) // 32), dtype=torch.int32, device=X.device)
    ds = dropout.c_struct()
    _check(lib().qlora_dropout_mask(_ptr(X), M, d, ctypes.byref(ds), _ptr(X_kept),
                                    _ptr(keep_bits), _stream(X.device)), "qlora_dropout_mask")
    return X_kept, keep_bits


@dataclass
class FwdItem:
    q: NF4Weight
    X: torch.Tensor
    A: torch.Tensor
    B: torch.Tensor
    lora_alpha: float
    Y: torch.Tensor
    workspace: torch.Tensor
    T_save: Optional[torch.Tensor] = None


def qlora_linear_fwd_many(items: Sequence[FwdItem], M: int) -> None:
    arr = (_FwdItem * len(items))()
    for i, it in enumerate(items):
        r = it.A.shape[0]
        _need(it.X, torch.bfloat16, (M, it.q.d_in), "X")
        _need(it.A, torch.bfloat16, (r, it.q.d_in), "A")
        _need(it.B, torch.bfloat16, (it.q.d_out, r), "B")
        _need(it.Y, torch.bfloat16, (M, it.q.d_out), "Y")
        arr[i] = _FwdItem(it.q.c_struct(), it.X.data_ptr(), it.A.data_ptr(), it.B.data_ptr(), r,
                          float(it.lora_alpha), it.Y.data_ptr(),
                          it.T_save.data_ptr() if it.T_save is not None else None,
                          it.workspace.data_ptr(), it.workspace.numel())
    dev = items[0].X.device
    _check(lib().qlora_linear_fwd_many(len(items), arr, M, _stream(dev)), "qlora_linear_fwd_many")


def _bwd(q, X, dY, A, B, lora_alpha, T_saved, need_dx, dX, dA, dB, workspace, dropout):
    M = X.shape[0]
    r = A.shape[0]
    dev = X.device
    _need(X, torch.bfloat16, (M, q.d_in), "X")
    _need(dY, torch.bfloat16, (M, q.d_out), "dY")
    _need(A, torch.bfloat16, (r, q.d_in), "A")
    _need(B, torch.bfloat16, (q.d_out, r), "B")
    if T_saved is not None:
        _need(T_saved, torch.float32, (M, r), "T_saved")
    if need_dx and dX is None:
        dX = torch.empty((M, q.d_in), dtype=torch.bfloat16, device=dev)
    dA = dA if dA is not None else torch.empty((r, q.d_in), dtype=torch.float32, device=dev)
    dB = dB if dB is not None else torch.empty((q.d_out, r), dtype=torch.float32, device=dev)
    op = QLORA_OP_BWD if dropout is None else QLORA_OP_BWD_DROPOUT
    need = qlora_workspace_bytes(op, q.d_out, q.d_in, M, r)
    ws = workspace if workspace is not None else _workspace(need, dev)
    qs = q.c_struct()
    if dropout is None:
        _check(lib().qlora_linear_bwd(ctypes.byref(qs), _ptr(X), _ptr(dY), M, _ptr(A), _ptr(B),
                                      r, float(lora_alpha), _ptr(T_saved),
                                      _ptr(dX if need_dx else None), _ptr(dA), _ptr(dB),
                                      _ptr(ws), ws.numel(), _stream(dev)), "qlora_linear_bwd")
    else:
        ds = dropout.c_struct()
        _check(lib().qlora_linear_bwd_dropout(ctypes.byref(qs), _ptr(X), _ptr(dY), M, _ptr(A),
                                              _ptr(B), r, float(lora_alpha), ctypes.byref(ds),
                                              _ptr(T_saved), _ptr(dX if need_dx else None),
                                              _ptr(dA), _ptr(dB), _ptr(ws), ws.numel(),
                                              _stream(dev)), "qlora_linear_bwd_dropout")
    return (dX if need_dx else None), dA, dB


def qlora_linear_bwd(q: NF4Weight, X: torch.Tensor, dY: torch.Tensor, A: torch.Tensor,
                     B: torch.Tensor, lora_alpha: float, T_saved: Optional[torch.Tensor] = None,
                     need_dx: bool = True, dX: Optional[torch.Tensor] = None,
                     dA: Optional[torch.Tensor] = None, dB: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None):
    return _bwd(q, X, dY, A, B, lora_alpha, T_saved, need_dx, dX, dA, dB, workspace, None)


def qlora_linear_bwd_dropout(q: NF4Weight, X: torch.Tensor, dY: torch.Tensor, A: torch.Tensor,
                             B: torch.Tensor, lora_alpha: float, dropout: Dropout,
                             T_saved: Optional[torch.Tensor] = None, need_dx: bool = True,
                             dX: Optional[torch.Tensor] = None, dA: Optional[torch.Tensor] = None,
                             dB: Optional[torch.Tensor] = None,
                             workspace: Optional[torch.Tensor] = None):
    """Backward of qlora_linear_fwd_dropout (same X and dropout)."""
    return _bwd(q, X, dY, A, B, lora_alpha, T_saved, need_dx, dX, dA, dB, workspace, dropout)
