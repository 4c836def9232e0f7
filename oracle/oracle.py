"""TEST INFRASTRUCTURE ONLY -- Python face of the CPU oracle (qlora_oracle.c).

A thin ctypes wrapper over the plain C oracle plus numpy marshalling.  It
holds no arithmetic of its own beyond unit conversions (BF16 bit patterns to
FP32 values).  See qlora_oracle.c for the statement of each step and its
source on the pages ("第 04 篇：QLoRA 原理", cited [QP §x]; the compassingai
"QLoRA" concept page, cited [CP]).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
use this module.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qlora_oracle.c")
# QLORA_ORACLE_SANITIZE=1: the same source built with AddressSanitizer and
# UndefinedBehaviorSanitizer (gcc), for runs with libasan and libubsan
# preloaded
_SANITIZE = os.environ.get("QLORA_ORACLE_SANITIZE") == "1"
_LIB = os.path.join(_HERE, "libqlora_oracle_san.so" if _SANITIZE else "libqlora_oracle.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g"]

BLOCK = 64    # first-level block [QP §3.4]
GROUP = 256   # second-level block [QP §5.2]

_lib = None


def build(force: bool = False, sanitize: bool = _SANITIZE) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction); with
    sanitize, the sanitized build libqlora_oracle_san.so."""
    lib = os.path.join(_HERE, "libqlora_oracle_san.so" if sanitize else "libqlora_oracle.so")
    if force or not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(_SRC):
        tmp = lib + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
            *(SAN_FLAGS if sanitize else []),
            "-fPIC", "-shared", "-std=c11", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, lib)
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        lib.orc_codebook.argtypes = [P]
        lib.orc_nf4_index.argtypes = [ctypes.c_float]
        lib.orc_nf4_index.restype = ctypes.c_uint8
        lib.orc_fp8_decode.argtypes = [ctypes.c_uint8]
        lib.orc_fp8_decode.restype = ctypes.c_float
        lib.orc_fp8_encode.argtypes = [ctypes.c_float]
        lib.orc_fp8_encode.restype = ctypes.c_uint8
        lib.orc_bf16_rne.argtypes = [ctypes.c_float]
        lib.orc_bf16_rne.restype = ctypes.c_uint16
        lib.orc_scale_mean.argtypes = [P, I]
        lib.orc_scale_mean.restype = ctypes.c_float
        lib.orc_quantize_nf4.argtypes = [P, I, P, P, P, P, P]
        lib.orc_quantize_nf4_sel.argtypes = [P, I, P, P, P, P, P]
        lib.orc_quantize_nf4_blocked.argtypes = [P, I, I, I, P, P, P, P, P]
        lib.orc_dequant_bf16_blocked.argtypes = [P, P, P, ctypes.c_float, I, I, I, P]
        lib.orc_scale_mean_g.argtypes = [P, I, I]
        lib.orc_scale_mean_g.restype = ctypes.c_float
        lib.orc_restored_scale_g.argtypes = [P, P, ctypes.c_float, I, I]
        lib.orc_restored_scale_g.restype = ctypes.c_float
        lib.orc_restored_scale.argtypes = [P, P, ctypes.c_float, I]
        lib.orc_restored_scale.restype = ctypes.c_float
        lib.orc_dequant_bf16.argtypes = [P, P, P, ctypes.c_float, I, P]
        D = ctypes.c_double
        lib.orc_linear_fwd_rows.argtypes = [P, P, P, P, I, I, I, D, P, I, P, D, P]
        lib.orc_linear_bwd.argtypes = [P, P, P, P, P, I, I, I, I, D, P, I, P, D, P, P, P]
        lib.orc_lora_down.argtypes = [P, P, I, I, I, D, P, D, P]
        lib.orc_philox4x32_10.argtypes = [P, P, P]
        lib.orc_dropout_keep.argtypes = [I, I, ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64, P]
        lib.orc_merge.argtypes = [P, P, P, I, I, I, ctypes.c_float, P]
        lib.orc_sumsq.argtypes = [P, I]
        lib.orc_sumsq.restype = ctypes.c_double
        lib.orc_clip_coef.argtypes = [ctypes.c_double, ctypes.c_float]
        lib.orc_clip_coef.restype = ctypes.c_float
        F = ctypes.c_float
        lib.orc_adamw.argtypes = [P, P, P, P, P, I, F, F, F, F, F, I, F]
        lib.orc_map_nf4_index.argtypes = [P, I, P]
        lib.orc_map_fp8_encode.argtypes = [P, I, P]
        lib.orc_map_bf16_rne.argtypes = [P, I, P]
        lib.orc_num_threads.restype = ctypes.c_int
        lib.orc_set_num_threads.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for the oracle's later parallel loops."""
    _load().orc_set_num_threads(int(n))


# ---------------------------------------------------------------- scalars

def codebook() -> np.ndarray:
    out = np.zeros(16, np.float32)
    _load().orc_codebook(_ptr(out))
    return out


def nf4_index(x: np.ndarray) -> np.ndarray:
    """Nearest-level index of each FP32 value (ties to the lower index)."""
    x = _c(x, np.float32).ravel()
    out = np.empty(x.size, np.uint8)
    _load().orc_map_nf4_index(_ptr(x), x.size, _ptr(out))
    return out


def fp8_decode(code: int) -> float:
    return float(_load().orc_fp8_decode(int(code)))


def fp8_encode(y: np.ndarray) -> np.ndarray:
    y = _c(y, np.float32).ravel()
    out = np.empty(y.size, np.uint8)
    _load().orc_map_fp8_encode(_ptr(y), y.size, _ptr(out))
    return out


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """RNE to BF16; returns the uint16 bit patterns."""
    x = _c(x, np.float32).ravel()
    out = np.empty(x.size, np.uint16)
    _load().orc_map_bf16_rne(_ptr(x), x.size, _ptr(out))
    return out


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------- quantization

def scale_mean(absmax: np.ndarray) -> float:
    a = _c(absmax, np.float32)
    return float(_load().orc_scale_mean(_ptr(a), a.size))


def quantize_nf4(W: np.ndarray, return_absmax: bool = False):
    """NF4 + double quantization of an FP32 matrix (row-major flatten).

    Returns (codes uint8[n/2], scale_codes uint8[n/64], s2 float32[G], mean)."""
    W = _c(W, np.float32)
    n = W.size
    assert n % BLOCK == 0
    n1 = n // BLOCK
    G = (n1 + GROUP - 1) // GROUP
    codes = np.empty(n // 2, np.uint8)
    scodes = np.empty(n1, np.uint8)
    s2 = np.empty(G, np.float32)
    mean = np.zeros(1, np.float32)
    absmax = np.empty(n1, np.float32)
    _load().orc_quantize_nf4(_ptr(W), n, _ptr(codes), _ptr(scodes), _ptr(s2),
                             _ptr(mean), _ptr(absmax))
    out = (codes, scodes, s2, float(mean[0]))
    return out + (absmax,) if return_absmax else out


def quantize_nf4_sel(W: np.ndarray, group_sel: np.ndarray):
    """The layer format with NF4 codes only for the 256-block groups g where
    group_sel[g] is true (codes of other groups are 0); the FP8 scale codes,
    second-level scales and mean are computed for every block, as by
    quantize_nf4.  Returns (codes, scale_codes, s2, mean)."""
    W = _c(W, np.float32)
    n = W.size
    assert n % BLOCK == 0
    n1 = n // BLOCK
    G = (n1 + GROUP - 1) // GROUP
    sel = _c(np.asarray(group_sel, bool), np.uint8)
    assert sel.size == G
    codes = np.empty(n // 2, np.uint8)
    scodes = np.empty(n1, np.uint8)
    s2 = np.empty(G, np.float32)
    mean = np.zeros(1, np.float32)
    _load().orc_quantize_nf4_sel(_ptr(W), n, _ptr(sel), _ptr(codes), _ptr(scodes), _ptr(s2),
                                 _ptr(mean))
    return codes, scodes, s2, float(mean[0])


def quantize_nf4_blocked(W: np.ndarray, block: int, group: int, return_absmax: bool = False):
    """NF4 + double quantization of n = W.size values (flattened) with
    first-level blocks of `block` and second-level groups of `group` scales;
    a short last block or group is allowed.  [QP §5.5]

    Returns (codes uint8[ceil(n/2)], scale_codes uint8[n1], s2 float32[G], mean)."""
    W = _c(W, np.float32).ravel()
    n = W.size
    n1 = -(-n // block)
    G = -(-n1 // group)
    codes = np.empty((n + 1) // 2, np.uint8)
    scodes = np.empty(n1, np.uint8)
    s2 = np.empty(G, np.float32)
    mean = np.zeros(1, np.float32)
    absmax = np.empty(n1, np.float32)
    _load().orc_quantize_nf4_blocked(_ptr(W), n, block, group, _ptr(codes), _ptr(scodes),
                                     _ptr(s2), _ptr(mean), _ptr(absmax))
    out = (codes, scodes, s2, float(mean[0]))
    return out + (absmax,) if return_absmax else out


def dequant_bf16_blocked(codes, scodes, s2, mean: float, n: int, block: int,
                         group: int) -> np.ndarray:
    """Restored weights (BF16 bit patterns, uint16[n]) of the blocked format."""
    codes = _c(codes, np.uint8)
    scodes = _c(scodes, np.uint8)
    s2 = _c(s2, np.float32)
    out = np.empty(n, np.uint16)
    _load().orc_dequant_bf16_blocked(_ptr(codes), _ptr(scodes), _ptr(s2), float(mean), n,
                                     block, group, _ptr(out))
    return out


def restored_scale_g(scodes, s2, mean: float, b: int, group: int) -> float:
    sc = _c(scodes, np.uint8)
    s2 = _c(s2, np.float32)
    return float(_load().orc_restored_scale_g(_ptr(sc), _ptr(s2), float(mean), int(b), int(group)))


def scale_mean_g(absmax: np.ndarray, group: int) -> float:
    a = _c(absmax, np.float32)
    return float(_load().orc_scale_mean_g(_ptr(a), a.size, group))


def restored_scales(scodes: np.ndarray, s2: np.ndarray, mean: float) -> np.ndarray:
    lib = _load()
    sc = _c(scodes, np.uint8)
    s2 = _c(s2, np.float32)
    return np.array([lib.orc_restored_scale(_ptr(sc), _ptr(s2), mean, b)
                     for b in range(sc.size)], np.float32)


def dequant_bf16(codes, scodes, s2, mean: float, n: int) -> np.ndarray:
    """Restored weights as BF16 bit patterns, uint16[n]."""
    codes = _c(codes, np.uint8)
    scodes = _c(scodes, np.uint8)
    s2 = _c(s2, np.float32)
    out = np.empty(n, np.uint16)
    _load().orc_dequant_bf16(_ptr(codes), _ptr(scodes), _ptr(s2), float(mean), n, _ptr(out))
    return out


# ------------------------------------------------------------- LoRA linear

def merge(Wh, A, B, s: float) -> np.ndarray:
    """Merged FP32 weight Wh + s B A (FP64 evaluation, one FP32 rounding);
    s is the FP32 value alpha / r.  [QP §12.3]"""
    Wh, A, B = (_c(t, np.float32) for t in (Wh, A, B))
    d_out, d_in = Wh.shape
    r = A.shape[0]
    Wm = np.empty((d_out, d_in), np.float32)
    _load().orc_merge(_ptr(Wh), _ptr(A), _ptr(B), d_out, d_in, r, float(np.float32(s)), _ptr(Wm))
    return Wm


def sumsq(g: np.ndarray) -> float:
    """Sum of squares in the fixed order (groups of 256, then the tree over
    the group sums).  [QP §10.2]"""
    g = _c(g, np.float32).ravel()
    return float(_load().orc_sumsq(_ptr(g), g.size))


def clip_coef(S: float, max_norm: float) -> float:
    return float(_load().orc_clip_coef(float(S), float(max_norm)))


def adamw(p, g, m, v, lr, beta1, beta2, eps, wd, step, c=1.0, want_bf16=False):
    """One AdamW step on copies of (p, m, v); returns (p, m, v, p_bf16 bits or
    None).  [QP §7.3]"""
    p, m, v = (_c(t, np.float32).copy() for t in (p, m, v))
    g = _c(g, np.float32)
    p16 = np.empty(p.shape, np.uint16) if want_bf16 else None
    _load().orc_adamw(_ptr(p), _ptr(p16) if want_bf16 else ctypes.c_void_p(0), _ptr(g), _ptr(m),
                      _ptr(v), p.size, float(lr), float(beta1), float(beta2), float(eps),
                      float(wd), int(step), float(c))
    return p, m, v, p16


def _keep_args(keep, M, d_in, p):
    if keep is None:
        return ctypes.c_void_p(0), 1.0, None
    keep = _c(keep, np.uint8)
    assert keep.shape == (M, d_in)
    return _ptr(keep), 1.0 - float(np.float32(p)), keep


def linear_fwd(Wh, X, A, B, s: float, rows=None, keep=None, p: float = 0.0) -> np.ndarray:
    """Y[rows] = X[rows] Wh^T + s (D(X)[rows] A^T) B^T in FP64.

    Wh [d_out, d_in], X [M, d_in], A [r, d_in], B [d_out, r]: FP32 arrays of
    exact values.  rows defaults to every token row.  keep (uint8 [M, d_in])
    and p give the LoRA dropout D(x) = keep x / (1 - p); None: D(x) = x."""
    Wh, X, A, B = (_c(t, np.float32) for t in (Wh, X, A, B))
    d_out, d_in = Wh.shape
    r = A.shape[0]
    M = X.shape[0]
    rows = np.arange(M, dtype=np.int64) if rows is None else _c(rows, np.int64)
    Y = np.zeros((rows.size, d_out), np.float64)
    kp, q, _hold = _keep_args(keep, M, d_in, p)
    _load().orc_linear_fwd_rows(_ptr(Wh), _ptr(X), _ptr(A), _ptr(B), d_out, d_in, r,
                                float(s), _ptr(rows), rows.size, kp, q, _ptr(Y))
    return Y


def lora_down(X, A, s: float, keep=None, p: float = 0.0) -> np.ndarray:
    """T = s D(X) A^T in FP64, [M, r]: the LoRA branch's rank-r intermediate
    (see linear_fwd for keep / p).  [QP §2.2]"""
    X, A = (_c(t, np.float32) for t in (X, A))
    M, d_in = X.shape
    r = A.shape[0]
    T = np.zeros((M, r), np.float64)
    kp, q, _hold = _keep_args(keep, M, d_in, p)
    _load().orc_lora_down(_ptr(X), _ptr(A), M, d_in, r, float(s), kp, q, _ptr(T))
    return T


def linear_bwd(Wh, X, dY, A, B, s: float, rows=None, want_dx=True, want_da=True,
               want_db=True, keep=None, p: float = 0.0):
    """(dX[rows], dA, dB) in FP64 for upstream gradient dY; no dW exists.
    keep / p: the forward's LoRA dropout (see linear_fwd)."""
    Wh, X, dY, A, B = (_c(t, np.float32) for t in (Wh, X, dY, A, B))
    d_out, d_in = Wh.shape
    r = A.shape[0]
    M = X.shape[0]
    rows = np.arange(M, dtype=np.int64) if rows is None else _c(rows, np.int64)
    dX = np.zeros((rows.size, d_in), np.float64) if want_dx else None
    dA = np.zeros((r, d_in), np.float64) if want_da else None
    dB = np.zeros((d_out, r), np.float64) if want_db else None
    nul = ctypes.c_void_p(0)
    kp, q, _hold = _keep_args(keep, M, d_in, p)
    _load().orc_linear_bwd(_ptr(Wh), _ptr(X), _ptr(dY), _ptr(A), _ptr(B), M, d_out, d_in, r,
                           float(s), _ptr(rows), rows.size, kp, q,
                           _ptr(dX) if want_dx else nul, _ptr(dA) if want_da else nul,
                           _ptr(dB) if want_db else nul)
    return dX, dA, dB


def philox4x32_10(ctr, key) -> np.ndarray:
    """Philox4x32-10 of one 4-word counter under a 2-word key."""
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    out = np.zeros(4, np.uint32)
    _load().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def dropout_keep(M: int, d: int, p: float, seed: int, offset: int) -> np.ndarray:
    """uint8 [M, d] keep mask of the LoRA dropout (1 = kept).  [QP §6.3]"""
    keep = np.zeros((M, d), np.uint8)
    _load().orc_dropout_keep(M, d, float(p), int(seed), int(offset), _ptr(keep))
    return keep
