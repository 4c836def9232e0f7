"""The C-ABI library loads, exports every entry point include/qlora.h
declares, and rejects bad arguments on the host before touching a GPU.

No call here reaches a kernel: every call either is host-only or fails
argument validation (fake device addresses are never dereferenced)."""
import ctypes
import subprocess

import pytest

import bit_quantized_lora_quantize_amd as q
from bit_quantized_lora_quantize_amd import _lib

OK, ENULL, ESHAPE, EALIGN, EWS, EHIP = 0, -1, -2, -3, -4, -5


@pytest.fixture(scope="module")
def L():
    import os
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return q.lib()


def test_exports_every_declared_function(L):
    declared = q.header_functions()
    assert {"qlora_quantize_nf4", "qlora_dequant_bf16", "qlora_linear_fwd",
            "qlora_linear_bwd"} <= set(declared)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [f for f in declared if f not in exported]
    assert not missing, missing
    for f in declared:
        assert hasattr(L, f)


def test_wide_descriptor_test_build_exports_the_same(L):
    """libqlora_wide.so (the test build whose backward GEMM takes the per-step
    weight descriptors at every size) is built beside the library and exports
    the same entry points."""
    import os
    wide = os.path.join(os.path.dirname(_lib.LIB_PATH), "libqlora_wide.so")
    assert os.path.exists(wide), "libqlora_wide.so is not built"
    out = subprocess.run(["nm", "-D", "--defined-only", wide], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(q.header_functions()) <= exported


def _exports(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    return {line.split()[-1] for line in out.splitlines() if " T " in line}


def test_timing_hook_only_in_the_timing_build(L):
    """libqlora.so keeps no state between calls: the event hook that times
    single kernels is exported only by the benchmark build libqlora_timed.so
    (include/qlora_timing.h), which also exports every qlora.h entry point."""
    import os
    import re
    assert "qlora_time_next_weight_kernel" not in _exports(_lib.LIB_PATH)
    assert "qlora_time_next_weight_kernel" not in q.header_functions()
    assert os.path.exists(_lib.TIMED_LIB_PATH), "libqlora_timed.so is not built"
    timed = _exports(_lib.TIMED_LIB_PATH)
    text = open(os.path.join(os.path.dirname(_lib.HEADER_PATH), "qlora_timing.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    timing_fns = set(re.findall(r"\b(qlora_[a-z0-9_]+)\s*\(", text))
    assert timing_fns == {"qlora_time_next_weight_kernel"}
    assert set(q.header_functions()) | timing_fns <= timed
    peaks = os.path.join(os.path.dirname(_lib.LIB_PATH), "libqlora_peaks.so")
    assert {"qlora_peak_stream_read", "qlora_peak_mfma"} <= _exports(peaks)


def test_status_strings_and_version(L):
    assert q.qlora_abi_version() >> 16 == 1
    for s in (OK, ENULL, ESHAPE, EALIGN, EWS, EHIP):
        assert q.qlora_status_string(s) and q.qlora_status_string(s) != "unknown status"
    assert q.qlora_status_string(12345) == "unknown status"


def test_nf4_sizes_closed_form(L):
    """codes n/2, FP8 scale codes n/64, FP32 second-level scales ceil(n/64/256),
    one FP32 mean."""
    for d_out, d_in in ((256, 256), (4096, 4096), (11008, 4096), (4096, 11008), (3, 64),
                        (8192, 22016)):
        n = d_out * d_in
        assert q.qlora_nf4_sizes(d_out, d_in) == (n // 2, n // 64, 4 * (-(-(n // 64) // 256)), 4)
    with pytest.raises(q.QloraError):
        q.qlora_nf4_sizes(4, 100)
    with pytest.raises(q.QloraError):
        q.qlora_nf4_sizes(0, 64)


def test_workspace_sizes(L):
    ws = q.qlora_workspace_bytes
    assert ws(0, 256, 256) > 0
    assert ws(1, 4096, 4096, 16, 64) > 0 and ws(2, 4096, 4096, 4096, 64) > 0
    assert ws(1, 4096, 4096, 0, 64) > 0           # M = 0 is valid
    assert ws(2, 64, 128, 0, 8) > 0
    for M in (0, 1, 15, 16, 17, 31, 32, 33, 4096):
        for r in (1, 8, 64, 256):
            assert ws(1, 100, 192, M, r) > 0 and ws(2, 100, 192, M, r) > 0
    assert ws(1, 4096, 4096, 16, 0) == 0          # r out of range
    assert ws(1, 4096, 4096, 16, 257) == 0
    assert ws(1, 4096, 100, 16, 8) == 0           # d_in % 64 != 0
    assert ws(7, 4096, 4096, 16, 8) == 0          # unknown op
    # larger problems never need less
    assert ws(2, 4096, 4096, 4096, 64) >= ws(2, 4096, 4096, 2048, 64)


def _nf4(d_out=64, d_in=64, base=0x10000):
    return _lib._Nf4(d_out, d_in, base, base + 0x1000, base + 0x2000, base + 0x3000)


def test_quantize_argument_errors(L):
    P = ctypes.c_void_p
    good = _nf4()
    W, wsp = P(0x20000), P(0x30000)
    big = 1 << 30
    assert L.qlora_quantize_nf4(None, ctypes.byref(good), wsp, big, None) == ENULL
    assert L.qlora_quantize_nf4(W, None, wsp, big, None) == ENULL
    assert L.qlora_quantize_nf4(W, ctypes.byref(good), None, big, None) == ENULL
    assert L.qlora_quantize_nf4(P(0x20004), ctypes.byref(good), wsp, big, None) == EALIGN
    assert L.qlora_quantize_nf4(W, ctypes.byref(good), wsp, 16, None) == EWS
    bad = _nf4(64, 100)
    assert L.qlora_quantize_nf4(W, ctypes.byref(bad), wsp, big, None) == ESHAPE
    bad = _nf4(0, 64)
    assert L.qlora_quantize_nf4(W, ctypes.byref(bad), wsp, big, None) == ESHAPE
    mis = _lib._Nf4(64, 64, 0x10008, 0x11000, 0x12000, 0x13000)
    assert L.qlora_quantize_nf4(W, ctypes.byref(mis), wsp, big, None) == EALIGN
    nul = _lib._Nf4(64, 64, 0x10000, None, 0x12000, 0x13000)
    assert L.qlora_quantize_nf4(W, ctypes.byref(nul), wsp, big, None) == ENULL
    assert L.qlora_dequant_bf16(ctypes.byref(good), None, None) == ENULL
    assert L.qlora_dequant_bf16(ctypes.byref(good), P(0x40002), None) == EALIGN


def test_linear_argument_errors(L):
    P = ctypes.c_void_p
    w = _nf4(128, 64)
    X, A, B, Y, ws = P(0x50000), P(0x60000), P(0x70000), P(0x80000), P(0x90000)
    big = 1 << 30
    f = L.qlora_linear_fwd
    assert f(ctypes.byref(w), X, 4, A, B, 0, 16.0, Y, None, ws, big, None) == ESHAPE
    assert f(ctypes.byref(w), X, 4, A, B, 300, 16.0, Y, None, ws, big, None) == ESHAPE
    assert f(ctypes.byref(w), X, -1, A, B, 8, 16.0, Y, None, ws, big, None) == ESHAPE
    assert f(ctypes.byref(w), None, 4, A, B, 8, 16.0, Y, None, ws, big, None) == ENULL
    assert f(ctypes.byref(w), X, 4, A, B, 8, 16.0, None, None, ws, big, None) == ENULL
    assert f(ctypes.byref(w), P(0x50002), 4, A, B, 8, 16.0, Y, None, ws, big, None) == EALIGN
    assert f(ctypes.byref(w), X, 4, A, B, 8, 16.0, Y, P(0x1234), ws, big, None) == EALIGN
    assert f(ctypes.byref(w), X, 4, A, B, 8, 16.0, Y, None, ws, 64, None) == EWS
    assert f(ctypes.byref(w), X, 4, A, B, 8, 16.0, Y, None, None, big, None) == ENULL
    # size limits: at most 2^21 tokens, layer sides at most 2^21
    assert f(ctypes.byref(w), X, (1 << 21) + 1, A, B, 8, 16.0, Y, None, ws, big, None) == ESHAPE
    wide = _nf4(64, (1 << 21) + 64)
    assert f(ctypes.byref(wide), X, 4, A, B, 8, 16.0, Y, None, ws, big, None) == ESHAPE
    # M = 0 is an empty batch: valid, nothing to do, no GPU work
    assert f(ctypes.byref(w), None, 0, None, None, 8, 16.0, None, None, None, 0, None) == OK
    b = L.qlora_linear_bwd
    dA, dB = P(0xA0000), P(0xB0000)
    assert b(ctypes.byref(w), X, X, 4, A, B, 8, 16.0, None, None, None, dB, ws, big, None) == ENULL
    assert b(ctypes.byref(w), X, X, 4, A, B, 8, 16.0, None, None, dA, dB, ws, 64, None) == EWS
    assert b(ctypes.byref(w), X, P(0x50006), 4, A, B, 8, 16.0, None, None, dA, dB, ws, big,
             None) == EALIGN
    assert b(ctypes.byref(w), X, X, 4, A, B, 0, 16.0, None, None, dA, dB, ws, big, None) == ESHAPE
    assert b(ctypes.byref(w), X, X, (1 << 21) + 1, A, B, 8, 16.0, None, None, dA, dB, ws, big,
             None) == ESHAPE


def test_grouped_forward_argument_errors(L):
    items = (_lib._FwdItem * 9)()
    assert L.qlora_linear_fwd_many(0, items, 4, None) == ESHAPE
    assert L.qlora_linear_fwd_many(9, items, 4, None) == ESHAPE
    assert L.qlora_linear_fwd_many(1, None, 4, None) == ENULL
    # an all-zero item has no valid shape; with a shape but NULL buffers it is
    # a NULL error; either way nothing is enqueued
    assert L.qlora_linear_fwd_many(1, items, 4, None) == ESHAPE
    items[0].w.d_out, items[0].w.d_in, items[0].r = 64, 64, 8
    assert L.qlora_linear_fwd_many(1, items, 4, None) == ENULL


def test_merge_argument_errors(L):
    P = ctypes.c_void_p
    w, wo = _nf4(128, 64), _nf4(128, 64, base=0x40000)
    other = _nf4(64, 64, base=0x40000)
    A, B, Wm, ws = P(0x60000), P(0x70000), P(0x80000), P(0x90000)
    big = 1 << 30
    f = L.qlora_merge_nf4
    assert f(ctypes.byref(w), A, B, 0, 16.0, Wm, None, None, 0, None) == ESHAPE
    assert f(ctypes.byref(w), A, B, 257, 16.0, Wm, None, None, 0, None) == ESHAPE
    assert f(ctypes.byref(w), None, B, 8, 16.0, Wm, None, None, 0, None) == ENULL
    assert f(ctypes.byref(w), A, B, 8, 16.0, None, None, None, 0, None) == ENULL
    assert f(ctypes.byref(w), P(0x60002), B, 8, 16.0, Wm, None, None, 0, None) == EALIGN
    assert f(ctypes.byref(w), A, B, 8, 16.0, Wm, ctypes.byref(other), ws, big, None) == ESHAPE
    assert f(ctypes.byref(w), A, B, 8, 16.0, Wm, ctypes.byref(wo), None, big, None) == ENULL
    assert f(ctypes.byref(w), A, B, 8, 16.0, Wm, ctypes.byref(wo), ws, 16, None) == EWS


def test_optimizer_argument_errors(L):
    P = ctypes.c_void_p
    Prm = _lib._AdamwParam
    good = (Prm * 2)(Prm(0x10000, None, 0x20000, 0x30000, 0x40000, 100),
                     Prm(0x50000, 0x60000, 0x70000, 0x80000, 0x90000, 0))
    nograd = (Prm * 1)(Prm(0x10000, None, None, 0x30000, 0x40000, 100))
    neg = (Prm * 1)(Prm(0x10000, None, 0x20000, 0x30000, 0x40000, -1))
    f = L.qlora_adamw_step
    args = (1e-3, 0.9, 0.999, 1e-8, 0.0)
    assert f(0, None, *args, 1, None, 0.0, None) == OK      # nothing to do
    assert f(-1, good, *args, 1, None, 0.0, None) == ESHAPE
    assert f(2, good, *args, 0, None, 0.0, None) == ESHAPE  # step counts from 1
    assert f(2, good, 1e-3, 1.0, 0.999, 1e-8, 0.0, 1, None, 0.0, None) == ESHAPE
    assert f(2, good, 1e-3, 0.9, -0.1, 1e-8, 0.0, 1, None, 0.0, None) == ESHAPE
    assert f(2, None, *args, 1, None, 0.0, None) == ENULL
    assert f(1, nograd, *args, 1, None, 0.0, None) == ENULL
    assert f(1, neg, *args, 1, None, 0.0, None) == ESHAPE
    g = L.qlora_grad_sumsq
    acc, ws = P(0xA0000), P(0xB0000)
    need = L.qlora_sumsq_workspace_bytes(2, good)
    assert need >= 16 and L.qlora_sumsq_workspace_bytes(-1, good) == 0
    assert L.qlora_sumsq_workspace_bytes(1, neg) == 0
    big = (Prm * 1)(Prm(0x10000, None, 0x20000, 0x30000, 0x40000, 1 << 30))
    assert L.qlora_sumsq_workspace_bytes(1, big) >= (1 << 30) // 256 * 8
    huge = (Prm * 1)(Prm(0x10000, None, 0x20000, 0x30000, 0x40000, (1 << 32) + 1))
    assert L.qlora_sumsq_workspace_bytes(1, huge) == 0
    assert g(1, huge, acc, ws, 1 << 40, None) == ESHAPE
    assert f(1, huge, *args, 1, None, 0.0, None) == ESHAPE
    assert g(0, None, None, None, 0, None) == OK
    assert g(-1, good, acc, ws, need, None) == ESHAPE
    assert g(2, good, None, ws, need, None) == ENULL
    assert g(2, good, acc, None, need, None) == ENULL
    assert g(2, good, acc, P(0xB0008), need, None) == EALIGN
    assert g(2, good, acc, ws, need - 1, None) == EWS
    assert g(1, nograd, acc, ws, need, None) == ENULL
    assert g(1, neg, acc, ws, need, None) == ESHAPE


def test_dropout_argument_errors(L):
    P = ctypes.c_void_p
    D = _lib._Dropout
    ok, bad_hi, bad_neg = D(0.1, 1, 2), D(1.0, 1, 2), D(-0.1, 1, 2)
    X, Xk, bits = P(0x10000), P(0x20000), P(0x30000)
    f = L.qlora_dropout_mask
    assert f(X, 0, 64, ctypes.byref(ok), Xk, None, None) == OK     # nothing to do
    assert f(X, 4, 64, None, Xk, None, None) == ENULL
    assert f(X, 4, 64, ctypes.byref(bad_hi), Xk, None, None) == ESHAPE
    assert f(X, 4, 64, ctypes.byref(bad_neg), Xk, None, None) == ESHAPE
    assert f(X, 4, 60, ctypes.byref(ok), Xk, None, None) == ESHAPE  # d % 8
    assert f(X, 4, 64, ctypes.byref(ok), None, None, None) == ENULL
    assert f(None, 4, 64, ctypes.byref(ok), Xk, None, None) == ENULL
    assert f(X, 4, 64, ctypes.byref(ok), P(0x20004), None, None) == EALIGN
    assert f(X, (1 << 21) + 1, 64, ctypes.byref(ok), Xk, bits, None) == ESHAPE
    w = _nf4(128, 64)
    A, B, Y, ws = P(0x60000), P(0x70000), P(0x80000), P(0x90000)
    fw = L.qlora_linear_fwd_dropout
    assert fw(ctypes.byref(w), X, 4, A, B, 8, 16.0, None, Y, None, ws, 1 << 30, None) == ENULL
    assert fw(ctypes.byref(w), X, 4, A, B, 8, 16.0, ctypes.byref(bad_hi), Y, None, ws, 1 << 30,
              None) == ESHAPE
    need = q.qlora_workspace_bytes(q.QLORA_OP_FWD_DROPOUT, 128, 64, 4, 8)
    assert need > q.qlora_workspace_bytes(q.QLORA_OP_FWD, 128, 64, 4, 8)
    assert fw(ctypes.byref(w), X, 4, A, B, 8, 16.0, ctypes.byref(ok), Y, None, ws, need - 1,
              None) == EWS
    bw = L.qlora_linear_bwd_dropout
    dA, dB = P(0xA0000), P(0xB0000)
    needb = q.qlora_workspace_bytes(q.QLORA_OP_BWD_DROPOUT, 128, 64, 40, 8)
    # M > 16: keep words in both layouts (no masked copy of X); M <= 16: the
    # masked copy of X and the keep words of the GEMM
    assert needb >= q.qlora_workspace_bytes(q.QLORA_OP_BWD, 128, 64, 40, 8) + 40 * 2 * 4 + 64 * 2 * 4
    assert (q.qlora_workspace_bytes(q.QLORA_OP_BWD_DROPOUT, 128, 64, 4, 8) >=
            q.qlora_workspace_bytes(q.QLORA_OP_BWD, 128, 64, 4, 8) + 4 * 64 * 2 + 64 * 4)
    misaligned = D(0.1, 1, 2, 0x40004, 0x50000)
    assert bw(ctypes.byref(w), X, X, 40, A, B, 8, 16.0, ctypes.byref(misaligned), None, None, dA,
              dB, ws, needb, None) == EALIGN
    assert bw(ctypes.byref(w), X, X, 40, A, B, 8, 16.0, None, None, None, dA, dB, ws, needb,
              None) == ENULL
    assert bw(ctypes.byref(w), X, X, 40, A, B, 8, 16.0, ctypes.byref(ok), None, None, dA, dB, ws,
              needb - 1, None) == EWS
    assert bw(ctypes.byref(w), X, X, 40, A, B, 0, 16.0, ctypes.byref(ok), None, None, dA, dB, ws,
              needb, None) == ESHAPE


def test_blocked_sizes_and_argument_errors(L):
    P = ctypes.c_void_p
    assert q.qlora_nf4_blocked_sizes(1001, 32, 16) == (501, 32, 8)
    assert q.qlora_nf4_blocked_sizes(64 * 256 * 3, 64, 256) == (64 * 384, 768, 12)
    for bad in ((0, 64, 256), (100, 48, 256), (100, 16, 256), (100, 8192, 256), (100, 64, 8),
                (100, 64, 2048), (100, 64, 100), ((1 << 40) + 1, 64, 256)):
        with pytest.raises(q.QloraError):
            q.qlora_nf4_blocked_sizes(*bad)
        assert q.qlora_quantize_blocked_workspace_bytes(*bad) == 0
    need = q.qlora_quantize_blocked_workspace_bytes(1000, 32, 16)
    assert need >= 32 * 4 + 8
    B = _lib._Nf4Blocked
    good = B(1000, 32, 16, 0x10000, 0x20000, 0x30000, 0x40000)
    W, ws = P(0x50000), P(0x60000)
    f = L.qlora_quantize_nf4_blocked
    assert f(W, None, ws, need, None) == ENULL
    assert f(W, ctypes.byref(B(1000, 24, 16, 0x10000, 0x20000, 0x30000, 0x40000)), ws, need,
             None) == ESHAPE
    assert f(W, ctypes.byref(B(1000, 32, 16, 0, 0x20000, 0x30000, 0x40000)), ws, need,
             None) == ENULL
    assert f(W, ctypes.byref(B(1000, 32, 16, 0x10008, 0x20000, 0x30000, 0x40000)), ws, need,
             None) == EALIGN
    assert f(None, ctypes.byref(good), ws, need, None) == ENULL
    assert f(P(0x50004), ctypes.byref(good), ws, need, None) == EALIGN
    assert f(W, ctypes.byref(good), ws, need - 1, None) == EWS
    g = L.qlora_dequant_bf16_blocked
    assert g(ctypes.byref(good), None, None) == ENULL
    assert g(ctypes.byref(good), P(0x70002), None) == EALIGN


def test_noalloc_forward_host_checks(L):
    """qlora_linear_fwd_noalloc checks its arguments like qlora_linear_fwd and
    rejects a call whose workspace exceeds the library's fixed device scratch
    with its own status -- all before any GPU call.  Every LLaMA-7B and -65B
    projection shape fits at r = 64 up to 40000 tokens, as its declaration
    states."""
    from bit_quantized_lora_quantize_amd import inputs
    P = ctypes.c_void_p
    ESCRATCH = q.QLORA_ERR_SCRATCH
    assert q.qlora_status_string(ESCRATCH) != "unknown status"
    f = L.qlora_linear_fwd_noalloc
    X, A, B, Y = P(0x50000), P(0x60000), P(0x70000), P(0x80000)
    w = _nf4(128, 64)
    assert f(ctypes.byref(w), X, 4, A, B, 0, 16.0, Y, None, None) == ESHAPE
    assert f(ctypes.byref(w), None, 4, A, B, 8, 16.0, Y, None, None) == ENULL
    assert f(ctypes.byref(w), P(0x50002), 4, A, B, 8, 16.0, Y, None, None) == EALIGN
    assert f(ctypes.byref(w), None, 0, None, None, 8, 16.0, None, None, None) == OK
    lim = q.QLORA_STATIC_SCRATCH_BYTES
    wbig = _nf4(4096, 4096)
    M = 1 << 20
    assert q.qlora_workspace_bytes(q.QLORA_OP_FWD, 4096, 4096, M, 256) > lim
    assert f(ctypes.byref(wbig), X, M, A, B, 256, 16.0, Y, None, None) == ESCRATCH
    for M in (1, 4, 16, 17, 2048, 4096, 40000):
        for _, d_out, d_in in inputs.LLAMA_7B + inputs.LLAMA_65B:
            assert q.qlora_workspace_bytes(q.QLORA_OP_FWD, d_out, d_in, M, 64) <= lim
