"""GPU parity of the NF4 LoRA linear layer, forward and backward, against the
CPU oracle: Y, dX, dA, dB within 1e-2 normwise-max and 2e-3 relative-
Frobenius error of the FP64-accumulating oracle; T = s X A^T likewise."""
import numpy as np
import pytest
import torch

import bit_quantized_lora_quantize_amd as q
from bit_quantized_lora_quantize_amd import inputs
from parity_util import (assert_close, assert_quant_equal, f32, oracle_quant, rel_errors, say,
                         wide_weight_library)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
ALPHA = 16.0


def _layer(d_out, d_in, M, r, config, layer=0, proj=0, device="cpu"):
    W = inputs.weight(d_out, d_in, config=config, layer=layer, device=device, proj=proj)
    A, B = inputs.lora_factors(d_out, d_in, r, config=config, layer=layer, device=device,
                               proj=proj)
    X = inputs.activations(M, d_in, config, layer, inputs.T_X, device=device, proj=proj)
    dY = inputs.activations(M, d_out, config, layer, inputs.T_DY, device=device, proj=proj)
    return W, A, B, X, dY


def _check_layer(orc, W, A, B, X, dY, rows=None, label="", check_bwd=True):
    d_out, d_in = W.shape
    M, r = X.shape[0], A.shape[0]
    s = ALPHA / r
    say(f"linear parity: {label} d_out={d_out} d_in={d_in} M={M} r={r}")
    ref_q, _, Wh = oracle_quant(orc, W.cpu())
    w = q.qlora_quantize_nf4(W.to(DEV).contiguous())
    Xd, Ad, Bd, dYd = (t.to(DEV).contiguous() for t in (X, A, B, dY))
    T = torch.empty((M, r), dtype=torch.float32, device=DEV)
    Y = q.qlora_linear_fwd(w, Xd, Ad, Bd, ALPHA, T_save=T)
    torch.cuda.synchronize()
    assert_quant_equal(w, ref_q)
    Xn, An, Bn, dYn = (f32(t) for t in (X, A, B, dY))
    sel = slice(None) if rows is None else rows
    Yr = orc.linear_fwd(Wh, Xn, An, Bn, s, rows=rows)
    assert_close("Y", f32(Y)[sel], Yr)
    assert_close("T", f32(T), orc.lora_down(Xn, An, s), fro_tol=1e-4, max_tol=1e-4)
    if not check_bwd:
        return
    dXr, dAr, dBr = orc.linear_bwd(Wh, Xn, dYn, An, Bn, s, rows=rows)
    dX, dA, dB = q.qlora_linear_bwd(w, Xd, dYd, Ad, Bd, ALPHA, T_saved=T)
    dX2, dA2, dB2 = q.qlora_linear_bwd(w, Xd, dYd, Ad, Bd, ALPHA, T_saved=None)
    torch.cuda.synchronize()
    assert_close("dX", f32(dX)[sel], dXr)
    assert_close("dA", f32(dA), dAr)
    assert_close("dB", f32(dB), dBr)
    # recomputing T inside the backward gives the same bytes
    assert torch.equal(dX.view(torch.int16), dX2.view(torch.int16))
    assert torch.equal(dA, dA2) and torch.equal(dB, dB2)


SMALL = [  # (d_out, d_in, M, r)
    (256, 256, 16, 8),      # the 256 x 256, 16-token, rank-8 configuration
    (64, 64, 1, 1),
    (100, 192, 3, 4),
    (130, 320, 17, 16),
    (64, 128, 100, 64),
    (300, 256, 16, 256),
    (1, 64, 5, 3),
    (513, 1088, 33, 24),
    (200, 4096, 16, 64),
    (96, 512, 129, 7),
    (72, 192, 70, 100),     # large-M rank path, r in (64, 128]
    (136, 256, 48, 256),    # large-M rank path at the maximum rank
    (200, 256, 40, 128),    # large-M rank path, r in (64, 128], B read as stored
    (264, 320, 300, 40),    # two row tiles of the weight kernel, ragged in M and N
    (264, 320, 1100, 40),   # three 512-token tiles of the GEMM, ragged in M, N and K
]


# backward activation paths: straight into LDS (d_out % 32 == 0), 16-byte
# register loads (d_out % 8 == 0) and element loads (otherwise)
WIDE = [(256, 512, 300, 16), (264, 320, 1100, 40), (130, 320, 17, 16)]


@pytest.mark.parametrize("shape", WIDE)
def test_linear_wide_weight_descriptors(orc, shape):
    """The backward GEMM's per-step weight descriptors (taken in production for
    packed weights beyond 2^31 bytes) against the oracle, through the test
    build that takes them at every size."""
    d_out, d_in, M, r = shape
    with wide_weight_library():
        _check_layer(orc, *_layer(d_out, d_in, M, r, 140 + WIDE.index(shape)), label=f"wide {shape}")


@pytest.mark.parametrize("shape", SMALL)
def test_linear_small(orc, shape):
    d_out, d_in, M, r = shape
    cfg = 0 if shape == (256, 256, 16, 8) else 80 + (d_out + d_in + M + r) % 9
    _check_layer(orc, *_layer(d_out, d_in, M, r, cfg), label=str(shape))


def test_linear_empty_batch(orc):
    d_out, d_in, r = 64, 128, 8
    W, A, B, _, _ = _layer(d_out, d_in, 1, r, 70)
    w = q.qlora_quantize_nf4(W.to(DEV))
    X = torch.empty((0, d_in), dtype=torch.bfloat16, device=DEV)
    dY = torch.empty((0, d_out), dtype=torch.bfloat16, device=DEV)
    Y = q.qlora_linear_fwd(w, X, A.to(DEV), B.to(DEV), ALPHA)
    dA = torch.full((r, d_in), 7.0, device=DEV)
    dB = torch.full((d_out, r), 7.0, device=DEV)
    dX, dA, dB = q.qlora_linear_bwd(w, X, dY, A.to(DEV), B.to(DEV), ALPHA, dA=dA, dB=dB)
    torch.cuda.synchronize()
    assert Y.shape == (0, d_out) and dX.shape == (0, d_in)
    assert torch.count_nonzero(dA) == 0 and torch.count_nonzero(dB) == 0


def test_special_cases(orc):
    """W = 0: Y is the LoRA branch alone.  B = 0: dA = 0 exactly.  A = 0: dB = 0."""
    d_out, d_in, M, r = 96, 256, 12, 8
    W, A, B, X, dY = _layer(d_out, d_in, M, r, 71)
    _check_layer(orc, torch.zeros_like(W), A, B, X, dY, label="W = 0")
    w = q.qlora_quantize_nf4(W.to(DEV))
    Xd, dYd = X.to(DEV), dY.to(DEV)
    _, dA, _ = q.qlora_linear_bwd(w, Xd, dYd, A.to(DEV), torch.zeros_like(B).to(DEV), ALPHA)
    _, _, dB = q.qlora_linear_bwd(w, Xd, dYd, torch.zeros_like(A).to(DEV), B.to(DEV), ALPHA)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dA) == 0 and torch.count_nonzero(dB) == 0


@pytest.mark.parametrize("shape", [(264, 320, 300, 40), (200, 256, 40, 128),
                                   (136, 256, 48, 256), (256, 512, 300, 16)])
def test_u_from_b_as_stored_matches_transposed(orc, shape):
    """For large M the backward's U = s dY B reads B as stored (whole 16-byte
    pieces of its rows, transposing LDS reads) when B is 16-byte aligned, and
    goes through a transposed copy of B otherwise: the same products, so the
    same bits in dX, dA and dB."""
    d_out, d_in, M, r = shape
    W, A, B, X, dY = (t.to(DEV) for t in _layer(d_out, d_in, M, r, 73))
    w = q.qlora_quantize_nf4(W)
    buf = torch.zeros(B.numel() + 8, dtype=B.dtype, device=DEV)
    Bu = buf[1:1 + B.numel()].view(d_out, r)   # 2 bytes past a 16-byte boundary
    Bu.copy_(B)
    assert B.data_ptr() % 16 == 0 and Bu.data_ptr() % 16 == 2
    res = [q.qlora_linear_bwd(w, X, dY, A, Bx, ALPHA) for Bx in (B, Bu)]
    torch.cuda.synchronize()
    for x, y in zip(*res):
        assert torch.equal(x, y)


@pytest.mark.parametrize("shape", [(320, 1024, 16, 64),      # weight-streaming forward
                                   (264, 320, 1100, 40),     # K splits, token splits, ragged
                                   (1024, 2048, 2200, 64)])  # several splits of every kind
def test_deterministic(orc, shape):
    """Split reductions add their partials in a fixed order: the same call
    twice gives the same bits, on the small-M path and on the large-M one."""
    d_out, d_in, M, r = shape
    W, A, B, X, dY = (t.to(DEV) for t in _layer(d_out, d_in, M, r, 72))
    w = q.qlora_quantize_nf4(W)
    outs = []
    for _ in range(2):
        T = torch.empty((M, r), dtype=torch.float32, device=DEV)
        Y = q.qlora_linear_fwd(w, X, A, B, ALPHA, T_save=T)
        dX, dA, dB = q.qlora_linear_bwd(w, X, dY, A, B, ALPHA)
        outs.append((Y.clone(), T.clone(), dX.clone(), dA.clone(), dB.clone()))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                           b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16))


def test_grouped_forward_matches_oracle(orc):
    """qlora_linear_fwd_many over projections of different shapes (M = 4)."""
    M, r = 4, 64
    shapes = [(256, 512), (1000, 256), (64, 1088)]
    items, refs = [], []
    for i, (d_out, d_in) in enumerate(shapes):
        W, A, B, X, _ = _layer(d_out, d_in, M, r, 73, proj=i)
        _, _, Wh = oracle_quant(orc, W)
        refs.append(orc.linear_fwd(Wh, f32(X), f32(A), f32(B), ALPHA / r))
        w = q.qlora_quantize_nf4(W.to(DEV))
        ws = torch.empty(q.qlora_workspace_bytes(q.QLORA_OP_FWD, d_out, d_in, M, r),
                         dtype=torch.uint8, device=DEV)
        Y = torch.empty((M, d_out), dtype=torch.bfloat16, device=DEV)
        items.append(q.FwdItem(w, X.to(DEV), A.to(DEV), B.to(DEV), ALPHA, Y, ws))
    q.qlora_linear_fwd_many(items, M)
    torch.cuda.synchronize()
    for it, ref in zip(items, refs):
        assert_close(f"Y[{it.q.d_out}x{it.q.d_in}]", f32(it.Y), ref)


@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("proj", [0, 4, 6])
def test_llama7b_decode_forward(orc, M, proj):
    """Decode-sized forward (M = 1, 4, 16; r = 64) on the 7B projection
    shapes, full output compared."""
    name, d_out, d_in = inputs.LLAMA_7B[proj]
    W, A, B, X, dY = _layer(d_out, d_in, M, 64, 2, proj=proj, device=DEV)
    _check_layer(orc, W, A, B, X, dY, label=f"7B {name}", check_bwd=False)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_llama7b_decode_grouped_as_benched(orc, M):
    """The decode call the benchmark times: qlora_linear_fwd_many over all
    seven projections of the 7B layer (the benchmark's seeds: config 2, layer
    0) at M tokens, r = 64.  Quantized state bit for bit, every Y element and
    T against the oracle.  The grouped call plans its K split over the whole
    layer, unlike a single call, so Y may differ from a single call's in FP32
    summation order (the count is printed); T does not depend on the split
    and must equal the single call's bit for bit."""
    r = 64
    items, singles, weights = [], [], []
    for p, (name, d_out, d_in) in enumerate(inputs.LLAMA_7B):
        W = inputs.weight(d_out, d_in, 2, 0, device=DEV, proj=p)
        A, B = inputs.lora_factors(d_out, d_in, r, 2, 0, device=DEV, proj=p)
        X = inputs.activations(M, d_in, 2, 0, inputs.T_X, device=DEV, proj=p)
        w = q.qlora_quantize_nf4(W)
        ws = torch.empty(q.qlora_workspace_bytes(q.QLORA_OP_FWD, d_out, d_in, M, r),
                         dtype=torch.uint8, device=DEV)
        Y = torch.empty((M, d_out), dtype=torch.bfloat16, device=DEV)
        T = torch.empty((M, r), dtype=torch.float32, device=DEV)
        items.append(q.FwdItem(w, X, A, B, ALPHA, Y, ws, T_save=T))
        weights.append(W)
    q.qlora_linear_fwd_many(items, M)
    for it in items:
        Ts = torch.empty_like(it.T_save)
        singles.append((q.qlora_linear_fwd(it.q, it.X, it.A, it.B, ALPHA, T_save=Ts), Ts))
    torch.cuda.synchronize()
    say(f"7B grouped decode M={M}: 7 projections in one call")
    differs = 0
    for p, (it, W, (Ys, Ts)) in enumerate(zip(items, weights, singles)):
        name = inputs.LLAMA_7B[p][0]
        ref_q, _, Wh = oracle_quant(orc, W.cpu())
        assert_quant_equal(it.q, ref_q)
        Xn, An, Bn = (f32(t) for t in (it.X, it.A, it.B))
        assert_close(f"{name} Y", f32(it.Y), orc.linear_fwd(Wh, Xn, An, Bn, ALPHA / r))
        assert_close(f"{name} T", f32(it.T_save), orc.lora_down(Xn, An, ALPHA / r),
                     fro_tol=1e-4, max_tol=1e-4)
        assert torch.equal(it.T_save, Ts), f"{name}: grouped T differs from the single call's"
        differs += int(not torch.equal(it.Y.view(torch.int16), Ys.view(torch.int16)))
    say(f"  projections whose grouped Y differs bitwise from the single call: {differs}")


@pytest.mark.parametrize("proj", [0, 4, 6])
def test_llama7b_training_shape(orc, proj):
    """M = 4096 tokens, r = 64, fwd + bwd on the 7B projection shapes: Y and
    dX on 24 sampled token rows (first, last, random), dA and dB in full."""
    name, d_out, d_in = inputs.LLAMA_7B[proj]
    M = 4096
    W, A, B, X, dY = _layer(d_out, d_in, M, 64, 3, proj=proj, device=DEV)
    rng = np.random.default_rng(proj)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 22, replace=False)]))
    _check_layer(orc, W, A, B, X, dY, rows=rows, label=f"7B {name} train")


def test_linear_tokens_beyond_2gib(orc):
    """Activations larger than 2 GiB, so that byte offsets over a whole
    tensor would not fit 32 bits: M = 5 x 65536 tokens of width 4096 (2.7 GB
    each for X and dY).  X and dY are five stacked copies of a 65536-token
    block.  Every row of Y, T and dX is computed by per-row arithmetic that
    does not depend on where the row sits, so each copy must reproduce the
    block's rows bit for bit; dA and dB sum over tokens, so they must equal
    five times the block's own within FP32 rounding.  The block itself is
    checked against the oracle on sampled rows."""
    d_out = d_in = 4096
    M0, copies, r = 65536, 5, 64
    W, A, B, X0, dY0 = _layer(d_out, d_in, M0, r, 90, device=DEV)
    w = q.qlora_quantize_nf4(W)
    X = X0.repeat(copies, 1).contiguous()
    dY = dY0.repeat(copies, 1).contiguous()
    T0 = torch.empty((M0, r), dtype=torch.float32, device=DEV)
    Y0 = q.qlora_linear_fwd(w, X0, A, B, ALPHA, T_save=T0)
    dX0, dA0, dB0 = q.qlora_linear_bwd(w, X0, dY0, A, B, ALPHA, T_saved=T0)
    T = torch.empty((copies * M0, r), dtype=torch.float32, device=DEV)
    Y = q.qlora_linear_fwd(w, X, A, B, ALPHA, T_save=T)
    dX, dA, dB = q.qlora_linear_bwd(w, X, dY, A, B, ALPHA, T_saved=T)
    torch.cuda.synchronize()
    say(f"large-M: M={copies * M0} d={d_in} X {X.numel() * 2 / 2**30:.2f} GiB")
    for c in range(copies):
        rows = slice(c * M0, (c + 1) * M0)
        assert torch.equal(Y[rows].view(torch.int16), Y0.view(torch.int16)), f"Y copy {c}"
        assert torch.equal(T[rows], T0), f"T copy {c}"
        assert torch.equal(dX[rows].view(torch.int16), dX0.view(torch.int16)), f"dX copy {c}"
    for name, got, ref in (("dA", dA, dA0), ("dB", dB, dB0)):
        fro, mx = rel_errors(f32(got), copies * f32(ref).astype(np.float64))
        say(f"  {name} vs {copies} x block: fro {fro:.2e} max {mx:.2e}")
        assert fro <= 1e-5 and mx <= 1e-5, (name, fro, mx)
    # the block against the oracle on sampled token rows
    _, _, Wh = oracle_quant(orc, W.cpu())
    rows = np.arange(0, M0, 4093)
    s = ALPHA / r
    Xn, An, Bn, dYn = (f32(t) for t in (X0, A, B, dY0))
    assert_close("Y rows", f32(Y0)[rows], orc.linear_fwd(Wh, Xn, An, Bn, s, rows=rows))
    dXr, _, _ = orc.linear_bwd(Wh, Xn, dYn, An, Bn, s, rows=rows, want_da=False, want_db=False)
    assert_close("dX rows", f32(dX0)[rows], dXr)
