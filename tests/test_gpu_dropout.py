"""GPU parity of the LoRA dropout ([QP §6.3]): the Philox keep mask and the
masked LoRA input bit for bit against the CPU oracle; the training-mode
forward and backward within the floating-point tolerances; p = 0 equal to the
plain layer bit for bit."""
import numpy as np
import pytest
import torch

import bit_quantized_lora_quantize_amd as q
from bit_quantized_lora_quantize_amd import inputs
from parity_util import assert_close, bits16, f32, oracle_quant, say, wide_weight_library

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
ALPHA = 16.0
P = 0.05  # the LoRA dropout of the principles page's configuration (§9.4)


def _pack_keep(keep):
    """keep [M, d] (0/1) -> words [d, ceil(M/32)], bit m % 32 of word m / 32."""
    M, d = keep.shape
    ldw = (M + 31) // 32
    pad = np.zeros((ldw * 32, d), np.uint64)
    pad[:M] = keep
    w = np.zeros((d, ldw), np.uint64)
    for j in range(32):
        w |= pad[j::32].T << np.uint64(j)
    return w.astype(np.uint32)


@pytest.mark.parametrize("shape", [(1, 64), (37, 136), (100, 4096), (4096, 4096), (33, 11008)])
def test_dropout_mask_bit_exact(orc, shape):
    M, d = shape
    drop = q.Dropout(0.1, seed=0xDEADBEEF12345 + M, offset=7 * d)
    say(f"dropout mask parity: M={M} d={d}")
    X = inputs.activations(M, d, 90, tensor=inputs.T_X)
    Xk, bits = q.qlora_dropout_mask(X.to(DEV), drop, want_bits=True)
    torch.cuda.synchronize()
    keep = orc.dropout_keep(M, d, drop.p, drop.seed, drop.offset)
    ref = np.where(keep.astype(bool), bits16(X).reshape(M, d), np.uint16(0))
    assert np.array_equal(bits16(Xk).reshape(M, d), ref), "masked input differs"
    assert np.array_equal(bits.cpu().numpy().view(np.uint32), _pack_keep(keep)), "keep words differ"


def _layer(d_out, d_in, M, r, config):
    W = inputs.weight(d_out, d_in, config=config)
    A, B = inputs.lora_factors(d_out, d_in, r, config=config)
    X = inputs.activations(M, d_in, config, 0, inputs.T_X)
    dY = inputs.activations(M, d_out, config, 0, inputs.T_DY)
    return W, A, B, X, dY


def _check_dropout(orc, shape, cfg, p=P, rows=None):
    d_out, d_in, M, r = shape
    s = ALPHA / r
    drop = q.Dropout(p, seed=1000 + cfg, offset=3 * cfg + 1)
    say(f"dropout linear parity: {shape} p={p}")
    W, A, B, X, dY = _layer(d_out, d_in, M, r, cfg)
    _, _, Wh = oracle_quant(orc, W)
    keep = orc.dropout_keep(M, d_in, p, drop.seed, drop.offset)
    w = q.qlora_quantize_nf4(W.to(DEV))
    Xd, Ad, Bd, dYd = (t.to(DEV) for t in (X, A, B, dY))
    T = torch.empty((M, r), dtype=torch.float32, device=DEV)
    Y = q.qlora_linear_fwd_dropout(w, Xd, Ad, Bd, ALPHA, drop, T_save=T)
    dX, dA, dB = q.qlora_linear_bwd_dropout(w, Xd, dYd, Ad, Bd, ALPHA, drop, T_saved=T)
    dX2, dA2, dB2 = q.qlora_linear_bwd_dropout(w, Xd, dYd, Ad, Bd, ALPHA, drop, T_saved=None)
    torch.cuda.synchronize()
    Xn, An, Bn, dYn = (f32(t) for t in (X, A, B, dY))
    sel = slice(None) if rows is None else rows
    assert_close("Y", f32(Y)[sel], orc.linear_fwd(Wh, Xn, An, Bn, s, rows=rows, keep=keep, p=p))
    assert_close("T", f32(T), orc.lora_down(Xn, An, s, keep=keep, p=p), fro_tol=1e-4,
                 max_tol=1e-4)
    dXr, dAr, dBr = orc.linear_bwd(Wh, Xn, dYn, An, Bn, s, rows=rows, keep=keep, p=p)
    assert_close("dX", f32(dX)[sel], dXr)
    assert_close("dA", f32(dA), dAr)
    assert_close("dB", f32(dB), dBr)
    # the regenerated mask and the recomputed T give the same bytes
    assert torch.equal(dX.view(torch.int16), dX2.view(torch.int16))
    assert torch.equal(dA, dA2) and torch.equal(dB, dB2)


SHAPES = [  # (d_out, d_in, M, r): small-M weight streaming and the fused GEMM
    (256, 256, 16, 8),
    (100, 192, 3, 4),
    (130, 320, 17, 16),
    (64, 128, 100, 64),
    (513, 1088, 33, 24),
    (264, 320, 300, 40),
    (96, 512, 129, 7),
    (264, 320, 1100, 40),   # three 512-token GEMM tiles, ragged
]


@pytest.mark.parametrize("shape", SHAPES)
def test_dropout_linear(orc, shape):
    _check_dropout(orc, shape, 110 + SHAPES.index(shape))


def test_dropout_wide_weight_descriptors(orc):
    """The masked backward GEMM with per-step weight descriptors (the test
    build that takes them at every size) against the oracle."""
    with wide_weight_library():
        _check_dropout(orc, (264, 320, 1100, 40), 145)
        _check_dropout(orc, (256, 512, 300, 16), 146)


def test_dropout_high_rate(orc):
    """p = 0.5: half the LoRA input gone, the branch doubled."""
    _check_dropout(orc, (192, 256, 40, 16), 120, p=0.5)


@pytest.mark.parametrize("M", [4, 300])
def test_dropout_p0_equals_plain_layer(orc, M):
    """With p = 0 nothing is dropped and the scale is unchanged: every output
    equals the plain layer's bit for bit (small-M and GEMM paths)."""
    d_out, d_in, r = 200, 320, 16
    W, A, B, X, dY = (t.to(DEV) for t in _layer(d_out, d_in, M, r, 121))
    w = q.qlora_quantize_nf4(W)
    drop = q.Dropout(0.0, seed=5, offset=6)
    T1 = torch.empty((M, r), dtype=torch.float32, device=DEV)
    T2 = torch.empty_like(T1)
    Y1 = q.qlora_linear_fwd(w, X, A, B, ALPHA, T_save=T1)
    Y2 = q.qlora_linear_fwd_dropout(w, X, A, B, ALPHA, drop, T_save=T2)
    g1 = q.qlora_linear_bwd(w, X, dY, A, B, ALPHA)
    g2 = q.qlora_linear_bwd_dropout(w, X, dY, A, B, ALPHA, drop)
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))
    assert torch.equal(T1, T2)
    assert torch.equal(g1[0].view(torch.int16), g2[0].view(torch.int16))
    assert torch.equal(g1[1], g2[1]) and torch.equal(g1[2], g2[2])


@pytest.mark.parametrize("proj", [0, 6])
def test_dropout_llama7b_training_shape(orc, proj):
    """M = 4096 tokens, r = 64, p = 0.05 on a 7B projection (q or down),
    sampled rows against the oracle."""
    name, d_out, d_in = inputs.LLAMA_7B[proj]
    M, r = 4096, 64
    rows = np.array([0, 1, 255, 256, 2047, 4000, 4095])
    say(f"dropout 7B {name}")
    _check_dropout(orc, (d_out, d_in, M, r), 130 + proj, rows=rows)


def test_dropout_empty_batch_and_extreme_parameters(orc):
    """M = 0 does nothing (and zeroes dA, dB); p = 0.99 keeps about one in a
    hundred and still matches the oracle; seeds and offsets use all 64 bits."""
    d_out, d_in, r = 64, 128, 8
    W, A, B, X, dY = _layer(d_out, d_in, 1, r, 125)
    w = q.qlora_quantize_nf4(W.to(DEV))
    X0 = torch.empty((0, d_in), dtype=torch.bfloat16, device=DEV)
    dY0 = torch.empty((0, d_out), dtype=torch.bfloat16, device=DEV)
    drop = q.Dropout(0.5, seed=(1 << 64) - 1, offset=(1 << 63) + 5)
    Y = q.qlora_linear_fwd_dropout(w, X0, A.to(DEV), B.to(DEV), ALPHA, drop)
    dA = torch.full((r, d_in), 3.0, device=DEV)
    dB = torch.full((d_out, r), 3.0, device=DEV)
    _, dA, dB = q.qlora_linear_bwd_dropout(w, X0, dY0, A.to(DEV), B.to(DEV), ALPHA, drop,
                                           dA=dA, dB=dB)
    torch.cuda.synchronize()
    assert Y.shape == (0, d_out)
    assert torch.count_nonzero(dA) == 0 and torch.count_nonzero(dB) == 0
    Xm = inputs.activations(70, 136, 126, tensor=inputs.T_X)
    Xk, bits = q.qlora_dropout_mask(Xm.to(DEV), drop, want_bits=True)
    keep = orc.dropout_keep(70, 136, drop.p, drop.seed, drop.offset)
    torch.cuda.synchronize()
    ref = np.where(keep.astype(bool), bits16(Xm).reshape(70, 136), np.uint16(0))
    assert np.array_equal(bits16(Xk).reshape(70, 136), ref)
    assert np.array_equal(bits.cpu().numpy().view(np.uint32), _pack_keep(keep))
    _check_dropout(orc, (96, 192, 48, 8), 127, p=0.99)


def _pack_rows(keep):
    """keep [M, d] (0/1) -> words [M, d/32], bit k % 32 of word k / 32."""
    M, d = keep.shape
    w = np.zeros((M, d // 32), np.uint64)
    for j in range(32):
        w |= keep[:, j::32].astype(np.uint64) << np.uint64(j)
    return w.astype(np.uint32)


@pytest.mark.parametrize("shape", [(256, 1024, 300, 64), (4096, 4096, 4096, 64)])
def test_dropout_saved_mask(orc, shape):
    """The forward writes its mask into the caller's keep_rows / keep_cols
    (equal to the oracle's mask in both layouts), and the backward that reads
    them gives the same dX, dA and dB bit for bit as the backward that
    regenerates the mask."""
    d_out, d_in, M, r = shape
    say(f"dropout saved mask: {shape}")
    W, A, B, X, dY = _layer(d_out, d_in, M, r, 11)
    w = q.qlora_quantize_nf4(W.to(DEV))
    X, dY, A, B = X.to(DEV), dY.to(DEV), A.to(DEV), B.to(DEV)
    drop = q.Dropout(P, seed=77, offset=5)
    saved = drop.saved_mask(M, d_in, DEV)
    T = torch.empty((M, r), dtype=torch.float32, device=DEV)
    Y = q.qlora_linear_fwd_dropout(w, X, A, B, ALPHA, saved, T_save=T)
    Y2 = q.qlora_linear_fwd_dropout(w, X, A, B, ALPHA, drop)
    g_saved = q.qlora_linear_bwd_dropout(w, X, dY, A, B, ALPHA, saved, T_saved=T)
    g_regen = q.qlora_linear_bwd_dropout(w, X, dY, A, B, ALPHA, drop, T_saved=T)
    torch.cuda.synchronize()
    keep = orc.dropout_keep(M, d_in, P, drop.seed, drop.offset)
    assert np.array_equal(saved.keep_cols.cpu().numpy().view(np.uint32), _pack_keep(keep))
    assert np.array_equal(saved.keep_rows.cpu().numpy().view(np.uint32), _pack_rows(keep))
    assert np.array_equal(bits16(Y), bits16(Y2)), "saving the mask changed Y"
    for a, b, name in zip(g_saved, g_regen, ("dX", "dA", "dB")):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), name
