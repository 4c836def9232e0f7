"""GPU parity of the LLaMA-65B-shaped stack: 80 layers x 7 projections
(hidden 8192, FFN 22016), NF4 with FP8 double quantization resident in HBM
(about 33.4 GB packed), forward + backward at M = 2048 tokens, r = 64,
alpha = 16 -- built with the same seeds and the same shared activation and
workspace buffers as the benchmark's stack.

  - every layer: the FP8 scale codes, second-level scales and mean of all
    seven projections bit for bit; NF4 codes and restored BF16 weights bit
    for bit on 16 sampled 256-block groups per projection (first, last and
    random; the oracle's per-weight level search over all 64.8 B weights
    would take many minutes of CPU);
  - layers 0 and 79: every projection in full -- quantized state bit for
    bit, T and dA, dB in full, Y and dX on 32 token rows;
  - layer 40 after the whole stack has run one training step on the shared
    buffers: its outputs (captured as the stack ran) against the oracle, and
    a rerun of the layer on the buffers the later layers left behind equal
    to them bit for bit.
Tolerances as everywhere: normwise-max 1e-2, relative-Frobenius 2e-3 for
floating-point outputs; 1e-4 for the FP32 T."""
import numpy as np
import pytest
import torch

import bit_quantized_lora_quantize_amd as q
from bit_quantized_lora_quantize_amd import inputs
from parity_util import assert_close, assert_quant_equal, bits16, f32, oracle_quant, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
ALPHA, R, M, CFG = 16.0, 64, 2048, 4
LAYERS = inputs.LLAMA_65B_LAYERS
GROUP_WEIGHTS = 64 * 256            # weights under one second-level scale
MID = 40


@pytest.fixture(scope="module")
def stack():
    """The resident stack: weights of layer l, projection p from seeds
    (config 4, layer l, projection p), as the benchmark draws them."""
    say(f"65B stack: quantizing {LAYERS} x 7 projections on the GPU")
    layers = []
    for l in range(LAYERS):
        items = []
        for p, (name, d_out, d_in) in enumerate(inputs.LLAMA_65B):
            W = inputs.weight(d_out, d_in, CFG, l, device=DEV, proj=p)
            w = q.qlora_quantize_nf4(W)
            del W
            A, B = inputs.lora_factors(d_out, d_in, R, CFG, l, device=DEV, proj=p)
            items.append(dict(name=name, p=p, w=w, A=A, B=B, d_out=d_out, d_in=d_in))
        layers.append(items)
    torch.cuda.synchronize()
    say(f"65B stack resident: {sum(it['w'].nbytes() for L in layers for it in L) / 1e9:.2f} GB")
    yield layers
    del layers
    torch.cuda.empty_cache()


def _first_proj_of_shape():
    first = {}
    for p, (_, d_out, d_in) in enumerate(inputs.LLAMA_65B):
        first.setdefault((d_out, d_in), p)
    return first


@pytest.fixture(scope="module")
def acts():
    """Activations, outputs and workspaces per projection shape, shared by
    every layer (X and dY drawn from layer 0's seeds of the shape's first
    projection), as in the benchmark."""
    buf = {}
    for (d_out, d_in), p in _first_proj_of_shape().items():
        buf[(d_out, d_in)] = dict(
            X=inputs.activations(M, d_in, CFG, 0, inputs.T_X, device=DEV, proj=p),
            dY=inputs.activations(M, d_out, CFG, 0, inputs.T_DY, device=DEV, proj=p),
            Y=torch.empty((M, d_out), dtype=torch.bfloat16, device=DEV),
            dX=torch.empty((M, d_in), dtype=torch.bfloat16, device=DEV),
            dA=torch.empty((R, d_in), dtype=torch.float32, device=DEV),
            dB=torch.empty((d_out, R), dtype=torch.float32, device=DEV),
            T=torch.empty((M, R), dtype=torch.float32, device=DEV),
            wsf=torch.empty(q.qlora_workspace_bytes(q.QLORA_OP_FWD, d_out, d_in, M, R),
                            dtype=torch.uint8, device=DEV),
            wsb=torch.empty(q.qlora_workspace_bytes(q.QLORA_OP_BWD, d_out, d_in, M, R),
                            dtype=torch.uint8, device=DEV))
    return buf


def _step(it, a):
    q.qlora_linear_fwd(it["w"], a["X"], it["A"], it["B"], ALPHA, Y=a["Y"], T_save=a["T"],
                       workspace=a["wsf"])
    q.qlora_linear_bwd(it["w"], a["X"], a["dY"], it["A"], it["B"], ALPHA, T_saved=a["T"],
                       dX=a["dX"], dA=a["dA"], dB=a["dB"], workspace=a["wsb"])


def _rows(seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, M - 1], rng.choice(np.arange(1, M - 1), 30,
                                                             replace=False)]))


def _check_outputs(orc, label, it, Wh, a, Y, T, dX, dA, dB, rows):
    s = ALPHA / R
    Xn, An, Bn, dYn = (f32(t) for t in (a["X"], it["A"], it["B"], a["dY"]))
    assert_close(f"{label} Y", f32(Y)[rows], orc.linear_fwd(Wh, Xn, An, Bn, s, rows=rows))
    assert_close(f"{label} T", f32(T), orc.lora_down(Xn, An, s), fro_tol=1e-4, max_tol=1e-4)
    dXr, dAr, dBr = orc.linear_bwd(Wh, Xn, dYn, An, Bn, s, rows=rows)
    assert_close(f"{label} dX", f32(dX)[rows], dXr)
    assert_close(f"{label} dA", f32(dA), dAr)
    assert_close(f"{label} dB", f32(dB), dBr)


@pytest.mark.parametrize("layer", range(LAYERS))
def test_stack65b_quantized_state(orc, stack, layer):
    rng = np.random.default_rng(6500 + layer)
    for it in stack[layer]:
        W = inputs.weight(it["d_out"], it["d_in"], CFG, layer, device=DEV, proj=it["p"])
        Wn = W.cpu().numpy()
        del W
        G = Wn.size // GROUP_WEIGHTS
        sel = np.zeros(G, bool)
        sel[[0, G - 1]] = True
        sel[rng.choice(np.arange(1, G - 1), 14, replace=False)] = True
        codes, scodes, s2, mean = orc.quantize_nf4_sel(Wn, sel)
        del Wn
        w = it["w"]
        assert np.array_equal(w.scale_codes.cpu().numpy(), scodes), f"{it['name']}: FP8 codes"
        assert np.array_equal(w.scale2.cpu().numpy().view(np.uint32), s2.view(np.uint32)), \
            f"{it['name']}: second-level scales"
        assert np.float32(w.scale_mean.item()).view(np.uint32) == np.float32(mean).view(np.uint32)
        gi = np.flatnonzero(sel)
        gi_d = torch.from_numpy(gi).to(DEV)
        got = w.codes.view(G, GROUP_WEIGHTS // 2)[gi_d].cpu().numpy()
        assert np.array_equal(got, codes.reshape(G, -1)[gi]), f"{it['name']}: NF4 codes"
        Wh = q.qlora_dequant_bf16(w)
        got = bits16(Wh.view(G, GROUP_WEIGHTS)[gi_d])
        del Wh
        half = GROUP_WEIGHTS // 2
        ref = np.concatenate([orc.dequant_bf16(codes[g * half:(g + 1) * half],
                                               scodes[g * 256:(g + 1) * 256], s2[g:g + 1], mean,
                                               GROUP_WEIGHTS) for g in gi])
        assert np.array_equal(got, ref), f"{it['name']}: restored BF16 weights"
    say(f"layer {layer}: scale state of 7 projections and 16 groups each bit-exact")


@pytest.mark.parametrize("proj", range(7))
@pytest.mark.parametrize("layer", [0, LAYERS - 1])
def test_stack65b_layer_in_full(orc, stack, acts, layer, proj):
    it = stack[layer][proj]
    W = inputs.weight(it["d_out"], it["d_in"], CFG, layer, device=DEV, proj=proj)
    ref_q, _, Wh = oracle_quant(orc, W.cpu())
    del W
    assert_quant_equal(it["w"], ref_q)
    a = acts[(it["d_out"], it["d_in"])]
    _step(it, a)
    torch.cuda.synchronize()
    _check_outputs(orc, f"layer {layer} {it['name']}", it, Wh, a, a["Y"], a["T"], a["dX"],
                   a["dA"], a["dB"], _rows(650 + 7 * layer + proj))


def test_stack65b_mid_layer_after_full_run(orc, stack, acts):
    captured = {}
    for l in range(LAYERS):
        for it in stack[l]:
            a = acts[(it["d_out"], it["d_in"])]
            _step(it, a)
            if l == MID:
                captured[it["p"]] = tuple(a[k].clone() for k in ("Y", "T", "dX", "dA", "dB"))
    torch.cuda.synchronize()
    say(f"65B stack: one training step over {LAYERS} layers done; checking layer {MID}")
    for it in stack[MID]:
        a = acts[(it["d_out"], it["d_in"])]
        _step(it, a)                      # workspaces as the later layers left them
        torch.cuda.synchronize()
        for k, ref in zip(("Y", "T", "dX", "dA", "dB"), captured[it["p"]]):
            got = a[k]
            same = torch.equal(got.view(torch.int16), ref.view(torch.int16)) \
                if got.dtype == torch.bfloat16 else torch.equal(got, ref)
            assert same, f"{it['name']} {k}: rerun differs from the stack run"
        W = inputs.weight(it["d_out"], it["d_in"], CFG, MID, device=DEV, proj=it["p"])
        _, _, Wh = oracle_quant(orc, W.cpu())
        del W
        _check_outputs(orc, f"layer {MID} {it['name']}", it, Wh, a, *captured[it["p"]],
                       _rows(6540 + it["p"]))
