"""GPU parity of NF4 quantization with double quantization and of double
dequantization to BF16: bit-exact against the CPU oracle."""
import numpy as np
import pytest
import torch

import bit_quantized_lora_quantize_amd as q
from bit_quantized_lora_quantize_amd import inputs
from parity_util import assert_quant_equal, bits16, oracle_quant, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _roundtrip(orc, W: torch.Tensor, label: str):
    say(f"quant parity: {label} shape={tuple(W.shape)}")
    ref, wh_bits, _ = oracle_quant(orc, W)
    w = q.qlora_quantize_nf4(W.to(DEV).contiguous())
    Wb = q.qlora_dequant_bf16(w)
    torch.cuda.synchronize()
    assert_quant_equal(w, ref)
    assert np.array_equal(bits16(Wb), wh_bits), "restored BF16 weights differ"
    return w


@pytest.mark.parametrize("shape", [(256, 256), (1, 64), (3, 64), (5, 192), (37, 320),
                                   (100, 4096), (257, 1024), (64, 11008)])
def test_quantize_dequant_bit_exact(orc, shape):
    d_out, d_in = shape
    W = inputs.weight(d_out, d_in, config=0 if shape == (256, 256) else 90 + d_in % 7,
                      outliers=d_out * d_in >= 64 * 1000)
    _roundtrip(orc, W, "seeded N(0,0.02)")


def test_zero_and_planted_blocks(orc):
    """Zero blocks (index 7), blocks of exact codebook values sharing one
    absmax (s2 = 0 groups, restored scale = mean) and ordinary blocks mixed."""
    c = torch.tensor(orc.codebook())
    g = torch.Generator().manual_seed(5)
    d_out, d_in = 48, 1024                    # 768 blocks, 3 groups
    W = torch.randn(d_out, d_in, generator=g) * 0.02
    # first 256 blocks (group 0): planted codebook values * 2^-4
    idx = torch.randint(0, 16, (256, 64), generator=g)
    idx[:, 0], idx[:, 1] = 0, 15
    W.view(-1)[: 256 * 64] = (c[idx] * 2.0 ** -4).reshape(-1)
    W.view(-1)[256 * 64: 300 * 64] = 0.0      # zero blocks in group 1
    _roundtrip(orc, W.float().contiguous(), "zero + planted blocks")


def test_all_zero_matrix(orc):
    w = _roundtrip(orc, torch.zeros(16, 256), "all zero")
    assert int(w.codes.cpu().numpy().min()) == 0x77


def test_deterministic_repeat(orc):
    W = inputs.weight(300, 2048, config=91, outliers=True).to(DEV)
    w1 = q.qlora_quantize_nf4(W)
    w2 = q.qlora_quantize_nf4(W)
    b1, b2 = q.qlora_dequant_bf16(w1), q.qlora_dequant_bf16(w2)
    torch.cuda.synchronize()
    for a, b in ((w1.codes, w2.codes), (w1.scale_codes, w2.scale_codes),
                 (w1.scale2, w2.scale2), (w1.scale_mean, w2.scale_mean)):
        assert torch.equal(a, b)
    assert torch.equal(b1.view(torch.int16), b2.view(torch.int16))


def test_reuse_output_and_workspace(orc):
    """Quantizing into existing buffers with a caller workspace (state kept
    from a previous, different matrix must not leak)."""
    W1 = inputs.weight(64, 4096, config=92).to(DEV)
    W2 = inputs.weight(64, 4096, config=93, outliers=True)
    ws = torch.empty(q.qlora_workspace_bytes(q.QLORA_OP_QUANTIZE, 64, 4096), dtype=torch.uint8,
                     device=DEV)
    w = q.qlora_quantize_nf4(W1, workspace=ws)
    q.qlora_quantize_nf4(W2.to(DEV), out=w, workspace=ws)
    torch.cuda.synchronize()
    ref, _, _ = oracle_quant(orc, W2)
    assert_quant_equal(w, ref)


@pytest.mark.parametrize("name,d_out,d_in", inputs.LLAMA_7B)
def test_llama7b_layer_roundtrip(orc, name, d_out, d_in):
    """The 7B decoder layer's projections at full size, N(0, 0.02) with 0.1%
    outliers at 10 std: codes, FP8 scales, s2, mean and restored BF16 weights
    bit-exact."""
    proj = [p[0] for p in inputs.LLAMA_7B].index(name)
    W = inputs.weight(d_out, d_in, config=1, layer=0, outliers=True, device=DEV, proj=proj)
    _roundtrip(orc, W.cpu(), f"7B layer {name}")


def test_large_group_tree(orc):
    """8192 x 22016 (the 65B down projection): 11008 second-level groups, so
    the scale-mean tree runs its global-memory levels before the LDS ones."""
    W = inputs.weight(8192, 22016, config=4, layer=0, device=DEV, proj=6)
    _roundtrip(orc, W.cpu(), "65B down_proj")


@pytest.mark.parametrize("shape", [(257, 1024), (4096, 4096)])
def test_quantized_state_file_roundtrip(orc, tmp_path, shape):
    """The quantized state is the four buffers the principles page lists for
    a stored 4-bit weight (§5.3): packed codes, 8-bit block-scale codes, the
    FP32 second-level scales and the mean.  Copied to the host, written to a
    file, read back into fresh device buffers and dequantized, it restores
    the same BF16 bytes as the original buffers (and as the oracle)."""
    d_out, d_in = shape
    W = inputs.weight(d_out, d_in, config=7, layer=0, outliers=True)
    w = _roundtrip(orc, W, "state file round trip")
    ref = q.qlora_dequant_bf16(w)
    path = tmp_path / "nf4_state.npz"
    np.savez(path, codes=w.codes.cpu().numpy(), scale_codes=w.scale_codes.cpu().numpy(),
             scale2=w.scale2.cpu().numpy(), scale_mean=w.scale_mean.cpu().numpy(),
             shape=np.array([d_out, d_in], dtype=np.int64))
    del w
    torch.cuda.synchronize()
    with np.load(path) as f:                      # no pickles: plain arrays only
        d_out2, d_in2 = (int(v) for v in f["shape"])
        w2 = q.NF4Weight(d_out2, d_in2,
                         torch.from_numpy(f["codes"]).to(DEV),
                         torch.from_numpy(f["scale_codes"]).to(DEV),
                         torch.from_numpy(f["scale2"]).to(DEV),
                         torch.from_numpy(f["scale_mean"]).to(DEV))
    out = q.qlora_dequant_bf16(w2)
    torch.cuda.synchronize()
    assert (d_out2, d_in2) == (d_out, d_in)
    assert np.array_equal(bits16(out), bits16(ref)), "reloaded state restores different bytes"


def test_quantize_many_matches_single_calls(orc):
    """The grouped call on the 7B layer's seven projections plus two small
    and ragged tensors (9 > 8 would be refused, so 8 items): every state and
    every restored BF16 weight equals a single call's, bit for bit, and the
    small ones equal the oracle's."""
    shapes = [(4096, 4096), (11008, 4096), (4096, 11008), (4096, 4096), (11008, 4096),
              (4096, 4096), (37, 320), (1, 64)]
    Ws = [inputs.weight(d_out, d_in, config=5, layer=0, outliers=True, device=DEV, proj=i)
          for i, (d_out, d_in) in enumerate(shapes)]
    say("quantize_many: 8 tensors")
    many = q.qlora_quantize_nf4_many(Ws)
    outs = q.qlora_dequant_bf16_many(many)
    for i, W in enumerate(Ws):
        one = q.qlora_quantize_nf4(W)
        torch.cuda.synchronize()
        for name in ("codes", "scale_codes", "scale2", "scale_mean"):
            a, b = getattr(many[i], name), getattr(one, name)
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"item {i} {name}"
        assert np.array_equal(bits16(outs[i]), bits16(q.qlora_dequant_bf16(one))), f"item {i} bf16"
    for i in (6, 7):
        ref, wh_bits, _ = oracle_quant(orc, Ws[i].cpu())
        assert_quant_equal(many[i], ref)
        assert np.array_equal(bits16(outs[i]), wh_bits)


def test_quantize_many_refuses_bad_counts():
    W = torch.zeros((64, 64), dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):
        q.qlora_quantize_nf4_many([W] * 9)
    with pytest.raises(ValueError):
        q.qlora_quantize_nf4_many([])


def test_quantize_many_with_large_group_tree(orc):
    """A list whose middle tensor has 11008 second-level groups (8192 x 22016,
    the 65B down projection): its tree runs the global-memory levels between
    the list's two launches.  Equal to single calls bit for bit, and the
    small ragged neighbours equal the oracle."""
    shapes = [(5, 192), (8192, 22016), (257, 1024)]
    Ws = [inputs.weight(d_out, d_in, config=6, layer=1, device=DEV, proj=i)
          for i, (d_out, d_in) in enumerate(shapes)]
    say("quantize_many: list with an 11008-group tensor")
    many = q.qlora_quantize_nf4_many(Ws)
    for i, W in enumerate(Ws):
        one = q.qlora_quantize_nf4(W)
        torch.cuda.synchronize()
        for name in ("codes", "scale_codes", "scale2", "scale_mean"):
            assert torch.equal(getattr(many[i], name).view(torch.uint8),
                               getattr(one, name).view(torch.uint8)), f"item {i} {name}"
    for i in (0, 2):
        ref, _, _ = oracle_quant(orc, Ws[i].cpu())
        assert_quant_equal(many[i], ref)
