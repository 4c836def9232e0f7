"""GPU parity of the LoRA merge into the NF4 base ([QP §12.3]): the merged
FP32 weight Wh + s B A and its requantized NF4 state, bit-exact against the
CPU oracle."""
import numpy as np
import pytest
import torch

import bit_quantized_lora_quantize_amd as q
from bit_quantized_lora_quantize_amd import inputs
from parity_util import assert_quant_equal, f32, oracle_quant, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
ALPHA = 16.0


@pytest.mark.parametrize("shape", [(256, 256, 8), (37, 320, 16), (130, 192, 100),
                                   (4096, 4096, 64), (11008, 4096, 64)])
def test_merge_and_requantize_bit_exact(orc, shape):
    d_out, d_in, r = shape
    cfg = 95 + (d_out + d_in + r) % 5
    W = inputs.weight(d_out, d_in, config=cfg)
    A, B = inputs.lora_factors(d_out, d_in, r, config=cfg)
    say(f"merge parity: {d_out}x{d_in} r={r}")
    _, _, Wh = oracle_quant(orc, W)
    s = np.float32(ALPHA) / np.float32(r)
    Wm_ref = orc.merge(Wh, f32(A), f32(B), float(s))
    ref_q = orc.quantize_nf4(Wm_ref)
    w = q.qlora_quantize_nf4(W.to(DEV))
    Wm, wq = q.qlora_merge_nf4(w, A.to(DEV), B.to(DEV), ALPHA)
    torch.cuda.synchronize()
    assert np.array_equal(Wm.cpu().numpy().view(np.uint32), Wm_ref.view(np.uint32)), \
        "merged FP32 weights differ"
    assert_quant_equal(wq, ref_q)


def test_merge_zero_adapter(orc):
    """B = 0: the merged weight is the restored weight, and requantizing it
    reproduces the NF4 indices of the base."""
    d_out, d_in, r = 512, 1024, 32
    W = inputs.weight(d_out, d_in, config=97)
    A, _ = inputs.lora_factors(d_out, d_in, r, config=97)
    w = q.qlora_quantize_nf4(W.to(DEV))
    Wh = q.qlora_dequant_bf16(w).float()
    Wm, wq = q.qlora_merge_nf4(w, A.to(DEV), torch.zeros((d_out, r), dtype=torch.bfloat16,
                                                         device=DEV), ALPHA)
    torch.cuda.synchronize()
    assert torch.equal(Wm, Wh)
    assert torch.equal(wq.codes, w.codes)


def test_merge_without_requantize(orc):
    d_out, d_in, r = 64, 128, 4
    W = inputs.weight(d_out, d_in, config=98)
    A, B = inputs.lora_factors(d_out, d_in, r, config=98)
    w = q.qlora_quantize_nf4(W.to(DEV))
    Wm, wq = q.qlora_merge_nf4(w, A.to(DEV), B.to(DEV), ALPHA, requantize=False)
    torch.cuda.synchronize()
    assert wq is None
    _, _, Wh = oracle_quant(orc, W)
    ref = orc.merge(Wh, f32(A), f32(B), float(np.float32(ALPHA) / np.float32(r)))
    assert np.array_equal(Wm.cpu().numpy().view(np.uint32), ref.view(np.uint32))
