"""The forward entry point that allocates nothing (qlora_linear_fwd_noalloc,
for callers that cannot allocate: HIP graph capture, serving loops) against
qlora_linear_fwd with a caller workspace: same kernels, so Y and T must be
equal bit for bit.  Two calls in a row on each path, the second smaller, so
the second runs on the scratch the first left behind."""
import pytest
import torch

import bit_quantized_lora_quantize_amd as q
from bit_quantized_lora_quantize_amd import inputs
from parity_util import say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
ALPHA = 16.0


def _case(d_out, d_in, M, r, config):
    W = inputs.weight(d_out, d_in, config, device=DEV)
    A, B = inputs.lora_factors(d_out, d_in, r, config, device=DEV)
    X = inputs.activations(M, d_in, config, 0, inputs.T_X, device=DEV)
    return q.qlora_quantize_nf4(W), X, A, B


@pytest.mark.parametrize("pair", [
    ((11008, 4096, 16, 64), (4096, 4096, 4, 64)),     # weight streaming, M <= 16
    ((4096, 11008, 2048, 64), (1000, 512, 300, 16)),  # fused GEMM
    ((4096, 4096, 4096, 64), (4096, 4096, 1, 8)),     # GEMM, then weight streaming
])
def test_noalloc_forward_equals_workspace_forward(pair):
    for n, (d_out, d_in, M, r) in enumerate(pair):
        say(f"noalloc forward: call {n + 1}, d_out={d_out} d_in={d_in} M={M} r={r}")
        w, X, A, B = _case(d_out, d_in, M, r, 150 + n)
        T_ref = torch.empty((M, r), dtype=torch.float32, device=DEV)
        Y_ref = q.qlora_linear_fwd(w, X, A, B, ALPHA, T_save=T_ref)
        Y = torch.full((M, d_out), 7.0, dtype=torch.bfloat16, device=DEV)
        T = torch.full((M, r), 7.0, dtype=torch.float32, device=DEV)
        q.qlora_linear_fwd_noalloc(w, X, A, B, ALPHA, Y, T_save=T)
        Y2 = torch.empty_like(Y)
        q.qlora_linear_fwd_noalloc(w, X, A, B, ALPHA, Y2)       # T kept in the scratch
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), Y_ref.view(torch.int16))
        assert torch.equal(T, T_ref)
        assert torch.equal(Y2.view(torch.int16), Y_ref.view(torch.int16))


def test_noalloc_forward_rejects_oversized_call():
    w, X, A, B = _case(4096, 4096, 1, 8, 160)
    M, r = 1 << 17, 256
    assert q.qlora_workspace_bytes(q.QLORA_OP_FWD, 4096, 4096, M, r) > q.QLORA_STATIC_SCRATCH_BYTES
    Xb = torch.zeros((M, 4096), dtype=torch.bfloat16, device=DEV)
    Ab = torch.zeros((r, 4096), dtype=torch.bfloat16, device=DEV)
    Bb = torch.zeros((4096, r), dtype=torch.bfloat16, device=DEV)
    Y = torch.empty((M, 4096), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(q.QloraError) as e:
        q.qlora_linear_fwd_noalloc(w, Xb, Ab, Bb, ALPHA, Y)
    assert e.value.status == q.QLORA_ERR_SCRATCH
