"""Shared helpers of the GPU parity tests (not a test module).

The HIP path and the oracle receive the same seeded bytes; the oracle never
sees a value the HIP path produced.  Tolerances (floating-point outputs vs the
FP64-accumulating oracle): normwise-max relative 1e-2 and relative-Frobenius
2e-3; quantized bytes and restored BF16 weights are compared bit for bit."""
import os
import sys

import numpy as np
import pytest
import torch

FRO_TOL = 2e-3
MAX_TOL = 1e-2


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    nref = np.linalg.norm(ref)
    fro = np.linalg.norm(got - ref) / nref if nref > 0 else np.linalg.norm(got)
    mref = np.abs(ref).max() if ref.size else 0.0
    mx = np.abs(got - ref).max() / mref if mref > 0 else (np.abs(got).max() if got.size else 0.0)
    return float(fro), float(mx)


def assert_close(name, got, ref, fro_tol=FRO_TOL, max_tol=MAX_TOL):
    fro, mx = rel_errors(got, ref)
    say(f"  {name}: rel-Frobenius {fro:.3e}  normwise-max {mx:.3e}")
    assert fro <= fro_tol and mx <= max_tol, f"{name}: fro {fro:.3e} max {mx:.3e}"


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16).ravel()


def oracle_quant(orc, W: torch.Tensor):
    """Oracle quantization and restored weights (FP32 values) of an FP32 W."""
    Wn = W.detach().cpu().numpy()
    codes, scodes, s2, mean = orc.quantize_nf4(Wn)
    wh_bits = orc.dequant_bf16(codes, scodes, s2, mean, Wn.size)
    return (codes, scodes, s2, mean), wh_bits, orc.bf16_bits_to_f32(wh_bits).reshape(Wn.shape)


def assert_quant_equal(w, ref):
    codes, scodes, s2, mean = ref
    assert np.array_equal(w.codes.cpu().numpy(), codes), "NF4 codes differ"
    assert np.array_equal(w.scale_codes.cpu().numpy(), scodes), "FP8 scale codes differ"
    assert np.array_equal(w.scale2.cpu().numpy().view(np.uint32), s2.view(np.uint32)), \
        "second-level scales differ"
    assert np.float32(w.scale_mean.item()).view(np.uint32) == np.float32(mean).view(np.uint32), \
        "scale mean differs"


def wide_weight_library():
    """Run the enclosed calls on libqlora_wide.so, the in-tree test build whose
    backward GEMM builds its weight descriptors per K step at every size (the
    production library does so only for packed weights beyond 2^31 bytes)."""
    from bit_quantized_lora_quantize_amd import _lib
    path = os.path.join(os.path.dirname(_lib.LIB_PATH), "libqlora_wide.so")
    if not os.path.exists(path):
        pytest.fail("libqlora_wide.so is not built (python -m bit_quantized_lora_quantize_amd.build_lib)")
    return _lib.library(path)
