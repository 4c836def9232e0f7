"""Seeded synthetic inputs for tests, the smoke check and the benchmark.

Only random draws and shapes live here -- none of the method's arithmetic.
Both the HIP path and the CPU oracle receive the very same bytes from these
generators (drawn once, then copied where needed).

Recipe (std = standard deviation):
  W  FP32 ~ N(0, 0.02), optionally with round(0.001 n) outliers at +-10 std
     (+-0.2, random sign) at positions drawn without replacement;
  A  ~ N(0, 1/r), B ~ N(0, 0.01), both rounded to BF16;
  X, dY ~ N(0, 1) rounded to BF16;
  optimizer state: FP32 gradient ~ N(0, 1e-3), first moment ~ N(0, 1e-4),
  second moment = (a draw of N(0, 1e-3))^2 (non-negative, as after earlier
  steps).
Seeds: seed(config, layer, tensor) = 1000 config + 16 layer + tensor.  A
torch.Generator on the target device draws the values, so CPU and GPU draws
of one seed differ; every comparison moves one draw between devices.
"""
from __future__ import annotations

import torch

T_W, T_A, T_B, T_X, T_DY, T_OUT_POS, T_OUT_SIGN, T_G, T_M, T_V = range(10)

# Decoder-layer projections as (name, d_out, d_in) = nn.Linear weight shapes.
LLAMA_7B = [("q_proj", 4096, 4096), ("k_proj", 4096, 4096), ("v_proj", 4096, 4096),
            ("o_proj", 4096, 4096), ("gate_proj", 11008, 4096), ("up_proj", 11008, 4096),
            ("down_proj", 4096, 11008)]
LLAMA_65B = [("q_proj", 8192, 8192), ("k_proj", 8192, 8192), ("v_proj", 8192, 8192),
             ("o_proj", 8192, 8192), ("gate_proj", 22016, 8192), ("up_proj", 22016, 8192),
             ("down_proj", 8192, 22016)]
LLAMA_65B_LAYERS = 80

W_STD = 0.02
OUTLIER_FRAC = 0.001
OUTLIER_SIGMAS = 10.0
B_STD = 0.01


def seed(config: int, layer: int, tensor: int) -> int:
    return 1000 * config + 16 * layer + tensor


def _gen(s: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(s))
    return g


def normal(shape, std: float, s: int, device="cpu", dtype=torch.float32) -> torch.Tensor:
    """N(0, std) drawn in FP32, then cast to `dtype` (RNE for BF16)."""
    t = torch.randn(*shape, generator=_gen(s, device), device=device, dtype=torch.float32)
    return (t * std).to(dtype)


def weight(d_out: int, d_in: int, config: int, layer: int = 0, outliers: bool = False,
           device="cpu", proj: int = 0) -> torch.Tensor:
    """FP32 W[d_out, d_in] ~ N(0, 0.02) (+ optional 10-std outliers)."""
    base = seed(config, layer, T_W) + 100000 * proj
    W = normal((d_out, d_in), W_STD, base, device)
    if outliers:
        n = W.numel()
        k = int(round(OUTLIER_FRAC * n))
        pos = torch.randperm(n, generator=_gen(base + T_OUT_POS, device), device=device)[:k]
        sign = torch.randint(0, 2, (k,), generator=_gen(base + T_OUT_SIGN, device),
                             device=device).to(torch.float32) * 2 - 1
        W.view(-1)[pos] = sign * (OUTLIER_SIGMAS * W_STD)
    return W


def lora_factors(d_out: int, d_in: int, r: int, config: int, layer: int = 0, device="cpu",
                 proj: int = 0):
    """A[r, d_in] ~ N(0, 1/r), B[d_out, r] ~ N(0, 0.01), BF16."""
    off = 100000 * proj
    A = normal((r, d_in), 1.0 / r, seed(config, layer, T_A) + off, device, torch.bfloat16)
    B = normal((d_out, r), B_STD, seed(config, layer, T_B) + off, device, torch.bfloat16)
    return A, B


def activations(M: int, d: int, config: int, layer: int = 0, tensor: int = T_X, device="cpu",
                proj: int = 0) -> torch.Tensor:
    """X or dY ~ N(0, 1) in BF16."""
    return normal((M, d), 1.0, seed(config, layer, tensor) + 100000 * proj, device,
                  torch.bfloat16)


def optimizer_state(n: int, config: int, layer: int = 0, step: int = 0, device="cpu"):
    """(grad, m, v) FP32 [n]; `step` varies the gradient draw only."""
    g = normal((n,), 1e-3, seed(config, layer, T_G) + 100000 * step, device)
    m = normal((n,), 1e-4, seed(config, layer, T_M), device)
    v = normal((n,), 1e-3, seed(config, layer, T_V), device) ** 2
    return g, m, v
