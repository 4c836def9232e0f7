"""Pins of the CPU oracle to facts fixed by the pages and by mathematics.

None of these re-types the oracle's own formula: each checks a printed
value, a closed form, an invariant, a special case with a known answer, an
independent library routine, or an exhaustive sweep against an independent
method.  Sources: "第 04 篇：QLoRA 原理" (cited [QP §x]) and the compassingai
"QLoRA" concept page (cited [CP, heading]).
"""
import math

import numpy as np
import pytest
import torch

from conftest import read_golden_kv, read_golden_values




# --------------------------------------------------------------- codebook

def test_codebook_matches_printed_table(orc):
    """[QP §4.3] prints the 16 NF4 values; the oracle uses exactly those."""
    printed = np.array([float(v) for v in read_golden_values("nf4_codebook.txt")], np.float32)
    assert printed.size == 16
    np.testing.assert_array_equal(orc.codebook(), printed)


def test_codebook_properties(orc):
    """[QP §4.3]: unequal gaps, denser near zero, an exact zero, halves built
    separately so the levels are not a mirror image; [QP §3.3] likewise."""
    c = orc.codebook().astype(np.float64)
    assert np.all(np.diff(c) > 0)
    assert c[0] == -1.0 and c[15] == 1.0 and c[7] == 0.0
    assert (c < 0).sum() == 7 and (c > 0).sum() == 8
    assert c[8] != -c[6]                       # not mirrored
    gaps = np.diff(c)
    assert gaps[7] < gaps[0] and gaps[6] < gaps[14]   # denser near 0
    assert len(set(np.round(gaps, 7))) > 2            # not equally spaced


def test_codebook_is_normal_quantile_construction(orc):
    """[QP §4.2-4.3]: equal-probability quantiles of N(0,1), one half with an
    extra level, merged with a single zero and normalized to [-1, 1].  The
    page does not print the outer probability; the fitted p = 0.9677083
    reproduces every printed level to within 1e-7 (the printed decimals carry
    7 digits), and the oracle's FP32 levels are those decimals."""
    from scipy.stats import norm
    p = 0.9677083
    pos = norm.ppf(np.linspace(p, 0.5, 9)[:-1])     # 8 positive levels
    neg = -norm.ppf(np.linspace(p, 0.5, 8)[:-1])    # 7 negative levels
    v = np.sort(np.concatenate([pos, [0.0], neg]))
    v = v / np.abs(v).max()
    printed = np.array([float(t) for t in read_golden_values("nf4_codebook.txt")])
    assert np.abs(v - printed).max() < 1e-7
    assert np.abs(orc.codebook().astype(np.float64) - printed).max() < 3e-8


# ------------------------------------------------------------ NF4 index

def _threshold_index(orc, x):
    """Independent index rule: count the midpoints strictly below x, with
    2*midpoint = c_i + c_{i+1} formed exactly in FP64 and 2x exact."""
    c = orc.codebook().astype(np.float64)
    return np.searchsorted(c[:-1] + c[1:], 2.0 * x.astype(np.float64), side="left").astype(np.uint8)


def test_nf4_index_exhaustive_outer_range(orc):
    """Every FP32 x with 2^-5 <= |x| <= 1 (all 15 midpoints lie in this
    range): nearest level with ties to the lower index equals the
    midpoint-count rule."""
    lo, hi = 0x3D000000, 0x3F800000       # 2^-5 .. 1.0
    step = 1 << 24
    for sign in (0, 0x80000000):
        for start in range(lo, hi + 1, step):
            bits = np.arange(start, min(start + step, hi + 1), dtype=np.uint64)
            x = (bits | sign).astype(np.uint32).view(np.float32)
            np.testing.assert_array_equal(orc.nf4_index(x), _threshold_index(orc, x))


def test_nf4_index_inner_range_is_zero_level(orc):
    """|x| < 2^-5 lies strictly between the midpoints around 0, so the index
    is 7.  The index is monotone in x, so checking a dense sample plus both
    ends of the range covers it."""
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 0x3D000000, size=1 << 20, dtype=np.uint64)
    bits = np.concatenate([bits, [0, 1, 0x3CFFFFFF, 0x00800000]]).astype(np.uint32)
    for sign in (0, 0x80000000):
        x = (bits | np.uint32(sign)).view(np.float32)
        assert np.all(orc.nf4_index(x) == 7)


def test_nf4_index_ties_resolve_low(orc):
    """Midpoints that FP32 represents exactly are real ties; the reading is
    'lower index'.  At least one such midpoint exists (see DESIGN)."""
    c = orc.codebook().astype(np.float64)
    ties = 0
    for i in range(15):
        m = (c[i] + c[i + 1]) / 2
        if float(np.float32(m)) == m:
            ties += 1
            assert orc.nf4_index(np.array([m], np.float32))[0] == i
    assert ties >= 1


# ------------------------------------------------------------------ FP8

def test_fp8_decode_all_codes_match_library(orc):
    """All 256 E4M3FN codes decode as torch's float8_e4m3fn (OCP) does."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = np.array([orc.fp8_decode(int(k)) for k in codes], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert orc.fp8_decode(0x7E) == 448.0 and orc.fp8_decode(0x01) == 2.0 ** -9


def _fp8_probe_values():
    """Every FP32 value within 64 ulps of each midpoint between adjacent
    E4M3FN magnitudes and of each magnitude, both signs, plus a strided
    sweep of all patterns below 464."""
    mags = np.array([float(torch.tensor(k, dtype=torch.uint8).view(torch.float8_e4m3fn).float())
                     for k in range(0x7F)], np.float64)
    centers = np.concatenate([mags, (mags[:-1] + mags[1:]) / 2])
    cb = np.float32(centers).view(np.uint32).astype(np.int64)
    offs = np.arange(-64, 65, dtype=np.int64)
    near = (cb[:, None] + offs[None, :]).ravel()
    near = near[(near >= 0) & (near < 0x43E80000)]
    strided = np.arange(0, 0x43E80000, 997, dtype=np.int64)
    pos = np.concatenate([near, strided]).astype(np.uint32)
    return np.concatenate([pos, pos | np.uint32(0x80000000)]).view(np.float32)


def test_fp8_encode_matches_library_rne(orc):
    """Nearest-even FP8 encoding equals torch's float8_e4m3fn cast (RNE) on
    every probe below 464 in magnitude (torch turns larger values into NaN;
    the reading there is saturation, checked next)."""
    y = _fp8_probe_values()
    got = orc.fp8_encode(y)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got, ref)


def test_fp8_encode_saturates_and_keeps_sign(orc):
    y = np.array([464.0, 480.0, 1e6, np.inf, -1e30, -np.inf, -0.0, 0.0, -1e-30], np.float32)
    np.testing.assert_array_equal(orc.fp8_encode(y),
                                  np.array([0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x80, 0x00, 0x80], np.uint8))


# ----------------------------------------------------------------- BF16

def test_bf16_rne_matches_library(orc):
    """RNE to BF16 equals torch's float32 -> bfloat16 cast: every low-half
    pattern for a set of high halves (zero, subnormals, ordinary values, the
    largest finite), and a strided sweep of all finite patterns."""
    highs = np.array([0x0000, 0x0001, 0x007F, 0x0080, 0x3F80, 0x3F81, 0x4049,
                      0x7F7E, 0x7F7F, 0x0123, 0x3C00, 0x4000], np.uint32)
    low = np.arange(1 << 16, dtype=np.uint32)
    bits = (highs[:, None] << 16 | low[None, :]).ravel()
    bits = np.concatenate([bits, np.arange(0, 0x7F800000, 4099, dtype=np.uint32)])
    bits = np.concatenate([bits, bits | np.uint32(0x80000000)])
    x = bits.view(np.float32)
    got = orc.bf16_rne(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, ref)


# ------------------------------------------------------------ scale mean

def test_scale_mean_is_the_mean(orc):
    """The tree-summed mean equals the exactly rounded mean of the absmax
    values to within one FP32 rounding, for ragged group counts."""
    rng = np.random.default_rng(2)
    for n1 in (1, 7, 256, 257, 1000, 4096, 12352, 70001):
        a = np.abs(rng.normal(0, 0.05, n1)).astype(np.float32)
        exact = math.fsum(a.astype(np.float64).tolist()) / n1
        got = orc.scale_mean(a)
        assert abs(got - exact) <= 0.5 * np.spacing(np.float32(exact)) * (1 + 1e-6)


# ------------------------------------------------------------ quantize

def _planted_exact_matrix(orc, d_out, d_in, k, seed):
    """Blocks holding codebook values times 2^k, each block containing both
    -1 and +1 so every absmax is exactly 2^k; returns (W, planted indices)."""
    rng = np.random.default_rng(seed)
    n = d_out * d_in
    idx = rng.integers(0, 16, size=n).astype(np.uint8)
    idx = idx.reshape(-1, 64)
    idx[:, 0] = 0
    idx[:, 1] = 15
    for b in range(idx.shape[0]):
        rng.shuffle(idx[b])
    idx = idx.ravel()
    W = (orc.codebook()[idx].astype(np.float64) * 2.0 ** k).astype(np.float32)
    return W.reshape(d_out, d_in), idx


def test_quantize_planted_codebook_blocks(orc):
    """Special case with a known answer: every block is a permutation of
    codebook values scaled by 2^k containing both ends, so absmax = 2^k
    everywhere, the mean is 2^k, every centred scale is 0 (s2 = 0, FP8 code
    0), each index is the planted one, and the restored weights are
    RNE_bf16(c) * 2^k exactly.  Also fixes the nibble order (element 2j in
    the low nibble)."""
    for k in (-3, -7, 0):
        W, idx = _planted_exact_matrix(orc, 8, 192, k, seed=10 + k)
        codes, scodes, s2, mean = orc.quantize_nf4(W)
        packed = (idx[0::2] | (idx[1::2] << 4)).astype(np.uint8)
        np.testing.assert_array_equal(codes, packed)
        assert mean == 2.0 ** k
        assert np.all(s2 == 0) and np.all(scodes == 0)
        wh = orc.bf16_bits_to_f32(orc.dequant_bf16(codes, scodes, s2, mean, W.size))
        c_bf16 = orc.bf16_bits_to_f32(orc.bf16_rne(orc.codebook()))
        np.testing.assert_array_equal(wh, (c_bf16[idx].astype(np.float64) * 2.0 ** k).astype(np.float32))


def test_quantize_zero_blocks(orc):
    """A zero block has absmax 0 and maps every element to the exact-zero
    level (index 7, byte 0x77); an all-zero matrix restores to zeros."""
    W = np.zeros((4, 128), np.float32)
    codes, scodes, s2, mean = orc.quantize_nf4(W)
    assert np.all(codes == 0x77) and mean == 0.0 and np.all(s2 == 0) and np.all(scodes == 0)
    wh = orc.bf16_bits_to_f32(orc.dequant_bf16(codes, scodes, s2, mean, W.size))
    assert np.all(wh == 0)
    W = np.random.default_rng(3).normal(0, 0.02, (4, 128)).astype(np.float32)
    W[1, 64:128] = 0
    codes, *_ = orc.quantize_nf4(W)
    assert np.all(codes.reshape(4, 64)[1, 32:] == 0x77)


def _unpack(codes):
    return np.stack([codes & 15, codes >> 4], axis=1).ravel().astype(np.int64)


def test_quantize_roundtrip_error_bound(orc):
    """[QP §3.5, §5.4] error decomposition: without DQ, |w - c_idx a| is at
    most half the local level gap times a (nearest level); with DQ the
    restored weight adds |c_idx| |a - a_hat| and the BF16 rounding.
    Weights N(0, 0.02) with 0.1% outliers at 10 sigma; ragged group count."""
    rng = np.random.default_rng(4)
    d_out, d_in = 96, 704
    W = rng.normal(0, 0.02, (d_out, d_in)).astype(np.float32)
    flat = W.ravel()
    pos = rng.choice(flat.size, size=max(1, flat.size // 1000), replace=False)
    flat[pos] = np.where(rng.random(pos.size) < 0.5, -0.2, 0.2).astype(np.float32)
    W = flat.reshape(d_out, d_in)
    codes, scodes, s2, mean, absmax = orc.quantize_nf4(W, return_absmax=True)
    c = orc.codebook().astype(np.float64)
    idx = _unpack(codes)
    w = W.ravel().astype(np.float64)
    a = np.repeat(absmax.astype(np.float64), 64)
    np.testing.assert_array_equal(absmax, np.abs(W.reshape(-1, 64)).max(axis=1))
    # nearest level: the chosen level is at least as close as both neighbours
    x = w / a
    d_chosen = np.abs(x - c[idx])
    d_left = np.abs(x - c[np.maximum(idx - 1, 0)])
    d_right = np.abs(x - c[np.minimum(idx + 1, 15)])
    assert np.all(d_chosen <= d_left + 1e-7) and np.all(d_chosen <= d_right + 1e-7)
    gap = np.maximum(np.diff(c)[np.clip(idx - 1, 0, 14)], np.diff(c)[np.clip(idx, 0, 14)])
    assert np.all(np.abs(w - c[idx] * a) <= a * gap / 2 * (1 + 1e-6) + 1e-9)
    # DQ: restored scale within half an FP8 step of s2 (plus FP32 rounding)
    ah = np.repeat(orc.restored_scales(scodes, s2, mean).astype(np.float64), 64)
    s2b = np.repeat(np.repeat(s2.astype(np.float64), 256)[: absmax.size], 64)
    y = np.abs(a - mean) / np.where(s2b > 0, s2b, 1)
    fp8_half_step = np.where(y < 2 ** -6, 2.0 ** -10, 2.0 ** (np.floor(np.log2(np.maximum(y, 2 ** -6))) - 4))
    assert np.all(np.abs(a - ah) <= s2b * fp8_half_step * (1 + 1e-5) + 4 * np.spacing(np.float32(a.max())))
    wh = orc.bf16_bits_to_f32(orc.dequant_bf16(codes, scodes, s2, mean, W.size)).astype(np.float64)
    bound = a * gap / 2 + np.abs(c[idx]) * np.abs(a - ah) + np.abs(wh) * 2.0 ** -8 + 1e-9
    assert np.all(np.abs(w - wh) <= bound * (1 + 1e-5))


def test_second_level_group_max_maps_to_448(orc):
    """Symmetric second level: in each group the largest |centred scale|
    encodes to the largest finite FP8 magnitude (448)."""
    rng = np.random.default_rng(5)
    W = rng.normal(0, 0.02, (40, 64 * 40)).astype(np.float32)
    codes, scodes, s2, mean, absmax = orc.quantize_nf4(W, return_absmax=True)
    G = s2.size
    for g in range(G):
        d = absmax[g * 256:(g + 1) * 256] - np.float32(mean)
        j = int(np.argmax(np.abs(d)))
        assert scodes[g * 256 + j] & 0x7F == 0x7E
        assert (scodes[g * 256 + j] >> 7) == (1 if d[j] < 0 else 0)


# ------------------------------------------------------- bits per parameter

def _storage_bits_per_param(n):
    n1 = n // 64
    G = -(-n1 // 256)
    return (n // 2 + n1 + 4 * G + 4) * 8 / n


def test_bits_per_param_closed_form_and_printed_figures():
    """[QP §5.1, §5.3]; [CP, 雙重量化]: 32/64 = 0.5 bit of scales without DQ,
    8/64 + 32/(64*256) with DQ, a saving of about 0.37 bit/param; for 65B
    parameters about 3.0 GB = 2.82 GiB saved and 33.53 GB = 31.23 GiB in
    total (codes plus scales)."""
    fig = read_golden_kv("dq_memory_figures.txt")
    b1, b2 = int(fig["block1"]), int(fig["block2"])
    no_dq = 32 / b1
    dq = 8 / b1 + 32 / (b1 * b2)
    assert no_dq == 0.5 and abs(dq - 0.126953125) < 1e-15
    assert round(no_dq - dq, 2) == fig["saving_bits_per_param"]
    P = 65e9
    saved = P * (no_dq - dq) / 8
    assert round(saved / 1e9, 1) == fig["saving_65b_GB"]
    assert round(saved / 2 ** 30, 2) == fig["saving_65b_GiB"]
    total = P * (4 + dq) / 8
    assert round(total / 1e9, 2) == fig["total_65b_GB"]
    assert round(total / 2 ** 30, 2) == fig["total_65b_GiB"]
    # the buffers the oracle returns realise this rate (+ one FP32 mean)
    for n in (4096 * 4096, 11008 * 4096, 256 * 256):
        assert abs(_storage_bits_per_param(n) - (4 + dq + 32 / n)) < 1e-12


def test_quantize_buffer_sizes(orc):
    W = np.random.default_rng(6).normal(0, 0.02, (3, 64 * 300)).astype(np.float32)
    codes, scodes, s2, mean = orc.quantize_nf4(W)
    n = W.size
    assert codes.size == n // 2 and scodes.size == n // 64 and s2.size == -(-(n // 64) // 256)
    assert (codes.nbytes + scodes.nbytes + s2.nbytes + 4) * 8 / n == _storage_bits_per_param(n)


# ------------------------------------------------------------ LoRA linear

def _small_layer(seed, d_out=24, d_in=128, M=5, r=3):
    rng = np.random.default_rng(seed)
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).float().numpy()
    Wh = bf(rng.normal(0, 0.02, (d_out, d_in)))
    X = bf(rng.normal(0, 1, (M, d_in)))
    A = bf(rng.normal(0, 1 / r, (r, d_in)))
    B = bf(rng.normal(0, 0.01, (d_out, r)))
    dY = bf(rng.normal(0, 1, (M, d_out)))
    return Wh, X, A, B, dY


def test_forward_equals_merged_weight_product(orc):
    """[QP §12.3] merge identity: y = (W + s B A) x.  The merged weight is
    built with Python fractions-free FP64 loops over a tiny layer and applied
    to x; the oracle's branch form must agree to FP64 rounding."""
    Wh, X, A, B, _ = _small_layer(7, d_out=5, d_in=64, M=3, r=2)
    s = 16 / 2
    d_out, d_in = Wh.shape
    r = A.shape[0]
    merged = [[float(Wh[o, c]) + s * sum(float(B[o, i]) * float(A[i, c]) for i in range(r))
               for c in range(d_in)] for o in range(d_out)]
    ref = np.array([[sum(merged[o][c] * float(X[m, c]) for c in range(d_in))
                     for o in range(d_out)] for m in range(X.shape[0])])
    np.testing.assert_allclose(orc.linear_fwd(Wh, X, A, B, s), ref, rtol=1e-12, atol=1e-14)


def test_forward_one_hot_tokens_read_columns(orc):
    """A one-hot token e_k reads column k of the restored weight (B = 0), and
    the LoRA branch alone (W = 0, A = one-hot rows) reads s * B columns: a
    transposed operand would read rows instead."""
    Wh, X, A, B, _ = _small_layer(8, d_out=7, d_in=64, M=3, r=4)
    ks = [0, 17, 63]
    E = np.zeros((3, 64), np.float32)
    E[np.arange(3), ks] = 1
    Y = orc.linear_fwd(Wh, E, A, np.zeros_like(B), 2.0)
    np.testing.assert_array_equal(Y, Wh[:, ks].T.astype(np.float64))
    A1 = np.zeros((4, 64), np.float32)
    A1[2, 17] = 1
    Y = orc.linear_fwd(np.zeros_like(Wh), E, A1, B, 0.25)
    np.testing.assert_array_equal(Y[1], 0.25 * B[:, 2].astype(np.float64))
    np.testing.assert_array_equal(Y[0], 0 * Y[0])


def _inner(a, b):
    return float(np.sum(np.asarray(a, np.float64) * np.asarray(b, np.float64)))


@pytest.mark.parametrize("shape", [(24, 128, 5, 3), (64, 64, 1, 1), (33, 192, 9, 8)])
def test_backward_adjoint_identities(orc, shape):
    """[QP §2.4]: gradients for X, A, B and none for W.  Y is linear in each
    of X, A, B separately, so <dY, Y(V)> = <grad, V> exactly: this pins the
    backward (dX, dA, dB) to the forward with no shared formula."""
    d_out, d_in, M, r = shape
    Wh, X, A, B, dY = _small_layer(9 + M, d_out, d_in, M, r)
    s = 16.0 / r
    rng = np.random.default_rng(11)
    dX, dA, dB = orc.linear_bwd(Wh, X, dY, A, B, s)
    VX = rng.normal(size=X.shape).astype(np.float32)
    lhs = _inner(dY, orc.linear_fwd(Wh, VX, A, B, s))
    assert abs(lhs - _inner(dX, VX)) <= 1e-10 * (abs(lhs) + 1)
    VA = rng.normal(size=A.shape).astype(np.float32)
    lhs = _inner(dY, orc.linear_fwd(np.zeros_like(Wh), X, VA, B, s))
    assert abs(lhs - _inner(dA, VA)) <= 1e-10 * (abs(lhs) + 1)
    VB = rng.normal(size=B.shape).astype(np.float32)
    lhs = _inner(dY, orc.linear_fwd(np.zeros_like(Wh), X, A, VB, s))
    assert abs(lhs - _inner(dB, VB)) <= 1e-10 * (abs(lhs) + 1)


def test_backward_special_cases(orc):
    """B = 0 gives dA = 0; A = 0 gives dB = 0; W = 0 and B = 0 give dX = 0."""
    Wh, X, A, B, dY = _small_layer(12)
    _, dA, _ = orc.linear_bwd(Wh, X, dY, A, np.zeros_like(B), 2.0)
    assert np.all(dA == 0)
    _, _, dB = orc.linear_bwd(Wh, X, dY, np.zeros_like(A), B, 2.0)
    assert np.all(dB == 0)
    dX, _, _ = orc.linear_bwd(np.zeros_like(Wh), X, dY, A, np.zeros_like(B), 2.0)
    assert np.all(dX == 0)


def test_rows_subset_matches_full(orc):
    """Sampled-row evaluation returns the same rows as the full evaluation."""
    Wh, X, A, B, dY = _small_layer(13, M=9)
    rows = np.array([8, 0, 4])
    np.testing.assert_array_equal(orc.linear_fwd(Wh, X, A, B, 0.5, rows=rows),
                                  orc.linear_fwd(Wh, X, A, B, 0.5)[rows])
    np.testing.assert_array_equal(orc.linear_bwd(Wh, X, dY, A, B, 0.5, rows=rows)[0],
                                  orc.linear_bwd(Wh, X, dY, A, B, 0.5)[0][rows])


def test_lora_down_one_hot_tokens_read_columns(orc):
    """[QP §2.2] T = s D(X) A^T: a one-hot token e_k gives s times column k
    of A (a transposed operand would give a row); with dropout, a kept one-hot
    token gives s A[:, k] / (1 - p) and a dropped one gives 0."""
    _, _, A, _, _ = _small_layer(40, d_out=4, d_in=64, M=2, r=5)
    ks = [3, 40, 63]
    E = np.zeros((3, 64), np.float32)
    E[np.arange(3), ks] = 1
    T = orc.lora_down(E, A, 0.25)
    np.testing.assert_array_equal(T, 0.25 * A[:, ks].T.astype(np.float64))
    keep = np.ones(E.shape, np.uint8)
    keep[1, 40] = 0
    T = orc.lora_down(E, A, 0.25, keep=keep, p=0.5)   # 1 - p = 0.5: exact scaling
    np.testing.assert_array_equal(T[[0, 2]], 0.5 * A[:, [3, 63]].T.astype(np.float64))
    assert np.all(T[1] == 0)


def test_lora_down_is_the_forward_and_backward_intermediate(orc):
    """T is the quantity that both the forward and dB use: with W = 0 and a
    one-hot B row (B[o] = e_i), Y[:, o] = T[:, i]; with a one-hot dY row
    (dY[m] = e_o, other rows 0), dB[o, :] = T[m, :].  Both hold bit for bit."""
    Wh, X, A, B, dY = _small_layer(41, d_out=6, d_in=128, M=4, r=3)
    s = 16.0 / 3
    T = orc.lora_down(X, A, s)
    B1 = np.zeros_like(B)
    B1[2, 1] = 1
    Y = orc.linear_fwd(np.zeros_like(Wh), X, A, B1, s)
    np.testing.assert_array_equal(Y[:, 2], T[:, 1])
    dY1 = np.zeros_like(dY)
    dY1[3, 5] = 1
    _, _, dB = orc.linear_bwd(Wh, X, dY1, A, B, s, want_dx=False, want_da=False)
    np.testing.assert_array_equal(dB[5], T[3])
    keep = orc.dropout_keep(*X.shape, 0.2, 3, 4)
    Tk = orc.lora_down(X, A, s, keep=keep, p=0.2)
    Y = orc.linear_fwd(np.zeros_like(Wh), X, A, B1, s, keep=keep, p=0.2)
    np.testing.assert_array_equal(Y[:, 2], Tk[:, 1])


def test_quantize_selected_groups_match_full(orc):
    """The sampled-group quantization gives the full quantization's codes on
    the selected groups, zero codes elsewhere, and the full scale state."""
    rng = np.random.default_rng(42)
    W = rng.normal(0, 0.02, (40, 1024)).astype(np.float32)   # 640 blocks, 3 groups
    W.ravel()[rng.choice(W.size, 40, replace=False)] = 0.2
    full = orc.quantize_nf4(W)
    sel = np.array([True, False, True])
    part = orc.quantize_nf4_sel(W, sel)
    np.testing.assert_array_equal(part[1], full[1])
    np.testing.assert_array_equal(part[2].view(np.uint32), full[2].view(np.uint32))
    assert np.float32(part[3]) == np.float32(full[3])
    per_group = 256 * 64 // 2
    for g, on in enumerate(sel):
        got = part[0][g * per_group:(g + 1) * per_group]
        ref = full[0][g * per_group:(g + 1) * per_group]
        np.testing.assert_array_equal(got, ref if on else np.zeros_like(ref))


# ------------------------------------------------------------------ LoRA merge

def test_merge_planted_powers_of_two(orc):
    """[QP §12.3] merge with a known answer: a planted base (codebook values
    times 2^-4, restored exactly), a rank-1 adapter with B = 2^-5 and
    A = +-2^-6 and s = 2, so every merged value Wh + s B A = Wh +- 2^-10 is
    representable and the FP32 rounding is exact."""
    W, idx = _planted_exact_matrix(orc, 4, 128, -4, seed=31)
    codes, scodes, s2, mean = orc.quantize_nf4(W)
    Wh = orc.bf16_bits_to_f32(orc.dequant_bf16(codes, scodes, s2, mean, W.size)).reshape(4, 128)
    sign = np.where(np.arange(128) % 3 == 0, -1.0, 1.0)
    A = (sign * 2.0 ** -6).astype(np.float32).reshape(1, 128)
    B = np.full((4, 1), 2.0 ** -5, np.float32)
    Wm = orc.merge(Wh, A, B, 2.0)
    expect = Wh.astype(np.float64) + sign[None, :] * 2.0 ** -10
    np.testing.assert_array_equal(Wm, expect.astype(np.float32))
    assert np.all(expect.astype(np.float32) == expect)


def test_merge_zero_adapter_requantizes_to_same_codes(orc):
    """A zero adapter leaves the restored weight unchanged (bit for bit), and
    quantizing it again reproduces every NF4 index: each block's largest
    element restores to +-bf16(scale) and becomes +-1 after the new absmax
    division, and every other element moves by at most a BF16 rounding,
    far less than half the smallest gap between levels."""
    rng = np.random.default_rng(5)
    W = rng.normal(0, 0.02, (16, 256)).astype(np.float32)
    codes, scodes, s2, mean = orc.quantize_nf4(W)
    Wh = orc.bf16_bits_to_f32(orc.dequant_bf16(codes, scodes, s2, mean, W.size)).reshape(16, 256)
    A = rng.normal(0, 0.1, (4, 256)).astype(np.float32)
    Wm = orc.merge(Wh, A, np.zeros((16, 4), np.float32), 4.0)
    np.testing.assert_array_equal(Wm, Wh)
    codes2, *_ = orc.quantize_nf4(Wm)
    np.testing.assert_array_equal(codes2, codes)


def test_merge_applied_equals_lora_forward(orc):
    """The merged weight applied to tokens equals the unmerged LoRA forward
    up to the one FP32 rounding of each merged element."""
    Wh, X, A, B, _ = _small_layer(11, d_out=24, d_in=128, M=6, r=4)
    s = np.float32(16.0) / np.float32(4)
    Wm = orc.merge(Wh, A, B, float(s))
    got = X.astype(np.float64) @ Wm.astype(np.float64).T
    ref = orc.linear_fwd(Wh, X, A, B, float(s))
    # |rounding| <= 2^-24 |Wm| per element
    bound = np.abs(X).astype(np.float64) @ (np.abs(Wm).astype(np.float64).T * 2.0 ** -24)
    assert np.all(np.abs(got - ref) <= bound + 1e-300)


# ---------------------------------------------------------- optimizer step

def test_sumsq_is_the_sum_of_squares(orc):
    """The fixed-order FP64 sum of squares equals the exactly rounded sum
    (math.fsum of the exact squares) within n FP64 roundings."""
    for n in (1, 255, 256, 257, 70000):
        g = np.random.default_rng(n).normal(0, 1, n).astype(np.float32)
        S = orc.sumsq(g)
        ref = math.fsum(float(x) * float(x) for x in g)
        assert abs(S - ref) <= n * 2.0 ** -52 * ref


def test_adamw_first_step_moves_by_lr(orc):
    """From zero moments the first bias-corrected step is lr * g / (|g| +
    eps), i.e. each weight moves by lr against its gradient's sign."""
    rng = np.random.default_rng(2)
    p0 = rng.normal(0, 1, 512).astype(np.float32)
    g = rng.normal(0, 1, 512).astype(np.float32)
    lr, eps = 2e-4, 1e-8
    p, m, v, _ = orc.adamw(p0, g, np.zeros(512, np.float32), np.zeros(512, np.float32),
                           lr, 0.9, 0.999, eps, 0.0, 1)
    step = p0.astype(np.float64) - p
    expect = lr * np.sign(g)
    tol = lr * (eps / np.abs(g) + 8 * 2.0 ** -24) + 2 * np.spacing(np.abs(p0))
    assert np.all(np.abs(step - expect) <= tol)


def test_adamw_weight_decay_alone_is_geometric(orc):
    """Zero gradients leave the moments at zero and the update is the
    decoupled decay alone: p_t = p_0 (1 - lr wd)^t."""
    rng = np.random.default_rng(4)
    p = rng.normal(0, 1, 300).astype(np.float32)
    m = np.zeros(300, np.float32)
    v = np.zeros(300, np.float32)
    z = np.zeros(300, np.float32)
    lr, wd, T = 1e-2, 0.1, 20
    q = p.copy()
    for t in range(1, T + 1):
        q, m, v, _ = orc.adamw(q, z, m, v, lr, 0.9, 0.999, 1e-8, wd, t)
    assert np.all(m == 0) and np.all(v == 0)
    np.testing.assert_allclose(q, p.astype(np.float64) * (1 - lr * wd) ** T, rtol=T * 2.0 ** -22)


def test_adamw_matches_torch_adamw(orc):
    """Special case that reduces to a library routine: the oracle's steps
    follow torch.optim.AdamW (FP32, decoupled decay) to within FP32
    rounding-order differences over several steps."""
    rng = np.random.default_rng(9)
    p0 = rng.normal(0, 0.1, (64, 96)).astype(np.float32)
    grads = [rng.normal(0, 1e-2, (64, 96)).astype(np.float32) for _ in range(6)]
    lr, b1, b2, eps, wd = 2e-4, 0.9, 0.999, 1e-8, 0.01
    tp = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.AdamW([tp], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd,
                            foreach=False)
    p, m, v = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
    for t, g in enumerate(grads, 1):
        tp.grad = torch.from_numpy(g.copy())
        opt.step()
        p, m, v, _ = orc.adamw(p, g, m, v, lr, b1, b2, eps, wd, t)
    np.testing.assert_allclose(p, tp.detach().numpy(), rtol=0, atol=1e-6)


def test_clip_coefficient_matches_torch_and_is_scale_invariant(orc):
    """The clip coefficient agrees with torch.nn.utils.clip_grad_norm_ for
    the same gradients, and scaling every gradient by k leaves the clipped
    gradients unchanged (to FP32 rounding)."""
    rng = np.random.default_rng(12)
    gs = [rng.normal(0, 1, n).astype(np.float32) for n in (1000, 4096, 77)]
    S = sum(orc.sumsq(g) for g in gs)
    c = orc.clip_coef(S, 0.3)
    ts = [torch.nn.Parameter(torch.zeros(len(g))) for g in gs]
    for t, g in zip(ts, gs):
        t.grad = torch.from_numpy(g.copy())
    torch.nn.utils.clip_grad_norm_(ts, 0.3)
    for t, g in zip(ts, gs):
        np.testing.assert_allclose(t.grad.numpy(), g * c, rtol=2e-6)
    k = 37.0
    S2 = sum(orc.sumsq((g * k).astype(np.float32)) for g in gs)
    c2 = orc.clip_coef(S2, 0.3)
    for g in gs:
        np.testing.assert_allclose((g * k).astype(np.float32) * c2, g * c, rtol=1e-6)
    assert orc.clip_coef(1e-6, 0.3) == 1.0


# ------------------------------------------------------------ LoRA dropout

def test_philox_known_answers(orc):
    """Philox4x32-10 reproduces the generator's published known answers
    (fixture philox4x32_10_kat.txt, with its citation)."""
    for line in read_golden_values("philox4x32_10_kat.txt"):
        w = [int(t, 16) for t in line.split()]
        out = orc.philox4x32_10(w[0:4], w[4:6])
        assert [int(x) for x in out] == w[6:10]


@pytest.mark.parametrize("p", [0.0, 0.05, 0.1, 0.5])
def test_dropout_keep_rate_and_uniformity(orc, p):
    """Each element is dropped with probability p: the kept fraction lies
    within 5 binomial standard deviations of 1 - p, per row group of four
    and per column (a wrong word index or counter would skew one of them)."""
    M, d = 512, 1024
    keep = orc.dropout_keep(M, d, p, seed=0x1234_5678_9ABC, offset=3)
    n = keep.size
    q = 1 - np.float32(p)
    if p == 0:
        assert keep.all()
        return
    sd = math.sqrt(n * p * (1 - p))
    assert abs(keep.sum() - n * q) <= 5 * sd
    for j in range(4):  # rows m with m % 4 == j use output word j
        sub = keep[j::4]
        assert abs(sub.sum() - sub.size * q) <= 5 * math.sqrt(sub.size * p * (1 - p))
    cols = keep.sum(axis=0)
    assert abs(cols.mean() - M * q) <= 5 * math.sqrt(M * p * (1 - p) / d)


def test_dropout_masks_differ_by_seed_and_offset_only(orc):
    """Same (seed, offset): the same mask (the backward regenerates the
    forward's); another offset or seed: an independent mask, agreeing on
    about q^2 + p^2 of the elements."""
    p, M, d = 0.1, 256, 512
    a = orc.dropout_keep(M, d, p, 11, 0)
    assert np.array_equal(a, orc.dropout_keep(M, d, p, 11, 0))
    for b in (orc.dropout_keep(M, d, p, 11, 1), orc.dropout_keep(M, d, p, 12, 0),
              orc.dropout_keep(M, d, p, 11, 1 << 32)):
        agree = float((a == b).mean())
        assert abs(agree - (0.81 + 0.01)) < 0.01


def test_dropout_linear_special_cases(orc):
    """Keeping everything at p = 0 is the plain layer; keeping everything at
    p scales the LoRA branch by 1 / (1 - p) exactly; dropped inputs do not
    reach the LoRA branch, kept ones do."""
    Wh, X, A, B, dY = _small_layer(21, d_out=16, d_in=128, M=6, r=4)
    s = 4.0
    ones = np.ones(X.shape, np.uint8)
    np.testing.assert_array_equal(orc.linear_fwd(Wh, X, A, B, s, keep=ones, p=0.0),
                                  orc.linear_fwd(Wh, X, A, B, s))
    for got, ref in zip(orc.linear_bwd(Wh, X, dY, A, B, s, keep=ones, p=0.0),
                        orc.linear_bwd(Wh, X, dY, A, B, s)):
        np.testing.assert_array_equal(got, ref)
    Z = np.zeros_like(Wh)
    p = 0.25  # 1 - p = 0.75: a power-of-two ratio keeps the scaling exact
    np.testing.assert_allclose(orc.linear_fwd(Z, X, A, B, s, keep=ones, p=p),
                               orc.linear_fwd(Z, X, A, B, s) / 0.75, rtol=1e-13)
    keep = orc.dropout_keep(*X.shape, 0.3, 5, 9)
    X2 = X.copy()
    X2[keep == 0] = 123.0
    np.testing.assert_array_equal(orc.linear_fwd(Z, X2, A, B, s, keep=keep, p=0.3),
                                  orc.linear_fwd(Z, X, A, B, s, keep=keep, p=0.3))
    X3 = X.copy()
    X3[keep == 1] += 1.0
    assert not np.array_equal(orc.linear_fwd(Z, X3, A, B, s, keep=keep, p=0.3),
                              orc.linear_fwd(Z, X, A, B, s, keep=keep, p=0.3))


@pytest.mark.parametrize("shape", [(24, 128, 5, 3), (33, 192, 9, 8)])
def test_dropout_backward_adjoint_identities(orc, shape):
    """With the mask fixed, Y is still linear in X, A and B separately, so
    <dY, Y(V)> = <grad, V> pins the dropout backward (the mask on dX's LoRA
    term, the dropped input in dA) to the dropout forward."""
    d_out, d_in, M, r = shape
    Wh, X, A, B, dY = _small_layer(30 + M, d_out, d_in, M, r)
    s, p = 16.0 / r, 0.1
    keep = orc.dropout_keep(M, d_in, p, 77, 1)
    rng = np.random.default_rng(31)
    dX, dA, dB = orc.linear_bwd(Wh, X, dY, A, B, s, keep=keep, p=p)
    VX = rng.normal(size=X.shape).astype(np.float32)
    lhs = _inner(dY, orc.linear_fwd(Wh, VX, A, B, s, keep=keep, p=p))
    assert abs(lhs - _inner(dX, VX)) <= 1e-10 * (abs(lhs) + 1)
    VA = rng.normal(size=A.shape).astype(np.float32)
    lhs = _inner(dY, orc.linear_fwd(np.zeros_like(Wh), X, VA, B, s, keep=keep, p=p))
    assert abs(lhs - _inner(dA, VA)) <= 1e-10 * (abs(lhs) + 1)
    VB = rng.normal(size=B.shape).astype(np.float32)
    lhs = _inner(dY, orc.linear_fwd(np.zeros_like(Wh), X, A, VB, s, keep=keep, p=p))
    assert abs(lhs - _inner(dB, VB)) <= 1e-10 * (abs(lhs) + 1)


# ------------------------------------------------ general block sizes [QP §5.5]

def _planted_blocks(orc, n, B1, k, seed):
    """n values in blocks of B1 (last block shorter when n % B1 != 0), each
    block a shuffle of codebook indices that contains both ends (0 and 15),
    scaled by 2^k; returns (W, planted indices)."""
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, 16, size=n).astype(np.uint8)
    for b0 in range(0, n, B1):
        blk = idx[b0:b0 + B1]
        blk[0], blk[1] = 0, 15
        rng.shuffle(blk)
    W = (orc.codebook()[idx].astype(np.float64) * 2.0 ** k).astype(np.float32)
    return W, idx


@pytest.mark.parametrize("B1,B2,n", [(32, 256, 32 * 700 + 6), (128, 16, 128 * 50 + 127),
                                     (1024, 256, 1024 * 9 + 2), (4096, 1024, 4096 * 3 + 7),
                                     (64, 64, 64 * 1000)])
def test_blocked_planted_codebook_blocks(orc, B1, B2, n):
    """Known answer at any block size, with a short last block and (odd n)
    a half-used last byte: absmax = 2^k everywhere, mean 2^k, s2 = 0 and
    FP8 code 0, the planted indices (element 2j low nibble; no element's
    nibble is 0), and restored weights RNE_bf16(c) 2^k exactly."""
    k = -5
    W, idx = _planted_blocks(orc, n, B1, k, seed=B1 + n)
    codes, scodes, s2, mean = orc.quantize_nf4_blocked(W, B1, B2)
    n1 = -(-n // B1)
    assert codes.size == (n + 1) // 2 and scodes.size == n1 and s2.size == -(-n1 // B2)
    pad = np.concatenate([idx, np.zeros(n % 2, np.uint8)])
    np.testing.assert_array_equal(codes, (pad[0::2] | (pad[1::2] << 4)).astype(np.uint8))
    assert mean == 2.0 ** k and np.all(s2 == 0) and np.all(scodes == 0)
    wh = orc.bf16_bits_to_f32(orc.dequant_bf16_blocked(codes, scodes, s2, mean, n, B1, B2))
    c_bf16 = orc.bf16_bits_to_f32(orc.bf16_rne(orc.codebook()))
    np.testing.assert_array_equal(wh, (c_bf16[idx].astype(np.float64) * 2.0 ** k).astype(np.float32))


def _block_absmax(w, B):
    n1 = -(-w.size // B)
    pad = np.zeros(n1 * B, np.float32)
    pad[:w.size] = np.abs(w)
    return pad.reshape(n1, B).max(axis=1)


def test_blocked_tail_absmax_and_nesting(orc):
    """The absmax of every block, the short last one included, is the max
    over exactly its elements (brute force), and blocks of 2B are unions of
    two blocks of B: absmax_2B[b] = max(absmax_B[2b], absmax_B[2b+1])."""
    rng = np.random.default_rng(40)
    n = 1_000_003
    w = rng.normal(0, 0.02, n).astype(np.float32)
    prev = None
    for B1 in (32, 64, 128, 256, 512, 2048):
        *_, a = orc.quantize_nf4_blocked(w, B1, 256, return_absmax=True)
        np.testing.assert_array_equal(a, _block_absmax(w, B1))
        if prev is not None and B1 == 2 * prev[0]:
            p = np.concatenate([prev[1], np.zeros(prev[1].size % 2, np.float32)])
            np.testing.assert_array_equal(a, np.maximum(p[0::2], p[1::2]))
        prev = (B1, a)


@pytest.mark.parametrize("B2", [16, 64, 1024])
def test_blocked_scale_mean_any_group(orc, B2):
    """The tree-summed mean with groups of B2 equals the exactly rounded
    mean within one FP32 rounding."""
    rng = np.random.default_rng(B2)
    for n1 in (1, B2 - 1, B2 + 1, 5 * B2 + 3, 40001):
        a = np.abs(rng.normal(0, 0.05, n1)).astype(np.float32)
        exact = math.fsum(a.astype(np.float64).tolist()) / n1
        assert abs(orc.scale_mean_g(a, B2) - exact) <= 0.5 * np.spacing(np.float32(exact)) * (1 + 1e-6)


@pytest.mark.parametrize("B1,B2", [(32, 256), (256, 64), (128, 1024)])
def test_blocked_roundtrip_error_bound(orc, B1, B2):
    """The error decomposition bound of the layer format at other block
    sizes, on a length that leaves a short last block and group."""
    rng = np.random.default_rng(41)
    n = 300_001
    w = rng.normal(0, 0.02, n).astype(np.float32)
    pos = rng.choice(n, size=n // 1000, replace=False)
    w[pos] = np.where(rng.random(pos.size) < 0.5, -0.2, 0.2).astype(np.float32)
    codes, scodes, s2, mean, absmax = orc.quantize_nf4_blocked(w, B1, B2, return_absmax=True)
    c = orc.codebook().astype(np.float64)
    idx = _unpack(codes)[:n]
    a = np.repeat(absmax.astype(np.float64), B1)[:n]
    gap = np.maximum(np.diff(c)[np.clip(idx - 1, 0, 14)], np.diff(c)[np.clip(idx, 0, 14)])
    wd = w.astype(np.float64)
    assert np.all(np.abs(wd - c[idx] * a) <= a * gap / 2 * (1 + 1e-6) + 1e-9)
    s2b = np.repeat(np.repeat(s2.astype(np.float64), B2)[: absmax.size], B1)[:n]
    ah = np.repeat([orc.restored_scale_g(scodes, s2, mean, b, B2) for b in range(absmax.size)],
                   B1)[:n].astype(np.float64)
    y = np.abs(a - mean) / np.where(s2b > 0, s2b, 1)
    half = np.where(y < 2 ** -6, 2.0 ** -10, 2.0 ** (np.floor(np.log2(np.maximum(y, 2 ** -6))) - 4))
    assert np.all(np.abs(a - ah) <= s2b * half * (1 + 1e-5) + 4 * np.spacing(np.float32(a.max())))
    wh = orc.bf16_bits_to_f32(
        orc.dequant_bf16_blocked(codes, scodes, s2, mean, n, B1, B2)).astype(np.float64)
    bound = a * gap / 2 + np.abs(c[idx]) * np.abs(a - ah) + np.abs(wh) * 2.0 ** -8 + 1e-9
    assert np.all(np.abs(wd - wh) <= bound * (1 + 1e-5))


def test_blocked_group_max_maps_to_448(orc):
    rng = np.random.default_rng(42)
    w = rng.normal(0, 0.02, 64 * 64 * 9 + 100).astype(np.float32)
    B1, B2 = 64, 64
    codes, scodes, s2, mean, absmax = orc.quantize_nf4_blocked(w, B1, B2, return_absmax=True)
    for g in range(s2.size):
        d = absmax[g * B2:(g + 1) * B2] - np.float32(mean)
        j = int(np.argmax(np.abs(d)))
        assert scodes[g * B2 + j] & 0x7F == 0x7E


def test_blocked_metadata_and_error_follow_block_size(orc):
    """[QP §5.5]: scale metadata is about 8/B1 + 32/(B1 B2) bits per weight
    (inversely proportional to B1), and smaller blocks give a lower
    quantization error on normal weights with outliers."""
    rng = np.random.default_rng(43)
    n = 64 * 4096
    w = rng.normal(0, 0.02, n).astype(np.float32)
    pos = rng.choice(n, size=n // 1000, replace=False)
    w[pos] = np.where(rng.random(pos.size) < 0.5, -0.2, 0.2).astype(np.float32)
    errs = []
    for B1 in (32, 64, 256, 1024):
        codes, scodes, s2, mean = orc.quantize_nf4_blocked(w, B1, 256)
        bits = (codes.nbytes + scodes.nbytes + s2.nbytes + 4) * 8 / n
        assert abs(bits - (4 + 8 / B1 + 32 / (B1 * 256) + 32 / n)) < 32 / n + 1e-12
        wh = orc.bf16_bits_to_f32(orc.dequant_bf16_blocked(codes, scodes, s2, mean, n, B1, 256))
        errs.append(float(np.mean(np.abs(wh.astype(np.float64) - w))))
    assert errs == sorted(errs), errs
