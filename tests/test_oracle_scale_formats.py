"""Pins of the oracle's FP32 scale formats (block grid and per-row).

The block_f32 format has the BF16 grid's shape and index with FP32 values
(nemotron_mamba2.rs listing, `set_fp8_weights`); row_f32 holds one FP32 scale
per weight row (Qwen3SsmLayer docs, `set_fp8_rowwise_prefill_weights`). Each
is pinned by exact rational sums on tiny shapes, by reduction to the already
pinned BF16 block format where the values allow it, by a library fp64 matmul,
and by the invariants a scale must satisfy (which outputs it may touch, exact
power-of-two scaling). A scale read at the wrong index (k-block for a row
scale, n-block for the wrong row, a transposed grid) fails one of them.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from gemm_mamba_ssm_amd import inputs


def torch_decode(W):
    return torch.from_numpy(np.array(W, copy=True)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_bf16(bits):
    return torch.from_numpy(np.array(bits, copy=True).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def independent_dequant(W, S, fmt):
    """E4M3 via torch; block scales expanded with np.repeat, row scales broadcast."""
    N, K = W.shape
    if fmt == "row_f32":
        return torch_decode(W) * S.astype(np.float64)[:, None]
    s = S.astype(np.float64)
    return torch_decode(W) * np.repeat(np.repeat(s, 128, axis=0), 128, axis=1)[:N, :K]


def odd_scales(shape, seed):
    """FP32 scales with full 24-bit mantissas (not BF16-representable)."""
    rng = np.random.default_rng(seed)
    s = (2.0 ** rng.integers(-9, -3, shape)) * (1 + rng.random(shape))
    s = s.astype(np.float32)
    s.flat[0] = np.float32(0.1)                  # a classic inexact value
    return s


FMT_SHAPES = [(m, n, k) for m in (1, 3) for n in (128, 200) for k in (144, 256)]


@pytest.mark.parametrize("fmt", ["block_f32", "row_f32"])
@pytest.mark.parametrize("M,N,K", FMT_SHAPES)
def test_bruteforce_exact_rational(fmt, M, N, K):
    A = inputs.activations(M, K, seed=M + N + K)
    W, _ = inputs.weights(N, K, 0.02, seed=N * K)
    S = odd_scales((N,) if fmt == "row_f32" else inputs.scale_grid(N, K), seed=M * N)
    ref, den = oracle.w8a16(A, W, S, fmt)
    a = [[Fraction(float(x)) for x in row] for row in torch_bf16(A)]
    e = torch_decode(W)
    for m in range(M):
        for n in range(N):
            if fmt == "row_f32":
                s_of = [Fraction(float(S[n]))] * K
            else:
                s_of = [Fraction(float(S[n // 128, k // 128])) for k in range(K)]
            terms = [a[m][k] * Fraction(float(e[n, k])) * s_of[k] for k in range(K)]
            exact = sum(terms, Fraction(0))
            mag = sum((abs(t) for t in terms), Fraction(0))
            assert abs(Fraction(ref[m, n]) - exact) <= Fraction(1, 10 ** 12) * mag, (m, n)
            assert abs(Fraction(den[m, n]) - mag) <= Fraction(1, 10 ** 12) * mag, (m, n)


def test_f32_grid_with_bf16_values_equals_bf16_grid():
    A = inputs.activations(5, 400, seed=21)
    W, S = inputs.weights(300, 400, 0.02, seed=22)
    S32 = torch_bf16(S).astype(np.float32)           # the same values, stored as FP32
    r0, d0 = oracle.w8a16(A, W, S)
    r1, d1 = oracle.w8a16(A, W, S32, "block_f32")
    assert np.array_equal(r0, r1) and np.array_equal(d0, d1)
    assert np.array_equal(oracle.dequant(W, S), oracle.dequant(W, S32, "block_f32"))


def test_row_scales_constant_per_band_equal_block_grid():
    N, K = 300, 400
    nb, kb = inputs.scale_grid(N, K)
    band = np.array([0.0078125, 0.01171875, 0.375], np.float32)   # BF16-representable
    R = np.repeat(band, 128)[:N]
    S = torch.from_numpy(np.repeat(band[:, None], kb, axis=1)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    A = inputs.activations(4, K, seed=23)
    W, _ = inputs.weights(N, K, 0.02, seed=24)
    r0, d0 = oracle.w8a16(A, W, S)
    r1, d1 = oracle.w8a16(A, W, R, "row_f32")
    assert np.array_equal(r0, r1) and np.array_equal(d0, d1)


@pytest.mark.parametrize("fmt", ["block_f32", "row_f32"])
def test_dequant_distinct_scales_index(fmt):
    N, K = 300, 400
    rng = np.random.default_rng(3)
    W = rng.integers(0, 256, (N, K)).astype(np.uint8)
    W[(W & 0x7F) == 0x7F] = 0x38
    if fmt == "row_f32":
        S = np.array([2.0 ** (n % 8) * (1 + n / 1024) for n in range(N)], np.float32)
        assert len(set(S.tolist())) == N
    else:
        nb, kb = inputs.scale_grid(N, K)
        S = np.array([[2.0 ** (i % 8) * (1 + j / 1024 + i / 7) for j in range(kb)] for i in range(nb)], np.float32)
        assert len(set(S.ravel().tolist())) == nb * kb
    got = oracle.dequant(W, S, fmt)
    assert np.array_equal(got, independent_dequant(W, S, fmt))
    for n, k in [(0, 0), (127, 127), (128, 127), (127, 128), (299, 399), (256, 384), (5, 390)]:
        e = float(torch_decode(W[n:n + 1, k:k + 1])[0, 0])
        s = float(S[n]) if fmt == "row_f32" else float(S[n // 128, k // 128])
        assert got[n, k] == e * s


@pytest.mark.parametrize("fmt", ["block_f32", "row_f32"])
@pytest.mark.parametrize("M,N,K", [(5, 300, 1040), (16, 1000, 640)])
def test_matches_library_fp64_matmul(fmt, M, N, K):
    A = inputs.activations(M, K, seed=M + N)
    W, S = inputs.weights_fmt(N, K, 0.02, M + K, fmt)
    ref, den = oracle.w8a16(A, W, S, fmt)
    a = torch_bf16(A)
    wd = independent_dequant(W, S, fmt)
    assert np.all(np.abs(ref - a @ wd.T) <= 1e-12 * (np.abs(a) @ np.abs(wd).T) + 1e-300)
    assert np.allclose(den, np.abs(a) @ np.abs(wd).T, rtol=1e-12, atol=0)


def test_row_scale_touches_only_its_column():
    A = inputs.activations(3, 272, seed=31)
    W, R = inputs.weights_fmt(200, 272, 0.02, 32, "row_f32")
    ref, den = oracle.w8a16(A, W, R, "row_f32")
    R2 = R.copy()
    R2[77] *= np.float32(2)                          # exact
    R2[150] *= np.float32(-0.5)                      # exact
    ref2, _ = oracle.w8a16(A, W, R2, "row_f32")
    other = np.ones(200, bool)
    other[[77, 150]] = False
    assert np.array_equal(ref2[:, other], ref[:, other])
    assert np.array_equal(ref2[:, 77], 2 * ref[:, 77])
    assert np.array_equal(ref2[:, 150], -0.5 * ref[:, 150])


def test_block_f32_scale_touches_only_its_block():
    M, N, K = 3, 300, 400
    A = inputs.activations(M, K, seed=41)
    W, S = inputs.weights_fmt(N, K, 0.02, 42, "block_f32")
    ref, den = oracle.w8a16(A, W, S, "block_f32")
    S2 = S.copy()
    S2[2, 1] *= np.float32(4)
    ref2, _ = oracle.w8a16(A, W, S2, "block_f32")
    cols = slice(256, 300)
    assert np.array_equal(ref2[:, :256], ref[:, :256])
    a = torch_bf16(A)
    wd = independent_dequant(W, S, "block_f32")
    block = a[:, 128:256] @ wd[cols, 128:256].T
    assert np.all(np.abs((ref2[:, cols] - ref[:, cols]) - 3 * block) <= 1e-12 * 8 * den[:, cols])


def test_points_match_full_formats():
    A = inputs.activations(7, 272, seed=51)
    for fmt in ("block_f32", "row_f32"):
        W, S = inputs.weights_fmt(333, 272, 0.02, 52, fmt)
        ref, den = oracle.w8a16(A, W, S, fmt)
        rng = np.random.default_rng(1)
        mi, ni = rng.integers(0, 7, 300), rng.integers(0, 333, 300)
        r, d = oracle.w8a16_points(A, W, S, mi, ni, fmt)
        assert np.array_equal(r, ref[mi, ni]) and np.array_equal(d, den[mi, ni])


def test_scale_format_contract():
    A = inputs.activations(2, 256, seed=4)
    W, S = inputs.weights(200, 256, 0.02, 5)
    grid32 = torch_bf16(S).astype(np.float32)
    row32 = np.ones(200, np.float32)
    with pytest.raises(ValueError):
        oracle.w8a16(A, W, row32, "block_f32")       # per-row vector as a grid
    with pytest.raises(ValueError):
        oracle.w8a16(A, W, grid32, "row_f32")        # grid as a per-row vector
    with pytest.raises(ValueError):
        oracle.w8a16(A, W, row32[:199], "row_f32")
    with pytest.raises(TypeError):
        oracle.w8a16(A, W, S, "block_f32")           # BF16 bits as FP32
    with pytest.raises(TypeError):
        oracle.w8a16(A, W, grid32, "block_bf16")
    with pytest.raises(ValueError):
        oracle.w8a16(A, W, S, "tensor_f32")


@pytest.mark.parametrize("fmt", ["block_f32", "row_f32"])
def test_quantizer_round_trip(fmt):
    """The generators' codes times their scales reproduce the draws to E4M3 precision."""
    N, K = 260, 300
    W, S = inputs.weights_fmt(N, K, 0.02, 61, fmt)
    rng = np.random.default_rng(61)
    w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    wd = independent_dequant(W, S, fmt)
    # half an E4M3 ulp of the value, or half the subnormal quantum 2^-9 (code
    # 0x08 is 2^-6), in units of the scale; a little slack for w / s in fp32
    half_sub = 2.0 ** -4 * independent_dequant(np.full_like(W, 0x08), S, fmt)
    assert np.all(np.abs(wd - w) <= 1.0001 * (2.0 ** -4 * np.abs(w) + half_sub))
    codes = torch_decode(W)
    if fmt == "row_f32":
        assert np.all(np.abs(codes).max(axis=1) == 448)
    else:
        assert np.abs(codes[:128, :128]).max() == 448
