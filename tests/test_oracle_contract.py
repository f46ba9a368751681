"""Pins of the oracle's block-scaled contraction.

The oracle's sum is checked against exact rational sums (brute force on tiny
shapes), a library fp64 matmul fed by torch's independent E4M3 decode, a
hand-worked golden example, and the invariants any bilinear block-scaled
product must satisfy. A dropped term, a wrong sign, a wrong scale index or a
transposed operand in the oracle fails at least one of these.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from gemm_mamba_ssm_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_decode(W):
    return torch.from_numpy(np.array(W, copy=True)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_bf16(bits):
    return torch.from_numpy(np.array(bits, copy=True).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def independent_dequant(W, S):
    """E4M3 via torch, scales expanded with np.repeat over 128x128 blocks."""
    N, K = W.shape
    s = torch_bf16(S)
    s_full = np.repeat(np.repeat(s, 128, axis=0), 128, axis=1)[:N, :K]
    return torch_decode(W) * s_full


def rand_operands(M, N, K, seed, sigma=0.02):
    A = inputs.activations(M, K, seed)
    Wq, S = inputs.weights(N, K, sigma, seed + 1)
    return A, Wq, S


def test_worked_example_golden():
    M, N, K = 2, 130, 256
    A = np.zeros((M, K), np.uint16)
    W = np.zeros((N, K), np.uint8)
    A[0, 0], A[0, 1], A[0, 128], A[0, 255] = 0x3F80, 0x4000, 0xBF00, 0x4040
    A[1, 1], A[1, 200] = 0x3F80, 0x4080
    W[0, 0], W[0, 1], W[0, 128], W[0, 255] = 0x38, 0x40, 0xB8, 0x01
    W[129, 1], W[129, 200] = 0x7E, 0x09
    S = np.array([[0x3F00, 0x4000], [0x3E80, 0x3C00]], np.uint16)
    ref, den = oracle.w8a16(A, W, S)
    n_checked = 0
    with open(os.path.join(GOLDEN, "worked_example.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            m, n, r, d = line.split()
            assert ref[int(m), int(n)] == float(r), (m, n)
            assert den[int(m), int(n)] == float(d), (m, n)
            n_checked += 1
    assert n_checked == 6


TINY_SHAPES = [(1, 384, 256)] + [(m, n, k) for m in (1, 2, 3) for n in (128, 200, 256) for k in (128, 144, 256)]


@pytest.mark.parametrize("M,N,K", TINY_SHAPES)
def test_bruteforce_exact_rational(M, N, K):
    A, W, S = rand_operands(M, N, K, seed=100 + M * 7 + N + K)
    # salt in extreme codes so subnormals, +-448 and -0 take part
    rng = np.random.default_rng(N * K)
    W = W.copy()
    idx = rng.integers(0, W.size, 40)
    W.flat[idx] = rng.choice(np.array([0x01, 0x07, 0x08, 0x7E, 0xFE, 0x80, 0x81], np.uint8), 40)
    ref, den = oracle.w8a16(A, W, S)
    a = [[Fraction(float(x)) for x in row] for row in torch_bf16(A)]
    wd = [[Fraction(float(x)) for x in row] for row in independent_dequant(W, S)]
    for m in range(M):
        for n in range(N):
            terms = [a[m][k] * wd[n][k] for k in range(K)]
            exact = sum(terms, Fraction(0))
            mag = sum((abs(t) for t in terms), Fraction(0))
            assert abs(Fraction(ref[m, n]) - exact) <= Fraction(1, 10 ** 12) * mag, (m, n)
            assert abs(Fraction(den[m, n]) - mag) <= Fraction(1, 10 ** 12) * mag, (m, n)


def test_tiny_workload_bruteforce():
    (p,) = inputs.WORKLOADS["tiny_gemv"]
    A, W, S = inputs.make(p)
    ref, den = oracle.w8a16(A, W, S)
    a = [Fraction(float(x)) for x in torch_bf16(A)[0]]
    wd = independent_dequant(W, S)
    for n in range(p.N):
        exact = sum((a[k] * Fraction(float(wd[n, k])) for k in range(p.K)), Fraction(0))
        assert abs(Fraction(ref[0, n]) - exact) <= Fraction(1, 10 ** 12) * Fraction(den[0, n])


@pytest.mark.parametrize("M,N,K", [(5, 300, 1040), (16, 1000, 640), (64, 257, 272)])
def test_matches_library_fp64_matmul(M, N, K):
    A, W, S = rand_operands(M, N, K, seed=M + N + K)
    ref, den = oracle.w8a16(A, W, S)
    a = torch_bf16(A)
    wd = independent_dequant(W, S)
    lib = a @ wd.T
    libden = np.abs(a) @ np.abs(wd).T
    assert np.all(np.abs(ref - lib) <= 1e-12 * libden + 1e-300)
    assert np.allclose(den, libden, rtol=1e-12, atol=0)


def test_dequant_distinct_scales_index():
    N, K = 300, 400                      # grid 3 x 4, ragged in both dims
    nb, kb = inputs.scale_grid(N, K)
    s_vals = np.array([[2.0 ** (i % 8) * (1 + j / 128) for j in range(kb)] for i in range(nb)], np.float32)
    S = torch.from_numpy(s_vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert len(set(S.ravel().tolist())) == nb * kb
    rng = np.random.default_rng(3)
    W = rng.integers(0, 256, (N, K)).astype(np.uint8)
    W[(W & 0x7F) == 0x7F] = 0x38
    got = oracle.dequant(W, S)
    want = independent_dequant(W, S)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))
    # spot-check the index by hand: element (n, k) -> S[n // 128, k // 128]
    for n, k in [(0, 0), (127, 127), (128, 127), (127, 128), (299, 399), (256, 384)]:
        e = float(torch_decode(W[n:n + 1, k:k + 1])[0, 0])
        assert got[n, k] == e * float(s_vals[n // 128, k // 128])


def test_points_match_full():
    A, W, S = rand_operands(7, 333, 272, seed=9)
    ref, den = oracle.w8a16(A, W, S)
    rng = np.random.default_rng(1)
    mi = rng.integers(0, 7, 500)
    ni = rng.integers(0, 333, 500)
    r, d = oracle.w8a16_points(A, W, S, mi, ni)
    assert np.array_equal(r, ref[mi, ni])
    assert np.array_equal(d, den[mi, ni])
    with pytest.raises(IndexError):
        oracle.w8a16_points(A, W, S, [7], [0])


def test_shape_contract():
    A, W, S = rand_operands(2, 200, 256, seed=4)
    with pytest.raises(ValueError):
        oracle.w8a16(A, W, S[:, :1])             # per-row-like truncated grid
    with pytest.raises(ValueError):
        oracle.w8a16(A, W, np.zeros((200,), np.uint16))   # per-row [N] scale
    with pytest.raises(ValueError):
        oracle.w8a16(A[:, :128], W, S)
    with pytest.raises(TypeError):
        oracle.w8a16(A.astype(np.float32), W, S)


# --- invariants of the block-scaled bilinear product -------------------------

def test_zero_weights_give_exact_zero():
    A, W, S = rand_operands(3, 260, 384, seed=5)
    ref, den = oracle.w8a16(A, np.zeros_like(W), S)
    assert np.all(ref == 0) and np.all(den == 0)


def test_one_hot_row_returns_dequantized_column():
    M, N, K = 4, 300, 400
    A, W, S = rand_operands(M, N, K, seed=6)
    A = np.zeros_like(A)
    cols = [0, 131, 255, 399]
    for m, j in enumerate(cols):
        A[m, j] = 0x3F80                    # 1.0
    ref, _ = oracle.w8a16(A, W, S)
    wd = independent_dequant(W, S)
    for m, j in enumerate(cols):
        assert np.array_equal(ref[m], wd[:, j])


def test_scale_doubling_changes_only_that_block():
    M, N, K = 3, 300, 400
    A, W, S = rand_operands(M, N, K, seed=8)
    ref, den = oracle.w8a16(A, W, S)
    S2 = S.copy()
    nb, kbk = 1, 2
    S2[nb, kbk] += 0x80                     # +1 in the BF16 exponent: exactly x2
    assert torch_bf16(S2[nb:nb + 1, kbk:kbk + 1])[0, 0] == 2 * torch_bf16(S[nb:nb + 1, kbk:kbk + 1])[0, 0]
    ref2, _ = oracle.w8a16(A, W, S2)
    cols = slice(nb * 128, min(N, nb * 128 + 128))
    other = np.ones(N, bool)
    other[cols] = False
    assert np.array_equal(ref2[:, other], ref[:, other])
    a = torch_bf16(A)
    wd = independent_dequant(W, S)
    ks = slice(kbk * 128, min(K, kbk * 128 + 128))
    block = a[:, ks] @ wd[cols, ks].T
    assert np.all(np.abs((ref2[:, cols] - ref[:, cols]) - block) <= 1e-12 * den[:, cols] * 2)


def test_sign_and_power_of_two_scaling_are_exact():
    A, W, S = rand_operands(4, 256, 512, seed=10)
    ref, _ = oracle.w8a16(A, W, S)
    neg, _ = oracle.w8a16(A ^ np.uint16(0x8000), W, S)
    assert np.array_equal(neg, -ref)
    dbl, _ = oracle.w8a16(A + np.uint16(0x80), W, S)   # every A value doubled (no overflow here)
    assert np.array_equal(dbl, 2 * ref)
    wneg, _ = oracle.w8a16(A, W ^ np.uint8(0x80), S)
    assert np.array_equal(wneg, -ref)


def test_row_permutation():
    A, W, S = rand_operands(6, 200, 256, seed=12)
    ref, _ = oracle.w8a16(A, W, S)
    perm = np.array([3, 0, 5, 1, 4, 2])
    got, _ = oracle.w8a16(A[perm], W, S)
    assert np.array_equal(got, ref[perm])
