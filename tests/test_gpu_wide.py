"""GPU parity of the 256 x 256-tile prefill GEMM (all calls through the C ABI).

The GEMM entry takes this kernel when its 256 x 256 tiles fill every round of
CU-many tiles to at least 85 %, which on a 256-CU MI355X needs about 256 or
more tiles. The shapes below are chosen for that:
  * M = 256, N = 65536, K = 64: exactly one round (256 tiles), one k-step;
  * M = 257, N = 63963, K = 144: two rounds of 250 tiles each, a one-row
    second M-tile, a ragged last N-tile (N % 4 = 3: the per-element store
    path) and a k-tail of 16 (K = 2 * 64 + 16);
  * M = 1000, N = 16300, K = 528: one round (4 x 64 tiles) with ragged M,
    ragged last N-tile, N % 4 = 0 (the 8-byte store path) and K = 8 * 64 + 16.
The weights are converted as bf16(e * s) in the kernel (one rounding of the
exact product), which the tolerance covers; where the answer is unique the
checks are bit for bit: a one-hot activation row returns bf16_rne(e * s),
zero weights give zero, 2A gives 2out (and -A gives -out up to a few last-bit
differences in a million, see the test), row permutations
permute the output, doubling one scale leaves every other column alone, and
an FP32 grid that holds BF16 values reproduces the BF16 grid's bits.
"""
import numpy as np
import pytest
import torch

import oracle
from gemm_mamba_ssm_amd import binding, inputs

pytestmark = pytest.mark.gpu

RTOL, ATOL = 4e-3, 1e-6
SHAPES = [(256, 65536, 64), (257, 63963, 144), (1000, 16300, 528)]


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    binding.load()
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dtype, device):
    raw = np.ascontiguousarray(a)
    view = raw.view(np.int16) if raw.dtype == np.uint16 else raw
    return torch.from_numpy(view.copy()).view(dtype).to(device)


def bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def gemm(A, W, S, device, fmt=None):
    sdt = torch.bfloat16 if S.dtype == np.uint16 else torch.float32
    out = binding.w8a16_gemm(to_dev(A, torch.bfloat16, device), to_dev(W, torch.uint8, device), to_dev(S, sdt, device),
                             scale_format=fmt)
    torch.cuda.synchronize()
    return bits(out)


def assert_within_tol(got_bits, ref, den, what):
    g = oracle.bf16_value(got_bits)
    tol = RTOL * den + ATOL
    err = np.abs(g - ref)
    bad = ~(err <= tol)
    say(f"  {what}: {err.size} elements, max err/tol {float(np.max(err / tol)):.4f}")
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; first {np.argwhere(bad)[:5].tolist()}"


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_wide_every_element(dev, M, N, K):
    say(f"wide gemm M={M} N={N} K={K}")
    A = inputs.activations(M, K, 1300 + M)
    W, S = inputs.weights(N, K, 0.02, 1400 + K)
    got = gemm(A, W, S, dev)
    ref, den = oracle.w8a16(A, W, S)
    assert_within_tol(got, ref, den, f"wide M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", SHAPES[1:])
def test_wide_residual_epilogue_bits(dev, M, N, K):
    say(f"wide gemm + residual M={M} N={N} K={K}")
    A = inputs.activations(M, K, 1500 + M)
    W, S = inputs.weights(N, K, 0.02, 1600 + K)
    R = inputs.activations(M, N, 1700 + N)
    dA, dW, dS = to_dev(A, torch.bfloat16, dev), to_dev(W, torch.uint8, dev), to_dev(S, torch.bfloat16, dev)
    y = binding.w8a16_gemm(dA, dW, dS)
    z = binding.w8a16_gemm_residual(dA, dW, dS, to_dev(R, torch.bfloat16, dev))
    torch.cuda.synchronize()
    want = oracle.bf16_rne(oracle.bf16_value(R) + oracle.bf16_value(bits(y)))
    assert np.array_equal(bits(z), want)


@pytest.mark.parametrize("fmt", ["block_f32", "row_f32"])
def test_wide_scale_formats(dev, fmt):
    M, N, K = SHAPES[1]
    say(f"wide gemm {fmt} M={M} N={N} K={K}")
    A = inputs.activations(M, K, 1800)
    W, S = inputs.weights_fmt(N, K, 0.02, 1900, fmt)
    got = gemm(A, W, S, dev, fmt)
    ref, den = oracle.w8a16(A, W, S, fmt=fmt)
    assert_within_tol(got, ref, den, f"wide {fmt}")


def test_wide_f32_grid_of_bf16_values_gives_bf16_bits(dev):
    M, N, K = SHAPES[2]
    A = inputs.activations(M, K, 2000)
    W, S = inputs.weights(N, K, 0.02, 2100)
    S32 = oracle.bf16_value(S).astype(np.float32)
    assert np.array_equal(gemm(A, W, S32, dev, "block_f32"), gemm(A, W, S, dev))


def test_wide_one_hot_rows(dev):
    M, N, K = 256, 65536, 1040
    W, S = inputs.weights(N, K, 0.02, 2200)
    A = np.zeros((M, K), np.uint16)
    cols = (np.arange(M) * 97 + 5) % K
    A[np.arange(M), cols] = 0x3F80
    got = gemm(A, W, S, dev)
    want = oracle.bf16_rne(oracle.dequant(W, S)[:, cols].T)
    # unique up to the sign of zero (a -0 weight times +1 may sum to +0)
    assert np.array_equal(oracle.bf16_value(got), oracle.bf16_value(want))


def test_wide_zero_weights(dev):
    M, N, K = SHAPES[0]
    A = inputs.activations(M, K, 2300)
    W, S = inputs.weights(N, K, 0.02, 2400)
    got = gemm(A, np.zeros_like(W), S, dev)
    assert np.all((got & 0x7FFF) == 0)


def test_wide_sign_scaling_permutation_and_determinism(dev):
    M, N, K = SHAPES[1]
    A = inputs.activations(M, K, 2500)
    W, S = inputs.weights(N, K, 0.02, 2600)
    base = gemm(A, W, S, dev)
    assert np.array_equal(gemm(A, W, S, dev), base), "not deterministic"
    # -A: the matrix cores' fp32 accumulation is not exactly sign-symmetric
    # in its last bit (measured on MI355X: 6 to 9 of 16.7 million outputs
    # differ, all near-cancellations of magnitude ~1e-4 and within 2 BF16
    # ulp), so the negation is checked as: all but a few in a million outputs
    # negate bit for bit, and the rest are within 2 ulp (each is within the
    # tolerance by the every-element test).
    neg = gemm(A ^ np.uint16(0x8000), W, S, dev)
    diff = oracle.bf16_value(neg) != -oracle.bf16_value(base)
    assert diff.sum() <= 1e-5 * diff.size, f"{int(diff.sum())} outputs do not negate"
    ulps = np.abs((neg.astype(np.int32) & 0x7FFF) - (base.astype(np.int32) & 0x7FFF))[diff]
    assert np.all(ulps <= 2), ulps.max()
    A2 = np.where((A & 0x7FFF) == 0, A, A + np.uint16(0x80))      # A * 2 exactly
    assert np.array_equal(oracle.bf16_value(gemm(A2, W, S, dev)), 2 * oracle.bf16_value(base))
    perm = np.random.default_rng(5).permutation(M)               # every row sums over the whole K alike
    assert np.array_equal(gemm(A[perm], W, S, dev), base[perm])


def test_wide_scale_doubling_touches_only_its_block(dev):
    M, N, K = SHAPES[2]
    A = inputs.activations(M, K, 2700)
    W, S = inputs.weights(N, K, 0.02, 2800)
    base = gemm(A, W, S, dev)
    S2 = S.copy()
    S2[77, 2] += 0x80                                            # x2 exactly
    got = gemm(A, W, S2, dev)
    cols = np.zeros(N, bool)
    cols[77 * 128:78 * 128] = True
    assert np.array_equal(got[:, ~cols], base[:, ~cols])
    ref, den = oracle.w8a16(A, W, S2)
    assert_within_tol(got, ref, den, "scale x2")


# Columns split between the two tile families: when 256 x 256 tiles cover
# at least one whole round of CU-many tiles but the rest is less than 85 %
# of a round, whole rounds of them take the first columns (a multiple of
# 256) and the 128-row tiles the remaining ones, written at their column
# offset with the full row stride. M = 1000, N = 18000, K = 1040: 4 x 71
# tiles of 256 x 256; the first 4 x 64 take columns 0..16383, and 8 x 13
# tiles of 128 x 128 (a ragged last one: 1616 = 12 * 128 + 80) the rest
# (K is not a multiple of 256, so whole tiles; with a workspace they split).
# M = 1024, N = 18560, K = 4096 (the 1024-token in_proj; every element in
# test_gpu_parity.py) takes the k-split workgroups for its 8 x 17 rest.
SPLIT_N = (1000, 18000, 1040)


@pytest.mark.parametrize("fmt", [None, "block_f32", "row_f32"])
def test_wide_split_columns_every_element(dev, fmt):
    M, N, K = SPLIT_N
    say(f"wide + 128-row tiles {fmt or 'block_bf16'} M={M} N={N} K={K}")
    A = inputs.activations(M, K, 3100)
    if fmt is None:
        W, S = inputs.weights(N, K, 0.02, 3200)
    else:
        W, S = inputs.weights_fmt(N, K, 0.02, 3200, fmt)
    got = gemm(A, W, S, dev, fmt)
    ref, den = oracle.w8a16(A, W, S, fmt=fmt or "block_bf16")
    assert_within_tol(got, ref, den, f"split columns {fmt}")


def test_wide_split_columns_residual_and_workspace(dev):
    M, N, K = SPLIT_N
    A = inputs.activations(M, K, 3300)
    W, S = inputs.weights(N, K, 0.02, 3400)
    R = inputs.activations(M, N, 3500)
    dA, dW, dS = to_dev(A, torch.bfloat16, dev), to_dev(W, torch.uint8, dev), to_dev(S, torch.bfloat16, dev)
    y = binding.w8a16_gemm(dA, dW, dS)
    z = binding.w8a16_gemm_residual(dA, dW, dS, to_dev(R, torch.bfloat16, dev))
    ws = binding.gemm_workspace(M, N, K, dev)
    assert ws is not None
    yw = binding.w8a16_gemm_ws(dA, dW, dS, ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits(z), oracle.bf16_rne(oracle.bf16_value(R) + oracle.bf16_value(bits(y))))
    ref, den = oracle.w8a16(A, W, S)
    assert_within_tol(bits(yw), ref, den, "split columns, tail tiles split through the workspace")
    # the 256 x 256 part is the same kernel either way: its columns are bit-identical
    assert np.array_equal(bits(yw)[:, :16384], bits(y)[:, :16384])


# Long K on the 256 x 256 tiles: K = 16400 holds 129 k-blocks, so the tile's
# scale row spans three of the four per-lane scale registers, and the k-tail
# is 16. M = 1000, N = 16384: one round of 4 x 64 tiles. Checked on a whole
# row in every 128-row block and a whole column in every 128-column block.
def test_wide_long_k_every_tile(dev):
    M, N, K = 1000, 16384, 16400
    say(f"wide gemm long K M={M} N={N} K={K}")
    A = inputs.activations(M, K, 3600)
    W, S = inputs.weights(N, K, 0.02, 3700)
    got = gemm(A, W, S, dev)
    rows = np.unique(np.r_[np.arange(0, M, 128) + 37, M - 1].clip(0, M - 1))
    cols = np.unique(np.r_[np.arange(0, N, 128) + 91, N - 1].clip(0, N - 1))
    ref, den = oracle.w8a16(A[rows], W, S)
    assert_within_tol(got[rows], ref, den, f"long K: {rows.size} whole rows")
    mi = np.repeat(np.arange(M), cols.size)
    ni = np.tile(cols, M)
    ref, den = oracle.w8a16_points(A, W, S, mi, ni)
    assert_within_tol(got[mi, ni], ref, den, f"long K: {cols.size} whole columns")
