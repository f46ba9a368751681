"""GPU parity of the FP32 scale formats against the CPU oracle.

block_f32: the BF16 grid's shape and index with FP32 values (nemotron_mamba2.rs
listing, `set_fp8_weights`); row_f32: one FP32 scale per weight row, applied to
the finished fp32 row sum (Qwen3SsmLayer docs,
`set_fp8_rowwise_prefill_weights`). Every path is covered for each format:
the GEMV kernels (M <= 3, K > 8192, or K > 4096 below 12 rows), the skinny kernel
(4 <= M <= 16 via the GEMV entry, M <= 16 via the GEMM entry; K <= 4096, or
K <= 8192 from 12 rows on), the mid-size kernel (17 <= M <= 256; more of it in
test_gpu_mid.py), and the GEMM's 32-, 64- and 128-row tiles (K past 32768, or
M past 256) and its k-split workgroups. Bar as for the BF16
grid: |gpu - ref| <= 4e-3 * sum_k |A * Wdeq| + 1e-6 on every element, and
bit-exact where the answer is unique (an FP32 grid holding BF16 values gives
the BF16 grid's bits; a power-of-two row scale scales its column's bits).
"""
import numpy as np
import pytest
import torch

import oracle
from gemm_mamba_ssm_amd import binding, inputs

pytestmark = pytest.mark.gpu

RTOL, ATOL = 4e-3, 1e-6
FORMATS = ["block_f32", "row_f32"]


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


def scale_to_dev(S, device):
    return to_dev(S, torch.bfloat16 if S.dtype == np.uint16 else torch.float32, device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def run(fn, A, W, S, device, fmt=None):
    out = fn(to_dev(A, torch.bfloat16, device), to_dev(W, torch.uint8, device), scale_to_dev(S, device),
             scale_format=fmt)
    torch.cuda.synchronize()
    return bf16_bits(out)


def assert_within_tol(got_bits, ref, den, what):
    g = oracle.bf16_value(got_bits)
    tol = RTOL * den + ATOL
    err = np.abs(g - ref)
    bad = ~(err <= tol)
    say(f"  {what}: {err.size} elements, max err/tol {float(np.max(err / tol)) if err.size else 0.0:.4f}")
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; first {np.argwhere(bad)[:5].tolist()}"


GEMV_SHAPES = [(1, 1000, 1040), (1, 18560, 4096), (1, 4096, 8192), (3, 300, 16384), (2, 7, 16),
               (4, 1000, 1040), (8, 259, 272), (16, 18560, 4096), (9, 300, 8192), (13, 130, 3072),
               (3, 9000, 1040)]
GEMM_SHAPES = [(1, 384, 256), (16, 1000, 4096), (3, 140000, 1040), (20, 4096, 8192), (31, 300, 4112),
               (33, 1000, 1040), (40, 98400, 528), (129, 1000, 1040), (300, 257, 4096), (66, 65704, 1040),
               (65, 89603, 1040), (513, 640, 1024), (200, 12200, 1280), (20, 1000, 36880), (40, 300, 40960),
               (768, 4096, 256)]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("M,N,K", GEMV_SHAPES)
def test_gemv_every_element(dev, fmt, M, N, K):
    say(f"gemv {fmt} M={M} N={N} K={K}")
    A = inputs.activations(M, K, 1200 + M)
    W, S = inputs.weights_fmt(N, K, 0.02, 1300 + N + K, fmt)
    got = run(binding.w8a16_gemv, A, W, S, dev)
    ref, den = oracle.w8a16(A, W, S, fmt)
    assert_within_tol(got, ref, den, f"gemv {fmt} M={M} N={N} K={K}")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_every_element(dev, fmt, M, N, K):
    say(f"gemm {fmt} M={M} N={N} K={K}")
    A = inputs.activations(M, K, 1400 + M)
    W, S = inputs.weights_fmt(N, K, 0.02, 1500 + N + K, fmt)
    got = run(binding.w8a16_gemm, A, W, S, dev)
    ref, den = oracle.w8a16(A, W, S, fmt)
    assert_within_tol(got, ref, den, f"gemm {fmt} M={M} N={N} K={K}")


@pytest.mark.parametrize("fmt", FORMATS)
def test_prefill_1k_in_proj_sampled(dev, fmt):
    p = inputs.WORKLOADS["prefill_1k"][0]
    say(f"gemm {fmt} {p.name} M={p.M} N={p.N} K={p.K} (sampled)")
    A = inputs.activations(p.M, p.K, p.seed_a)
    W, S = inputs.weights_fmt(p.N, p.K, p.sigma, p.seed_w, fmt)
    got = run(binding.w8a16_gemm, A, W, S, dev)
    rng = np.random.default_rng(5)
    rows = np.array([0, 1, 517, p.M - 1])
    cols = np.array([0, 127, 128, 9000, p.N - 1])
    mi = np.concatenate([np.repeat(rows, p.N), np.repeat(np.arange(p.M), cols.size), rng.integers(0, p.M, 20000)])
    ni = np.concatenate([np.tile(np.arange(p.N), rows.size), np.tile(cols, p.M), rng.integers(0, p.N, 20000)])
    ref, den = oracle.w8a16_points(A, W, S, mi, ni, fmt)
    assert_within_tol(got[mi, ni], ref, den, f"{fmt} prefill_1k/{p.name}")


ALL_PATHS = [("gemv", 1, 1000, 1040), ("gemv", 3, 300, 8192), ("gemv", 8, 1000, 1040), ("gemm", 16, 1000, 2048),
             ("gemm", 24, 4096, 8192), ("gemm", 50, 1000, 1040), ("gemm", 200, 1000, 1040),
             ("gemm", 72, 78339, 1040), ("gemm", 256, 12288, 512),
             ("gemm", 12, 300, 6160), ("gemm", 20, 1000, 36880), ("gemm", 768, 4096, 256), ("gemm", 300, 1000, 1040)]
ENTRY = {"gemv": binding.w8a16_gemv, "gemm": binding.w8a16_gemm}


@pytest.mark.parametrize("entry,M,N,K", ALL_PATHS)
def test_f32_grid_of_bf16_values_matches_bf16_grid_bits(dev, entry, M, N, K):
    """The same scale values in either block format give the same bits."""
    say(f"{entry} f32-vs-bf16 grid M={M} N={N} K={K}")
    A = inputs.activations(M, K, 1600 + M)
    W, S = inputs.weights(N, K, 0.02, 1700 + N)
    S32 = ((S.astype(np.uint32) << 16).view(np.float32)).copy()
    a = run(ENTRY[entry], A, W, S, dev)
    b = run(ENTRY[entry], A, W, S32, dev, fmt="block_f32")
    assert np.array_equal(a, b)


@pytest.mark.parametrize("entry,M,N,K", ALL_PATHS)
def test_row_scale_power_of_two_and_locality(dev, entry, M, N, K):
    """Doubling one row scale doubles exactly that output column; halving and
    negating another does the same; every other column keeps its bits."""
    say(f"{entry} row-scale invariants M={M} N={N} K={K}")
    A = inputs.activations(M, K, 1800 + M)
    W, R = inputs.weights_fmt(N, K, 0.02, 1900 + N, "row_f32")
    base = run(ENTRY[entry], A, W, R, dev)
    R2 = R.copy()
    c1, c2 = 5, N - 2
    R2[c1] *= np.float32(2)
    R2[c2] *= np.float32(-0.5)
    got = run(ENTRY[entry], A, W, R2, dev)
    other = np.ones(N, bool)
    other[[c1, c2]] = False
    assert np.array_equal(got[:, other], base[:, other])
    v = oracle.bf16_value(base)
    g = oracle.bf16_value(got)
    assert np.array_equal(g[:, c1], 2 * v[:, c1])
    # halving may meet BF16's subnormal range only for tiny sums; none here
    assert np.array_equal(g[:, c2], -0.5 * v[:, c2])


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("entry", ["gemv", "gemm"])
def test_one_hot_rows(dev, fmt, entry):
    """A one-hot row returns its dequantized weight column, rounded, bit-exact."""
    M = 6 if entry == "gemv" else 40
    N, K = 300, 1040
    W, S = inputs.weights_fmt(N, K, 0.02, 31, fmt)
    A = np.zeros((M, K), np.uint16)
    cols = (np.arange(M) * 97 + 5) % K
    A[np.arange(M), cols] = 0x3F80
    got = run(ENTRY[entry], A, W, S, dev)
    # The one non-zero term is the E4M3 value e; the kernels scale it in fp32
    # (e * s has up to 4 + 24 significant bits, so that product is rounded
    # once to fp32) and round the result to BF16. The same two roundings,
    # taken on the exact values, give the one correct answer.
    e = oracle.dequant(W, np.ones_like(S), fmt)[:, cols].T
    s_cols = (S[None, :].repeat(M, 0) if fmt == "row_f32"
              else np.repeat(S, 128, axis=0)[:N][:, cols // 128].T)
    prod32 = (e.astype(np.float32) * s_cols.astype(np.float32)).astype(np.float64)
    want = oracle.bf16_rne(prod32)
    assert np.array_equal(oracle.bf16_value(got), oracle.bf16_value(want))


@pytest.mark.parametrize("fmt", FORMATS)
def test_misaligned_fp32_scale_refused(dev, fmt):
    W, S = inputs.weights_fmt(256, 256, 0.02, 81, fmt)
    dW = to_dev(W, torch.uint8, dev)
    raw = torch.zeros(S.size * 4 + 2, dtype=torch.uint8, device=dev)
    dA = torch.ones((2, 256), dtype=torch.bfloat16, device=dev)
    out = torch.empty((2, 256), dtype=torch.bfloat16, device=dev)
    code = binding.SCALE_FORMATS[fmt]
    for raw_fn in (binding.gemv_ex_raw, binding.gemm_ex_raw):
        st = raw_fn(dA.data_ptr(), dW.data_ptr(), raw.data_ptr() + 2, code, out.data_ptr(), 2, 256, 256, 0)
        assert st == binding.ERR_ALIGN
    torch.cuda.synchronize()
