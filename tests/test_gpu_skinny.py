"""GPU parity of the one-shot skinny form (one 16-row weight block per
workgroup, every weight load issued up front, the activations in LDS), all
calls through the C ABI.

The host takes this form for 1 <= M <= 16 when the activations, padded to the
waves' k-blocks, fit 128 KB of LDS and, with more 16-row weight blocks than
CUs, 32 KB; the GEMV entry from M = 2 on, the GEMM entry for every M. The
shapes below are chosen for that (on a 256-CU MI355X):
  * M = 2, N = 4100, K = 4096: 257 blocks (more than the CUs), 16 KB of
    activations, a ragged last block (N % 16 = 4);
  * M = 3, N = 129, K = 4112: 8 k-blocks per wave, a k-tail of 16, 9 blocks;
  * M = 8, N = 4096, K = 8192: 128 KB of activations (the Mamba-2 out_proj);
  * M = 5, N = 1000, K = 1040: 2 k-blocks per wave, a ragged k-block;
  * M = 4, N = 18560, K = 4096: the Mamba-2 in_proj, 1160 blocks;
  * M = 1 through the GEMM entry; M = 16 with a short K;
  * activations in two phases of half of K (more than 128 KB of them with
    every weight block on a CU of its own, or more than 32 KB with more
    blocks than CUs): M = 16, N = 4096, K = 8192 (the Mamba-2 out_proj), M = 9
    with a ragged N, M = 16 with a k-tail of 16, M = 8 with 257 blocks.
From 17 rows on the GEMM entry takes the mid-size kernel (test_gpu_mid.py).
"""
import numpy as np
import pytest
import torch

import oracle
from gemm_mamba_ssm_amd import binding, inputs

pytestmark = pytest.mark.gpu

RTOL, ATOL = 4e-3, 1e-6
SHAPES = [(2, 4100, 4096), (3, 129, 4112), (8, 4096, 8192), (5, 1000, 1040), (4, 18560, 4096), (1, 4096, 8192),
          (16, 300, 2048), (16, 4096, 8192), (9, 300, 8192), (16, 129, 4112), (8, 4100, 4096)]


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


def assert_within_tol(got_bits, ref, den, what):
    g = oracle.bf16_value(got_bits)
    tol = RTOL * den + ATOL
    err = np.abs(g - ref)
    bad = ~(err <= tol)
    say(f"  {what}: {err.size} elements, max err/tol {float(np.max(err / tol)):.4f}")
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; first {np.argwhere(bad)[:5].tolist()}"


def run(entry, A, W, S, device, fmt=None):
    sdt = torch.bfloat16 if S.dtype == np.uint16 else torch.float32
    fn = binding.w8a16_gemv if entry == "gemv" else binding.w8a16_gemm
    out = fn(to_dev(A, torch.bfloat16, device), to_dev(W, torch.uint8, device), to_dev(S, sdt, device),
             scale_format=fmt)
    torch.cuda.synchronize()
    return bits(out)


# The GEMV entry keeps the VALU GEMV at M = 1 and takes at most 16 rows, so
# those shapes run through the GEMM entry only.
@pytest.mark.parametrize("entry,M,N,K", [(e, *s) for e in ("gemv", "gemm") for s in SHAPES
                                         if e == "gemm" or 1 < s[0] <= 16])
def test_one_shot_every_element(dev, entry, M, N, K):
    say(f"one-shot skinny via {entry} M={M} N={N} K={K}")
    A = inputs.activations(M, K, 4100 + M)
    W, S = inputs.weights(N, K, 0.02, 4200 + N + K)
    got = run(entry, A, W, S, dev)
    ref, den = oracle.w8a16(A, W, S)
    assert_within_tol(got, ref, den, f"{entry} M={M} N={N} K={K}")


def test_one_shot_matches_between_entries(dev):
    M, N, K = SHAPES[0]
    A = inputs.activations(M, K, 4300)
    W, S = inputs.weights(N, K, 0.02, 4400)
    assert np.array_equal(run("gemv", A, W, S, dev), run("gemm", A, W, S, dev))


@pytest.mark.parametrize("M,N,K", [(2, 4100, 4096), (6, 4096, 8192), (12, 4096, 8192), (16, 4096, 8192)])
def test_one_shot_residual_epilogue_bits(dev, M, N, K):
    say(f"one-shot skinny + residual M={M} N={N} K={K}")
    A = inputs.activations(M, K, 4500 + M)
    W, S = inputs.weights(N, K, 0.02, 4600 + K)
    R = inputs.activations(M, N, 4700 + N)
    dA, dW, dS = to_dev(A, torch.bfloat16, dev), to_dev(W, torch.uint8, dev), to_dev(S, torch.bfloat16, dev)
    y = binding.w8a16_gemm(dA, dW, dS)
    z = binding.w8a16_gemm_residual(dA, dW, dS, to_dev(R, torch.bfloat16, dev))
    torch.cuda.synchronize()
    assert np.array_equal(bits(z), oracle.bf16_rne(oracle.bf16_value(R) + oracle.bf16_value(bits(y))))


@pytest.mark.parametrize("fmt", ["block_f32", "row_f32"])
@pytest.mark.parametrize("M,N,K", [(3, 129, 4112), (6, 4096, 8192), (14, 300, 8192), (16, 300, 8192)])
def test_one_shot_scale_formats(dev, fmt, M, N, K):
    say(f"one-shot skinny {fmt} M={M} N={N} K={K}")
    A = inputs.activations(M, K, 4800 + M)
    W, S = inputs.weights_fmt(N, K, 0.02, 4900 + K, fmt)
    for entry in ("gemv", "gemm") if M <= 16 else ("gemm",):
        got = run(entry, A, W, S, dev, fmt)
        ref, den = oracle.w8a16(A, W, S, fmt=fmt)
        assert_within_tol(got, ref, den, f"{entry} {fmt}")


def test_one_shot_invariants(dev):
    M, N, K = 8, 4096, 8192
    W, S = inputs.weights(N, K, 0.02, 5000)
    # one-hot rows return the rounded dequantized weight column, exactly
    A1 = np.zeros((M, K), np.uint16)
    cols = (np.arange(M) * 997 + 11) % K
    A1[np.arange(M), cols] = 0x3F80
    got = run("gemv", A1, W, S, dev)
    want = oracle.bf16_rne(oracle.dequant(W, S)[:, cols].T)
    assert np.array_equal(oracle.bf16_value(got), oracle.bf16_value(want))
    # zero weights give zero; -A, 2A and row permutations are exact; deterministic
    A = inputs.activations(M, K, 5100)
    assert np.all((run("gemv", A, np.zeros_like(W), S, dev) & 0x7FFF) == 0)
    base = run("gemv", A, W, S, dev)
    assert np.array_equal(run("gemv", A, W, S, dev), base)
    # -A: the matrix cores' fp32 accumulation is not exactly sign-symmetric in
    # its last bit (a few outputs in ten million, near-cancellations within
    # 2 BF16 ulp); all but such outputs negate bit for bit
    neg = run("gemv", A ^ np.uint16(0x8000), W, S, dev)
    diff = oracle.bf16_value(neg) != -oracle.bf16_value(base)
    assert diff.sum() <= max(1, 1e-5 * diff.size), f"{int(diff.sum())} outputs do not negate"
    ulps = np.abs((neg.astype(np.int32) & 0x7FFF) - (base.astype(np.int32) & 0x7FFF))[diff]
    assert np.all(ulps <= 2)
    A2 = np.where((A & 0x7FFF) == 0, A, A + np.uint16(0x80))
    assert np.array_equal(oracle.bf16_value(run("gemv", A2, W, S, dev)), 2 * oracle.bf16_value(base))
    perm = np.random.default_rng(9).permutation(M)
    assert np.array_equal(run("gemv", A[perm], W, S, dev), base[perm])
    # doubling one scale block changes its 128 columns only
    S2 = S.copy()
    S2[5, 17] += 0x80
    got = run("gemv", A, W, S2, dev)
    c = np.zeros(N, bool)
    c[5 * 128:6 * 128] = True
    assert np.array_equal(got[:, ~c], base[:, ~c])
