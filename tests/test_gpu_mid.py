"""GPU parity of the mid-size GEMM kernel (17..256 rows of A, K <= 32768):
one workgroup of 8 waves per small output tile, A and W staged through LDS by
DMA, K split across waves within each stage. All calls through the C ABI
(w8a16_gemm and its variants), every element against the oracle.

The host picks the tile from M, N, K and the CU count; on a 256-CU MI355X
the shapes below reach every tile (rows x columns) of the kernel:
  * 16 x 32: M = 17 with N = 130 and K = 144 (ragged M, N and K), M = 33 with
    N = 7 and K = 64 (fewer columns than a block, K below one stage), M = 20
    on the Mamba-2 out_proj;
  * 16 x 64: M = 129 with N = 1000 and K = 1040 (a K tail of 16), the
    out_proj at M = 64, K = 32768 (the largest K this kernel takes);
  * 32 x 64: the out_proj at M = 128, M = 30 with K = 4112;
  * 64 x 64: the out_proj at M = 256, M = 240 with N = 3100 and K = 1552;
  * 32 x 80: the in_proj at M = 32, M = 20 with K = 2064;
  * 64 x 80: the in_proj at M = 64, M = 250 with N = 5000 and K = 3008;
  * 64 x 160: the in_proj at M = 128, M = 40 with N = 98400 (three rounds of
    tiles over the CUs);
  * 128 x 160: the in_proj at M = 256, M = 66 with N = 65704 (two rounds),
    M = 130 with K = 128 (one stage).
"""
import numpy as np
import pytest
import torch

import oracle
from gemm_mamba_ssm_amd import binding, inputs

pytestmark = pytest.mark.gpu

RTOL, ATOL = 4e-3, 1e-6

SHAPES = [(17, 130, 144), (33, 7, 64), (20, 4096, 8192),
          (129, 1000, 1040), (64, 4096, 8192), (100, 2000, 32768),
          (128, 4096, 8192), (30, 9000, 4112),
          (256, 4096, 8192), (240, 3100, 1552),
          (32, 18560, 4096), (20, 18560, 2064),
          (64, 18560, 4096), (250, 5000, 3008),
          (128, 18560, 4096), (40, 98400, 528),
          (256, 18560, 4096), (66, 65704, 1040), (130, 18560, 128)]


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


def bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def assert_within_tol(got_bits, ref, den, what):
    g = oracle.bf16_value(got_bits)
    tol = RTOL * den + ATOL
    err = np.abs(g - ref)
    bad = ~(err <= tol)
    say(f"  {what}: {err.size} elements, max err/tol {float(np.max(err / tol)):.4f}")
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; first {np.argwhere(bad)[:5].tolist()}"


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_mid_every_element(dev, M, N, K):
    say(f"mid-size gemm M={M} N={N} K={K}")
    A = inputs.activations(M, K, 6100 + M)
    W, S = inputs.weights(N, K, 0.02, 6200 + N + K)
    out = binding.w8a16_gemm(to_dev(A, torch.bfloat16, dev), to_dev(W, torch.uint8, dev),
                             to_dev(S, torch.bfloat16, dev))
    got = bits(out)
    again = bits(binding.w8a16_gemm(to_dev(A, torch.bfloat16, dev), to_dev(W, torch.uint8, dev),
                                    to_dev(S, torch.bfloat16, dev)))
    assert np.array_equal(got, again), "not deterministic"
    ref, den = oracle.w8a16(A, W, S)
    assert_within_tol(got, ref, den, f"M={M} N={N} K={K}")


# Edges: K = 16 (one stage, one k-chunk), N = 1, the largest K at the fewest
# and the most rows, every dimension ragged.
EDGE_SHAPES = [(20, 50, 16), (256, 1, 32768), (17, 16, 32768), (255, 129, 4112), (200, 3, 48)]


@pytest.mark.parametrize("M,N,K", EDGE_SHAPES)
def test_mid_edges_every_element(dev, M, N, K):
    say(f"mid-size gemm edge M={M} N={N} K={K}")
    A = inputs.activations(M, K, 7100 + M)
    W, S = inputs.weights(N, K, 0.02, 7200 + N + K)
    out = binding.w8a16_gemm(to_dev(A, torch.bfloat16, dev), to_dev(W, torch.uint8, dev),
                             to_dev(S, torch.bfloat16, dev))
    ref, den = oracle.w8a16(A, W, S)
    assert_within_tol(bits(out), ref, den, f"M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(129, 1000, 1040), (64, 4096, 8192)])
def test_mid_scale_grid_at_two_byte_offset(dev, M, N, K):
    """A BF16 scale grid that starts 2 bytes past a 4-byte boundary (a view at
    an odd element offset): the kernel copies the grid rows as aligned dwords,
    so the bits must equal those from an aligned copy of the same grid."""
    say(f"mid-size gemm, scale grid at offset 2, M={M} N={N} K={K}")
    A = inputs.activations(M, K, 7300 + M)
    W, S = inputs.weights(N, K, 0.02, 7400 + K)
    dA, dW, dS = to_dev(A, torch.bfloat16, dev), to_dev(W, torch.uint8, dev), to_dev(S, torch.bfloat16, dev)
    store = torch.zeros(dS.numel() + 1, dtype=torch.bfloat16, device=dev)
    shifted = store[1:].view(dS.shape)
    shifted.copy_(dS)
    assert shifted.data_ptr() % 4 == 2
    aligned = bits(binding.w8a16_gemm(dA, dW, dS))
    odd = bits(binding.w8a16_gemm(dA, dW, shifted))
    assert np.array_equal(aligned, odd)
    ref, den = oracle.w8a16(A, W, S)
    assert_within_tol(odd, ref, den, f"offset grid M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(17, 130, 144), (128, 4096, 8192), (64, 18560, 4096), (66, 65704, 1040)])
def test_mid_residual_epilogue_bits(dev, M, N, K):
    """out = bf16(residual + y) exactly, y = the same GEMM without the residual."""
    say(f"mid-size gemm + residual M={M} N={N} K={K}")
    A = inputs.activations(M, K, 6300 + M)
    W, S = inputs.weights(N, K, 0.02, 6400 + K)
    R = inputs.activations(M, N, 6500 + N)
    dA, dW, dS = to_dev(A, torch.bfloat16, dev), to_dev(W, torch.uint8, dev), to_dev(S, torch.bfloat16, dev)
    y = binding.w8a16_gemm(dA, dW, dS)
    z = binding.w8a16_gemm_residual(dA, dW, dS, to_dev(R, torch.bfloat16, dev))
    torch.cuda.synchronize()
    assert np.array_equal(bits(z), oracle.bf16_rne(oracle.bf16_value(R) + oracle.bf16_value(bits(y))))


@pytest.mark.parametrize("fmt", ["block_f32", "row_f32"])
@pytest.mark.parametrize("M,N,K", [(17, 130, 144), (100, 2000, 32768), (256, 4096, 8192), (128, 18560, 4096),
                                   (40, 98400, 528)])
def test_mid_scale_formats(dev, fmt, M, N, K):
    say(f"mid-size gemm {fmt} M={M} N={N} K={K}")
    A = inputs.activations(M, K, 6600 + M)
    W, S = inputs.weights_fmt(N, K, 0.02, 6700 + K, fmt)
    out = binding.w8a16_gemm(to_dev(A, torch.bfloat16, dev), to_dev(W, torch.uint8, dev), scale_to_dev(S, dev),
                             scale_format=fmt)
    ref, den = oracle.w8a16(A, W, S, fmt=fmt)
    assert_within_tol(bits(out), ref, den, f"{fmt} M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(20, 18560, 8192), (48, 18560, 2048), (128, 4096, 8192), (256, 4096, 8192),
                                   (17, 140000, 1040)])
def test_mid_needs_no_workspace(dev, M, N, K):
    """These shapes took the split schedule before the mid-size kernel; now
    they need no workspace, and the workspace entry gives the plain entry's
    bits (with a workspace given or not)."""
    assert binding.gemm_workspace_size(M, N, K) == 0
    A = inputs.activations(M, K, 6800 + M)
    W, S = inputs.weights(N, K, 0.02, 6900 + N)
    dA, dW, dS = to_dev(A, torch.bfloat16, dev), to_dev(W, torch.uint8, dev), to_dev(S, torch.bfloat16, dev)
    plain = bits(binding.w8a16_gemm(dA, dW, dS))
    spare = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    st = binding.gemm_ws_raw(dA.data_ptr(), dW.data_ptr(), dS.data_ptr(), out.data_ptr(), M, N, K,
                             spare.data_ptr(), spare.numel(), torch.cuda.current_stream(dev).cuda_stream)
    assert st == binding.OK, binding.strerror(st)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), plain)
