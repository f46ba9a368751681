"""GPU check of w8a16_gemm_noalloc, the GEMM entry point that allocates
nothing: its split schedule's partial tiles go to the library's static
scratch array instead of a caller's workspace. Called through the C ABI, it
must give the same bits as w8a16_gemm_ws with a workspace of
w8a16_gemm_workspace_size bytes (the same kernels and schedule), on two calls
in a row, the second on a smaller shape (the scratch then holds the first
call's partial tiles), and stay within the oracle's tolerance."""
import numpy as np
import pytest
import torch

import oracle
from gemm_mamba_ssm_amd import binding, inputs

pytestmark = pytest.mark.gpu

RTOL, ATOL = 4e-3, 1e-6


def say(*a):
    print(*a, flush=True)


def to_dev(a: np.ndarray, dtype, device):
    raw = np.ascontiguousarray(a)
    view = raw.view(np.int16) if raw.dtype == np.uint16 else raw
    return torch.from_numpy(view.copy()).view(dtype).to(device)


def bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def operands(M, N, K, seed, device):
    A = inputs.activations(M, K, seed)
    W, S = inputs.weights(N, K, 0.02, seed + 1)
    return (A, W, S), (to_dev(A, torch.bfloat16, device), to_dev(W, torch.uint8, device),
                       to_dev(S, torch.bfloat16, device))


def run_noalloc(dA, dW, dS, M, N, K, stream):
    out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dA.device)
    st = binding.gemm_noalloc_raw(dA.data_ptr(), dW.data_ptr(), dS.data_ptr(), out.data_ptr(), M, N, K, stream)
    assert st == binding.OK, binding.strerror(st)
    return out


def run_ws(dA, dW, dS, M, N, K, stream):
    need = binding.gemm_workspace_size(M, N, K)
    assert need > 0, "the shape is meant to take the split schedule"
    ws = torch.empty(need, dtype=torch.uint8, device=dA.device)
    out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dA.device)
    st = binding.gemm_ws_raw(dA.data_ptr(), dW.data_ptr(), dS.data_ptr(), out.data_ptr(), M, N, K,
                             ws.data_ptr(), need, stream)
    assert st == binding.OK, binding.strerror(st)
    return out, ws


# First a shape whose split needs the whole 64 MiB (384 tokens through the
# Mamba-2 in_proj), then a smaller one with a ragged tile in M, N and K.
SHAPES = [(384, 18560, 4096), (300, 1000, 1040)]


def test_noalloc_matches_the_workspace_entry_on_two_calls_in_a_row():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    binding.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev).cuda_stream
    assert binding.gemm_workspace_size(*SHAPES[0]) == binding.gemm_noalloc_scratch_bytes()
    for i, (M, N, K) in enumerate(SHAPES):
        say(f"w8a16_gemm_noalloc call {i + 1}: M={M} N={N} K={K}")
        host, (dA, dW, dS) = operands(M, N, K, 7100 + 10 * i, dev)
        got = run_noalloc(dA, dW, dS, M, N, K, stream)
        want, ws = run_ws(dA, dW, dS, M, N, K, stream)
        torch.cuda.synchronize()
        g, w = bits(got), bits(want)
        assert np.array_equal(g, w), f"{int((g != w).sum())} of {g.size} outputs differ from w8a16_gemm_ws"
        # rows in every 128-row tile against the oracle (the whole output on the small shape)
        rows = np.arange(M) if M * N <= 200000 else np.unique(np.r_[np.arange(0, M, 41), M - 1])
        ref, den = oracle.w8a16(host[0][rows], host[1], host[2])
        err = np.abs(oracle.bf16_value(g[rows]) - ref)
        tol = RTOL * den + ATOL
        say(f"  {rows.size} rows x {N}: max err/tol {float(np.max(err / tol)):.4f}")
        assert np.all(err <= tol)
        del ws
