"""HIP-graph capture of one Mamba-2 layer decode step, every kernel from this
library: in_proj with its RMSNorm fused, the conv1d update, the SSM decode,
out_proj with the gated RMSNorm and the residual fused (z and dt read in place
from the in_proj output).

No kernel here allocates or clears memory, so the four launches can be
captured. The graph is replayed several times, with eager work and
synchronizations between the replays; before each replay the states are
restored from a saved copy, and every replay's outputs and updated states
must equal the eager run's bit for bit.
"""
import numpy as np
import pytest
import torch

from gemm_mamba_ssm_amd import binding, inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    binding.load()
    return torch.device("cuda:0")


def bf(a: np.ndarray, device):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16).copy()).view(torch.bfloat16).to(device)


def u8(a: np.ndarray, device):
    return torch.from_numpy(np.ascontiguousarray(a).copy()).to(device)


@pytest.mark.parametrize("M", [1, 2])
def test_layer_decode_step_graph_replays_match_eager(dev, M):
    H, P, S_, G, DC = 16, 64, 128, 2, 4                  # a narrow layer of the same structure
    d_inner = H * P
    d_xbc = d_inner + 2 * G * S_
    hidden = 1024
    n_in = d_inner + d_xbc + H
    eps = inputs.NORM_EPS
    W_in, S_in = inputs.weights(n_in, hidden, 0.02, 9101)
    W_out, S_out = inputs.weights(hidden, d_inner, 0.02, 9102)
    dW_in, dS_in, dW_out, dS_out = u8(W_in, dev), bf(S_in, dev), u8(W_out, dev), bf(S_out, dev)
    w_in = bf(inputs.norm_weight(hidden, 9103), dev)
    w_out = bf(inputs.norm_weight(d_inner, 9104), dev)
    cw, cb = (bf(a, dev) for a in inputs.conv_params(d_xbc, DC, 9105))
    a_log, d_param, dt_bias = (torch.from_numpy(a).to(dev) for a in inputs.ssm_params(H, 9106))
    x = bf(inputs.activations(M, hidden, 9107), dev)
    conv0 = torch.from_numpy(inputs.conv_state(M, d_xbc, DC, 9108)).to(dev)
    ssm0 = torch.from_numpy(inputs.ssm_state(M, H, P, S_, 9109)).to(dev)
    conv_state, ssm_state = conv0.clone(), ssm0.clone()
    proj = torch.empty((M, n_in), dtype=torch.bfloat16, device=dev)
    xbc = torch.empty((M, d_xbc), dtype=torch.bfloat16, device=dev)
    y = torch.empty((M, d_inner), dtype=torch.bfloat16, device=dev)
    out = torch.empty((M, hidden), dtype=torch.bfloat16, device=dev)

    def step():
        binding.w8a16_gemv_fused(x, dW_in, dS_in, norm_weight=w_in, eps=eps, out=proj)
        binding.w8a16_conv1d_update(conv_state, proj[:, d_inner:d_inner + d_xbc], cw, cb, out=xbc)
        binding.w8a16_ssm_decode(ssm_state, xbc, proj[:, d_inner + d_xbc:], a_log, d_param, dt_bias, G, out=y)
        binding.w8a16_gemv_fused(y, dW_out, dS_out, norm_weight=w_out, eps=eps, gate=proj[:, :d_inner],
                                 residual=x, out=out)

    def restore():
        conv_state.copy_(conv0)
        ssm_state.copy_(ssm0)

    step()                                             # eager reference
    torch.cuda.synchronize()
    ref = [t.clone() for t in (proj, xbc, y, out, conv_state, ssm_state)]
    assert torch.isfinite(out.float()).all()

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):                      # warm-up on the capture stream, outside capture
        restore()
        step()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(4):
        for t in (proj, xbc, y, out):                  # eager work between replays
            t.fill_(7.0)
        restore()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (proj, xbc, y, out, conv_state, ssm_state)
        for name, g, r in zip(("proj", "xbc", "y", "out", "conv_state", "ssm_state"), got, ref):
            assert torch.equal(g.view(torch.int16) if g.dtype == torch.bfloat16 else g.view(torch.int32),
                               r.view(torch.int16) if r.dtype == torch.bfloat16 else r.view(torch.int32)), \
                f"replay {rep}: {name} differs from the eager run"


# GEMM shapes of every tile schedule: whole 128 x 128 tiles (24 of them; with
# a workspace, split), the k-split inside the workgroup (256 tiles), the
# 256 x 256 tiles (one round of 256), the skinny kernel's one-shot form (two
# activation phases of 128 KB of dynamic LDS), 32-row tiles past the
# mid-size kernel's K (split with a workspace), and the mid-size kernel.
CAPTURE_SHAPES = [(300, 1000, 1040), (1024, 4096, 512), (512, 32768, 64), (16, 4096, 8192), (20, 4100, 40960),
                  (20, 18560, 8192), (129, 1000, 1040), (256, 4096, 8192)]
SPLIT_WITH_WORKSPACE = {(300, 1000, 1040), (20, 4100, 40960)}


@pytest.mark.parametrize("M,N,K", CAPTURE_SHAPES)
@pytest.mark.parametrize("with_workspace", [False, True])
def test_gemm_captured_as_first_call_on_a_fresh_stream(dev, M, N, K, with_workspace):
    """The GEMM allocates nothing, so its first call on a new stream can be
    inside a capture; with a caller workspace the split tiles' partial sums
    and the second (combine) kernel are captured too. Every replay, with eager
    work between replays, equals the eager result bit for bit."""
    A = bf(inputs.activations(M, K, 9200 + M), dev)
    W, S = inputs.weights(N, K, 0.02, 9300 + N)
    dW, dS = u8(W, dev), bf(S, dev)
    ws = binding.gemm_workspace(M, N, K, dev) if with_workspace else None
    if with_workspace:
        assert (ws is not None) == ((M, N, K) in SPLIT_WITH_WORKSPACE), "the schedule this shape is meant to take"
    ref = binding.w8a16_gemm_ws(A, dW, dS, ws) if with_workspace else binding.w8a16_gemm(A, dW, dS)
    torch.cuda.synchronize()
    out = torch.empty_like(ref)
    fresh = torch.cuda.Stream(device=dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=fresh):
        if with_workspace:
            binding.w8a16_gemm_ws(A, dW, dS, ws, out=out)
        else:
            binding.w8a16_gemm(A, dW, dS, out=out)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(3.0)                                 # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {rep} differs"
