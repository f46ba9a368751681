"""GPU parity of the Mamba-2 decode step (conv1d update, SSM decode; the
forward steps 3 to 5 of the nemotron_mamba2.rs module docs) against the CPU
oracle, over several tokens so that the carried states are checked too.

* conv1d update: the FP32 conv state holds copies of BF16 inputs, so it must
  match the oracle bit for bit after every token; each output within one
  BF16 step of the oracle's rounding of the exact value (fp32 arithmetic
  against fp64), at most 1 % of them off.
* SSM decode: the FP32 state against the fp64 oracle with a relative bound
  that grows with the tokens (1e-5 of |h| before and after each update,
  summed over the tokens: the kernel rounds every operation to fp32 and its
  exp / softplus are within a few ulp); each output within one BF16 step of
  its value plus 1e-4 of sum_n |C h| + |D x|.
* An SSM step with dt = 0 leaves the state bit-identical.
* in_proj with the conv epilogue (w8a16_gemv_in_proj): the conv state comes
  out shifted bit for bit with the projection's output as its newest entry
  (within the product tolerance of the oracle), the other columns within that
  tolerance too, the conv outputs within the oracle's chain's value plus one
  output rounding and the effect of a one-step difference in the conv input;
  and, where it groups rows like w8a16_gemv_fused, bit for bit the result of
  the two launches it replaces.
"""
import numpy as np
import pytest
import torch

import oracle
from gemm_mamba_ssm_amd import binding, inputs

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    binding.load()
    return torch.device("cuda:0")


def bf(a: np.ndarray, device):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16).copy()).view(torch.bfloat16).to(device)


def f32(a: np.ndarray, device):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32).copy()).to(device)


def bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def check_step_bits(got, want, what):
    g, w = got.astype(np.int32), want.astype(np.int32)
    same_sign = (g & 0x8000) == (w & 0x8000)
    zero = ((g & 0x7FFF) == 0) & ((w & 0x7FFF) == 0)
    ok = zero | (same_sign & (np.abs((g & 0x7FFF) - (w & 0x7FFF)) <= 1))
    frac = float(np.mean(g != w))
    say(f"  {what}: {g.size} values, {frac * 100:.3f} % one step off")
    assert ok.all(), f"{what}: {int((~ok).sum())} values more than one BF16 step off"
    assert frac <= 0.01, f"{what}: {frac * 100:.2f} % differ"


# --- conv1d update ----------------------------------------------------------------

@pytest.mark.parametrize("B,dim,d_conv,ld_x", [(1, 10240, 4, 18560), (3, 37, 4, 40), (2, 300, 2, 300),
                                               (1, 513, 3, 600), (4, 64, 8, 64), (2, 257, 1, 300)])
def test_conv1d_update_tokens(dev, B, dim, d_conv, ld_x):
    say(f"conv1d B={B} dim={dim} d_conv={d_conv} ld_x={ld_x}")
    w, bias = inputs.conv_params(dim, d_conv, 7000 + dim)
    s0 = inputs.conv_state(B, dim, d_conv, 7100 + dim)
    ref_state = s0.astype(np.float64)
    d_state = f32(s0, dev)
    dw, db = bf(w, dev), bf(bias, dev)
    for t in range(5):
        row = inputs.activations(B, ld_x, 7200 + t)
        x_dev = bf(row, dev)[:, 8 if ld_x - dim >= 8 else 0:]             # a column slice of a wider row
        off = 8 if ld_x - dim >= 8 else 0
        got = binding.w8a16_conv1d_update(d_state, x_dev, dw, db)
        torch.cuda.synchronize()
        _, want = oracle.conv1d_update(ref_state, np.ascontiguousarray(row[:, off:]), w, bias)
        check_step_bits(bits(got), want, f"conv t={t}")
        assert np.array_equal(d_state.cpu().numpy().astype(np.float64), ref_state), f"state differs after t={t}"


# --- SSM decode -----------------------------------------------------------------

SSM_SHAPES = [  # (B, heads, head_dim, state, groups)
    (1, 128, 64, 128, 8),       # the hidden-4096 layer
    (2, 128, 64, 128, 8),
    (1, 6, 5, 12, 3),           # ragged rows per workgroup, 3 of 32 lanes per row busy
    (2, 4, 8, 256, 2),          # two chunks per lane
    (1, 8, 9, 160, 1),          # partial second chunk
    (3, 16, 16, 64, 16),
]


@pytest.mark.parametrize("B,heads,hd,st,groups", SSM_SHAPES)
def test_ssm_decode_tokens(dev, B, heads, hd, st, groups):
    say(f"ssm B={B} heads={heads} head_dim={hd} state={st} groups={groups}")
    a_log, d_param, dt_bias = inputs.ssm_params(heads, 8000 + heads)
    h0 = inputs.ssm_state(B, heads, hd, st, 8100 + st)
    ref = h0.astype(np.float64)
    d_h = f32(h0, dev)
    da, dd, dbias = f32(a_log, dev), f32(d_param, dev), f32(dt_bias, dev)
    width = heads * hd + 2 * groups * st
    acc_tol = np.zeros_like(ref)
    for t in range(4):
        row = inputs.activations(B, width + 3, 8200 + t)                # rows with a little slack (ld_xbc)
        dt_row = inputs.activations(B, heads + 5, 8300 + t)
        prev = ref.copy()
        y_ref, y_bits, den = oracle.ssm_decode(ref, row, dt_row, a_log, d_param, dt_bias, groups)
        got = binding.w8a16_ssm_decode(d_h, bf(row, dev), bf(dt_row, dev), da, dd, dbias, groups)
        torch.cuda.synchronize()
        acc_tol += 1e-5 * (np.abs(prev) + np.abs(ref))
        h_gpu = d_h.cpu().numpy().astype(np.float64)
        err = np.abs(h_gpu - ref)
        say(f"  t={t}: state max err/tol {float(np.max(err / (acc_tol + 1e-30))):.4f}")
        assert np.all(err <= acc_tol + 1e-30), f"state outside tolerance at t={t}"
        y = oracle.bf16_value(bits(got))
        tol = 2.0 ** -8 * np.abs(y_ref) + 1e-4 * den + 1e-30
        yerr = np.abs(y - y_ref)
        say(f"  t={t}: y max err/tol {float(np.max(yerr / tol)):.4f}")
        assert np.all(yerr <= tol), f"outputs outside tolerance at t={t}"


def test_ssm_zero_dt_keeps_state_bits(dev):
    B, heads, hd, st, groups = 1, 8, 8, 64, 2
    a_log, d_param, dt_bias = inputs.ssm_params(heads, 8401)
    h0 = inputs.ssm_state(B, heads, hd, st, 8402)
    d_h = f32(h0, dev)
    row = inputs.activations(B, heads * hd + 2 * groups * st, 8403)
    dt_row = np.full((B, heads), 0xC2C8, np.uint16)                     # -100: softplus underflows to 0
    binding.w8a16_ssm_decode(d_h, bf(row, dev), bf(dt_row, dev), f32(a_log, dev), f32(d_param, dev),
                             f32(dt_bias, dev), groups, dt_min=0.0)
    torch.cuda.synchronize()
    assert np.array_equal(d_h.cpu().numpy().view(np.uint32), h0.view(np.uint32))


def test_mamba2_rejections_on_device(dev):
    h = torch.zeros((1, 4, 2, 6), dtype=torch.float32, device=dev)
    xbc = torch.zeros((1, 64), dtype=torch.bfloat16, device=dev)
    dt = torch.zeros((1, 4), dtype=torch.bfloat16, device=dev)
    p = torch.zeros(4, dtype=torch.float32, device=dev)
    out = torch.empty((1, 8), dtype=torch.bfloat16, device=dev)
    st = binding.ssm_decode_raw(h.data_ptr(), xbc.data_ptr(), 64, dt.data_ptr(), 4, p.data_ptr(), p.data_ptr(),
                                p.data_ptr(), out.data_ptr(), 8, 1, 4, 2, 6, 2, 0.0, 1e9, 0)
    assert st == binding.ERR_SHAPE                                       # state 6 is not a multiple of 4
    with pytest.raises(ValueError):
        binding.w8a16_ssm_decode(h, xbc, dt, p, p, p, groups=3)
    torch.cuda.synchronize()


# --- in_proj with the RMSNorm prologue and the conv1d epilogue (one launch) --------------------

def _in_proj_case(M, hidden, d_inner, d_xbc, heads, d_conv, seed):
    n_in = d_inner + d_xbc + heads
    x = inputs.activations(M, hidden, seed)
    nw = inputs.norm_weight(hidden, seed + 1)
    W, S = inputs.weights(n_in, hidden, 0.02, seed + 2)
    cw, cb = inputs.conv_params(d_xbc, d_conv, seed + 3)
    st = inputs.conv_state(M, d_xbc, d_conv, seed + 4)
    return n_in, x, nw, W, S, cw, cb, st


IN_PROJ_SHAPES = [  # (M, hidden, d_inner, d_xbc, heads, d_conv)
    (1, 4096, 8192, 10240, 128, 4),     # the hidden-4096 layer
    (2, 4096, 8192, 10240, 128, 4),
    (3, 1024, 1024, 1536, 16, 3),
    (4, 16384, 512, 768, 8, 4),         # two chunks per lane
    (4, 1024, 1024, 1536, 16, 4),       # halved row groups for the conv epilogue
    (8, 2048, 512, 640, 8, 2),
    (2, 1024, 1024, 1536, 16, 6),       # d_conv > 4: the taps one by one
]


@pytest.mark.parametrize("M,hidden,d_inner,d_xbc,heads,d_conv", IN_PROJ_SHAPES)
def test_gemv_in_proj_conv_epilogue(dev, M, hidden, d_inner, d_xbc, heads, d_conv):
    say(f"gemv_in_proj M={M} hidden={hidden} xBC={d_xbc} d_conv={d_conv}")
    eps = inputs.NORM_EPS
    n_in, x, nw, W, S, cw, cb, st0 = _in_proj_case(M, hidden, d_inner, d_xbc, heads, d_conv, 9500 + M)
    dx, dnw, dW, dS, dcw, dcb = bf(x, dev), bf(nw, dev), torch.from_numpy(W).to(dev), bf(S, dev), bf(cw, dev), bf(cb, dev)
    d_state = f32(st0, dev)
    got = bits(binding.w8a16_gemv_in_proj(dx, dW, dS, dnw, eps, d_state, dcw, dcb, d_inner))
    new_state = d_state.cpu().numpy()
    torch.cuda.synchronize()
    conv_cols = slice(d_inner, d_inner + d_xbc)
    # the state: shifted bit for bit, and its newest entry is the projection's output
    assert np.array_equal(new_state[:, :, :-1].view(np.uint32), st0[:, :, 1:].view(np.uint32))
    _, a = oracle.rmsnorm(x, nw, eps)
    ref, den = oracle.w8a16(a, W, S)
    new_in = new_state[:, :, -1].astype(np.float64)
    err = np.abs(new_in - ref[:, conv_cols])
    assert np.all(err <= 4e-3 * den[:, conv_cols] + 1e-6), "conv input (the projection) outside tolerance"
    g = oracle.bf16_value(got)
    other = np.ones(n_in, bool)
    other[conv_cols] = False
    assert np.all(np.abs(g[:, other] - ref[:, other]) <= 4e-3 * den[:, other] + 1e-6), "z / dt outside tolerance"
    # the conv outputs against the oracle's own chain (its projection, rounded to BF16, as the conv input).
    # The kernel's input may be one BF16 step (2^-7 relative at most) from the oracle's where the product
    # lies near a rounding midpoint; silu' < 1.1, so that moves the output by at most 1.1 |w_last| 2^-7 |x|,
    # on top of the output's own rounding (2^-8 relative).
    ex, want = oracle.conv1d_update(st0.astype(np.float64), oracle.bf16_rne(ref[:, conv_cols]), cw, cb)
    x_ref = oracle.bf16_value(oracle.bf16_rne(ref[:, conv_cols]))
    w_last = np.abs(oracle.bf16_value(cw[:, -1]))[None, :]
    tol = 2.0 ** -8 * np.abs(ex) + 1.1 * w_last * 2.0 ** -7 * np.abs(x_ref) + 1e-30
    cerr = np.abs(oracle.bf16_value(got[:, conv_cols]) - ex)
    say(f"  in_proj conv M={M}: max err/tol {float(np.max(cerr / tol)):.4f}, "
        f"{float(np.mean(got[:, conv_cols] != want)) * 100:.3f} % of outputs differ from the oracle's rounding")
    assert np.all(cerr <= tol), "conv outputs outside tolerance"
    # same row groups as the fused GEMV (M <= 3, or two chunks per lane): bit-identical to the two launches
    if M <= 3 or hidden > 8192:
        proj = binding.w8a16_gemv_fused(dx, dW, dS, norm_weight=dnw, eps=eps)
        d2 = f32(st0, dev)
        conv = binding.w8a16_conv1d_update(d2, proj[:, conv_cols], dcw, dcb)
        torch.cuda.synchronize()
        chain = bits(proj)
        chain[:, conv_cols] = bits(conv)
        assert np.array_equal(got, chain)
        assert np.array_equal(d2.cpu().numpy().view(np.uint32), new_state.view(np.uint32))
