"""Pins of the oracle's norm prologues and residual epilogue.

The layer's forward steps (nemotron_mamba2.rs module docs) put an RMS norm
scaled by its weight before in_proj (step 1), the gated norm
rms_norm(y, ssm_norm) * silu(z) before out_proj (step 6) and a residual add
after out_proj (step 8). The oracle's fp64 norm is checked against torch's own
RMSNorm and SiLU in float64, against closed forms (constant rows, a zero gate,
a zero weight) and against the invariants of a norm (scale invariance at
eps = 0, row independence); the residual add against exact sums.
"""
import numpy as np
import pytest
import torch

import oracle
from gemm_mamba_ssm_amd import inputs


def bf16_to_f64(bits):
    return torch.from_numpy(np.array(bits, copy=True).view(np.int16)).view(torch.bfloat16).to(torch.float64)


@pytest.mark.parametrize("M,K", [(1, 4096), (3, 8192), (5, 272), (2, 16)])
@pytest.mark.parametrize("gated", [False, True])
def test_matches_torch_float64(M, K, gated):
    x = inputs.activations(M, K, 11 + K)
    w = inputs.norm_weight(K, 12 + K)
    z = inputs.activations(M, K, 13 + K) if gated else None
    eps = inputs.NORM_EPS
    exact, bits = oracle.rmsnorm(x, w, eps, gate=z)
    xt, wt = bf16_to_f64(x), bf16_to_f64(w)
    want = torch.nn.functional.rms_norm(xt, (K,), weight=wt, eps=eps)
    if gated:
        want = want * torch.nn.functional.silu(bf16_to_f64(z))
    want = want.numpy()
    assert np.all(np.abs(exact - want) <= 1e-13 * np.abs(want) + 1e-300)
    assert np.array_equal(bits, oracle.bf16_rne(exact))


@pytest.mark.parametrize("M,K,G", [(2, 8192, 1024), (3, 4096, 2048), (1, 16384, 1024), (4, 2048, 2048),
                                   (2, 272, 16)])
@pytest.mark.parametrize("gated", [False, True])
def test_grouped_matches_torch_float64(M, K, G, gated):
    """The grouped norm is torch's RMSNorm over each group of G channels (the
    row reshaped to [K / G, G]), then the per-channel weight (and gate)."""
    x = inputs.activations(M, K, 21 + K + G)
    w = inputs.norm_weight(K, 22 + K)
    z = inputs.activations(M, K, 23 + K) if gated else None
    eps = inputs.NORM_EPS
    exact, bits = oracle.rmsnorm(x, w, eps, gate=z, group=G)
    xt = bf16_to_f64(x).reshape(M, K // G, G)
    want = torch.nn.functional.rms_norm(xt, (G,), eps=eps).reshape(M, K) * bf16_to_f64(w)
    if gated:
        want = want * torch.nn.functional.silu(bf16_to_f64(z))
    want = want.numpy()
    assert np.all(np.abs(exact - want) <= 1e-13 * np.abs(want) + 1e-300)
    assert np.array_equal(bits, oracle.bf16_rne(exact))


def test_grouped_norm_whole_row_and_group_independence():
    """group = K is the whole-row norm, bit for bit; each group is normalized
    on its own: at eps = 0 scaling one group of x by a power of two changes
    no output, and changing another group's values leaves a group's outputs
    as they were."""
    M, K, G = 3, 4096, 1024
    x = inputs.activations(M, K, 31)
    w = inputs.norm_weight(K, 32)
    z = inputs.activations(M, K, 33)
    e_row, b_row = oracle.rmsnorm(x, w, 1e-5, gate=z)
    e_k, b_k = oracle.rmsnorm(x, w, 1e-5, gate=z, group=K)
    assert np.array_equal(b_row, b_k) and np.array_equal(e_row, e_k)
    e0, _ = oracle.rmsnorm(x, w, 0.0, gate=z, group=G)
    xs = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16)
    xs[:, G:2 * G] *= 4.0                                  # exact in BF16
    x2 = xs.view(torch.int16).numpy().view(np.uint16)
    e1, _ = oracle.rmsnorm(x2, w, 0.0, gate=z, group=G)
    assert np.array_equal(e0, e1)
    x3 = x.copy()
    x3[:, 3 * G:] = inputs.activations(M, G, 34)
    e3, _ = oracle.rmsnorm(x3, w, 1e-5, gate=z, group=G)
    e4, _ = oracle.rmsnorm(x, w, 1e-5, gate=z, group=G)
    assert np.array_equal(e3[:, :3 * G], e4[:, :3 * G])
    assert not np.array_equal(e_row, e4)                   # the grouping matters


def test_silu_matches_torch_and_identities():
    z = np.concatenate([np.linspace(-30, 30, 2001), [0.0, 1e-8, -1e-8, 80.0, -80.0]])
    got = np.array([oracle.silu(v) for v in z])
    want = torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    assert np.all(np.abs(got - want) <= 1e-15 * np.abs(want) + 1e-300)
    assert oracle.silu(0.0) == 0.0
    # silu(z) - silu(-z) = z (sigmoid(z) + sigmoid(-z) = 1)
    for v in (0.5, 3.0, 7.25):
        assert abs((oracle.silu(v) - oracle.silu(-v)) - v) <= 1e-15 * v


def test_constant_rows_closed_form():
    K = 256
    vals = np.array([1.0, 0.25, -2.0, 64.0, -0.125], np.float32)
    x = torch.from_numpy(np.repeat(vals[:, None], K, axis=1)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    w = np.full(K, 0x3F80, np.uint16)                      # 1.0
    exact, bits = oracle.rmsnorm(x, w, 0.0)
    # a power-of-two constant c normalizes to sign(c) exactly
    assert np.array_equal(exact, np.sign(vals.astype(np.float64))[:, None].repeat(K, 1))
    eps = 0.5
    exact, _ = oracle.rmsnorm(x, w, eps)
    c = vals.astype(np.float64)[:, None]
    assert np.allclose(exact, c / np.sqrt(c * c + eps), rtol=1e-15, atol=0)


def test_zero_gate_and_zero_weight_give_zero():
    M, K = 2, 512
    x = inputs.activations(M, K, 21)
    w = inputs.norm_weight(K, 22)
    _, bits = oracle.rmsnorm(x, w, 1e-5, gate=np.zeros((M, K), np.uint16))
    assert np.all((bits & 0x7FFF) == 0)
    _, bits = oracle.rmsnorm(x, np.zeros(K, np.uint16), 1e-5)
    assert np.all((bits & 0x7FFF) == 0)


def test_scale_invariance_and_row_independence():
    M, K = 4, 1024
    x = inputs.activations(M, K, 31)
    w = inputs.norm_weight(K, 32)
    z = inputs.activations(M, K, 33)
    e0, b0 = oracle.rmsnorm(x, w, 0.0, gate=z)
    x2 = np.where((x & 0x7FFF) == 0, x, x + np.uint16(0x80))      # every value doubled
    e1, b1 = oracle.rmsnorm(x2, w, 0.0, gate=z)
    assert np.array_equal(b0, b1) and np.array_equal(e0, e1)
    perm = np.array([2, 0, 3, 1])
    e2, b2 = oracle.rmsnorm(x[perm], w, 1e-5, gate=z[perm])
    e3, b3 = oracle.rmsnorm(x, w, 1e-5, gate=z)
    assert np.array_equal(b2, b3[perm])


def test_gate_multiplies_elementwise():
    M, K = 2, 384
    x = inputs.activations(M, K, 41)
    w = inputs.norm_weight(K, 42)
    z = inputs.activations(M, K, 43)
    plain, _ = oracle.rmsnorm(x, w, 1e-5)
    gated, _ = oracle.rmsnorm(x, w, 1e-5, gate=z)
    s = torch.nn.functional.silu(bf16_to_f64(z)).numpy()
    assert np.all(np.abs(gated - plain * s) <= 1e-15 * np.abs(plain * s) + 1e-300)


def test_residual_add():
    res = np.array([0x3F80, 0xBF80, 0x4000, 0x0000, 0x3F80, 0x4480], np.uint16)   # 1, -1, 2, 0, 1, 1024
    ref = np.array([0.5, 0.5, -2.0, 3.0, 1.0 / 3.0, 5.0])
    out = oracle.residual_add(res, ref)
    # 1 + 0.5 = 1.5; -1 + 0.5 = -0.5; 2 - 2 = 0; 0 + 3 = 3;
    # 1 + bf16(1/3) = 1 + 0.333984375 -> bf16 1.3359375; 1024 + 5 = 1029 rounds to 1032 (ulp 8)
    want = torch.tensor([1.5, -0.5, 0.0, 3.0, 1.3359375, 1032.0], dtype=torch.float64)
    assert np.array_equal(oracle.bf16_value(out), want.numpy())
    # against torch's BF16 add on random data (equal-magnitude values: no double rounding)
    r = inputs.activations(1, 4096, 51)[0]
    f = oracle.bf16_value(inputs.activations(1, 4096, 52)[0]) * 0.75
    got = oracle.residual_add(r, f)
    t = (bf16_to_f64(r).to(torch.float32) + torch.from_numpy(f).to(torch.bfloat16).to(torch.float32)).to(torch.bfloat16)
    assert np.array_equal(got, t.view(torch.int16).numpy().view(np.uint16))


def test_norm_contract():
    x = inputs.activations(2, 256, 1)
    w = inputs.norm_weight(256, 2)
    with pytest.raises(ValueError):
        oracle.rmsnorm(x, w[:128], 1e-5)
    with pytest.raises(ValueError):
        oracle.rmsnorm(x, w, 1e-5, gate=x[:1])
    with pytest.raises(TypeError):
        oracle.rmsnorm(x.astype(np.float32), w, 1e-5)
    with pytest.raises(ValueError):
        oracle.rmsnorm(x, w, 1e-5, group=100)
