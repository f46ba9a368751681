"""Pins of the oracle's Mamba-2 decode step (conv1d update with bias and SiLU;
SSM state update and output), the forward steps 3 to 5 of the nemotron_mamba2.rs
module docs, read as the standard Mamba-2 recurrence.

The conv update is checked against numpy's convolution over a token
sequence; the SSM state against scipy's first-order IIR filter (the state of
one (head, p, n) is a first-order recurrence in time) and against the closed
form of a geometric series for constant inputs; the output against a direct
contraction of those states; softplus against torch; the group mapping, the
dt clamp and the skip term by construction.
"""
import numpy as np
import pytest
import scipy.signal
import torch

import oracle
from gemm_mamba_ssm_amd import inputs


def bf16_f64(bits):
    return torch.from_numpy(np.array(bits, copy=True).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def to_bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def silu(v):
    return torch.nn.functional.silu(torch.from_numpy(np.asarray(v, np.float64))).numpy()


def test_softplus_matches_torch():
    v = np.linspace(-30, 19, 981)
    got = np.array([oracle.softplus(t) for t in v])
    want = torch.nn.functional.softplus(torch.from_numpy(v)).numpy()
    assert np.all(np.abs(got - want) <= 1e-14 * np.abs(want) + 1e-300)


@pytest.mark.parametrize("d_conv", [2, 3, 4])
def test_conv_update_is_a_causal_convolution(d_conv):
    B, dim, T = 2, 37, 9
    w, bias = inputs.conv_params(dim, d_conv, 11 + d_conv)
    xs = [inputs.activations(B, dim + 5, 100 + t) for t in range(T)]      # rows longer than dim (ld_x)
    state = np.zeros((B, dim, d_conv))
    outs = []
    for t in range(T):
        exact, bits = oracle.conv1d_update(state, xs[t], w, bias)
        assert np.array_equal(bits, oracle.bf16_rne(exact))
        outs.append(exact)
    wf, bf = bf16_f64(w), bf16_f64(bias)
    for b in range(B):
        for c in range(dim):
            seq = np.array([bf16_f64(xs[t][b, c:c + 1])[0] for t in range(T)])
            # causal: out_t = sum_w weight[w] * x_{t - (d_conv - 1) + w}, zeros before t = 0
            pre = np.convolve(seq, wf[c][::-1])[:T] + bf[c]
            got = np.array([outs[t][b, c] for t in range(T)])
            assert np.allclose(got, silu(pre), rtol=1e-13, atol=1e-300), (b, c)
            # the state ends holding the last d_conv inputs, oldest first
            assert np.array_equal(state[b, c], seq[T - d_conv:])


def test_conv_one_hot_tap_and_zero_weights():
    B, dim, d_conv = 1, 8, 4
    state = inputs.conv_state(B, dim, d_conv, 3).astype(np.float64)
    x = inputs.activations(B, dim, 4)
    w = np.zeros((dim, d_conv), np.uint16)
    w[:, 1] = 0x3F80                                      # 1.0 on tap 1
    bias = np.zeros(dim, np.uint16)
    before = state.copy()
    exact, _ = oracle.conv1d_update(state, x, w, bias)
    # after the shift, tap 1 holds what tap 2 held before
    assert np.allclose(exact[0], silu(before[0, :, 2]), rtol=1e-15, atol=0)
    state2 = before.copy()
    exact0, bits0 = oracle.conv1d_update(state2, x, np.zeros_like(w), to_bf16(np.full(dim, 0.5)))
    assert np.all(exact0 == silu(0.5))


def test_ssm_state_is_a_first_order_filter():
    """Constant dt per head, time-varying x and B: each state element follows
    h_t = dA h_{t-1} + dt B_t[n] x_t[p], i.e. lfilter([1], [1, -dA], u)."""
    Bn, heads, hd, st, groups, T = 1, 4, 3, 5, 2, 12
    a_log, d_param, dt_bias = inputs.ssm_params(heads, 7)
    d_inner = heads * hd
    h = np.zeros((Bn, heads, hd, st))
    dt_raw = inputs.activations(Bn, heads, 8)                      # the same every step
    rows = [inputs.activations(Bn, d_inner + 2 * groups * st, 200 + t) for t in range(T)]
    ys = []
    for t in range(T):
        y, bits, den = oracle.ssm_decode(h, rows[t], dt_raw, a_log, d_param, dt_bias, groups)
        assert np.array_equal(bits, oracle.bf16_rne(y))
        ys.append(y[0])
    per = heads // groups
    for hh in range(heads):
        g = hh // per
        dt = np.log1p(np.exp(bf16_f64(dt_raw[0, hh:hh + 1])[0] + np.float64(dt_bias[hh])))
        dA = np.exp(dt * -np.exp(np.float64(a_log[hh])))
        for p in range(hd):
            for n in range(st):
                u = np.array([dt * bf16_f64(rows[t][0, d_inner + g * st + n:d_inner + g * st + n + 1])[0]
                              * bf16_f64(rows[t][0, hh * hd + p:hh * hd + p + 1])[0] for t in range(T)])
                traj = scipy.signal.lfilter([1.0], [1.0, -dA], u)
                assert abs(h[0, hh, p, n] - traj[-1]) <= 1e-12 * (np.abs(traj).max() + 1e-300)
    # the output of the last step: y = sum_n C[n] h[n] + D x
    last = rows[-1][0]
    C = bf16_f64(last[d_inner + groups * st:d_inner + 2 * groups * st]).reshape(groups, st)
    xv = bf16_f64(last[:d_inner]).reshape(heads, hd)
    want = np.array([[C[hh // per] @ h[0, hh, p] + np.float64(d_param[hh]) * xv[hh, p] for p in range(hd)]
                     for hh in range(heads)]).ravel()
    assert np.allclose(ys[-1], want, rtol=1e-12, atol=1e-15)


def test_ssm_geometric_series_closed_form():
    """Constant x, B, dt for T steps from h0: h_T = dA^T h0 + u (1 - dA^T) / (1 - dA)."""
    Bn, heads, hd, st, groups, T = 2, 2, 2, 3, 1, 25
    a_log, d_param, dt_bias = inputs.ssm_params(heads, 9)
    h0 = inputs.ssm_state(Bn, heads, hd, st, 10).astype(np.float64)
    h = h0.copy()
    row = inputs.activations(Bn, heads * hd + 2 * groups * st, 11)
    dt_raw = inputs.activations(Bn, heads, 12)
    for _ in range(T):
        oracle.ssm_decode(h, row, dt_raw, a_log, d_param, dt_bias, groups)
    for b in range(Bn):
        for hh in range(heads):
            dt = oracle.softplus(bf16_f64(dt_raw[b, hh:hh + 1])[0] + np.float64(dt_bias[hh]))
            dA = np.exp(dt * -np.exp(np.float64(a_log[hh])))
            Bv = bf16_f64(row[b, heads * hd:heads * hd + st])
            xv = bf16_f64(row[b, hh * hd:(hh + 1) * hd])
            u = dt * np.outer(xv, Bv)
            want = dA ** T * h0[b, hh] + u * (1 - dA ** T) / (1 - dA)
            assert np.allclose(h[b, hh], want, rtol=1e-11, atol=1e-14)


def test_ssm_output_selects_c_of_its_group_closed_form():
    """Output pin independent of the oracle's contraction: C of group g is one-hot
    at state index n_g (and a two-hot mix), B, x, dt constant, so every state
    element follows the geometric series h_t = dA^t h0 + u (1 - dA^t) / (1 - dA)
    and the output after step t is y[h, p] = h_t[h, p, n_g(h)] + D[h] x[h, p]
    (resp. 2 h_t[.., a] - h_t[.., b] / 2 + D x). A C read from the wrong group or
    from B's columns, or outputs in another order, pick other state elements."""
    Bn, heads, hd, st, groups, T = 1, 8, 3, 5, 4, 6
    a_log, d_param, dt_bias = inputs.ssm_params(heads, 21)
    d_inner = heads * hd
    per = heads // groups
    h0 = inputs.ssm_state(Bn, heads, hd, st, 22).astype(np.float64)
    row = inputs.activations(Bn, d_inner + 2 * groups * st, 23)       # x and B random
    pick = [(2 * g + 1) % st for g in range(groups)]
    c0 = d_inner + groups * st
    row[0, c0:] = 0
    for g in range(groups):
        row[0, c0 + g * st + pick[g]] = 0x3F80                          # C_g = e_pick[g]
    dt_raw = inputs.activations(Bn, heads, 24)
    dt = np.array([oracle.softplus(bf16_f64(dt_raw[0, hh:hh + 1])[0] + np.float64(dt_bias[hh])) for hh in range(heads)])
    dA = np.exp(dt * -np.exp(np.float64(a_log)))
    xv = bf16_f64(row[0, :d_inner]).reshape(heads, hd)
    Bv = bf16_f64(row[0, d_inner:d_inner + groups * st]).reshape(groups, st)

    def h_closed(t):
        u = dt[:, None, None] * xv[:, :, None] * Bv[np.arange(heads) // per][:, None, :]
        a = dA[:, None, None]
        return a ** t * h0[0] + u * (1 - a ** t) / (1 - a)

    h = h0.copy()
    for t in range(1, T + 1):
        y, _, _ = oracle.ssm_decode(h, row, dt_raw, a_log, d_param, dt_bias, groups)
        ht = h_closed(t)
        want = np.array([[ht[hh, p, pick[hh // per]] + np.float64(d_param[hh]) * xv[hh, p] for p in range(hd)]
                         for hh in range(heads)])
        assert np.allclose(y[0].reshape(heads, hd), want, rtol=1e-12, atol=1e-15), t
    # a two-hot C: y = 2 h[a] - h[b] / 2 + D x, from the same closed form
    a_i, b_i = 0, st - 1
    row[0, c0:] = 0
    for g in range(groups):
        row[0, c0 + g * st + a_i] = 0x4000                              # 2.0
        row[0, c0 + g * st + b_i] = 0xBF00                              # -0.5
    h = h0.copy()
    for t in range(1, 3):
        y, _, _ = oracle.ssm_decode(h, row, dt_raw, a_log, d_param, dt_bias, groups)
    ht = h_closed(2)
    want = 2 * ht[:, :, a_i] - 0.5 * ht[:, :, b_i] + np.float64(d_param)[:, None] * xv
    assert np.allclose(y[0].reshape(heads, hd), want, rtol=1e-12, atol=1e-15)


def test_ssm_groups_clamp_and_skip():
    Bn, heads, hd, st, groups = 1, 8, 2, 4, 4
    a_log, d_param, dt_bias = inputs.ssm_params(heads, 13)
    d_inner = heads * hd
    row = np.zeros((Bn, d_inner + 2 * groups * st), np.uint16)
    row[0, :d_inner] = inputs.activations(1, d_inner, 14)[0]
    row[0, d_inner + 3 * st:d_inner + 4 * st] = 0x3F80                 # B of group 3 only
    dt_raw = inputs.activations(Bn, heads, 15)
    h = np.zeros((Bn, heads, hd, st))
    y, _, _ = oracle.ssm_decode(h, row, dt_raw, a_log, d_param, dt_bias, groups)
    per = heads // groups
    changed = np.any(h[0] != 0, axis=(1, 2))
    assert np.array_equal(changed, np.arange(heads) // per == 3)
    # C = 0: the output is the skip term D x exactly
    xv = bf16_f64(row[0, :d_inner]).reshape(heads, hd)
    assert np.array_equal(y[0].reshape(heads, hd), np.float64(d_param)[:, None] * xv)
    # dt clamp: dt_min above every softplus value makes dt = dt_min
    h = np.ones((Bn, heads, hd, st))
    row[:] = 0
    oracle.ssm_decode(h, row, dt_raw, a_log, d_param, dt_bias, groups, dt_min=0.5, dt_max=1e9)
    want = np.exp(0.5 * -np.exp(np.float64(a_log)))
    assert np.allclose(h[0], want[:, None, None] * np.ones((heads, hd, st)), rtol=1e-15, atol=0)


def test_ssm_contract():
    h = np.zeros((1, 4, 2, 3))
    row = np.zeros((1, 4 * 2 + 2 * 2 * 3), np.uint16)
    p = inputs.ssm_params(4, 1)
    with pytest.raises(ValueError):
        oracle.ssm_decode(h, row, np.zeros((1, 4), np.uint16), *p, groups=3)     # heads % groups
    with pytest.raises(ValueError):
        oracle.ssm_decode(h, row[:, :-1], np.zeros((1, 4), np.uint16), *p, groups=2)
    with pytest.raises(TypeError):
        oracle.ssm_decode(h.astype(np.float32), row, np.zeros((1, 4), np.uint16), *p, groups=2)
