"""GPU parity of the norm prologues and the residual epilogue (the Mamba-2
layer's forward steps 1, 6 and 8 around its projections; nemotron_mamba2.rs
module docs) against the CPU oracle.

* w8a16_rmsnorm: every element within one BF16 step of the oracle's rounding
  of the exact fp64 value (the kernel works in fp32, so a value that lies
  within fp32 error of a rounding midpoint may round the other way), and at
  most 1 % of the elements so.
* The products: |gpu - ref| <= 4e-3 * den + 1e-6 as for the plain projection,
  with ref and den the oracle's product over the oracle's normalized
  activations; with the residual, against residual + ref with one more BF16
  rounding (2^-8 of the value) allowed.
* The epilogue alone is checked bit for bit: out = bf16(residual + y) where y
  is the same path's output without the residual, on every GEMM path.
"""
import numpy as np
import pytest
import torch

import oracle
from gemm_mamba_ssm_amd import binding, inputs

pytestmark = pytest.mark.gpu

RTOL, ATOL = 4e-3, 1e-6
EPS = inputs.NORM_EPS


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


def u8(a: np.ndarray, device):
    return torch.from_numpy(np.ascontiguousarray(a).copy()).to(device)


def bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def check_close(got_bits, want, den, what, extra_rel=0.0):
    g = oracle.bf16_value(got_bits)
    tol = RTOL * den + extra_rel * np.abs(want) + ATOL
    err = np.abs(g - want)
    bad = ~(err <= tol)
    say(f"  {what}: {err.size} elements, max err/tol {float(np.max(err / tol)) if err.size else 0.0:.4f}")
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; first {np.argwhere(bad)[:5].tolist()}"


def bf16_sum_bits(a_bits, b_bits):
    """BF16 bits of a + b for two BF16 arrays (fp32 add, one rounding): the
    residual epilogue's exact property, written independently of the oracle."""
    ta = torch.from_numpy(np.ascontiguousarray(a_bits).view(np.int16)).view(torch.bfloat16).float()
    tb = torch.from_numpy(np.ascontiguousarray(b_bits).view(np.int16)).view(torch.bfloat16).float()
    return (ta + tb).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def check_norm_bits(got, want, what):
    """Each element equals the oracle's BF16 or is its neighbour (same sign)."""
    g = got.astype(np.int32)
    w = want.astype(np.int32)
    same_sign = (g & 0x8000) == (w & 0x8000)
    step = np.abs((g & 0x7FFF) - (w & 0x7FFF))
    zero = ((g & 0x7FFF) == 0) & ((w & 0x7FFF) == 0)
    ok = zero | (same_sign & (step <= 1))
    frac = float(np.mean(g != w))
    say(f"  {what}: {g.size} values, {frac * 100:.3f} % one step off")
    assert ok.all(), f"{what}: {int((~ok).sum())} values more than one BF16 step off; first {np.argwhere(~ok)[:5].tolist()}"
    assert frac <= 0.01, f"{what}: {frac * 100:.2f} % of the values differ"


# --- standalone norm ------------------------------------------------------------

@pytest.mark.parametrize("gated", [False, True])
# K picks the kernel: up to 2048 / 4096 / 8192 / 16384 values hold 1 / 2 / 4 / 8
# chunks per thread in registers; longer rows loop over the row twice.
@pytest.mark.parametrize("M,K", [(1, 4096), (3, 8192), (1024, 4096), (5, 16), (2, 16400), (17, 272),
                                 (2, 16384), (4, 12288), (3, 2064)])
def test_rmsnorm(dev, gated, M, K):
    say(f"rmsnorm gated={gated} M={M} K={K}")
    x = inputs.activations(M, K, 3100 + K)
    w = inputs.norm_weight(K, 3200 + K)
    z = inputs.activations(M, K, 3300 + K) if gated else None
    got = binding.w8a16_rmsnorm(bf(x, dev), bf(w, dev), EPS, gate=bf(z, dev) if gated else None)
    torch.cuda.synchronize()
    _, want = oracle.rmsnorm(x, w, EPS, gate=z)
    check_norm_bits(bits(got), want, f"rmsnorm gated={gated} M={M} K={K}")


# Grouped norm (the published Mamba-2 gated norm: groups of K / n_groups
# channels): whole-row bits with group = K, the oracle's grouped norm otherwise.
@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("M,K,G", [(3, 8192, 1024), (1024, 8192, 1024), (2, 16384, 2048), (5, 4096, 4096),
                                   (4, 2048, 1024), (2, 12288, 3072), (3, 1024, 1024)])
def test_rmsnorm_grouped(dev, gated, M, K, G):
    say(f"rmsnorm grouped gated={gated} M={M} K={K} group={G}")
    x = inputs.activations(M, K, 3150 + K + G)
    w = inputs.norm_weight(K, 3250 + K)
    z = inputs.activations(M, K, 3350 + K) if gated else None
    dx, dw, dz = bf(x, dev), bf(w, dev), bf(z, dev) if gated else None
    got = bits(binding.w8a16_rmsnorm(dx, dw, EPS, gate=dz, group=G))
    _, want = oracle.rmsnorm(x, w, EPS, gate=z, group=G)
    check_norm_bits(got, want, f"rmsnorm grouped gated={gated} M={M} K={K} group={G}")
    if G == K:
        assert np.array_equal(got, bits(binding.w8a16_rmsnorm(dx, dw, EPS, gate=dz)))


def test_rmsnorm_zero_row_and_big_eps(dev):
    M, K = 3, 512
    x = inputs.activations(M, K, 3401)
    x[1] = 0                                           # an all-zero row normalizes to zero
    w = inputs.norm_weight(K, 3402)
    for eps in (EPS, 4.0):
        got = bits(binding.w8a16_rmsnorm(bf(x, dev), bf(w, dev), eps))
        _, want = oracle.rmsnorm(x, w, eps)
        assert np.all((got[1] & 0x7FFF) == 0)
        check_norm_bits(got, want, f"rmsnorm eps={eps}")


# --- fused decode GEMV ------------------------------------------------------------

FUSED_SHAPES = [(1, 18560, 4096), (1, 4096, 8192), (1, 8192, 16384), (2, 1000, 1040), (3, 300, 16384),
                (4, 1000, 4096), (6, 259, 272), (8, 4096, 8192), (1, 7, 16)]


@pytest.mark.parametrize("M,N,K", FUSED_SHAPES)
def test_gemv_fused_norm_prologue(dev, M, N, K):
    """in_proj form: RMSNorm of the layer input, then the projection."""
    say(f"gemv_fused rmsnorm M={M} N={N} K={K}")
    x = inputs.activations(M, K, 3500 + M)
    w = inputs.norm_weight(K, 3600 + K)
    Wq, S = inputs.weights(N, K, 0.02, 3700 + N)
    got = binding.w8a16_gemv_fused(bf(x, dev), u8(Wq, dev), bf(S, dev), norm_weight=bf(w, dev), eps=EPS)
    torch.cuda.synchronize()
    _, a = oracle.rmsnorm(x, w, EPS)
    ref, den = oracle.w8a16(a, Wq, S)
    check_close(bits(got), ref, den, f"fused norm M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", FUSED_SHAPES)
def test_gemv_fused_gated_norm_and_residual(dev, M, N, K):
    """out_proj form: gated RMSNorm of y with z, the projection, the residual add."""
    say(f"gemv_fused gated+residual M={M} N={N} K={K}")
    y = inputs.activations(M, K, 3800 + M)
    z = inputs.activations(M, K, 3900 + M)
    w = inputs.norm_weight(K, 4000 + K)
    res = inputs.activations(M, N, 4100 + N)
    Wq, S = inputs.weights(N, K, 0.02, 4200 + N)
    got = binding.w8a16_gemv_fused(bf(y, dev), u8(Wq, dev), bf(S, dev), norm_weight=bf(w, dev), eps=EPS,
                                   gate=bf(z, dev), residual=bf(res, dev))
    torch.cuda.synchronize()
    _, a = oracle.rmsnorm(y, w, EPS, gate=z)
    ref, den = oracle.w8a16(a, Wq, S)
    want = oracle.bf16_value(res) + ref
    check_close(bits(got), want, den, f"fused gated+res M={M} N={N} K={K}", extra_rel=2.0 ** -8)


@pytest.mark.parametrize("M,N,K,G", [(1, 4096, 8192, 1024), (2, 4096, 8192, 2048), (4, 1000, 16384, 1024),
                                     (8, 4096, 8192, 1024), (1, 18560, 4096, 1024), (3, 300, 16384, 8192),
                                     (1, 4096, 8192, 8192)])
def test_gemv_fused_grouped_gated_norm(dev, M, N, K, G):
    """out_proj form with the gated norm over groups of G channels (the
    published Mamba-2 norm with K / G groups), the projection and the
    residual; group = K gives the whole-row bits."""
    say(f"gemv_fused grouped gated+residual M={M} N={N} K={K} group={G}")
    y = inputs.activations(M, K, 3810 + M)
    z = inputs.activations(M, K, 3910 + M)
    w = inputs.norm_weight(K, 4010 + K)
    res = inputs.activations(M, N, 4110 + N)
    Wq, S = inputs.weights(N, K, 0.02, 4210 + N)
    dy, dz, dw, dr = bf(y, dev), bf(z, dev), bf(w, dev), bf(res, dev)
    dW, dS = u8(Wq, dev), bf(S, dev)
    got = bits(binding.w8a16_gemv_fused(dy, dW, dS, norm_weight=dw, eps=EPS, gate=dz, residual=dr, group=G))
    _, a = oracle.rmsnorm(y, w, EPS, gate=z, group=G)
    ref, den = oracle.w8a16(a, Wq, S)
    want = oracle.bf16_value(res) + ref
    check_close(got, want, den, f"fused grouped M={M} N={N} K={K} group={G}", extra_rel=2.0 ** -8)
    if G == K:
        whole = bits(binding.w8a16_gemv_fused(dy, dW, dS, norm_weight=dw, eps=EPS, gate=dz, residual=dr))
        assert np.array_equal(got, whole)


@pytest.mark.parametrize("M", [1, 3, 8])
def test_gemv_fused_gate_read_in_place(dev, M):
    """The gate as a column slice of a wider row (z of the in_proj output row
    [z | xBC | dt]): the same bits as with a contiguous copy of it."""
    N, K = 4096, 8192
    y = inputs.activations(M, K, 4310 + M)
    zrow = inputs.activations(M, K + 2208, 4320 + M)                  # z in columns 8 .. 8 + K
    w = inputs.norm_weight(K, 4330)
    res = inputs.activations(M, N, 4340 + M)
    Wq, S = inputs.weights(N, K, 0.02, 4350)
    dy, dW, dS, dw, dr = bf(y, dev), u8(Wq, dev), bf(S, dev), bf(w, dev), bf(res, dev)
    zdev = bf(zrow, dev)
    z_slice = zdev[:, 8:8 + K]
    z_copy = z_slice.contiguous()
    a = bits(binding.w8a16_gemv_fused(dy, dW, dS, norm_weight=dw, eps=EPS, gate=z_slice, residual=dr))
    b = bits(binding.w8a16_gemv_fused(dy, dW, dS, norm_weight=dw, eps=EPS, gate=z_copy, residual=dr))
    assert np.array_equal(a, b)
    _, act = oracle.rmsnorm(y, w, EPS, gate=np.ascontiguousarray(zrow[:, 8:8 + K]))
    ref, den = oracle.w8a16(act, Wq, S)
    check_close(a, oracle.bf16_value(res) + ref, den, f"gate slice M={M}", extra_rel=2.0 ** -8)


@pytest.mark.parametrize("M", [1, 2, 3])
def test_gemv_fused_without_prologue_matches_plain_bits(dev, M):
    """With neither norm nor residual the fused kernel computes the plain GEMV's
    sums in the same order (M <= 3 runs the same GEMV kernel)."""
    N, K = 1000, 4096
    A = inputs.activations(M, K, 4300 + M)
    Wq, S = inputs.weights(N, K, 0.02, 4400)
    dA, dW, dS = bf(A, dev), u8(Wq, dev), bf(S, dev)
    plain = bits(binding.w8a16_gemv(dA, dW, dS))
    fused = bits(binding.w8a16_gemv_fused(dA, dW, dS))
    assert np.array_equal(plain, fused)
    res = inputs.activations(M, N, 4500 + M)
    with_res = bits(binding.w8a16_gemv_fused(dA, dW, dS, residual=bf(res, dev)))
    assert np.array_equal(with_res, bf16_sum_bits(res, plain))


# --- residual epilogue of the GEMM (every path) ------------------------------------

GEMM_RES_SHAPES = [(1, 384, 256), (16, 1000, 4096), (20, 4096, 8192), (40, 98400, 528), (129, 1000, 1040),
                   (300, 257, 4096), (66, 65704, 1040), (513, 640, 1024), (200, 12200, 1280),
                   (12, 300, 6160), (20, 1000, 36880), (768, 4096, 256)]


@pytest.mark.parametrize("M,N,K", GEMM_RES_SHAPES)
def test_gemm_residual_epilogue_bits(dev, M, N, K):
    """out = bf16(residual + y) exactly, y = the same GEMM without the residual
    (skinny kernel, mid-size kernel, 32-, 64- and 128-row tiles, the k-split
    workgroups)."""
    say(f"gemm_residual M={M} N={N} K={K}")
    A = inputs.activations(M, K, 4600 + M)
    Wq, S = inputs.weights(N, K, 0.02, 4700 + N + K)
    res = inputs.activations(M, N, 4800 + M)
    dA, dW, dS = bf(A, dev), u8(Wq, dev), bf(S, dev)
    y = bits(binding.w8a16_gemm(dA, dW, dS))
    got = bits(binding.w8a16_gemm_residual(dA, dW, dS, bf(res, dev)))
    assert np.array_equal(got, bf16_sum_bits(res, y))
    if M * N * K <= 2 ** 31:
        ref, den = oracle.w8a16(A, Wq, S)
        check_close(got, oracle.bf16_value(res) + ref, den, f"gemm_residual M={M} N={N} K={K}",
                    extra_rel=2.0 ** -8)


def test_prefill_two_step_layer_ends(dev):
    """Prefill form: w8a16_rmsnorm then the GEMM (in_proj), and the gated norm
    then the GEMM with the residual (out_proj), at the 1024-token shapes,
    checked on sampled rows, columns and points."""
    p_in, p_out = inputs.WORKLOADS["prefill_1k"]
    rng = np.random.default_rng(9)
    for p, gated in ((p_in, False), (p_out, True)):
        say(f"prefill two-step {p.name} M={p.M} N={p.N} K={p.K}")
        x = inputs.activations(p.M, p.K, p.seed_a)
        w = inputs.norm_weight(p.K, 5000 + p.K)
        z = inputs.activations(p.M, p.K, 5100) if gated else None
        _, Wq, S = inputs.make(p)
        dW, dS = u8(Wq, dev), bf(S, dev)
        a_dev = binding.w8a16_rmsnorm(bf(x, dev), bf(w, dev), EPS, gate=bf(z, dev) if gated else None)
        _, a = oracle.rmsnorm(x, w, EPS, gate=z)
        check_norm_bits(bits(a_dev), a, f"{p.name} norm")
        mi = np.concatenate([np.repeat([0, p.M - 1], p.N), rng.integers(0, p.M, 20000)])
        ni = np.concatenate([np.tile(np.arange(p.N), 2), rng.integers(0, p.N, 20000)])
        ref, den = oracle.w8a16_points(a, Wq, S, mi, ni)
        if gated:
            res = inputs.activations(p.M, p.N, 5200)
            got = bits(binding.w8a16_gemm_residual(a_dev, dW, dS, bf(res, dev)))
            check_close(got[mi, ni], oracle.bf16_value(res[mi, ni]) + ref, den, f"{p.name} + residual",
                        extra_rel=2.0 ** -8)
        else:
            got = bits(binding.w8a16_gemm(a_dev, dW, dS))
            check_close(got[mi, ni], ref, den, f"{p.name}")
        torch.cuda.synchronize()


def test_fused_rejections_on_device(dev):
    Wq, S = inputs.weights(256, 256, 0.02, 5301)
    dW, dS = u8(Wq, dev), bf(S, dev)
    A = torch.ones((9, 256), dtype=torch.bfloat16, device=dev)
    out = torch.empty((9, 256), dtype=torch.bfloat16, device=dev)
    st = binding.gemv_fused_raw(A.data_ptr(), 0, 0, 1e-5, dW.data_ptr(), dS.data_ptr(), 0, out.data_ptr(),
                                9, 256, 256, 0)
    assert st == binding.ERR_SHAPE
    res = torch.zeros((2, 256), dtype=torch.bfloat16, device=dev)
    st = binding.gemm_residual_raw(A.data_ptr(), dW.data_ptr(), dS.data_ptr(), res.data_ptr(), res.data_ptr(),
                                   2, 256, 256, 0)
    assert st == binding.ERR_ALIAS
    torch.cuda.synchronize()
