"""C-ABI checks that need no GPU: the library loads, exports every function
include/w8a16.h declares, and rejects bad arguments on the host before any
HIP call. Also the binding's refusals of wrong dtypes and scale layouts."""
import os
import re

import pytest
import torch

from gemm_mamba_ssm_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w8a16.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w8a16_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = binding.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_strerror_covers_every_status():
    for st in (binding.OK, binding.ERR_NULL, binding.ERR_SHAPE, binding.ERR_ALIGN,
               binding.ERR_LAUNCH, binding.ERR_ALIAS, binding.ERR_ARG, binding.ERR_WORKSPACE,
               binding.ERR_SCRATCH):
        s = binding.strerror(st)
        assert s and "unknown" not in s
    assert "unknown" in binding.strerror(12345)


FAKE = 1 << 40          # an aligned address that is never dereferenced (checks fail first)


@pytest.mark.parametrize("fn", [binding.gemv_raw, binding.gemm_raw])
def test_rejections_before_any_hip_call(fn):
    ok = dict(A=FAKE, Wq=FAKE + (1 << 30), scale=FAKE + (2 << 30), out=FAKE + (3 << 30))

    def call(M=4, N=256, K=256, **over):
        a = dict(ok, **over)
        return fn(a["A"], a["Wq"], a["scale"], a["out"], M, N, K, 0)

    assert call(K=0) == binding.ERR_SHAPE
    assert call(K=8) == binding.ERR_SHAPE
    assert call(K=264 - 1) == binding.ERR_SHAPE
    assert call(K=136) == binding.ERR_SHAPE            # not a multiple of 16
    assert call(M=-1) == binding.ERR_SHAPE
    assert call(N=-5) == binding.ERR_SHAPE
    assert call(M=1 << 31) == binding.ERR_SHAPE
    assert call(M=0) == binding.OK                      # no-op
    assert call(N=0) == binding.OK
    assert call(M=0, A=0, out=0) == binding.OK         # no-op needs no buffers
    assert call(A=0) == binding.ERR_NULL
    assert call(Wq=0) == binding.ERR_NULL
    assert call(scale=0) == binding.ERR_NULL
    assert call(out=0) == binding.ERR_NULL
    assert call(A=FAKE + 8) == binding.ERR_ALIGN
    assert call(Wq=FAKE + (1 << 30) + 4) == binding.ERR_ALIGN
    assert call(scale=FAKE + (2 << 30) + 1) == binding.ERR_ALIGN
    assert call(out=FAKE + (3 << 30) + 1) == binding.ERR_ALIGN
    assert call(out=FAKE) == binding.ERR_ALIAS           # out on top of A
    assert call(out=FAKE + (1 << 30) + 1024) == binding.ERR_ALIAS   # inside Wq
    # out's last 16 bytes reach into the scale grid
    assert call(out=FAKE + (2 << 30) - 2 * 4 * 256 + 16) == binding.ERR_ALIAS


@pytest.mark.parametrize("fn", [binding.gemv_ex_raw, binding.gemm_ex_raw])
def test_scale_format_rejections(fn):
    A, W, S, O = FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30)
    M, N, K = 4, 256, 256
    for bad in (-1, 3, 1000):
        assert fn(A, W, S, bad, O, M, N, K, 0) == binding.ERR_ARG
        assert fn(A, W, S, bad, O, 0, N, K, 0) == binding.ERR_ARG      # checked even for a no-op
    for fmt in (binding.SCALE_BLOCK_BF16, binding.SCALE_BLOCK_F32, binding.SCALE_ROW_F32):
        assert fn(A, W, S, fmt, O, 0, N, K, 0) == binding.OK
        assert fn(A, W, 0, fmt, O, M, N, K, 0) == binding.ERR_NULL
        assert fn(A, W, S + 1, fmt, O, M, N, K, 0) == binding.ERR_ALIGN
    # FP32 scales need 4-byte alignment, BF16 ones only 2
    assert fn(A, W, S + 2, binding.SCALE_BLOCK_F32, O, M, N, K, 0) == binding.ERR_ALIGN
    assert fn(A, W, S + 2, binding.SCALE_ROW_F32, O, M, N, K, 0) == binding.ERR_ALIGN
    # the overlap check uses each format's own size: N*4 bytes of row
    # scales, 2x2 blocks of 4 (FP32) or 2 (BF16) bytes
    out_row_end = S + 4 * N - 2                          # out's first element inside the row scales
    assert fn(A, W, S, binding.SCALE_ROW_F32, out_row_end, M, N, K, 0) == binding.ERR_ALIAS
    out_f32_end = S + 4 * 4 - 2
    assert fn(A, W, S, binding.SCALE_BLOCK_F32, out_f32_end, M, N, K, 0) == binding.ERR_ALIAS


def test_gemv_limits():
    F = FAKE
    args = (F, F + (1 << 30), F + (2 << 30), F + (3 << 30))
    assert binding.gemv_raw(*args, 17, 256, 256, 0) == binding.ERR_SHAPE
    assert binding.gemv_raw(*args, 8, 256, binding.GEMV_MAX_K_SMALL_M + 16, 0) == binding.ERR_SHAPE
    assert binding.gemv_raw(*args, 9, 256, binding.GEMV_MAX_K + 16, 0) == binding.ERR_SHAPE


def test_dequant_rejections():
    F = FAKE
    assert binding.dequant_raw(F, F + (1 << 30), F + (2 << 30), 256, 100, 0) == binding.ERR_SHAPE
    assert binding.dequant_raw(F, F + (1 << 30), F + (2 << 30), 0, 256, 0) == binding.OK
    assert binding.dequant_raw(0, F + (1 << 30), F + (2 << 30), 256, 256, 0) == binding.ERR_NULL
    assert binding.dequant_raw(F, F + (1 << 30), F + (2 << 30) + 4, 256, 256, 0) == binding.ERR_ALIGN
    assert binding.dequant_raw(F, F + (1 << 30), F, 256, 256, 0) == binding.ERR_ALIAS


def _cpu_operands(M=2, N=300, K=256):
    A = torch.zeros((M, K), dtype=torch.bfloat16)
    W = torch.zeros((N, K), dtype=torch.uint8)
    S = torch.zeros(binding.scale_grid(N, K), dtype=torch.bfloat16)
    return A, W, S


def test_binding_refuses_wrong_layouts():
    A, W, S = _cpu_operands()
    N, K = W.shape
    bad_scales = [
        torch.zeros((N,), dtype=torch.bfloat16),                       # per-row [N]
        torch.zeros((), dtype=torch.bfloat16),                         # scalar
        torch.zeros((1,), dtype=torch.float32),                        # raw 4-byte scalar
        torch.zeros((N + 1,), dtype=torch.float32),                    # per-row, wrong length
        torch.zeros(binding.scale_grid(N, K)[::-1], dtype=torch.float32),    # transposed fp32 grid
        torch.zeros(binding.scale_grid(N, K)[::-1], dtype=torch.bfloat16),   # transposed shape
        torch.zeros((3, 4), dtype=torch.bfloat16)[:, :2],              # right shape, not contiguous
        torch.zeros((2 * N,), dtype=torch.float32)[::2],               # per-row, not contiguous
        torch.zeros(binding.scale_grid(N, K), dtype=torch.float16),    # no such format
    ]
    for s in bad_scales:
        for fn in (binding.w8a16_gemv, binding.w8a16_gemm):
            with pytest.raises(ValueError, match="scale"):
                fn(A, W, s)
    grid32 = torch.zeros(binding.scale_grid(N, K), dtype=torch.float32)
    row32 = torch.zeros((N,), dtype=torch.float32)
    for s, fmt in [(grid32, "row_f32"), (row32, "block_f32"), (S, "block_f32"), (grid32, "block_bf16"),
                   (S, "per_tensor")]:
        with pytest.raises(ValueError, match="scale"):
            binding.w8a16_gemm(A, W, s, scale_format=fmt)             # explicit format disagrees
    assert binding.scale_format_of(S) == "block_bf16"
    assert binding.scale_format_of(grid32) == "block_f32"
    assert binding.scale_format_of(row32) == "row_f32"
    for s in (S, grid32, row32):                                        # valid layouts reach the device check
        with pytest.raises(ValueError, match="HIP device"):
            binding.w8a16_gemm(A, W, s)
    with pytest.raises(ValueError):
        binding.w8a16_gemm(A.float(), W, S)                            # A not bf16
    with pytest.raises(ValueError):
        binding.w8a16_gemm(A, W.to(torch.int8), S)                     # not E4M3 bytes
    with pytest.raises(ValueError):
        binding.w8a16_gemm(A[:, :128], W, S)                           # K mismatch
    with pytest.raises(ValueError):
        binding.w8a16_gemv(torch.zeros((17, K), dtype=torch.bfloat16), W, S)
    with pytest.raises(ValueError):
        binding.w8a16_gemm(A, W, S)                                    # CPU tensors
    with pytest.raises(ValueError):
        binding.w8a16_dequant(W, S[:, :1])


def test_norm_and_fused_rejections():
    F = FAKE
    X, G, Wn, O = F, F + (1 << 30), F + (2 << 30), F + (3 << 30)
    nan = float("nan")
    # w8a16_rmsnorm(x, gate, weight, eps, out, M, K)
    assert binding.rmsnorm_raw(X, G, Wn, 1e-5, O, 4, 8, 0) == binding.ERR_SHAPE          # K < 16
    assert binding.rmsnorm_raw(X, G, Wn, 1e-5, O, 4, 264, 0) == binding.ERR_SHAPE          # K % 16
    assert binding.rmsnorm_raw(X, G, Wn, 1e-5, O, -1, 256, 0) == binding.ERR_SHAPE
    assert binding.rmsnorm_raw(X, G, Wn, nan, O, 4, 256, 0) == binding.ERR_ARG
    assert binding.rmsnorm_raw(X, G, Wn, -1.0, O, 4, 256, 0) == binding.ERR_ARG
    assert binding.rmsnorm_raw(X, G, Wn, float("inf"), O, 4, 256, 0) == binding.ERR_ARG
    assert binding.rmsnorm_raw(X, G, Wn, 1e-5, O, 0, 256, 0) == binding.OK               # no-op
    assert binding.rmsnorm_raw(0, G, Wn, 1e-5, O, 4, 256, 0) == binding.ERR_NULL
    assert binding.rmsnorm_raw(X, G, 0, 1e-5, O, 4, 256, 0) == binding.ERR_NULL
    assert binding.rmsnorm_raw(X, G, Wn, 1e-5, 0, 4, 256, 0) == binding.ERR_NULL
    assert binding.rmsnorm_raw(X + 2, G, Wn, 1e-5, O, 4, 256, 0) == binding.ERR_ALIGN
    assert binding.rmsnorm_raw(X, G + 2, Wn, 1e-5, O, 4, 256, 0) == binding.ERR_ALIGN
    assert binding.rmsnorm_raw(X, G, Wn + 8, 1e-5, O, 4, 256, 0) == binding.ERR_ALIGN
    assert binding.rmsnorm_raw(X, G, Wn, 1e-5, X + 16, 4, 256, 0) == binding.ERR_ALIAS   # out over x
    assert binding.rmsnorm_raw(X, G, Wn, 1e-5, G, 4, 256, 0) == binding.ERR_ALIAS        # out over gate
    assert binding.rmsnorm_raw(X, G, Wn, 1e-5, Wn - 16, 4, 256, 0) == binding.ERR_ALIAS  # out reaches weight
    # group: 0 or K, else a multiple of 1024 dividing K <= 16384
    assert binding.rmsnorm_raw(X, G, Wn, 1e-5, O, 0, 8192, 0, group=512) == binding.ERR_SHAPE
    assert binding.rmsnorm_raw(X, G, Wn, 1e-5, O, 0, 8192, 0, group=3072) == binding.ERR_SHAPE   # 8192 % 3072
    assert binding.rmsnorm_raw(X, G, Wn, 1e-5, O, 0, 32768, 0, group=1024) == binding.ERR_SHAPE  # K > 16384
    assert binding.rmsnorm_raw(X, G, Wn, 1e-5, O, 0, 8192, 0, group=-1024) == binding.ERR_SHAPE
    assert binding.rmsnorm_raw(X, G, Wn, 1e-5, O, 0, 8192, 0, group=16384) == binding.ERR_SHAPE  # > K
    assert binding.rmsnorm_raw(X, G, Wn, 1e-5, O, 0, 8192, 0, group=2048) == binding.OK          # no-op, valid
    assert binding.rmsnorm_raw(X, G, Wn, 1e-5, O, 0, 32768, 0, group=32768) == binding.OK        # group = K
    # w8a16_gemv_fused(A, gate, norm_weight, eps, Wq, scale, residual, out, M, N, K)
    A, Wq, S = F + (4 << 30), F + (5 << 30), F + (6 << 30)
    R = F + (7 << 30)
    fused = binding.gemv_fused_raw
    assert fused(A, G, 0, 1e-5, Wq, S, R, O, 1, 256, 256, 0) == binding.ERR_ARG       # gate without norm
    assert fused(A, 0, Wn, nan, Wq, S, R, O, 1, 256, 256, 0) == binding.ERR_ARG
    assert fused(A, 0, Wn, 1e-5, Wq, S, R, O, 9, 256, 256, 0) == binding.ERR_SHAPE    # M > 8
    assert fused(A, 0, Wn, 1e-5, Wq, S, R, O, 5, 256, 8192 + 16, 0) == binding.ERR_SHAPE
    assert fused(A, 0, Wn, 1e-5, Wq, S, R, O, 4, 256, 16384 + 16, 0) == binding.ERR_SHAPE
    assert fused(A, 0, Wn, 1e-5, Wq, S, R, O, 0, 256, 256, 0) == binding.OK           # no-op
    assert fused(A, G, Wn, 1e-5, Wq, S, R, O, 1, 256, 256, 0, ld_gate=255) == binding.ERR_SHAPE   # ld_gate < K
    assert fused(A, G, Wn, 1e-5, Wq, S, R, O, 1, 256, 256, 0, ld_gate=260) == binding.ERR_SHAPE   # ld_gate % 8
    assert fused(A, 0, Wn + 8, 1e-5, Wq, S, R, O, 1, 256, 256, 0) == binding.ERR_ALIGN
    assert fused(A, G + 8, Wn, 1e-5, Wq, S, R, O, 1, 256, 256, 0) == binding.ERR_ALIGN
    assert fused(A, 0, Wn, 1e-5, Wq, S, R + 1, O, 1, 256, 256, 0) == binding.ERR_ALIGN
    assert fused(A, 0, Wn, 1e-5, Wq, S, O, O, 1, 256, 256, 0) == binding.ERR_ALIAS    # residual is out
    assert fused(A, 0, O + 64, 1e-5, Wq, S, R, O, 1, 256, 256, 0) == binding.ERR_ALIAS   # out over norm weight
    assert fused(A, G, Wn, 1e-5, Wq, S, R, G + 2, 1, 256, 256, 0) == binding.ERR_ALIAS    # out over gate
    assert fused(A, 0, 0, 1e-5, Wq, S, 0, A, 1, 256, 256, 0) == binding.ERR_ALIAS        # out over A
    assert fused(A, G, Wn, 1e-5, Wq, S, R, O, 1, 4096, 8192, 0, group=1000) == binding.ERR_SHAPE
    assert fused(A, G, Wn, 1e-5, Wq, S, R, O, 0, 4096, 8192, 0, group=1024) == binding.OK     # no-op, valid
    # w8a16_gemm_residual(A, Wq, scale, residual, out, M, N, K)
    assert binding.gemm_residual_raw(A, Wq, S, 0, O, 4, 256, 256, 0) == binding.ERR_NULL
    assert binding.gemm_residual_raw(A, Wq, S, R + 1, O, 4, 256, 256, 0) == binding.ERR_ALIGN
    assert binding.gemm_residual_raw(A, Wq, S, O + 256, O, 4, 256, 256, 0) == binding.ERR_ALIAS
    assert binding.gemm_residual_raw(A, Wq, S, R, O, 0, 256, 256, 0) == binding.OK


def test_binding_refuses_bad_norm_arguments():
    A, W, S = _cpu_operands(M=2, N=300, K=256)
    w = torch.ones(256, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="weight"):
        binding.w8a16_rmsnorm(A, w[:128], 1e-5)
    with pytest.raises(ValueError, match="gate"):
        binding.w8a16_rmsnorm(A, w, 1e-5, gate=A[:1])
    with pytest.raises(ValueError, match="eps"):
        binding.w8a16_rmsnorm(A, w, float("nan"))
    with pytest.raises(ValueError, match="eps"):
        binding.w8a16_gemv_fused(A, W, S, norm_weight=w, eps=-1.0)
    with pytest.raises(ValueError, match="group"):
        binding.w8a16_rmsnorm(A, w, 1e-5, group=100)
    with pytest.raises(ValueError, match="group"):
        binding.w8a16_gemv_fused(A, W, S, norm_weight=w, group=128)
    with pytest.raises(ValueError, match="gate needs"):
        binding.w8a16_gemv_fused(A, W, S, gate=A)
    with pytest.raises(ValueError, match="residual"):
        binding.w8a16_gemv_fused(A, W, S, residual=torch.zeros((2, 299), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="M <= 4"):
        binding.w8a16_gemv_fused(torch.zeros((9, 256), dtype=torch.bfloat16), W, S)
    with pytest.raises(ValueError, match="residual"):
        binding.w8a16_gemm_residual(A, W, S, torch.zeros((2, 300), dtype=torch.float32))
    with pytest.raises(ValueError, match="HIP device"):
        binding.w8a16_gemm_residual(A, W, S, torch.zeros((2, 300), dtype=torch.bfloat16))


def test_mamba2_step_rejections():
    F = FAKE
    St, X, Wt, Bi, O = F, F + (1 << 30), F + (2 << 30), F + (3 << 30), F + (4 << 30)
    conv = binding.conv1d_update_raw
    # conv1d_update(state, x, ld_x, weight, bias, out, ld_out, batch, dim, d_conv)
    assert conv(St, X, 64, Wt, Bi, O, 64, 1, 64, 0, 0) == binding.ERR_SHAPE        # d_conv < 1
    assert conv(St, X, 64, Wt, Bi, O, 64, 1, 64, 9, 0) == binding.ERR_SHAPE        # d_conv > 8
    assert conv(St, X, 63, Wt, Bi, O, 64, 1, 64, 4, 0) == binding.ERR_SHAPE        # ld_x < dim
    assert conv(St, X, 64, Wt, Bi, O, 63, 1, 64, 4, 0) == binding.ERR_SHAPE
    assert conv(St, X, 64, Wt, Bi, O, 64, 65536, 64, 4, 0) == binding.ERR_SHAPE
    assert conv(St, X, 64, Wt, Bi, O, 64, 0, 64, 4, 0) == binding.OK               # no-op
    assert conv(0, X, 64, Wt, Bi, O, 64, 1, 64, 4, 0) == binding.ERR_NULL
    assert conv(St, X, 64, Wt, 0, O, 64, 1, 64, 4, 0) == binding.ERR_NULL
    assert conv(St + 2, X, 64, Wt, Bi, O, 64, 1, 64, 4, 0) == binding.ERR_ALIGN
    assert conv(St, X + 1, 64, Wt, Bi, O, 64, 1, 64, 4, 0) == binding.ERR_ALIGN
    assert conv(St, X, 64, Wt, Bi, X + 64, 64, 1, 64, 4, 0) == binding.ERR_ALIAS   # out over x
    assert conv(St, X, 64, Wt, Bi, St + 100, 64, 1, 64, 4, 0) == binding.ERR_ALIAS  # out over the state
    assert conv(St, St + 256, 64, Wt, Bi, O, 64, 1, 64, 4, 0) == binding.ERR_ALIAS  # x inside the state
    # ssm_decode(h, xbc, ld_xbc, dt, ld_dt, a_log, D, dt_bias, out, ld_out, batch, heads, hd, state, groups, dt_min, dt_max)
    H, Xb, Dt, Al, Dp, Db = F, F + (1 << 30), F + (2 << 30), F + (3 << 30), F + (3 << 30) + 4096, F + (3 << 30) + 8192
    ssm = binding.ssm_decode_raw
    w = 8 * 4 + 2 * 2 * 16                                                      # heads 8, hd 4, groups 2, state 16

    def call(**kw):
        a = dict(h=H, xbc=Xb, ld_xbc=w, dt=Dt, ld_dt=8, al=Al, dp=Dp, db=Db, out=O, ld_out=32, batch=1, heads=8,
                 hd=4, state=16, groups=2, dmin=0.0, dmax=1e9)
        a.update(kw)
        return ssm(a["h"], a["xbc"], a["ld_xbc"], a["dt"], a["ld_dt"], a["al"], a["dp"], a["db"], a["out"],
                   a["ld_out"], a["batch"], a["heads"], a["hd"], a["state"], a["groups"], a["dmin"], a["dmax"], 0)

    assert call(groups=3) == binding.ERR_SHAPE                                  # heads % groups
    assert call(state=18) == binding.ERR_SHAPE                                  # state % 4
    assert call(state=260) == binding.ERR_SHAPE                                 # state > 256
    assert call(ld_xbc=w - 1) == binding.ERR_SHAPE
    assert call(ld_dt=7) == binding.ERR_SHAPE
    assert call(ld_out=31) == binding.ERR_SHAPE
    assert call(dmin=-1.0) == binding.ERR_ARG
    assert call(dmin=2.0, dmax=1.0) == binding.ERR_ARG
    assert call(dmax=float("nan")) == binding.ERR_ARG
    assert call(batch=0) == binding.OK
    assert call(h=0) == binding.ERR_NULL
    assert call(db=0) == binding.ERR_NULL
    assert call(h=H + 8) == binding.ERR_ALIGN                                   # state needs 16 bytes
    assert call(al=Al + 2) == binding.ERR_ALIGN
    assert call(out=Xb + 16) == binding.ERR_ALIAS
    assert call(out=H + 64) == binding.ERR_ALIAS
    assert call(xbc=H + 128) == binding.ERR_ALIAS                                # xbc inside the state
    assert call(out=Dp) == binding.ERR_ALIAS                                     # out over D


def test_in_proj_rejections():
    F = FAKE
    A, Wn, Wq, S, St, Cw, Cb, O = (F + (i << 30) for i in range(8))
    ip = binding.gemv_in_proj_raw
    # gemv_in_proj(A, norm_weight, eps, Wq, scale, conv_state, conv_weight, conv_bias, begin, dim, d_conv, out, M, N, K)
    assert ip(A, Wn, 1e-5, Wq, S, St, Cw, Cb, 100, 200, 4, O, 1, 256, 256, 0) == binding.ERR_SHAPE   # past N
    assert ip(A, Wn, 1e-5, Wq, S, St, Cw, Cb, 0, 0, 4, O, 1, 256, 256, 0) == binding.ERR_SHAPE      # no columns
    assert ip(A, Wn, 1e-5, Wq, S, St, Cw, Cb, 0, 64, 9, O, 1, 256, 256, 0) == binding.ERR_SHAPE     # d_conv > 8
    assert ip(A, Wn, float("nan"), Wq, S, St, Cw, Cb, 0, 64, 4, O, 1, 256, 256, 0) == binding.ERR_ARG
    assert ip(A, Wn, 1e-5, Wq, S, St, Cw, Cb, 0, 64, 4, O, 9, 256, 256, 0) == binding.ERR_SHAPE     # M > 8
    assert ip(A, Wn, 1e-5, Wq, S, St, Cw, Cb, 0, 64, 4, O, 0, 256, 256, 0) == binding.OK            # no-op
    assert ip(A, 0, 1e-5, Wq, S, St, Cw, Cb, 0, 64, 4, O, 1, 256, 256, 0) == binding.ERR_NULL
    assert ip(A, Wn, 1e-5, Wq, S, 0, Cw, Cb, 0, 64, 4, O, 1, 256, 256, 0) == binding.ERR_NULL
    assert ip(A, Wn, 1e-5, Wq, S, St + 2, Cw, Cb, 0, 64, 4, O, 1, 256, 256, 0) == binding.ERR_ALIGN
    assert ip(A, Wn + 8, 1e-5, Wq, S, St, Cw, Cb, 0, 64, 4, O, 1, 256, 256, 0) == binding.ERR_ALIGN
    assert ip(A, Wn, 1e-5, Wq, S, O + 64, Cw, Cb, 0, 64, 4, O, 1, 256, 256, 0) == binding.ERR_ALIAS  # state in out
    assert ip(A, Wn, 1e-5, Wq, S, St, Cw, Cb, 0, 64, 4, Cw - 64, 1, 256, 256, 0) == binding.ERR_ALIAS
    assert ip(A, Wn, 1e-5, Wq, S, A + 16, Cw, Cb, 0, 64, 4, O, 1, 256, 256, 0) == binding.ERR_ALIAS   # state over A


def test_gemm_workspace_size_follows_the_split_schedule():
    """Host-only: which shapes split their tiles (and need a workspace) on a
    256-CU device; computed from M, N, K and the CU count, nothing launched."""
    ws = binding.gemm_workspace_size
    assert ws(-1, 256, 256) == binding.ERR_SHAPE
    assert ws(4, 256, 136) == binding.ERR_SHAPE
    assert ws(0, 4096, 8192) == 0
    assert ws(8, 18560, 4096) == 0                      # skinny kernel: no split
    assert ws(1024, 18560, 4096) == 0                   # whole 128 x 128 tiles
    assert ws(1024, 4096, 8192) == 0                    # k split inside the workgroup
    assert ws(8192, 35072, 8192) == 0                   # 256 x 256 tiles
    need = ws(512, 4096, 8192)                          # 128 tiles of 128 x 128 on 512 slots
    assert need > 0 and need % (128 * 128 * 4) == 0
    assert ws(16, 4096, 8192) == 0                      # one-shot skinny kernel (every weight block on a CU)
    for m in (17, 32, 128, 256):                        # mid-size kernel: K split inside the workgroup
        assert ws(m, 4096, 8192) == 0 and ws(m, 18560, 4096) == 0
    assert ws(32, 18560, 40960) > 0                     # K past the mid-size kernel: 145 tiles of 32 x 128
    assert ws(384, 18560, 4096) == 64 << 20             # 435 tiles of 128 x 128 cut over 512 workgroups


def test_gemm_ws_rejections_before_any_hip_call():
    A, Wq, scale, out = FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30)
    M, N, K = 512, 4096, 8192
    need = binding.gemm_workspace_size(M, N, K)
    assert need > 0
    wsp = FAKE + (4 << 30)
    call = binding.gemm_ws_raw
    assert call(A, Wq, scale, out, M, N, K, wsp + 16, need, 0) == binding.ERR_ALIGN
    assert call(A, Wq, scale, out, M, N, K, wsp, need - 1, 0) == binding.ERR_WORKSPACE
    assert call(A, Wq, scale, out, M, N, K, wsp, -1, 0) == binding.ERR_ARG
    assert call(A, Wq, scale, out, M, N, K, out, need, 0) == binding.ERR_ALIAS
    assert call(A, Wq, scale, out, M, N, 136, wsp, need, 0) == binding.ERR_SHAPE
    assert call(A, Wq, scale, out, 0, N, K, wsp, 0, 0) == binding.OK        # no-op


def test_gemm_noalloc_scratch_and_rejections_before_any_hip_call():
    # 64 MiB: two 128 x 128 fp32 partial tiles for each of 512 workgroups,
    # the largest split schedule on a 256-CU device
    assert binding.gemm_noalloc_scratch_bytes() == 64 << 20
    for M, N, K in ((32, 18560, 40960), (512, 4096, 8192), (384, 18560, 4096), (300, 1000, 1040)):
        assert 0 < binding.gemm_workspace_size(M, N, K) <= binding.gemm_noalloc_scratch_bytes()
    A, Wq, scale, out = FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30)
    call = binding.gemm_noalloc_raw
    assert call(A, Wq, scale, out, 128, 4096, 136, 0) == binding.ERR_SHAPE
    assert call(A, Wq, scale, out, -1, 4096, 8192, 0) == binding.ERR_SHAPE
    assert call(0, Wq, scale, out, 128, 4096, 8192, 0) == binding.ERR_NULL
    assert call(A + 2, Wq, scale, out, 128, 4096, 8192, 0) == binding.ERR_ALIGN
    assert call(A, Wq, scale, A, 128, 4096, 8192, 0) == binding.ERR_ALIAS
    assert call(A, Wq, scale, out, 0, 4096, 8192, 0) == binding.OK          # no-op


def test_hbm_read_rejections_before_any_hip_call():
    call = binding.hbm_read_raw
    assert call(FAKE, 100, 256, 8, FAKE + (1 << 30), 0) == binding.ERR_SHAPE          # not a multiple of 16
    assert call(FAKE, (1 << 31) + 16, 256, 8, FAKE + (1 << 30), 0) == binding.ERR_SHAPE
    assert call(FAKE, -16, 256, 8, FAKE + (1 << 30), 0) == binding.ERR_SHAPE
    assert call(FAKE, 1 << 20, 96, 8, FAKE + (1 << 30), 0) == binding.ERR_ARG
    assert call(FAKE, 1 << 20, 256, 3, FAKE + (1 << 30), 0) == binding.ERR_ARG
    assert call(0, 1 << 20, 256, 8, FAKE + (1 << 30), 0) == binding.ERR_NULL
    assert call(FAKE + 8, 1 << 20, 256, 8, FAKE + (1 << 30), 0) == binding.ERR_ALIGN
    assert call(FAKE, 0, 256, 8, 0, 0) == binding.OK                                 # no-op
