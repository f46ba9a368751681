"""Python binding of libw8a16.so: argument marshalling only.

Every function here checks torch tensors (dtype, shape, contiguity, device),
then calls the C ABI declared in ``include/w8a16.h`` on the current torch HIP
stream. All arithmetic runs in the HIP kernels; there is no fallback path, and
a missing library raises.

Scale formats (``scale_format``; by default taken from the scale tensor):

* ``"block_bf16"`` - [ceil(N/128), ceil(K/128)] BF16 grid (NemotronMamba2Layer
  docs, ``set_fp8_weights``);
* ``"block_f32"``  - the same grid in FP32 (nemotron_mamba2.rs listing,
  ``set_fp8_weights``, which takes an f32 scale grid);
* ``"row_f32"``    - one FP32 scale per weight row, [N] (Qwen3SsmLayer docs,
  ``set_fp8_rowwise_prefill_weights``).

The layout check mirrors those pages: a scale tensor of the wrong shape would
be read past its end inside the kernel, and the Qwen3SsmLayer docs note that
a mix-up between the block and per-row formats is only caught by an explicit
check, so the format must agree with the tensor's dtype and shape exactly.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libw8a16.so")
BLOCK = 128

EXPORTS = ("w8a16_gemv", "w8a16_gemm", "w8a16_gemv_ex", "w8a16_gemm_ex", "w8a16_gemm_workspace_size",
           "w8a16_gemm_ws", "w8a16_rmsnorm", "w8a16_gemv_fused", "w8a16_gemm_residual", "w8a16_conv1d_update",
           "w8a16_gemv_in_proj", "w8a16_ssm_decode", "w8a16_dequant", "w8a16_strerror",
           "w8a16_gemm_noalloc", "w8a16_gemm_noalloc_scratch_bytes", "w8a16_hbm_read")

# enum w8a16_scale_format
SCALE_BLOCK_BF16, SCALE_BLOCK_F32, SCALE_ROW_F32 = 0, 1, 2
SCALE_FORMATS = {"block_bf16": SCALE_BLOCK_BF16, "block_f32": SCALE_BLOCK_F32, "row_f32": SCALE_ROW_F32}

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_LAUNCH, ERR_ALIAS, ERR_ARG, ERR_WORKSPACE = 0, -1, -2, -3, -4, -5, -6, -7
ERR_SCRATCH = -8
WORKSPACE_ALIGN = 256
GEMV_MAX_M = 16
GEMV_MAX_K_SMALL_M = 16384   # M <= 8
GEMV_MAX_K = 8192            # M >= 9
FUSED_MAX_M = 8              # w8a16_gemv_fused: M <= 4 with K <= 16384, M <= 8 with K <= 8192
FUSED_MAX_M_LONG_K = 4

_lib = None


class W8A16Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed with status {status}: {strerror(status)}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libw8a16.so (built in-tree); raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m gemm_mamba_ssm_amd.build` "
            "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    for name in ("w8a16_gemv", "w8a16_gemm"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [P, P, P, P, I64, I64, I64, P]
    for name in ("w8a16_gemv_ex", "w8a16_gemm_ex"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [P, P, P, ctypes.c_int, P, I64, I64, I64, P]
    lib.w8a16_gemm_workspace_size.restype = I64
    lib.w8a16_gemm_workspace_size.argtypes = [I64, I64, I64]
    lib.w8a16_gemm_ws.restype = ctypes.c_int
    lib.w8a16_gemm_ws.argtypes = [P, P, P, P, I64, I64, I64, P, I64, P]
    lib.w8a16_gemm_noalloc.restype = ctypes.c_int
    lib.w8a16_gemm_noalloc.argtypes = [P, P, P, P, I64, I64, I64, P]
    lib.w8a16_gemm_noalloc_scratch_bytes.restype = I64
    lib.w8a16_gemm_noalloc_scratch_bytes.argtypes = []
    lib.w8a16_hbm_read.restype = ctypes.c_int
    lib.w8a16_hbm_read.argtypes = [P, I64, ctypes.c_int, ctypes.c_int, P, P]
    F = ctypes.c_float
    lib.w8a16_rmsnorm.restype = ctypes.c_int
    lib.w8a16_rmsnorm.argtypes = [P, P, P, F, I64, P, I64, I64, P]
    lib.w8a16_gemv_fused.restype = ctypes.c_int
    lib.w8a16_gemv_fused.argtypes = [P, P, I64, P, F, I64, P, P, P, P, I64, I64, I64, P]
    lib.w8a16_gemm_residual.restype = ctypes.c_int
    lib.w8a16_gemm_residual.argtypes = [P, P, P, P, P, I64, I64, I64, P]
    lib.w8a16_conv1d_update.restype = ctypes.c_int
    lib.w8a16_conv1d_update.argtypes = [P, P, I64, P, P, P, I64, I64, I64, I64, P]
    lib.w8a16_gemv_in_proj.restype = ctypes.c_int
    lib.w8a16_gemv_in_proj.argtypes = [P, P, F, P, P, P, P, P, I64, I64, I64, P, I64, I64, I64, P]
    lib.w8a16_ssm_decode.restype = ctypes.c_int
    lib.w8a16_ssm_decode.argtypes = [P, P, I64, P, I64, P, P, P, P, I64, I64, I64, I64, I64, I64, F, F, P]
    lib.w8a16_dequant.restype = ctypes.c_int
    lib.w8a16_dequant.argtypes = [P, P, P, I64, I64, P]
    lib.w8a16_strerror.restype = ctypes.c_char_p
    lib.w8a16_strerror.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load().w8a16_strerror(int(status)).decode()


# --- raw pointer calls (integers in, status out) ------------------------------

def gemv_raw(A: int, Wq: int, scale: int, out: int, M: int, N: int, K: int, stream: int = 0) -> int:
    return load().w8a16_gemv(A, Wq, scale, out, M, N, K, stream)


def gemm_raw(A: int, Wq: int, scale: int, out: int, M: int, N: int, K: int, stream: int = 0) -> int:
    return load().w8a16_gemm(A, Wq, scale, out, M, N, K, stream)


def gemm_workspace_size(M: int, N: int, K: int) -> int:
    """Bytes of workspace w8a16_gemm_ws needs for (M, N, K) on the current device (0: none)."""
    return load().w8a16_gemm_workspace_size(M, N, K)


def gemm_ws_raw(A: int, Wq: int, scale: int, out: int, M: int, N: int, K: int, workspace: int,
                workspace_bytes: int, stream: int = 0) -> int:
    return load().w8a16_gemm_ws(A, Wq, scale, out, M, N, K, workspace or None, workspace_bytes, stream)


def gemm_noalloc_raw(A: int, Wq: int, scale: int, out: int, M: int, N: int, K: int, stream: int = 0) -> int:
    return load().w8a16_gemm_noalloc(A, Wq, scale, out, M, N, K, stream)


def gemm_noalloc_scratch_bytes() -> int:
    """Bytes of the library's static scratch that w8a16_gemm_noalloc uses per GPU."""
    return load().w8a16_gemm_noalloc_scratch_bytes()


def hbm_read_raw(buf: int, nbytes: int, threads: int, loads: int, sink: int, stream: int = 0) -> int:
    """Plain read of nbytes at buf (the HBM floor the GEMV is compared against); writes nothing."""
    return load().w8a16_hbm_read(buf, nbytes, threads, loads, sink, stream)


def gemv_ex_raw(A: int, Wq: int, scale: int, scale_format: int, out: int, M: int, N: int, K: int,
                stream: int = 0) -> int:
    return load().w8a16_gemv_ex(A, Wq, scale, scale_format, out, M, N, K, stream)


def gemm_ex_raw(A: int, Wq: int, scale: int, scale_format: int, out: int, M: int, N: int, K: int,
                stream: int = 0) -> int:
    return load().w8a16_gemm_ex(A, Wq, scale, scale_format, out, M, N, K, stream)


def rmsnorm_raw(x: int, gate: int, weight: int, eps: float, out: int, M: int, K: int, stream: int = 0,
                group: int = 0) -> int:
    return load().w8a16_rmsnorm(x, gate or None, weight, eps, group, out, M, K, stream)


def gemv_fused_raw(A: int, gate: int, norm_weight: int, eps: float, Wq: int, scale: int, residual: int,
                   out: int, M: int, N: int, K: int, stream: int = 0, ld_gate: int | None = None,
                   group: int = 0) -> int:
    return load().w8a16_gemv_fused(A, gate or None, K if ld_gate is None else ld_gate, norm_weight or None, eps,
                                   group, Wq, scale, residual or None, out, M, N, K, stream)


def gemm_residual_raw(A: int, Wq: int, scale: int, residual: int, out: int, M: int, N: int, K: int,
                      stream: int = 0) -> int:
    return load().w8a16_gemm_residual(A, Wq, scale, residual, out, M, N, K, stream)


def conv1d_update_raw(conv_state: int, x: int, ld_x: int, weight: int, bias: int, out: int, ld_out: int,
                      batch: int, dim: int, d_conv: int, stream: int = 0) -> int:
    return load().w8a16_conv1d_update(conv_state, x, ld_x, weight, bias, out, ld_out, batch, dim, d_conv, stream)


def gemv_in_proj_raw(A: int, norm_weight: int, eps: float, Wq: int, scale: int, conv_state: int, conv_weight: int,
                     conv_bias: int, conv_begin: int, conv_dim: int, d_conv: int, out: int, M: int, N: int, K: int,
                     stream: int = 0) -> int:
    return load().w8a16_gemv_in_proj(A, norm_weight, eps, Wq, scale, conv_state, conv_weight, conv_bias,
                                     conv_begin, conv_dim, d_conv, out, M, N, K, stream)


def ssm_decode_raw(h_state: int, xbc: int, ld_xbc: int, dt_raw: int, ld_dt: int, a_log: int, d_param: int,
                   dt_bias: int, out: int, ld_out: int, batch: int, heads: int, head_dim: int, state: int,
                   groups: int, dt_min: float, dt_max: float, stream: int = 0) -> int:
    return load().w8a16_ssm_decode(h_state, xbc, ld_xbc, dt_raw, ld_dt, a_log, d_param, dt_bias, out, ld_out,
                                   batch, heads, head_dim, state, groups, dt_min, dt_max, stream)


def dequant_raw(Wq: int, scale: int, out: int, N: int, K: int, stream: int = 0) -> int:
    return load().w8a16_dequant(Wq, scale, out, N, K, stream)


# --- torch tensors ------------------------------------------------------------

def scale_grid(N: int, K: int) -> tuple[int, int]:
    return ((N + BLOCK - 1) // BLOCK, (K + BLOCK - 1) // BLOCK)


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _check_codes(Wq: torch.Tensor) -> tuple[int, int]:
    _need(Wq.dtype in (torch.uint8, torch.float8_e4m3fn),
          f"Wq must hold E4M3 bytes (torch.uint8 or torch.float8_e4m3fn), got {Wq.dtype}")
    _need(Wq.dim() == 2, f"Wq must be [N, K], got shape {tuple(Wq.shape)}")
    N, K = Wq.shape
    _need(K >= 16 and K % 16 == 0, f"K must be a multiple of 16 and >= 16, got {K}")
    _need(Wq.is_contiguous(), "Wq must be contiguous (row-major [N, K])")
    return N, K


def _check_weights(Wq: torch.Tensor, scale: torch.Tensor) -> tuple[int, int]:
    """E4M3 codes with the BF16 block grid (the dequant path's only format)."""
    N, K = _check_codes(Wq)
    _need(scale.dtype == torch.bfloat16,
          f"scale must be the BF16 block-scale grid, got dtype {scale.dtype}")
    _need(tuple(scale.shape) == scale_grid(N, K),
          f"scale must be the [ceil(N/128), ceil(K/128)] = {list(scale_grid(N, K))} block grid, "
          f"got shape {list(scale.shape)} (per-row or scalar scales are a different format)")
    _need(scale.is_contiguous(), "scale must be contiguous (row-major by n-block)")
    return N, K


def scale_format_of(scale: torch.Tensor) -> str:
    """The format a scale tensor's dtype and rank stand for."""
    if scale.dtype == torch.bfloat16:
        return "block_bf16"
    if scale.dtype == torch.float32:
        return "row_f32" if scale.dim() == 1 else "block_f32"
    raise ValueError(f"scale must be bfloat16 (block grid) or float32 (block grid or per-row), got {scale.dtype}")


def _check_scaled_weights(Wq: torch.Tensor, scale: torch.Tensor, scale_format: str | None) -> tuple[int, int, int]:
    """(N, K, format code) for E4M3 codes and a scale tensor of any format."""
    N, K = _check_codes(Wq)
    fmt = scale_format_of(scale) if scale_format is None else scale_format
    _need(fmt in SCALE_FORMATS, f"unknown scale_format {fmt!r} (one of {sorted(SCALE_FORMATS)})")
    want_dtype = torch.bfloat16 if fmt == "block_bf16" else torch.float32
    want_shape = (N,) if fmt == "row_f32" else scale_grid(N, K)
    _need(scale.dtype == want_dtype and tuple(scale.shape) == want_shape,
          f"{fmt} scales must be a {want_dtype} tensor of shape {list(want_shape)}, "
          f"got {scale.dtype} {list(scale.shape)}")
    _need(scale.is_contiguous(), "scale must be contiguous")
    return N, K, SCALE_FORMATS[fmt]


def _check_device(*tensors: torch.Tensor):
    dev = tensors[0].device
    _need(dev.type == "cuda", f"tensors must be on a HIP device, got {dev}")
    for t in tensors[1:]:
        _need(t.device == dev, f"all tensors must be on {dev}, got {t.device}")


def _stream_handle(device: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream)


def _product(fn_name: str, A, Wq, scale, out, stream, max_m=None, scale_format=None):
    _need(A.dtype == torch.bfloat16, f"A must be bfloat16, got {A.dtype}")
    _need(A.dim() == 2, f"A must be [M, K], got shape {tuple(A.shape)}")
    N, K, fmt = _check_scaled_weights(Wq, scale, scale_format)
    M = A.shape[0]
    _need(A.shape[1] == K, f"A is {list(A.shape)} but Wq is {list(Wq.shape)}")
    _need(A.is_contiguous(), "A must be contiguous (row-major [M, K])")
    if max_m is not None:
        _need(M <= max_m, f"{fn_name} takes at most {max_m} rows, got M={M} (use w8a16_gemm)")
    if out is None:
        _check_device(A, Wq, scale)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    else:
        _need(out.dtype == torch.bfloat16 and tuple(out.shape) == (M, N) and out.is_contiguous(),
              f"out must be a contiguous bfloat16 [{M}, {N}] tensor")
        _check_device(A, Wq, scale, out)
    with torch.cuda.device(A.device):
        handle = _stream_handle(A.device, stream)
        if fmt == SCALE_BLOCK_BF16:
            st = getattr(load(), fn_name)(A.data_ptr(), Wq.data_ptr(), scale.data_ptr(), out.data_ptr(),
                                          M, N, K, handle)
        else:
            fn_name += "_ex"
            st = getattr(load(), fn_name)(A.data_ptr(), Wq.data_ptr(), scale.data_ptr(), fmt, out.data_ptr(),
                                          M, N, K, handle)
    if st != OK:
        raise W8A16Error(fn_name, st)
    return out


def w8a16_gemv(A: torch.Tensor, Wq: torch.Tensor, scale: torch.Tensor,
               out: torch.Tensor | None = None, stream=None, scale_format: str | None = None) -> torch.Tensor:
    """Decode GEMV, M = 1..16: out[M, N] = A[M, K] x dequant(Wq[N, K], scale)^T (BF16).

    ``scale`` is a BF16 or FP32 block grid or an FP32 per-row vector; see the
    module docstring for ``scale_format``."""
    return _product("w8a16_gemv", A, Wq, scale, out, stream, max_m=GEMV_MAX_M, scale_format=scale_format)


def w8a16_gemm(A: torch.Tensor, Wq: torch.Tensor, scale: torch.Tensor,
               out: torch.Tensor | None = None, stream=None, scale_format: str | None = None) -> torch.Tensor:
    """Prefill GEMM, any M: out[M, N] = A[M, K] x dequant(Wq[N, K], scale)^T (BF16).

    ``scale`` as for :func:`w8a16_gemv`."""
    return _product("w8a16_gemm", A, Wq, scale, out, stream, scale_format=scale_format)


def gemm_workspace(M: int, N: int, K: int, device=None) -> torch.Tensor | None:
    """A workspace tensor for w8a16_gemm_ws at (M, N, K) (None if the shape needs none).

    Allocated by torch here, once, by the caller's choice: the library itself
    allocates nothing."""
    device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    with torch.cuda.device(device):
        nbytes = gemm_workspace_size(M, N, K)
    if nbytes < 0:
        raise W8A16Error("w8a16_gemm_workspace_size", nbytes)
    if nbytes == 0:
        return None
    # torch's caching allocator returns 512-byte aligned blocks
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def w8a16_gemm_ws(A: torch.Tensor, Wq: torch.Tensor, scale: torch.Tensor, workspace: torch.Tensor | None,
                  out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The GEMM with a caller-supplied workspace (BF16 block grid): shapes whose
    tiles do not fill the GPU split their k-blocks between workgroups, the
    partial sums going through ``workspace`` (a uint8 device tensor of at
    least gemm_workspace_size(M, N, K) bytes; None runs w8a16_gemm)."""
    _need(A.dtype == torch.bfloat16 and A.dim() == 2 and A.is_contiguous(), "A must be a contiguous bfloat16 [M, K]")
    N, K, fmt = _check_scaled_weights(Wq, scale, "block_bf16")
    M = A.shape[0]
    _need(A.shape[1] == K, f"A is {list(A.shape)} but Wq is {list(Wq.shape)}")
    if workspace is not None:
        _need(workspace.dtype == torch.uint8 and workspace.is_contiguous(), "workspace must be a contiguous uint8 tensor")
        _check_device(A, workspace)
    if out is None:
        _check_device(A, Wq, scale)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    else:
        _need(out.dtype == torch.bfloat16 and tuple(out.shape) == (M, N) and out.is_contiguous(),
              f"out must be a contiguous bfloat16 [{M}, {N}] tensor")
        _check_device(A, Wq, scale, out)
    with torch.cuda.device(A.device):
        st = gemm_ws_raw(A.data_ptr(), Wq.data_ptr(), scale.data_ptr(), out.data_ptr(), M, N, K,
                         workspace.data_ptr() if workspace is not None else 0,
                         workspace.numel() if workspace is not None else 0, _stream_handle(A.device, stream))
    if st != OK:
        raise W8A16Error("w8a16_gemm_ws", st)
    return out


def w8a16_dequant(Wq: torch.Tensor, scale: torch.Tensor, out: torch.Tensor | None = None,
                  stream=None) -> torch.Tensor:
    """Dequantize only (test path): FP32 [N, K] = E4M3(Wq) * block scale, exact."""
    N, K = _check_weights(Wq, scale)
    if out is None:
        _check_device(Wq, scale)
        out = torch.empty((N, K), dtype=torch.float32, device=Wq.device)
    else:
        _need(out.dtype == torch.float32 and tuple(out.shape) == (N, K) and out.is_contiguous(),
              f"out must be a contiguous float32 [{N}, {K}] tensor")
        _check_device(Wq, scale, out)
    with torch.cuda.device(Wq.device):
        st = load().w8a16_dequant(Wq.data_ptr(), scale.data_ptr(), out.data_ptr(), N, K,
                                  _stream_handle(Wq.device, stream))
    if st != OK:
        raise W8A16Error("w8a16_dequant", st)
    return out


# --- norm prologues and the residual epilogue ----------------------------------
# (nemotron_mamba2.rs module docs, forward steps 1, 6 and 8.)

def _check_bf16(t: torch.Tensor, name: str, shape: tuple):
    _need(t.dtype == torch.bfloat16, f"{name} must be bfloat16, got {t.dtype}")
    _need(tuple(t.shape) == tuple(shape), f"{name} must be {list(shape)}, got {list(t.shape)}")
    _need(t.is_contiguous(), f"{name} must be contiguous")


def _eps(eps) -> float:
    e = float(eps)
    _need(e >= 0.0 and e < 3.0e38, f"eps must be finite and >= 0, got {eps}")
    return e


def _group(group, K: int) -> int:
    g = 0 if group is None else int(group)
    _need(g in (0, K) or (g > 0 and g % 1024 == 0 and K % g == 0 and K <= 16384),
          f"group must be K, or a multiple of 1024 dividing K <= 16384, got {group} for K = {K}")
    return g


def w8a16_rmsnorm(x: torch.Tensor, weight: torch.Tensor, eps: float, gate: torch.Tensor | None = None,
                  out: torch.Tensor | None = None, stream=None, group: int | None = None) -> torch.Tensor:
    """bf16(x * rsqrt(mean(x^2) + eps) * weight [* silu(gate)]) per row of x [M, K] (BF16), the mean
    over each group of `group` channels (None: the whole row)."""
    _need(x.dim() == 2, f"x must be [M, K], got shape {tuple(x.shape)}")
    M, K = x.shape
    grp = _group(group, K)
    _check_bf16(x, "x", (M, K))
    _check_bf16(weight, "weight", (K,))
    if gate is not None:
        _check_bf16(gate, "gate", (M, K))
    e = _eps(eps)
    if out is None:
        _check_device(*[t for t in (x, weight, gate) if t is not None])
        out = torch.empty((M, K), dtype=torch.bfloat16, device=x.device)
    else:
        _check_bf16(out, "out", (M, K))
        _check_device(*[t for t in (x, weight, gate, out) if t is not None])
    with torch.cuda.device(x.device):
        st = load().w8a16_rmsnorm(x.data_ptr(), gate.data_ptr() if gate is not None else None, weight.data_ptr(),
                                  e, grp, out.data_ptr(), M, K, _stream_handle(x.device, stream))
    if st != OK:
        raise W8A16Error("w8a16_rmsnorm", st)
    return out


def w8a16_gemv_fused(A: torch.Tensor, Wq: torch.Tensor, scale: torch.Tensor,
                     norm_weight: torch.Tensor | None = None, eps: float = 1e-5,
                     gate: torch.Tensor | None = None, residual: torch.Tensor | None = None,
                     out: torch.Tensor | None = None, stream=None, group: int | None = None) -> torch.Tensor:
    """Decode GEMV with the norm prologue (norm_weight, optional gate; the norm
    over groups of `group` channels, None: the whole row) and the residual
    epilogue fused: out = [residual +] (norm(A) x dequant(Wq)^T), BF16.
    The gate may be a column slice of a wider row-major tensor (z of the
    in_proj output), as long as its rows are contiguous and 16-byte aligned."""
    _need(A.dim() == 2, f"A must be [M, K], got shape {tuple(A.shape)}")
    N, K = _check_weights(Wq, scale)
    M = A.shape[0]
    _check_bf16(A, "A", (M, K))
    _need(gate is None or norm_weight is not None, "a gate needs a norm weight")
    if norm_weight is not None:
        _check_bf16(norm_weight, "norm_weight", (K,))
    ld_gate = K
    if gate is not None:
        ld_gate = _rows(gate, "gate", torch.bfloat16, M, K)
        _need(gate.shape[1] == K, f"gate must have K = {K} columns, got {gate.shape[1]}")
    if residual is not None:
        _check_bf16(residual, "residual", (M, N))
    e = _eps(eps)
    grp = _group(group, K) if norm_weight is not None else 0
    _need(M <= FUSED_MAX_M and (K <= GEMV_MAX_K if M > FUSED_MAX_M_LONG_K else K <= GEMV_MAX_K_SMALL_M),
          f"w8a16_gemv_fused takes M <= 4 with K <= {GEMV_MAX_K_SMALL_M} or M <= 8 with K <= {GEMV_MAX_K}, "
          f"got M={M}, K={K} (use w8a16_rmsnorm + w8a16_gemm_residual)")
    ins = [t for t in (A, Wq, scale, norm_weight, gate, residual) if t is not None]
    if out is None:
        _check_device(*ins)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    else:
        _check_bf16(out, "out", (M, N))
        _check_device(*ins, out)
    ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
    with torch.cuda.device(A.device):
        st = load().w8a16_gemv_fused(A.data_ptr(), ptr(gate), ld_gate, ptr(norm_weight), e, grp, Wq.data_ptr(),
                                     scale.data_ptr(), ptr(residual), out.data_ptr(), M, N, K,
                                     _stream_handle(A.device, stream))
    if st != OK:
        raise W8A16Error("w8a16_gemv_fused", st)
    return out


def w8a16_gemm_residual(A: torch.Tensor, Wq: torch.Tensor, scale: torch.Tensor, residual: torch.Tensor,
                        out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Prefill GEMM with the residual epilogue: out = bf16(residual + bf16(A x dequant(Wq)^T))."""
    _need(A.dim() == 2, f"A must be [M, K], got shape {tuple(A.shape)}")
    N, K = _check_weights(Wq, scale)
    M = A.shape[0]
    _check_bf16(A, "A", (M, K))
    _check_bf16(residual, "residual", (M, N))
    if out is None:
        _check_device(A, Wq, scale, residual)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    else:
        _check_bf16(out, "out", (M, N))
        _check_device(A, Wq, scale, residual, out)
    with torch.cuda.device(A.device):
        st = load().w8a16_gemm_residual(A.data_ptr(), Wq.data_ptr(), scale.data_ptr(), residual.data_ptr(),
                                        out.data_ptr(), M, N, K, _stream_handle(A.device, stream))
    if st != OK:
        raise W8A16Error("w8a16_gemm_residual", st)
    return out


# --- Mamba-2 decode step (forward steps 3 to 5) ----------------------------------

def _rows(t: torch.Tensor, name: str, dtype, batch: int, width: int) -> int:
    """Row stride of a [batch, >= width] tensor whose rows are contiguous."""
    _need(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    _need(t.dim() == 2 and t.shape[0] == batch and t.shape[1] >= width and t.stride(1) == 1,
          f"{name} must be [{batch}, >= {width}] with contiguous rows, got {list(t.shape)} strides {t.stride()}")
    return t.stride(0) if batch > 1 else t.shape[1]


def w8a16_conv1d_update(conv_state: torch.Tensor, x: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor,
                        out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """One conv1d update step: conv_state (float32 [B, dim, d_conv], updated in
    place) takes x [B, >= dim] (BF16 rows, e.g. a column slice of the in_proj
    output); returns bf16(silu(bias + sum_w state * weight)) [B, dim]."""
    _need(conv_state.dtype == torch.float32 and conv_state.dim() == 3 and conv_state.is_contiguous(),
          "conv_state must be a contiguous float32 [B, dim, d_conv] tensor")
    B, dim, d_conv = conv_state.shape
    ld_x = _rows(x, "x", torch.bfloat16, B, dim)
    _check_bf16(weight, "weight", (dim, d_conv))
    _check_bf16(bias, "bias", (dim,))
    if out is None:
        _check_device(conv_state, x, weight, bias)
        out = torch.empty((B, dim), dtype=torch.bfloat16, device=x.device)
    else:
        _check_device(conv_state, x, weight, bias, out)
    ld_out = _rows(out, "out", torch.bfloat16, B, dim)
    with torch.cuda.device(x.device):
        st = load().w8a16_conv1d_update(conv_state.data_ptr(), x.data_ptr(), ld_x, weight.data_ptr(),
                                        bias.data_ptr(), out.data_ptr(), ld_out, B, dim, d_conv,
                                        _stream_handle(x.device, stream))
    if st != OK:
        raise W8A16Error("w8a16_conv1d_update", st)
    return out


def w8a16_ssm_decode(h_state: torch.Tensor, xbc: torch.Tensor, dt_raw: torch.Tensor, a_log: torch.Tensor,
                     d_param: torch.Tensor, dt_bias: torch.Tensor, groups: int, dt_min: float = 1e-9,
                     dt_max: float = 1e9, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """One SSM decode step: h_state (float32 [B, heads, head_dim, state],
    updated in place), xbc = [x | B | C] rows (BF16 [B, >= width]), dt_raw
    (BF16 [B, >= heads]); returns y [B, heads * head_dim] (BF16)."""
    _need(h_state.dtype == torch.float32 and h_state.dim() == 4 and h_state.is_contiguous(),
          "h_state must be a contiguous float32 [B, heads, head_dim, state] tensor")
    B, heads, hd, st_ = h_state.shape
    _need(groups >= 1 and heads % groups == 0, f"heads ({heads}) must be a multiple of groups ({groups})")
    ld_x = _rows(xbc, "xbc", torch.bfloat16, B, heads * hd + 2 * groups * st_)
    ld_dt = _rows(dt_raw, "dt_raw", torch.bfloat16, B, heads)
    for t, name in ((a_log, "a_log"), (d_param, "d_param"), (dt_bias, "dt_bias")):
        _need(t.dtype == torch.float32 and tuple(t.shape) == (heads,) and t.is_contiguous(),
              f"{name} must be a contiguous float32 [{heads}] tensor")
    if out is None:
        _check_device(h_state, xbc, dt_raw, a_log, d_param, dt_bias)
        out = torch.empty((B, heads * hd), dtype=torch.bfloat16, device=xbc.device)
    else:
        _check_device(h_state, xbc, dt_raw, a_log, d_param, dt_bias, out)
    ld_out = _rows(out, "out", torch.bfloat16, B, heads * hd)
    with torch.cuda.device(xbc.device):
        st = load().w8a16_ssm_decode(h_state.data_ptr(), xbc.data_ptr(), ld_x, dt_raw.data_ptr(), ld_dt,
                                     a_log.data_ptr(), d_param.data_ptr(), dt_bias.data_ptr(), out.data_ptr(),
                                     ld_out, B, heads, hd, st_, groups, float(dt_min), float(dt_max),
                                     _stream_handle(xbc.device, stream))
    if st != OK:
        raise W8A16Error("w8a16_ssm_decode", st)
    return out


def w8a16_gemv_in_proj(x: torch.Tensor, Wq: torch.Tensor, scale: torch.Tensor, norm_weight: torch.Tensor,
                       eps: float, conv_state: torch.Tensor, conv_weight: torch.Tensor, conv_bias: torch.Tensor,
                       conv_begin: int, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The decode step's in_proj in one launch: RMSNorm of x, the projection,
    and the conv1d update applied in place to the output columns
    [conv_begin, conv_begin + dim) (conv_state float32 [M, dim, d_conv],
    updated). Returns out [M, N] (BF16)."""
    _need(x.dim() == 2, f"x must be [M, K], got shape {tuple(x.shape)}")
    N, K = _check_weights(Wq, scale)
    M = x.shape[0]
    _check_bf16(x, "x", (M, K))
    _check_bf16(norm_weight, "norm_weight", (K,))
    _need(conv_state.dtype == torch.float32 and conv_state.dim() == 3 and conv_state.is_contiguous()
          and conv_state.shape[0] == M, f"conv_state must be a contiguous float32 [{M}, dim, d_conv] tensor")
    dim, d_conv = conv_state.shape[1], conv_state.shape[2]
    _check_bf16(conv_weight, "conv_weight", (dim, d_conv))
    _check_bf16(conv_bias, "conv_bias", (dim,))
    _need(0 <= conv_begin and conv_begin + dim <= N, f"conv columns [{conv_begin}, {conv_begin + dim}) exceed N = {N}")
    e = _eps(eps)
    _need(M <= FUSED_MAX_M and (K <= GEMV_MAX_K if M > FUSED_MAX_M_LONG_K else K <= GEMV_MAX_K_SMALL_M),
          f"w8a16_gemv_in_proj takes M <= 4 with K <= {GEMV_MAX_K_SMALL_M} or M <= 8 with K <= {GEMV_MAX_K}")
    ins = [x, Wq, scale, norm_weight, conv_state, conv_weight, conv_bias]
    if out is None:
        _check_device(*ins)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    else:
        _check_bf16(out, "out", (M, N))
        _check_device(*ins, out)
    with torch.cuda.device(x.device):
        st = load().w8a16_gemv_in_proj(x.data_ptr(), norm_weight.data_ptr(), e, Wq.data_ptr(), scale.data_ptr(),
                                       conv_state.data_ptr(), conv_weight.data_ptr(), conv_bias.data_ptr(),
                                       conv_begin, dim, d_conv, out.data_ptr(), M, N, K,
                                       _stream_handle(x.device, stream))
    if st != OK:
        raise W8A16Error("w8a16_gemv_in_proj", st)
    return out
