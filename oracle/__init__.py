"""CPU oracle for the w8a16 block-scaled FP8 projection (test infrastructure).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The GPU library does
not import it and shares no code with it.

The arithmetic lives in ``w8a16_oracle.c`` (plain C, fp64, closed-form E4M3
decode); this module compiles it with gcc and marshals numpy arrays into it.
The operation is the one the Qwen3SsmLayer docs give for the w8a16 GEMV
(``set_fp8_decode_weights``), with the block-scale index of the
NemotronMamba2Layer docs (``set_fp8_weights``):

    out[m, n] = sum_k A[m, k] * E4M3(W[n, k]) * S[n // 128, k // 128]

Arrays are raw bit patterns: A and S are ``uint16`` BF16 bits, W is ``uint8``
E4M3 codes. Results are fp64.

Scale formats (``fmt``): ``"block_bf16"`` (S as above), ``"block_f32"`` (S a
``float32`` grid of the same shape; nemotron_mamba2.rs listing,
``set_fp8_weights``) and ``"row_f32"`` (S a ``float32`` [N] vector, one scale
per weight row; Qwen3SsmLayer docs, ``set_fp8_rowwise_prefill_weights``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w8a16_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_w8a16.so")
BLOCK = 128
FORMATS = {"block_bf16": 0, "block_f32": 1, "row_f32": 2}

_lib = None


def build() -> str:
    """Compile the oracle with gcc (OpenMP over independent output elements)."""
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
           _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_bf16_value.restype = ctypes.c_double
    lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_rne.restype = ctypes.c_uint16
    lib.oracle_bf16_rne.argtypes = [ctypes.c_double]
    for name in ("oracle_e4m3_values", "oracle_bf16_values", "oracle_bf16_rne_array"):
        getattr(lib, name).restype = None
        getattr(lib, name).argtypes = [P, I64, P]
    lib.oracle_dequant.restype = None
    lib.oracle_dequant.argtypes = [P, P, I64, I64, P]
    lib.oracle_w8a16.restype = None
    lib.oracle_w8a16.argtypes = [P, P, P, I64, I64, I64, P, P]
    lib.oracle_w8a16_points.restype = None
    lib.oracle_w8a16_points.argtypes = [P, P, P, I64, I64, I64, P, P, I64, P, P]
    C = ctypes.c_int
    lib.oracle_dequant_fmt.restype = None
    lib.oracle_dequant_fmt.argtypes = [P, P, C, I64, I64, P]
    lib.oracle_w8a16_fmt.restype = None
    lib.oracle_w8a16_fmt.argtypes = [P, P, P, C, I64, I64, I64, P, P]
    lib.oracle_w8a16_points_fmt.restype = None
    lib.oracle_w8a16_points_fmt.argtypes = [P, P, P, C, I64, I64, I64, P, P, I64, P, P]
    lib.oracle_silu.restype = ctypes.c_double
    lib.oracle_silu.argtypes = [ctypes.c_double]
    lib.oracle_rmsnorm.restype = None
    lib.oracle_rmsnorm.argtypes = [P, P, P, ctypes.c_double, I64, I64, I64, P, P]
    lib.oracle_residual_add.restype = None
    lib.oracle_residual_add.argtypes = [P, P, I64, P]
    D = ctypes.c_double
    lib.oracle_conv1d_update.restype = None
    lib.oracle_conv1d_update.argtypes = [P, P, I64, P, P, I64, I64, I64, P, P]
    lib.oracle_softplus.restype = D
    lib.oracle_softplus.argtypes = [D]
    lib.oracle_ssm_decode.restype = None
    lib.oracle_ssm_decode.argtypes = [P, P, I64, P, I64, P, P, P, I64, I64, I64, I64, I64, D, D, P, P, P]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return np.ascontiguousarray(a)


def scale_grid(N: int, K: int) -> tuple[int, int]:
    """Shape of the block-scale grid: [ceil(N/128), ceil(K/128)]."""
    return ((N + BLOCK - 1) // BLOCK, (K + BLOCK - 1) // BLOCK)


def _check_scales(S, fmt: str, N: int, K: int) -> np.ndarray:
    if fmt not in FORMATS:
        raise ValueError(f"unknown scale format {fmt!r}")
    S = _c(S, np.uint16 if fmt == "block_bf16" else np.float32)
    want = (N,) if fmt == "row_f32" else scale_grid(N, K)
    if S.shape != want:
        raise ValueError(f"{fmt} scales must have shape {want}, got {S.shape}")
    return S


def _check_operands(A, W, S, fmt="block_bf16"):
    A = _c(A, np.uint16)
    W = _c(W, np.uint8)
    if A.ndim != 2 or W.ndim != 2:
        raise ValueError("A and W must be 2-D")
    M, K = A.shape
    N, K2 = W.shape
    if K2 != K:
        raise ValueError(f"A is [{M},{K}] but W is [{N},{K2}]")
    S = _check_scales(S, fmt, N, K)
    return A, W, S, M, N, K


def e4m3_value(codes) -> np.ndarray:
    """Closed-form E4M3 decode of each byte (NaN for 0x7F / 0xFF)."""
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().oracle_e4m3_values(_ptr(c), c.size, _ptr(out))
    return out


def bf16_value(bits) -> np.ndarray:
    """Exact value of each BF16 bit pattern."""
    b = _c(bits, np.uint16)
    out = np.empty(b.shape, np.float64)
    _load().oracle_bf16_values(_ptr(b), b.size, _ptr(out))
    return out


def bf16_rne(x) -> np.ndarray:
    """BF16 bit pattern nearest each fp64 value (ties to even)."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(a.shape, np.uint16)
    _load().oracle_bf16_rne_array(_ptr(a), a.size, _ptr(out))
    return out


def dequant(W, S, fmt: str = "block_bf16") -> np.ndarray:
    """Wdeq[n, k] = E4M3(W[n, k]) * its scale, in fp64 (exact).

    The scale is S[n//128, k//128] for the block formats, S[n] for row_f32."""
    W = _c(W, np.uint8)
    N, K = W.shape
    S = _check_scales(S, fmt, N, K)
    out = np.empty((N, K), np.float64)
    if fmt == "block_bf16":
        _load().oracle_dequant(_ptr(W), _ptr(S), N, K, _ptr(out))
    else:
        _load().oracle_dequant_fmt(_ptr(W), _ptr(S), FORMATS[fmt], N, K, _ptr(out))
    return out


def w8a16(A, W, S, fmt: str = "block_bf16") -> tuple[np.ndarray, np.ndarray]:
    """Whole result: (ref, den), each [M, N] fp64.

    ref[m, n] = sum_k A[m,k] * Wdeq[n,k] (k ascending, fp64);
    den[m, n] = sum_k |A[m,k] * Wdeq[n,k]|.
    """
    A, W, S, M, N, K = _check_operands(A, W, S, fmt)
    ref = np.empty((M, N), np.float64)
    den = np.empty((M, N), np.float64)
    if fmt == "block_bf16":
        _load().oracle_w8a16(_ptr(A), _ptr(W), _ptr(S), M, N, K, _ptr(ref), _ptr(den))
    else:
        _load().oracle_w8a16_fmt(_ptr(A), _ptr(W), _ptr(S), FORMATS[fmt], M, N, K, _ptr(ref), _ptr(den))
    return ref, den


def w8a16_points(A, W, S, mi, ni, fmt: str = "block_bf16") -> tuple[np.ndarray, np.ndarray]:
    """(ref, den) at the listed output coordinates (mi[p], ni[p])."""
    A, W, S, M, N, K = _check_operands(A, W, S, fmt)
    mi = np.ascontiguousarray(np.asarray(mi, dtype=np.int64))
    ni = np.ascontiguousarray(np.asarray(ni, dtype=np.int64))
    if mi.shape != ni.shape or mi.ndim != 1:
        raise ValueError("mi and ni must be 1-D and of equal length")
    if mi.size and (mi.min() < 0 or mi.max() >= M or ni.min() < 0 or ni.max() >= N):
        raise IndexError("output coordinate out of range")
    ref = np.empty(mi.size, np.float64)
    den = np.empty(mi.size, np.float64)
    if fmt == "block_bf16":
        _load().oracle_w8a16_points(_ptr(A), _ptr(W), _ptr(S), M, N, K,
                                    _ptr(mi), _ptr(ni), mi.size, _ptr(ref), _ptr(den))
    else:
        _load().oracle_w8a16_points_fmt(_ptr(A), _ptr(W), _ptr(S), FORMATS[fmt], M, N, K,
                                        _ptr(mi), _ptr(ni), mi.size, _ptr(ref), _ptr(den))
    return ref, den


def silu(z: float) -> float:
    """z / (1 + exp(-z)) in fp64."""
    return float(_load().oracle_silu(float(z)))


def rmsnorm(x, weight, eps: float, gate=None, group=None) -> tuple[np.ndarray, np.ndarray]:
    """RMSNorm of BF16 x [M, K] times BF16 weight [K] (times silu(gate)), over
    consecutive groups of `group` channels of each row (None: the whole row).

    Returns (exact fp64 values [M, K], their BF16 bits [M, K])
    (nemotron_mamba2.rs module docs, forward steps 1 and 6)."""
    x = _c(x, np.uint16)
    w = _c(weight, np.uint16)
    if x.ndim != 2 or w.shape != (x.shape[1],):
        raise ValueError(f"x must be [M, K] and weight [K], got {x.shape} and {w.shape}")
    G = x.shape[1] if group is None else int(group)
    if G < 1 or x.shape[1] % G != 0:
        raise ValueError(f"group must divide K = {x.shape[1]}, got {group}")
    g = None
    if gate is not None:
        g = _c(gate, np.uint16)
        if g.shape != x.shape:
            raise ValueError(f"gate must match x {x.shape}, got {g.shape}")
    M, K = x.shape
    exact = np.empty((M, K), np.float64)
    bits = np.empty((M, K), np.uint16)
    _load().oracle_rmsnorm(_ptr(x), _ptr(g) if g is not None else None, _ptr(w), float(eps), G, M, K,
                           _ptr(exact), _ptr(bits))
    return exact, bits


def residual_add(residual, ref) -> np.ndarray:
    """BF16 bits of residual + bf16(ref): the residual add after the projection."""
    r = _c(residual, np.uint16)
    f = np.ascontiguousarray(np.asarray(ref, dtype=np.float64))
    if r.shape != f.shape:
        raise ValueError(f"residual {r.shape} and ref {f.shape} differ")
    out = np.empty(r.shape, np.uint16)
    _load().oracle_residual_add(_ptr(r), _ptr(f), r.size, _ptr(out))
    return out


def softplus(v: float) -> float:
    """log(1 + e^v) in fp64."""
    return float(_load().oracle_softplus(float(v)))


def conv1d_update(state, x, weight, bias, ld_x: int | None = None):
    """One conv1d update step (nemotron_mamba2.rs module docs, forward step 3).

    state: float64 [B, dim, d_conv], updated in place (oldest input first);
    x: BF16 bits [B, ld_x] (the first dim channels are used); weight: BF16
    [dim, d_conv]; bias: BF16 [dim]. Returns (exact fp64 [B, dim], BF16 bits)."""
    if not (isinstance(state, np.ndarray) and state.dtype == np.float64 and state.flags.c_contiguous
            and state.ndim == 3):
        raise TypeError("state must be a C-contiguous float64 [B, dim, d_conv] array (updated in place)")
    Bn, dim, d_conv = state.shape
    x = _c(x, np.uint16)
    w = _c(weight, np.uint16)
    bi = _c(bias, np.uint16)
    ld = x.shape[1] if ld_x is None else ld_x
    if x.ndim != 2 or x.shape[0] != Bn or x.shape[1] < dim or ld != x.shape[1]:
        raise ValueError(f"x must be [B, >= dim] with ld_x its row length, got {x.shape} (ld_x {ld})")
    if w.shape != (dim, d_conv) or bi.shape != (dim,):
        raise ValueError(f"weight must be {(dim, d_conv)} and bias {(dim,)}, got {w.shape}, {bi.shape}")
    exact = np.empty((Bn, dim), np.float64)
    bits = np.empty((Bn, dim), np.uint16)
    _load().oracle_conv1d_update(_ptr(state), _ptr(x), ld, _ptr(w), _ptr(bi), Bn, dim, d_conv,
                                 _ptr(exact), _ptr(bits))
    return exact, bits


def ssm_decode(hstate, xbc, dt_raw, a_log, d_param, dt_bias, groups: int, dt_min: float = 1e-9,
               dt_max: float = 1e9):
    """One Mamba-2 SSM decode step (nemotron_mamba2.rs module docs, forward
    steps 4 and 5; `ssm_decode` argument list).

    hstate: float64 [B, heads, head_dim, state], updated in place; xbc: BF16
    bits [B, ld] holding x | B | C from column 0; dt_raw: BF16 bits [B, >=
    heads]; a_log, d_param, dt_bias: float32 [heads]. Returns (y exact fp64
    [B, heads*head_dim], y BF16 bits, den)."""
    if not (isinstance(hstate, np.ndarray) and hstate.dtype == np.float64 and hstate.flags.c_contiguous
            and hstate.ndim == 4):
        raise TypeError("hstate must be a C-contiguous float64 [B, heads, head_dim, state] array")
    Bn, heads, hd, st = hstate.shape
    if groups < 1 or heads % groups:
        raise ValueError(f"heads ({heads}) must be a multiple of groups ({groups})")
    xbc = _c(xbc, np.uint16)
    dt = _c(dt_raw, np.uint16)
    need = heads * hd + 2 * groups * st
    if xbc.ndim != 2 or xbc.shape[0] != Bn or xbc.shape[1] < need:
        raise ValueError(f"xbc must be [B, >= {need}], got {xbc.shape}")
    if dt.ndim != 2 or dt.shape[0] != Bn or dt.shape[1] < heads:
        raise ValueError(f"dt_raw must be [B, >= {heads}], got {dt.shape}")
    al, dp, db = (_c(v, np.float32) for v in (a_log, d_param, dt_bias))
    if al.shape != (heads,) or dp.shape != (heads,) or db.shape != (heads,):
        raise ValueError("a_log, d_param and dt_bias must be float32 [heads]")
    y = np.empty((Bn, heads * hd), np.float64)
    bits = np.empty((Bn, heads * hd), np.uint16)
    den = np.empty((Bn, heads * hd), np.float64)
    _load().oracle_ssm_decode(_ptr(hstate), _ptr(xbc), xbc.shape[1], _ptr(dt), dt.shape[1], _ptr(al), _ptr(dp),
                              _ptr(db), Bn, heads, hd, st, groups, float(dt_min), float(dt_max),
                              _ptr(y), _ptr(bits), _ptr(den))
    return y, bits, den


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())
