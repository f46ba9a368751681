"""Seeded synthetic inputs for the w8a16 block-scaled FP8 projection.

This module only *makes* inputs; it holds none of the projection's own
arithmetic (no E4M3 decode, no product). Both the GPU path's tests and the CPU
oracle's tests draw from it, and it imports neither.

Recipe (the pages give no data; these stand in for the Mamba-2 layer's
in_proj / out_proj weights and activations):

* RNG: ``numpy.random.default_rng(seed)`` (PCG64), float32 standard normals.
* Activations A [M, K]: N(0, 1) rounded to BF16 (round-to-nearest-even).
* Weights: w [N, K] ~ N(0, sigma). For every 128x128 block (edge blocks may be
  partial), ``scale = bf16(max|w| / 448)``; the codes are the E4M3 values
  nearest (ties to even) to ``clamp(w / scale, -448, 448)``, with ``w / scale``
  taken against the BF16-rounded scale so that code * scale reproduces w. A
  block whose max is 0 gets scale 0 and all-zero codes. NaN codes (0x7F, 0xFF)
  never occur.

Encoding to E4M3 uses torch's ``float8_e4m3fn`` cast (OCP E4M3, saturating
input already clamped to +-448); the tests cross-check that cast against a
hand-written round-to-nearest-even encoder.

All arrays returned are raw bit patterns: A and scales as ``uint16`` BF16 bits,
weights as ``uint8`` E4M3 codes.

Norm inputs: the layer input, the gate z and the residual are drawn like A
(N(0, 1) rounded to BF16); a norm weight is ``1 + 0.1 * N(0, 1)`` rounded to
BF16; epsilon is ``NORM_EPS``.

Mamba-2 decode-step inputs (``MAMBA2_4K`` dimensions): the xBC row and dt_raw
are drawn like A; conv weights N(0, 0.5) and bias N(0, 0.1) in BF16; conv
states hold earlier BF16 inputs as float32; SSM states N(0, 0.1) float32;
``ssm_params`` draws a_log, D and dt_bias (float32) in the usual ranges.

The FP32 scale formats (``weights_fmt``) use the same draws; ``block_f32``
keeps ``max|w| / 448`` of each block in float32 (no BF16 rounding), and
``row_f32`` takes it over each whole weight row instead, as a float32 [N]
vector.
"""
from __future__ import annotations

import functools
import hashlib
from dataclasses import dataclass

import numpy as np
import torch

BLOCK = 128
E4M3_MAX = 448.0


def scale_grid(N: int, K: int) -> tuple[int, int]:
    return ((N + BLOCK - 1) // BLOCK, (K + BLOCK - 1) // BLOCK)


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def activations(M: int, K: int, seed: int) -> np.ndarray:
    """A [M, K] as BF16 bits: N(0, 1) float32 draws rounded to BF16."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    return _f32_to_bf16_bits(x)


def quantize_blocks(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Block-quantize float32 w [N, K] to (E4M3 codes [N, K], BF16 scale bits)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    nb, kb = scale_grid(N, K)
    pad = np.zeros((nb * BLOCK, kb * BLOCK), np.float32)
    pad[:N, :K] = w
    blocks = pad.reshape(nb, BLOCK, kb, BLOCK)
    amax = np.abs(blocks).max(axis=(1, 3))                  # [nb, kb] float32
    s_bits = _f32_to_bf16_bits(amax / np.float32(E4M3_MAX))  # float32 divide, then bf16
    s = _bf16_bits_to_f32(s_bits)
    codes = np.empty((N, K), np.uint8)
    for bi in range(nb):                                     # one row-band at a time (memory)
        r0, r1 = bi * BLOCK, min(N, (bi + 1) * BLOCK)
        s_cols = np.repeat(s[bi], BLOCK)[:K]                  # [K] scale per column
        safe = np.where(s_cols == 0, np.float32(1), s_cols)
        q = w[r0:r1] / safe[None, :]
        q = np.where(s_cols[None, :] == 0, np.float32(0), q)
        q = np.clip(q, -E4M3_MAX, E4M3_MAX).astype(np.float32)
        codes[r0:r1] = (torch.from_numpy(q).to(torch.float8_e4m3fn)
                        .view(torch.uint8).numpy())
    return codes, s_bits


def _encode_e4m3(q: np.ndarray) -> np.ndarray:
    q = np.clip(q, -E4M3_MAX, E4M3_MAX).astype(np.float32)
    return torch.from_numpy(np.ascontiguousarray(q)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def quantize_blocks_f32(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Block-quantize float32 w [N, K] to (E4M3 codes, float32 scale grid)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    nb, kb = scale_grid(N, K)
    pad = np.zeros((nb * BLOCK, kb * BLOCK), np.float32)
    pad[:N, :K] = w
    amax = np.abs(pad.reshape(nb, BLOCK, kb, BLOCK)).max(axis=(1, 3))
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    codes = np.empty((N, K), np.uint8)
    for bi in range(nb):
        r0, r1 = bi * BLOCK, min(N, (bi + 1) * BLOCK)
        s_cols = np.repeat(s[bi], BLOCK)[:K]
        safe = np.where(s_cols == 0, np.float32(1), s_cols)
        q = np.where(s_cols[None, :] == 0, np.float32(0), w[r0:r1] / safe[None, :])
        codes[r0:r1] = _encode_e4m3(q)
    return codes, s


def quantize_rows_f32(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Row-quantize float32 w [N, K] to (E4M3 codes, float32 [N] row scales)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    s = (np.abs(w).max(axis=1) / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(s == 0, np.float32(1), s)
    codes = np.empty(w.shape, np.uint8)
    for r0 in range(0, w.shape[0], BLOCK):
        r1 = min(w.shape[0], r0 + BLOCK)
        q = np.where(s[r0:r1, None] == 0, np.float32(0), w[r0:r1] / safe[r0:r1, None])
        codes[r0:r1] = _encode_e4m3(q)
    return codes, s


SCALE_FORMATS = ("block_bf16", "block_f32", "row_f32")

# Norm epsilon of the layer's RMSNorms (the pages do not give it; 1e-5 is the
# usual value for this model family).
NORM_EPS = 1e-5


# Mamba-2 mixer of the hidden-4096 layer: d_inner = heads * head_dim = 8192,
# xBC = d_inner + 2 * groups * state = 10240 channels, and the in_proj output
# row [z | xBC | dt] is 8192 + 10240 + 128 = 18560 wide (IN_4K's N).
MAMBA2_4K = dict(heads=128, head_dim=64, state=128, groups=8, d_conv=4)


def ssm_params(heads: int, seed: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(a_log, d_param, dt_bias), float32 [heads]: a_log = log U(1, 16) (so
    A = -exp(a_log) lies in [-16, -1]), D = 1 + 0.1 * N(0, 1), and dt_bias ~
    U(-6.9, -2.25) (softplus of it lies between about 0.001 and 0.1)."""
    rng = np.random.default_rng(seed)
    a_log = np.log(rng.uniform(1.0, 16.0, heads)).astype(np.float32)
    d_param = (1.0 + 0.1 * rng.standard_normal(heads)).astype(np.float32)
    dt_bias = rng.uniform(-6.9, -2.25, heads).astype(np.float32)
    return a_log, d_param, dt_bias


def conv_params(dim: int, d_conv: int, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """(weight [dim, d_conv], bias [dim]) as BF16 bits: N(0, 0.5) and N(0, 0.1)."""
    rng = np.random.default_rng(seed)
    w = (0.5 * rng.standard_normal((dim, d_conv))).astype(np.float32)
    b = (0.1 * rng.standard_normal(dim)).astype(np.float32)
    return _f32_to_bf16_bits(w), _f32_to_bf16_bits(b)


def conv_state(B: int, dim: int, d_conv: int, seed: int) -> np.ndarray:
    """A conv state of earlier inputs, float32 [B, dim, d_conv]: N(0, 1) values
    rounded to BF16 (the inputs it holds are BF16)."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((B, dim, d_conv), dtype=np.float32)
    return _bf16_bits_to_f32(_f32_to_bf16_bits(v)).reshape(B, dim, d_conv).copy()


def ssm_state(B: int, heads: int, head_dim: int, state: int, seed: int) -> np.ndarray:
    """An SSM state, float32 [B, heads, head_dim, state] ~ N(0, 0.1)."""
    rng = np.random.default_rng(seed)
    return (0.1 * rng.standard_normal((B, heads, head_dim, state), dtype=np.float32)).astype(np.float32)


def norm_weight(K: int, seed: int) -> np.ndarray:
    """A norm's weight [K] as BF16 bits: 1 + 0.1 * N(0, 1), rounded to BF16."""
    rng = np.random.default_rng(seed)
    w = np.float32(1) + np.float32(0.1) * rng.standard_normal(K, dtype=np.float32)
    return _f32_to_bf16_bits(w)


def weights_fmt(N: int, K: int, sigma: float, seed: int, fmt: str) -> tuple[np.ndarray, np.ndarray]:
    """(Wq [N, K] E4M3 codes, scales in format fmt) from the same draws as weights()."""
    if fmt == "block_bf16":
        return weights(N, K, sigma, seed)
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(sigma)
    if fmt == "block_f32":
        return quantize_blocks_f32(w)
    if fmt == "row_f32":
        return quantize_rows_f32(w)
    raise ValueError(f"unknown scale format {fmt!r}")


def weights(N: int, K: int, sigma: float, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """(Wq [N, K] E4M3 codes, S [ceil(N/128), ceil(K/128)] BF16 bits)."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(sigma)
    return quantize_blocks(w)


def sha256(*arrays: np.ndarray) -> str:
    h = hashlib.sha256()
    for a in arrays:
        a = np.ascontiguousarray(a)
        h.update(str(a.dtype).encode())
        h.update(str(a.shape).encode())
        h.update(a.tobytes())
    return h.hexdigest()


# ---------------------------------------------------------------------------
# Workloads. Shapes follow the Nemotron-H Mamba-2 layer: in_proj maps the
# hidden state to [z, xBC, dt] (N = 2*d_inner + 2*groups*state + heads) and
# out_proj maps d_inner back to the hidden size.
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Projection:
    name: str          # "in_proj" / "out_proj" / "tiny"
    M: int
    N: int
    K: int
    sigma: float
    seed_a: int
    seed_w: int

    @property
    def grid(self):
        return scale_grid(self.N, self.K)

    def bytes_moved(self) -> int:
        """Algorithmic HBM bytes: W codes, scales, A and the BF16 output once each."""
        nb, kb = self.grid
        return self.N * self.K + 2 * nb * kb + 2 * self.M * self.K + 2 * self.M * self.N

    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


# Hidden 4096, d_inner 8192, 8 groups x 128 state, 128 heads.
IN_4K = dict(N=18560, K=4096)
OUT_4K = dict(N=4096, K=8192)
# Hidden 8192, d_inner 16384, 8 groups x 128 state, 256 heads.
IN_8K = dict(N=35072, K=8192)
OUT_8K = dict(N=8192, K=16384)

WORKLOADS: dict[str, list[Projection]] = {
    # 2x3 grid of 128x128 scale blocks, one token.
    "tiny_gemv": [Projection("tiny", 1, 384, 256, 0.02, 1, 2)],
    # One decode token through both projections (hidden 4096).
    "decode_m1": [Projection("in_proj", 1, **IN_4K, sigma=0.02, seed_a=1001, seed_w=1002),
                  Projection("out_proj", 1, **OUT_4K, sigma=0.02, seed_a=1004, seed_w=1003)],
    # 1024-token prefill through both projections, same weights as decode_m1.
    "prefill_1k": [Projection("in_proj", 1024, **IN_4K, sigma=0.02, seed_a=3001, seed_w=1002),
                   Projection("out_proj", 1024, **OUT_4K, sigma=0.02, seed_a=3004, seed_w=1003)],
    # 8192-token prefill through the larger layer (hidden 8192).
    "prefill_8k_large": [Projection("in_proj", 8192, **IN_8K, sigma=0.01, seed_a=4001, seed_w=4002),
                         Projection("out_proj", 8192, **OUT_8K, sigma=0.01, seed_a=4004, seed_w=4003)],
    # One decode token through the larger layer.
    "decode_m1_large": [Projection("in_proj", 1, **IN_8K, sigma=0.01, seed_a=4011, seed_w=4002),
                        Projection("out_proj", 1, **OUT_8K, sigma=0.01, seed_a=4014, seed_w=4003)],
}

MULTISEQ_M = (2, 4, 8, 16)
for _m in MULTISEQ_M:
    # M decode sequences against the hidden-4096 weights (weights read once for all rows).
    WORKLOADS[f"multiseq_m{_m}"] = [
        Projection("in_proj", _m, **IN_4K, sigma=0.02, seed_a=2000 + _m, seed_w=1002),
        Projection("out_proj", _m, **OUT_4K, sigma=0.02, seed_a=2100 + _m, seed_w=1003)]


@functools.lru_cache(maxsize=8)
def _weights_cached(N, K, sigma, seed):
    Wq, S = weights(N, K, sigma, seed)
    Wq.setflags(write=False)
    S.setflags(write=False)
    return Wq, S


def make(p: Projection) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(A bits [M,K], Wq [N,K], S bits) for one projection of a workload."""
    Wq, S = _weights_cached(p.N, p.K, p.sigma, p.seed_w)
    return activations(p.M, p.K, p.seed_a), Wq, S
