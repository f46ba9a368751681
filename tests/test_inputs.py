"""The seeded input generator: determinism, the quantization recipe, and an
independent check of its E4M3 encoding (torch cast vs a hand RNE encoder)."""
import json
import math
import os

import numpy as np
import torch

from gemm_mamba_ssm_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _e4m3_grid():
    """All finite non-negative E4M3 values, from the format's bit fields."""
    vals = [m / 512 for m in range(8)]
    for e in range(1, 16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            vals.append(math.ldexp(1 + m / 8, e - 7))
    return vals


def _hand_rne_encode(x: float) -> int:
    """Nearest E4M3 code to x (|x| <= 448), ties to the even mantissa."""
    grid = _e4m3_grid()
    a = abs(x)
    best = min(range(len(grid)), key=lambda i: (abs(grid[i] - a), i % 2))
    # among equidistant neighbours pick the even code (grid index parity = mantissa parity)
    lo = max(i for i in range(len(grid)) if grid[i] <= a)
    hi = min(len(grid) - 1, lo + 1)
    if grid[hi] - a == a - grid[lo] and hi != lo:
        best = lo if lo % 2 == 0 else hi
    code = best
    return (0x80 | code) if (x < 0 or (x == 0 and math.copysign(1, x) < 0)) else code


def test_torch_e4m3_cast_matches_hand_encoder():
    rng = np.random.default_rng(5)
    xs = list(rng.uniform(-448, 448, 3000)) + list(rng.standard_normal(3000) * 0.05)
    grid = _e4m3_grid()
    xs += [(grid[i] + grid[i + 1]) / 2 for i in range(len(grid) - 1)]        # every tie
    xs += [-(grid[i] + grid[i + 1]) / 2 for i in range(0, len(grid) - 1, 3)]
    xs = np.array(xs, np.float32)
    got = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for x, g in zip(xs.tolist(), got.tolist()):
        assert g == _hand_rne_encode(x), (x, hex(g))


def test_deterministic_and_seed_sensitive():
    a1 = inputs.activations(2, 256, 3)
    a2 = inputs.activations(2, 256, 3)
    a3 = inputs.activations(2, 256, 4)
    assert np.array_equal(a1, a2) and not np.array_equal(a1, a3)
    w1 = inputs.weights(200, 256, 0.02, 9)
    w2 = inputs.weights(200, 256, 0.02, 9)
    assert all(np.array_equal(x, y) for x, y in zip(w1, w2))


def test_manifest():
    with open(os.path.join(GOLDEN, "input_manifest.json")) as f:
        want = json.load(f)
    (p,) = inputs.WORKLOADS["tiny_gemv"]
    A, W, S = inputs.make(p)
    assert want["tiny_gemv"] == {"A": inputs.sha256(A), "W": inputs.sha256(W), "S": inputs.sha256(S)}
    A = inputs.activations(3, 512, 77)
    W, S = inputs.weights(300, 384, 0.02, 78)
    assert want["m3_n300_k384_seed77"] == {"A": inputs.sha256(A), "W": inputs.sha256(W), "S": inputs.sha256(S)}


def _bf16(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_quantization_recipe():
    N, K, sigma = 300, 400, 0.02
    rng = np.random.default_rng(21)
    w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(sigma)
    w[128:256, 256:384] = 0                         # one all-zero block
    W, S = inputs.quantize_blocks(w)
    assert S.shape == (3, 4) and W.shape == (N, K) and W.dtype == np.uint8
    assert not np.any((W & 0x7F) == 0x7F), "no NaN codes"
    s = _bf16(S)
    assert s[1, 2] == 0 and np.all(W[128:256, 256:384] == 0)
    e = torch.from_numpy(W.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.abs(e).max() <= 448
    for bi in range(3):
        for bj in range(4):
            blk = w[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
            amax = np.abs(blk).max()
            want = torch.tensor([amax / np.float32(448)], dtype=torch.float32).to(torch.bfloat16).item()
            assert s[bi, bj] == want
            if amax > 0:
                # each block reaches (close to) full E4M3 range
                eb = e[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
                assert np.abs(eb).max() >= 416
    # reconstruction error: half an E4M3 step (relative 2^-4 for normals, 2^-10 abs below)
    s_full = np.repeat(np.repeat(s, 128, 0), 128, 1)[:N, :K]
    err = np.abs(e * s_full - w)
    bound = np.maximum(np.abs(w) * 2.0 ** -4, 2.0 ** -10 * s_full) * 1.0001 + 2 * s_full * 2.0 ** -4
    assert np.all(err <= bound)


def test_workload_table():
    w = inputs.WORKLOADS
    (p,) = w["tiny_gemv"]
    assert (p.M, p.N, p.K) == (1, 384, 256) and p.grid == (3, 2)
    ip, op = w["decode_m1"]
    assert (ip.N, ip.K, op.N, op.K) == (18560, 4096, 4096, 8192)
    assert ip.N == 2 * 8192 + 2 * 8 * 128 + 128
    assert ip.bytes_moved() + op.bytes_moved() == 109_659_456
    assert sum(p.flops() for p in w["prefill_1k"]) == 224_412_041_216
    ip, op = w["prefill_8k_large"]
    assert ip.N == 2 * 16384 + 2 * 8 * 128 + 256 and (op.N, op.K) == (8192, 16384)
    for m in inputs.MULTISEQ_M:
        assert w[f"multiseq_m{m}"][0].M == m
