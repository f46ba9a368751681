"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: bit-exact for the dequant-only path (E4M3 decode and scale indexing);
for the products every checked element satisfies
    |gpu - ref| <= 4e-3 * sum_k |A[m,k] * Wdeq[n,k]| + 1e-6
(one BF16 output ulp plus fp32 reordering), with ref and the sum from the
fp64 oracle on the same seeded inputs. Every element is checked, up to the
1024-token prefill; the 8192-token prefill of the large layer is checked along
a whole row and a whole column of every 128 x 128 output block. Invariants with a unique answer
(one-hot rows, zero weights, sign and power-of-two scaling, row permutation,
run-to-run determinism) are checked bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from gemm_mamba_ssm_amd import binding, inputs

pytestmark = pytest.mark.gpu

RTOL, ATOL = 4e-3, 1e-6


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    binding.load()
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dtype, device):
    raw = np.ascontiguousarray(a)
    view = raw.view(np.int16) if raw.dtype == np.uint16 else raw
    return torch.from_numpy(view.copy()).view(dtype).to(device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def upload(A, W, S, device):
    return (to_dev(A, torch.bfloat16, device), to_dev(W, torch.uint8, device),
            to_dev(S, torch.bfloat16, device))


def assert_within_tol(got_bits, ref, den, what):
    g = oracle.bf16_value(got_bits)
    tol = RTOL * den + ATOL
    err = np.abs(g - ref)
    bad = ~(err <= tol)
    ratio = float(np.max(err / tol)) if err.size else 0.0
    say(f"  {what}: {err.size} elements, max err/tol {ratio:.4f}")
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} elements outside tolerance; first {np.argwhere(bad)[:5].tolist()}"
    return ratio


def run(fn, A, W, S, device):
    dA, dW, dS = upload(A, W, S, device)
    out = fn(dA, dW, dS)
    torch.cuda.synchronize()
    return bf16_bits(out)


# --- dequant-only path: bit-exact ---------------------------------------------

def _all_codes_weights(N, K, seed):
    rng = np.random.default_rng(seed)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    W = finite[rng.integers(0, finite.size, (N, K))]
    W.flat[:finite.size] = finite                          # every finite code at least once
    return W


def _distinct_scales(N, K, seed):
    nb, kb = inputs.scale_grid(N, K)
    rng = np.random.default_rng(seed)
    vals = np.exp2(rng.integers(-20, 21, (nb, kb))) * (1 + rng.integers(0, 128, (nb, kb)) / 128)
    S = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return S


@pytest.mark.parametrize("N,K", [(300, 1040), (128, 128), (1, 16), (257, 4096), (129, 16400)])
def test_dequant_bit_exact(dev, N, K):
    say(f"dequant N={N} K={K}")
    W = _all_codes_weights(N, K, N + K) if N * K >= 254 else np.full((N, K), 0xB9, np.uint8)
    S = _distinct_scales(N, K, 7 * N + K)
    dW, dS = to_dev(W, torch.uint8, dev), to_dev(S, torch.bfloat16, dev)
    got = binding.w8a16_dequant(dW, dS)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    exact = oracle.dequant(W, S)
    want = exact.astype(np.float32)                        # exact: e*s fits fp32
    assert np.array_equal(want.astype(np.float64), exact)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), \
        f"{int((got.view(np.uint32) != want.view(np.uint32)).sum())} mismatching elements"


# --- GEMV ------------------------------------------------------------------------

@pytest.mark.parametrize("workload", ["tiny_gemv", "decode_m1", "decode_m1_large"]
                         + [f"multiseq_m{m}" for m in inputs.MULTISEQ_M])
def test_gemv_workloads_every_element(dev, workload):
    for p in inputs.WORKLOADS[workload]:
        say(f"gemv {workload} {p.name} M={p.M} N={p.N} K={p.K}")
        A, W, S = inputs.make(p)
        got = run(binding.w8a16_gemv, A, W, S, dev)
        ref, den = oracle.w8a16(A, W, S)
        assert_within_tol(got, ref, den, f"{workload}/{p.name}")


@pytest.mark.parametrize("M", list(range(1, 17)))
def test_gemv_every_m_ragged(dev, M):
    N, K = 1000, 1040                       # ragged against 128-blocks, row groups and 1024-wide slices
    say(f"gemv ragged M={M} N={N} K={K}")
    A = inputs.activations(M, K, 500 + M)
    W, S = inputs.weights(N, K, 0.02, 600 + M)
    got = run(binding.w8a16_gemv, A, W, S, dev)
    ref, den = oracle.w8a16(A, W, S)
    assert_within_tol(got, ref, den, f"gemv M={M}")


@pytest.mark.parametrize("M,N,K", [(4, 300, 16384), (8, 300, 16384), (9, 300, 8192), (16, 129, 8192),
                                   (1, 7, 16), (3, 1, 48), (1, 130, 3072), (2, 259, 12288),
                                   (1, 2049, 8208), (1, 33, 16384), (7, 4096, 1024)])
def test_gemv_k_edges(dev, M, N, K):
    say(f"gemv edge M={M} N={N} K={K}")
    A = inputs.activations(M, K, 700 + K)
    W, S = inputs.weights(N, K, 0.02, 800 + N)
    got = run(binding.w8a16_gemv, A, W, S, dev)
    ref, den = oracle.w8a16(A, W, S)
    assert_within_tol(got, ref, den, f"gemv M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(2, 8193, 16), (3, 9000, 1040), (4, 8195, 8192), (3, 18560, 4096),
                                   (2, 18560, 4096), (4, 18560, 4096)])
def test_gemv_few_tokens_on_the_gemv_kernel(dev, M, N, K):
    """2..4 rows with at least 8 four-row weight groups per CU (N >= 8192 on
    256 CUs) and K <= 8192 run the GEMV kernel with the single-token launch
    shape rather than the skinny kernel: ragged N (a last group of 1..3 rows),
    K of one k-chunk, K not a multiple of 128, the largest K of one chunk per
    lane, and the Mamba-2 in_proj."""
    say(f"gemv few tokens M={M} N={N} K={K}")
    A = inputs.activations(M, K, 900 + M)
    W, S = inputs.weights(N, K, 0.02, 1000 + N)
    got = run(binding.w8a16_gemv, A, W, S, dev)
    again = run(binding.w8a16_gemv, A, W, S, dev)
    assert np.array_equal(got, again), "not deterministic"
    ref, den = oracle.w8a16(A, W, S)
    assert_within_tol(got, ref, den, f"gemv M={M} N={N} K={K}")


# --- GEMM ------------------------------------------------------------------------

# Paths of the GEMM entry (w8a16_gemm, which computes every tile whole in one
# workgroup and uses no workspace). M <= 16 takes the skinny kernel: its
# one-shot form (one 16-row weight block per workgroup, activations in LDS)
# where its plan fits (every weight block on a CU of its own: N = 130..4100
# here; more blocks than CUs with 64 KB of activations or less: N = 140000 /
# 166400 with M = 3 / 5, N = 4100 with M = 2), else its ring form (M = 16,
# N = 18560, K = 4096). 17 <= M <= 256 with K <= 32768 takes the mid-size
# kernel (small tiles, one per workgroup; every tile shape of it in
# test_gpu_mid.py): here ragged M, N and K, K below one stage, several rounds
# of tiles over the CUs (N = 65704, 78339, 89603, 98400). Past those, the
# tiles are 32 x 128 for M <= 32 and 64 x 128 for M <= 64 (M = 7 with K =
# 8208 past the one-shot form's 64 k-blocks; M = 20 and 40 with K above
# 32768), 128 x 128 above (several rounds of them at M = 300, N = 40000);
# 128 x 128 tiles numbering 192..256 (on 256 CUs) with K a multiple of 256
# split their k-steps between two wave groups of one workgroup (M = 1000,
# N = 3000, K = 1280: ragged M and N, 10 k-steps per group). The 256 x 256
# tiles and the split schedules of w8a16_gemm_ws have their own tests
# (test_gpu_wide.py, below).
@pytest.mark.parametrize("M,N,K", [(1, 384, 256), (17, 130, 144), (127, 300, 272), (129, 1000, 1040),
                                   (300, 257, 4096), (256, 256, 128), (1, 1, 16), (64, 4096, 512),
                                   (513, 640, 1024), (130, 18560, 128), (66, 65704, 1040),
                                   (72, 78339, 1040), (65, 89603, 1040), (32, 18560, 4096), (20, 4096, 8192),
                                   (3, 140000, 1040), (5, 166400, 528), (33, 1000, 1040), (48, 18560, 2048),
                                   (40, 98400, 528), (31, 300, 4112), (16, 18560, 4096), (9, 1000, 4096),
                                   (7, 1000, 8208), (2, 4100, 1936), (200, 12200, 1280), (256, 12288, 512),
                                   (130, 38300, 512), (16, 4096, 8192), (13, 1000, 4224), (12, 300, 6160),
                                   (20, 1000, 36880), (40, 300, 40960), (1000, 3000, 1280), (300, 40000, 272)])
def test_gemm_every_element(dev, M, N, K):
    say(f"gemm M={M} N={N} K={K}")
    A = inputs.activations(M, K, 900 + M)
    W, S = inputs.weights(N, K, 0.02, 1000 + N + K)
    got = run(binding.w8a16_gemm, A, W, S, dev)
    ref, den = oracle.w8a16(A, W, S)
    assert_within_tol(got, ref, den, f"gemm M={M} N={N} K={K}")


@pytest.mark.parametrize("proj", [0, 1])
def test_gemm_prefill_1k_every_element(dev, proj):
    """The 1024-token prefill through in_proj (1024 x 18560 x 4096) or out_proj
    (1024 x 4096 x 8192): every element against the oracle, which takes its
    rows in chunks (about a minute of host time per projection)."""
    p = inputs.WORKLOADS["prefill_1k"][proj]
    say(f"gemm prefill_1k {p.name} M={p.M} N={p.N} K={p.K} (every element)")
    A, W, S = inputs.make(p)
    got = run(binding.w8a16_gemm, A, W, S, dev)
    worst = 0.0
    for r0 in range(0, p.M, 128):
        ref, den = oracle.w8a16(A[r0:r0 + 128], W, S)
        worst = max(worst, assert_within_tol(got[r0:r0 + 128], ref, den, f"{p.name} rows {r0}.."))
    say(f"  {p.name}: max err/tol over all rows {worst:.4f}")


def _tile_rows_cols(M, N, tile=128):
    """One row in every 128-row block and one column in every 128-column block
    (a different offset inside each block), so every output tile of every tile
    shape (128 x 128 and 256 x 256) is checked along a whole row and a whole
    column."""
    rows = np.array([min(M - 1, b * tile + (37 * b + 5) % tile) for b in range((M + tile - 1) // tile)])
    cols = np.array([min(N - 1, b * tile + (53 * b + 11) % tile) for b in range((N + tile - 1) // tile)])
    return rows, cols


@pytest.mark.parametrize("proj", [0, 1])
def test_gemm_prefill_8k_every_tile(dev, proj):
    """The 8192-token prefill of the large layer: a whole row in every 128-row
    block and a whole column in every 128-column block, against the oracle."""
    p = inputs.WORKLOADS["prefill_8k_large"][proj]
    say(f"gemm prefill_8k_large {p.name} M={p.M} N={p.N} K={p.K} (a row and a column per tile)")
    A, W, S = inputs.make(p)
    got = run(binding.w8a16_gemm, A, W, S, dev)
    rows, cols = _tile_rows_cols(p.M, p.N)
    ref, den = oracle.w8a16(A[rows], W, S)
    assert_within_tol(got[rows], ref, den, f"{p.name}: {rows.size} whole rows")
    mi = np.repeat(np.arange(p.M), cols.size)
    ni = np.tile(cols, p.M)
    ref, den = oracle.w8a16_points(A, W, S, mi, ni)
    assert_within_tol(got[mi, ni], ref, den, f"{p.name}: {cols.size} whole columns")


# Long K past what the 256 x 256 tiles and the skinny kernel take (K = 65552,
# 513 k-blocks with a k-tail of 16): 128 x 128 tiles, every element.
def test_gemm_long_k_every_element(dev):
    M, N, K = 130, 300, 65552
    say(f"gemm long K M={M} N={N} K={K}")
    A = inputs.activations(M, K, 7700)
    W, S = inputs.weights(N, K, 0.02, 7800)
    got = run(binding.w8a16_gemm, A, W, S, dev)
    ref, den = oracle.w8a16(A, W, S)
    assert_within_tol(got, ref, den, f"gemm M={M} N={N} K={K}")


def test_gemv_matches_gemm_on_decode_shapes(dev):
    for p in inputs.WORKLOADS["multiseq_m8"]:
        A, W, S = inputs.make(p)
        gv = run(binding.w8a16_gemv, A, W, S, dev)
        gm = run(binding.w8a16_gemm, A, W, S, dev)
        ref, den = oracle.w8a16(A, W, S)
        assert_within_tol(gv, ref, den, "gemv")
        assert_within_tol(gm, ref, den, "gemm")


# --- invariants with a unique answer ------------------------------------------------

ENTRY = {"gemv": binding.w8a16_gemv, "gemm": binding.w8a16_gemm}


@pytest.mark.parametrize("entry,M", [("gemv", 4), ("gemv", 16), ("gemm", 130), ("gemm", 20), ("gemm", 40)])
def test_one_hot_rows_return_rounded_dequantized_columns(dev, entry, M):
    N, K = 300, 1040
    W, S = inputs.weights(N, K, 0.02, 31)
    A = np.zeros((M, K), np.uint16)
    cols = (np.arange(M) * 97 + 5) % K
    A[np.arange(M), cols] = 0x3F80
    got = run(ENTRY[entry], A, W, S, dev)
    want = oracle.bf16_rne(oracle.dequant(W, S)[:, cols].T)
    # unique up to the sign of zero (a -0 weight times +1 may sum to +0)
    assert np.array_equal(oracle.bf16_value(got), oracle.bf16_value(want))


@pytest.mark.parametrize("entry", ["gemv", "gemm"])
def test_zero_weights_give_exact_zero(dev, entry):
    A = inputs.activations(8, 1040, 41)
    W, S = inputs.weights(300, 1040, 0.02, 42)
    got = run(ENTRY[entry], A, np.zeros_like(W), S, dev)
    assert np.all((got & 0x7FFF) == 0)


@pytest.mark.parametrize("entry,M", [("gemv", 6), ("gemm", 200), ("gemm", 24), ("gemm", 56)])
def test_sign_scaling_permutation_and_determinism(dev, entry, M):
    N, K = 520, 2048
    A = inputs.activations(M, K, 51)
    W, S = inputs.weights(N, K, 0.02, 52)
    fn = ENTRY[entry]
    base = run(fn, A, W, S, dev)
    again = run(fn, A, W, S, dev)
    assert np.array_equal(base, again), "not deterministic"
    neg = run(fn, A ^ np.uint16(0x8000), W, S, dev)
    assert np.array_equal(neg, base ^ np.uint16(0x8000)) or np.array_equal(
        oracle.bf16_value(neg), -oracle.bf16_value(base))
    A2 = np.where((A & 0x7FFF) == 0, A, A + np.uint16(0x80))   # A * 2 exactly
    dbl = run(fn, A2, W, S, dev)
    assert np.array_equal(oracle.bf16_value(dbl), 2 * oracle.bf16_value(base))
    # Rows are independent and every row of a tile goes through the same
    # k-split (for the GEMM at this shape every tile splits at the same
    # k-blocks), so permuting the rows permutes the output bits.
    perm = np.random.default_rng(3).permutation(M)
    got = run(fn, A[perm], W, S, dev)
    assert np.array_equal(got, base[perm])


@pytest.mark.parametrize("entry,M", [("gemv", 3), ("gemm", 150), ("gemm", 10), ("gemm", 60)])
def test_scale_doubling_touches_only_its_block(dev, entry, M):
    N, K = 300, 1040
    A = inputs.activations(M, K, 61)
    W, S = inputs.weights(N, K, 0.02, 62)
    fn = ENTRY[entry]
    base = run(fn, A, W, S, dev)
    S2 = S.copy()
    S2[1, 3] += 0x80                                  # x2 exactly
    got = run(fn, A, W, S2, dev)
    cols = np.zeros(N, bool)
    cols[128:256] = True
    assert np.array_equal(got[:, ~cols], base[:, ~cols])
    ref, den = oracle.w8a16(A, W, S2)
    assert_within_tol(got, ref, den, "scale x2")


@pytest.mark.parametrize("entry", ["gemv", "gemm"])
def test_output_guard_band_untouched(dev, entry):
    M, N, K = 5, 333, 1040
    A = inputs.activations(M, K, 71)
    W, S = inputs.weights(N, K, 0.02, 72)
    dA, dW, dS = upload(A, W, S, dev)
    pad = 4096
    buf = torch.full((pad + M * N + pad,), -7.0, dtype=torch.bfloat16, device=dev)
    out = buf[pad:pad + M * N].view(M, N)
    ENTRY[entry](dA, dW, dS, out=out)
    torch.cuda.synchronize()
    assert torch.all(buf[:pad] == -7.0) and torch.all(buf[pad + M * N:] == -7.0)
    ref, den = oracle.w8a16(A, W, S)
    assert_within_tol(bf16_bits(out), ref, den, f"{entry} into a view")


@pytest.mark.parametrize("entry", ["gemv", "gemm"])
def test_empty_and_rejected_calls(dev, entry):
    W, S = inputs.weights(256, 256, 0.02, 81)
    dW, dS = to_dev(W, torch.uint8, dev), to_dev(S, torch.bfloat16, dev)
    out = ENTRY[entry](torch.empty((0, 256), dtype=torch.bfloat16, device=dev), dW, dS)
    assert tuple(out.shape) == (0, 256)
    dA = torch.ones((2, 256), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        ENTRY[entry](dA, dW, dS.reshape(-1))           # wrong scale layout refused before launch
    st = (binding.gemv_raw if entry == "gemv" else binding.gemm_raw)(
        dA.data_ptr(), dW.data_ptr(), dS.data_ptr(), dA.data_ptr(), 2, 256, 256, 0)
    assert st == binding.ERR_ALIAS
    torch.cuda.synchronize()


# Shapes whose tiles split their k-blocks between workgroups when a workspace
# is given (w8a16_gemm_ws): fewer tiles than slots (32-, 64- and 128-row
# tiles; the 32- and 64-row ones with K past the mid-size kernel's 32768),
# a whole round plus a split remainder (M = 300, N = 33000) and one split
# tile. (The schedule that fills the whole 64 MiB, M = 384 on the Mamba-2
# in_proj, runs in test_zz_no_alloc.py.)
SPLIT_SHAPES = [(300, 1000, 1040), (300, 257, 4096), (512, 2048, 4096), (20, 1000, 36880), (40, 4100, 40960),
                (300, 33000, 272)]


@pytest.mark.parametrize("M,N,K", SPLIT_SHAPES)
def test_gemm_ws_split_tiles_every_element(dev, M, N, K):
    say(f"gemm_ws M={M} N={N} K={K}")
    A = inputs.activations(M, K, 950 + M)
    W, S = inputs.weights(N, K, 0.02, 1050 + N + K)
    ws = binding.gemm_workspace(M, N, K, dev)
    assert ws is not None, "this shape splits"
    dA, dW, dS = upload(A, W, S, dev)
    got = binding.w8a16_gemm_ws(dA, dW, dS, ws)
    again = binding.w8a16_gemm_ws(dA, dW, dS, ws)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), again.view(torch.int16)), "not deterministic"
    ref, den = oracle.w8a16(A, W, S)
    assert_within_tol(bf16_bits(got), ref, den, f"gemm_ws M={M} N={N} K={K}")


def test_gemm_ws_on_two_streams_with_two_workspaces(dev):
    """Two split GEMMs run concurrently on two streams, each with its own
    workspace: neither result is disturbed, and repeats agree bit for bit."""
    shapes = [(300, 1000, 1040, 21), (300, 257, 4096, 22)]
    ops = []
    for M, N, K, seed in shapes:
        A = inputs.activations(M, K, seed)
        W, S = inputs.weights(N, K, 0.02, seed + 100)
        ops.append((A, W, S, *upload(A, W, S, dev), binding.gemm_workspace(M, N, K, dev)))
        assert ops[-1][-1] is not None, "this shape splits"
    streams = [torch.cuda.Stream(device=dev) for _ in shapes]
    outs = []
    torch.cuda.synchronize()
    for rep in range(3):
        for (A, W, S, dA, dW, dS, ws), s in zip(ops, streams):
            with torch.cuda.stream(s):
                outs.append(binding.w8a16_gemm_ws(dA, dW, dS, ws))
    torch.cuda.synchronize()
    for i, (A, W, S, *_) in enumerate(ops):
        ref, den = oracle.w8a16(A, W, S)
        got = [bf16_bits(outs[rep * len(ops) + i]) for rep in range(3)]
        assert_within_tol(got[0], ref, den, f"stream {i}")
        assert all(np.array_equal(g, got[0]) for g in got[1:]), "repeats differ"


def test_gemm_on_two_streams_at_once(dev):
    """Two GEMMs run concurrently on two streams (no shared state: the plain
    entry point uses no workspace), each result exact to the oracle's bar."""
    shapes = [(129, 1000, 1040, 11), (300, 257, 4096, 12)]
    ops = []
    for M, N, K, seed in shapes:
        A = inputs.activations(M, K, seed)
        W, S = inputs.weights(N, K, 0.02, seed + 100)
        ops.append((A, W, S, *upload(A, W, S, dev)))
    streams = [torch.cuda.Stream(device=dev) for _ in shapes]
    outs = []
    torch.cuda.synchronize()
    for rep in range(3):
        for (A, W, S, dA, dW, dS), s in zip(ops, streams):
            with torch.cuda.stream(s):
                outs.append(binding.w8a16_gemm(dA, dW, dS))
    torch.cuda.synchronize()
    for i, (A, W, S, *_) in enumerate(ops):
        ref, den = oracle.w8a16(A, W, S)
        got = [bf16_bits(outs[rep * len(ops) + i]) for rep in range(3)]
        assert_within_tol(got[0], ref, den, f"stream {i}")
        assert all(np.array_equal(g, got[0]) for g in got[1:]), "repeats differ"


def test_stream_ordering(dev):
    """The call is enqueued on the caller's stream and ordered with other work on it."""
    p = inputs.WORKLOADS["tiny_gemv"][0]
    A, W, S = inputs.make(p)
    dA, dW, dS = upload(A, W, S, dev)
    s = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(s):
        out = torch.full((1, p.N), 3.0, dtype=torch.bfloat16, device=dev)
        binding.w8a16_gemv(dA, dW, dS, out=out)
        res = out.clone()
    s.synchronize()
    ref, den = oracle.w8a16(A, W, S)
    assert_within_tol(bf16_bits(res), ref, den, "stream")
