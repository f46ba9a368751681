// Decode GEMV for the w8a16 block-scaled FP8 projection, M = 1..16 rows of A.
//
//   out[m][n] = sum_k A[m][k] * E4M3(W[n][k]) * scale[n/128][k/128]
// (Qwen3SsmLayer docs, `set_fp8_decode_weights`; NemotronMamba2Layer docs,
// `set_fp8_weights` for the block index). Decode runs it once per token per
// projection (nemotron_mamba2.rs module docs, forward steps 2 and 7), and the
// multi-sequence decode applies one weight pass to all rows
// (TransformerLayer docs, `decode_multi_seq`).
//
// The GEMV is HBM-bound: each weight byte is read exactly once per call. The
// layout that follows from that on CDNA4:
//  * A workgroup holds `nwaves` wavefronts; wave w owns the K-slice
//    [w*1024*J, (w+1)*1024*J). Lane l of that wave owns the 16-value chunks
//    k = slice + j*1024 + 16*l (j < J), so one wave-wide 16-byte load covers
//    1 KB of a weight row, fully coalesced.
//  * The lane's activations for its chunks (MR rows x J chunks x 16 BF16)
//    stay in registers for the whole kernel; the weight rows stream past.
//  * Each 16-byte weight chunk is decoded once (8 packed E4M3->BF16
//    converts, exact) and used for all MR rows with v_dot2_f32_bf16. A chunk
//    lies inside one 128-wide scale block, so its 16-term partial sum is
//    multiplied by that block's scale in fp32 (exact dequantization).
//  * Partial sums are reduced across the 64 lanes with DPP row operations and
//    across the waves of the workgroup through LDS, always in the same order,
//    so results are deterministic. No atomics.
#include "w8a16_device.h"
#include "w8a16_host.h"

namespace w8a16 {
namespace {

constexpr int kChunk = 16;             // K values (bytes of W) per lane per load
constexpr int kWaveK = 64 * kChunk;    // K values covered by one wave-wide load
constexpr int kMaxWaves = 8;      // 512 threads: up to 256 VGPRs per lane

template <int MR, int J, int RB>
__global__ void __launch_bounds__(kMaxWaves * 64)
gemv_kernel(const uint16_t* __restrict__ A, const uint8_t* __restrict__ W,
            const uint16_t* __restrict__ S, uint16_t* __restrict__ out,
            int N, int K, int groups_per_block) {
    static_assert(kScaleBlock % RB == 0, "a row group must stay inside one scale block");
    static_assert(RB * MR <= 64, "one output per lane after the reduction");
    __shared__ float red[2][kMaxWaves][RB * MR];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const int k_blocks = (K + kScaleBlock - 1) / kScaleBlock;
    const int k_wave = wave * (kWaveK * J);

    // Activations of this lane's chunks, as packed BF16 pairs (k, k+1).
    uint32_t a[MR][J][8];
    bool kvalid[J];
    int kch[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        kch[j] = k_wave + j * kWaveK + lane * kChunk;
        kvalid[j] = kch[j] < K;
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            u32x4_t lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
            if (kvalid[j]) {
                const uint16_t* p = A + static_cast<int64_t>(m) * K + kch[j];
                lo = load16(p);
                hi = load16(p + 8);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                a[m][j][t] = lo[t];
                a[m][j][4 + t] = hi[t];
            }
        }
    }

    const int groups = (N + RB - 1) / RB;
    const int g_begin = blockIdx.x * groups_per_block;
    const int g_end = min(groups, g_begin + groups_per_block);
    int parity = 0;
    for (int g = g_begin; g < g_end; ++g, parity ^= 1) {
        const int n0 = g * RB;

        u32x4_t w[RB][J];
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int j = 0; j < J; ++j) {
                if (n0 + r < N && kvalid[j])
                    w[r][j] = load_stream16(W + static_cast<int64_t>(n0 + r) * K + kch[j]);
                else
                    w[r][j] = u32x4_t{0u, 0u, 0u, 0u};
            }
        // All RB rows sit in scale row-block n0/128 (RB divides 128).
        float s[J];
#pragma unroll
        for (int j = 0; j < J; ++j)
            s[j] = kvalid[j] ? bf16_bits_to_f32(S[scale_index(n0, kch[j], k_blocks)]) : 0.0f;

        float acc[RB][MR];
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int m = 0; m < MR; ++m) acc[r][m] = 0.0f;

#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                bf16x2_t wv[8];
                e4m3x16_to_bf16(w[r][j], wv);
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    float p = 0.0f;
#pragma unroll
                    for (int t = 0; t < 8; ++t)
                        p = __builtin_amdgcn_fdot2_f32_bf16(
                            wv[t], __builtin_bit_cast(bf16x2_t, a[m][j][t]), p, false);
                    acc[r][m] = fmaf(p, s[j], acc[r][m]);
                }
            }

        // Lane t ends up holding output t = r*MR + m of this group.
        float mine = 0.0f;
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const float v = wave_sum(acc[r][m]);
                if (lane == r * MR + m) mine = v;
            }

        if (nwaves == 1) {
            if (lane < RB * MR) {
                const int r = lane / MR, m = lane % MR;
                if (n0 + r < N)
                    out[static_cast<int64_t>(m) * N + n0 + r] = f32_to_bf16_bits(mine);
            }
        } else {
            if (lane < RB * MR) red[parity][wave][lane] = mine;
            __syncthreads();
            if (wave == 0 && lane < RB * MR) {
                float tot = 0.0f;
                for (int v = 0; v < nwaves; ++v) tot += red[parity][v][lane];
                const int r = lane / MR, m = lane % MR;
                if (n0 + r < N)
                    out[static_cast<int64_t>(m) * N + n0 + r] = f32_to_bf16_bits(tot);
            }
            // The next group writes red[parity ^ 1]; red[parity] is rewritten
            // only after the next barrier, which wave 0 reaches after reading it.
        }
    }
}

typedef void (*gemv_fn)(const uint16_t*, const uint8_t*, const uint16_t*, uint16_t*, int, int, int);

// Largest chunk count per lane that keeps MR*J*8 activation registers <= 64.
constexpr int max_chunks(int mr) { return mr == 1 ? 8 : mr == 2 ? 4 : mr <= 4 ? 2 : 1; }

// W rows per iteration: about 16 loads in flight per lane, at most 64 partial
// sums (32 when MR > 8, where the activations already take 72-128 registers).
constexpr int rows_per_iter(int mr, int j) {
    int rb = 16 / j;
    rb = rb < 2 ? 2 : (rb > 8 ? 8 : rb);
    while (rb * mr > (mr > 8 ? 32 : 64)) rb /= 2;
    return rb;
}

template <int MR, int J>
gemv_fn pick_j() {
    return &gemv_kernel<MR, J, rows_per_iter(MR, J)>;
}

template <int MR>
gemv_fn pick(int j) {
    if constexpr (max_chunks(MR) >= 8)
        if (j == 8) return pick_j<MR, 8>();
    if constexpr (max_chunks(MR) >= 4)
        if (j == 4) return pick_j<MR, 4>();
    if constexpr (max_chunks(MR) >= 2)
        if (j == 2) return pick_j<MR, 2>();
    return pick_j<MR, 1>();
}

gemv_fn select_kernel(int mr, int j) {
    switch (mr) {
        case 1: return pick<1>(j);
        case 2: return pick<2>(j);
        case 3: return pick<3>(j);
        case 4: return pick<4>(j);
        case 5: return pick<5>(j);
        case 6: return pick<6>(j);
        case 7: return pick<7>(j);
        case 8: return pick<8>(j);
        case 9: return pick<9>(j);
        case 10: return pick<10>(j);
        case 11: return pick<11>(j);
        case 12: return pick<12>(j);
        case 13: return pick<13>(j);
        case 14: return pick<14>(j);
        case 15: return pick<15>(j);
        default: return pick<16>(j);
    }
}

int rows_per_iter_rt(int mr, int j) { return rows_per_iter(mr, j); }

}  // namespace
}  // namespace w8a16

extern "C" int w8a16_gemv(const void* A, const void* Wq, const void* scale, void* out,
                          int64_t M, int64_t N, int64_t K, void* stream) {
    using namespace w8a16;
    bool noop = false;
    int st = check_product_args(A, Wq, scale, out, M, N, K, &noop);
    if (st != W8A16_OK || noop) return st;
    if (M > W8A16_GEMV_MAX_M || K > (M <= 4 ? W8A16_GEMV_MAX_K_SMALL_M : W8A16_GEMV_MAX_K))
        return W8A16_ERR_SHAPE;

    const int mr = static_cast<int>(M);
    const int jneed = static_cast<int>(ceil_div(K, kWaveK));
    int j = 1;
    while (j < jneed && j < max_chunks(mr)) j *= 2;
    const int nwaves = static_cast<int>(ceil_div(K, static_cast<int64_t>(kWaveK) * j));
    if (nwaves > kMaxWaves) return W8A16_ERR_SHAPE;
    const int rb = rows_per_iter_rt(mr, j);

    const int64_t groups = ceil_div(N, rb);
    const int64_t target_blocks = static_cast<int64_t>(device_cu_count()) * 32 / nwaves;
    const int64_t per_block = ceil_div(groups, target_blocks < 1 ? 1 : target_blocks);
    const int64_t blocks = ceil_div(groups, per_block);

    return launch(select_kernel(mr, j), dim3(static_cast<unsigned>(blocks)), dim3(64 * nwaves),
                  static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(A),
                  static_cast<const uint8_t*>(Wq), static_cast<const uint16_t*>(scale),
                  static_cast<uint16_t*>(out), static_cast<int>(N), static_cast<int>(K),
                  static_cast<int>(per_block));
}
