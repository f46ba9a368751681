// Prefill GEMM for the w8a16 block-scaled FP8 projection (any M).
//
//   out[m][n] = sum_k A[m][k] * E4M3(W[n][k]) * scale[n/128][k/128]
// (Qwen3SsmLayer docs, `set_fp8_decode_weights`; NemotronMamba2Layer docs,
// `set_fp8_weights`). Prefill reads the weights once for all prompt tokens
// as one GEMM with M = tokens (TransformerLayer docs, `prefill`).
//
// The pages measure (nemotron_mamba2.rs, `set_bf16_weights` docs) that a
// prefill GEMM which dequantizes its weight tile again in every M-block
// pays N*K*M/M_TILE converts. Here each staged weight tile is converted once
// per workgroup and shared by all TM rows and all waves of that workgroup;
// the converts run on the VALU beside the matrix cores.
//
// Tiling (CDNA4, 64-wide wavefronts, bf16 MFMA v_mfma_f32_32x32x16_bf16):
//  * workgroup tile TM x TN x TK = 128 x 128 x 64, 4 waves in a 2 x 2 grid,
//    each wave a 64 x 64 sub-tile = 2 x 2 MFMA blocks of 32 x 32;
//  * both operands are K-contiguous (A [M][K], W [N][K]), so each MFMA
//    operand lane reads 8 consecutive k (16 bytes) from an LDS row;
//  * LDS rows are 64 BF16 = 8 chunks of 16 bytes; chunk c of row r is stored
//    at c ^ (r & 7) so the 32 rows an MFMA operand read touches spread over
//    all banks;
//  * two LDS stages: tile kt+1 is fetched from HBM into registers while tile
//    kt is multiplied, then written (A as is, W converted) to the other stage;
//  * TN = 128 and TK = 64 divide the 128 x 128 scale blocks, so each staged W
//    tile has exactly one scale, folded into the conversion as
//    bf16_rne(E4M3 * s) (the fp32 product is exact; one rounding to BF16).
#include "w8a16_device.h"
#include "w8a16_host.h"

namespace w8a16 {
namespace {

constexpr int TM = 128, TN = 128, TK = 64;
constexpr int kThreads = 256;
constexpr int kRowChunks = TK / 8;     // 16-byte BF16 chunks per LDS row

static_assert(kScaleBlock % TN == 0 && kScaleBlock % TK == 0, "one scale per staged W tile");

__device__ __forceinline__ int swz(int row, int chunk) { return row * TK + ((chunk ^ (row & 7)) * 8); }

__global__ void __launch_bounds__(kThreads)
gemm_kernel(const uint16_t* __restrict__ A, const uint8_t* __restrict__ W,
            const uint16_t* __restrict__ S, uint16_t* __restrict__ out,
            int M, int N, int K, int tiles_n) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][TM * TK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][TN * TK];

    const int tile = blockIdx.x;
    const int tm = tile / tiles_n, tn = tile % tiles_n;
    const int m0 = tm * TM, n0 = tn * TN;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int k_blocks = (K + kScaleBlock - 1) / kScaleBlock;
    const int nk = (K + TK - 1) / TK;

    u32x4_t ra[4];   // A tile: 128 rows x 8 chunks of 8 BF16 -> 4 chunks per thread
    u32x4_t rb[2];   // W tile: 128 rows x 4 chunks of 16 E4M3 -> 2 chunks per thread

    auto fetch = [&](int kt) {
        const int k0 = kt * TK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + kThreads * i;
            const int row = q >> 3, c = q & 7;
            const int m = m0 + row, k = k0 + c * 8;
            ra[i] = (m < M && k < K) ? load16(A + static_cast<int64_t>(m) * K + k)
                                     : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int q = tid + kThreads * i;
            const int row = q >> 2, c16 = q & 3;
            const int n = n0 + row, k = k0 + c16 * 16;
            rb[i] = (n < N && k < K) ? load16(W + static_cast<int64_t>(n) * K + k)
                                     : u32x4_t{0u, 0u, 0u, 0u};
        }
    };

    auto stage_store = [&](int st, int kt) {
        const float s = bf16_bits_to_f32(S[scale_index(n0, static_cast<int64_t>(kt) * TK, k_blocks)]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + kThreads * i;
            const int row = q >> 3, c = q & 7;
            *reinterpret_cast<u32x4_t*>(&As[st][swz(row, c)]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int q = tid + kThreads * i;
            const int row = q >> 2, c16 = q & 3;
            uint32_t cv[8];
            e4m3x16_scaled_to_bf16(rb[i], s, cv);
            *reinterpret_cast<u32x4_t*>(&Bs[st][swz(row, 2 * c16)]) = u32x4_t{cv[0], cv[1], cv[2], cv[3]};
            *reinterpret_cast<u32x4_t*>(&Bs[st][swz(row, 2 * c16 + 1)]) = u32x4_t{cv[4], cv[5], cv[6], cv[7]};
        }
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[bi][bj][v] = 0.0f;

    const int li = lane & 31, kg = lane >> 5;

    fetch(0);
    stage_store(0, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        if (kt + 1 < nk) fetch(kt + 1);
#pragma unroll
        for (int ks = 0; ks < TK / 16; ++ks) {
            const int c = 2 * ks + kg;
            bf16x8_t af[2], bf[2];
#pragma unroll
            for (int bi = 0; bi < 2; ++bi) {
                const int row = wm * 64 + bi * 32 + li;
                af[bi] = *reinterpret_cast<const bf16x8_t*>(&As[st][swz(row, c)]);
            }
#pragma unroll
            for (int bj = 0; bj < 2; ++bj) {
                const int row = wn * 64 + bj * 32 + li;
                bf[bj] = *reinterpret_cast<const bf16x8_t*>(&Bs[st][swz(row, c)]);
            }
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                for (int bj = 0; bj < 2; ++bj)
                    acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[bi], bf[bj], acc[bi][bj], 0, 0, 0);
        }
        if (kt + 1 < nk) stage_store(st ^ 1, kt + 1);
        __syncthreads();
    }

    // 32x32 MFMA result layout: lane l holds column l % 32; value v is row
    // 8*(v/4) + 4*(l/32) + v%4 of the block.
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) {
            const int n = n0 + wn * 64 + bj * 32 + li;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = m0 + wm * 64 + bi * 32 + 8 * (v >> 2) + 4 * kg + (v & 3);
                if (m < M && n < N)
                    out[static_cast<int64_t>(m) * N + n] = f32_to_bf16_bits(acc[bi][bj][v]);
            }
        }
}

}  // namespace
}  // namespace w8a16

extern "C" int w8a16_gemm(const void* A, const void* Wq, const void* scale, void* out,
                          int64_t M, int64_t N, int64_t K, void* stream) {
    using namespace w8a16;
    bool noop = false;
    int st = check_product_args(A, Wq, scale, out, M, N, K, &noop);
    if (st != W8A16_OK || noop) return st;
    const int64_t tiles_n = ceil_div(N, TN);
    const int64_t tiles = ceil_div(M, TM) * tiles_n;
    if (tiles > INT32_MAX) return W8A16_ERR_SHAPE;
    return launch(&gemm_kernel, dim3(static_cast<unsigned>(tiles)), dim3(kThreads),
                  static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(A),
                  static_cast<const uint8_t*>(Wq), static_cast<const uint16_t*>(scale),
                  static_cast<uint16_t*>(out), static_cast<int>(M), static_cast<int>(N),
                  static_cast<int>(K), static_cast<int>(tiles_n));
}
