// Dequantize-only path: exposes the device E4M3 decode (the packed convert the
// GEMV and GEMM feed their dot products and MFMAs with) and the block-scale
// index, so both can be checked bit for bit: out = float(E4M3) * s in fp32,
// which is exact (weights and scale grid as in the Qwen3SsmLayer docs,
// `set_fp8_decode_weights`, and the NemotronMamba2Layer docs, `set_fp8_weights`).
// One thread per 16-byte weight chunk; four 16-byte fp32 stores.
#include "w8a16_device.h"
#include "w8a16_host.h"

namespace w8a16 {
namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads)
dequant_kernel(const uint8_t* __restrict__ W, const uint16_t* __restrict__ S, float* __restrict__ out,
               int64_t N, int K) {
    const int64_t chunks_per_row = K / 16;
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (idx >= N * chunks_per_row) return;
    const int64_t n = idx / chunks_per_row;
    const int k = static_cast<int>(idx % chunks_per_row) * 16;
    const int k_blocks = (K + kScaleBlock - 1) / kScaleBlock;
    const u32x4_t w = load16(W + n * K + k);
    const float s = bf16_bits_to_f32(S[scale_index(n, k, k_blocks)]);
    float r[16];
    bf16x2_t v[8];
    e4m3x16_to_bf16(w, v);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        r[2 * t] = static_cast<float>(v[t].x) * s;
        r[2 * t + 1] = static_cast<float>(v[t].y) * s;
    }
    f32x4_t* o = reinterpret_cast<f32x4_t*>(out + n * K + k);
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = f32x4_t{r[4 * q], r[4 * q + 1], r[4 * q + 2], r[4 * q + 3]};
}

}  // namespace
}  // namespace w8a16

extern "C" int w8a16_dequant(const void* Wq, const void* scale, float* out, int64_t N, int64_t K,
                             void* stream) {
    using namespace w8a16;
    if (N < 0 || K < 16 || (K % 16) != 0 || N > INT32_MAX || K > INT32_MAX) return W8A16_ERR_SHAPE;
    if (N == 0) return W8A16_OK;
    if (!Wq || !scale || !out) return W8A16_ERR_NULL;
    if (!aligned(Wq, 16) || !aligned(scale, 2) || !aligned(out, 16)) return W8A16_ERR_ALIGN;
    const int64_t scale_bytes = ceil_div(N, kScaleBlockHost) * ceil_div(K, kScaleBlockHost) * 2;
    if (overlaps(out, N * K * 4, Wq, N * K) || overlaps(out, N * K * 4, scale, scale_bytes))
        return W8A16_ERR_ALIAS;
    const int64_t blocks = ceil_div(N * (K / 16), kThreads);
    if (blocks > INT32_MAX) return W8A16_ERR_SHAPE;
    return launch(&dequant_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads),
                  static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(Wq),
                  static_cast<const uint16_t*>(scale), out, N, static_cast<int>(K));
}
