// Row-wise RMSNorm and gated RMSNorm of BF16 activations, the prologues of
// the Mamba-2 projections (nemotron_mamba2.rs module docs, forward step 1:
// RMS norm scaled by its weight before in_proj; step 6: the gated norm
// rms_norm(y, ssm_norm) * silu(z) before out_proj):
//
//   r        = 1 / sqrt(mean_k x[m][k]^2 + eps)
//   out[m][k] = bf16(x[m][k] * r * w[k] [* silu(z[m][k])])
//
// The decode GEMV fuses this into its activation load (w8a16_gemv_fused);
// this standalone kernel serves the prefill GEMM, whose operands go from HBM
// straight into LDS. It is HBM-bound: one read of x (and z), one write of
// out; the weight and the second read of the row come from L2.
//
// One workgroup per row: the 256 threads take 16-byte chunks of the row,
// add their squares (fp32), the workgroup sums them in a fixed order, then
// every thread normalizes its chunks.
#include "w8a16_device.h"
#include "w8a16_host.h"

namespace w8a16 {
namespace {

constexpr int kNormThreads = 256;

template <bool GATED>
__global__ void __launch_bounds__(kNormThreads)
rmsnorm_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ gate,
               const uint16_t* __restrict__ weight, float eps, uint16_t* __restrict__ out, int K) {
    __shared__ float part[kNormThreads / 64];
    const int64_t row = blockIdx.x;
    const uint16_t* xr = x + row * K;
    const int chunks = K / 8;
    float ss = 0.0f;
    for (int c = threadIdx.x; c < chunks; c += kNormThreads) ss += sumsq8(load16(xr + 8 * c));
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float r = rms_factor((part[0] + part[1]) + (part[2] + part[3]), K, eps);
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    for (int c = threadIdx.x; c < chunks; c += kNormThreads) {
        const u32x4_t g = GATED ? load16(gate + row * K + 8 * c) : zero;
        *reinterpret_cast<u32x4_t*>(out + row * K + 8 * c) =
            norm8<GATED>(load16(xr + 8 * c), load16(weight + 8 * c), g, r);
    }
}
static_assert(kNormThreads == 256, "the workgroup sum above adds four waves");

}  // namespace

int check_norm_args(const void* x, const void* gate, const void* weight, float eps, const void* out,
                    int64_t M, int64_t K, bool* noop) {
    *noop = false;
    if (M < 0 || K < 16 || (K % 16) != 0 || M > INT32_MAX || K > INT32_MAX) return W8A16_ERR_SHAPE;
    if (!(eps >= 0.0f) || eps > 3.0e38f) return W8A16_ERR_ARG;   // also rejects NaN
    if (M == 0) {
        *noop = true;
        return W8A16_OK;
    }
    if (!x || !weight || !out) return W8A16_ERR_NULL;
    if (!aligned(x, 16) || !aligned(weight, 16) || !aligned(out, 16) || (gate && !aligned(gate, 16)))
        return W8A16_ERR_ALIGN;
    const int64_t bytes = M * K * 2;
    if (overlaps(out, bytes, x, bytes) || overlaps(out, bytes, weight, K * 2) ||
        (gate && overlaps(out, bytes, gate, bytes)))
        return W8A16_ERR_ALIAS;
    return W8A16_OK;
}

}  // namespace w8a16

extern "C" int w8a16_rmsnorm(const void* x, const void* gate, const void* weight, float eps, void* out,
                             int64_t M, int64_t K, void* stream) {
    using namespace w8a16;
    bool noop = false;
    const int st = check_norm_args(x, gate, weight, eps, out, M, K, &noop);
    if (st != W8A16_OK || noop) return st;
    auto xs = static_cast<const uint16_t*>(x), gs = static_cast<const uint16_t*>(gate);
    auto ws = static_cast<const uint16_t*>(weight);
    auto os = static_cast<uint16_t*>(out);
    const dim3 grid(static_cast<unsigned>(M)), block(kNormThreads);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int k = static_cast<int>(K);
    return gate ? launch(&rmsnorm_kernel<true>, grid, block, s, xs, gs, ws, eps, os, k)
                : launch(&rmsnorm_kernel<false>, grid, block, s, xs, gs, ws, eps, os, k);
}
