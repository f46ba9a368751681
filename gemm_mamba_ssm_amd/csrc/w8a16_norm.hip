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
// out; the weight comes from L2.
//
// One workgroup per row: the 256 threads take 16-byte chunks of the row and
// load them, with the weight's (and the gate's) chunks, into registers at
// once (up to 8 chunks per thread, K <= 16384; longer rows loop and read the
// row twice), add their squares (fp32), the workgroup sums them in a fixed
// order, then every thread normalizes its chunks.
#include "w8a16_device.h"
#include "w8a16_host.h"

namespace w8a16 {
namespace {

constexpr int kNormThreads = 256;

// The workgroup's sum of its threads' values, in a fixed order.
__device__ __forceinline__ float block_sum(float v, float* part) {
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
    __syncthreads();
    return (part[0] + part[1]) + (part[2] + part[3]);
}

// CH > 0: chunk c = threadIdx.x + i * 256 (i < CH) is held in registers;
// CH == 0: any K, chunks looped over twice.
template <bool GATED, int CH>
__global__ void __launch_bounds__(kNormThreads)
rmsnorm_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ gate,
               const uint16_t* __restrict__ weight, float eps, uint16_t* __restrict__ out, int K) {
    __shared__ float part[kNormThreads / 64];
    const int64_t row = blockIdx.x;
    const uint16_t* xr = x + row * K;
    const uint16_t* gr = GATED ? gate + row * K : nullptr;
    uint16_t* orow = out + row * K;
    const int chunks = K / 8;
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    if constexpr (CH > 0) {
        u32x4_t xv[CH], wv[CH], gv[CH];
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = threadIdx.x + i * kNormThreads;
            const bool ok = c < chunks;
            xv[i] = ok ? load16(xr + 8 * c) : zero;
            wv[i] = ok ? load16(weight + 8 * c) : zero;
            gv[i] = GATED && ok ? load16(gr + 8 * c) : zero;
        }
#pragma unroll
        for (int i = 0; i < CH; ++i) ss += sumsq8(xv[i]);
        const float r = rms_factor(block_sum(ss, part), K, eps);
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = threadIdx.x + i * kNormThreads;
            if (c < chunks) *reinterpret_cast<u32x4_t*>(orow + 8 * c) = norm8<GATED>(xv[i], wv[i], gv[i], r);
        }
    } else {
        float ss = 0.0f;
        for (int c = threadIdx.x; c < chunks; c += kNormThreads) ss += sumsq8(load16(xr + 8 * c));
        const float r = rms_factor(block_sum(ss, part), K, eps);
        for (int c = threadIdx.x; c < chunks; c += kNormThreads) {
            const u32x4_t g = GATED ? load16(gr + 8 * c) : zero;
            *reinterpret_cast<u32x4_t*>(orow + 8 * c) = norm8<GATED>(load16(xr + 8 * c), load16(weight + 8 * c), g, r);
        }
    }
}

template <bool GATED>
int launch_norm(const uint16_t* x, const uint16_t* g, const uint16_t* w, float eps, uint16_t* o, int64_t M,
                int64_t K, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(M)), block(kNormThreads);
    const int k = static_cast<int>(K);
    const int64_t per_thread = ceil_div(K / 8, kNormThreads);
    if (per_thread <= 1) return launch(&rmsnorm_kernel<GATED, 1>, grid, block, s, x, g, w, eps, o, k);
    if (per_thread <= 2) return launch(&rmsnorm_kernel<GATED, 2>, grid, block, s, x, g, w, eps, o, k);
    if (per_thread <= 4) return launch(&rmsnorm_kernel<GATED, 4>, grid, block, s, x, g, w, eps, o, k);
    if (per_thread <= 8) return launch(&rmsnorm_kernel<GATED, 8>, grid, block, s, x, g, w, eps, o, k);
    return launch(&rmsnorm_kernel<GATED, 0>, grid, block, s, x, g, w, eps, o, k);
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
    hipStream_t s = static_cast<hipStream_t>(stream);
    return gate ? launch_norm<true>(xs, gs, ws, eps, os, M, K, s) : launch_norm<false>(xs, gs, ws, eps, os, M, K, s);
}
