// Row-wise RMSNorm and gated RMSNorm of BF16 activations, the prologues of
// the Mamba-2 projections (nemotron_mamba2.rs module docs, forward step 1:
// RMS norm scaled by its weight before in_proj; step 6: the gated norm
// rms_norm(y, ssm_norm) * silu(z) before out_proj):
//
//   r        = 1 / sqrt(mean_k x[m][k]^2 + eps)
//   out[m][k] = bf16(x[m][k] * r * w[k] [* silu(z[m][k])])
//
// with the mean over each group of `group` consecutive channels of the row
// (the whole row when group = K; the pages name no grouping, so it is the
// caller's: the published Mamba-2 gated norm takes K / n_groups).
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
// order, then every thread normalizes its chunks. In groups (a multiple of
// 1024 channels, K <= 16384): each wave's 512 channels of a chunk round lie
// in one group; the waves' sums go to LDS and one thread per group adds its
// parts in order.
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
               const uint16_t* __restrict__ weight, float eps, uint16_t* __restrict__ out, int K, int group) {
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
        if (group == K) {
#pragma unroll
            for (int i = 0; i < CH; ++i) ss += sumsq8(xv[i]);
            const float r = rms_factor(block_sum(ss, part), K, eps);
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int c = threadIdx.x + i * kNormThreads;
                if (c < chunks) *reinterpret_cast<u32x4_t*>(orow + 8 * c) = norm8<GATED>(xv[i], wv[i], gv[i], r);
            }
        } else {
            // Round i, wave w covers channels 2048 i + 512 w .. + 511, inside
            // one group; its sum of squares goes to gpart[i][w].
            __shared__ float gpart[CH][kNormThreads / 64];
            __shared__ float grs[kMaxNormGroups];
            const int wave = threadIdx.x >> 6;
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const float v = wave_sum(sumsq8(xv[i]));
                if ((threadIdx.x & 63) == 0) gpart[i][wave] = v;
            }
            __syncthreads();
            if (static_cast<int>(threadIdx.x) < K / group) {
                const int g = threadIdx.x;
                float t = 0.0f;
                for (int i = 0; i < CH; ++i)
                    for (int w = 0; w < kNormThreads / 64; ++w) {
                        const int ch = 8 * kNormThreads * i + 512 * w;
                        if (ch < K && ch / group == g) t += gpart[i][w];
                    }
                grs[g] = rms_factor(t, group, eps);
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int c = threadIdx.x + i * kNormThreads;
                if (c < chunks)
                    *reinterpret_cast<u32x4_t*>(orow + 8 * c) = norm8<GATED>(xv[i], wv[i], gv[i], grs[8 * c / group]);
            }
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
                int64_t K, int64_t group, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(M)), block(kNormThreads);
    const int k = static_cast<int>(K), gr = static_cast<int>(group);
    const int64_t per_thread = ceil_div(K / 8, kNormThreads);
    if (per_thread <= 1) return launch(&rmsnorm_kernel<GATED, 1>, grid, block, s, x, g, w, eps, o, k, gr);
    if (per_thread <= 2) return launch(&rmsnorm_kernel<GATED, 2>, grid, block, s, x, g, w, eps, o, k, gr);
    if (per_thread <= 4) return launch(&rmsnorm_kernel<GATED, 4>, grid, block, s, x, g, w, eps, o, k, gr);
    if (per_thread <= 8) return launch(&rmsnorm_kernel<GATED, 8>, grid, block, s, x, g, w, eps, o, k, gr);
    return launch(&rmsnorm_kernel<GATED, 0>, grid, block, s, x, g, w, eps, o, k, gr);   // group == K only
}
static_assert(kNormThreads == 256, "the workgroup sum above adds four waves");

}  // namespace

int check_norm_args(const void* x, const void* gate, const void* weight, float eps, int64_t group,
                    const void* out, int64_t M, int64_t K, bool* noop) {
    *noop = false;
    if (M < 0 || K < 16 || (K % 16) != 0 || M > INT32_MAX || K > INT32_MAX) return W8A16_ERR_SHAPE;
    if (!norm_group_valid(group, K)) return W8A16_ERR_SHAPE;
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

extern "C" int w8a16_rmsnorm(const void* x, const void* gate, const void* weight, float eps, int64_t group,
                             void* out, int64_t M, int64_t K, void* stream) {
    using namespace w8a16;
    bool noop = false;
    const int st = check_norm_args(x, gate, weight, eps, group, out, M, K, &noop);
    if (st != W8A16_OK || noop) return st;
    auto xs = static_cast<const uint16_t*>(x), gs = static_cast<const uint16_t*>(gate);
    auto ws = static_cast<const uint16_t*>(weight);
    auto os = static_cast<uint16_t*>(out);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t gr = group == 0 ? K : group;
    return gate ? launch_norm<true>(xs, gs, ws, eps, os, M, K, gr, s)
                : launch_norm<false>(xs, gs, ws, eps, os, M, K, gr, s);
}
