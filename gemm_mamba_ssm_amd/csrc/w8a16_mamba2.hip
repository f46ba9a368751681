// The Mamba-2 decode step between the layer's two projections
// (nemotron_mamba2.rs module docs, forward steps 3 to 5; the argument lists
// and launch shapes of `conv1d_update_biased` and `ssm_decode` in that
// listing), read as the standard Mamba-2 recurrence for one token:
//
//  conv1d update (per sequence b, channel c; state = the last d_conv inputs,
//  oldest first, FP32):
//    state[c] <- [state[c][1..], x[c]]
//    out[c]   = bf16( silu( bias[c] + sum_w state[c][w] * weight[c][w] ) )
//
//  SSM decode (per sequence b, head h of group g = h / (heads / groups);
//  xbc = the conv output row [x | B | C]; state FP32 [heads][head_dim][state]):
//    dt = clamp(softplus(dt_raw[h] + dt_bias[h]), dt_min, dt_max)
//    dA = exp(-dt * exp(a_log[h]))
//    h[p][n] <- dA * h[p][n] + dt * B[g][n] * x[h][p]
//    y[h][p] = bf16( sum_n C[g][n] * h[p][n] + D[h] * x[h][p] )
//
// Both are HBM-bound on their state (the SSM state of the hidden-4096 layer
// is 4 MB per sequence, read and written once per token). The SSM kernel
// gives each row (h, p) of the state to 32 lanes that hold 4 consecutive
// states each (16-byte loads and stores; two chunks per lane for state
// <= 256), 8 rows per workgroup, so one token's 128 heads x 64 rows make
// 1024 workgroups; the row's output sum is a fixed butterfly over its 32
// lanes (deterministic).
#include "w8a16_device.h"
#include "w8a16_host.h"

namespace w8a16 {
namespace {

constexpr int kConvThreads = 256;
constexpr int kRowsPerWg = 8;          // SSM state rows (h, p) per workgroup
constexpr int kLanesPerRow = 32;
constexpr int kMaxState = 256;         // 2 chunks of 4 states per lane

__device__ __forceinline__ float bf16v(const uint16_t* p) { return bf16_bits_to_f32(*p); }

__global__ void __launch_bounds__(kConvThreads)
conv1d_update_kernel(float* __restrict__ state, const uint16_t* __restrict__ x, int64_t ld_x,
                     const uint16_t* __restrict__ weight, const uint16_t* __restrict__ bias,
                     uint16_t* __restrict__ out, int64_t ld_out, int dim, int d_conv) {
    const int c = blockIdx.x * kConvThreads + threadIdx.x;
    const int64_t b = blockIdx.y;
    if (c >= dim) return;
    out[b * ld_out + c] = conv_update_channel(state + (b * dim + c) * d_conv, weight + static_cast<int64_t>(c) * d_conv,
                                              bias + c, x[b * ld_x + c], d_conv);
}

// softplus(v) = log(1 + e^v), in the form that neither overflows nor cancels.
__device__ __forceinline__ float softplus(float v) {
    return v > 0.0f ? v + log1pf(expf(-v)) : log1pf(expf(v));
}

// NCH = 4-state chunks per lane (1 for state <= 128, 2 for state <= 256).
template <int NCH>
__global__ void __launch_bounds__(kRowsPerWg * kLanesPerRow)
ssm_decode_kernel(float* __restrict__ hstate, const uint16_t* __restrict__ xbc, int64_t ld_xbc,
                  const uint16_t* __restrict__ dt_raw, int64_t ld_dt, const float* __restrict__ a_log,
                  const float* __restrict__ d_param, const float* __restrict__ dt_bias,
                  uint16_t* __restrict__ out, int64_t ld_out, int heads, int head_dim, int st, int groups,
                  float dt_min, float dt_max) {
    const int row_blocks = (head_dim + kRowsPerWg - 1) / kRowsPerWg;
    const int h = blockIdx.x / row_blocks;
    const int p = (blockIdx.x % row_blocks) * kRowsPerWg + static_cast<int>(threadIdx.x) / kLanesPerRow;
    const int lane = threadIdx.x % kLanesPerRow;
    const int64_t b = blockIdx.y;
    if (p >= head_dim) return;                   // whole 32-lane rows leave together
    const int g = h / (heads / groups);
    const int64_t d_inner = static_cast<int64_t>(heads) * head_dim;
    const uint16_t* row = xbc + b * ld_xbc;
    const uint16_t* Bg = row + d_inner + static_cast<int64_t>(g) * st;
    const uint16_t* Cg = row + d_inner + static_cast<int64_t>(groups) * st + static_cast<int64_t>(g) * st;
    float* hp = hstate + ((b * heads + h) * head_dim + p) * st;

    // Every load first, the state's (from HBM) at the head, so that the
    // memory round trips overlap instead of following one another.
    f32x4_t hv[NCH];
    float bv[NCH][4], cv[NCH][4];
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
        const int n0 = 4 * (lane + q * kLanesPerRow);
        if (n0 < st) hv[q] = *reinterpret_cast<const f32x4_t*>(hp + n0);
    }
    const float raw = bf16v(dt_raw + b * ld_dt + h) + dt_bias[h];
    const float a_h = a_log[h], d_h = d_param[h];
    const float xv = bf16v(row + static_cast<int64_t>(h) * head_dim + p);
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
        const int n0 = 4 * (lane + q * kLanesPerRow);
        if (n0 < st)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bv[q][i] = bf16v(Bg + n0 + i);
                cv[q][i] = bf16v(Cg + n0 + i);
            }
    }

    const float dt = fminf(fmaxf(softplus(raw), dt_min), dt_max);
    const float dA = expf(-dt * expf(a_h));
    const float dtx = dt * xv;
    float y = 0.0f;
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
        const int n0 = 4 * (lane + q * kLanesPerRow);
        if (n0 >= st) break;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            hv[q][i] = dA * hv[q][i] + bv[q][i] * dtx;
            y = fmaf(cv[q][i], hv[q][i], y);
        }
        *reinterpret_cast<f32x4_t*>(hp + n0) = hv[q];
    }
#pragma unroll
    for (int d = kLanesPerRow / 2; d >= 1; d /= 2) y += __shfl_xor(y, d, kLanesPerRow);
    if (lane == 0) out[b * ld_out + static_cast<int64_t>(h) * head_dim + p] = f32_to_bf16_bits(y + d_h * xv);
}

// [p, p + bytes) for a [rows][ld] array of which each row uses `used` elements.
inline int64_t span_bytes(int64_t rows, int64_t ld, int64_t used, int64_t elem) {
    return rows > 0 ? ((rows - 1) * ld + used) * elem : 0;
}

}  // namespace
}  // namespace w8a16

extern "C" int w8a16_conv1d_update(void* conv_state, const void* x, int64_t ld_x, const void* weight,
                                   const void* bias, void* out, int64_t ld_out, int64_t batch, int64_t dim,
                                   int64_t d_conv, void* stream) {
    using namespace w8a16;
    if (batch < 0 || dim < 1 || d_conv < 1 || d_conv > kMaxConvTaps || ld_x < dim || ld_out < dim ||
        batch > 65535 || dim > INT32_MAX || ld_x > INT32_MAX || ld_out > INT32_MAX)
        return W8A16_ERR_SHAPE;
    if (batch == 0) return W8A16_OK;
    if (!conv_state || !x || !weight || !bias || !out) return W8A16_ERR_NULL;
    if (!aligned(conv_state, 4) || !aligned(x, 2) || !aligned(weight, 2) || !aligned(bias, 2) || !aligned(out, 2))
        return W8A16_ERR_ALIGN;
    const int64_t sb = batch * dim * d_conv * 4, xb = span_bytes(batch, ld_x, dim, 2);
    const int64_t ob = span_bytes(batch, ld_out, dim, 2), wb = dim * d_conv * 2;
    if (overlaps(out, ob, x, xb) || overlaps(out, ob, conv_state, sb) || overlaps(out, ob, weight, wb) ||
        overlaps(out, ob, bias, dim * 2) || overlaps(conv_state, sb, x, xb) || overlaps(conv_state, sb, weight, wb) ||
        overlaps(conv_state, sb, bias, dim * 2))
        return W8A16_ERR_ALIAS;
    const dim3 grid(static_cast<unsigned>(ceil_div(dim, kConvThreads)), static_cast<unsigned>(batch));
    return launch(&conv1d_update_kernel, grid, dim3(kConvThreads), static_cast<hipStream_t>(stream),
                  static_cast<float*>(conv_state), static_cast<const uint16_t*>(x), ld_x,
                  static_cast<const uint16_t*>(weight), static_cast<const uint16_t*>(bias),
                  static_cast<uint16_t*>(out), ld_out, static_cast<int>(dim), static_cast<int>(d_conv));
}

extern "C" int w8a16_ssm_decode(void* h_state, const void* xbc, int64_t ld_xbc, const void* dt_raw, int64_t ld_dt,
                                const float* a_log, const float* d_param, const float* dt_bias, void* out,
                                int64_t ld_out, int64_t batch, int64_t heads, int64_t head_dim, int64_t state,
                                int64_t groups, float dt_min, float dt_max, void* stream) {
    using namespace w8a16;
    if (batch < 0 || heads < 1 || head_dim < 1 || groups < 1 || heads % groups != 0 || state < 4 ||
        state % 4 != 0 || state > kMaxState || batch > 65535 || heads > 65536 || head_dim > 65536)
        return W8A16_ERR_SHAPE;
    const int64_t d_inner = heads * head_dim, width = d_inner + 2 * groups * state;
    if (ld_xbc < width || ld_dt < heads || ld_out < d_inner || ld_xbc > INT32_MAX || ld_dt > INT32_MAX ||
        ld_out > INT32_MAX)
        return W8A16_ERR_SHAPE;
    if (!(dt_min >= 0.0f) || !(dt_max >= dt_min) || dt_max > 3.0e38f) return W8A16_ERR_ARG;   // also NaN
    if (batch == 0) return W8A16_OK;
    if (!h_state || !xbc || !dt_raw || !a_log || !d_param || !dt_bias || !out) return W8A16_ERR_NULL;
    if (!aligned(h_state, 16) || !aligned(xbc, 2) || !aligned(dt_raw, 2) || !aligned(a_log, 4) ||
        !aligned(d_param, 4) || !aligned(dt_bias, 4) || !aligned(out, 2))
        return W8A16_ERR_ALIGN;
    const int64_t hb = batch * d_inner * state * 4, xb = span_bytes(batch, ld_xbc, width, 2);
    const int64_t db = span_bytes(batch, ld_dt, heads, 2), ob = span_bytes(batch, ld_out, d_inner, 2);
    const void* params[3] = {a_log, d_param, dt_bias};
    if (overlaps(out, ob, xbc, xb) || overlaps(out, ob, dt_raw, db) || overlaps(out, ob, h_state, hb) ||
        overlaps(h_state, hb, xbc, xb) || overlaps(h_state, hb, dt_raw, db))
        return W8A16_ERR_ALIAS;
    for (const void* q : params)
        if (overlaps(out, ob, q, heads * 4) || overlaps(h_state, hb, q, heads * 4)) return W8A16_ERR_ALIAS;
    const int64_t wgs = heads * ceil_div(head_dim, kRowsPerWg);
    if (wgs > INT32_MAX) return W8A16_ERR_SHAPE;
    const dim3 grid(static_cast<unsigned>(wgs), static_cast<unsigned>(batch)), block(kRowsPerWg * kLanesPerRow);
    hipStream_t s = static_cast<hipStream_t>(stream);
    auto hs = static_cast<float*>(h_state);
    auto xs = static_cast<const uint16_t*>(xbc);
    auto ds = static_cast<const uint16_t*>(dt_raw);
    auto os = static_cast<uint16_t*>(out);
    const int H = static_cast<int>(heads), P = static_cast<int>(head_dim), S = static_cast<int>(state),
              G = static_cast<int>(groups);
    if (state <= 4 * kLanesPerRow)
        return launch(&ssm_decode_kernel<1>, grid, block, s, hs, xs, ld_xbc, ds, ld_dt, a_log, d_param, dt_bias, os,
                      ld_out, H, P, S, G, dt_min, dt_max);
    return launch(&ssm_decode_kernel<2>, grid, block, s, hs, xs, ld_xbc, ds, ld_dt, a_log, d_param, dt_bias, os,
                  ld_out, H, P, S, G, dt_min, dt_max);
}
