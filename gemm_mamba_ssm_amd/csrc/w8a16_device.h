// Device-side building blocks shared by the GEMV, GEMM and dequant kernels:
// E4M3 -> BF16 decode with the gfx950 packed converts, the block-scale index,
// BF16 <-> FP32 and the wavefront reduction. gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a16 {

// Scale blocks are 128 x 128 (NemotronMamba2Layer docs, `set_fp8_weights`).
constexpr int kScaleBlock = 128;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Index of the scale of weight element (n, k) in the row-major
// [ceil(N/128)][ceil(K/128)] grid: (n / 128) * ceil(K/128) + k / 128.
__device__ __forceinline__ int64_t scale_index(int64_t n, int64_t k, int64_t k_blocks) {
    return (n / kScaleBlock) * k_blocks + k / kScaleBlock;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits) {
    return __uint_as_float(bits << 16);
}

// fp32 -> BF16 bits, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Two E4M3 codes (bytes 0-1 of `w` if !hi, bytes 2-3 if hi) -> two BF16.
// Every finite E4M3 value (3 mantissa bits, exponents 2^-9 .. 2^8) is exactly
// representable in BF16, and a scale of 1.0 leaves it unchanged: exact.
__device__ __forceinline__ bf16x2_t e4m3x2_to_bf16(uint32_t w, bool hi) {
    return hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
              : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
}

// 16 E4M3 codes (one 16-byte load) -> 16 BF16, as 8 packed pairs in order.
__device__ __forceinline__ void e4m3x16_to_bf16(u32x4_t w, bf16x2_t (&out)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = e4m3x2_to_bf16(w[i], false);
        out[2 * i + 1] = e4m3x2_to_bf16(w[i], true);
    }
}

// DPP lane moves (within rows of 16 lanes). Controls from the GCN/CDNA DPP encoding.
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;   // row_ror:4
constexpr int kDppRowRor8 = 0x128;   // row_ror:8

template <int Ctrl>
__device__ __forceinline__ float dpp_move(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), Ctrl, 0xF, 0xF, false));
}

// Sum over the 64 lanes of a wavefront, in a fixed order (deterministic).
// Within each row of 16 lanes: quad sums, then pairs of quads, then the
// row; across the four rows: read each row's sum and add (r0+r1)+(r2+r3).
// The result is uniform (the same in every lane).
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_move<kDppQuadXor1>(v);
    v += dpp_move<kDppQuadXor2>(v);
    v += dpp_move<kDppRowRor4>(v);
    v += dpp_move<kDppRowRor8>(v);
    float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

// Scale formats (enum w8a16_scale_format): the kernels take one as a template
// parameter.
constexpr int kScaleBlockBf16 = 0, kScaleBlockF32 = 1, kScaleRowF32 = 2;

// Scale of k-block `idx` of the block grid (index (n/128) * ceil(K/128) +
// k/128) in format SF; 1 for the per-row format, whose scale multiplies the
// finished row sum instead (row_scale).
template <int SF>
__device__ __forceinline__ float block_scale(const void* S, int64_t idx) {
    if constexpr (SF == kScaleBlockBf16)
        return bf16_bits_to_f32(static_cast<const uint16_t*>(S)[idx]);
    else if constexpr (SF == kScaleBlockF32)
        return static_cast<const float*>(S)[idx];
    else
        return 1.0f;
}

// The same scale as raw bits (BF16 bits, or FP32 bits), for callers that
// load it early and decode it where it is used.
template <int SF>
__device__ __forceinline__ uint32_t block_scale_bits(const void* S, int64_t idx) {
    if constexpr (SF == kScaleBlockBf16)
        return static_cast<const uint16_t*>(S)[idx];
    else if constexpr (SF == kScaleBlockF32)
        return __float_as_uint(static_cast<const float*>(S)[idx]);
    else
        return __float_as_uint(1.0f);
}

template <int SF>
__device__ __forceinline__ float scale_from_bits(uint32_t bits) {
    if constexpr (SF == kScaleBlockBf16)
        return bf16_bits_to_f32(bits);
    else
        return __uint_as_float(bits);
}

// Scale of weight row n in format SF: the FP32 [N] entry, 1 for the block formats.
template <int SF>
__device__ __forceinline__ float row_scale(const void* S, int64_t n) {
    if constexpr (SF == kScaleRowF32)
        return static_cast<const float*>(S)[n];
    else
        return 1.0f;
}

__device__ __forceinline__ u32x4_t load16(const void* p) {
    return *reinterpret_cast<const u32x4_t*>(p);
}

// --- norm prologues and the residual epilogue (nemotron_mamba2.rs module
// docs, forward steps 1, 6 and 8) ---

// What a fused projection does around the product (kernel argument): a
// norm prologue on the activations when `weight` is set (gated by silu(gate)
// when `gate` is set too), and a residual epilogue when `residual` is set.
struct Fusion {
    const uint16_t* gate;       // [M] rows of K BF16, ld_gate apart, or nullptr
    const uint16_t* weight;     // [K] BF16 norm weight, or nullptr (no norm)
    const uint16_t* residual;   // [M][N] BF16, or nullptr
    int64_t ld_gate;
    float eps;
    int group;                  // channels per norm group: K (the whole row) or a multiple of 1024 dividing K
    // conv1d update on output columns [conv_begin, conv_begin + conv_dim)
    // (the in_proj form): FP32 state [M][conv_dim][d_conv], BF16 taps
    // [conv_dim][d_conv] and bias [conv_dim].
    float* conv_state;
    const uint16_t* conv_weight;
    const uint16_t* conv_bias;
    int conv_begin, conv_dim, d_conv;
};

// SiLU in fp32: z / (1 + e^-z), with the hardware exponential and reciprocal
// (a few ulp of fp32; every use rounds the result, or a product with it, to
// BF16). The IEEE-exact expf and division take about five times the VALU
// work, which showed in the gated norm prologue of the decode GEMV. Large
// |z| is exact in the limit: e^-z -> 0 gives z, e^-z -> inf gives -0.
__device__ __forceinline__ float silu(float z) {
    return __fdividef(z, 1.0f + __expf(-z));
}

// Sum of squares of 8 BF16 values (4 packed pairs).
__device__ __forceinline__ float sumsq8(u32x4_t x) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = bf16_bits_to_f32(x[i] & 0xFFFFu), hi = bf16_bits_to_f32(x[i] >> 16);
        s = fmaf(lo, lo, s);
        s = fmaf(hi, hi, s);
    }
    return s;
}

// 8 normalized activations: bf16(x * r * w), or bf16(x * r * w * silu(g))
// when GATED, in fp32 with one rounding at the end.
template <bool GATED>
__device__ __forceinline__ u32x4_t norm8(u32x4_t x, u32x4_t w, u32x4_t g, float r) {
    u32x4_t o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float lo = bf16_bits_to_f32(x[i] & 0xFFFFu) * r * bf16_bits_to_f32(w[i] & 0xFFFFu);
        float hi = bf16_bits_to_f32(x[i] >> 16) * r * bf16_bits_to_f32(w[i] >> 16);
        if constexpr (GATED) {
            lo *= silu(bf16_bits_to_f32(g[i] & 0xFFFFu));
            hi *= silu(bf16_bits_to_f32(g[i] >> 16));
        }
        o[i] = static_cast<uint32_t>(f32_to_bf16_bits(lo)) | (static_cast<uint32_t>(f32_to_bf16_bits(hi)) << 16);
    }
    return o;
}

// 1 / sqrt(mean of squares + eps) of K values (a row, or one group of it).
__device__ __forceinline__ float rms_factor(float sumsq, int K, float eps) {
    return 1.0f / sqrtf(sumsq / static_cast<float>(K) + eps);
}

// The residual add after the projection: both operands are BF16 tensors, so
// the projection's sum is rounded to BF16 first (y), then the sum of the two.
__device__ __forceinline__ uint16_t residual_add_bits(uint16_t y, uint16_t residual) {
    return f32_to_bf16_bits(bf16_bits_to_f32(residual) + bf16_bits_to_f32(y));
}

__device__ __forceinline__ uint16_t residual_out(float sum, uint16_t residual) {
    return residual_add_bits(f32_to_bf16_bits(sum), residual);
}

constexpr int kMaxConvTaps = 8;        // d_conv at most (checked by the entry points)
constexpr int kConvFastTaps = 4;       // d_conv up to this reads its operands in one round trip

// conv1d update of one channel (nemotron_mamba2.rs module docs, forward step
// 3): the FP32 state s[0..d_conv) of the last inputs, oldest first, is
// shifted and takes the new BF16 input x; returns bf16(silu(bias + sum_t
// s[t] * w[t])), summed in tap order.
// For d_conv <= 4 (the Mamba-2 layers) every operand is loaded before the
// sums and stores, one memory round trip: the 4 state values and taps are
// read unconditionally (a tap past d_conv re-reads the last one and is not
// used), so no branch makes the compiler wait for each value as it arrives.
// Longer convolutions take the taps one by one, in the same order.
__device__ __forceinline__ uint16_t conv_update_channel(float* s, const uint16_t* w, const uint16_t* bias_p, uint16_t x,
                                                        int d_conv) {
    const float xv = bf16_bits_to_f32(x);
    if (d_conv <= kConvFastTaps) {
        float sv[kConvFastTaps];
        uint32_t wb[kConvFastTaps];
#pragma unroll
        for (int t = 0; t < kConvFastTaps; ++t) {
            const int i = min(t, d_conv - 1);
            sv[t] = s[i];
            wb[t] = w[i];
        }
        float acc = bf16_bits_to_f32(*bias_p);
#pragma unroll
        for (int t = 0; t + 1 < kConvFastTaps; ++t)
            if (t + 1 < d_conv) acc = fmaf(sv[t + 1], bf16_bits_to_f32(wb[t]), acc);
#pragma unroll
        for (int t = 0; t < kConvFastTaps; ++t)
            if (t + 1 == d_conv) acc = fmaf(xv, bf16_bits_to_f32(wb[t]), acc);
#pragma unroll
        for (int t = 0; t < kConvFastTaps; ++t)
            if (t < d_conv) s[t] = t + 1 < d_conv ? sv[t + 1] : xv;
        return f32_to_bf16_bits(silu(acc));
    }
    float acc = bf16_bits_to_f32(*bias_p);
    for (int t = 0; t + 1 < d_conv; ++t) {
        const float v = s[t + 1];
        s[t] = v;
        acc = fmaf(v, bf16_bits_to_f32(w[t]), acc);
    }
    s[d_conv - 1] = xv;
    acc = fmaf(xv, bf16_bits_to_f32(w[d_conv - 1]), acc);
    return f32_to_bf16_bits(silu(acc));
}

}  // namespace w8a16
