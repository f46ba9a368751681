// Host-side argument checks and kernel launch shared by the entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w8a16.h"

namespace w8a16 {

constexpr int64_t kScaleBlockHost = 128;   // 128 x 128 scale blocks

// Compute units of the current device (cached per device).
int device_cu_count();

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// [lo, lo + bytes) and [lo2, lo2 + bytes2) intersect?
inline bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return abytes > 0 && bbytes > 0 && a0 < b0 + static_cast<uintptr_t>(bbytes) &&
           b0 < a0 + static_cast<uintptr_t>(abytes);
}

inline bool scale_format_valid(int f) {
    return f == W8A16_SCALE_BLOCK_BF16 || f == W8A16_SCALE_BLOCK_F32 || f == W8A16_SCALE_ROW_F32;
}

// Bytes of the scale buffer in format f.
inline int64_t scale_bytes(int f, int64_t N, int64_t K) {
    if (f == W8A16_SCALE_ROW_F32) return N * 4;
    return ceil_div(N, kScaleBlockHost) * ceil_div(K, kScaleBlockHost) * (f == W8A16_SCALE_BLOCK_F32 ? 4 : 2);
}

// Checks shared by the GEMV and GEMM entry points. Returns W8A16_OK or an
// error; *noop is set when there is nothing to compute (M == 0 or N == 0).
inline int check_product_args(const void* A, const void* Wq, const void* scale, const void* out,
                              int64_t M, int64_t N, int64_t K, bool* noop, int fmt = W8A16_SCALE_BLOCK_BF16) {
    *noop = false;
    if (!scale_format_valid(fmt)) return W8A16_ERR_ARG;
    if (M < 0 || N < 0 || K < 16 || (K % 16) != 0 || M > INT32_MAX || N > INT32_MAX ||
        K > INT32_MAX)
        return W8A16_ERR_SHAPE;
    if (M == 0 || N == 0) {
        *noop = true;
        return W8A16_OK;
    }
    if (!A || !Wq || !scale || !out) return W8A16_ERR_NULL;
    if (!aligned(A, 16) || !aligned(Wq, 16) || !aligned(scale, fmt == W8A16_SCALE_BLOCK_BF16 ? 2 : 4) ||
        !aligned(out, 2))
        return W8A16_ERR_ALIGN;
    const int64_t out_bytes = M * N * 2;
    const int64_t scale_bytes = w8a16::scale_bytes(fmt, N, K);
    if (overlaps(out, out_bytes, A, M * K * 2) || overlaps(out, out_bytes, Wq, N * K) ||
        overlaps(out, out_bytes, scale, scale_bytes))
        return W8A16_ERR_ALIAS;
    return W8A16_OK;
}

// Channels per norm group: 0 or K (the whole row), or a multiple of 1024
// that divides K with K <= 16384 (each wave's channels then lie in one group,
// and the groups' sums fit the kernels' LDS).
constexpr int64_t kNormGroupUnit = 1024, kMaxNormGroups = 16;
inline bool norm_group_valid(int64_t group, int64_t K) {
    if (group == 0 || group == K) return true;
    return group > 0 && group % kNormGroupUnit == 0 && K % group == 0 && K <= kNormGroupUnit * kMaxNormGroups;
}

// Checks of the norm arguments (w8a16_norm.hip): shapes, eps, group, NULL,
// 16-byte alignment, and `out` [M][K] overlapping an input.
int check_norm_args(const void* x, const void* gate, const void* weight, float eps, int64_t group,
                    const void* out, int64_t M, int64_t K, bool* noop);

// Skinny GEMM (w8a16_skinny.hip): 1 <= M <= kSkinnyMaxM rows, K <= kSkinnyMaxK, weights
// streamed from HBM straight into the matrix-core operands. Arguments as for
// w8a16_gemm (already checked by the caller); enqueues one kernel on `stream`.
// K above kSkinnyOnePassK takes two passes over the weight block, which pays
// from kSkinnyTwoPassMinM rows on (measured on the Mamba-2 out_proj, K = 8192:
// 18.4 against 21.7 us for the GEMV at M = 16, but 15.2 against 10.1 at M = 4).
constexpr int64_t kSkinnyMaxM = 16;
constexpr int64_t kSkinnyOnePassK = 4096;
constexpr int64_t kSkinnyMaxK = 8192;
constexpr int64_t kSkinnyTwoPassMinM = 12;
constexpr int64_t kSkinnyLdsMaxM = 16;          // the one-shot form: one 16-row block of A
inline bool skinny_fits(int64_t M, int64_t K) {
    return M >= 1 && M <= kSkinnyMaxM &&
           (K <= kSkinnyOnePassK || (K <= kSkinnyMaxK && M >= kSkinnyTwoPassMinM));
}
// One-shot skinny form (one 16-row weight block per workgroup, every weight
// load issued up front, activations in LDS; M <= kSkinnyLdsMaxM): whether it
// applies to (M, N, K) on `cus` CUs, its k-blocks per wave and its
// activation phases (1 to 8).
bool skinny_lds_plan(int64_t M, int64_t N, int64_t K, int cus, int* kb, int* phases);
inline bool skinny_lds_fits(int64_t M, int64_t N, int64_t K, int cus) {
    int kb = 0, phases = 1;
    return skinny_lds_plan(M, N, K, cus, &kb, &phases);
}
int skinny_lds_gemm(const void* A, const void* Wq, const void* scale, int fmt, const void* residual, void* out,
                    int64_t M, int64_t N, int64_t K, hipStream_t stream);
// `residual` ([M][N] BF16, or nullptr) adds the residual epilogue.
int skinny_gemm(const void* A, const void* Wq, const void* scale, int fmt, const void* residual, void* out,
                int64_t M, int64_t N, int64_t K, hipStream_t stream);

// Mid-size GEMM (w8a16_mid.hip): kMidMinM..kMidMaxM rows, K <= kMidMaxK; one
// workgroup per small output tile, K split across its waves, A and W streamed
// into registers. mid_plan returns the tile shape for (M, N, K) on `cus` CUs
// (an index, or -1 when the kernel does not apply); mid_gemm launches it
// (`residual` as for skinny_gemm, BF16 block scales only; `ldo` the row
// stride of out and residual, in elements).
constexpr int64_t kMidMinM = 17;
constexpr int64_t kMidMaxM = 256;
constexpr int64_t kMidMaxK = 32768;
int mid_plan(int64_t M, int64_t N, int64_t K, int cus);
int mid_gemm(const void* A, const void* Wq, const void* scale, int fmt, const void* residual, void* out, int64_t M,
             int64_t N, int64_t K, int64_t ldo, hipStream_t stream);

// Prefill GEMM with 256 x 256 tiles (w8a16_gemm_wide.hip): the weight
// convert is done once per workgroup tile, with the block scale folded in.
// K up to 32768; arguments as for w8a16_gemm (already checked by the
// caller), `residual` as for skinny_gemm (BF16 block scales only).
bool wide_gemm_fits(int64_t M, int64_t N, int64_t K, int64_t ldo);
// Whether the 256 x 256 tiles keep the grid busy: at least one tile per CU
// and every round of CU-many tiles at least 85 % full (a nearly empty last
// round costs a whole tile time; the 128-row kernels then finish first).
bool wide_gemm_pays(int64_t M, int64_t N, int64_t K, int cus);
// Columns [0, n) that whole rounds of CU-many 256 x 256 tiles cover (a
// multiple of 256, 0 if not even one round fits); the rest of the columns go
// to the 128-row tiles.
int64_t wide_gemm_columns(int64_t M, int64_t N, int64_t K, int cus);
// ldo: the row stride of out and residual, in elements (>= N).
int wide_gemm(const void* A, const void* Wq, const void* scale, int fmt, const void* residual, void* out,
              int64_t M, int64_t N, int64_t K, int64_t ldo, hipStream_t stream);

// Launch `kernel` with exactly the argument types of its signature; the HIP
// launch status becomes W8A16_OK / W8A16_ERR_LAUNCH.
template <typename... KArgs>
inline int launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                  KArgs... args) {
    void* argv[] = {static_cast<void*>(&args)...};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, stream);
    return e == hipSuccess ? W8A16_OK : W8A16_ERR_LAUNCH;
}

// Raise `kernel`'s dynamic LDS limit to at least `bytes` on the current
// device (a HIP call only when that raises it); false if that fails.
bool allow_large_lds(const void* kernel, size_t bytes);

// The same with `lds_bytes` of dynamic LDS (above 64 KB the kernel's limit
// is raised first).
template <typename... KArgs>
inline int launch_with_lds(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds_bytes, hipStream_t stream,
                           KArgs... args) {
    if (lds_bytes > 64 * 1024 && !allow_large_lds(reinterpret_cast<const void*>(kernel), lds_bytes))
        return W8A16_ERR_LAUNCH;
    void* argv[] = {static_cast<void*>(&args)...};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, lds_bytes, stream);
    return e == hipSuccess ? W8A16_OK : W8A16_ERR_LAUNCH;
}

}  // namespace w8a16
