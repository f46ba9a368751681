// Skinny GEMM for the w8a16 block-scaled FP8 projection, M <= 16 rows and
// K <= 8192:
//
//   out[m][n] = sum_k A[m][k] * E4M3(W[n][k]) * scale[n/128][k/128]
// (Qwen3SsmLayer docs, `set_fp8_decode_weights`; NemotronMamba2Layer docs,
// `set_fp8_weights`). A few tokens at once (TransformerLayer docs,
// `decode_multi_seq`, and the K-token verify of speculative decoding) read
// every weight once for all rows, so the time is the weight stream from HBM.
//
// The layout follows the decode GEMV (keep many weight loads in flight, keep
// the activations in registers) with the matrix cores doing the products:
//  * K is split across the S waves of a workgroup: wave w owns a contiguous
//    range of at most KB 128-wide k-blocks, and holds the activations of that
//    range (all M rows, as MFMA A operands) in registers for the whole pass;
//    K above 4096 takes two passes, each over half the k-blocks, and the
//    second pass adds its sums to the first's (kept in LDS, fp32);
//  * a workgroup walks a contiguous range of 16-row weight blocks; for each,
//    every wave streams its 16 x (KB * 128)-byte slice straight from HBM into
//    registers, D - 1 blocks ahead (a ring of D blocks; D = 2 measured
//    fastest on the Mamba-2 in_proj shape, D = 3 and 4 were slower);
//  * each k-block is two v_mfma_f32_16x16x32_bf16 steps per 16 rows of A;
//    lane l carries row l % 16 and k = 64c + 16(l / 16) + 8h + [0, 8) of
//    chunk c, step h, for both operands, so one 16-byte load of W feeds both
//    steps of a chunk, and the block scale is applied exactly in fp32
//    (acc += scale * blk);
//  * the S partial 16 x 16 tiles of a block meet in LDS and are added in wave
//    order (ascending k): the result is deterministic;
//  * scale formats: BF16 or FP32 block grids are folded per k-block as above;
//    an FP32 per-row scale multiplies the finished sum of its column before
//    the BF16 rounding (the workgroup's row scales are staged in LDS).
#include <algorithm>
#include <type_traits>

#include "w8a16_device.h"
#include "w8a16_host.h"

namespace w8a16 {
namespace {

constexpr int kRows = 16;                  // weight rows per workgroup (one MFMA column block)
constexpr int kMaxWaves = 16;              // per workgroup
constexpr int kMaxBlocksPerWg = 32;        // 16-row weight blocks per workgroup at most
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kBufferFlags = 0x00020000;   // raw buffer, 32-bit data format
static_assert(kScaleBlock % kRows == 0, "a workgroup's rows share one scale row");

// 8 E4M3 codes (two dwords) -> 8 BF16, exact.
__device__ __forceinline__ bf16x8_t e4m3x8(uint32_t lo, uint32_t hi) {
    const bf16x2_t p0 = e4m3x2_to_bf16(lo, false), p1 = e4m3x2_to_bf16(lo, true);
    const bf16x2_t p2 = e4m3x2_to_bf16(hi, false), p3 = e4m3x2_to_bf16(hi, true);
    return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// MB = 16-row blocks of A (the entry points use 1: M <= 16); KB = k-blocks per
// wave at most (the activations of KB k-blocks take 16 * MB * KB VGPRs); D =
// weight blocks in flight per wave; MAXW = waves per workgroup at most; SF =
// scale format; NPASS = passes over K (1 or 2): in pass p, wave w owns the
// k-blocks from (p * waves + w) * KB, so 16 waves cover K <= NPASS * 4096.
template <int MB, int KB, int D, int MAXW, int SF, int NPASS>
__global__ void __launch_bounds__(64 * MAXW)
skinny_kernel(const uint16_t* __restrict__ A, const uint8_t* __restrict__ W, const void* __restrict__ S,
              const uint16_t* __restrict__ res, uint16_t* __restrict__ out, int M, int N, int K,
              int blocks_per_wg) {
    constexpr bool kRowScale = SF == kScaleRowF32;
    // Partial tiles of the waves, double-buffered by block parity:
    // [parity][wave][mb][lane] x 4 floats.
    __shared__ f32x4_t red[2][MAXW * MB * 64];
    // The workgroup's outputs, written out after the loop (so that the loop
    // issues no vector-memory stores, which would share the loads' counter).
    __shared__ uint16_t outs[kMaxBlocksPerWg * 256 * MB];
    // Per-row scales of the workgroup's weight rows (row format only).
    __shared__ float row_s[kRowScale ? kMaxBlocksPerWg * kRows : 1];
    // Sums of the earlier passes, per output (two passes only).
    static_assert(NPASS == 1 || NPASS == 2, "one or two passes over K");
    __shared__ float part[NPASS > 1 ? kMaxBlocksPerWg * 256 * MB : 1];

    const int waves = blockDim.x / 64;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int lane = threadIdx.x % 64;
    const int r = lane % 16, g = lane / 16;
    const int k_blocks = (K + kScaleBlock - 1) / kScaleBlock;
    const int nblk = (N + kRows - 1) / kRows;
    const int blk0 = blockIdx.x * blocks_per_wg, blk1 = min(nblk, blk0 + blocks_per_wg);
    if (blk0 >= blk1) return;                        // uniform over the workgroup

    // Per-row scales of the workgroup's rows to LDS (read after the first
    // barrier of the loop).
    constexpr int kScaleBytes = SF == kScaleBlockBf16 ? 2 : 4;
    const int scale_elems = kRowScale ? N : ((N + kScaleBlock - 1) / kScaleBlock) * k_blocks;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(S), 0, scale_elems * kScaleBytes, kBufferFlags);
    if constexpr (kRowScale) {
        for (int i = threadIdx.x; i < (blk1 - blk0) * kRows; i += blockDim.x) {
            const int n = blk0 * kRows + i;
            row_s[i] = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(rs, n < N ? static_cast<uint32_t>(n) * 4 : kOutOfRange, 0, 0));
        }
    }
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(A), 0, M * K * 2, kBufferFlags);
    const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
    int parity = 0;

    // Each pass loads its activations and scales, then streams every weight
    // block of the workgroup through the ring; the ring drains at the end of
    // a pass, so the waits are the same in every pass.
    for (int pass = 0; pass < NPASS; ++pass) {
        const int kb0 = (pass * waves + wave) * KB;      // this wave's k-blocks: [kb0, kb0 + KB) within k_blocks

        // Lane's k of chunk c of the wave's j-th k-block (K % 16 == 0, so a
        // lane's 16 bytes are all inside K or all outside).
        auto kof = [&](int j, int c) { return (kb0 + j) * kScaleBlock + 64 * c + 16 * g; };
        uint32_t w_off[KB][2];
#pragma unroll
        for (int j = 0; j < KB; ++j)
#pragma unroll
            for (int c = 0; c < 2; ++c) w_off[j][c] = kof(j, c) < K ? static_cast<uint32_t>(r * K + kof(j, c)) : kOutOfRange;

        // Activations of the wave's k-range, [mb][j][c][h]: 8 BF16 each.
        u32x4_t a[MB][KB][2][2];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < KB; ++j)
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int k = kof(j, c) + 8 * h;
                        a[mb][j][c][h] =
                            __builtin_amdgcn_raw_buffer_load_b128(ra, k < K ? ((mb * 16 + r) * K + k) * 2 : kOutOfRange, 0, 0);
                    }

        // Block scales of the workgroup's rows and the wave's k-blocks: lane l
        // holds scale row srow0 + l / KB, k-block kb0 + l % KB (a workgroup's rows
        // span at most kMaxBlocksPerWg * 16 / 128 + 2 scale rows). Per-row
        // scales are in LDS instead.
        constexpr int kScaleRows = 64 / KB;
        static_assert(kMaxBlocksPerWg * kRows / kScaleBlock + 2 <= kScaleRows, "one scale load per workgroup");
        const int srow0 = blk0 * kRows / kScaleBlock;
        float s_lane = 1.0f;
        if constexpr (SF == kScaleBlockBf16 || SF == kScaleBlockF32) {
            const int srow = srow0 + lane / KB, kb = kb0 + lane % KB;
            const bool ok = srow * kScaleBlock < N && kb < k_blocks;
            const uint32_t off = ok ? static_cast<uint32_t>(srow * k_blocks + kb) * kScaleBytes : kOutOfRange;
            if constexpr (SF == kScaleBlockBf16)
                s_lane = bf16_bits_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0));
            else
                s_lane = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
        }

        // Weights of row block b into a ring slot: [j][c], 16 bytes each; rows
        // past N read zeros (beyond the buffer's range). Blocks past the
        // workgroup's range get an empty range and load zeros: the loads are the
        // same in every step (so the waits are too, also the compiler's own).
        u32x4_t wr[D][KB][2];
        auto issue = [&](int b, u32x4_t (&dst)[KB][2]) {
            const bool live = b < blk1;
            const int n0 = (live ? b : blk0) * kRows;
            const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint8_t*>(W + static_cast<int64_t>(n0) * K), 0, live ? min(kRows, N - n0) * K : 0,
                kBufferFlags);
#pragma unroll
            for (int j = 0; j < KB; ++j)
#pragma unroll
                for (int c = 0; c < 2; ++c) dst[j][c] = __builtin_amdgcn_raw_buffer_load_b128(rw, w_off[j][c], 0, 0);
        };
#pragma unroll
        for (int d = 0; d < D; ++d) issue(blk0 + d, wr[d]);

        // Block bb in ring slot d: wait for its loads (the later blocks' stay in
        // flight), multiply, refill the slot with block bb + D, then reduce.
        auto block = [&](int bb, u32x4_t (&w)[KB][2]) {
            // Loads in flight, oldest first: this block, then the D - 1 later ones.
            wait_vmem<(D - 1) * 2 * KB>();
            __builtin_amdgcn_sched_barrier(0);
            const int srow = bb * kRows / kScaleBlock;   // srow - srow0 < kScaleRows
            f32x4_t acc[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[mb] = zero;
#pragma unroll
            for (int j = 0; j < KB; ++j) {
                const float s =
                    __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s_lane), (srow - srow0) * KB + j));
                f32x4_t blk[MB];
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const bf16x8_t bw0 = e4m3x8(w[j][c][0], w[j][c][1]), bw1 = e4m3x8(w[j][c][2], w[j][c][3]);
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb)
                            blk[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8_t, a[mb][j][c][h]), h ? bw1 : bw0,
                                (c == 0 && h == 0) ? zero : blk[mb], 0, 0, 0);
                }
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[mb][v] = fmaf(blk[mb][v], s, acc[mb][v]);
            }
            issue(bb + D, w);
            // 16x16 MFMA result layout: lane l holds column l % 16, rows
            // 4(l/16) + v. Thread t < 256 * MB then writes output (row, column) =
            // (t / 16, t % 16): the sum over the waves in k order.
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) red[parity][(wave * MB + mb) * 64 + lane] = acc[mb];
            __syncthreads();
            if (threadIdx.x < 256 * MB) {                // blockDim.x >= 256 * MB
                const int t = threadIdx.x;
                const int row = t / 16, col = t % 16;
                const int mb = row / 16, rr = row % 16;
                const int l = col + 16 * (rr / 4), v = rr % 4;
                float sum = red[parity][mb * 64 + l][v];
                for (int w2 = 1; w2 < waves; ++w2) sum += red[parity][(w2 * MB + mb) * 64 + l][v];
                if (bb < blk1) {
                    // Two passes: the first pass's sum, then the second's added to
                    // it (the same thread writes and reads an output's slot).
                    const int o = (bb - blk0) * 256 * MB + t;
                    if constexpr (NPASS > 1) {
                        if (pass == 0) part[o] = sum;
                        else sum = part[o] + sum;
                    }
                    if (pass == NPASS - 1) {
                        if constexpr (kRowScale) sum *= row_s[(bb - blk0) * kRows + col];
                        outs[o] = f32_to_bf16_bits(sum);
                    }
                }
            }
            // red[parity] is written again two blocks later, after the next
            // barrier, which every thread reaches only once done reading it.
            parity ^= 1;
        };
        // D blocks per iteration, the last iteration padded with blocks past the
        // range (their weights load as zeros and their outputs are dropped): the
        // loads and waits are the same in every iteration.
        static_assert(D >= 2 && D <= 4, "ring of 2 to 4 blocks");
        for (int b = blk0; b < blk1; b += D) {
            block(b, wr[0]);
            block(b + 1, wr[1]);
            if constexpr (D >= 3) block(b + 2, wr[2]);
            if constexpr (D >= 4) block(b + 3, wr[3]);
        }
        wait_vmem<0>();                                  // the zero loads past the range
    }
    __syncthreads();
    // Output (row, column n0 + col) of block b sits at outs[(b - blk0) * 256 *
    // MB + row * 16 + col]; threads take 16-column runs of one row.
    const int per_row = blk1 - blk0;
    for (int i = threadIdx.x; i < per_row * 16 * 16 * MB; i += blockDim.x) {
        const int row = i / (per_row * 16), rest = i % (per_row * 16);
        const int b = rest / 16, col = rest % 16;
        const int n = (blk0 + b) * kRows + col;
        if (row < M && n < N) {
            const int64_t o = static_cast<int64_t>(row) * N + n;
            const uint16_t y = outs[b * 256 * MB + row * 16 + col];
            out[o] = res ? residual_add_bits(y, res[o]) : y;      // residual epilogue, if any
        }
    }
}

// ---------------------------------------------------------------------------
// One-shot form: every weight load of a workgroup is issued at its start, as
// the decode GEMV's one-group workgroups do, so the HBM pipe never waits for
// a workgroup's arithmetic or barriers, and the workgroups are small and many
// (one 16-row weight block each), which a plain read of W measures as the
// fastest way to stream it. The registers the ring form spends on
// activations go to the weights here: the activations (all M rows, all of K,
// at most 128 KB; above that, half of K at a time in two phases) are copied
// to LDS by DMA at the start of every workgroup and each wave reads its MFMA
// A operands from LDS. 8 waves per workgroup; in each phase wave w owns the
// phase's k-blocks [w*KB/PH, (w+1)*KB/PH); the 8 partial 16 x 16 tiles are
// added in LDS in wave order, so the result is deterministic. (Measured and
// not kept, on the Mamba-2 shapes: several blocks per workgroup, strided or
// contiguous, one workgroup per CU: 20-23 against 17-18 us for in_proj at
// M = 1..4; the activations in registers instead of LDS: 10.6-33 against
// 9.0-26 us.)
constexpr int kLdsWaves = 8;
constexpr int kLdsABytes = 128 * 1024;          // activation region of one phase: M * Kpad * 2 / PH bytes at most

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void lds_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Activation chunk (8 BF16 of one row, logical chunk q = k / 8) at LDS chunk
// (q & ~15) | ((q ^ m) & 15) of row m: the 16 rows an MFMA operand read
// touches at one k land in 16 different 16-byte slots of a 256-byte line.
__device__ __forceinline__ int a_chunk_swz(int q, int m) { return (q & ~15) | ((q ^ m) & 15); }

template <int KB, int PH, int SF>
__global__ void __launch_bounds__(64 * kLdsWaves, 1)
skinny_lds_kernel(const uint16_t* __restrict__ A, const uint8_t* __restrict__ W, const void* __restrict__ S,
                  const uint16_t* __restrict__ res, uint16_t* __restrict__ out, int M, int N, int K) {
    constexpr bool kRowScale = SF == kScaleRowF32;
    constexpr int KBP = KB / PH;                        // k-blocks per wave and phase
    static_assert(PH >= 1 && PH <= 8 && KB % PH == 0, "phases of whole k-blocks");
    constexpr int MB = 1;                               // one 16-row block of A
    constexpr int kLoads = KB * 2;                      // weight loads per lane
    static_assert(kLoads < 64, "vmcnt field");
    extern __shared__ __attribute__((aligned(16))) uint8_t a_lds[];   // M * kph * 2 bytes, rounded to 1 KB
    __shared__ f32x4_t red[kLdsWaves * 64];
    __shared__ uint16_t outs[256 * MB];
    __shared__ float row_s[kRowScale ? kRows : 1];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int lane = threadIdx.x % 64;
    const int r = lane % 16, g = lane / 16;
    const int k_blocks = (K + kScaleBlock - 1) / kScaleBlock;
    const int kph = kLdsWaves * KBP * kScaleBlock;      // K of one phase (K padded to the waves' k-blocks / PH)
    const int b = blockIdx.x;                           // this workgroup's 16-row weight block
    const int n0 = b * kRows;
    // Global k-block of the wave's j-th k-block (phase j / KBP).
    auto kblock = [&](int j) { return (j / KBP) * (kLdsWaves * KBP) + wave * KBP + j % KBP; };

    // Activations of phase p to LDS by DMA: LDS chunk e (16 bytes) holds row
    // e / cph, logical chunk q (k = p * kph + 8q) with a_chunk_swz(q, m) ==
    // e % cph; chunks past K read as zero.
    const int cph = kph / 8;                            // 16-byte chunks per row and phase
    const int nch = M * cph;
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(A), 0, M * K * 2, kBufferFlags);
    auto stage_a = [&](int p) {
        for (int i = wave; i * 64 < nch; i += kLdsWaves) {
            const int e = i * 64 + lane;
            const int m = e / cph, pc = e - m * cph;
            const int k = p * kph + a_chunk_swz(pc, m) * 8;   // the swizzle is its own inverse
            const uint32_t off = (e < nch && k < K) ? static_cast<uint32_t>((m * K + k) * 2) : kOutOfRange;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(a_lds + i * 1024), 16, off, 0, 0, 0);
        }
    };
    stage_a(0);

    // Scales: lane l holds the block's scale for the wave's k-block l % KB
    // (block formats); the row format's 16 row scales go to LDS.
    constexpr int kScaleBytes = SF == kScaleBlockBf16 ? 2 : 4;
    const int scale_elems = kRowScale ? N : ((N + kScaleBlock - 1) / kScaleBlock) * k_blocks;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(S), 0, scale_elems * kScaleBytes, kBufferFlags);
    float s_lane = 1.0f;
    if constexpr (SF == kScaleBlockBf16 || SF == kScaleBlockF32) {
        const int kb = kblock(lane % KB);
        const uint32_t off =
            kb < k_blocks ? static_cast<uint32_t>((n0 / kScaleBlock) * k_blocks + kb) * kScaleBytes : kOutOfRange;
        if constexpr (SF == kScaleBlockBf16)
            s_lane = bf16_bits_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0));
        else
            s_lane = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
    } else {
        if (threadIdx.x < kRows) {
            const int n = n0 + threadIdx.x;
            row_s[threadIdx.x] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                rs, n < N ? static_cast<uint32_t>(n) * 4 : kOutOfRange, 0, 0));
        }
    }

    // Every weight load of the workgroup, phase by phase: k-block j, chunk c
    // (16 codes of row r from k = kblock(j)*128 + 64c + 16g). Rows past N and
    // k past K read zeros.
    u32x4_t w[KB][2];
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(W + static_cast<int64_t>(n0) * K), 0, min(kRows, N - n0) * K, kBufferFlags);
#pragma unroll
    for (int j = 0; j < KB; ++j)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int k = kblock(j) * kScaleBlock + 64 * c + 16 * g;
            w[j][c] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rw, k < K ? static_cast<uint32_t>(r * K + k) : kOutOfRange, 0, 0));
        }
    __builtin_amdgcn_sched_barrier(0);

    // MFMA A operand of row block mb, (k-block j, chunk c, half h): row
    // min(16mb + r, M - 1) (rows past M feed output rows that are never
    // stored), k = kblock(j)*128 + 64c + 16g + 8h, the same k-slot order as
    // the weights. One decoded weight fragment feeds all MB row blocks.
    int am[MB];
    const uint8_t* a_row[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        am[mb] = min(16 * mb + r, M - 1);
        a_row[mb] = a_lds + am[mb] * (cph * 16);
    }
    const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
    f32x4_t acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = zero;
#pragma unroll
    for (int p = 0; p < PH; ++p) {
        if (p == 0) {
            // The activations (and scales) are older than every weight load:
            // wait for them (and this wave's LDS writes) only, then make the
            // DMA's LDS writes visible. (__syncthreads would also wait for
            // every weight load in flight.)
            __builtin_amdgcn_s_waitcnt((kLoads & 15) | (0x7 << 4) | ((kLoads >> 4) << 14));
        } else {
            // Every wave is done reading phase p - 1's activations; stage
            // phase p's (the youngest loads: waiting for them waits for all).
            __builtin_amdgcn_s_waitcnt(15 | (0x7 << 4) | (0x3 << 14));   // LDS reads only
            lds_sync();
            stage_a(p);
            __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
        }
        lds_sync();
#pragma unroll
        for (int jj = 0; jj < KBP; ++jj) {
            const int j = p * KBP + jj;
            const float s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s_lane), j));
            f32x4_t blk[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) blk[mb] = zero;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const bf16x8_t bw0 = e4m3x8(w[j][c][0], w[j][c][1]), bw1 = e4m3x8(w[j][c][2], w[j][c][3]);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int q = ((wave * KBP + jj) * kScaleBlock + 64 * c + 16 * g + 8 * h) / 8;
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        const u32x4_t av = *reinterpret_cast<const u32x4_t*>(a_row[mb] + a_chunk_swz(q, am[mb]) * 16);
                        blk[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                                          h ? bw1 : bw0, blk[mb], 0, 0, 0);
                    }
                }
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[mb][v] = fmaf(blk[mb][v], s, acc[mb][v]);
        }
    }
    // Lane l holds output column l % 16, rows 16mb + 4(l/16) + v; thread
    // t < 256 adds output (row 16mb + t / 16, column t % 16) over the waves
    // in order of their k-blocks (phase-major, so the order is fixed), one
    // row block at a time.
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        red[wave * 64 + lane] = acc[mb];
        __syncthreads();
        if (threadIdx.x < 256) {
            const int t = threadIdx.x, rr = t / 16, col = t % 16;
            const int l = col + 16 * (rr / 4), v = rr % 4;
            float sum = red[l][v];
#pragma unroll
            for (int w2 = 1; w2 < kLdsWaves; ++w2) sum += red[w2 * 64 + l][v];
            if constexpr (kRowScale) sum *= row_s[col];
            outs[mb * 256 + t] = f32_to_bf16_bits(sum);
        }
        __syncthreads();
    }
    // Outputs: (row, column) at outs[row * 16 + column].
    for (int e = threadIdx.x; e < M * 16; e += blockDim.x) {
        const int row = e / 16, col = e % 16, n = n0 + col;
        if (n < N) {
            const int64_t o = static_cast<int64_t>(row) * N + n;
            const uint16_t y = outs[row * 16 + col];
            out[o] = res ? residual_add_bits(y, res[o]) : y;
        }
    }
}

template <int KB, int SF>
int launch_lds(int phases, dim3 grid, hipStream_t s, const uint16_t* a, const uint8_t* w, const void* scale,
               const uint16_t* r, uint16_t* o, int m, int n, int k) {
    const size_t lds = static_cast<size_t>((m * KB / phases * kLdsWaves * kScaleBlock * 2 + 1023) / 1024 * 1024);
    const dim3 block(64 * kLdsWaves);
    switch (phases) {
        case 8:
            if constexpr (KB % 8 == 0)
                return launch_with_lds(&skinny_lds_kernel<KB, 8, SF>, grid, block, lds, s, a, w, scale, r, o, m, n, k);
            break;
        case 4:
            if constexpr (KB % 4 == 0)
                return launch_with_lds(&skinny_lds_kernel<KB, 4, SF>, grid, block, lds, s, a, w, scale, r, o, m, n, k);
            break;
        case 2:
            if constexpr (KB % 2 == 0)
                return launch_with_lds(&skinny_lds_kernel<KB, 2, SF>, grid, block, lds, s, a, w, scale, r, o, m, n, k);
            break;
        default:
            return launch_with_lds(&skinny_lds_kernel<KB, 1, SF>, grid, block, lds, s, a, w, scale, r, o, m, n, k);
    }
    return W8A16_ERR_SHAPE;
}

}  // namespace

// The one-shot form where it applies (skinny_lds_plan); otherwise the ring
// form: M <= 16, K <= 8192 (one pass over K up to 4096, two above). Waves per
// workgroup: enough that each holds at most two k-blocks of activations per
// pass, at least 4. The grid aims at about 16 resident waves per CU, each
// workgroup taking a contiguous range of 16-row weight blocks.
int skinny_gemm(const void* A, const void* Wq, const void* scale, int fmt, const void* residual, void* out,
                int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    if (skinny_lds_fits(M, N, K, device_cu_count()))
        return skinny_lds_gemm(A, Wq, scale, fmt, residual, out, M, N, K, stream);
    if (M < 1 || M > kSkinnyMaxM) return W8A16_ERR_SHAPE;
    if (!skinny_fits(M, K)) return W8A16_ERR_SHAPE;
    const int kb_max = 2;
    const int64_t k_blocks = ceil_div(K, kScaleBlockHost);
    // Buffer offsets and sizes are 32-bit.
    if (static_cast<int64_t>(kRows) * K >= static_cast<int64_t>(kOutOfRange) ||
        scale_bytes(fmt, N, K) >= static_cast<int64_t>(kOutOfRange))
        return W8A16_ERR_SHAPE;
    const int passes = k_blocks > kMaxWaves * kb_max ? 2 : 1;
    int waves = static_cast<int>(ceil_div(k_blocks, kb_max * passes));
    waves = std::max(waves, 4);
    const int64_t nblk = ceil_div(N, kRows);
    if (nblk > INT32_MAX) return W8A16_ERR_SHAPE;
    const int64_t resident = std::max<int64_t>(1, 16 / waves) * device_cu_count();
    const int64_t per_wg = std::min<int64_t>(kMaxBlocksPerWg, ceil_div(nblk, resident));
    const dim3 grid(static_cast<unsigned>(ceil_div(nblk, per_wg))), block(64 * waves);
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K), p = static_cast<int>(per_wg);
    auto a = static_cast<const uint16_t*>(A);
    auto w = static_cast<const uint8_t*>(Wq);
    auto o = static_cast<uint16_t*>(out);
    auto r = static_cast<const uint16_t*>(residual);
    switch (fmt) {
        case W8A16_SCALE_BLOCK_BF16:
            return passes == 1
                       ? launch(&skinny_kernel<1, 2, 2, 16, kScaleBlockBf16, 1>, grid, block, stream, a, w, scale, r, o, m, n, k, p)
                       : launch(&skinny_kernel<1, 2, 2, 16, kScaleBlockBf16, 2>, grid, block, stream, a, w, scale, r, o, m, n, k, p);
        case W8A16_SCALE_BLOCK_F32:
            return passes == 1
                       ? launch(&skinny_kernel<1, 2, 2, 16, kScaleBlockF32, 1>, grid, block, stream, a, w, scale, r, o, m, n, k, p)
                       : launch(&skinny_kernel<1, 2, 2, 16, kScaleBlockF32, 2>, grid, block, stream, a, w, scale, r, o, m, n, k, p);
        case W8A16_SCALE_ROW_F32:
            return passes == 1
                       ? launch(&skinny_kernel<1, 2, 2, 16, kScaleRowF32, 1>, grid, block, stream, a, w, scale, r, o, m, n, k, p)
                       : launch(&skinny_kernel<1, 2, 2, 16, kScaleRowF32, 2>, grid, block, stream, a, w, scale, r, o, m, n, k, p);
        default:
            return W8A16_ERR_ARG;
    }
}

// The one-shot form's k-blocks per wave for (M, N, K) on `cus` CUs; false
// where it does not apply: K above 8 * 8 k-blocks, activations above the
// LDS budget, or (with more weight blocks than CUs) above 32 KB, where fewer
// than three workgroups fit a CU and the ring form is faster (measured on the
// Mamba-2 in_proj: 23 against 20 us at M = 8).
bool skinny_lds_plan(int64_t M, int64_t N, int64_t K, int cus, int* kb, int* phases) {
    if (M < 1 || M > kSkinnyLdsMaxM || N < 1 || K < 16 || cus < 1) return false;
    const int64_t k_blocks = ceil_div(K, kScaleBlockHost);
    int per_wave = 1;
    while (per_wave * kLdsWaves < k_blocks) per_wave *= 2;
    if (per_wave > 8) return false;
    if (static_cast<int64_t>(kRows) * K >= static_cast<int64_t>(kOutOfRange)) return false;
    const int64_t nblk = ceil_div(N, kRows);
    if (nblk > INT32_MAX) return false;
    const int64_t a_bytes = M * per_wave * kLdsWaves * kScaleBlockHost * 2;
    // Activations over the LDS budget go in phases of a part of K each; each
    // phase's copy waits for the previous phase's products. The budget:
    // 128 KB where every weight block has a CU of its own, else 32 KB (so
    // that several workgroups share a CU and cover each other's copies) and
    // no more than two phases (measured on the Mamba-2 in_proj: 19.5 against
    // 20.0 us for the ring form at M = 8 in two phases; 23.1 against 21.4 at
    // M = 16 in four).
    const bool own_cu = nblk <= cus;
    const int64_t budget = own_cu ? kLdsABytes : 32 * 1024;
    int ph = 1;
    while (a_bytes > ph * budget && ph < (own_cu ? 8 : 2)) ph *= 2;
    if (a_bytes > ph * budget || per_wave % ph != 0) return false;
    *phases = ph;
    *kb = per_wave;
    return true;
}

int skinny_lds_gemm(const void* A, const void* Wq, const void* scale, int fmt, const void* residual, void* out,
                    int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    int kb = 0, phases = 1;
    if (!skinny_lds_plan(M, N, K, device_cu_count(), &kb, &phases)) return W8A16_ERR_SHAPE;
    if (scale_bytes(fmt, N, K) >= static_cast<int64_t>(kOutOfRange)) return W8A16_ERR_SHAPE;
    const dim3 grid(static_cast<unsigned>(ceil_div(N, kRows)));
    auto a = static_cast<const uint16_t*>(A);
    auto w = static_cast<const uint8_t*>(Wq);
    auto o = static_cast<uint16_t*>(out);
    auto r = static_cast<const uint16_t*>(residual);
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
    auto by_kb = [&](auto sf) {
        constexpr int SF = decltype(sf)::value;
        switch (kb) {
            case 1: return launch_lds<1, SF>(phases, grid, stream, a, w, scale, r, o, m, n, k);
            case 2: return launch_lds<2, SF>(phases, grid, stream, a, w, scale, r, o, m, n, k);
            case 4: return launch_lds<4, SF>(phases, grid, stream, a, w, scale, r, o, m, n, k);
            default: return launch_lds<8, SF>(phases, grid, stream, a, w, scale, r, o, m, n, k);
        }
    };
    switch (fmt) {
        case W8A16_SCALE_BLOCK_BF16: return by_kb(std::integral_constant<int, kScaleBlockBf16>{});
        case W8A16_SCALE_BLOCK_F32: return by_kb(std::integral_constant<int, kScaleBlockF32>{});
        case W8A16_SCALE_ROW_F32: return by_kb(std::integral_constant<int, kScaleRowF32>{});
        default: return W8A16_ERR_ARG;
    }
}

}  // namespace w8a16
