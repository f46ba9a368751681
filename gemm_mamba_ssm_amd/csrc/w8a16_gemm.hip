// Prefill GEMM for the w8a16 block-scaled FP8 projection (any M).
//
//   out[m][n] = sum_k A[m][k] * E4M3(W[n][k]) * scale[n/128][k/128]
// (Qwen3SsmLayer docs, `set_fp8_decode_weights`; NemotronMamba2Layer docs,
// `set_fp8_weights`). Prefill reads the weights once for all prompt tokens
// as one GEMM with M = tokens (TransformerLayer docs, `prefill`).
//
// The pages measure (nemotron_mamba2.rs, `set_bf16_weights` docs) that a
// prefill GEMM which rewrites a dequantized weight tile in shared memory for
// every M-block pays N*K*M/M_TILE of that work. Here the raw E4M3 bytes are
// staged once per workgroup tile and never rewritten: each wave decodes the
// 16-byte rows it feeds to the matrix cores in registers, with the exact
// packed E4M3->BF16 convert, right before the MFMA that uses them.
//
// Tiling (CDNA4: 64-wide wavefronts, bf16 MFMA v_mfma_f32_32x32x16_bf16,
// 160 KB LDS with 64 four-byte banks, direct-to-LDS buffer loads):
//  * workgroup tile TM x TN x TK = 128 x 128 x 64, 4 waves in a 2 x 2 grid,
//    each wave a 64 x 64 sub-tile = 2 x 2 MFMA blocks of 32 x 32;
//  * A (BF16) and W (E4M3 bytes) tiles go from HBM straight into LDS with
//    buffer_load_dwordx4 ... lds (no register staging, no ds_write); lanes
//    whose 16 bytes fall outside the matrix get an offset past the buffer's
//    range and so load zeros (M, N and K tails need no branches);
//  * three LDS stages: the tile for step kt+2 is in flight while step kt is
//    multiplied;
//  * LDS layouts are XOR-swizzled so both the 16-byte DMA writes and the
//    one-row-per-lane operand reads hit 16 distinct 16-byte slots of a
//    256-byte bank line: A rows are 128 bytes (chunk c of row r at
//    c ^ ((r >> 1) & 7)), W rows are 64 bytes (chunk c at c ^ ((r >> 2) & 3));
//  * the MFMA's k-slots are assigned so that one 16-byte W read (16
//    consecutive k of one row) feeds two consecutive MFMA steps: lane group g
//    of the step (j, h) carries k = 32j + 16g + 8h + [0, 8) for both operands;
//  * the block scale is applied exactly, in fp32: the MFMAs of one 128-wide
//    k-block accumulate into `blk`, which is then added to the result as
//    acc += scale * blk (TN = 128 keeps a wave's columns in one scale row).
#include <type_traits>

#include "w8a16_device.h"
#include "w8a16_host.h"

namespace w8a16 {
namespace {

constexpr int TM = 128, TN = 128, TK = 64;
constexpr int kThreads = 256;
constexpr int kStages = 3;
constexpr int kATileBytes = TM * TK * 2;            // 16 KB of BF16
constexpr int kWTileBytes = TN * TK;                // 8 KB of E4M3
constexpr int kStageBytes = kATileBytes + kWTileBytes;
constexpr int kAChunksPerThread = kATileBytes / 16 / kThreads;   // 4
constexpr int kWChunksPerThread = kWTileBytes / 16 / kThreads;   // 2
constexpr uint32_t kOutOfRange = 0x80000000u;       // buffer offset that reads as zero
constexpr int kBufferFlags = 0x00020000;            // raw buffer, 32-bit data format

static_assert(kScaleBlock % TN == 0 && kScaleBlock == 2 * TK, "two k-steps per scale block");

typedef __attribute__((address_space(3))) void lds_void;

// Byte offset of 16-byte chunk `c` of row `r` inside a staged tile.
__device__ __forceinline__ int a_slot(int r, int c) { return r * (TK * 2) + ((c ^ ((r >> 1) & 7)) << 4); }
__device__ __forceinline__ int w_slot(int r, int c) { return r * TK + ((c ^ ((r >> 2) & 3)) << 4); }

// Workgroups are handed to the 8 XCDs round-robin (block b runs on XCD b % 8),
// and each XCD has its own L2. Remap so that XCD x receives a contiguous range
// of tile ids, ordered with the M-tile fastest: the M-tiles that share one
// weight strip then run on the same XCD, and the strip is fetched into that
// L2 once. The map is a bijection on [0, tiles).
constexpr int kXcds = 8;

__device__ __forceinline__ int xcd_tile(int b, int tiles) {
    const int q = tiles / kXcds, r = tiles % kXcds;
    const int x = b % kXcds;
    return x * q + min(x, r) + b / kXcds;
}

// 8 E4M3 codes (two dwords) -> 8 BF16, exact.
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
    const bf16x2_t p0 = e4m3x2_to_bf16(lo, false), p1 = e4m3x2_to_bf16(lo, true);
    const bf16x2_t p2 = e4m3x2_to_bf16(hi, false), p3 = e4m3x2_to_bf16(hi, true);
    return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Wait until at most N vector-memory operations of this wave are in flight
// (the LDS-DMA loads of the stages after the one about to be read).
template <int N>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

__global__ void __launch_bounds__(kThreads, 2)
gemm_kernel(const uint16_t* __restrict__ A, const uint8_t* __restrict__ W,
            const uint16_t* __restrict__ S, uint16_t* __restrict__ out,
            int M, int N, int K, int tiles_m) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * kStageBytes];

    const int tile = xcd_tile(blockIdx.x, gridDim.x);
    const int tm = tile % tiles_m, tn = tile / tiles_m;
    const int m0 = tm * TM, n0 = tn * TN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int li = lane & 31, lg = lane >> 5;
    const int k_blocks = (K + kScaleBlock - 1) / kScaleBlock;
    const int nk = (K + TK - 1) / TK;

    // Buffer resources over this tile's rows of A and W: rows past M or N lie
    // beyond num_records and read as zero.
    const int rows_a = min(TM, M - m0), rows_w = min(TN, N - n0);
    const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(A + static_cast<int64_t>(m0) * K), 0, rows_a * K * 2, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rsrc_w = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(W + static_cast<int64_t>(n0) * K), 0, rows_w * K, kBufferFlags);

    // Per-thread DMA source offsets at k0 = 0 (the lane's LDS destination is
    // fixed by the instruction: base + 16 * lane).
    uint32_t a_off[kAChunksPerThread], w_off[kWChunksPerThread];
    int a_k[kAChunksPerThread], w_k[kWChunksPerThread];
#pragma unroll
    for (int i = 0; i < kAChunksPerThread; ++i) {
        const int o = i * (kThreads * 16) + wave * 1024 + lane * 16;     // byte offset in the A tile
        const int r = o / (TK * 2), p = (o / 16) % 8, c = p ^ ((r >> 1) & 7);
        a_k[i] = c * 8;
        a_off[i] = static_cast<uint32_t>(r * K + c * 8) * 2;
    }
#pragma unroll
    for (int i = 0; i < kWChunksPerThread; ++i) {
        const int o = i * (kThreads * 16) + wave * 1024 + lane * 16;     // byte offset in the W tile
        const int r = o / TK, p = (o / 16) % 4, c = p ^ ((r >> 2) & 3);
        w_k[i] = c * 16;
        w_off[i] = static_cast<uint32_t>(r * K + c * 16);
    }

    // DMA of k-step kt into stage `slot`. A full k-step passes k0 as the
    // scalar offset; the K-tail step checks each lane's k and sends lanes past
    // K out of range (they load zeros).
    auto issue = [&](int kt, int slot) {
        const int k0 = kt * TK;
        uint8_t* base = smem + slot * kStageBytes;
        const bool full = k0 + TK <= K;
#pragma unroll
        for (int i = 0; i < kAChunksPerThread; ++i) {
            lds_void* dst = (lds_void*)(base + i * (kThreads * 16) + wave * 1024);
            if (full)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_a, dst, 16, a_off[i], k0 * 2, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsrc_a, dst, 16, (k0 + a_k[i] < K) ? a_off[i] + k0 * 2 : kOutOfRange, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < kWChunksPerThread; ++i) {
            lds_void* dst = (lds_void*)(base + kATileBytes + i * (kThreads * 16) + wave * 1024);
            if (full)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_w, dst, 16, w_off[i], k0, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsrc_w, dst, 16, (k0 + w_k[i] < K) ? w_off[i] + k0 : kOutOfRange, 0, 0, 0);
        }
    };

    // Lane-constant operand addresses inside a stage; the stage is added as
    // an immediate offset. A: [bi][j][h], W: [bj][j].
    int a_addr[2][2][2], w_addr[2][2];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h) a_addr[bi][j][h] = a_slot(wm * 64 + bi * 32 + li, 4 * j + 2 * lg + h);
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
        for (int j = 0; j < 2; ++j) w_addr[bj][j] = kATileBytes + w_slot(wn * 64 + bj * 32 + li, 2 * j + lg);

    f32x16_t acc[2][2], blk[2][2];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[bi][bj][v] = 0.0f;
    const f32x16_t zero = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f,
                           0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};

    // One k-step on stage SLOT: 12 operand reads, 32 converts, 16 MFMAs. The
    // first k-step of a scale block starts the block accumulator from zero.
    auto compute = [&](auto slot_c, auto first_c) {
        constexpr int kSlot = decltype(slot_c)::value;
        constexpr bool kFirst = decltype(first_c)::value;
        const uint8_t* stage = smem + kSlot * kStageBytes;
#pragma unroll
        for (int j = 0; j < 2; ++j) {               // two 32-wide k spans
            bf16x8_t bw[2][2];                      // [bj][h]
#pragma unroll
            for (int bj = 0; bj < 2; ++bj) {
                const u32x4_t q = *reinterpret_cast<const u32x4_t*>(stage + w_addr[bj][j]);
                bw[bj][0] = e4m3x8_to_bf16(q[0], q[1]);
                bw[bj][1] = e4m3x8_to_bf16(q[2], q[3]);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                bf16x8_t av[2];
#pragma unroll
                for (int bi = 0; bi < 2; ++bi)
                    av[bi] = *reinterpret_cast<const bf16x8_t*>(stage + a_addr[bi][j][h]);
#pragma unroll
                for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                    for (int bj = 0; bj < 2; ++bj)
                        blk[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            av[bi], bw[bj][h], (kFirst && j == 0 && h == 0) ? zero : blk[bi][bj], 0, 0, 0);
            }
        }
    };

    // The tile's scale row, 64 k-blocks at a time: lane l holds block base + l,
    // so the main loop issues no vector memory operation besides the DMA.
    const uint16_t* s_row = S + static_cast<int64_t>(tn) * k_blocks;
    auto load_scales = [&](int base) {
        return (base + lane < k_blocks) ? bf16_bits_to_f32(s_row[base + lane]) : 0.0f;
    };
    float s_lane = load_scales(0);

    auto fold = [&](int kb) {
        if ((kb & 63) == 0 && kb > 0) s_lane = load_scales(kb);
        const float s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s_lane), kb & 63));
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
            for (int bj = 0; bj < 2; ++bj)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[bi][bj][v] = fmaf(blk[bi][bj][v], s, acc[bi][bj][v]);
    };

    // k-step kt reads stage kt % 3. Before it: wait for this wave's DMA of kt
    // (at most the next step's loads remain in flight), then a barrier, after
    // which every wave's DMA of kt has landed and every wave is done reading
    // stage (kt + 2) % 3 == (kt - 1) % 3, which is refilled with step kt + 2.
    // FIRST: kt is even (the first k-step of a scale block); the unrolled
    // loop below starts at multiples of 6, so the parity is static.
    auto step = [&](auto slot_c, auto first_c, int kt) {
        constexpr int kSlot = decltype(slot_c)::value;
        constexpr bool kFirst = decltype(first_c)::value;
        if (kt + 1 < nk)
            wait_vmem<kAChunksPerThread + kWChunksPerThread>();
        else
            wait_vmem<0>();
        __builtin_amdgcn_s_barrier();
        if (kt + 2 < nk) issue(kt + 2, (kSlot + 2) % kStages);
        compute(slot_c, first_c);
        if (!kFirst || kt + 1 == nk) fold(kt >> 1);
    };

    issue(0, 0);
    if (nk > 1) issue(1, 1);
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using F = std::true_type;
    using L = std::false_type;
    for (int kt = 0; kt < nk; kt += 2 * kStages) {   // six k-steps: stages 0,1,2,0,1,2
        step(S0{}, F{}, kt);
        if (kt + 1 < nk) step(S1{}, L{}, kt + 1);
        if (kt + 2 < nk) step(S2{}, F{}, kt + 2);
        if (kt + 3 < nk) step(S0{}, L{}, kt + 3);
        if (kt + 4 < nk) step(S1{}, F{}, kt + 4);
        if (kt + 5 < nk) step(S2{}, L{}, kt + 5);
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
                const int m = m0 + wm * 64 + bi * 32 + 8 * (v >> 2) + 4 * lg + (v & 3);
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
    // Buffer offsets are 32-bit: one tile's rows of A must span less than 2 GiB.
    if (static_cast<int64_t>(TM) * K * 2 >= static_cast<int64_t>(kOutOfRange)) return W8A16_ERR_SHAPE;
    const int64_t tiles_m = ceil_div(M, TM);
    const int64_t tiles = tiles_m * ceil_div(N, TN);
    if (tiles > INT32_MAX) return W8A16_ERR_SHAPE;
    return launch(&gemm_kernel, dim3(static_cast<unsigned>(tiles)), dim3(kThreads),
                  static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(A),
                  static_cast<const uint8_t*>(Wq), static_cast<const uint16_t*>(scale),
                  static_cast<uint16_t*>(out), static_cast<int>(M), static_cast<int>(N),
                  static_cast<int>(K), static_cast<int>(tiles_m));
}
