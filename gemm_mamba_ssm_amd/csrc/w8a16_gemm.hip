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
// staged once per workgroup tile and LDS is never rewritten, but the decode
// itself is still repeated: each wave decodes the 16-byte rows it feeds to
// the matrix cores in registers (the exact packed E4M3->BF16 convert, right
// before the MFMA that uses them), so every weight is decoded by the two
// waves that share its columns in each 128-row M-tile, 2*N*K*ceil(M/128)
// converts in all, on the vector ALU beside the matrix cores. (The 256 x 256
// tiles of w8a16_gemm_wide.hip halve that per token.)
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
//
// Schedule. Without a workspace every tile is computed whole by one
// workgroup. With one (w8a16_gemm_ws, or the static scratch of
// w8a16_gemm_noalloc) the grid is persistent, G = 2 workgroups per CU: the
// 128 x 128 output tiles rarely come in a multiple of G, so whole-tile waves
// would leave up to half of the chip idle in the last wave. Instead:
//  * shared part: the tiles past the last whole round of G are cut into
//    units of one 128-wide k-block, and the units are dealt to the workgroups
//    in equal contiguous ranges, so every workgroup gets the same work. A tile
//    whose k-blocks fall in two or more ranges is "split": each range stores
//    its fp32 partial tile to a workspace slot;
//  * full rounds: then, while at least G whole tiles remain, workgroup w
//    computes tile r*G + w whole (r = 0, 1, ...);
//  * a second kernel on the same stream adds the partial tiles of every
//    split tile in k order (so the bits never depend on timing) and writes
//    its BF16 result. The kernel boundary orders the two, so no workgroup
//    ever waits for another and no atomics or flags are needed.
// The shared part runs first so that the partial stores drain while the
// workgroups go on with their whole tiles.
//
// When the 128 x 128 tiles about match the CUs (the out_proj's 256), one
// workgroup of two 4-wave groups takes each tile instead: each group runs half
// of the tile's k-steps on its own LDS stages, and the two fp32 halves are
// added in LDS at the end, so nothing goes through memory twice and no second
// kernel runs (BigSplit below).
#include <mutex>
#include <type_traits>
#include <utility>

#include "w8a16_device.h"
#include "w8a16_host.h"

namespace w8a16 {
namespace {

constexpr int TN = 128, TK = 64;                    // every tile is 128 columns: one scale block
constexpr int kThreads = 256;                       // 4 waves
constexpr uint32_t kOutOfRange = 0x80000000u;       // buffer offset that reads as zero
constexpr int kBufferFlags = 0x00020000;            // raw buffer, 32-bit data format

static_assert(kScaleBlock == TN && kScaleBlock == 2 * TK, "one scale block per tile column, two k-steps per block");

// Tile shape of one kernel instance: the 4 waves form a WAVES_M x (4 /
// WAVES_M) grid, each wave BI x BJ MFMA blocks of 32 x 32.
//  * Big      (M > 64):  128 x 128, 2 x 2 waves of 64 x 64, 2 workgroups per CU;
//  * Skinny64 (M <= 64):  64 x 128, 1 x 4 waves of 64 x 32, 3 workgroups per CU;
//  * Skinny32 (M <= 32):  32 x 128, 1 x 4 waves of 32 x 32, 4 workgroups per CU.
// The skinny tiles do not pad M to 128 rows (at M = 16 that would be 8x the
// MFMA work) and keep more workgroups and more stages in flight per CU, since
// there the weights stream from HBM with little work per byte.
template <int WAVES_M, int BI_, int BJ_, int WG_PER_CU, int STAGES, int MIN_SHARE, int KSPLIT = 1>
struct TileShape {
    static constexpr int WM = WAVES_M, WN = 4 / WAVES_M, BI = BI_, BJ = BJ_;
    static constexpr int kSplit = KSPLIT;                      // k-groups of 4 waves per workgroup
    static constexpr int kThreadsWg = kThreads * KSPLIT;
    static constexpr int TM = WM * BI * 32;
    static constexpr int kWgPerCu = WG_PER_CU;                 // resident workgroups per CU
    static constexpr int kStages = STAGES;                     // LDS ring (kStages - 1 steps in flight)
    static constexpr int kATileBytes = TM * TK * 2;            // BF16
    static constexpr int kWTileBytes = TN * TK;                // E4M3
    static constexpr int kStageBytes = kATileBytes + kWTileBytes;
    static constexpr int kAChunksPerThread = kATileBytes / 16 / kThreads;
    static constexpr int kWChunksPerThread = kWTileBytes / 16 / kThreads;
    static constexpr int kChunks = kAChunksPerThread + kWChunksPerThread;
    static constexpr int kTileFloats = TM * TN;                // one fp32 partial tile
    static constexpr int kMinShareBlocks = MIN_SHARE;          // fewest k-blocks a shared tile hands one workgroup
    static_assert(WN * BJ * 32 == TN, "4 waves cover the 128 columns");
    static_assert(kAChunksPerThread >= 1 && kATileBytes % (16 * kThreads) == 0, "whole DMA chunks per thread");
    static_assert(kStages * kStageBytes * kWgPerCu * KSPLIT <= 160 * 1024, "LDS of the resident workgroups");
    static_assert(KSPLIT == 1 || (KSPLIT == 2 && TM * TN * 4 <= 2 * kStages * kStageBytes), "combine buffer in LDS");
    static_assert((kStages - 2) * kChunks < 64, "vmcnt field");
};
using BigTile = TileShape<2, 2, 2, 2, 3, 4>;
// The 128 x 128 tile with the k-range of every tile split between two groups
// of 4 waves in one workgroup (one workgroup per CU), added through LDS at the
// end: for as many tiles as CUs, no partial tiles go through memory and no
// combine kernel runs. Whole tiles only, with a multiple of 4 k-steps.
using BigSplit = TileShape<2, 2, 2, 1, 3, 4, 2>;
using Skinny64 = TileShape<1, 2, 1, 3, 3, 4>;
using Skinny32 = TileShape<1, 1, 1, 4, 3, 4>;

typedef __attribute__((address_space(3))) void lds_void;

// How the output tiles are spread over the G workgroups (logical index w):
// tiles [shared_tile0, tiles) form shared_units = (tiles - shared_tile0) *
// k_blocks units (unit (t - shared_tile0) * k_blocks + kb is k-block kb of
// tile t), and workgroup w < shared_groups takes units [start(w), start(w+1))
// with start(w) = floor(w * shared_units / shared_groups); then full rounds
// give workgroup w the tiles r * G + w, r < full_rounds.
struct Schedule {
    int64_t ldo;         // row stride of out and of the residual, in elements (>= N)
    int tiles_m;         // tile t covers rows (t % tiles_m) * TM and columns (t / tiles_m) * TN
    int k_blocks;        // ceil(K / 128)
    int full_rounds;
    int shared_groups;   // 0 when every tile is computed whole
    int shared_tile0;
    int shared_r;        // shared_units % shared_groups
    int64_t shared_q;    // shared_units / shared_groups
};

// start(w) = w * q + floor(w * r / shared_groups), which equals
// floor(w * shared_units / shared_groups) without a 64-bit division
// (w * r < shared_groups^2 fits in 32 bits).
__device__ __forceinline__ int64_t share_start(const Schedule& sc, int w) {
    return static_cast<int64_t>(w) * sc.shared_q + (w * sc.shared_r) / sc.shared_groups;
}

// Byte offset of 16-byte chunk `c` of row `r` inside a staged tile.
__device__ __forceinline__ int a_slot(int r, int c) { return r * (TK * 2) + ((c ^ ((r >> 1) & 7)) << 4); }
__device__ __forceinline__ int w_slot(int r, int c) { return r * TK + ((c ^ ((r >> 2) & 3)) << 4); }

// Workgroups are handed to the 8 XCDs round-robin (block b runs on XCD b % 8),
// and each XCD has its own L2. Remap so that XCD x receives a contiguous range
// of logical workgroups, which own neighbouring tiles (M-tile fastest): the
// M-tiles that share one weight strip then run on the same XCD, and the strip
// is fetched into that L2 once. The map is a bijection on [0, count).
constexpr int kXcds = 8;

__device__ __forceinline__ int xcd_remap(int b, int count) {
    const int q = count / kXcds, r = count % kXcds;
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

// A copy of x that the compiler cannot see through: values derived from it
// are computed where they are used, instead of being hoisted to the top of
// the kernel and kept in registers across the main loop.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Workgroup barrier for the stage hand-off. The memory clobbers keep the
// compiler from moving LDS accesses across it; the hardware needs no fence
// here, because each wave has already waited (s_waitcnt) for its own DMA and
// its LDS reads complete before their MFMAs issue. A workgroup-scope fence
// would also wait for every in-flight DMA load and serialize the pipeline.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Wait until at most `younger` later k-steps' DMA (C::kChunks loads each) of
// this wave are in flight; younger <= C::kStages - 2.
template <class C>
__device__ __forceinline__ void wait_steps(int younger) {
    static_assert(C::kStages == 3 || C::kStages == 4, "one or two later steps in flight");
    if constexpr (C::kStages == 4) {
        if (younger >= 2) {
            wait_vmem<2 * C::kChunks>();
            return;
        }
    }
    if (__builtin_expect(younger >= 1, 1))
        wait_vmem<C::kChunks>();
    else
        wait_vmem<0>();
}

// The GEMM for tile shape C and scale format SF, with the residual epilogue
// out = bf16(res + bf16(sum)) when RES (nemotron_mamba2.rs module docs,
// forward step 8); each combination has its own kernel below (with its own
// occupancy bound).
template <class C, int SF, bool RES>
__device__ __forceinline__ void gemm_body(const uint16_t* __restrict__ A, const uint8_t* __restrict__ W,
                                          const void* __restrict__ S, const uint16_t* __restrict__ res,
                                          uint16_t* __restrict__ out,
                                          float* __restrict__ partials, int M, int N, int K, const Schedule& sc) {
    constexpr int TM = C::TM, BI = C::BI, BJ = C::BJ, kStages = C::kStages;
    constexpr int kAChunksPerThread = C::kAChunksPerThread, kWChunksPerThread = C::kWChunksPerThread;
    constexpr int kATileBytes = C::kATileBytes, kStageBytes = C::kStageBytes;
    constexpr int kWaveRows = BI * 32, kWaveCols = BJ * 32;
    // One LDS array only: a second __shared__ variable makes the compiler
    // attach alias scopes to LDS accesses, after which it waits for every
    // in-flight DMA before each LDS read (the explicit waits below already
    // order them).
    constexpr int KS = C::kSplit;
    __shared__ __attribute__((aligned(16))) uint8_t smem_all[KS * kStages * kStageBytes];

    const int G = gridDim.x;
    const int w = xcd_remap(blockIdx.x, G);
    // k-group g of the workgroup (KS = 2) has its own LDS stages and its own
    // half of every tile's k-steps; wave and tid are local to the group.
    const int kgroup = KS == 2 ? __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kThreads) : 0;
    uint8_t* const smem = smem_all + kgroup * (kStages * kStageBytes);
    const int tid = threadIdx.x % kThreads, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int li = lane & 31, lg = lane >> 5;
    const int k_blocks = sc.k_blocks;
    const int nk = (K + TK - 1) / TK;

    // Per-thread DMA source offsets at k0 = 0, the same for every tile (the
    // lane's LDS destination is fixed by the instruction: base + 16 * lane).
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

    // Lane-constant operand addresses inside a stage; the stage is added as
    // an immediate offset. A: [bi][j][h], W: [bj][j].
    int a_addr[BI][2][2], w_addr[BJ][2];
#pragma unroll
    for (int bi = 0; bi < BI; ++bi)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                a_addr[bi][j][h] = a_slot(wm * kWaveRows + bi * 32 + li, 4 * j + 2 * lg + h);
#pragma unroll
    for (int bj = 0; bj < BJ; ++bj)
#pragma unroll
        for (int j = 0; j < 2; ++j) w_addr[bj][j] = kATileBytes + w_slot(wn * kWaveCols + bj * 32 + li, 2 * j + lg);

    const f32x16_t zero = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f,
                           0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    f32x16_t acc[BI][BJ], blk[BI][BJ];

    // 32x32 MFMA result layout: lane l holds column l % 32; value v is row
    // 8*(v/4) + 4*(l/32) + v%4 of the block.
    // A per-row scale multiplies the finished sum (1 for the block formats).
    // ONLY_BI >= 0 writes that 32-row block of the wave's rows only.
    auto store_tile = [&](const f32x16_t (&r)[BI][BJ], int m0, int n0, int only_bi = -1) {
        const int l = opaque(lane), li = l & 31, lg = l >> 5;
#pragma unroll
        for (int bi = 0; bi < BI; ++bi)
#pragma unroll
            for (int bj = 0; bj < BJ; ++bj) {
                if (only_bi >= 0 && bi != only_bi) continue;
                const int n = n0 + wn * kWaveCols + bj * 32 + li;
                float rs = 1.0f;
                if constexpr (SF == kScaleRowF32) rs = n < N ? row_scale<SF>(S, n) : 0.0f;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int m = m0 + wm * kWaveRows + bi * 32 + 8 * (v >> 2) + 4 * lg + (v & 3);
                    if (m < M && n < N) {
                        const int64_t o = static_cast<int64_t>(m) * sc.ldo + n;
                        if constexpr (RES)
                            out[o] = residual_out(r[bi][bj][v] * rs, res[o]);
                        else
                            out[o] = f32_to_bf16_bits(r[bi][bj][v] * rs);
                    }
                }
            }
    };

    // Shared-range state: this workgroup's units [u, u_end) and the local
    // index of the first tile they touch.
    int64_t u = 0, u_end = 0;
    if (w < sc.shared_groups) {
        u = share_start(sc, w);
        u_end = share_start(sc, w + 1);
    }
    const int first_shared = static_cast<int>(u / k_blocks);
    int round = 0;

    for (;;) {
        // Next piece of work: tile t, k-blocks [kb0, kb1).
        int t, kb0, kb1;
        if (u < u_end) {
            const int ts = static_cast<int>(u / k_blocks);
            kb0 = static_cast<int>(u - static_cast<int64_t>(ts) * k_blocks);
            kb1 = static_cast<int>(min(static_cast<int64_t>(k_blocks), kb0 + (u_end - u)));
            t = sc.shared_tile0 + ts;
            u += kb1 - kb0;
        } else if (round < sc.full_rounds) {
            t = round * G + w;
            kb0 = 0;
            kb1 = k_blocks;
            ++round;
        } else {
            break;
        }
        const int tm = t % sc.tiles_m, tn = t / sc.tiles_m;
        const int m0 = tm * TM, n0 = tn * TN;
        // k-steps [ks0, ks0 + len) of this piece (ks0 even, len >= 1); with
        // two k-groups (whole tiles, a multiple of 4 k-steps) group g takes
        // the g-th half, which starts a scale block.
        const int len = (min(2 * kb1, nk) - 2 * kb0) / KS;
        const int ks0 = 2 * kb0 + kgroup * len;
        kb0 += kgroup * (len / 2);

        // Buffer resources over this tile's rows of A and W: rows past M or
        // N lie beyond num_records and read as zero.
        const int rows_a = min(TM, M - m0), rows_w = min(TN, N - n0);
        const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(A + static_cast<int64_t>(m0) * K), 0, rows_a * K * 2, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rsrc_w = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(W + static_cast<int64_t>(n0) * K), 0, rows_w * K, kBufferFlags);

        // DMA of k-step ks0 + kt into stage `slot`. A full k-step passes k0
        // as the scalar offset; the K-tail step checks each lane's k and sends
        // lanes past K out of range (they load zeros).
        // DMA of a k-step known to lie inside K (not the last k-step).
        auto issue_full = [&](int kt, int slot) {
            const int k0 = (ks0 + kt) * TK;
            uint8_t* base = smem + slot * kStageBytes;
#pragma unroll
            for (int i = 0; i < kAChunksPerThread; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsrc_a, (lds_void*)(base + i * (kThreads * 16) + wave * 1024), 16, a_off[i], k0 * 2, 0, 0);
#pragma unroll
            for (int i = 0; i < kWChunksPerThread; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsrc_w, (lds_void*)(base + kATileBytes + i * (kThreads * 16) + wave * 1024), 16, w_off[i], k0, 0, 0);
        };
        auto issue = [&](int kt, int slot) {
            const int k0 = (ks0 + kt) * TK;
            uint8_t* base = smem + slot * kStageBytes;
            auto dst_a = [&](int i) { return (lds_void*)(base + i * (kThreads * 16) + wave * 1024); };
            auto dst_w = [&](int i) { return (lds_void*)(base + kATileBytes + i * (kThreads * 16) + wave * 1024); };
            if (__builtin_expect(k0 + TK <= K, 1)) {   // one branch per step, not one per load
#pragma unroll
                for (int i = 0; i < kAChunksPerThread; ++i)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_a, dst_a(i), 16, a_off[i], k0 * 2, 0, 0);
#pragma unroll
                for (int i = 0; i < kWChunksPerThread; ++i)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_w, dst_w(i), 16, w_off[i], k0, 0, 0);
            } else {
#pragma unroll
                for (int i = 0; i < kAChunksPerThread; ++i)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rsrc_a, dst_a(i), 16, (k0 + a_k[i] < K) ? a_off[i] + k0 * 2 : kOutOfRange, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < kWChunksPerThread; ++i)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rsrc_w, dst_w(i), 16, (k0 + w_k[i] < K) ? w_off[i] + k0 : kOutOfRange, 0, 0, 0);
            }
        };

        // One k-step on stage SLOT: the operand reads, 4 * BJ * 4 converts and
        // 4 * BI * BJ MFMAs. All reads are issued first (the scheduling
        // barrier keeps them there), so the MFMAs wait on them in order
        // instead of on one read at a time. The first k-step of a scale block
        // starts the block accumulator from zero.
        auto compute = [&](auto slot_c, auto first_c) {
            constexpr int kSlot = decltype(slot_c)::value;
            constexpr bool kFirst = decltype(first_c)::value;
            const uint8_t* stage = smem + kSlot * kStageBytes;
            u32x4_t wq[BJ][2];                          // [bj][j]
            bf16x8_t av[BI][2][2];                      // [bi][j][h]
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
                for (int bj = 0; bj < BJ; ++bj) wq[bj][j] = *reinterpret_cast<const u32x4_t*>(stage + w_addr[bj][j]);
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int bi = 0; bi < BI; ++bi)
                        av[bi][j][h] = *reinterpret_cast<const bf16x8_t*>(stage + a_addr[bi][j][h]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 2; ++j) {               // two 32-wide k spans
                bf16x8_t bw[BJ][2];                     // [bj][h]
#pragma unroll
                for (int bj = 0; bj < BJ; ++bj) {
                    bw[bj][0] = e4m3x8_to_bf16(wq[bj][j][0], wq[bj][j][1]);
                    bw[bj][1] = e4m3x8_to_bf16(wq[bj][j][2], wq[bj][j][3]);
                }
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int bi = 0; bi < BI; ++bi)
#pragma unroll
                        for (int bj = 0; bj < BJ; ++bj)
                            blk[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                av[bi][j][h], bw[bj][h], (kFirst && j == 0 && h == 0) ? zero : blk[bi][bj], 0, 0, 0);
            }
        };

        // The tile's scale row, 64 k-blocks at a time: lane l holds block
        // s_base + l, so the main loop issues no vector memory operation
        // besides the DMA (one reload per 64 k-blocks).
        const int64_t s_row = static_cast<int64_t>(tn) * k_blocks;
        auto load_scales = [&](int base) {
            return (base + lane < k_blocks) ? block_scale<SF>(S, s_row + base + lane) : 0.0f;
        };
        int s_base = kb0 & ~63;
        float s_lane = load_scales(s_base);

        auto fold = [&](int kb) {
            if (__builtin_expect(kb - s_base >= 64, 0)) {
                s_base += 64;
                s_lane = load_scales(s_base);
            }
            const float s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s_lane), kb - s_base));
#pragma unroll
            for (int bi = 0; bi < BI; ++bi)
#pragma unroll
                for (int bj = 0; bj < BJ; ++bj)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[bi][bj][v] = fmaf(blk[bi][bj][v], s, acc[bi][bj][v]);
        };

#pragma unroll
        for (int bi = 0; bi < BI; ++bi)
#pragma unroll
            for (int bj = 0; bj < BJ; ++bj) acc[bi][bj] = zero;

        // k-step kt (relative to ks0) reads stage kt % kStages. Before it:
        // wait for this wave's DMA of kt (the later steps' loads may remain
        // in flight), then a barrier, after which every wave's DMA of kt has
        // landed and every wave is done reading stage (kt - 1) % kStages,
        // which is refilled with step kt + kStages - 1. FIRST: kt is even
        // (ks0 is even, so this is the first k-step of a scale block); the
        // unrolled loop below starts at multiples of 2 * kStages, so the
        // stage and the parity are static.
        // A step of a steady chunk (one that ends at least kStages steps
        // before the piece): the wait count is fixed, the step it issues is a
        // full one, and it is not the last step.
        auto steady_step = [&](auto slot_c, auto first_c, int kt) {
            constexpr int kSlot = decltype(slot_c)::value;
            constexpr bool kFirst = decltype(first_c)::value;
            wait_vmem<(kStages - 2) * C::kChunks>();
            lds_barrier();
            issue_full(kt + kStages - 1, (kSlot + kStages - 1) % kStages);
            compute(slot_c, first_c);
            // kt + 1 < len here, so this folds after the odd steps only; the
            // run-time form keeps each step its own block for the compiler
            // (with a compile-time condition it schedules two steps as one
            // and spills).
            if (!kFirst || kt + 1 == len) fold(kb0 + (kt >> 1));
        };
        auto step = [&](auto slot_c, auto first_c, int kt) {
            constexpr int kSlot = decltype(slot_c)::value;
            constexpr bool kFirst = decltype(first_c)::value;
            wait_steps<C>(min(len - 1, kt + kStages - 2) - kt);
            lds_barrier();
            if (__builtin_expect(kt + kStages - 1 < len, 1)) issue(kt + kStages - 1, (kSlot + kStages - 1) % kStages);
            compute(slot_c, first_c);
            if (!kFirst || __builtin_expect(kt + 1 == len, 0)) fold(kb0 + (kt >> 1));
        };

        // Every wave is done reading the stages of the previous piece.
        lds_barrier();
#pragma unroll
        for (int i = 0; i + 1 < kStages; ++i)
            if (i < len) issue(i, i);
        constexpr int kUnroll = 2 * kStages;             // stages 0 .. kStages-1, twice
        static_assert(kUnroll == 6, "the unrolled steps below");
        int kt = 0;
        for (; kt + kUnroll + kStages - 1 < len; kt += kUnroll) {   // steady chunks
            steady_step(std::integral_constant<int, 0>{}, std::true_type{}, kt);
            steady_step(std::integral_constant<int, 1 % kStages>{}, std::false_type{}, kt + 1);
            steady_step(std::integral_constant<int, 2 % kStages>{}, std::true_type{}, kt + 2);
            steady_step(std::integral_constant<int, 3 % kStages>{}, std::false_type{}, kt + 3);
            steady_step(std::integral_constant<int, 4 % kStages>{}, std::true_type{}, kt + 4);
            steady_step(std::integral_constant<int, 5 % kStages>{}, std::false_type{}, kt + 5);
        }
        for (; kt + kUnroll <= len; kt += kUnroll) {      // whole chunks: no per-step length checks
            step(std::integral_constant<int, 0>{}, std::true_type{}, kt);
            step(std::integral_constant<int, 1 % kStages>{}, std::false_type{}, kt + 1);
            step(std::integral_constant<int, 2 % kStages>{}, std::true_type{}, kt + 2);
            step(std::integral_constant<int, 3 % kStages>{}, std::false_type{}, kt + 3);
            step(std::integral_constant<int, 4 % kStages>{}, std::true_type{}, kt + 4);
            step(std::integral_constant<int, 5 % kStages>{}, std::false_type{}, kt + 5);
        }
        if (kt < len) {                                     // the last, partial chunk
            step(std::integral_constant<int, 0>{}, std::true_type{}, kt);
            if (kt + 1 < len) step(std::integral_constant<int, 1 % kStages>{}, std::false_type{}, kt + 1);
            if (kt + 2 < len) step(std::integral_constant<int, 2 % kStages>{}, std::true_type{}, kt + 2);
            if (kt + 3 < len) step(std::integral_constant<int, 3 % kStages>{}, std::false_type{}, kt + 3);
            if (kt + 4 < len) step(std::integral_constant<int, 4 % kStages>{}, std::true_type{}, kt + 4);
        }

        if constexpr (KS == 2) {
            // The two groups' sums meet in LDS (lane-major, no bank
            // conflicts): group g hands over its 32-row blocks bi != g, adds
            // the other group's block bi == g to its own (a + b, the same
            // bits either way round) and writes those rows.
            static_assert(BI == 2, "one 32-row block per group");
            lds_barrier();                          // every wave is done with the stages
            float* xs = reinterpret_cast<float*>(smem_all);
            auto slot = [&](int bi, int bj, int v) { return ((wave * BI * BJ + bi * BJ + bj) * 16 + v) * 64 + lane; };
#pragma unroll
            for (int bi = 0; bi < BI; ++bi)
#pragma unroll
                for (int bj = 0; bj < BJ; ++bj)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (bi != kgroup) xs[slot(bi, bj, v)] = acc[bi][bj][v];
            lds_barrier();
#pragma unroll
            for (int bi = 0; bi < BI; ++bi)
#pragma unroll
                for (int bj = 0; bj < BJ; ++bj)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (bi == kgroup) acc[bi][bj][v] += xs[slot(bi, bj, v)];
            store_tile(acc, m0, n0, kgroup);
            continue;
        } else if (kb0 == 0 && kb1 == k_blocks) {        // the whole tile: write it
            store_tile(acc, m0, n0);
            continue;
        }

        // Part of a split tile: store it row-major to this range's slot 0 if
        // the tile is the first of the range, else to slot 1 (a range has at
        // most two split tiles: its first and its last). Plain stores, no
        // wait: the combine kernel reads them after this kernel has ended.
        const int ts = t - sc.shared_tile0;
        float* mine = partials + (2 * static_cast<int64_t>(w) + (ts == first_shared ? 0 : 1)) * C::kTileFloats;
        const int l = opaque(lane), li = l & 31, lg = l >> 5;
#pragma unroll
        for (int bi = 0; bi < BI; ++bi)
#pragma unroll
            for (int bj = 0; bj < BJ; ++bj) {
                const int col = wn * kWaveCols + bj * 32 + li;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = wm * kWaveRows + bi * 32 + 8 * (v >> 2) + 4 * lg + (v & 3);
                    mine[row * TN + col] = acc[bi][bj][v];
                }
            }
    }
}

// One kernel per (tile shape, scale format, residual); suffixes: s1 = FP32
// block scales, r = FP32 row scales, res = residual epilogue.
#define W8A16_GEMM_KERNEL(NAME, C, SF, RES)                                                          \
    __global__ void __launch_bounds__(C::kThreadsWg, C::kWgPerCu)                                    \
    NAME(const uint16_t* __restrict__ A, const uint8_t* __restrict__ W, const void* __restrict__ S,   \
         const uint16_t* __restrict__ res, uint16_t* __restrict__ out, float* __restrict__ partials,  \
         int M, int N, int K, Schedule sc) {                                                         \
        gemm_body<C, SF, RES>(A, W, S, res, out, partials, M, N, K, sc);                             \
    }                                                                                                \
    template <>                                                                                      \
    struct GemmKernel<C, SF, RES> {                                                                  \
        static constexpr auto fn = &NAME;                                                            \
    };
template <class C, int SF, bool RES> struct GemmKernel;
W8A16_GEMM_KERNEL(gemm_kernel_128, BigTile, kScaleBlockBf16, false)
W8A16_GEMM_KERNEL(gemm_kernel_64, Skinny64, kScaleBlockBf16, false)
W8A16_GEMM_KERNEL(gemm_kernel_32, Skinny32, kScaleBlockBf16, false)
W8A16_GEMM_KERNEL(gemm_kernel_128_s1, BigTile, kScaleBlockF32, false)
W8A16_GEMM_KERNEL(gemm_kernel_64_s1, Skinny64, kScaleBlockF32, false)
W8A16_GEMM_KERNEL(gemm_kernel_32_s1, Skinny32, kScaleBlockF32, false)
W8A16_GEMM_KERNEL(gemm_kernel_128_r, BigTile, kScaleRowF32, false)
W8A16_GEMM_KERNEL(gemm_kernel_64_r, Skinny64, kScaleRowF32, false)
W8A16_GEMM_KERNEL(gemm_kernel_32_r, Skinny32, kScaleRowF32, false)
W8A16_GEMM_KERNEL(gemm_kernel_128_res, BigTile, kScaleBlockBf16, true)
W8A16_GEMM_KERNEL(gemm_kernel_64_res, Skinny64, kScaleBlockBf16, true)
W8A16_GEMM_KERNEL(gemm_kernel_32_res, Skinny32, kScaleBlockBf16, true)
W8A16_GEMM_KERNEL(gemm_kernel_128k2, BigSplit, kScaleBlockBf16, false)
W8A16_GEMM_KERNEL(gemm_kernel_128k2_s1, BigSplit, kScaleBlockF32, false)
W8A16_GEMM_KERNEL(gemm_kernel_128k2_r, BigSplit, kScaleRowF32, false)
W8A16_GEMM_KERNEL(gemm_kernel_128k2_res, BigSplit, kScaleBlockBf16, true)
#undef W8A16_GEMM_KERNEL

// Combine of the split tiles. The host lists, for every split tile, the
// workgroup that computed its first k-blocks (the tile is the last of that
// workgroup's range). Workgroup (i, y) of the combine handles rows
// 32y .. 32y+31 of split tile i: each thread adds four float4 (rows r, r+8,
// r+16, r+24 at 4 consecutive columns) over the parts in k order, issuing
// the loads of kCombineBatch parts before their additions, and writes BF16.
constexpr int kMaxSplits = 1536;                       // list capacity (3 KB of kernel arguments)
constexpr int kCombineRows = 32;
constexpr int kCombineBatch = 4;
static_assert(kThreads == 8 * (TN / 4), "8 rows of float4 per pass");

struct SplitList {
    uint16_t first[kMaxSplits];
};

template <class C, int SF, bool RES>
__global__ void __launch_bounds__(kThreads)
combine_kernel(const float* __restrict__ partials, uint16_t* __restrict__ out, const void* __restrict__ S,
               const uint16_t* __restrict__ res, int M, int N, Schedule sc, SplitList list) {
    constexpr int TM = C::TM, kTileFloats = C::kTileFloats;
    const int w = list.first[blockIdx.x];
    const int k_blocks = sc.k_blocks;
    const int ts = static_cast<int>((share_start(sc, w + 1) - 1) / k_blocks);
    // Parts: workgroups w .. last, the ranges that intersect tile ts (w + 1
    // starts inside it, since w ends inside it).
    const int64_t tile_begin = static_cast<int64_t>(ts) * k_blocks, tile_end = tile_begin + k_blocks;
    int last = w + 1;
    while (last + 1 < sc.shared_groups && share_start(sc, last + 1) < tile_end) ++last;

    const int t = sc.shared_tile0 + ts;
    const int m0 = (t % sc.tiles_m) * TM, n0 = (t / sc.tiles_m) * TN;
    const int row0 = blockIdx.y * kCombineRows + threadIdx.x / (TN / 4), col = (threadIdx.x % (TN / 4)) * 4;
    f32x4_t sum[4];
    for (int p0 = w; p0 <= last; p0 += kCombineBatch) {
        f32x4_t x[kCombineBatch][4];
#pragma unroll
        for (int i = 0; i < kCombineBatch; ++i) {
            const int p = p0 + i;
            if (p <= last) {
                // Slot 0 if tile ts is the first tile of p's range (the range
                // starts inside it or at its start), else slot 1.
                const int slot = share_start(sc, p) >= tile_begin ? 0 : 1;
                const float* src = partials + (2 * static_cast<int64_t>(p) + slot) * kTileFloats + row0 * TN + col;
#pragma unroll
                for (int r = 0; r < 4; ++r) x[i][r] = *reinterpret_cast<const f32x4_t*>(src + r * 8 * TN);
            }
        }
#pragma unroll
        for (int i = 0; i < kCombineBatch; ++i) {
            const int p = p0 + i;
            if (p <= last) {
#pragma unroll
                for (int r = 0; r < 4; ++r) sum[r] = (p == w) ? x[i][r] : sum[r] + x[i][r];
            }
        }
    }
    float rs[4];                                       // per-row scales of the 4 columns (1 for block formats)
#pragma unroll
    for (int e = 0; e < 4; ++e) rs[e] = n0 + col + e < N ? row_scale<SF>(S, n0 + col + e) : 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = m0 + row0 + r * 8;
        if (m >= M) break;
        const int64_t o = static_cast<int64_t>(m) * sc.ldo + n0 + col;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (n0 + col + e < N) {
                if constexpr (RES)
                    out[o + e] = residual_out(sum[r][e] * rs[e], res[o + e]);
                else
                    out[o + e] = f32_to_bf16_bits(sum[r][e] * rs[e]);
            }
    }
}

// Choose the schedule; returns the grid size. `slots` is the number of
// workgroups resident at once. Whole tiles, one per workgroup, when they fill
// the slots evenly or the last wave is at least a quarter full (splitting k
// then costs more in partial-tile traffic than the idle slots); otherwise
// whole rounds of `slots` tiles plus a shared part over the rest, with at
// least `min_share` k-blocks per workgroup.
int plan(int64_t tiles, int64_t tiles_m, int k_blocks, int slots, int min_share, Schedule* sc) {
    *sc = Schedule{};
    sc->tiles_m = static_cast<int>(tiles_m);
    sc->k_blocks = k_blocks;
    const int64_t rounds = tiles / slots;
    const int64_t rest = tiles - rounds * slots;
    if (rest == 0 || (rounds > 0 && 4 * rest >= slots)) {
        sc->full_rounds = 1;
        return static_cast<int>(tiles);
    }
    const int64_t units = rest * k_blocks;
    const int64_t groups = std::min<int64_t>(slots, std::max<int64_t>(rest, units / min_share));
    sc->full_rounds = static_cast<int>(rounds);
    sc->shared_tile0 = static_cast<int>(rounds * slots);
    sc->shared_groups = static_cast<int>(groups);
    sc->shared_q = units / groups;
    sc->shared_r = static_cast<int>(units % groups);
    return rounds > 0 ? slots : static_cast<int>(groups);
}

// Host copy of share_start.
int64_t host_share_start(const Schedule& sc, int w) {
    return static_cast<int64_t>(w) * sc.shared_q + (static_cast<int64_t>(w) * sc.shared_r) / sc.shared_groups;
}

// The split tiles, each named by the workgroup that computes its first
// k-blocks: w whose range ends inside a tile that it also starts.
int list_splits(const Schedule& sc, SplitList* list) {
    int n = 0;
    for (int w = 0; w + 1 < sc.shared_groups; ++w) {
        const int64_t end = host_share_start(sc, w + 1);
        if (end % sc.k_blocks == 0) continue;
        const int64_t tile_begin = (end - 1) / sc.k_blocks * sc.k_blocks;
        if (host_share_start(sc, w) <= tile_begin) list->first[n++] = static_cast<uint16_t>(w);
    }
    return n;
}

// Bytes of partial tiles the split schedule of tile shape C needs (0 when
// it computes whole tiles only): two slots per workgroup of the shared part.
template <class C>
int64_t split_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if constexpr (C::kSplit == 2) {
        return 0;
    } else {
        const int64_t tiles_m = ceil_div(M, C::TM), tiles = tiles_m * ceil_div(N, TN);
        if (tiles > INT32_MAX) return 0;
        Schedule sc;
        plan(tiles, tiles_m, static_cast<int>(ceil_div(K, kScaleBlockHost)),
             std::min(C::kWgPerCu * device_cu_count(), kMaxSplits), C::kMinShareBlocks, &sc);
        return sc.shared_groups > 0 ? 2 * static_cast<int64_t>(sc.shared_groups) * C::kTileFloats * 4 : 0;
    }
}

// Plan and launch the GEMM (and, if tiles are split, the combine) with tile
// shape C and scale format SF. Without a workspace (partials == nullptr)
// every tile is computed whole by one workgroup.
template <class C, int SF, bool RES>
int run_gemm(const void* A, const void* Wq, const void* scale, const void* residual, void* out, int64_t M,
             int64_t N, int64_t K, int64_t ldo, float* partials, size_t workspace_bytes, hipStream_t s) {
    // Buffer offsets are 32-bit: one tile's rows of A must span less than 2 GiB.
    if (static_cast<int64_t>(C::TM) * K * 2 >= static_cast<int64_t>(kOutOfRange)) return W8A16_ERR_SHAPE;
    const int64_t tiles_m = ceil_div(M, C::TM);
    const int64_t tiles = tiles_m * ceil_div(N, TN);
    if (tiles > INT32_MAX) return W8A16_ERR_SHAPE;
    const int k_blocks = static_cast<int>(ceil_div(K, kScaleBlockHost));
    const int slots = std::min(C::kWgPerCu * device_cu_count(), kMaxSplits);
    Schedule sc;
    int grid;
    const bool may_split = C::kSplit == 1 && partials != nullptr;
    if (!may_split) {
        sc = Schedule{};                             // whole tiles, one per workgroup
        sc.ldo = ldo;
        sc.tiles_m = static_cast<int>(tiles_m);
        sc.k_blocks = k_blocks;
        sc.full_rounds = 1;
        grid = static_cast<int>(tiles);
    } else {
        grid = plan(tiles, tiles_m, k_blocks, slots, C::kMinShareBlocks, &sc);
        sc.ldo = ldo;
        if (sc.shared_groups > 0 &&
            workspace_bytes < static_cast<size_t>(2) * sc.shared_groups * C::kTileFloats * sizeof(float))
            return W8A16_ERR_WORKSPACE;
    }
    int st = launch(GemmKernel<C, SF, RES>::fn, dim3(static_cast<unsigned>(grid)), dim3(C::kThreadsWg), s,
                    static_cast<const uint16_t*>(A), static_cast<const uint8_t*>(Wq), scale,
                    static_cast<const uint16_t*>(residual), static_cast<uint16_t*>(out), partials,
                    static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), sc);
    if constexpr (C::kSplit == 2) {
        return st;                                   // whole tiles: nothing to combine
    } else {
        if (st != W8A16_OK || sc.shared_groups == 0) return st;
        SplitList list;
        const int splits = list_splits(sc, &list);
        if (splits == 0) return W8A16_OK;
        return launch(&combine_kernel<C, SF, RES>, dim3(static_cast<unsigned>(splits), C::TM / kCombineRows),
                      dim3(kThreads), s, static_cast<const float*>(partials), static_cast<uint16_t*>(out), scale,
                      static_cast<const uint16_t*>(residual), static_cast<int>(M), static_cast<int>(N), sc, list);
    }
}

// The kernel family for (M, N, K) on this device; depends on nothing else.
//  kWideSplitN: 256 x 256 tiles for whole rounds of CU-many tiles over the
//  first columns, the rest of the columns (less than a round) with the
//  128-row tiles; e.g. the 1024-token in_proj: 256 tiles over columns
//  0..16383, then 8 x 17 tiles of 128 x 128.
enum class Path { kSkinny, kMid, kTile32, kTile64, kWide, kWideSplitN, kBigSplit, kBigTile };

Path choose_path(int64_t M, int64_t N, int64_t K, int64_t* n_wide = nullptr) {
    if (mid_plan(M, N, K, device_cu_count()) >= 0) return Path::kMid;
    if (skinny_fits(M, K) || skinny_lds_fits(M, N, K, device_cu_count())) return Path::kSkinny;
    if (M <= Skinny32::TM) return Path::kTile32;
    if (M <= Skinny64::TM) return Path::kTile64;
    const int cus = device_cu_count();
    if (wide_gemm_pays(M, N, K, cus)) return Path::kWide;
    const int64_t nw = wide_gemm_columns(M, N, K, cus);
    if (nw > 0 && nw < N) {
        if (n_wide) *n_wide = nw;
        return Path::kWideSplitN;
    }
    // About as many 128 x 128 tiles as CUs (at least three quarters of them,
    // so no more than a quarter idles) and whole k-steps in two equal halves
    // of whole scale blocks: one workgroup per tile, k split inside it.
    const int64_t tiles = ceil_div(M, BigTile::TM) * ceil_div(N, TN);
    if (tiles <= cus && 4 * tiles >= 3 * cus && K % (4 * TK) == 0) return Path::kBigSplit;
    return Path::kBigTile;
}

// The 128-row kernel for the columns the 256 x 256 tiles leave: the k-split
// workgroups when the tiles fit one per CU, else whole (or, with a
// workspace, split) tiles.
bool tail_in_bigsplit(int64_t M, int64_t N, int64_t K) {
    return ceil_div(M, BigTile::TM) * ceil_div(N, TN) <= device_cu_count() && K % (4 * TK) == 0;
}

int64_t workspace_bytes_for(int64_t M, int64_t N, int64_t K) {
    int64_t nw = 0;
    switch (choose_path(M, N, K, &nw)) {
        case Path::kTile32: return split_workspace_bytes<Skinny32>(M, N, K);
        case Path::kTile64: return split_workspace_bytes<Skinny64>(M, N, K);
        case Path::kBigTile: return split_workspace_bytes<BigTile>(M, N, K);
        case Path::kWideSplitN:
            return tail_in_bigsplit(M, N - nw, K) ? 0 : split_workspace_bytes<BigTile>(M, N - nw, K);
        default: return 0;
    }
}

template <int SF, bool RES>
int gemm_by_shape(const void* A, const void* Wq, const void* scale, const void* residual, void* out, int64_t M,
                  int64_t N, int64_t K, hipStream_t s, float* partials = nullptr, size_t workspace_bytes = 0) {
    int64_t nw = 0;
    switch (choose_path(M, N, K, &nw)) {
        case Path::kSkinny: return skinny_gemm(A, Wq, scale, SF, residual, out, M, N, K, s);
        case Path::kMid: return mid_gemm(A, Wq, scale, SF, residual, out, M, N, K, N, s);
        case Path::kTile32:
            return run_gemm<Skinny32, SF, RES>(A, Wq, scale, residual, out, M, N, K, N, partials, workspace_bytes, s);
        case Path::kTile64:
            return run_gemm<Skinny64, SF, RES>(A, Wq, scale, residual, out, M, N, K, N, partials, workspace_bytes, s);
        case Path::kWide: return wide_gemm(A, Wq, scale, SF, residual, out, M, N, K, N, s);
        case Path::kWideSplitN: {
            // Columns [0, nw) on 256 x 256 tiles, [nw, N) on 128 x 128 tiles:
            // the weight rows, their scale rows (nw is a multiple of 128) and
            // the output columns of the second part start at nw.
            int st = wide_gemm(A, Wq, scale, SF, residual, out, M, nw, K, N, s);
            if (st != W8A16_OK) return st;
            const int64_t nt = N - nw;
            const void* W2 = static_cast<const uint8_t*>(Wq) + nw * K;
            const void* S2 = SF == kScaleRowF32
                                 ? static_cast<const void*>(static_cast<const float*>(scale) + nw)
                                 : static_cast<const void*>(static_cast<const uint8_t*>(scale) +
                                                            (nw / kScaleBlockHost) * ceil_div(K, kScaleBlockHost) *
                                                                (SF == kScaleBlockBf16 ? 2 : 4));
            void* O2 = static_cast<uint16_t*>(out) + nw;
            const void* R2 = residual ? static_cast<const uint16_t*>(residual) + nw : nullptr;
            if (tail_in_bigsplit(M, nt, K))
                return run_gemm<BigSplit, SF, RES>(A, W2, S2, R2, O2, M, nt, K, N, nullptr, 0, s);
            return run_gemm<BigTile, SF, RES>(A, W2, S2, R2, O2, M, nt, K, N, partials, workspace_bytes, s);
        }
        case Path::kBigSplit:
            return run_gemm<BigSplit, SF, RES>(A, Wq, scale, residual, out, M, N, K, N, nullptr, 0, s);
        default:
            return run_gemm<BigTile, SF, RES>(A, Wq, scale, residual, out, M, N, K, N, partials, workspace_bytes, s);
    }
}

}  // namespace
}  // namespace w8a16

extern "C" int w8a16_gemm_ex(const void* A, const void* Wq, const void* scale, int scale_format, void* out,
                             int64_t M, int64_t N, int64_t K, void* stream) {
    using namespace w8a16;
    bool noop = false;
    const int st = check_product_args(A, Wq, scale, out, M, N, K, &noop, scale_format);
    if (st != W8A16_OK || noop) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (scale_format) {
        case W8A16_SCALE_BLOCK_F32:
            return gemm_by_shape<kScaleBlockF32, false>(A, Wq, scale, nullptr, out, M, N, K, s);
        case W8A16_SCALE_ROW_F32:
            return gemm_by_shape<kScaleRowF32, false>(A, Wq, scale, nullptr, out, M, N, K, s);
        default:
            return gemm_by_shape<kScaleBlockBf16, false>(A, Wq, scale, nullptr, out, M, N, K, s);
    }
}

extern "C" int w8a16_gemm(const void* A, const void* Wq, const void* scale, void* out,
                          int64_t M, int64_t N, int64_t K, void* stream) {
    return w8a16_gemm_ex(A, Wq, scale, W8A16_SCALE_BLOCK_BF16, out, M, N, K, stream);
}

extern "C" int64_t w8a16_gemm_workspace_size(int64_t M, int64_t N, int64_t K) {
    using namespace w8a16;
    if (M < 0 || N < 0 || K < 16 || (K % 16) != 0 || M > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
        return W8A16_ERR_SHAPE;
    if (M == 0 || N == 0) return 0;
    return workspace_bytes_for(M, N, K);
}

extern "C" int w8a16_gemm_ws(const void* A, const void* Wq, const void* scale, void* out, int64_t M, int64_t N,
                             int64_t K, void* workspace, int64_t workspace_bytes, void* stream) {
    using namespace w8a16;
    bool noop = false;
    const int st = check_product_args(A, Wq, scale, out, M, N, K, &noop);
    if (st != W8A16_OK || noop) return st;
    if (workspace == nullptr)
        return gemm_by_shape<kScaleBlockBf16, false>(A, Wq, scale, nullptr, out, M, N, K,
                                                     static_cast<hipStream_t>(stream));
    if (workspace_bytes < 0) return W8A16_ERR_ARG;
    if (!aligned(workspace, 256)) return W8A16_ERR_ALIGN;
    if (workspace_bytes < workspace_bytes_for(M, N, K)) return W8A16_ERR_WORKSPACE;
    if (overlaps(workspace, workspace_bytes, out, M * N * 2) || overlaps(workspace, workspace_bytes, A, M * K * 2) ||
        overlaps(workspace, workspace_bytes, Wq, N * K) ||
        overlaps(workspace, workspace_bytes, scale, scale_bytes(W8A16_SCALE_BLOCK_BF16, N, K)))
        return W8A16_ERR_ALIAS;
    return gemm_by_shape<kScaleBlockBf16, false>(A, Wq, scale, nullptr, out, M, N, K, static_cast<hipStream_t>(stream),
                                                 static_cast<float*>(workspace), static_cast<size_t>(workspace_bytes));
}

// Scratch of the allocation-free GEMM: the split schedule's fp32 partial
// tiles, in a device array of the code object (each GPU holds its own copy,
// from the first call on it until the process ends). 64 MiB is what the
// largest split schedule on a 256-CU device needs: two 128 x 128 fp32 tiles
// for each of 512 workgroups.
constexpr int64_t kScratchBytes = 64ll << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace w8a16 {
namespace {

constexpr int kScratchDevices = 64;

// The scratch array's device address on the current device, looked up once
// per device with that device current (host code names the array only
// through this address). nullptr when the lookup fails.
float* scratch_on_current_device() {
    static std::mutex mu;
    static float* addr[kScratchDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
        addr[dev] = static_cast<float*>(p);
    }
    return addr[dev];
}

}  // namespace
}  // namespace w8a16

extern "C" int64_t w8a16_gemm_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" int w8a16_gemm_noalloc(const void* A, const void* Wq, const void* scale, void* out, int64_t M, int64_t N,
                                  int64_t K, void* stream) {
    using namespace w8a16;
    bool noop = false;
    const int st = check_product_args(A, Wq, scale, out, M, N, K, &noop);
    if (st != W8A16_OK || noop) return st;
    const int64_t need = workspace_bytes_for(M, N, K);
    if (need > kScratchBytes) return W8A16_ERR_SCRATCH;
    if (need == 0)                                   // whole tiles: no scratch
        return gemm_by_shape<kScaleBlockBf16, false>(A, Wq, scale, nullptr, out, M, N, K,
                                                     static_cast<hipStream_t>(stream));
    float* ws = scratch_on_current_device();
    if (ws == nullptr) return W8A16_ERR_LAUNCH;
    // Every partial tile is written by its workgroup before the combine
    // kernel reads it, so nothing in the scratch needs clearing first.
    return gemm_by_shape<kScaleBlockBf16, false>(A, Wq, scale, nullptr, out, M, N, K, static_cast<hipStream_t>(stream),
                                                 ws, static_cast<size_t>(kScratchBytes));
}

extern "C" int w8a16_gemm_residual(const void* A, const void* Wq, const void* scale, const void* residual,
                                   void* out, int64_t M, int64_t N, int64_t K, void* stream) {
    using namespace w8a16;
    bool noop = false;
    const int st = check_product_args(A, Wq, scale, out, M, N, K, &noop);
    if (st != W8A16_OK || noop) return st;
    if (!residual) return W8A16_ERR_NULL;
    if (!aligned(residual, 2)) return W8A16_ERR_ALIGN;
    const int64_t out_bytes = M * N * 2;
    if (overlaps(out, out_bytes, residual, out_bytes)) return W8A16_ERR_ALIAS;
    return gemm_by_shape<kScaleBlockBf16, true>(A, Wq, scale, residual, out, M, N, K,
                                                static_cast<hipStream_t>(stream));
}
