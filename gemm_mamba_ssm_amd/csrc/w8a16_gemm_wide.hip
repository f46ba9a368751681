// Prefill GEMM with 256 x 256 output tiles, weights converted in the
// workgroup that stages them.
//
//   out[m][n] = sum_k A[m][k] * E4M3(W[n][k]) * scale[n/128][k/128]
// (Qwen3SsmLayer docs, `set_fp8_decode_weights`; NemotronMamba2Layer docs,
// `set_fp8_weights`). Prefill is one GEMM with M = prompt tokens
// (TransformerLayer docs, `prefill`).
//
// The pages measure (nemotron_mamba2.rs, doc text of `set_bf16_weights`) that
// redoing the weight dequant for every M-block costs N*K*M/M_TILE converts and
// a visible share of a 1k-token prefill. Here a workgroup owns 256 output rows
// and stages each weight tile once for all of them; the two waves that share
// a weight column (rows 0..127 and 128..255 of the tile) each convert it in
// registers right before their MFMAs, so the convert work is N*K*M/128 and
// runs on the vector ALU beside the matrix cores (two waves per SIMD: one
// wave's converts issue while the other's MFMAs run).
//
// The block scale is folded into the convert: each weight becomes
// bf16(e * s) (e * s is exact in fp32 for a BF16 scale; one rounding to BF16),
// so the matrix cores accumulate the scaled product directly in fp32 over the
// whole K range, with no per-k-block partial sums and no fold instructions.
// A one-hot activation row therefore returns bf16_rne(e * s), the rounded
// dequantized weight, exactly.
//
// CDNA4 mapping (64-wide wavefronts, v_mfma_f32_32x32x16_bf16, 160 KB LDS):
//  * workgroup tile 256 x 256 x 64 (k-step), 8 waves in a 2 x 4 grid, one
//    workgroup per CU, two waves per SIMD: each wave computes a 128 x 64
//    sub-tile = 4 x 2 MFMA blocks of 32 x 32, 128 fp32 accumulators per lane;
//  * A (BF16, 32 KB per k-step) and W (E4M3, 16 KB) go from HBM/L2 straight
//    into LDS with buffer_load_dwordx4 ... lds (no register staging);
//  * three LDS stages (144 KB): the tiles of steps kt+1 and kt+2 are in
//    flight while step kt is multiplied;
//  * LDS rows are XOR-swizzled so the 16-byte DMA writes and the operand
//    reads are free of bank conflicts: A rows are 128 bytes (chunk c of row r
//    at c ^ ((r >> 1) & 7)), W rows are 64 bytes (chunk c at c ^ ((r >> 2) & 3));
//  * the MFMA's k-slots are permuted identically for A and W so that one
//    16-byte W read (16 consecutive k of one row) feeds two MFMA k-steps:
//    lane group g of MFMA step (j, h) carries k = 32j + 16g + 8h + [0, 8);
//  * persistent grid (one workgroup per CU) walking the tiles with an
//    XCD-aware order: each XCD takes a contiguous range of tiles, M-tile
//    fastest, so the 256-column weight strip of a range is fetched into that
//    XCD's L2 once for all of its M-tiles.
#include <algorithm>
#include <type_traits>

#include "w8a16_device.h"
#include "w8a16_host.h"

namespace w8a16 {
namespace {

constexpr int kTM = 256, kTN = 256, kTK = 64;
constexpr int kWaves = 8, kThreads = 64 * kWaves;
constexpr int kStages = 3;
constexpr int kATile = kTM * kTK * 2;                   // 32 KB of BF16
constexpr int kWTile = kTN * kTK;                       // 16 KB of E4M3
constexpr int kStageBytes = kATile + kWTile;
constexpr int kAChunks = kATile / (16 * kThreads);      // 16-byte DMA loads per lane per k-step
constexpr int kWChunks = kWTile / (16 * kThreads);
constexpr int kGroup = kAChunks + kWChunks;             // DMA loads of one k-step, per wave
constexpr int kWaveRows = 128, kWaveCols = 64;
constexpr int BI = kWaveRows / 32, BJ = kWaveCols / 32; // MFMA blocks of a wave
constexpr int kScaleRegs = 4;                           // scale row in 4 x 64 lanes: k_blocks <= 256
constexpr uint32_t kOutOfRange = 0x80000000u;           // buffer offset that reads as zero
constexpr int kBufferFlags = 0x00020000;                // raw buffer, 32-bit data format
constexpr int kXcds = 8;
constexpr int kBandM = 4;                               // M-tiles per band of the tile order
constexpr int kStRow = 528;                             // LDS row stride of the staged output tile (bytes)
static_assert(kTM * kStRow <= kStages * kStageBytes, "the output tile fits in the stages");

static_assert(kAChunks == 4 && kWChunks == 2, "DMA layout below");
static_assert(2 * kWaveRows == kTM && 4 * kWaveCols == kTN, "2 x 4 waves");
static_assert(kStages * kStageBytes <= 160 * 1024, "LDS");
static_assert(2 * kGroup < 64, "vmcnt field");

typedef __attribute__((address_space(3))) void lds_void;

// Workgroups are handed to the 8 XCDs round-robin (block b runs on XCD
// b % 8); remap so that XCD x holds a contiguous range of logical workgroups.
// A bijection on [0, count).
__device__ __forceinline__ int xcd_remap(int b, int count) {
    const int q = count / kXcds, r = count % kXcds;
    const int x = b % kXcds;
    return x * q + min(x, r) + b / kXcds;
}

// Wait until at most N vector-memory and L LDS operations of this wave are
// in flight (L = 15: no LDS wait).
template <int N, int L>
__device__ __forceinline__ void wait_vmem_lgkm() {
    static_assert(N < 64 && L < 16, "vmcnt / lgkmcnt fields");
    __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (L << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for the stage hand-off (see the k-step below for why no
// fence is needed); the clobbers keep LDS accesses on their side of it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// A copy of x that the compiler cannot see through: values derived from it
// are computed where they are used instead of being hoisted out of the loops
// and kept in registers.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// The source of the 16 bytes that lane `lane` of wave `wave` writes with DMA
// load i: A byte i * 8192 + wave * 1024 + 16 * lane of the stage is chunk
// c ^ ((r >> 1) & 7) of row r (8 BF16 from k = 8c); W byte i * 8192 +
// wave * 1024 + 16 * lane (after the A tile) is chunk c ^ ((r >> 2) & 3) of
// row r (16 codes from k = 16c).
__device__ __forceinline__ int dma_byte(int i, int wave, int lane) { return i * (kThreads * 16) + wave * 1024 + lane * 16; }
__device__ __forceinline__ int a_row(int i, int wave, int lane) { return dma_byte(i, wave, lane) >> 7; }
__device__ __forceinline__ int a_kc(int i, int wave, int lane) {
    const int o = dma_byte(i, wave, lane);
    return (((o >> 4) & 7) ^ (((o >> 7) >> 1) & 7)) * 8;
}
__device__ __forceinline__ int w_row(int i, int wave, int lane) { return dma_byte(i, wave, lane) >> 6; }
__device__ __forceinline__ int w_kc(int i, int wave, int lane) {
    const int o = dma_byte(i, wave, lane);
    return (((o >> 4) & 3) ^ (((o >> 6) >> 2) & 3)) * 16;
}

// 8 E4M3 codes (two dwords) -> 8 BF16 weights for the matrix cores. Block
// formats: bf16(e * s), with e * s exact in fp32 for a BF16 scale (4 + 8
// significant bits) and rounded once; an FP32 scale rounds e * s to fp32
// first. Row format: e itself (exact), the row scale multiplies the sum.
template <int SF>
__device__ __forceinline__ bf16x8_t decode8(uint32_t lo, uint32_t hi, float s) {
    if constexpr (SF == kScaleRowF32) {
        const bf16x2_t p0 = e4m3x2_to_bf16(lo, false), p1 = e4m3x2_to_bf16(lo, true);
        const bf16x2_t p2 = e4m3x2_to_bf16(hi, false), p3 = e4m3x2_to_bf16(hi, true);
        return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    } else {
        const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false) * s;
        const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true) * s;
        const f32x2_t c = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false) * s;
        const f32x2_t d = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true) * s;
        const bf16x2_t pa = __builtin_convertvector(a, bf16x2_t), pb = __builtin_convertvector(b, bf16x2_t);
        const bf16x2_t pc = __builtin_convertvector(c, bf16x2_t), pd = __builtin_convertvector(d, bf16x2_t);
        return bf16x8_t{pa[0], pa[1], pb[0], pb[1], pc[0], pc[1], pd[0], pd[1]};
    }
}

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef int v2i32_t __attribute__((ext_vector_type(2)));
typedef int v4i32_t __attribute__((ext_vector_type(4)));

// Two fp32 -> two BF16 (round to nearest even) in one dword, first in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{x, y}, bf16x2_t));
}

// The residual add of two packed BF16 pairs (y + residual, each rounded once).
__device__ __forceinline__ uint32_t residual_add_bf16x2(uint32_t y, uint32_t r) {
    return static_cast<uint32_t>(residual_add_bits(static_cast<uint16_t>(y & 0xFFFFu), static_cast<uint16_t>(r & 0xFFFFu))) |
           (static_cast<uint32_t>(residual_add_bits(static_cast<uint16_t>(y >> 16), static_cast<uint16_t>(r >> 16))) << 16);
}

template <int SF, bool RES>
__global__ void __launch_bounds__(kThreads, 1)
wide_gemm_kernel(const uint16_t* __restrict__ A, const uint8_t* __restrict__ W, const void* __restrict__ S,
                 const uint16_t* __restrict__ res, uint16_t* __restrict__ out, int M, int N, int K, int ldo_elems,
                 int tiles_m, int tiles, bool vec_out) {
    // One LDS array only (a second one makes the compiler wait for every
    // in-flight DMA before each LDS read).
    __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * kStageBytes];

    const int G = gridDim.x;
    const int wg = xcd_remap(blockIdx.x, G);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;            // rows 128 wm.., columns 64 wn..
    const int li = lane & 31, lg = lane >> 5;
    const int nk = (K + kTK - 1) / kTK;
    const int k_blocks = (K + 127) / 128;
    const int n_blocks = (N + 127) / 128;
    const int tiles_n = tiles / tiles_m;

    // DMA source offsets at k = 0 (the same for every tile); the lane's LDS
    // destination is fixed by the instruction: base + 16 * lane.
    uint32_t a_off[kAChunks], w_off[kWChunks];
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) a_off[i] = static_cast<uint32_t>(a_row(i, wave, lane) * K + a_kc(i, wave, lane)) * 2;
#pragma unroll
    for (int i = 0; i < kWChunks; ++i) w_off[i] = static_cast<uint32_t>(w_row(i, wave, lane) * K + w_kc(i, wave, lane));

    // Operand read offsets inside a stage. A: row 128 wm + 32 bi + li (bi adds
    // bi * 4096), chunk 4j + 2lg + h for MFMA step q = 2j + h. W: row
    // 64 wn + 32 bj + li (bj adds 2048), chunk 2j + lg.
    int a_rd[4], w_rd[2];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        a_rd[q] = (kWaveRows * wm + li) * 128 + ((((q >> 1) * 4 + 2 * lg + (q & 1)) ^ ((li >> 1) & 7)) << 4);
#pragma unroll
    for (int j = 0; j < 2; ++j)
        w_rd[j] = kATile + (kWaveCols * wn + li) * 64 + (((2 * j + lg) ^ ((li >> 2) & 3)) << 4);

    f32x16_t acc[BI][BJ];

    for (int t = wg; t < tiles; t += G) {
        // Tiles go in bands of kBandM M-tiles: inside a band, M-tile fastest.
        // An XCD's 32 concurrent tiles then share 4 A row-blocks and 8
        // weight strips in its L2 (with all M-tiles in one order, a long
        // prompt would stream the whole of A through every XCD per round).
        const int band = t / (kBandM * tiles_n), in_band = t - band * (kBandM * tiles_n);
        const int band_m = min(kBandM, tiles_m - band * kBandM);
        const int tm = band * kBandM + in_band % band_m, tn = in_band / band_m;
        const int m0 = tm * kTM, n0 = tn * kTN;
        const int rows_a = min(kTM, M - m0), rows_w = min(kTN, N - n0);
        const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(A + static_cast<int64_t>(m0) * K), 0, rows_a * K * 2, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rsrc_w = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(W + static_cast<int64_t>(n0) * K), 0, rows_w * K, kBufferFlags);

        // The scale row of this wave's columns (one 128-column block):
        // lane l of register r holds k-block 64 r + l. Loaded before the
        // DMA, so the first DMA wait covers it too.
        const int nb = (n0 + kWaveCols * wn) / 128;
        uint32_t s_vec[kScaleRegs];
#pragma unroll
        for (int r = 0; r < kScaleRegs; ++r) {
            const int kb = r * 64 + lane;
            s_vec[r] = (nb < n_blocks && kb < k_blocks) ? block_scale_bits<SF>(S, static_cast<int64_t>(nb) * k_blocks + kb)
                                                        : 0u;
        }
        // Scale of k-block kb (wave-uniform); 0 past K (those weights are zero).
        auto scale_of = [&](int kb) -> float {
            if constexpr (SF == kScaleRowF32) {
                return 1.0f;
            } else {
                uint32_t bits = 0;
#pragma unroll
                for (int r = 0; r < kScaleRegs; ++r)
                    if ((kb >> 6) == r) bits = __builtin_amdgcn_readlane(s_vec[r], kb & 63);
                return scale_from_bits<SF>(bits);
            }
        };

        // DMA of k-step ks into stage `slot`, load c of this wave (0..3: A,
        // 4..5: W). FULL: the step lies inside K; otherwise lanes past K (and
        // every lane of a step past K) load zeros.
        auto issue_one = [&](auto full_c, int ks, int slot, int c) {
            constexpr bool kFull = decltype(full_c)::value;
            const int k0 = ks * kTK;
            uint8_t* base = smem + slot * kStageBytes + wave * 1024;
            if (c < kAChunks) {
                const int i = c;
                uint32_t voff = a_off[i], soff = static_cast<uint32_t>(k0) * 2;
                if constexpr (!kFull) {
                    voff = (k0 + a_kc(i, wave, opaque(lane)) < K) ? a_off[i] + soff : kOutOfRange;
                    soff = 0;
                }
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_a, (lds_void*)(base + i * (kThreads * 16)), 16, voff,
                                                         soff, 0, 0);
            } else {
                const int i = c - kAChunks;
                uint32_t voff = w_off[i], soff = static_cast<uint32_t>(k0);
                if constexpr (!kFull) {
                    voff = (k0 + w_kc(i, wave, opaque(lane)) < K) ? w_off[i] + soff : kOutOfRange;
                    soff = 0;
                }
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_w, (lds_void*)(base + kATile + i * (kThreads * 16)),
                                                         16, voff, soff, 0, 0);
            }
        };
        auto issue = [&](int ks, int slot) {
#pragma unroll
            for (int c = 0; c < kGroup; ++c) issue_one(std::false_type{}, ks, slot, c);
        };

        // Every wave is done with the previous tile's stages.
        lds_barrier();
#pragma nounroll
        for (int i = 0; i < kStages - 1; ++i) {
            const int ks = __builtin_amdgcn_readfirstlane(opaque(i));
            issue(ks, ks);
        }
#pragma unroll
        for (int bi = 0; bi < BI; ++bi)
#pragma unroll
            for (int bj = 0; bj < BJ; ++bj)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[bi][bj][v] = 0.0f;

        // Operands of MFMA step q (q = 2j + h): A rows av[q & 1], converted
        // weights bw[q & 1]; wq holds the raw weights of the current k-step.
        bf16x8_t av[2][BI], bw[2][BJ];
        u32x4_t wq[BJ][2];
        float s = 0.0f;
        // The weights and the first A operands of k-step ks from stage slot.
        auto first_operands = [&](int ks, int slot) {
            const uint8_t* st = smem + slot * kStageBytes;
#pragma unroll
            for (int bj = 0; bj < BJ; ++bj)
#pragma unroll
                for (int j = 0; j < 2; ++j) wq[bj][j] = *reinterpret_cast<const u32x4_t*>(st + w_rd[j] + bj * 2048);
            s = scale_of(ks >> 1);
#pragma unroll
            for (int bi = 0; bi < BI; ++bi) av[0][bi] = *reinterpret_cast<const bf16x8_t*>(st + a_rd[0] + bi * 4096);
#pragma unroll
            for (int bj = 0; bj < BJ; ++bj) bw[0][bj] = decode8<SF>(wq[bj][0][0], wq[bj][0][1], s);
        };
        wait_vmem_lgkm<kGroup, 15>();                  // this wave's DMA of step 0
        lds_barrier();
        first_operands(0, 0);

        // k-step kt multiplies stage kt % 3. Its MFMA steps 0..2 issue the DMA
        // of step kt + 2 into stage (kt + 2) % 3, which every wave finished
        // reading before the barrier of step kt - 1 (below). Before MFMA step
        // 3: this wave's DMA of step kt + 1 has landed (only the loads of
        // step kt + 2 may be in flight) and its reads of this stage have
        // completed; then the barrier, after which every wave's DMA of step
        // kt + 1 has landed, so MFMA step 3 overlaps the reads and converts
        // of the first operands of step kt + 1. The barrier thus never
        // leaves the matrix cores without operands.
        auto step = [&](auto full_c, int kt, int slot) {
            const int slot1 = slot == 2 ? 0 : slot + 1, slot2 = slot == 0 ? 2 : slot - 1;
            const uint8_t* st = smem + slot * kStageBytes;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                __builtin_amdgcn_sched_barrier(0);
                constexpr int kDma0[4] = {0, 2, 4, -1}, kDma1[4] = {1, 3, 5, -1};
                if (q < 3) {
                    issue_one(full_c, kt + 2, slot2, kDma0[q]);
                    issue_one(full_c, kt + 2, slot2, kDma1[q]);
                    const int j = (q + 1) >> 1, h = (q + 1) & 1;
#pragma unroll
                    for (int bi = 0; bi < BI; ++bi)
                        av[(q + 1) & 1][bi] = *reinterpret_cast<const bf16x8_t*>(st + a_rd[q + 1] + bi * 4096);
#pragma unroll
                    for (int bj = 0; bj < BJ; ++bj)
                        bw[(q + 1) & 1][bj] = decode8<SF>(wq[bj][j][2 * h], wq[bj][j][2 * h + 1], s);
                } else {
                    wait_vmem_lgkm<kGroup, 0>();
                    lds_barrier();
                    first_operands(kt + 1, slot1);
                }
#pragma unroll
                for (int bi = 0; bi < BI; ++bi)
#pragma unroll
                    for (int bj = 0; bj < BJ; ++bj)
                        acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bw[q & 1][bj], av[q & 1][bi],
                                                                              acc[bi][bj], 0, 0, 0);
                // 8 MFMAs with the DMA, the LDS reads and the converts of the
                // next operands between them.
#pragma unroll
                for (int i = 0; i < BI * BJ; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                      // MFMA
                    if (q < 3 && (i == 1 || i == 5)) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // DMA
                    if (i < BI + (q == 3 ? 4 : 0)) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);                      // VALU
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        };

        // Steps whose DMA (of step kt + 2) lies inside K, then the rest.
        const int nfull = max(0, K / kTK - 2);
        int kt = 0, slot = 0;
        for (; kt < nfull; ++kt, slot = slot == 2 ? 0 : slot + 1) step(std::true_type{}, kt, slot);
        for (; kt < nk; ++kt, slot = slot == 2 ? 0 : slot + 1) step(std::false_type{}, kt, slot);

        // The MFMAs take the weights as their first operand, so block (bi, bj)
        // holds the transposed product: lane l has output row 32 bi + l % 32
        // of the wave, and its value v = 4a + b is column 32 bj + 8a +
        // 4 (l / 32) + b. Each lane thus owns runs of 4 consecutive columns of
        // one row (8 bytes of the output). Buffer stores over this tile's
        // rows: rows past M fall past the range and are dropped, columns past
        // N get an out-of-range offset.
        // The row stride is recomputed here (not hoisted out of the tile loop
        // with its multiples, which would hold that many scalar registers).
        const int ldo = __builtin_amdgcn_readfirstlane(opaque(ldo_elems)) * 2;
        const int rows_out = min(kTM, M - m0);
        const int out_bytes = (rows_out - 1) * ldo + N * 2;        // through column N - 1 of the last row
        const __amdgpu_buffer_rsrc_t rsrc_o = __builtin_amdgcn_make_buffer_rsrc(
            out + static_cast<int64_t>(m0) * ldo_elems, 0, out_bytes, kBufferFlags);
        __amdgpu_buffer_rsrc_t rsrc_r = rsrc_o;
        if constexpr (RES)
            rsrc_r = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(res + static_cast<int64_t>(m0) * ldo_elems), 0, out_bytes, kBufferFlags);
        const int l = opaque(lane);
        const int row = kWaveRows * wm + (l & 31);                  // + 32 bi
        const int col = n0 + kWaveCols * wn + 4 * (l >> 5);         // + 32 bj + 8 a
        if (vec_out) {
            // N and the row stride multiples of 8, out 16-byte aligned: the
            // tile is staged in LDS as BF16 (rows 528 bytes apart, so the
            // 8-byte writes of 32 lanes with 32 different rows spread over
            // the banks) and written back as whole 512-byte rows, 16 bytes
            // per lane: 16 wide stores per lane instead of 32 narrow ones,
            // each instruction covering two whole rows of the tile. Before
            // the stages are reused: every DMA of this wave (the zero loads
            // past K included) has landed and its LDS reads have completed,
            // then the barrier.
            wait_vmem_lgkm<0, 0>();
            lds_barrier();
#pragma unroll
            for (int bj = 0; bj < BJ; ++bj)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int n = col + 32 * bj + 8 * a;
                    float rs[4] = {1.0f, 1.0f, 1.0f, 1.0f};
                    if constexpr (SF == kScaleRowF32)
#pragma unroll
                        for (int b = 0; b < 4; ++b) rs[b] = n < N ? row_scale<SF>(S, n + b) : 0.0f;
#pragma unroll
                    for (int bi = 0; bi < BI; ++bi) {
                        const uint32_t lo = pack_bf16x2(acc[bi][bj][4 * a] * rs[0], acc[bi][bj][4 * a + 1] * rs[1]);
                        const uint32_t hi = pack_bf16x2(acc[bi][bj][4 * a + 2] * rs[2], acc[bi][bj][4 * a + 3] * rs[3]);
                        *reinterpret_cast<u32x2_t*>(smem + (row + 32 * bi) * kStRow + (n - n0) * 2) = u32x2_t{lo, hi};
                    }
                }
            lds_barrier();
            const int tr = tid >> 5, tc = tid & 31;                  // 16 rows of 32 x 16 bytes per round
            const int n = n0 + 8 * tc;
#pragma unroll 4
            for (int r = 0; r < kTM / 16; ++r) {
                const int orow = 16 * r + tr;
                u32x4_t v = *reinterpret_cast<const u32x4_t*>(smem + orow * kStRow + tc * 16);
                const uint32_t voff = n < N ? static_cast<uint32_t>(orow * ldo + 2 * n) : kOutOfRange;
                if constexpr (RES) {
                    const u32x4_t rv = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc_r, voff, 0, 0));
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = residual_add_bf16x2(v[i], rv[i]);
                }
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i32_t, v), rsrc_o, voff, 0, 0);
            }
        } else {
#pragma unroll
            for (int bj = 0; bj < BJ; ++bj)
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const int n = col + 32 * bj + 8 * a + b;
                        const float rs = (SF == kScaleRowF32 && n < N) ? row_scale<SF>(S, n) : 1.0f;
#pragma unroll
                        for (int bi = 0; bi < BI; ++bi) {
                            const uint32_t voff = n < N ? static_cast<uint32_t>(row * ldo + 2 * n) : kOutOfRange;
                            const int soff = 32 * bi * ldo;
                            uint16_t y = f32_to_bf16_bits(acc[bi][bj][4 * a + b] * rs);
                            if constexpr (RES) {
                                const uint16_t r = __builtin_bit_cast(
                                    uint16_t, __builtin_amdgcn_raw_buffer_load_b16(rsrc_r, voff, soff, 0));
                                y = residual_add_bits(y, r);
                            }
                            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(short, y), rsrc_o, voff, soff, 0);
                        }
                    }
        }
    }
}

}  // namespace

bool wide_gemm_fits(int64_t M, int64_t N, int64_t K, int64_t ldo) {
    // Buffer offsets are 32-bit: one tile's rows of A, W and out must span
    // less than 2 GiB, so that an out-of-range offset plus any in-range part
    // stays past the range.
    return M >= 1 && N >= 1 && ldo >= N && K <= 128 * 64 * kScaleRegs &&
           static_cast<int64_t>(kTM) * K * 2 < static_cast<int64_t>(kOutOfRange) &&
           static_cast<int64_t>(kTN) * K < static_cast<int64_t>(kOutOfRange) &&
           static_cast<int64_t>(kTM) * ldo * 2 < static_cast<int64_t>(kOutOfRange);
}

bool wide_gemm_pays(int64_t M, int64_t N, int64_t K, int cus) {
    if (!wide_gemm_fits(M, N, K, N) || cus <= 0) return false;
    const int64_t tiles = ceil_div(M, kTM) * ceil_div(N, kTN);
    const int64_t rounds = ceil_div(tiles, cus);
    return tiles >= cus && 100 * tiles >= 85 * rounds * cus;
}

int64_t wide_gemm_columns(int64_t M, int64_t N, int64_t K, int cus) {
    if (!wide_gemm_fits(M, N, K, N) || cus <= 0) return 0;
    const int64_t tiles_m = ceil_div(M, kTM), tiles_n = ceil_div(N, kTN);
    const int64_t rounds = tiles_m * tiles_n / cus;
    return std::min(tiles_n, rounds * cus / tiles_m) * kTN;
}

int wide_gemm(const void* A, const void* Wq, const void* scale, int fmt, const void* residual, void* out, int64_t M,
              int64_t N, int64_t K, int64_t ldo, hipStream_t stream) {
    if (!wide_gemm_fits(M, N, K, ldo)) return W8A16_ERR_SHAPE;
    const int64_t tiles_m = ceil_div(M, kTM), tiles = tiles_m * ceil_div(N, kTN);
    if (tiles > INT32_MAX) return W8A16_ERR_SHAPE;
    const int grid = static_cast<int>(std::min<int64_t>(tiles, device_cu_count()));
    // 8-byte output stores need every run of 4 columns 8-byte aligned.
    const bool vec_out = N % 8 == 0 && ldo % 8 == 0 && aligned(out, 16) && (!residual || aligned(residual, 16));
    auto go = [&](auto kernel) {
        return launch(kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), stream,
                      static_cast<const uint16_t*>(A), static_cast<const uint8_t*>(Wq), scale,
                      static_cast<const uint16_t*>(residual), static_cast<uint16_t*>(out), static_cast<int>(M),
                      static_cast<int>(N), static_cast<int>(K), static_cast<int>(ldo), static_cast<int>(tiles_m),
                      static_cast<int>(tiles), vec_out);
    };
    if (residual) return go(&wide_gemm_kernel<kScaleBlockBf16, true>);
    switch (fmt) {
        case kScaleBlockF32: return go(&wide_gemm_kernel<kScaleBlockF32, false>);
        case kScaleRowF32: return go(&wide_gemm_kernel<kScaleRowF32, false>);
        default: return go(&wide_gemm_kernel<kScaleBlockBf16, false>);
    }
}

}  // namespace w8a16
