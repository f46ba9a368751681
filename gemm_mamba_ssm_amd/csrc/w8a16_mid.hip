// Mid-size GEMM for the w8a16 block-scaled FP8 projection: a few dozen to a
// few hundred rows of A (a batch of decode tokens, a short prompt, the
// K-token verify of speculative decoding):
//
//   out[m][n] = sum_k A[m][k] * E4M3(W[n][k]) * scale[n/128][k/128]
// (Qwen3SsmLayer docs, `set_fp8_decode_weights`; NemotronMamba2Layer docs,
// `set_fp8_weights`; TransformerLayer docs, `decode_multi_seq`: the weights
// are read once for all rows).
//
// At these sizes the 128 x 128 tiles of the prefill GEMM are too few to
// occupy the chip (the Mamba-2 out_proj at 128 tokens has 32 of them for 256
// CUs), and the matrix cores are far from busy: what bounds a CU is the bytes
// it must bring in from L2 for its output tile, K * (2 * TM + TN) for a tile
// of TM rows and TN columns over all of K (BF16 A, E4M3 W). With one tile per
// CU that is least for TN about 2 * TM, so the host picks small tiles of 16 *
// MB rows and 16 * NB columns that come to about the CU count (out_proj at
// 128 tokens: 256 tiles of 32 x 64, 1 MB per CU instead of 3 MB).
//
// How fast a CU can pull those bytes depends on the access pattern of each
// wave-wide load (measured on MI355X, L2-resident data, one workgroup per
// CU): about 60 GB/s with 8 waves when the 16-byte pieces of a row sit on
// adjacent lanes, 33-38 GB/s when they are 16 lanes apart as the MFMA
// operand layout has them. So the tile goes through LDS:
//  * one workgroup of 8 waves per tile; each stage is 256 (or 128) of K:
//    A (TM rows x 512 bytes) and W (TN rows x 256 bytes) go from L2/HBM into
//    LDS with buffer_load ... lds, every wave-wide load covering whole rows
//    with the pieces of a row on adjacent lanes, STAGES stages in a ring;
//  * the 16-byte chunks of each LDS row are XOR-swizzled by row, so the MFMA
//    operand reads (16 rows at one k per quarter-wave) hit distinct banks;
//  * the 8 waves split the tile's column blocks (NQ ways), row blocks (MQ
//    ways) and each stage's k (KQ ways): each weight is decoded by MQ waves
//    (the exact packed convert), v_mfma_f32_16x16x32_bf16 does the products,
//    and the block scale is applied exactly in fp32 (acc += s * blk over the
//    wave's part of each scale block; the tile's scale rows are copied
//    into LDS once, by DMA ahead of the first stage, so that inside the
//    loop every wait on LDS is an exact count);
//  * a wave reads the next stage's operands from LDS into registers while
//    its MFMAs work on the current stage's (the stage's work is small next
//    to the latency of a barrier, an LDS read and an MFMA chain, which
//    otherwise add up every stage), one barrier per stage;
//  * the KQ partial tiles meet in LDS and are added in a fixed order
//    (deterministic), then the per-row scale (FP32 row format), the residual
//    epilogue and the BF16 stores.
#include <algorithm>
#include <type_traits>

#include "w8a16_device.h"
#include "w8a16_host.h"

namespace w8a16 {
namespace {

constexpr int kMidWaves = 8;
constexpr int kMidThreads = 64 * kMidWaves;
constexpr int kLdsBudget = 160 * 1024;
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kPastEnd = 0x7fffffff;             // scalar offset that puts every lane past a tile's buffer
constexpr int kBufferFlags = 0x00020000;         // raw buffer, 32-bit data format

typedef __attribute__((address_space(3))) void lds_void;
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for the stage hand-off; each wave has waited for its own
// DMA first (a workgroup fence would also wait for the loads still in flight).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Workgroup b runs on XCD b % 8; give XCD x a contiguous range of tiles (M
// fastest), so the tiles that share a weight strip read it through one L2.
__device__ __forceinline__ int mid_xcd_remap(int b, int count) {
    constexpr int kXcds = 8;
    const int q = count / kXcds, r = count % kXcds;
    const int x = b % kXcds;
    return x * q + min(x, r) + b / kXcds;
}

// Tile of MB x NB blocks of 16 x 16; the 8 waves split it MQ x NQ ways over
// row and column blocks and KQ ways over each stage's KS k (128 or 256: one
// or two scale blocks); STAGES stages in the LDS ring.
template <int MB_, int NB_, int MQ_, int NQ_, int KQ_, int KS_, int STAGES_>
struct MidCfg {
    static constexpr int MB = MB_, NB = NB_, MQ = MQ_, NQ = NQ_, KQ = KQ_, KS = KS_, STAGES = STAGES_;
    static constexpr int TM = 16 * MB, TN = 16 * NB;
    static constexpr int kARow = KS * 2, kWRow = KS;                     // bytes per staged row
    static constexpr int kABytes = TM * kARow, kWBytes = TN * kWRow;
    static constexpr int kStageBytes = kABytes + kWBytes;
    static constexpr int kInstr = kStageBytes / 1024;                    // wave-wide 1 KB loads per stage
    static constexpr int kLoads = (kInstr + kMidWaves - 1) / kMidWaves;  // per wave and stage
    static constexpr int kRing = STAGES * kStageBytes;
    static constexpr int kPartBytes = KQ * TM * TN * 4;
    static constexpr int kMain = kRing > kPartBytes ? kRing : kPartBytes;
    // Rows of the scale grid that TN consecutive columns can span, and the
    // LDS that holds them for K up to kMidMaxK (fp32-sized entries).
    static constexpr int kScaleRows = (TN - 1 + kScaleBlock - 1) / kScaleBlock + 1;
    static constexpr int kScaleTable = kScaleRows * static_cast<int>(kMidMaxK / kScaleBlock) * 4;
    static constexpr int kLds = kMain + 1024 + kScaleTable;
    static constexpr int MBW = MB / MQ, NBW = NB / NQ, KW = KS / KQ, kSteps = KW / 32;
    static constexpr int kStepsPerBlock = kSteps < 4 ? kSteps : 4;       // MFMA steps of a wave per scale block
    static_assert(KS == 128 || KS == 256, "one or two scale blocks per stage");
    static_assert(MQ * NQ * KQ == kMidWaves, "8 waves");
    static_assert(MB % MQ == 0 && NB % NQ == 0 && KW % 32 == 0, "whole blocks and MFMA steps per wave");
    static_assert(kABytes % 1024 == 0 && kWBytes % 1024 == 0, "whole 1 KB loads");
    static_assert(STAGES >= 2 && (STAGES - 1) * kLoads < 64, "vmcnt field");
    static_assert(kLds <= kLdsBudget, "LDS");
};

// Byte offset of logical 16-byte chunk c of row r in a staged tile (A rows
// of KS * 2 bytes, W rows of KS bytes): the chunks are XOR-swizzled by row so
// that 16 rows read at one k fall in distinct banks (64 four-byte banks).
template <int KS>
__device__ __forceinline__ int a_pos(int r, int c) { return r * (2 * KS) + ((c ^ (r & 15)) << 4); }
template <int KS>
__device__ __forceinline__ int w_pos(int r, int c) {
    return r * KS + ((c ^ (KS == 128 ? (r >> 1) & 7 : r & 15)) << 4);
}

// 8 E4M3 codes (two dwords) -> 8 BF16, exact.
__device__ __forceinline__ bf16x8_t e4m3x8(uint32_t lo, uint32_t hi) {
    const bf16x2_t p0 = e4m3x2_to_bf16(lo, false), p1 = e4m3x2_to_bf16(lo, true);
    const bf16x2_t p2 = e4m3x2_to_bf16(hi, false), p3 = e4m3x2_to_bf16(hi, true);
    return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// A wave's operands of one stage, in registers: A [i][step] 8 BF16, W
// [j][step] 8 E4M3 bytes, and the block scales of its k-blocks [j][block].
template <class C>
struct MidOps {
    bf16x8_t a[C::MBW][C::kSteps];
    u32x2_t w[C::NBW][C::kSteps];
    float s[C::NBW][C::kSteps / C::kStepsPerBlock];
};

// The finished fp32 sums of columns n .. n + 3 of output row m (n < N):
// the per-row scale (FP32 row format), BF16, the residual (out = bf16(res +
// bf16(sum)), nemotron_mamba2.rs module docs, forward step 8), and the store
// (8 bytes at once where `vec` says out and res allow it).
template <int SF, bool RES>
__device__ __forceinline__ void mid_store4(f32x4_t sum, const void* __restrict__ S, const uint16_t* __restrict__ res,
                                           uint16_t* __restrict__ out, int m, int n, int N, int64_t ldo, bool vec) {
    const int64_t o = static_cast<int64_t>(m) * ldo + n;
    uint16_t y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float v = sum[e];
        if constexpr (SF == kScaleRowF32) v *= n + e < N ? row_scale<SF>(S, n + e) : 0.0f;
        y[e] = f32_to_bf16_bits(v);
    }
    if (vec && n + 4 <= N) {
        if constexpr (RES) {
            const uint2 rv = *reinterpret_cast<const uint2*>(res + o);
            y[0] = residual_add_bits(y[0], rv.x & 0xFFFFu);
            y[1] = residual_add_bits(y[1], rv.x >> 16);
            y[2] = residual_add_bits(y[2], rv.y & 0xFFFFu);
            y[3] = residual_add_bits(y[3], rv.y >> 16);
        }
        *reinterpret_cast<uint2*>(out + o) =
            make_uint2(y[0] | (static_cast<uint32_t>(y[1]) << 16), y[2] | (static_cast<uint32_t>(y[3]) << 16));
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (n + e < N) out[o + e] = RES ? residual_add_bits(y[e], res[o + e]) : y[e];
    }
}

// Scale format SF; residual epilogue when RES (out = bf16(res + bf16(sum)),
// nemotron_mamba2.rs module docs, forward step 8); `ldo`: the row stride of
// out and res, in elements.
template <class C, int SF, bool RES>
__device__ __forceinline__ void mid_body(const uint16_t* __restrict__ A, const uint8_t* __restrict__ W,
                                         const void* __restrict__ S, const uint16_t* __restrict__ res,
                                         uint16_t* __restrict__ out, int M, int N, int K, int tiles_m, int64_t ldo) {
    constexpr bool kRowScale = SF == kScaleRowF32;
    constexpr int TM = C::TM, TN = C::TN, MBW = C::MBW, NBW = C::NBW, KW = C::KW, KS = C::KS;
    constexpr int STAGES = C::STAGES, kStage = C::kStageBytes, kLoads = C::kLoads;
    constexpr int kSteps = C::kSteps, kSpb = C::kStepsPerBlock, kBlocks = kSteps / kSpb;
    // One LDS array: the ring (afterwards the partial tiles), a 1 KB pad
    // that takes the loads of waves with no chunk left in a stage, and the
    // tile's block scales.
    __shared__ __attribute__((aligned(16))) uint8_t lds[C::kLds];
    uint8_t* const pad = lds + C::kMain;
    uint8_t* const stab = lds + C::kMain + 1024;

    const int t = mid_xcd_remap(blockIdx.x, gridDim.x);
    const int tm = t % tiles_m, tn = t / tiles_m;
    const int m0 = tm * TM, n0 = tn * TN;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / 64);
    const int lane = threadIdx.x % 64, r = lane % 16, g = lane / 16;
    const int kq = wave % C::KQ, mq = (wave / C::KQ) % C::MQ, nq = wave / (C::KQ * C::MQ);
    const int k_blocks = (K + kScaleBlock - 1) / kScaleBlock;
    const int n_stages = (K + KS - 1) / KS;
    const int j0 = n0 / kScaleBlock;

    // Buffer resources over the tile's rows of A and W: rows past M or N lie
    // beyond num_records and read as zero.
    const int rows_a = min(TM, M - m0), rows_w = min(TN, N - n0);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(A + static_cast<int64_t>(m0) * K), 0, rows_a * K * 2, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(W + static_cast<int64_t>(n0) * K), 0, rows_w * K, kBufferFlags);

    // This thread's DMA pieces: load i of a stage is the stage's 1 KB piece
    // wave + 8i (past the stage's pieces: the pad, reading nothing). In it
    // lane l fills LDS bytes [16l, 16l + 16): the row and position p of the
    // A or W part, holding logical chunk p ^ swizzle(row), i.e. the source
    // bytes at k = 8 * chunk (A) or 16 * chunk (W) of that row (the pieces of
    // a row sit on adjacent lanes). kof: that k within the stage; off: the
    // source offset at k0 = 0.
    int kof[kLoads];
    uint32_t off[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int o = (wave + kMidWaves * i) * 1024 + lane * 16;        // byte in the stage
        if (o < C::kABytes) {
            const int row = o / C::kARow, p = (o % C::kARow) / 16, c = (a_pos<KS>(row, p) % C::kARow) / 16;
            kof[i] = 8 * c;
            off[i] = static_cast<uint32_t>(row * K + 8 * c) * 2;
        } else {
            const int ow = o - C::kABytes;
            const int row = ow / C::kWRow, p = (ow % C::kWRow) / 16, c = (w_pos<KS>(row, p) % C::kWRow) / 16;
            kof[i] = 16 * c;
            off[i] = static_cast<uint32_t>(row * K + 16 * c);
        }
    }

    // DMA of stage st into ring slot `slot`. Pieces past the stage go to the
    // pad and stages past K (the ring's tail) read nothing: their scalar
    // offset puts every lane past the buffer, so every stage issues the same
    // loads with the same lane offsets (no branch and no new register per
    // stage: either costs the compiler's wait counts their precision). Only
    // the last stage of a K that is not a multiple of KS checks each lane.
    auto issue = [&](int st, int slot) __attribute__((always_inline)) {
        const int k0 = st * KS;
        uint8_t* const base = lds + slot * kStage;
        if (__builtin_expect(st + 1 < n_stages || K % KS == 0 || st >= n_stages, 1)) {
#pragma unroll
            for (int i = 0; i < kLoads; ++i) {
                const int piece = wave + kMidWaves * i;                       // uniform
                const bool real = piece < C::kInstr, isa = piece * 1024 < C::kABytes;
                lds_void* dst = (lds_void*)(real ? base + piece * 1024 : pad);
                const int so = !real || st >= n_stages ? kPastEnd : (isa ? k0 * 2 : k0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(isa ? ra : rw, dst, 16, off[i], so, 0, 0);
            }
        } else {
            const int kl = K - k0;
#pragma unroll
            for (int i = 0; i < kLoads; ++i) {
                const int piece = wave + kMidWaves * i;
                const bool real = piece < C::kInstr, isa = piece * 1024 < C::kABytes;
                lds_void* dst = (lds_void*)(real ? base + piece * 1024 : pad);
                const int so = !real ? kPastEnd : (isa ? k0 * 2 : k0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(isa ? ra : rw, dst, 16, kof[i] < kl ? off[i] : kOutOfRange,
                                                         so, 0, 0);
            }
        }
    };

    // Lane-constant operand addresses in a stage, per MFMA step s of the
    // wave's k-range (KW wide from kq * KW): lane group g carries k = kq * KW
    // + 32s + 8g + [0, 8) for both operands; A 16 bytes, W 8.
    int a_addr[MBW][kSteps], w_addr[NBW][kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        const int k = kq * KW + 32 * s + 8 * g;
#pragma unroll
        for (int i = 0; i < MBW; ++i) a_addr[i][s] = a_pos<KS>((mq * MBW + i) * 16 + r, k / 8);
#pragma unroll
        for (int j = 0; j < NBW; ++j)
            w_addr[j][s] = C::kABytes + w_pos<KS>((nq * NBW + j) * 16 + r, k / 16) + (k % 16);
    }
    // The tile's block scales, an fp32 table [row - j0][k-block] in LDS for
    // rows j0 .. j1 of the grid. Those rows lie one after another in memory;
    // they are copied once by DMA, as the dwords from the 4-byte boundary at
    // or below the first scale (a dword that holds a scale cannot cross a
    // page): FP32 straight into the table, BF16 into the ring's last slot
    // (free until the prologue refills it), from where the prologue widens
    // them into the table. Every wave issues kScaleLoads 256-byte loads
    // (past the copy: the pad, reading nothing), so the DMA counts stay the
    // same in every wave; they go before the ring's first stages, so the
    // wait for stage 0 covers them.
    constexpr bool kBf16Scale = SF == kScaleBlockBf16;
    constexpr int kEsz = kBf16Scale ? 2 : 4;
    constexpr int kScaleLoads =
        kRowScale ? 0 : (C::kScaleTable / (kEsz == 4 ? 1 : 2) + 4 + 255) / 256 / kMidWaves + 1;
    static_assert(kRowScale || C::kScaleTable / 2 + 256 + 4 <= kStage, "the BF16 copy fits a ring slot");
    const int j1 = min((n0 + TN - 1) / kScaleBlock, (N - 1) / kScaleBlock);
    const int n_scales = (j1 - j0 + 1) * k_blocks;
    uint8_t* const s_raw = kBf16Scale ? lds + (STAGES - 1) * kStage : stab;
    int s_lead = 0;
    if constexpr (!kRowScale) {
        const uintptr_t first = reinterpret_cast<uintptr_t>(S) + static_cast<uintptr_t>(j0) * k_blocks * kEsz;
        s_lead = static_cast<int>(first & 3);
        const int nrec = (s_lead + n_scales * kEsz + 3) & ~3;
        const int n_instr = (nrec + 255) / 256;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<void*>(first - s_lead), 0, nrec, kBufferFlags);
#pragma unroll
        for (int i = 0; i < kScaleLoads; ++i) {
            const int q = wave + kMidWaves * i;                                // uniform
            const bool real = q < n_instr;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(real ? s_raw + q * 256 : pad), 4, lane * 4,
                                                     real ? q * 256 : kPastEnd, 0, 0);
        }
    }
    // The table byte of each of the wave's column blocks' scale row (a block
    // past N reads row j0: its weights are zero), and the wave's first scale
    // block in a stage.
    int srow[NBW];
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
        const int n = n0 + (nq * NBW + j) * 16;
        srow[j] = ((n < N ? n / kScaleBlock : j0) - j0) * k_blocks * 4;
    }
    const int kb_wave = (kq * KW) / kScaleBlock;

    // The wave's operands of stage st from ring slot `slot`, and its scales
    // from the table (a scale block past K reads the last one: its products
    // are zero).
    auto read_ops = [&](int st, int slot, MidOps<C>& o) __attribute__((always_inline)) {
        const uint8_t* const base = lds + slot * kStage;
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
#pragma unroll
            for (int j = 0; j < NBW; ++j)
                // (a vector type: through the uint2 struct the compiler waits
                // for every DMA in flight before this read)
                o.w[j][s] = *reinterpret_cast<const u32x2_t*>(base + w_addr[j][s]);
#pragma unroll
            for (int i = 0; i < MBW; ++i) o.a[i][s] = *reinterpret_cast<const bf16x8_t*>(base + a_addr[i][s]);
        }
        if constexpr (!kRowScale) {
#pragma unroll
            for (int b = 0; b < kBlocks; ++b) {
                const int kb = min(st * (KS / kScaleBlock) + kb_wave + b, k_blocks - 1);
#pragma unroll
                for (int j = 0; j < NBW; ++j) o.s[j][b] = *reinterpret_cast<const float*>(stab + srow[j] + kb * 4);
            }
        }
    };

    const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
    f32x4_t acc[MBW][NBW];
#pragma unroll
    for (int i = 0; i < MBW; ++i)
#pragma unroll
        for (int j = 0; j < NBW; ++j) acc[i][j] = zero;

    // The wave's MFMAs on one stage's operands, with the exact fold per scale
    // block (acc += s * blk over the wave's part of the block).
    auto compute = [&](const MidOps<C>& o) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < kBlocks; ++b) {
            f32x4_t blk[MBW][NBW];
#pragma unroll
            for (int s = b * kSpb; s < (b + 1) * kSpb; ++s) {
                bf16x8_t bw[NBW];
#pragma unroll
                for (int j = 0; j < NBW; ++j) bw[j] = e4m3x8(o.w[j][s].x, o.w[j][s].y);
#pragma unroll
                for (int i = 0; i < MBW; ++i)
#pragma unroll
                    for (int j = 0; j < NBW; ++j) {
                        if constexpr (kRowScale)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.a[i][s], bw[j], acc[i][j], 0, 0, 0);
                        else
                            blk[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                o.a[i][s], bw[j], s == b * kSpb ? zero : blk[i][j], 0, 0, 0);
                    }
            }
            if constexpr (!kRowScale) {
#pragma unroll
                for (int j = 0; j < NBW; ++j)
#pragma unroll
                    for (int i = 0; i < MBW; ++i)
#pragma unroll
                        for (int v = 0; v < 4; ++v) acc[i][j][v] = fmaf(blk[i][j][v], o.s[j][b], acc[i][j][v]);
            }
        }
    };

    // Pipeline. The ring holds stages st + 1 .. st + STAGES while stage st is
    // multiplied from registers: each step waits for this wave's DMA of stage
    // st + 1 and for its own reads of stage st (already in registers), then a
    // barrier (every wave's DMA of st + 1 has landed and every wave is done
    // reading st), refills st's slot with stage st + STAGES, reads stage
    // st + 1's operands, and multiplies stage st.
#pragma unroll
    for (int sl = 0; sl + 1 < STAGES; ++sl) issue(sl, sl);
    MidOps<C> ops0, ops1;
    constexpr int kOpsRegs = MBW * kSteps * 4 + NBW * kSteps * 2 + NBW * kBlocks;
    constexpr bool kPinReads = 2 * kOpsRegs + 8 * MBW * NBW <= 200;
    wait_vmem<(STAGES - 2) * kLoads>();
    lds_barrier();
    if constexpr (kBf16Scale) {
        // BF16 -> fp32 is exact: the BF16 bits become the high half.
        for (int e = threadIdx.x; e < n_scales; e += kMidThreads)
            reinterpret_cast<float*>(stab)[e] =
                __uint_as_float(static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(s_raw + s_lead + 2 * e))
                                << 16);
        __builtin_amdgcn_s_waitcnt(0xC07F);                                // lgkmcnt(0): the table is written
        lds_barrier();
    }
    read_ops(0, 0, ops0);
    issue(STAGES - 1, STAGES - 1);
    auto step = [&](int st, int slot, const MidOps<C>& cur, MidOps<C>& nxt) __attribute__((always_inline)) {
        wait_vmem<(STAGES - 2) * kLoads>();
        __builtin_amdgcn_s_waitcnt(0xC07F);                                // lgkmcnt(0): this wave's reads of st
        lds_barrier();
        issue(st + STAGES, slot);
        const int nslot = slot + 1 == STAGES ? 0 : slot + 1;
        // (also after the last stage, reading a stale slot that is never
        // used: a branch here makes the compiler wait for these reads
        // before the MFMAs below)
        read_ops(st + 1, nslot, nxt);
        // Kept ahead of the products where the registers allow (the
        // scheduler would otherwise sink the reads below them, and their
        // latency would then show at the next barrier).
        if constexpr (kPinReads) __builtin_amdgcn_sched_barrier(0);
        compute(cur);
        return nslot;
    };
    int slot = 0;
    for (int st = 0; st < n_stages; st += 2) {
        slot = step(st, slot, ops0, ops1);
        if (st + 1 < n_stages) slot = step(st + 1, slot, ops1, ops0);
    }
    wait_vmem<0>();                                 // the zero loads past the last stage
    lds_barrier();                                  // every wave is done with the ring

    // Partial tiles, [kq][row][column] fp32 (16x16 MFMA result layout: lane l
    // holds column l % 16, rows 4(l/16) + v), then each thread takes runs of
    // 4 columns of a row: the sum over kq in order, the row scale, the
    // residual, BF16.
    float* const part = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int i = 0; i < MBW; ++i)
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                part[(kq * TM + (mq * MBW + i) * 16 + 4 * g + v) * TN + (nq * NBW + j) * 16 + r] = acc[i][j][v];
    __syncthreads();
    const bool vec = (reinterpret_cast<uintptr_t>(out) % 8) == 0 && (ldo % 4) == 0 &&
                     (!RES || (reinterpret_cast<uintptr_t>(res) % 8) == 0);
    for (int q = threadIdx.x; q < TM * (TN / 4); q += kMidThreads) {
        const int row = q / (TN / 4), col = (q % (TN / 4)) * 4;
        const int m = m0 + row, n = n0 + col;
        if (m >= M || n >= N) continue;
        f32x4_t sum = *reinterpret_cast<const f32x4_t*>(part + row * TN + col);
#pragma unroll
        for (int k2 = 1; k2 < C::KQ; ++k2) sum += *reinterpret_cast<const f32x4_t*>(part + (k2 * TM + row) * TN + col);
        mid_store4<SF, RES>(sum, S, res, out, m, n, N, ldo, vec);
    }
}

// The kernel is a thin wrapper: with the body (whose lambdas issue the LDS
// DMA) directly in a __global__ template, the host compilation pass emits no
// launch stub for it.
template <class C, int SF, bool RES>
__global__ void __launch_bounds__(kMidThreads, 1)
mid_kernel(const uint16_t* __restrict__ A, const uint8_t* __restrict__ W, const void* __restrict__ S,
           const uint16_t* __restrict__ res, uint16_t* __restrict__ out, int M, int N, int K, int tiles_m,
           int64_t ldo) {
    mid_body<C, SF, RES>(A, W, S, res, out, M, N, K, tiles_m, ldo);
}

// Tile shapes the planner chooses from (MB, NB), each with its split of the
// waves and as many stages as LDS allows.
struct MidShape {
    int mb, nb;
};
constexpr MidShape kMidShapes[] = {{1, 2}, {1, 4}, {2, 4}, {4, 4}, {2, 5}, {4, 5}, {4, 10}, {8, 10}};
// 256 of K per stage where a stage fits LDS about 3 times or more (measured
// faster than 128 with more stages: half the barriers); the 160-column tiles
// (the Mamba-2 in_proj at 128 and 256 tokens) stage 128.
using Mid0 = MidCfg<1, 2, 1, 2, 4, 256, 9>;
using Mid1 = MidCfg<1, 4, 1, 4, 2, 256, 6>;
using Mid2 = MidCfg<2, 4, 1, 4, 2, 256, 4>;
using Mid3 = MidCfg<4, 4, 1, 4, 2, 256, 3>;
using Mid4 = MidCfg<2, 5, 2, 1, 4, 256, 4>;
using Mid5 = MidCfg<4, 5, 2, 1, 4, 256, 3>;
using Mid6 = MidCfg<4, 10, 2, 2, 2, 128, 4>;
using Mid7 = MidCfg<8, 10, 4, 2, 1, 128, 3>;

template <class C, int SF, bool RES>
int launch_mid(const void* A, const void* Wq, const void* scale, const void* residual, void* out, int M, int N,
               int K, int64_t ldo, hipStream_t stream) {
    const int tiles_m = static_cast<int>(ceil_div(M, C::TM));
    const int64_t tiles = static_cast<int64_t>(tiles_m) * ceil_div(N, C::TN);
    return launch(&mid_kernel<C, SF, RES>, dim3(static_cast<unsigned>(tiles)), dim3(kMidThreads), stream,
                  static_cast<const uint16_t*>(A), static_cast<const uint8_t*>(Wq), scale,
                  static_cast<const uint16_t*>(residual), static_cast<uint16_t*>(out), M, N, K, tiles_m, ldo);
}

template <int SF, bool RES>
int mid_by_shape(int shape, const void* A, const void* Wq, const void* scale, const void* residual, void* out, int M,
                 int N, int K, int64_t ldo, hipStream_t s) {
    switch (shape) {
        case 0: return launch_mid<Mid0, SF, RES>(A, Wq, scale, residual, out, M, N, K, ldo, s);
        case 1: return launch_mid<Mid1, SF, RES>(A, Wq, scale, residual, out, M, N, K, ldo, s);
        case 2: return launch_mid<Mid2, SF, RES>(A, Wq, scale, residual, out, M, N, K, ldo, s);
        case 3: return launch_mid<Mid3, SF, RES>(A, Wq, scale, residual, out, M, N, K, ldo, s);
        case 4: return launch_mid<Mid4, SF, RES>(A, Wq, scale, residual, out, M, N, K, ldo, s);
        case 5: return launch_mid<Mid5, SF, RES>(A, Wq, scale, residual, out, M, N, K, ldo, s);
        case 6: return launch_mid<Mid6, SF, RES>(A, Wq, scale, residual, out, M, N, K, ldo, s);
        default: return launch_mid<Mid7, SF, RES>(A, Wq, scale, residual, out, M, N, K, ldo, s);
    }
}

}  // namespace

// Index into kMidShapes of the tile for (M, N, K) on `cus` CUs, or -1 when
// the mid-size kernel does not apply. A round of tiles costs a CU the larger
// of the bytes of its tile, K * (32 * MB + 16 * NB), at the feed this kernel
// reaches (measured 27-50 GB/s per CU on the Mamba-2 shapes; about 19 bytes
// per clock), and its matrix-core time, 512 * MB * NB * K flop at 4096 per
// clock over an efficiency of 0.5; the cheapest tile count wins (ties: the
// fewer tiles).
int mid_plan(int64_t M, int64_t N, int64_t K, int cus) {
    if (M < kMidMinM || M > kMidMaxM || K > kMidMaxK || cus <= 0) return -1;
    // 32-bit buffer offsets: a tile's rows of A, plus the zero-load offset.
    if (128 * 2 * K + 2 * K >= static_cast<int64_t>(kOutOfRange)) return -1;
    int best = -1;
    double best_cost = 0.0;
    int64_t best_tiles = 0;
    for (int i = 0; i < static_cast<int>(sizeof(kMidShapes) / sizeof(kMidShapes[0])); ++i) {
        const MidShape& sh = kMidShapes[i];
        const int64_t tiles = ceil_div(M, 16 * sh.mb) * ceil_div(N, 16 * sh.nb);
        if (tiles > INT32_MAX) continue;
        const double rounds = static_cast<double>(ceil_div(tiles, cus));
        const double feed = static_cast<double>(K) * (32 * sh.mb + 16 * sh.nb) / 19.0;
        const double mfma = static_cast<double>(K) * sh.mb * sh.nb * 512.0 / 4096.0 / 0.5;
        const double cost = rounds * std::max(feed, mfma);
        if (best < 0 || cost < best_cost * 0.999 || (cost <= best_cost * 1.001 && tiles < best_tiles)) {
            best = i;
            best_cost = cost;
            best_tiles = tiles;
        }
    }
    return best;
}

int mid_gemm(const void* A, const void* Wq, const void* scale, int fmt, const void* residual, void* out, int64_t M,
             int64_t N, int64_t K, int64_t ldo, hipStream_t stream) {
    const int shape = mid_plan(M, N, K, device_cu_count());
    if (shape < 0) return W8A16_ERR_SHAPE;
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
    if (residual != nullptr)
        return mid_by_shape<kScaleBlockBf16, true>(shape, A, Wq, scale, residual, out, m, n, k, ldo, stream);
    switch (fmt) {
        case W8A16_SCALE_BLOCK_F32:
            return mid_by_shape<kScaleBlockF32, false>(shape, A, Wq, scale, nullptr, out, m, n, k, ldo, stream);
        case W8A16_SCALE_ROW_F32:
            return mid_by_shape<kScaleRowF32, false>(shape, A, Wq, scale, nullptr, out, m, n, k, ldo, stream);
        default:
            return mid_by_shape<kScaleBlockBf16, false>(shape, A, Wq, scale, nullptr, out, m, n, k, ldo, stream);
    }
}

}  // namespace w8a16
