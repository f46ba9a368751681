// Decode GEMV for the w8a16 block-scaled FP8 projection, M = 1..16 rows of A.
//
//   out[m][n] = sum_k A[m][k] * E4M3(W[n][k]) * scale[n/128][k/128]
// (Qwen3SsmLayer docs, `set_fp8_decode_weights`; NemotronMamba2Layer docs,
// `set_fp8_weights` for the block index). Decode runs it once per token per
// projection (nemotron_mamba2.rs module docs, forward steps 2 and 7), and the
// multi-sequence decode applies one weight pass to all rows
// (TransformerLayer docs, `decode_multi_seq`).
//
// The GEMV is HBM-bound: each weight byte is read exactly once per call, so
// the design is about keeping enough 16-byte loads in flight on every CU:
//  * K is split across the `kw` waves of a workgroup: wave w owns
//    k in [w*1024*J, (w+1)*1024*J), and lane l of it the 16-value chunks
//    k = w*1024*J + j*1024 + 16*l (j < J). One wave-wide load covers 1 KB of a
//    weight row, fully coalesced. The lane's activations for its chunks
//    (MR x J x 16 BF16) stay in registers for the whole kernel.
//  * Each workgroup streams a contiguous range of row groups (RB rows each);
//    the loads of the next group are issued before the current one is
//    reduced (two register buffers), and the grid is sized so every CU holds
//    several workgroups.
//  * Each 16-byte weight chunk is decoded once (8 packed E4M3->BF16
//    converts, exact) and used for all MR rows with v_dot2_f32_bf16. A chunk
//    lies inside one 128-wide scale block, so its 16-term partial sum is
//    multiplied by that block's scale in fp32 (exact dequantization).
//  * The RB*MR partial sums of a lane are reduced across the wave with a
//    butterfly that halves the value count at every step (so the cost per
//    output shrinks as RB*MR grows), then across the kw waves through LDS.
//    The order of every sum is fixed: results are deterministic. No atomics.
//  * Fused form (w8a16_gemv_fused; nemotron_mamba2.rs module docs, forward
//    steps 1, 6 and 8): the activations a lane holds are normalized in place
//    before the loop (the row's sum of squares is reduced over the workgroup
//    in a fixed order; the norm weight and the gate are read for the lane's
//    chunks only), and the residual is added at the output store.
#include <algorithm>

#include "w8a16_device.h"
#include "w8a16_host.h"

namespace w8a16 {
namespace {

constexpr int kChunk = 16;             // K values (bytes of W) per lane per load
constexpr uint32_t kOutOfRange = 0x80000000u;   // buffer offset that reads as zero
constexpr int kBufferFlags = 0x00020000;        // raw buffer, 32-bit data format
constexpr int kNonTemporal = 2;                 // cache policy of the weight stream: read once
constexpr int kWaveK = 64 * kChunk;    // K values covered by one wave-wide load
constexpr int kMaxWaves = 8;           // 512 threads: up to 256 VGPRs per lane
constexpr int kWavesPerCu = 8;         // resident waves per CU the grid aims for

constexpr int pow2_ceil(int v) { return v <= 1 ? 1 : 2 * pow2_ceil((v + 1) / 2); }
constexpr int log2i(int v) { return v <= 1 ? 0 : 1 + log2i(v / 2); }

// Butterfly reduction of COUNT values per lane over the 64 lanes. At each
// distance D the lanes with bit D set keep the upper half of the values and
// the others the lower half; each adds its partner's copy of the half it
// keeps. Once one value is left the remaining distances add plainly. Lane l
// ends with the wave-wide sum of value index l >> (6 - log2(P)).
template <int P, int COUNT, int D>
__device__ __forceinline__ void butterfly(float (&v)[P], int lane) {
    if constexpr (D >= 1) {
        if constexpr (COUNT > 1) {
            const bool upper = (lane & D) != 0;
#pragma unroll
            for (int i = 0; i < COUNT / 2; ++i) {
                const float keep = upper ? v[i + COUNT / 2] : v[i];
                const float send = upper ? v[i] : v[i + COUNT / 2];
                v[i] = keep + __shfl_xor(send, D);
            }
            butterfly<P, COUNT / 2, D / 2>(v, lane);
        } else {
            v[0] += __shfl_xor(v[0], D);
            butterfly<P, 1, D / 2>(v, lane);
        }
    }
}

// What a kernel fuses around the product (w8a16_gemv_fused): nothing (the
// plain GEMV), the residual epilogue only, or the RMSNorm / gated RMSNorm
// prologue (each with the residual epilogue when one is passed); and the
// in_proj form (w8a16_gemv_in_proj): the RMSNorm prologue with the conv1d
// update applied to the xBC columns as they are stored.
constexpr int kFuseNone = 0, kFuseResidual = 1, kFuseNorm = 2, kFuseGated = 3, kFuseNormConv = 4;

template <int MR, int J, int RB, int SF, int FU>
struct Gemv {
    static constexpr int V = RB * MR;          // partial sums per lane per group
    static constexpr int P = pow2_ceil(V);     // padded to a power of two for the butterfly
    static_assert(P <= 64, "at most one output per lane");
    static_assert(kScaleBlock % RB == 0, "a row group must stay inside one scale block");
    static constexpr int kLaneShift = 6 - log2i(P);   // lane l holds value l >> kLaneShift

    struct Regs {
        u32x4_t w[RB][J];
        uint32_t s_bits[J];        // the block scales' bits, decoded where they are used
    };

    // Group g's scales and weight rows into r. A group past the workgroup's
    // range (valid false) issues the same loads, which read zeros (an empty
    // buffer range; the scale of row-block 0), so that the loop below has no
    // branch around a load and the compiler's waits stay exact.
    __device__ static __forceinline__ void load(Regs& r, const uint8_t* __restrict__ W,
                                                const void* __restrict__ S, int g, bool valid, int N, int K,
                                                int k_blocks, const int (&kch)[J], const bool (&kvalid)[J]) {
        const int n0 = valid ? g * RB : 0;
        // The scales first: all RB rows sit in scale row-block n0/128, and
        // every row's sum needs them, so waiting for them must not wait for
        // the weight rows issued after them. The load is unconditional (a
        // lane past K reads block 0 of the row-block and its scale is
        // replaced by 0 where it is used), so that no branch makes the
        // compiler wait for the value right after the load.
#pragma unroll
        for (int j = 0; j < J; ++j) r.s_bits[j] = block_scale_bits<SF>(S, scale_index(n0, kvalid[j] ? kch[j] : 0, k_blocks));
        __builtin_amdgcn_sched_barrier(0);
        // Buffer loads over the group's rows, so there is no branch around
        // them and the compiler can wait for each row alone: a chunk past K
        // gets an offset past num_records and reads as zero; a row past N
        // re-reads the group's last row (the scalar offset), and its sum is
        // never stored. The lane offset is the same for every row.
        const int rows = valid ? min(RB, N - n0) : 0;
        const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(W + static_cast<int64_t>(n0) * K), 0, rows * K, kBufferFlags);
        uint32_t voff[J];
#pragma unroll
        for (int j = 0; j < J; ++j) voff[j] = kvalid[j] ? static_cast<uint32_t>(kch[j]) : kOutOfRange;
        // In row order (the scheduler would otherwise issue them in any
        // order, e.g. the last row first), so that row i's products wait for
        // rows 0..i only.
#pragma unroll
        for (int i = 0; i < RB; ++i) {
#pragma unroll
            for (int j = 0; j < J; ++j)
                r.w[i][j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                rw, voff[j], max(min(i, rows - 1), 0) * K, kNonTemporal));
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Output (m, n): BF16 of the sum, the residual epilogue, or on the conv
    // columns the conv1d update of the channel with this BF16 output as its
    // new input (each channel's output is stored by exactly one lane).
    __device__ static __forceinline__ void store(uint16_t* __restrict__ out, const uint16_t* __restrict__ res,
                                                 const Fusion& fu, int m, int n, int N, float val) {
        const int64_t o = static_cast<int64_t>(m) * N + n;
        if constexpr (FU == kFuseNormConv) {
            const int c = n - fu.conv_begin;
            if (c >= 0 && c < fu.conv_dim) {
                out[o] = conv_update_channel(fu.conv_state + (static_cast<int64_t>(m) * fu.conv_dim + c) * fu.d_conv,
                                             fu.conv_weight + static_cast<int64_t>(c) * fu.d_conv, fu.conv_bias + c,
                                             f32_to_bf16_bits(val), fu.d_conv);
                return;
            }
        }
        if constexpr (FU != kFuseNone)
            if (res) {
                out[o] = residual_out(val, res[o]);
                return;
            }
        out[o] = f32_to_bf16_bits(val);
    }

    __device__ static __forceinline__ void process(const Regs& r, const uint32_t (&a)[MR][J][8], const bool (&kvalid)[J],
                                                   float (*red)[kMaxWaves][V], int parity,
                                                   uint16_t* __restrict__ out, const uint16_t* __restrict__ res,
                                                   const Fusion& fu, const void* __restrict__ S,
                                                   int g, int N, int lane, int wave, int nwaves) {
        float v[P];
#pragma unroll
        for (int i = 0; i < P; ++i) v[i] = 0.0f;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const float sj = kvalid[j] ? scale_from_bits<SF>(r.s_bits[j]) : 0.0f;
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                bf16x2_t wv[8];
                e4m3x16_to_bf16(r.w[i][j], wv);
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    float p = 0.0f;
#pragma unroll
                    for (int t = 0; t < 8; ++t)
                        p = __builtin_amdgcn_fdot2_f32_bf16(
                            wv[t], __builtin_bit_cast(bf16x2_t, a[m][j][t]), p, false);
                    v[i * MR + m] = fmaf(p, sj, v[i * MR + m]);
                }
                // Row by row: the scheduler would otherwise interleave the
                // rows' converts, and the first product would wait for the
                // group's last row (and for any loads issued after it).
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        butterfly<P, P, 32>(v, lane);

        const int idx = lane >> kLaneShift;                       // value this lane now holds
        const bool holder = (lane & ((1 << kLaneShift) - 1)) == 0 && idx < V;
        const int n0 = g * RB;
        if (nwaves == 1) {
            if (holder) {
                const int i = idx / MR, m = idx % MR;
                if (n0 + i < N)
                    store(out, res, fu, m, n0 + i, N, v[0] * row_scale<SF>(S, n0 + i));
            }
        } else {
            if (holder) red[parity][wave][idx] = v[0];
            __syncthreads();
            if (wave == 0 && lane < V) {
                float tot = 0.0f;
                for (int w = 0; w < nwaves; ++w) tot += red[parity][w][lane];
                const int i = lane / MR, m = lane % MR;
                if (n0 + i < N)
                    store(out, res, fu, m, n0 + i, N, tot * row_scale<SF>(S, n0 + i));
            }
            // The next group writes red[parity ^ 1]; red[parity] is written
            // again only after the next barrier, which wave 0 reaches after
            // it has read red[parity].
        }
    }
};

// The norm prologue on the activations a lane holds (rows of MR, chunks
// kch[j]), in place: a = bf16(x * r * weight [* silu(gate)]), r from the
// row's sum of squares over all K, reduced over the wave, then over the
// waves in order. issue() loads the norm weight (and, for one or two rows,
// the gate) while registers allow; the kernel calls it before the first
// weight group's loads, so that waiting for the activations and these
// operands never waits for the weight stream, and the reduction overlaps
// the weights' HBM latency.
template <int MR, int J, bool GATED>
struct NormOps {
    static constexpr bool kEarlyGate = GATED && MR * J <= 2, kEarlyWeight = MR * J < 8;
    u32x4_t wv[J][2];
    u32x4_t gv[kEarlyGate ? MR : 1][J][2];

    __device__ __forceinline__ void load_weight(const Fusion& fu, const int (&kch)[J], const bool (&kvalid)[J],
                                                int j) {
        const u32x4_t zero = {0u, 0u, 0u, 0u};
        wv[j][0] = kvalid[j] ? load16(fu.weight + kch[j]) : zero;
        wv[j][1] = kvalid[j] ? load16(fu.weight + kch[j] + 8) : zero;
    }

    __device__ __forceinline__ void issue(const Fusion& fu, int K, const int (&kch)[J], const bool (&kvalid)[J]) {
        const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < J; ++j) {
            if constexpr (kEarlyWeight) load_weight(fu, kch, kvalid, j);
            if constexpr (kEarlyGate)
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    const uint16_t* g = fu.gate + static_cast<int64_t>(m) * fu.ld_gate + kch[j];
                    gv[m][j][0] = kvalid[j] ? load16(g) : zero;
                    gv[m][j][1] = kvalid[j] ? load16(g + 8) : zero;
                }
        }
    }

    __device__ __forceinline__ void apply(uint32_t (&a)[MR][J][8], const Fusion& fu, int K, const int (&kch)[J],
                                          const bool (&kvalid)[J], int lane, int wave, int nwaves) {
        static_assert(MR * J <= 16, "one LDS slot per row and chunk");
        __shared__ float ssq[kMaxWaves][16];
        float r[MR][J];
        const int group = fu.group > 0 ? fu.group : K;
        if (group == K) {
            // One norm over the whole row: every chunk of row m shares r.
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                float ss = 0.0f;
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    ss += sumsq8(u32x4_t{a[m][j][0], a[m][j][1], a[m][j][2], a[m][j][3]});
                    ss += sumsq8(u32x4_t{a[m][j][4], a[m][j][5], a[m][j][6], a[m][j][7]});
                }
                r[m][0] = wave_sum(ss);
            }
            if (lane == 0)
#pragma unroll
                for (int m = 0; m < MR; ++m) ssq[wave][m] = r[m][0];
            __syncthreads();
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                float t = 0.0f;
                for (int w = 0; w < nwaves; ++w) t += ssq[w][m];
#pragma unroll
                for (int j = 0; j < J; ++j) r[m][j] = rms_factor(t, K, fu.eps);
            }
        } else {
            // In groups (a multiple of kWaveK channels): a wave's chunk j
            // (kWaveK channels from wave * kWaveK * J + j * kWaveK) lies in one
            // group; its sum goes to LDS, and each row's group adds the parts
            // of its chunks in order.
#pragma unroll
            for (int m = 0; m < MR; ++m)
#pragma unroll
                for (int j = 0; j < J; ++j)
                    r[m][j] = wave_sum(sumsq8(u32x4_t{a[m][j][0], a[m][j][1], a[m][j][2], a[m][j][3]}) +
                                       sumsq8(u32x4_t{a[m][j][4], a[m][j][5], a[m][j][6], a[m][j][7]}));
            if (lane == 0)
#pragma unroll
                for (int m = 0; m < MR; ++m)
#pragma unroll
                    for (int j = 0; j < J; ++j) ssq[wave][m * J + j] = r[m][j];
            __syncthreads();
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int g = (wave * kWaveK * J + j * kWaveK) / group;
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    float t = 0.0f;
                    for (int w = 0; w < nwaves; ++w)
                        for (int j2 = 0; j2 < J; ++j2) {
                            const int ch = w * kWaveK * J + j2 * kWaveK;
                            if (ch < K && ch / group == g) t += ssq[w][m * J + j2];
                        }
                    r[m][j] = rms_factor(t, group, fu.eps);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < J; ++j) {
            if (!kvalid[j]) continue;
            if constexpr (!kEarlyWeight) load_weight(fu, kch, kvalid, j);
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const u32x4_t xl = {a[m][j][0], a[m][j][1], a[m][j][2], a[m][j][3]};
                const u32x4_t xh = {a[m][j][4], a[m][j][5], a[m][j][6], a[m][j][7]};
                u32x4_t nl, nh;
                if constexpr (GATED) {
                    u32x4_t gl, gh;
                    if constexpr (kEarlyGate) {
                        gl = gv[m][j][0];
                        gh = gv[m][j][1];
                    } else {
                        const uint16_t* g = fu.gate + static_cast<int64_t>(m) * fu.ld_gate + kch[j];
                        gl = load16(g);
                        gh = load16(g + 8);
                    }
                    nl = norm8<true>(xl, wv[j][0], gl, r[m][j]);
                    nh = norm8<true>(xh, wv[j][1], gh, r[m][j]);
                } else {
                    const u32x4_t zero = {0u, 0u, 0u, 0u};
                    nl = norm8<false>(xl, wv[j][0], zero, r[m][j]);
                    nh = norm8<false>(xh, wv[j][1], zero, r[m][j]);
                }
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    a[m][j][t] = nl[t];
                    a[m][j][4 + t] = nh[t];
                }
            }
        }
    }
};

// How a workgroup walks its groups. kLoopAll: a double-buffered loop whose
// next-group loads are always issued (past the range they read zeros), so
// the compiler's waits stay per row; for several groups per workgroup.
// kOneGroup: exactly one group each (groups_per_block == 1), no loop.
// kLoopGuarded: the loop with the next-group loads behind a branch; with one
// group per workgroup, the plain (unfused) decode's form, measured faster
// there than kOneGroup (in_proj 13.57 against 13.71-13.74 us, out_proj 8.02-
// 8.04 against 8.19-8.23 us; the one-group form takes fewer registers and
// packs more workgroups per CU).
constexpr int kLoopAll = 0, kOneGroup = 1, kLoopGuarded = 2;

template <int MR, int J, int RB, int SF, int FU, int WALK>
__global__ void __launch_bounds__(kMaxWaves * 64)
gemv_kernel(const uint16_t* __restrict__ A, const uint8_t* __restrict__ W,
            const void* __restrict__ S, uint16_t* __restrict__ out,
            int N, int K, int groups_per_block, Fusion fu) {
    using G = Gemv<MR, J, RB, SF, FU>;
    constexpr bool kNorm = FU == kFuseNorm || FU == kFuseGated || FU == kFuseNormConv;
    __shared__ float red[2][kMaxWaves][G::V];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const int k_blocks = (K + kScaleBlock - 1) / kScaleBlock;

    const int groups = (N + RB - 1) / RB;
    const int g_begin = blockIdx.x * groups_per_block;
    const int g_end = min(groups, g_begin + groups_per_block);
    if (g_begin >= g_end) return;                              // uniform over the workgroup

    int kch[J];
    bool kvalid[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        kch[j] = wave * (kWaveK * J) + j * kWaveK + lane * kChunk;
        kvalid[j] = kch[j] < K;
    }

    // Activations of this lane's chunks, as packed BF16 pairs (k, k+1). They
    // are loaded before the first group's weights: a wave's memory loads
    // complete in issue order, so this way the first row's products wait
    // for the activations and that row only, and each later row is reduced
    // as it arrives while the rest of the group is still streaming in.
    // Chunks past K read as zero (beyond num_records).
    typename G::Regs ra, rb;
    uint32_t a[MR][J][8];
    const __amdgpu_buffer_rsrc_t rsrc_a =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(A), 0, MR * K * 2, kBufferFlags);
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const uint32_t off = static_cast<uint32_t>((m * K + kch[j]) * 2);
            const u32x4_t lo = __builtin_bit_cast(
                u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc_a, kvalid[j] ? off : kOutOfRange, 0, 0));
            const u32x4_t hi = __builtin_bit_cast(
                u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc_a, kvalid[j] ? off + 16 : kOutOfRange, 0, 0));
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                a[m][j][t] = lo[t];
                a[m][j][4 + t] = hi[t];
            }
        }

    if constexpr (kNorm) {
        NormOps<MR, J, FU == kFuseGated> no;
        no.issue(fu, K, kch, kvalid);
        G::load(ra, W, S, g_begin, true, N, K, k_blocks, kch, kvalid);
        no.apply(a, fu, K, kch, kvalid, lane, wave, nwaves);
    } else {
        G::load(ra, W, S, g_begin, true, N, K, k_blocks, kch, kvalid);
    }
    const uint16_t* res = FU != kFuseNone ? fu.residual : nullptr;

    if constexpr (WALK == kOneGroup) {
        G::process(ra, a, kvalid, red, 0, out, res, fu, S, g_begin, N, lane, wave, nwaves);
        return;
    }
    // Double buffer: the next group's loads go out before this group's
    // products.
    int parity = 0;
    for (int g = g_begin; g < g_end; g += 2) {
        if (WALK == kLoopAll || g + 1 < g_end) G::load(rb, W, S, g + 1, g + 1 < g_end, N, K, k_blocks, kch, kvalid);
        G::process(ra, a, kvalid, red, parity, out, res, fu, S, g, N, lane, wave, nwaves);
        parity ^= 1;
        if (g + 1 >= g_end) break;
        if (WALK == kLoopAll || g + 2 < g_end) G::load(ra, W, S, g + 2, g + 2 < g_end, N, K, k_blocks, kch, kvalid);
        G::process(rb, a, kvalid, red, parity, out, res, fu, S, g + 1, N, lane, wave, nwaves);
        parity ^= 1;
    }
}

typedef void (*gemv_fn)(const uint16_t*, const uint8_t*, const void*, uint16_t*, int, int, int, Fusion);

// Chunks per lane: 1 while K <= 8192 (8 waves of 1024), 2 up to 16384 (M <= 8).
constexpr int max_chunks(int mr) { return mr <= 8 ? 2 : 1; }

// Rows per group: up to 16 loads per lane per buffer, at most 64 partial sums
// per lane, and a power of two (so a group never straddles a scale block).
constexpr int rows_per_group(int mr, int j) {
    int rb = 16 / j;
    while (rb * mr > 64 && rb > 1) rb /= 2;
    if (mr * j * 8 >= 64 && rb * j > 8) rb = 8 / j;   // big activation footprint: 8 loads per buffer
    return rb;
}

// The in_proj form's conv epilogue needs a few more registers: a group of
// 64 partial sums per lane (4 rows x 16) is halved so that it does not spill.
constexpr int rows_for(int mr, int j, int fu) {
    const int rb = rows_per_group(mr, j);
    return fu == kFuseNormConv && mr * rb >= 64 ? rb / 2 : rb;
}

// The kernels of one configuration: for several groups per workgroup, and
// for one (the fused forms without a loop, the plain form with its guarded
// loop).
struct Choice {
    gemv_fn fn;
    gemv_fn fn_one;
    int rows_per_group;
};

template <int MR, int J, int RB, int SF, int FU>
Choice kernels() {
    return {&gemv_kernel<MR, J, RB, SF, FU, kLoopAll>,
            &gemv_kernel<MR, J, RB, SF, FU, FU == kFuseNone ? kLoopGuarded : kOneGroup>, RB};
}

template <int MR, int J, int SF, int FU>
Choice pick_j() {
    return kernels<MR, J, rows_for(MR, J, FU), SF, FU>();
}

// The fused kernels hold the norm's operands beside the activations; they
// fit in registers without spilling for M <= 4 (any K up to 16384) and for
// M <= 8 with K <= 8192 (one chunk per lane).
constexpr int64_t kFusedMaxM = 8, kFusedMaxMTwoChunks = 4;
inline bool fused_fits(int64_t M, int64_t K) {
    return M >= 1 && (M <= kFusedMaxMTwoChunks ? K <= W8A16_GEMV_MAX_K_SMALL_M
                                               : M <= kFusedMaxM && K <= kWaveK * kMaxWaves);
}

template <int MR, int SF, int FU>
Choice pick(int j) {
    if constexpr (max_chunks(MR) >= 2 && (FU == kFuseNone || MR <= kFusedMaxMTwoChunks))
        if (j == 2) return pick_j<MR, 2, SF, FU>();
    return pick_j<MR, 1, SF, FU>();
}

template <int MR, int SF, int FU>
Choice choose(int j) {
    return pick<MR, SF, FU>(j);
}

template <int SF>
Choice select_plain(int mr, int j);

template <int SF, int FU>
Choice select_kernel(int mr, int j) {
    if constexpr (FU != kFuseNone) {
        switch (mr) {
            case 1: return choose<1, SF, FU>(j);
            case 2: return choose<2, SF, FU>(j);
            case 3: return choose<3, SF, FU>(j);
            case 4: return choose<4, SF, FU>(j);
            case 5: return choose<5, SF, FU>(j);
            case 6: return choose<6, SF, FU>(j);
            case 7: return choose<7, SF, FU>(j);
            default: return choose<8, SF, FU>(j);
        }
    } else {
        return select_plain<SF>(mr, j);
    }
}

template <int SF>
Choice select_plain(int mr, int j) {
    switch (mr) {
        case 1: return choose<1, SF, kFuseNone>(j);
        case 2: return choose<2, SF, kFuseNone>(j);
        case 3: return choose<3, SF, kFuseNone>(j);
        case 4: return choose<4, SF, kFuseNone>(j);
        case 5: return choose<5, SF, kFuseNone>(j);
        case 6: return choose<6, SF, kFuseNone>(j);
        case 7: return choose<7, SF, kFuseNone>(j);
        case 8: return choose<8, SF, kFuseNone>(j);
        case 9: return choose<9, SF, kFuseNone>(j);
        case 10: return choose<10, SF, kFuseNone>(j);
        case 11: return choose<11, SF, kFuseNone>(j);
        case 12: return choose<12, SF, kFuseNone>(j);
        case 13: return choose<13, SF, kFuseNone>(j);
        case 14: return choose<14, SF, kFuseNone>(j);
        case 15: return choose<15, SF, kFuseNone>(j);
        default: return choose<16, SF, kFuseNone>(j);
    }
}

// A few tokens (2..4) on a shape with at least 8 four-row groups per CU and
// K of one chunk per lane (the Mamba-2 in_proj): the single-token launch
// shape, 4-row groups with one group per workgroup, every load issued at the
// start. Measured on the in_proj (K = 4096, N = 18560): 14.8 / 17.0 / 18.7 us
// at M = 2 / 3 / 4 against 18.6 / 19.1 / 20.1 us for the skinny MFMA kernel,
// which stays faster from M = 5 (17.8 against 21.2 us) and on the out_proj
// (8.6 against 9.1 us at M = 2).
constexpr int64_t kValuFewMaxM = 4;
inline bool valu_few_tokens(int64_t M, int64_t N, int64_t K, int64_t cus) {
    return M >= 2 && M <= kValuFewMaxM && K <= static_cast<int64_t>(kWaveK) * kMaxWaves && ceil_div(N, 4) >= 8 * cus;
}

// The launch of the GEMV for scale format SF, fused or not (arguments
// checked).
template <int SF, int FU>
int run_gemv(const void* A, const void* Wq, const void* scale, void* out, int64_t M, int64_t N, int64_t K,
             hipStream_t stream, Fusion fu = Fusion{}) {
    const int mr = static_cast<int>(M);
    const int j = K > static_cast<int64_t>(kWaveK) * kMaxWaves ? 2 : 1;
    const int nwaves = static_cast<int>(ceil_div(K, static_cast<int64_t>(kWaveK) * j));
    if (nwaves > kMaxWaves || j > max_chunks(mr)) return W8A16_ERR_SHAPE;
    Choice c = select_kernel<SF, FU>(mr, j);
    const int64_t cus = device_cu_count();
    int64_t per_block;
    if (mr == 1 && j == 1) {
        // Single-token decode, launch shape measured on the Mamba-2 projection
        // shapes: 4-row groups while they number at least 8 per CU (in_proj),
        // else 16-row groups while there is one for every CU (out_proj: 8.0
        // against 8.1 us with 8-row groups), else 8-row groups; one group per
        // workgroup up to about 18 workgroups per CU, then several.
        const int rb = ceil_div(N, 4) >= 8 * cus ? 4 : ceil_div(N, 16) >= cus ? 16 : 8;
        c = rb == 4 ? kernels<1, 1, 4, SF, FU>() : rb == 16 ? kernels<1, 1, 16, SF, FU>() : kernels<1, 1, 8, SF, FU>();
        per_block = std::max<int64_t>(1, ceil_div(N, rb) / (18 * cus));
        if constexpr (FU == kFuseNorm || FU == kFuseGated || FU == kFuseNormConv) {
            // Every workgroup normalizes the whole activation row before its
            // products, so the norm forms take more rows per workgroup:
            // 8-row groups, and two of them per workgroup behind the gated
            // norm (whose prologue also computes silu of the gate). Measured
            // on the Mamba-2 projections: in_proj 15.2 -> 14.3 us, out_proj
            // 10.0 -> 9.1 us.
            c = kernels<1, 1, 8, SF, FU>();
            per_block = FU == kFuseGated ? 2 : 1;
        }
    } else if (FU == kFuseNone && valu_few_tokens(M, N, K, cus)) {
        c = mr == 2 ? kernels<2, 1, 4, SF, FU>() : mr == 3 ? kernels<3, 1, 4, SF, FU>() : kernels<4, 1, 4, SF, FU>();
        per_block = std::max<int64_t>(1, ceil_div(N, 4) / (18 * cus));
    } else {
        const int64_t resident = cus * (kWavesPerCu / nwaves > 0 ? kWavesPerCu / nwaves : 1);
        per_block = ceil_div(ceil_div(N, c.rows_per_group), resident);
    }
    const int64_t groups = ceil_div(N, c.rows_per_group);
    const int64_t blocks = ceil_div(groups, per_block);

    return launch(per_block == 1 ? c.fn_one : c.fn, dim3(static_cast<unsigned>(blocks)), dim3(64 * nwaves), stream,
                  static_cast<const uint16_t*>(A), static_cast<const uint8_t*>(Wq), scale,
                  static_cast<uint16_t*>(out), static_cast<int>(N), static_cast<int>(K),
                  static_cast<int>(per_block), fu);
}

}  // namespace
}  // namespace w8a16

extern "C" int w8a16_gemv_ex(const void* A, const void* Wq, const void* scale, int scale_format, void* out,
                             int64_t M, int64_t N, int64_t K, void* stream) {
    using namespace w8a16;
    bool noop = false;
    const int st = check_product_args(A, Wq, scale, out, M, N, K, &noop, scale_format);
    if (st != W8A16_OK || noop) return st;
    if (M > W8A16_GEMV_MAX_M || K > (M <= 8 ? W8A16_GEMV_MAX_K_SMALL_M : W8A16_GEMV_MAX_K))
        return W8A16_ERR_SHAPE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // From 2 rows on, the skinny GEMM (the same single weight pass, products
    // on the matrix cores) is faster where its one-shot form applies
    // (measured on the Mamba-2 shapes: in_proj 17.3 against 18.8 us at M = 2;
    // out_proj 8.6 against 10.0 us at M = 4, 9.2 against 14.4 at M = 8); from
    // 4 rows on its ring form is too, where it applies (in_proj: 21 against
    // 23 us at M = 4, 22 against 49 us at M = 16): the products cost the VALU
    // GEMV more than the weight stream takes. Except for 2..4 rows on the
    // in_proj-sized shapes, which run the GEMV with the single-token launch
    // shape (valu_few_tokens).
    const int cus = device_cu_count();
    if (!valu_few_tokens(M, N, K, cus) &&
        ((M >= 2 && skinny_lds_fits(M, N, K, cus)) || (M >= 4 && skinny_fits(M, K))))
        return skinny_gemm(A, Wq, scale, scale_format, nullptr, out, M, N, K, s);
    switch (scale_format) {
        case W8A16_SCALE_BLOCK_F32: return run_gemv<kScaleBlockF32, kFuseNone>(A, Wq, scale, out, M, N, K, s);
        case W8A16_SCALE_ROW_F32: return run_gemv<kScaleRowF32, kFuseNone>(A, Wq, scale, out, M, N, K, s);
        default: return run_gemv<kScaleBlockBf16, kFuseNone>(A, Wq, scale, out, M, N, K, s);
    }
}

extern "C" int w8a16_gemv(const void* A, const void* Wq, const void* scale, void* out,
                          int64_t M, int64_t N, int64_t K, void* stream) {
    return w8a16_gemv_ex(A, Wq, scale, W8A16_SCALE_BLOCK_BF16, out, M, N, K, stream);
}

extern "C" int w8a16_gemv_fused(const void* A, const void* gate, int64_t ld_gate, const void* norm_weight, float eps,
                                int64_t group, const void* Wq, const void* scale, const void* residual, void* out,
                                int64_t M, int64_t N, int64_t K, void* stream) {
    using namespace w8a16;
    bool noop = false;
    int st = check_product_args(A, Wq, scale, out, M, N, K, &noop);
    if (st != W8A16_OK) return st;
    if (gate && !norm_weight) return W8A16_ERR_ARG;            // a gate belongs to the norm
    if (gate && (ld_gate < K || ld_gate % 8 != 0 || ld_gate > INT32_MAX)) return W8A16_ERR_SHAPE;
    if (norm_weight && (!(eps >= 0.0f) || eps > 3.0e38f)) return W8A16_ERR_ARG;   // also NaN
    if (norm_weight && !norm_group_valid(group, K)) return W8A16_ERR_SHAPE;
    if (noop) return W8A16_OK;
    if (!fused_fits(M, K)) return W8A16_ERR_SHAPE;
    if (norm_weight && (!aligned(norm_weight, 16) || (gate && !aligned(gate, 16)))) return W8A16_ERR_ALIGN;
    const int64_t out_bytes = M * N * 2;
    if (residual) {
        if (!aligned(residual, 2)) return W8A16_ERR_ALIGN;
        if (overlaps(out, out_bytes, residual, out_bytes)) return W8A16_ERR_ALIAS;
    }
    if ((norm_weight && overlaps(out, out_bytes, norm_weight, K * 2)) ||
        (gate && overlaps(out, out_bytes, gate, ((M - 1) * ld_gate + K) * 2)))
        return W8A16_ERR_ALIAS;
    Fusion fu{};
    fu.gate = static_cast<const uint16_t*>(gate);
    fu.weight = static_cast<const uint16_t*>(norm_weight);
    fu.residual = static_cast<const uint16_t*>(residual);
    fu.ld_gate = gate ? ld_gate : K;
    fu.eps = eps;
    fu.group = static_cast<int>(group == 0 ? K : group);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (gate) return run_gemv<kScaleBlockBf16, kFuseGated>(A, Wq, scale, out, M, N, K, s, fu);
    if (norm_weight) return run_gemv<kScaleBlockBf16, kFuseNorm>(A, Wq, scale, out, M, N, K, s, fu);
    return run_gemv<kScaleBlockBf16, kFuseResidual>(A, Wq, scale, out, M, N, K, s, fu);
}

extern "C" int w8a16_gemv_in_proj(const void* A, const void* norm_weight, float eps, const void* Wq, const void* scale,
                                  void* conv_state, const void* conv_weight, const void* conv_bias,
                                  int64_t conv_begin, int64_t conv_dim, int64_t d_conv, void* out,
                                  int64_t M, int64_t N, int64_t K, void* stream) {
    using namespace w8a16;
    bool noop = false;
    int st = check_product_args(A, Wq, scale, out, M, N, K, &noop);
    if (st != W8A16_OK) return st;
    if (!(eps >= 0.0f) || eps > 3.0e38f) return W8A16_ERR_ARG;   // also NaN
    if (conv_begin < 0 || conv_dim < 1 || conv_begin + conv_dim > N || d_conv < 1 || d_conv > kMaxConvTaps)
        return W8A16_ERR_SHAPE;
    if (noop) return W8A16_OK;
    if (!fused_fits(M, K)) return W8A16_ERR_SHAPE;
    if (!norm_weight || !conv_state || !conv_weight || !conv_bias) return W8A16_ERR_NULL;
    if (!aligned(norm_weight, 16) || !aligned(conv_state, 4) || !aligned(conv_weight, 2) || !aligned(conv_bias, 2))
        return W8A16_ERR_ALIGN;
    const int64_t out_bytes = M * N * 2, sb = M * conv_dim * d_conv * 4, wb = conv_dim * d_conv * 2;
    const void* reads[] = {A, Wq, scale, norm_weight, conv_weight, conv_bias};
    const int64_t read_bytes[] = {M * K * 2, N * K, scale_bytes(W8A16_SCALE_BLOCK_BF16, N, K), K * 2, wb, conv_dim * 2};
    if (overlaps(out, out_bytes, norm_weight, K * 2) || overlaps(out, out_bytes, conv_state, sb) ||
        overlaps(out, out_bytes, conv_weight, wb) || overlaps(out, out_bytes, conv_bias, conv_dim * 2))
        return W8A16_ERR_ALIAS;
    for (int i = 0; i < 6; ++i)
        if (overlaps(conv_state, sb, reads[i], read_bytes[i])) return W8A16_ERR_ALIAS;
    Fusion fu{};
    fu.weight = static_cast<const uint16_t*>(norm_weight);
    fu.ld_gate = K;
    fu.eps = eps;
    fu.conv_state = static_cast<float*>(conv_state);
    fu.conv_weight = static_cast<const uint16_t*>(conv_weight);
    fu.conv_bias = static_cast<const uint16_t*>(conv_bias);
    fu.conv_begin = static_cast<int>(conv_begin);
    fu.conv_dim = static_cast<int>(conv_dim);
    fu.d_conv = static_cast<int>(d_conv);
    return run_gemv<kScaleBlockBf16, kFuseNormConv>(A, Wq, scale, out, M, N, K, static_cast<hipStream_t>(stream), fu);
}
