/*
 * w8a16.h - C ABI of the MI355X (gfx950) w8a16 block-scaled FP8 projection.
 *
 * The operation (Qwen3SsmLayer docs, `set_fp8_decode_weights`, which gives the
 * w8a16 GEMV formula and the BF16 [N/BS, K/BS] scale buffer; NemotronMamba2Layer
 * docs, `set_fp8_weights`, which gives the 128-wide block index and the
 * [ceil(N/128), ceil(K/128)] grid):
 *
 *     out[m][n] = sum_k A[m][k] * E4M3(Wq[n][k]) * scale[n/128][k/128]
 *
 * Operands (all DEVICE pointers, row-major, no padding between rows):
 *   A      BF16  [M][K]                          activations (row stride K)
 *   Wq     E4M3  [N][K]  (one byte per value)    weights, K contiguous
 *   scale  BF16  [ceil(N/128)][ceil(K/128)]      block scales; element (n, k)
 *                                                uses scale[(n/128)*ceil(K/128) + k/128]
 *   out    BF16  [M][N]                          result (row stride N)
 * E4M3 is the OCP FP8 E4M3 ("FN") encoding: bias 7, largest finite 448, NaN
 * at 0x7F/0xFF (a NaN code propagates to the outputs it touches). Partial
 * edge blocks (N or K not multiples of 128) use their block's scale.
 * Accumulation is fp32; each output is rounded once to BF16 (nearest, ties
 * to even). The scale must be exactly the [ceil(N/128)][ceil(K/128)] BF16 grid:
 * the library cannot see allocation sizes, so a per-row [N] or scalar scale
 * buffer reads past its end (a device fault, not wrong numbers) - callers
 * must check the layout before calling, as the Python binding does.
 *
 * Ownership: the caller owns every buffer it passes; the library keeps no
 * pointer to them after a call returns, and allocates no device memory of its
 * own (no entry point calls hipMalloc). The decode-step entry points
 * (w8a16_conv1d_update, w8a16_ssm_decode) update the caller's state buffers in
 * place; every other entry point only writes `out`.
 * Streams: `stream` is a hipStream_t (NULL = the legacy default stream). Every
 * call only enqueues work on it and returns without synchronizing; the result
 * is ready once the stream reaches that point.
 * Errors: every argument is checked on the host BEFORE anything is enqueued;
 * a failed check returns a negative W8A16_ERR_* code and launches nothing.
 * W8A16_ERR_LAUNCH reports a HIP launch failure. The result is deterministic:
 * the same inputs give the same bits on every call.
 */
#ifndef W8A16_H
#define W8A16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum w8a16_status {
    W8A16_OK = 0,
    W8A16_ERR_NULL = -1,   /* a required pointer is NULL                        */
    W8A16_ERR_SHAPE = -2,  /* M, N or K out of range, or K not a multiple of 16 */
    W8A16_ERR_ALIGN = -3,  /* A or Wq not 16-byte aligned; scale/out not 2-byte */
    W8A16_ERR_LAUNCH = -4, /* the HIP launch failed                             */
    W8A16_ERR_ALIAS = -5,  /* out overlaps an input                             */
    W8A16_ERR_ARG = -6,    /* another argument is invalid                       */
    W8A16_ERR_WORKSPACE = -7, /* w8a16_gemm_ws: the workspace is too small        */
    W8A16_ERR_SCRATCH = -8  /* w8a16_gemm_noalloc: the shape needs more scratch
                               than w8a16_gemm_noalloc_scratch_bytes()          */
};

/*
 * Scale formats of the _ex entry points. w8a16_gemv and w8a16_gemm (below)
 * take the first; the others are the variants the pages name besides it:
 *  - W8A16_SCALE_BLOCK_BF16: BF16 [ceil(N/128)][ceil(K/128)] (the grid above);
 *  - W8A16_SCALE_BLOCK_F32: FP32, same grid and index (nemotron_mamba2.rs
 *    source listing, `set_fp8_weights`: its format check names FP32 block
 *    scales of that shape);
 *  - W8A16_SCALE_ROW_F32: FP32 [N], one scale per weight row:
 *    out[m][n] = sum_k A[m][k] * E4M3(Wq[n][k]) * scale[n] (Qwen3SsmLayer
 *    docs, `set_fp8_rowwise_prefill_weights`: per-row FP8 weights, a layout
 *    that must not reach a block-scaled kernel, since a mismatched buffer is
 *    read in bounds and gives wrong numbers).
 * The library cannot tell the formats apart from the pointer: the caller
 * passes the format that matches the buffer (the Python binding checks the
 * tensor's dtype and shape against it).
 */
enum w8a16_scale_format {
    W8A16_SCALE_BLOCK_BF16 = 0,
    W8A16_SCALE_BLOCK_F32 = 1,
    W8A16_SCALE_ROW_F32 = 2
};

/* Largest M the GEMV entry point accepts, and its largest K: 16384 when
 * M <= 8, 8192 otherwise (w8a16_gemm takes any M and K). */
#define W8A16_GEMV_MAX_M 16
#define W8A16_GEMV_MAX_K_SMALL_M 16384
#define W8A16_GEMV_MAX_K 8192

/*
 * Decode GEMV: one or a few tokens (TransformerLayer docs, `decode`: a
 * [1, hidden] BF16 row per token; `decode_multi_seq`: N sequences with the
 * weights read once for all of them). 1 <= M <= 16, N >= 0, K % 16 == 0,
 * 16 <= K <= 16384 for M <= 8 and 16 <= K <= 8192 for M >= 9.
 * M == 0 or N == 0 is a no-op returning W8A16_OK.
 * Each weight byte is read from HBM once per call for all M rows. M = 1
 * runs a GEMV on the vector ALU (dot products over 16-byte weight chunks,
 * reduced across the wavefront and the workgroup in a fixed order), and so
 * do M = 2..4 when K <= 8192 and the weights make at least 8 four-row groups
 * per compute unit (N >= 8192 on 256 CUs). Otherwise, from M = 2 on, where
 * the skinny path of w8a16_gemm applies (below), the call runs it (products
 * on the matrix cores; same result contract).
 */
int w8a16_gemv(const void* A, const void* Wq, const void* scale, void* out,
               int64_t M, int64_t N, int64_t K, void* stream);

/*
 * Prefill GEMM: M prompt tokens at once (TransformerLayer docs, `prefill`:
 * the weights are read once for all N tokens as one GEMM with M = N), and
 * the skinny case of a few tokens (speculative verify, batched decode).
 * M >= 0 (any), N >= 0, 16 <= K < 2^23, K % 16 == 0; M == 0 or N == 0 is a
 * no-op. Paths, chosen by M, N, K and the device's CU count only:
 *  - mid-size, 17 <= M <= 256 with K <= 32768 (one kernel, no workspace):
 *    one workgroup per output tile of 16 to 128 rows by 32 to 160 columns,
 *    the tile chosen so that the tiles about fill the CUs; its rows of A and
 *    its weight bytes stream into LDS, the waves split each stage's k and
 *    add their fp32 partial tiles in LDS in a fixed order, and the block
 *    scale multiplies each wave's fp32 partial sum over its part of a
 *    128-wide k-block;
 *  - skinny, M <= 16 (one kernel, no workspace; the weights stream from HBM
 *    straight into the matrix-core operands, each 16-row weight block read
 *    once for all M rows): K <= 8192 where one workgroup per 16-row block
 *    fits (the activations, in LDS, copied in up to 8 parts of K); else
 *    K <= 4096, or 12 <= M <= 16 with K <= 8192, with workgroups walking
 *    several blocks;
 *  - otherwise, M >= 65 where 256 x 256 output tiles fill every round of
 *    CU-many tiles to at least 85 % (e.g. the 8192-token prefill): one
 *    workgroup per CU walks those tiles; each weight is converted once per
 *    tile as bf16(e * s), the block scale folded in (e * s is exact in fp32,
 *    rounded once), and the matrix cores accumulate over the whole K range;
 *    where they cover at least one whole round but leave a sparse one (the
 *    1024-token in_proj), whole rounds of them take the first columns and
 *    the tiles below the rest;
 *  - otherwise output tiles of 32 (M <= 32), 64 (M <= 64; these two only
 *    for K past the mid-size kernel's) or 128 rows by 128 columns: the E4M3
 *    weight bytes of a tile are staged once per workgroup and decoded in
 *    registers, and the block scale multiplies each 128-wide k-block's fp32
 *    partial sum. 128-row tiles numbering between three quarters of the
 *    CUs and the CUs split their k-range between two halves of one
 *    workgroup, added in LDS. Every tile is computed whole by one
 *    workgroup: w8a16_gemm needs no workspace and allocates nothing (it may
 *    be captured in a HIP graph on any stream).
 * Every choice depends only on M, N, K and the device's compute-unit count,
 * so the bits are the same on every call.
 */
int w8a16_gemm(const void* A, const void* Wq, const void* scale, void* out,
               int64_t M, int64_t N, int64_t K, void* stream);

/*
 * The GEMV and the GEMM with the scale buffer in `scale_format` (an
 * enum w8a16_scale_format value; anything else returns W8A16_ERR_ARG).
 * Shapes, streams, paths and errors are those of w8a16_gemv / w8a16_gemm;
 * FP32 scales must be 4-byte aligned. Block scales are applied in fp32 to
 * each 128-wide k-block's partial sum; a row scale multiplies the finished
 * fp32 row sum once, before the BF16 rounding.
 * w8a16_gemv(...) is w8a16_gemv_ex(..., W8A16_SCALE_BLOCK_BF16, ...), and
 * likewise for the GEMM.
 */
int w8a16_gemv_ex(const void* A, const void* Wq, const void* scale, int scale_format, void* out,
                  int64_t M, int64_t N, int64_t K, void* stream);
int w8a16_gemm_ex(const void* A, const void* Wq, const void* scale, int scale_format, void* out,
                  int64_t M, int64_t N, int64_t K, void* stream);

/*
 * The GEMM with a caller-supplied workspace, for shapes whose 32-, 64- or
 * 128-row tiles do not fill the GPU (fewer tiles than it holds at once, or a
 * last wave less than a quarter full; e.g. a few hundred tokens against
 * weights with few rows, or a few dozen tokens with K past 32768): the
 * k-blocks of the remaining tiles are then split between workgroups, whose
 * fp32 partial tiles go to the workspace, and a second kernel enqueued on the
 * same stream adds them in k order (deterministic: the split depends only on
 * M, N, K and the CU count). Same operands, shapes, paths and result
 * contract as w8a16_gemm (BF16 block grid).
 * w8a16_gemm_workspace_size returns the bytes this needs for (M, N, K) on the
 * current device (0: the shape does not split), or W8A16_ERR_SHAPE for an
 * invalid shape.
 * workspace: device memory of workspace_bytes bytes, 256-byte aligned
 * (W8A16_ERR_ALIGN), not overlapping an operand (W8A16_ERR_ALIAS), at least
 * w8a16_gemm_workspace_size(M, N, K) bytes (else W8A16_ERR_WORKSPACE;
 * nothing is launched). NULL runs w8a16_gemm. The call owns the workspace
 * from enqueue until the stream passes the call: calls that may run at the
 * same time need separate workspaces.
 */
int64_t w8a16_gemm_workspace_size(int64_t M, int64_t N, int64_t K);
int w8a16_gemm_ws(const void* A, const void* Wq, const void* scale, void* out, int64_t M, int64_t N, int64_t K,
                  void* workspace, int64_t workspace_bytes, void* stream);

/*
 * The GEMM for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc) and
 * still want w8a16_gemm_ws's split schedule: the same kernels and the same
 * result, bit for bit, as w8a16_gemm_ws with a large enough workspace, but
 * the partial tiles go to a scratch array that the library holds in device
 * memory, w8a16_gemm_noalloc_scratch_bytes() bytes (64 MiB) per GPU, from
 * the first call on a GPU until the process ends. Nothing is allocated per
 * call. A shape whose schedule needs more scratch than that (none on a
 * 256-CU MI355X; w8a16_gemm_workspace_size reports the need) returns
 * W8A16_ERR_SCRATCH and launches nothing. Operands, shapes, alignment,
 * aliasing and the other errors are those of w8a16_gemm; W8A16_ERR_LAUNCH
 * also reports a failed lookup of the scratch array's device address.
 * Every call on one GPU shares that GPU's scratch: calls that may run at the
 * same time on one GPU (two streams, two host threads) race and must be
 * serialised by the caller. The scratch keeps the last call's partial tiles;
 * no call needs it cleared.
 */
int64_t w8a16_gemm_noalloc_scratch_bytes(void);
int w8a16_gemm_noalloc(const void* A, const void* Wq, const void* scale, void* out, int64_t M, int64_t N, int64_t K,
                       void* stream);

/*
 * Measurement helper, not a step of the projection: reads bytes of device
 * memory at buf once (16-byte loads, non-temporal like the decode GEMV's
 * weight loads), loads_per_lane loads per lane all issued before any is used,
 * in workgroups of `threads` threads. Its time is the plain-read floor that
 * the decode GEMV's weight stream (one read of N*K bytes) is compared against.
 * Writes nothing: sink (4-byte aligned, at least `threads` words) is only
 * named so that the loads are kept.
 * bytes: a multiple of 16, at most 2^31 (else W8A16_ERR_SHAPE; 0 is a no-op);
 * threads in {64, 128, 256, 512, 1024} and loads_per_lane in {1, 2, 4, 8, 16}
 * (else W8A16_ERR_ARG); buf 16-byte aligned (W8A16_ERR_ALIGN).
 */
int w8a16_hbm_read(const void* buf, int64_t bytes, int threads, int loads_per_lane, void* sink, void* stream);

/*
 * Norm prologues and the residual epilogue of the Mamba-2 layer around its
 * two projections (nemotron_mamba2.rs module docs, forward pass: step 1, RMS
 * norm scaled by its weight, before in_proj; step 6, the gated norm
 * rms_norm(y, ssm_norm) * silu(z), before out_proj; step 8, the residual add
 * after out_proj). The pages give neither epsilon nor a grouping of the
 * norm, so both are arguments: eps (finite, >= 0; anything else returns
 * W8A16_ERR_ARG) and group, the channels normalized together: 0 or K for
 * one norm over each whole row (the plain reading of rms_norm(y, ssm_norm)),
 * or a multiple of 1024 that divides K, with K <= 16384 (the published
 * Mamba-2 gated norm: group = K / n_groups); anything else returns
 * W8A16_ERR_SHAPE. For channel k in group g = k / group:
 *
 *   r[m][g] = 1 / sqrt( (sum_{k' in g} x[m][k']^2) / group + eps )
 *   a[m][k] = bf16( x[m][k] * r[m][g] * weight[k] [* silu(gate[m][k])] )
 *   silu(z) = z / (1 + e^-z)
 *
 * computed in fp32 with one rounding to BF16 at the end. The residual add
 * sums two BF16 tensors: out = bf16(residual + bf16(product)).
 *
 * w8a16_rmsnorm: a into out, all [M][K] BF16 (x, gate, out 16-byte aligned;
 * weight [K] BF16, 16-byte aligned; gate may be NULL for the plain norm). M
 * >= 0, K % 16 == 0, K >= 16. The prefill path: the GEMM then reads `out`.
 * out must not overlap an input (W8A16_ERR_ALIAS).
 */
int w8a16_rmsnorm(const void* x, const void* gate, const void* weight, float eps, int64_t group, void* out,
                  int64_t M, int64_t K, void* stream);

/*
 * Decode GEMV with the prologue and epilogue fused (one launch per
 * projection): A is the layer input x (in_proj, norm_weight set, gate NULL)
 * or the SSM output y (out_proj, gate = z); norm_weight NULL means no norm
 * (then gate must be NULL too, else W8A16_ERR_ARG); eps and group as for
 * w8a16_rmsnorm (group ignored without a norm). The gate's rows (K BF16
 * each) lie ld_gate elements apart, so z can be read in place from the
 * in_proj output row [z | xBC | dt] (ld_gate >= K, ld_gate % 8 == 0, gate
 * 16-byte aligned; ignored without a gate). residual ([M][N] BF16,
 * 2-byte aligned, or NULL) adds the epilogue; it must not overlap out.
 * The scale is the BF16 block grid; errors as for w8a16_gemv. Shapes: 1 <= M
 * <= 4 with K <= 16384, or 5 <= M <= 8 with K <= 8192 (the norm's operands
 * then fit in registers beside the activations); otherwise W8A16_ERR_SHAPE,
 * and the two-step form w8a16_rmsnorm + w8a16_gemm_residual applies. Every
 * M runs the GEMV kernel (the skinny path of w8a16_gemv is not fused).
 */
int w8a16_gemv_fused(const void* A, const void* gate, int64_t ld_gate, const void* norm_weight, float eps,
                     int64_t group, const void* Wq, const void* scale, const void* residual, void* out,
                     int64_t M, int64_t N, int64_t K, void* stream);

/*
 * Prefill GEMM with the residual epilogue: out = bf16(residual +
 * bf16(A x dequant(Wq)^T)), residual [M][N] BF16, 2-byte aligned, not NULL,
 * not overlapping out. Everything else as for w8a16_gemm (BF16 block grid).
 */
int w8a16_gemm_residual(const void* A, const void* Wq, const void* scale, const void* residual,
                        void* out, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * The Mamba-2 decode step between the two projections (nemotron_mamba2.rs
 * module docs, forward steps 3 to 5; argument lists and launch shapes of
 * `conv1d_update_biased` and `ssm_decode` in that listing). The pages name
 * the steps but do not write the formulas; these are the standard Mamba-2
 * recurrence for one token. All calls enqueue on `stream`; batch == 0 is a
 * no-op; arrays must not overlap (W8A16_ERR_ALIAS) except as stated.
 *
 * w8a16_conv1d_update: for each sequence b < batch and channel c < dim,
 *   conv_state[b][c][0..d_conv)   FP32, the last d_conv inputs (oldest first),
 *                                 updated in place: shifted by one, x appended;
 *   out[b*ld_out + c] = bf16( silu( bias[c] + sum_w conv_state[b][c][w] * weight[c][w] ) )
 * x [batch][ld_x] BF16 (the xBC part of the in_proj output row, ld_x >= dim);
 * weight [dim][d_conv] and bias [dim] BF16; out [batch][ld_out] BF16.
 * 1 <= d_conv <= 8, batch <= 65535. conv_state 4-byte aligned, the rest 2.
 */
int w8a16_conv1d_update(void* conv_state, const void* x, int64_t ld_x, const void* weight, const void* bias,
                        void* out, int64_t ld_out, int64_t batch, int64_t dim, int64_t d_conv, void* stream);

/*
 * w8a16_gemv_in_proj: the in_proj of the decode step in one launch. The
 * RMSNorm prologue of w8a16_gemv_fused (norm_weight required, no gate, no
 * residual), the projection, and the conv1d update above applied to the
 * output columns [conv_begin, conv_begin + conv_dim) as they are stored: for
 * column n = conv_begin + c of row m, the channel c takes the projection's
 * BF16 output as its new input, conv_state[m][c] is updated in place and
 * out[m][n] receives the conv output. The other columns hold the projection
 * (z and dt of the row [z | xBC | dt]). The result is bit-identical to
 * w8a16_gemv_fused followed by w8a16_conv1d_update on those columns, one
 * launch fewer. Shapes as for w8a16_gemv_fused; conv_begin + conv_dim <= N,
 * 1 <= d_conv <= 8; conv_state 4-byte aligned, taps [conv_dim][d_conv] and
 * bias [conv_dim] BF16, 2-byte aligned; no buffer may overlap another.
 */
int w8a16_gemv_in_proj(const void* A, const void* norm_weight, float eps, const void* Wq, const void* scale,
                       void* conv_state, const void* conv_weight, const void* conv_bias, int64_t conv_begin,
                       int64_t conv_dim, int64_t d_conv, void* out, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * w8a16_ssm_decode: for each sequence b and head h (group g = h / (heads /
 * groups)), with the conv output row xbc[b] = [x (heads*head_dim) | B
 * (groups*state) | C (groups*state)] (BF16, ld_xbc >= its width) and
 * dt_raw[b][h] (BF16, the dt part of the in_proj output, ld_dt >= heads):
 *   dt = clamp( softplus(dt_raw + dt_bias[h]), dt_min, dt_max )
 *   dA = exp( -dt * exp(a_log[h]) )
 *   h_state[b][h][p][n] <- dA * h_state[b][h][p][n] + dt * B[g][n] * x[h*head_dim + p]
 *   out[b*ld_out + h*head_dim + p] = bf16( sum_n C[g][n] * h_state[b][h][p][n] + d_param[h] * x[...] )
 * h_state FP32 [batch][heads][head_dim][state], updated in place, 16-byte
 * aligned; a_log, d_param, dt_bias FP32 [heads]; out BF16. state % 4 == 0,
 * 4 <= state <= 256, heads % groups == 0, 0 <= dt_min <= dt_max (finite;
 * else W8A16_ERR_ARG). Computed in fp32; the sum over n is a fixed
 * butterfly (deterministic).
 */
int w8a16_ssm_decode(void* h_state, const void* xbc, int64_t ld_xbc, const void* dt_raw, int64_t ld_dt,
                     const float* a_log, const float* d_param, const float* dt_bias, void* out, int64_t ld_out,
                     int64_t batch, int64_t heads, int64_t head_dim, int64_t state, int64_t groups,
                     float dt_min, float dt_max, void* stream);

/*
 * Dequantize only (a test path that exposes the device E4M3 decode and the
 * block-scale indexing the two entry points above use). out is FP32 [N][K]:
 *   out[n][k] = float(E4M3(Wq[n][k])) * scale[n/128][k/128]
 * which is exact (a 4-bit by 8-bit significand product). Same shape rules
 * as above; Wq and out must be 16-byte aligned, scale 2-byte aligned.
 */
int w8a16_dequant(const void* Wq, const void* scale, float* out,
                  int64_t N, int64_t K, void* stream);

/* Static description of a status code; never NULL. */
const char* w8a16_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* W8A16_H */
