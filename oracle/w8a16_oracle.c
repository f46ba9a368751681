/*
 * CPU oracle for the w8a16 block-scaled FP8 projection.
 *
 * TEST INFRASTRUCTURE ONLY. This file is a plain, slow, fp64 statement of what
 * the projection computes. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it. The GPU library shares no code,
 * header, table or helper with it, and nothing here calls the GPU.
 *
 * The operation (Qwen3SsmLayer docs, `set_fp8_decode_weights`: the w8a16 GEMV
 * formula; NemotronMamba2Layer docs, `set_fp8_weights`: the block-scale index):
 *
 *     out[m][n] = sum over k of  A[m][k] * E4M3(W[n][k]) * S[n / 128][k / 128]
 *
 *   A  : BF16 bit patterns, [M][K] row-major.
 *   W  : E4M3 bytes, [N][K] row-major (K contiguous).
 *   S  : BF16 bit patterns, [ceil(N/128)][ceil(K/128)] row-major, so the scale
 *        of element (n, k) sits at index (n / 128) * ceil(K/128) + (k / 128).
 *
 * Every product here is exact in fp64: a BF16 value has 8 significant bits,
 * an E4M3 value 4 and a BF16 scale 8, so A * E4M3 * S has at most 20 (at
 * most 36 with an FP32 scale). The sum runs over k in ascending order in
 * fp64. `den` is the same sum of absolute values; it scales the parity
 * tolerance.
 *
 * Scale formats (the `_fmt` functions; the others take format 0):
 *   0  BF16 block grid, as above;
 *   1  FP32 block grid, same shape and index (nemotron_mamba2.rs listing,
 *      `set_fp8_weights`: its format check names FP32 block scales);
 *   2  FP32 per-row scale R[n], [N] (Qwen3SsmLayer docs,
 *      `set_fp8_rowwise_prefill_weights`: per-row FP8 weights). The
 *      dequantized weight is then E4M3(W[n][k]) * R[n] for every k.
 *
 * Parity pins (the tests that tie this file to something other than itself):
 * E4M3 decode against the OCP 8-bit floating-point specification's special
 * values and against torch's float8_e4m3fn; BF16 decode against torch's
 * bfloat16 on all 65536 patterns; BF16 rounding against exact rational
 * rounding; the contraction against exact rational (fractions.Fraction) sums
 * on tiny shapes, against a library fp64 matmul, and against the invariants
 * of a bilinear block-scaled product (one-hot rows, zero weights, scale
 * doubling, sign and power-of-two scaling, row permutation).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

#define ORACLE_BLOCK 128

/*
 * E4M3 (OCP "OFP8" E4M3, the FN variant: bias 7, no infinities, NaN only at
 * S.1111.111). The pages call the weights E4M3 with a 448 maximum; this is
 * the closed form of that encoding, with no lookup table:
 *   exponent field 0  : (-1)^s * m * 2^-9            (subnormals, and +-0)
 *   exponent 15, m = 7: NaN
 *   otherwise         : (-1)^s * (1 + m/8) * 2^(E - 7)
 */
double oracle_e4m3_value(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* BF16 is the upper half of an IEEE binary32; widening it is exact. */
double oracle_bf16_value(uint16_t bits)
{
    union { uint32_t u; float f; } v;
    v.u = (uint32_t)bits << 16;
    return (double)v.f;
}

/*
 * Round a real (given exactly as a double) to BF16, round-to-nearest with
 * ties to even, directly from the double (no intermediate float, so there is
 * no double rounding). BF16: 8 significant bits, exponent range of binary32,
 * subnormal quantum 2^-133. Overflow past the largest finite value rounds to
 * infinity as in IEEE 754.
 */
uint16_t oracle_bf16_rne(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs(x);
    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0u);
    if (isinf(x))
        return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);               /* a = f * 2^e, f in [0.5, 1) -> unbiased exponent e-1 */
    int ue = e - 1;
    if (ue < -126)
        ue = -126;              /* subnormal range: fixed quantum */
    double quantum = ldexp(1.0, ue - 7);
    double q = nearbyint(a / quantum); /* exact division by a power of two; ties-to-even */
    double r = q * quantum;
    /* r has at most 9 significant bits only when q == 256 (carry), which is
     * still exactly representable in BF16 as the next binade's 1.0. */
    if (r >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80u);
    union { uint32_t u; float f; } v;
    v.f = (float)r;             /* exact: r is representable in binary32 */
    return (uint16_t)(sign | ((v.u >> 16) & 0x7FFFu));
}

static int64_t ceil_blocks(int64_t n) { return (n + ORACLE_BLOCK - 1) / ORACLE_BLOCK; }

/* The scale that multiplies E4M3(W[n][k]) in format fmt (exact in fp64). */
static double scale_of(const void* S, int fmt, int64_t K, int64_t n, int64_t k)
{
    int64_t idx = (n / ORACLE_BLOCK) * ceil_blocks(K) + (k / ORACLE_BLOCK);
    if (fmt == 0)
        return oracle_bf16_value(((const uint16_t*)S)[idx]);
    if (fmt == 1)
        return (double)((const float*)S)[idx];
    return (double)((const float*)S)[n];
}

/* Dequantized weight as a real: E4M3(W[n][k]) times its scale. */
static double wdeq(const uint8_t* W, const void* S, int fmt, int64_t K, int64_t n, int64_t k)
{
    return oracle_e4m3_value(W[n * K + k]) * scale_of(S, fmt, K, n, k);
}

/* out[n*K + k] = Wdeq[n][k], exact, [N][K] fp64. */
void oracle_dequant_fmt(const uint8_t* W, const void* S, int fmt, int64_t N, int64_t K, double* out)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            out[n * K + k] = wdeq(W, S, fmt, K, n, k);
}

void oracle_dequant(const uint8_t* W, const uint16_t* S, int64_t N, int64_t K, double* out)
{
    oracle_dequant_fmt(W, S, 0, N, K, out);
}

/* One output element: ref = sum_k A[m][k]*Wdeq[n][k] (k ascending), den = sum |.|. */
static void dot_one(const uint16_t* A, const uint8_t* W, const void* S, int fmt,
                    int64_t K, int64_t m, int64_t n, double* ref, double* den)
{
    double acc = 0.0, mag = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double t = oracle_bf16_value(A[m * K + k]) * wdeq(W, S, fmt, K, n, k);
        acc += t;
        mag += fabs(t);
    }
    *ref = acc;
    *den = mag;
}

/* Every element of the [M][N] result. Elements are independent; the threads
 * split the (m, n) pairs and never reorder a sum. */
void oracle_w8a16_fmt(const uint16_t* A, const uint8_t* W, const void* S, int fmt,
                      int64_t M, int64_t N, int64_t K, double* ref, double* den)
{
    int64_t total = M * N;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < total; ++i) {
        int64_t m = i / N, n = i % N;
        dot_one(A, W, S, fmt, K, m, n, &ref[i], &den[i]);
    }
}

void oracle_w8a16(const uint16_t* A, const uint8_t* W, const uint16_t* S,
                  int64_t M, int64_t N, int64_t K, double* ref, double* den)
{
    oracle_w8a16_fmt(A, W, S, 0, M, N, K, ref, den);
}

/* Selected elements (mi[p], ni[p]) of the result, for shapes too large to
 * compute whole. */
void oracle_w8a16_points_fmt(const uint16_t* A, const uint8_t* W, const void* S, int fmt,
                             int64_t M, int64_t N, int64_t K,
                             const int64_t* mi, const int64_t* ni, int64_t npts,
                             double* ref, double* den)
{
    (void)M; (void)N;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t p = 0; p < npts; ++p)
        dot_one(A, W, S, fmt, K, mi[p], ni[p], &ref[p], &den[p]);
}

void oracle_w8a16_points(const uint16_t* A, const uint8_t* W, const uint16_t* S,
                         int64_t M, int64_t N, int64_t K,
                         const int64_t* mi, const int64_t* ni, int64_t npts,
                         double* ref, double* den)
{
    oracle_w8a16_points_fmt(A, W, S, 0, M, N, K, mi, ni, npts, ref, den);
}

/*
 * Norm prologues and the residual epilogue around the projection (the
 * Mamba-2 layer's forward steps in the nemotron_mamba2.rs module docs: step 1,
 * RMS norm scaled by its weight, before in_proj; step 6, the gated norm
 * rms_norm(y, ssm_norm) * silu(z), before out_proj; step 8, the residual add
 * after out_proj). The pages give neither epsilon nor the norm's grouping, so
 * both are arguments: the norm runs over consecutive groups of `group`
 * channels of each row (group = K: one norm over the whole row, the plain
 * reading of rms_norm(y, ssm_norm); group = K / n_groups: the published
 * Mamba-2 gated norm, one norm per group of channels). For channel k in
 * group g = k / group:
 *
 *   r_g      = 1 / sqrt( (sum_{k' in g} x[k']^2) / group + eps )
 *   v[k]     = x[k] * r_g * weight[k]                  (RMSNorm)
 *   v[k]     = x[k] * r_g * weight[k] * silu(z[k])     (gated RMSNorm)
 *   silu(z)  = z / (1 + exp(-z))
 *
 * computed in fp64; `exact` receives v and `bits` its BF16 rounding (the
 * activation the projection then reads). group must divide K.
 */
double oracle_silu(double z)
{
    return z / (1.0 + exp(-z));
}

void oracle_rmsnorm(const uint16_t* x, const uint16_t* gate, const uint16_t* weight, double eps,
                    int64_t group, int64_t M, int64_t K, double* exact, uint16_t* bits)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t g0 = 0; g0 < K; g0 += group) {
            double ss = 0.0;
            for (int64_t k = g0; k < g0 + group; ++k) {
                double v = oracle_bf16_value(x[m * K + k]);
                ss += v * v;
            }
            double r = 1.0 / sqrt(ss / (double)group + eps);
            for (int64_t k = g0; k < g0 + group; ++k) {
                double v = oracle_bf16_value(x[m * K + k]) * r * oracle_bf16_value(weight[k]);
                if (gate)
                    v *= oracle_silu(oracle_bf16_value(gate[m * K + k]));
                exact[m * K + k] = v;
                bits[m * K + k] = oracle_bf16_rne(v);
            }
        }
    }
}

/*
 * Residual epilogue: the projection's output is a BF16 tensor, and the
 * residual add sums two BF16 tensors into a BF16 one:
 *   out[i] = bf16( residual[i] + bf16(ref[i]) ).
 */
void oracle_residual_add(const uint16_t* residual, const double* ref, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) {
        double y = oracle_bf16_value(oracle_bf16_rne(ref[i]));
        out[i] = oracle_bf16_rne(oracle_bf16_value(residual[i]) + y);
    }
}

/*
 * The Mamba-2 decode step between the two projections (nemotron_mamba2.rs
 * module docs, forward steps 3 to 5: the conv1d update on xBC with bias and
 * fused SiLU, the split into x, B and C, the SSM state update and output; the
 * argument lists of `conv1d_update_biased` and `ssm_decode` in that listing).
 * The pages do not write the formulas out; these are the standard Mamba-2
 * recurrence for one token (the reading is stated in the design notes).
 *
 * Conv1d update, for each sequence b and channel c, with a state of the last
 * d_conv inputs (oldest first):
 *   state[c][w] <- state[c][w + 1] (w < d_conv - 1), state[c][d_conv-1] <- x[c]
 *   out[c] = silu( sum_w state[c][w] * weight[c][w] + bias[c] )
 */
void oracle_conv1d_update(double* state, const uint16_t* x, int64_t ld_x, const uint16_t* weight,
                          const uint16_t* bias, int64_t B, int64_t dim, int64_t d_conv,
                          double* out_exact, uint16_t* out_bits)
{
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = 0; c < dim; ++c) {
            double* s = state + (b * dim + c) * d_conv;
            for (int64_t w = 0; w + 1 < d_conv; ++w)
                s[w] = s[w + 1];
            s[d_conv - 1] = oracle_bf16_value(x[b * ld_x + c]);
            double acc = oracle_bf16_value(bias[c]);
            for (int64_t w = 0; w < d_conv; ++w)
                acc += s[w] * oracle_bf16_value(weight[c * d_conv + w]);
            double v = oracle_silu(acc);
            out_exact[b * dim + c] = v;
            out_bits[b * dim + c] = oracle_bf16_rne(v);
        }
}

/* softplus(v) = log(1 + e^v). */
double oracle_softplus(double v)
{
    return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v));
}

/*
 * SSM decode, for each sequence b and head h (group g = h / (heads / groups)),
 * with the conv output row xbc = [x (heads * head_dim) | B (groups * state) |
 * C (groups * state)] and the state h[b][h][p][n]:
 *   dt   = clamp( softplus(dt_raw[h] + dt_bias[h]), dt_min, dt_max )
 *   a    = -exp(a_log[h]),  dA = exp(dt * a)
 *   h[p][n] <- dA * h[p][n] + dt * B[g][n] * x[h][p]
 *   y[h][p] = sum_n C[g][n] * h[p][n] + D[h] * x[h][p]
 * y_den receives sum_n |C[g][n] * h[p][n]| + |D[h] * x[h][p]| (for the parity
 * tolerance).
 */
void oracle_ssm_decode(double* hs, const uint16_t* xbc, int64_t ld_xbc, const uint16_t* dt_raw,
                       int64_t ld_dt, const float* a_log, const float* d_param, const float* dt_bias,
                       int64_t B, int64_t heads, int64_t head_dim, int64_t st, int64_t groups,
                       double dt_min, double dt_max, double* y_exact, uint16_t* y_bits, double* y_den)
{
    int64_t d_inner = heads * head_dim, per_group = heads / groups;
    for (int64_t b = 0; b < B; ++b) {
        const uint16_t* row = xbc + b * ld_xbc;
        for (int64_t h = 0; h < heads; ++h) {
            int64_t g = h / per_group;
            double dt = oracle_softplus(oracle_bf16_value(dt_raw[b * ld_dt + h]) + (double)dt_bias[h]);
            if (dt < dt_min) dt = dt_min;
            if (dt > dt_max) dt = dt_max;
            double dA = exp(dt * -exp((double)a_log[h]));
            const uint16_t* Bg = row + d_inner + g * st;
            const uint16_t* Cg = row + d_inner + groups * st + g * st;
            for (int64_t p = 0; p < head_dim; ++p) {
                double xv = oracle_bf16_value(row[h * head_dim + p]);
                double* hp = hs + ((b * heads + h) * head_dim + p) * st;
                double y = 0.0, den = 0.0;
                for (int64_t n = 0; n < st; ++n) {
                    hp[n] = dA * hp[n] + dt * oracle_bf16_value(Bg[n]) * xv;
                    double t = oracle_bf16_value(Cg[n]) * hp[n];
                    y += t;
                    den += fabs(t);
                }
                double skip = (double)d_param[h] * xv;
                y += skip;
                den += fabs(skip);
                int64_t o = b * d_inner + h * head_dim + p;
                y_exact[o] = y;
                y_bits[o] = oracle_bf16_rne(y);
                y_den[o] = den;
            }
        }
    }
}

/* Element-wise array forms of the scalar conversions above. */
void oracle_e4m3_values(const uint8_t* codes, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3_value(codes[i]);
}

void oracle_bf16_values(const uint16_t* bits, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_value(bits[i]);
}

void oracle_bf16_rne_array(const double* x, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_rne(x[i]);
}

/* Threads the parallel loops above would use (for reporting). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
