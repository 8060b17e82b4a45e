/*
 * oracle.c -- plain, slow, FP64 CPU reference for the weight-only INT4/INT2
 * quantised linear layer and the looped block that calls it.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this file's library.  The product path (the HIP
 * library under int2_quantized_gemm_amd/) never calls it, includes nothing from
 * it and shares no code with it; the two are compared element by element.
 *
 * Sources (TinyLoop documentation pages):
 *  - "Model" page, Parameters / VRAM cost: weights are INT2/INT4 packed codes
 *    plus FP16 scales and FP16 zeros per quantised layer; the residual stream
 *    buf.main is FP32 and the scratch buffers are FP16.
 *  - "β-Informed Deployment Features" page, CTX-TIER "Details of the shipped
 *    kernel": per-group asymmetric quantisation, groups of typically 128
 *    weights, INT2 scale = (max - min) / 3, four INT2 codes per byte, a row of
 *    codes is one output channel (INT4 row stride K/2 bytes, INT2 K/4 bytes);
 *    Phase 2b also meets per-row quantisation, one group spanning the whole
 *    row (group size = K).
 *  - "Warm-start mid-loop" page, internal flow: run_loop_iters_range applies
 *    iterations [L_used, new_L) in place on the residual; the shared block
 *    re-applies the same weights on every iteration.
 *
 * Where the pages are silent the readings below are used (each is listed in
 * the design notes):
 *  - zero point: integer z stored in FP16, dequant w^ = (q - z) * s;
 *  - range: lo = min(0, min W), hi = max(0, max W); s = fp16((hi-lo)/(2^b-1)),
 *    s := 1 when it rounds to 0; overflow of s is an error;
 *  - rounding: round-half-to-even everywhere (codes, z, FP16 conversions);
 *  - bit order: code j = k mod (32/b) of a uint32 word sits at bit
 *    16*(j mod 2) + b*floor(j/2): the even codes fill the low 16 bits and the
 *    odd codes the high 16 bits, each half from its least significant bit;
 *  - layout: codes [N][K*b/32] uint32, scales/zeros [N][K/G] FP16, N-major;
 *  - group size G: 128, or K for per-row groups (one scale and zero per
 *    output channel); K is a multiple of 128 either way;
 *  - glue between the projections: parameter-free LayerNorm (eps 1e-5,
 *    population variance), self-only attention (the V slice of qkv, columns
 *    [2D, 3D)), identity FFN activation (or SwiGLU when the block has a gate
 *    weight, see or_block); FP16 rounding at the LN outputs and at
 *    every GEMM output, FP64 residual.
 *
 * Parity unpinned against the pages: the glue readings above (LayerNorm,
 * self-only attention, identity FFN activation) and the integer zero-point
 * convention.  The pages print no values for them; the tests pin them only to
 * closed forms of these readings.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_EINVAL (-1)
#define OR_EUNSUPPORTED (-2)
#define OR_ENOMEM (-3)

/* ---------------------------------------------------------------- FP16 --- */

/* IEEE binary16 bits -> exact double value. */
double or_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);              /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);  /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* Nearest binary16 value to x (ties to even), returned as a double; values
 * that round beyond the largest finite half (65504) become +-inf.  Written from
 * the definition: the spacing of halves in [2^E, 2^(E+1)) is 2^(E-10) for
 * E >= -14, and 2^-24 below 2^-14 (subnormals). */
double or_round_half(double x)
{
    if (isnan(x) || x == 0.0 || isinf(x))
        return x;
    double a = fabs(x);
    int e2;
    frexp(a, &e2);          /* a = m * 2^e2, m in [0.5, 1) */
    int E = e2 - 1;         /* floor(log2(a)) */
    if (E < -14)
        E = -14;
    double quantum = ldexp(1.0, E - 10);
    double r = nearbyint(a / quantum) * quantum;   /* a/quantum is exact */
    if (r > 65504.0)
        r = INFINITY;
    return x < 0 ? -r : r;
}

/* Encode a double that is exactly a binary16 value (or +-inf) into its bits. */
uint16_t or_double_to_half_bits(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return 0x7e00;
    if (isinf(a))
        return sign | 0x7c00;
    if (a < ldexp(1.0, -14))
        return sign | (uint16_t)(a * ldexp(1.0, 24));
    int e2;
    frexp(a, &e2);
    int E = e2 - 1;
    uint16_t f = (uint16_t)(ldexp(a, 10 - E) - 1024.0);
    return sign | (uint16_t)((E + 15) << 10) | f;
}

/* Bit position of code j (0 <= j < 32/bits) inside its uint32 word. */
static int code_shift(int bits, int j)
{
    return 16 * (j & 1) + bits * (j >> 1);
}

/* ---------------------------------------------------------- validation --- */

static int check_format(int32_t bits, int32_t K, int32_t N, int32_t group)
{
    if (bits != 2 && bits != 4)
        return OR_EUNSUPPORTED;
    if (group != 128 && group != K)
        return OR_EUNSUPPORTED;
    if (K <= 0 || N <= 0 || K % 128 != 0)
        return OR_EINVAL;
    return OR_OK;
}

/* ---------------------------------------------------------------- pack --- */

/* Per (n, group): lo/hi over the group (with 0 included), s = fp16 of the FP64
 * quotient (hi - lo) / (2^b - 1) (CTX-TIER kernel details: scale = range / 3
 * for INT2), integer zero point z = rne(-lo / s), codes q = rne(W / s) + z,
 * both clamped to [0, 2^b - 1], packed along K into uint32 words (code j of a
 * word at bit code_shift(b, j)).  W is FP32 [K][ldw].  Returns OR_EINVAL for non-finite
 * W or a scale that overflows FP16. */
int or_pack(const float* W, int64_t ldw, int32_t K, int32_t N, int32_t bits,
            int32_t group, uint32_t* codes, uint16_t* scales, uint16_t* zeros)
{
    int st = check_format(bits, K, N, group);
    if (st)
        return st;
    if (ldw < N)
        return OR_EINVAL;
    const int qmax = (1 << bits) - 1;
    const int per_word = 32 / bits;
    const int64_t words_per_row = (int64_t)K / per_word;
    const int groups = K / group;
    int bad = 0;

    memset(codes, 0, sizeof(uint32_t) * (size_t)words_per_row * (size_t)N);
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int32_t n = 0; n < N; ++n) {
        for (int g = 0; g < groups; ++g) {
            double lo = 0.0, hi = 0.0;
            for (int k = g * group; k < (g + 1) * group; ++k) {
                double w = (double)W[(int64_t)k * ldw + n];
                if (!isfinite(w))
                    bad = 1;
                if (w < lo)
                    lo = w;
                if (w > hi)
                    hi = w;
            }
            double s = or_round_half((hi - lo) / (double)qmax);
            if (isinf(s) || isnan(s))
                bad = 1;
            if (s == 0.0)
                s = 1.0;
            double z = nearbyint(-lo / s);
            if (z < 0)
                z = 0;
            if (z > qmax)
                z = qmax;
            scales[(int64_t)n * groups + g] = or_double_to_half_bits(s);
            zeros[(int64_t)n * groups + g] = or_double_to_half_bits(z);
            for (int k = g * group; k < (g + 1) * group; ++k) {
                double w = (double)W[(int64_t)k * ldw + n];
                double q = nearbyint(w / s) + z;
                if (!(q >= 0))
                    q = 0;
                if (q > qmax)
                    q = qmax;
                codes[(int64_t)n * words_per_row + k / per_word] |=
                    ((uint32_t)q) << code_shift(bits, k % per_word);
            }
        }
    }
    return bad ? OR_EINVAL : OR_OK;
}

/* -------------------------------------------------------------- unpack --- */

/* q[n][k] = (codes[n][k / (32/b)] >> code_shift(b, k mod 32/b)) & (2^b - 1). */
int or_unpack(const uint32_t* codes, int32_t K, int32_t N, int32_t bits,
              uint8_t* q)
{
    int st = check_format(bits, K, N, 128);
    if (st)
        return st;
    const int per_word = 32 / bits;
    const int64_t words_per_row = (int64_t)K / per_word;
    const uint32_t mask = (1u << bits) - 1u;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            q[n * K + k] = (uint8_t)((codes[n * words_per_row + k / per_word] >>
                                      code_shift(bits, (int)(k % per_word))) & mask);
    return OR_OK;
}

/* ------------------------------------------------------------- dequant --- */

/* One output channel: w^[k] = (q[k] - z[g]) * s[g], g = k / group, in FP64
 * (exact: s is FP16 and |q - z| <= 15). */
static void dequant_row(const uint32_t* codes, const uint16_t* scales,
                        const uint16_t* zeros, int32_t K, int32_t bits,
                        int32_t group, int64_t n, double* out)
{
    const int per_word = 32 / bits;
    const int64_t words_per_row = (int64_t)K / per_word;
    const int groups = K / group;
    const uint32_t mask = (1u << bits) - 1u;
    for (int64_t k = 0; k < K; ++k) {
        uint32_t q = (codes[n * words_per_row + k / per_word] >>
                      code_shift(bits, (int)(k % per_word))) & mask;
        int64_t g = k / group;
        double s = or_half_to_double(scales[n * groups + g]);
        double z = or_half_to_double(zeros[n * groups + g]);
        out[k] = ((double)q - z) * s;
    }
}

/* out[n][k] = w^[k][n] (N-major, like the packed rows). */
int or_dequant(const uint32_t* codes, const uint16_t* scales,
               const uint16_t* zeros, int32_t K, int32_t N, int32_t bits,
               int32_t group, double* out)
{
    int st = check_format(bits, K, N, group);
    if (st)
        return st;
#pragma omp parallel for schedule(static)
    for (int32_t n = 0; n < N; ++n)
        dequant_row(codes, scales, zeros, K, bits, group, n, out + (int64_t)n * K);
    return OR_OK;
}

/* ---------------------------------------------------------------- GEMM --- */

typedef struct {
    int32_t bits, K, N, group;
    const uint32_t* codes;
    const uint16_t* scales;
    const uint16_t* zeros;
} or_weight;

/* Y[m][n] = sum over k ascending of X[m][k] * w^[k][n], all in FP64.
 * X is given as doubles (each an FP16 value on the path). */
static int gemm_d(const double* X, int64_t ldx, int32_t M, const or_weight* w,
                  double* Y, int64_t ldy)
{
    int st = check_format(w->bits, w->K, w->N, w->group);
    if (st)
        return st;
    const int32_t K = w->K, N = w->N;
    int oom = 0;
#pragma omp parallel reduction(| : oom)
    {
        /* every thread of the team must reach the worksharing loop, also one
         * whose buffer could not be allocated (it then skips its rows and the
         * call reports OR_ENOMEM) */
        double* row = (double*)malloc(sizeof(double) * (size_t)K);
        if (!row)
            oom = 1;
#pragma omp for schedule(static)
        for (int32_t n = 0; n < N; ++n) {
            if (!row)
                continue;
            dequant_row(w->codes, w->scales, w->zeros, K, w->bits, w->group, n, row);
            for (int32_t m = 0; m < M; ++m) {
                const double* x = X + (int64_t)m * ldx;
                double acc = 0.0;
                for (int32_t k = 0; k < K; ++k)
                    acc += x[k] * row[k];
                Y[(int64_t)m * ldy + n] = acc;
            }
        }
        free(row);
    }
    return oom ? OR_ENOMEM : OR_OK;
}

/* Public GEMM: X is FP16 bits [M][ldx]; Y is FP64 [M][ldy] (not rounded). */
int or_gemm(const uint16_t* X, int64_t ldx, int32_t M, const or_weight* w,
            double* Y, int64_t ldy)
{
    if (M < 0 || ldx < w->K || ldy < w->N)
        return OR_EINVAL;
    double* Xd = (double*)malloc(sizeof(double) * (size_t)(M ? M : 1) * (size_t)w->K);
    if (!Xd)
        return OR_ENOMEM;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < w->K; ++k)
            Xd[m * w->K + k] = or_half_to_double(X[m * ldx + k]);
    int st = gemm_d(Xd, w->K, M, w, Y, ldy);
    free(Xd);
    return st;
}

/* ---------------------------------------------------------- LayerNorm --- */

/* Parameter-free LayerNorm of one row of D values, FP64, rounded to FP16:
 * (h - mean) / sqrt(var + eps), population variance. */
static void layernorm_fp16(const double* h, int32_t D, double eps, double* out)
{
    double mean = 0.0;
    for (int32_t i = 0; i < D; ++i)
        mean += h[i];
    mean /= D;
    double var = 0.0;
    for (int32_t i = 0; i < D; ++i)
        var += (h[i] - mean) * (h[i] - mean);
    var /= D;
    double r = 1.0 / sqrt(var + eps);
    for (int32_t i = 0; i < D; ++i)
        out[i] = or_round_half((h[i] - mean) * r);
}

int or_layernorm(const double* h, int32_t M, int32_t D, double* out)
{
    for (int64_t m = 0; m < M; ++m)
        layernorm_fp16(h + m * D, D, 1e-5, out + m * D);
    return OR_OK;
}

/* ---------------------------------------------------------------- loop --- */

/* The block's weights.  gate.codes == NULL: four projections, identity FFN
 * activation.  Otherwise the FFN is SwiGLU ("Model" page, Parameters:
 * ffn_dim is the width of the gate and up projections; "β-Informed Deployment
 * Features" page, CTX-TIER Phase 2: the loop block's five weights attn_qkv,
 * attn_out, mlp_gate, mlp_up, mlp_down): a = fp16(silu(g) * u) with
 * g = fp16(x . Wgate), u = fp16(x . Wup), then down(a). */
typedef struct {
    int32_t D, F;
    or_weight qkv, out, up, down, gate;
} or_block;

/* silu(z) = z * sigmoid(z) = z / (1 + e^-z), in FP64. */
double or_silu(double z)
{
    return z / (1.0 + exp(-z));
}

static void round_all(double* v, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        v[i] = or_round_half(v[i]);
}

/* Iterations [L0, L1) of the shared block, in place on the FP64 residual h
 * [M][D] (warm-start page, internal flow: run_loop_iters_range).  Each
 * iteration with the same weights:
 *   x   = fp16(LN(h));   qkv = fp16(x @ Wqkv)          [M][3D]
 *   o   = fp16(qkv[:, 2D:3D] @ Wout);   h += o
 *   x   = fp16(LN(h));   u = fp16(x @ Wup)             [M][F]
 *   d   = fp16(u @ Wdown);              h += d
 * If the last_* pointers are non-NULL they receive the last iteration's
 * FP16-valued intermediates: norm (the second LN output), qkv, u and d. */
int or_loop_range(const or_block* b, double* h, int32_t M, int32_t L0,
                  int32_t L1, double* last_norm, double* last_qkv,
                  double* last_u, double* last_y, double* last_g)
{
    const int32_t D = b->D, F = b->F;
    const int gated = b->gate.codes != NULL;
    if (M < 0 || L0 < 0 || L1 < L0 || D <= 0 || F <= 0)
        return OR_EINVAL;
    if (b->qkv.K != D || b->qkv.N != 3 * D || b->out.K != D || b->out.N != D ||
        b->up.K != D || b->up.N != F || b->down.K != F || b->down.N != D)
        return OR_EINVAL;
    if (gated && (b->gate.K != D || b->gate.N != F))
        return OR_EINVAL;
    if (M == 0 || L0 == L1)
        return OR_OK;
    const size_t md = (size_t)M * D;
    double* x = (double*)malloc(sizeof(double) * md);
    double* qkv = (double*)malloc(sizeof(double) * md * 3);
    double* v = (double*)malloc(sizeof(double) * md);
    double* o = (double*)malloc(sizeof(double) * md);
    double* u = (double*)malloc(sizeof(double) * (size_t)M * F);
    double* g = gated ? (double*)malloc(sizeof(double) * (size_t)M * F) : NULL;
    int st = (x && qkv && v && o && u && (g || !gated)) ? OR_OK : OR_ENOMEM;
    for (int32_t l = L0; l < L1 && st == OR_OK; ++l) {
        or_layernorm(h, M, D, x);
        st = gemm_d(x, D, M, &b->qkv, qkv, 3 * D);
        if (st)
            break;
        round_all(qkv, (int64_t)md * 3);
        for (int64_t m = 0; m < M; ++m)
            memcpy(v + m * D, qkv + m * 3 * D + 2 * D, sizeof(double) * D);
        st = gemm_d(v, D, M, &b->out, o, D);
        if (st)
            break;
        round_all(o, (int64_t)md);
        for (size_t i = 0; i < md; ++i)
            h[i] += o[i];
        or_layernorm(h, M, D, x);
        st = gemm_d(x, D, M, &b->up, u, F);
        if (st)
            break;
        round_all(u, (int64_t)M * F);
        if (gated) {
            st = gemm_d(x, D, M, &b->gate, g, F);
            if (st)
                break;
            round_all(g, (int64_t)M * F);
            for (int64_t i = 0; i < (int64_t)M * F; ++i)
                u[i] = or_round_half(or_silu(g[i]) * u[i]);
        }
        st = gemm_d(u, F, M, &b->down, o, D);
        if (st)
            break;
        round_all(o, (int64_t)md);
        for (size_t i = 0; i < md; ++i)
            h[i] += o[i];
    }
    if (st == OR_OK) {
        if (last_norm)
            memcpy(last_norm, x, sizeof(double) * md);
        if (last_qkv)
            memcpy(last_qkv, qkv, sizeof(double) * md * 3);
        if (last_u)
            memcpy(last_u, u, sizeof(double) * (size_t)M * F);
        if (last_y)
            memcpy(last_y, o, sizeof(double) * md);
        if (last_g && gated)
            memcpy(last_g, g, sizeof(double) * (size_t)M * F);
    }
    free(x);
    free(qkv);
    free(v);
    free(o);
    free(u);
    free(g);
    return st;
}

/* --------------------------------------------------- array conveniences --- */

/* Element-wise or_round_half (used to compare against FP16 device outputs). */
void or_round_half_array(const double* x, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = or_round_half(x[i]);
}

void or_half_bits_array(const double* x, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = or_double_to_half_bits(or_round_half(x[i]));
}

void or_half_to_double_array(const uint16_t* h, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = or_half_to_double(h[i]);
}

/* Threads the oracle's OpenMP loops use (reported beside its timings). */
int or_num_threads(void)
{
    return omp_get_max_threads();
}

/* Sets the threads later OpenMP loops use (n >= 1); for timing the oracle on
 * one core as well as on all of them.  Results do not depend on it: every
 * parallel loop writes disjoint outputs and reduces only with a bitwise OR. */
void or_set_num_threads(int n)
{
    omp_set_num_threads(n >= 1 ? n : 1);
}
