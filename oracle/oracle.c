/*
 * CPU oracle for the quantised GEMV / expert-MLP path.
 *
 * TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's
 * CPU-baseline leg are the only callers.  The product path never loads this
 * library.  It shares no code, header, table or helper with the HIP path.
 *
 * Plain and slow on purpose.  Each quantity comes straight from its
 * definition, in double precision.  Outputs are computed one at a time, and
 * every sum runs in input order.  The only concurrency is OpenMP over
 * independent outputs, which reorders no sum.
 *
 * Sources (page title, then the passage):
 *  [G]  "colibri Vulkan compute backend complete guide" (xdnf.cn): the
 *       shader-level details section (formats: int8; int4 with two per byte
 *       and value nibble-8; int3-g64 with two planes and one f32 scale per
 *       64 inputs; MXFP4 e2m1 nibble with bit 3 the sign and f32 scales per
 *       32 inputs that the host expands), the API contract section (gate_up
 *       is silu(gate(x))*up(x); the expert group is the whole fused MLP of a
 *       batch) and the correctness section (int4 is offset binary,
 *       nibble - 8).
 *  [V]  "colibri -- Vulkan backend (docs/vulkan.md)": the arithmetic
 *       paragraph (the device multiplies the CPU's weights by f32
 *       activations, so the two differ only in summation order); the
 *       expert-tier engine table (format numbers 1, 2, 4, 5, 7 and SwiGLU);
 *       the tier's list of properties (each expert's output joins its row in
 *       routing order) and the GLM-5.2 paragraph (routed experts in rank
 *       order, then the shared expert).
 *  [A]  "opus colibri scout": the router row (strata's router does the
 *       softmax and the top-k in one dispatch).
 *       The f16-rows paragraph of [V] (format 14: f16 values, no scales, the
 *       low half of a word the even column, laid out like bf16's format 11)
 *       and the expert-tier engine table of [V] (format 10 F32, 11 BF16, 12
 *       FP8 in 128x128 blocks, 13 int8 with a scale per 64 inputs).
 *  [OCP] The OCP Microscaling (MX) Formats specification v1.0, FP4 E2M1:
 *       1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit, subnormal
 *       when the exponent field is 0.
 *  [OFP8] The OCP 8-bit floating point specification (OFP8), E4M3: 1 sign
 *       bit, 4 exponent bits with bias 7, 3 mantissa bits, subnormal when the
 *       exponent field is 0, no infinities, S.1111.111 is NaN.
 *  [IEEE] IEEE 754 binary16 (5 exponent bits, bias 15, 10 fraction bits) and
 *       binary32; bfloat16 is the upper 16 bits of a binary32 (8 exponent
 *       bits, bias 127, 7 fraction bits).  The all-ones exponent holds the
 *       infinities (fraction 0) and NaNs.
 *
 * Readings taken where the pages are silent (each is a listed reading, not
 * a page fact):
 *  - int4 and MXFP4 pairs: the low nibble of byte j holds input 2j and the
 *    high nibble input 2j+1 (by analogy with f16 rows, whose low half is the
 *    even column, in the f16-rows paragraph of [V]).
 *  - groups are gs consecutive inputs of one row; scales are row-major
 *    [O][K/gs].
 *  - int3-g64: the low plane holds 2 bits per input, 16 inputs per
 *    little-endian 32-bit word (input k at bits 2*(k mod 16)); the high
 *    plane holds 1 bit per input, 32 inputs per word (bit k mod 32);
 *    code = low | high << 2, value = code - 4.
 *  - a weight is the real product value * scale; the materialised f32
 *    weight is that product rounded once to nearest-even.
 *  - router weights multiply each expert's down output; the shared expert
 *    is added last with weight 1.
 *  - formats 10, 11 and 14 carry no scales (a weight is its stored value).
 *  - format 12: E4M3 codes [O][K] and one f32 scale per block of 128 rows x
 *    128 inputs, row-major [ceil(O/128)][K/128]; K is a multiple of 128.
 *  - format 13: int8 codes [O][K] with f32 scales [O][K/gs], groups of gs
 *    consecutive inputs as in format 4 (gs 64 in the pages' containers).
 *  - 16-bit values are little-endian words in column order, which puts the
 *    even column in the low half of each 32-bit word.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <omp.h>

typedef struct {
    int fmt;               /* 1 int8/row, 2 int4/row, 4 int4/gs, 5 int3-g64, 7 MXFP4,
                              10 f32, 11 bf16, 12 E4M3 128x128, 13 int8/gs, 14 f16 */
    long O, K, gs;         /* rows, inputs per row, inputs per scale */
    const void *q;         /* codes (fmt 5: the 2-bit plane) */
    const void *q2;        /* fmt 5: the 1-bit plane; otherwise unused */
    const float *scales;   /* [O][K/gs]; fmt 12 [ceil(O/128)][K/128]; unused by 10, 11, 14 */
} orc_matrix;

/* ------------------------------------------------------------------ */
/* Code values, from the format definitions.                            */
/* ------------------------------------------------------------------ */

/* One nibble of a packed pair: even input in the low nibble. */
static int nibble_at(const uint8_t *row, long k)
{
    uint8_t byte = row[k / 2];
    if (k % 2 == 0)
        return byte & 0x0F;
    return byte >> 4;
}

/* FP4 E2M1 value of a 4-bit code, from its bit fields [OCP]. */
double orc_e2m1(int code)
{
    int sign = (code >> 3) & 1;
    int expo = (code >> 1) & 3;
    int mant = code & 1;
    double mag;
    if (expo == 0)
        mag = 0.5 * mant;                       /* 2^(1-1) * (mant / 2) */
    else
        mag = ldexp(1.0 + 0.5 * mant, expo - 1);   /* 2^(expo-1) * (1 + mant/2) */
    return sign ? -mag : mag;
}

/* Value of a binary floating-point code from its fields [IEEE], [OFP8]:
   1 sign bit over ebits exponent bits (bias 2^(ebits-1) - 1) over mbits
   fraction bits; subnormal when the exponent field is 0.  ieee: the
   all-ones exponent holds infinities and NaNs; otherwise (E4M3) only the
   all-ones magnitude is NaN and every other code is finite. */
double orc_minifloat(uint32_t code, int ebits, int mbits, int ieee)
{
    uint32_t frac = code & ((1u << mbits) - 1);
    uint32_t expo = (code >> mbits) & ((1u << ebits) - 1);
    int sign = (code >> (ebits + mbits)) & 1;
    int bias = (1 << (ebits - 1)) - 1;
    uint32_t emax = (1u << ebits) - 1;
    double mag;
    if (ieee && expo == emax)
        mag = frac ? NAN : INFINITY;
    else if (!ieee && expo == emax && frac == (1u << mbits) - 1)
        mag = NAN;
    else if (expo == 0)
        mag = ldexp((double)frac, 1 - bias - mbits);               /* 2^(1-bias) * frac / 2^mbits */
    else
        mag = ldexp((double)((1u << mbits) + frac), (int)expo - bias - mbits);   /* 2^(e-bias) * (1.frac) */
    return sign ? -mag : mag;
}

/* int3 code 0..7 of input k from the two planes. */
static int int3_code(const uint32_t *low_row, const uint32_t *high_row, long k)
{
    int low = (int)((low_row[k / 16] >> (2 * (k % 16))) & 3u);
    int high = (int)((high_row[k / 32] >> (k % 32)) & 1u);
    return low | (high << 2);
}

/* The signed value v of weight (o, k) before scaling. */
double orc_code_value(const orc_matrix *m, long o, long k)
{
    switch (m->fmt) {
    case 1: {
        const int8_t *row = (const int8_t *)m->q + o * m->K;
        return (double)row[k];
    }
    case 2:
    case 4: {
        const uint8_t *row = (const uint8_t *)m->q + o * (m->K / 2);
        return (double)(nibble_at(row, k) - 8);
    }
    case 5: {
        const uint32_t *low_row = (const uint32_t *)m->q + o * (m->K / 16);
        const uint32_t *high_row = (const uint32_t *)m->q2 + o * (m->K / 32);
        return (double)(int3_code(low_row, high_row, k) - 4);
    }
    case 7: {
        const uint8_t *row = (const uint8_t *)m->q + o * (m->K / 2);
        return orc_e2m1(nibble_at(row, k));
    }
    case 10: {
        const float *row = (const float *)m->q + o * m->K;
        return (double)row[k];
    }
    case 11: {
        const uint16_t *row = (const uint16_t *)m->q + o * m->K;
        return orc_minifloat(row[k], 8, 7, 1);
    }
    case 12: {
        const uint8_t *row = (const uint8_t *)m->q + o * m->K;
        return orc_minifloat(row[k], 4, 3, 0);
    }
    case 13: {
        const int8_t *row = (const int8_t *)m->q + o * m->K;
        return (double)row[k];
    }
    case 14: {
        const uint16_t *row = (const uint16_t *)m->q + o * m->K;
        return orc_minifloat(row[k], 5, 10, 1);
    }
    }
    return NAN;
}

/* The scale that applies to weight (o, k). */
double orc_scale(const orc_matrix *m, long o, long k)
{
    if (m->fmt == 10 || m->fmt == 11 || m->fmt == 14)
        return 1.0;
    if (m->fmt == 12) {
        long blocks = m->K / 128;
        return (double)m->scales[(o / 128) * blocks + k / 128];
    }
    long groups = m->K / m->gs;
    return (double)m->scales[o * groups + k / m->gs];
}

/* Weight (o, k) as a real number: v * s.  Exact in double (v has at most
   8 significant bits and s 24, or s is 1 and v is a stored f32 or
   narrower float). */
double orc_weight(const orc_matrix *m, long o, long k)
{
    return orc_code_value(m, o, k) * orc_scale(m, o, k);
}

/* ------------------------------------------------------------------ */
/* Dequantisation: f32 weights, v * s rounded once to nearest-even.     */
/* ------------------------------------------------------------------ */

void orc_dequant(const orc_matrix *m, float *out)
{
    long o;
#pragma omp parallel for schedule(static)
    for (o = 0; o < m->O; o++)
        for (long k = 0; k < m->K; k++)
            out[o * m->K + k] = (float)orc_weight(m, o, k);
}

/* ------------------------------------------------------------------ */
/* GEMV: y[s][o] = sum_k w[o][k] * x[s][k], in double, k in order.      */
/* absn[s][o] = sum_k |w[o][k] * x[s][k]|, the per-row normaliser.      */
/* ------------------------------------------------------------------ */

static void row_dot(const orc_matrix *m, long o, const float *xf, const double *xd,
                    double *y, double *absn)
{
    double sum = 0.0, mag = 0.0;
    for (long k = 0; k < m->K; k++) {
        double xk = xf ? (double)xf[k] : xd[k];
        double term = orc_weight(m, o, k) * xk;
        sum += term;
        mag += fabs(term);
    }
    *y = sum;
    if (absn)
        *absn = mag;
}

void orc_gemv(const orc_matrix *m, const float *x, long S, double *y, double *absn)
{
    long idx;
#pragma omp parallel for schedule(static)
    for (idx = 0; idx < S * m->O; idx++) {
        long s = idx / m->O, o = idx % m->O;
        row_dot(m, o, x + s * m->K, NULL, &y[s * m->O + o], absn ? &absn[s * m->O + o] : NULL);
    }
}

/* Same with double inputs (used for the down projection of h). */
void orc_gemv_f64(const orc_matrix *m, const double *x, long S, double *y, double *absn)
{
    long idx;
#pragma omp parallel for schedule(static)
    for (idx = 0; idx < S * m->O; idx++) {
        long s = idx / m->O, o = idx % m->O;
        row_dot(m, o, NULL, x + s * m->K, &y[s * m->O + o], absn ? &absn[s * m->O + o] : NULL);
    }
}

/* ------------------------------------------------------------------ */
/* SwiGLU: h = silu(g) * u with silu(z) = z / (1 + exp(-z)).            */
/* ------------------------------------------------------------------ */

double orc_silu(double z)
{
    return z / (1.0 + exp(-z));
}

/* d silu / dz = sigma(z) * (1 + z * (1 - sigma(z))). */
static double silu_slope(double z)
{
    double sig = 1.0 / (1.0 + exp(-z));
    return sig * (1.0 + z * (1.0 - sig));
}

/*
 * gate_up over S tokens: g = G x, u = U x, h = silu(g) * u, each [S][I].
 * nh[s][i] bounds how far an f32 evaluation of h may move when g and u
 * carry errors proportional to their own normalisers (first order):
 *   nh = |silu'(g)| * absn_g * |u| + |silu(g)| * absn_u.
 * Any output pointer may be NULL except h.
 */
/*
 * gate_up with the clamped SwiGLU of [V]'s GLM paragraph (swiglu_limit L):
 *   g' = min(g, L), u' = min(max(u, -L), L), h = silu(g') * u'.
 * The pages give only what a limit of 0 does (every routed expert's output
 * is zero); this clamp is the reading that does that.  L = +inf is the
 * plain SwiGLU: both clamps are then the identity.  The normaliser carries
 * the clamped values; the clamps are 1-Lipschitz, so the first-order reach
 * of the errors in g and u is still |silu'(g')| A_g |u'| + |silu(g')| A_u.
 */
void orc_gate_up_clamped(const orc_matrix *G, const orc_matrix *U, const float *x, long S, double limit,
                         double *h, double *nh, double *g_out, double *u_out,
                         double *ag_out, double *au_out)
{
    long I = G->O, idx;
#pragma omp parallel for schedule(static)
    for (idx = 0; idx < S * I; idx++) {
        long s = idx / I, i = idx % I;
        double g, u, ag, au;
        row_dot(G, i, x + s * G->K, NULL, &g, &ag);
        row_dot(U, i, x + s * U->K, NULL, &u, &au);
        double gc = g > limit ? limit : g;   /* NaN stays NaN */
        double uc = u > limit ? limit : (u < -limit ? -limit : u);
        h[idx] = orc_silu(gc) * uc;
        if (nh)
            nh[idx] = fabs(silu_slope(gc)) * ag * fabs(uc) + fabs(orc_silu(gc)) * au;
        if (g_out) g_out[idx] = g;
        if (u_out) u_out[idx] = u;
        if (ag_out) ag_out[idx] = ag;
        if (au_out) au_out[idx] = au;
    }
}

void orc_gate_up(const orc_matrix *G, const orc_matrix *U, const float *x, long S,
                 double *h, double *nh, double *g_out, double *u_out,
                 double *ag_out, double *au_out)
{
    orc_gate_up_clamped(G, U, x, S, INFINITY, h, nh, g_out, u_out, ag_out, au_out);
}

static void mlp_one(const orc_matrix *gate, const orc_matrix *up, const orc_matrix *down,
                    const float *x, double limit, double *h, double *nh, double *dy, double *dabs)
{
    long I = gate->O, H = down->O;
    orc_gate_up_clamped(gate, up, x, 1, limit, h, nh, NULL, NULL, NULL, NULL);
    long o;
#pragma omp parallel for schedule(static)
    for (o = 0; o < H; o++) {
        double sum = 0.0, mag = 0.0;
        for (long k = 0; k < I; k++) {
            double wk = orc_weight(down, o, k);
            sum += wk * h[k];
            mag += fabs(wk) * (fabs(h[k]) + nh[k]);
        }
        dy[o] = sum;
        dabs[o] = mag;
    }
}

void orc_expert_group_clamped(const orc_matrix *gates, const orc_matrix *ups, const orc_matrix *downs,
                              long n_experts, long S, long k, const int32_t *ids, const float *w,
                              long shared, const float *x, double limit, double *y, double *absn,
                              double *h_work /* [I] */, double *nh_work /* [I] */,
                              double *dy_work /* [H] */, double *dabs_work /* [H] */)
{
    long H = downs[0].O;
    for (long t = 0; t < S; t++) {
        double *yt = y + t * H, *at = absn + t * H;
        for (long o = 0; o < H; o++) {
            yt[o] = 0.0;
            at[o] = 0.0;
        }
        for (long r = 0; r < k; r++) {
            long e = ids[t * k + r];
            if (e < 0 || e >= n_experts) {
                for (long o = 0; o < H; o++)
                    yt[o] = NAN;
                continue;
            }
            double wr = (double)w[t * k + r];
            mlp_one(&gates[e], &ups[e], &downs[e], x + t * gates[e].K, limit, h_work, nh_work,
                    dy_work, dabs_work);
            for (long o = 0; o < H; o++) {
                yt[o] += wr * dy_work[o];
                at[o] += fabs(wr) * dabs_work[o];
            }
        }
        if (shared >= 0) {
            mlp_one(&gates[shared], &ups[shared], &downs[shared], x + t * gates[shared].K,
                    limit, h_work, nh_work, dy_work, dabs_work);
            for (long o = 0; o < H; o++) {
                yt[o] += dy_work[o];
                at[o] += dabs_work[o];
            }
        }
    }
}

/* ------------------------------------------------------------------ */
/* Threads.                                                             */
/* ------------------------------------------------------------------ */

void orc_expert_group(const orc_matrix *gates, const orc_matrix *ups, const orc_matrix *downs,
                      long n_experts, long S, long k, const int32_t *ids, const float *w,
                      long shared, const float *x, double *y, double *absn,
                      double *h_work, double *nh_work, double *dy_work, double *dabs_work)
{
    orc_expert_group_clamped(gates, ups, downs, n_experts, S, k, ids, w, shared, x, INFINITY, y, absn,
                             h_work, nh_work, dy_work, dabs_work);
}

/*
 * The expert group's second half on hidden states given from outside
 * (steps 4 and 5 of the group's definition: down, then the combine in rank
 * order, then the shared expert with weight 1):
 *   y[t]    = sum_{r<k} w[t][r] * (D_{ids[t][r]} . h[t*k + r])  + D_shared . h[S*k + t]
 *   absn[t] = sum_{r<k} |w[t][r]| * A(D_{ids[t][r]}, h[t*k + r]) + A(D_shared, h[S*k + t])
 * with A(D, v)[o] = sum_i |D[o][i] * v[i]|, the GEMV's own per-row
 * normaliser.  h is f32 [S*k + S][I] in the slot order of the device's
 * scratch (slot t*k + r for token t's rank r, slot S*k + t for its shared
 * expert), so that a device's down and combine can be checked on the hidden
 * states the device itself computed.  An id outside [0, n_experts) makes its
 * token's row of y NaN.  shared < 0: no shared expert.
 */
void orc_expert_group_down(const orc_matrix *downs, long n_experts, long S, long k, const int32_t *ids,
                           const float *w, long shared, const float *h, double *y, double *absn)
{
    long H = downs[0].O, I = downs[0].K, idx;
#pragma omp parallel for schedule(static)
    for (idx = 0; idx < S * H; idx++) {
        long t = idx / H, o = idx % H;
        double sum = 0.0, mag = 0.0;
        int bad = 0;
        for (long r = 0; r < k; r++) {
            long e = ids[t * k + r];
            if (e < 0 || e >= n_experts) {
                bad = 1;
                continue;
            }
            double d, a, wr = (double)w[t * k + r];
            row_dot(&downs[e], o, h + (t * k + r) * I, NULL, &d, &a);
            sum += wr * d;
            mag += fabs(wr) * a;
        }
        if (shared >= 0) {
            double ds, as;
            row_dot(&downs[shared], o, h + (S * k + t) * I, NULL, &ds, &as);
            sum += ds;
            mag += as;
        }
        y[idx] = bad ? NAN : sum;
        absn[idx] = mag;
    }
}

/* ------------------------------------------------------------------ */
/* DeepSeek V4's rounding activation.                                   */
/* ------------------------------------------------------------------ */

/*
 * [V], the paragraph on DeepSeek V4's CPU expert and the tier's third
 * activation: gate and up are rounded to bf16 before the clamped SwiGLU;
 * the activation times the route weight is rounded to bf16; down's input
 * is rounded to E4M3 with one power-of-two scale per 128 values (the
 * smallest power of two that takes the block's largest magnitude below
 * 448); down's output is rounded to bf16; the rows of one token are added
 * with no further weight, in ascending expert id, then rank.
 *
 * Readings: every rounding is to nearest, ties to even; a block is 128
 * consecutive values of one slot's activation (I a multiple of 128); a block
 * whose values are all zero takes scale 1; the shared expert's weight is 1
 * and its row is added after the routed ones; the sum of a token's rows is
 * an f32 sum from 0 in that order (the engine's rows are f32).  x is taken
 * as given: the pages round it on the host before the call.
 */

/* v rounded to nearest-even in a binary format with mbits fraction bits and
 * smallest normal exponent emin, subnormals sharing the quantum 2^(emin -
 * mbits).  No largest exponent: callers stay inside the format's range.
 * bf16: (7, -126) [IEEE]; E4M3: (3, -6) [OFP8]. */
double orc_round_fmt(double v, int mbits, int emin)
{
    if (v == 0.0 || isnan(v) || isinf(v))
        return v;
    int e;
    frexp(fabs(v), &e);            /* |v| = f 2^e with f in [1/2, 1): the leading bit is 2^(e-1) */
    int lead = e - 1 < emin ? emin : e - 1;
    double quantum = ldexp(1.0, lead - mbits);
    return nearbyint(v / quantum) * quantum;   /* v / quantum is exact; the default mode is to nearest-even */
}

/* The smallest power of two s with m / s < 448; 1 when m is 0. */
double orc_v4_block_scale(double m)
{
    if (!(m > 0.0))
        return 1.0;
    double s = 1.0;
    while (m / s >= 448.0)
        s *= 2.0;
    while (m / (s / 2.0) < 448.0)
        s /= 2.0;
    return s;
}

/* One token's rows added in ascending (expert id, rank), then the shared
 * row: y[o] = f32 sum from 0.  rows: [k + has_shared][H], rank order, the
 * shared row last. */
void orc_v4_combine(const double *rows, const int32_t *ids, long k, int has_shared, long H, float *y)
{
    for (long o = 0; o < H; o++)
        y[o] = 0.0f;
    char done[k > 0 ? k : 1];
    for (long r = 0; r < k; r++)
        done[r] = 0;
    for (long n = 0; n < k; n++) {
        long pick = -1;
        for (long r = 0; r < k; r++)
            if (!done[r] && (pick < 0 || ids[r] < ids[pick]))
                pick = r;   /* the lowest id; among equal ids the lowest rank */
        done[pick] = 1;
        for (long o = 0; o < H; o++)
            y[o] = y[o] + (float)rows[pick * H + o];
    }
    if (has_shared)
        for (long o = 0; o < H; o++)
            y[o] = y[o] + (float)rows[k * H + o];
}

static double bf16(double v) { return orc_round_fmt(v, 7, -126); }

/* Is the bf16 rounding of a value known to within +-err not unique? */
static int bf16_open(double v, double err)
{
    return bf16(v - err) != bf16(v + err);
}

/*
 * One slot: e4[I] (down's input) and down's rounded outputs d[H].  A device
 * whose weighted activation may stray by act_rel of its value can take an
 * open bf16 decision either way; e4_lo, e4_hi bound what it then holds
 * (both candidates under both block scales those candidates allow: E4M3
 * rounding is monotone for a fixed scale, and the scale in the block's
 * maximum).  d_lo, d_hi bound down's rounded outputs for such an e4 and an
 * f32 sum that strays by down_err * sum|w e4|.  Returns the number of open
 * bf16 decisions before down: gate and up within gu_err * sum|w x|, the
 * weighted activation within act_rel of its value.
 */
static long v4_slot(const orc_matrix *gate, const orc_matrix *up, const orc_matrix *down, const float *x,
                    double limit, double wr, double gu_err, double act_rel, double down_err,
                    double *e4, double *e4_lo, double *e4_hi, double *d, double *d_lo, double *d_hi)
{
    long I = gate->O, H = down->O, open = 0, i;
#pragma omp parallel for schedule(static) reduction(+ : open)
    for (i = 0; i < I; i++) {
        double g, u, ag, au;
        row_dot(gate, i, x, NULL, &g, &ag);
        row_dot(up, i, x, NULL, &u, &au);
        open += bf16_open(g, gu_err * ag) + bf16_open(u, gu_err * au);
        double gb = bf16(g), ub = bf16(u);
        double gc = gb > limit ? limit : gb;
        double uc = ub > limit ? limit : (ub < -limit ? -limit : ub);
        double hv = orc_silu(gc) * uc * wr;
        open += bf16_open(hv, act_rel * fabs(hv));
        e4[i] = bf16(hv);
        e4_lo[i] = bf16(hv - act_rel * fabs(hv));
        e4_hi[i] = bf16(hv + act_rel * fabs(hv));
    }
    for (long b0 = 0; b0 < I; b0 += 128) {
        double m = 0.0, m_lo = 0.0, m_hi = 0.0;
        for (long j = b0; j < b0 + 128; j++) {
            if (fabs(e4[j]) > m || isnan(e4[j]))
                m = isnan(e4[j]) ? NAN : fabs(e4[j]);
            double a = fabs(e4_lo[j]), b = fabs(e4_hi[j]);
            double small = a < b ? a : b, big = a < b ? b : a;
            if (small > m_lo)
                m_lo = small;
            if (big > m_hi)
                m_hi = big;
        }
        double s = orc_v4_block_scale(m), s_lo = orc_v4_block_scale(m_lo), s_hi = orc_v4_block_scale(m_hi);
        for (long j = b0; j < b0 + 128; j++) {
            double c[4] = {orc_round_fmt(e4_lo[j] / s_lo, 3, -6) * s_lo, orc_round_fmt(e4_lo[j] / s_hi, 3, -6) * s_hi,
                           orc_round_fmt(e4_hi[j] / s_lo, 3, -6) * s_lo, orc_round_fmt(e4_hi[j] / s_hi, 3, -6) * s_hi};
            e4[j] = orc_round_fmt(e4[j] / s, 3, -6) * s;
            e4_lo[j] = e4_hi[j] = c[0];
            for (int q = 1; q < 4; q++) {
                if (c[q] < e4_lo[j])
                    e4_lo[j] = c[q];
                if (c[q] > e4_hi[j])
                    e4_hi[j] = c[q];
            }
        }
    }
    long o;
#pragma omp parallel for schedule(static)
    for (o = 0; o < H; o++) {
        double sum = 0.0, lo = 0.0, hi = 0.0, mag = 0.0;
        for (long j = 0; j < I; j++) {
            double wk = orc_weight(down, o, j);
            double p = wk * e4_lo[j], q = wk * e4_hi[j];
            sum += wk * e4[j];
            lo += p < q ? p : q;
            hi += p < q ? q : p;
            mag += fabs(p) > fabs(q) ? fabs(p) : fabs(q);
        }
        d[o] = bf16(sum);
        d_lo[o] = bf16(lo - down_err * mag);
        d_hi[o] = bf16(hi + down_err * mag);
    }
    return open;
}

/*
 * The expert group with DeepSeek V4's activation.  Outputs: h [S*k + S][I]
 * (down's input per slot, in the slot order of the device scratch: t*k + r,
 * then S*k + t for the shared expert) with its bounds h_lo, h_hi, y [S][H]
 * f32 and the f32 sums y_lo, y_hi of the rows' lower and upper candidates
 * (f32 addition is monotone in each operand, so a device whose only
 * differences are within the error bounds lands in [y_lo, y_hi]).  An id
 * outside [0, n_experts) makes its token's y NaN.  Returns the count of open
 * decisions before down.  The bounds assume gate and up themselves exact
 * (gu_err = 0, or no open decision there).
 */
long orc_expert_group_v4(const orc_matrix *gates, const orc_matrix *ups, const orc_matrix *downs,
                         long n_experts, long S, long k, const int32_t *ids, const float *w, long shared,
                         const float *x, double limit, double gu_err, double act_rel, double down_err,
                         double *h, double *h_lo, double *h_hi, float *y, float *y_lo, float *y_hi)
{
    long H = downs[0].O, I = gates[0].O, nr = S * k, open = 0;
    long nrow = k + (shared >= 0 ? 1 : 0);
    double *rows = malloc(sizeof(double) * (size_t)(3 * nrow * H + 1));
    if (!rows)
        return -1;
    double *lo = rows + nrow * H, *hi = lo + nrow * H;
    for (long t = 0; t < S; t++) {
        int bad = 0;
        for (long j = 0; j < nrow; j++) {
            long slot = j < k ? t * k + j : nr + t;
            long e = j < k ? ids[t * k + j] : shared;
            double wr = j < k ? (double)w[t * k + j] : 1.0;
            if (e < 0 || e >= n_experts) {
                bad = 1;
                for (long i = 0; i < I; i++)
                    h[slot * I + i] = h_lo[slot * I + i] = h_hi[slot * I + i] = NAN;
                continue;
            }
            open += v4_slot(&gates[e], &ups[e], &downs[e], x + t * gates[e].K, limit, wr, gu_err, act_rel,
                            down_err, h + slot * I, h_lo + slot * I, h_hi + slot * I, rows + j * H, lo + j * H,
                            hi + j * H);
        }
        if (bad) {
            for (long o = 0; o < H; o++)
                y[t * H + o] = y_lo[t * H + o] = y_hi[t * H + o] = NAN;
            continue;
        }
        orc_v4_combine(rows, ids + t * k, k, shared >= 0, H, y + t * H);
        orc_v4_combine(lo, ids + t * k, k, shared >= 0, H, y_lo + t * H);
        orc_v4_combine(hi, ids + t * k, k, shared >= 0, H, y_hi + t * H);
    }
    free(rows);
    return open;
}

/* ------------------------------------------------------------------ */
/* Router: logits -> scores -> top-k -> (ids, weights).                 */
/* ------------------------------------------------------------------ */

/*
 * One token's routing, from [V]'s engine tables (the host row of several
 * engines: the router's softmax, then top-k; MiMo's: sigmoid scores, a
 * correction bias that only picks, the top-k weights renormalised) and
 * the router row of [A] (softmax and top-k in one dispatch).
 *
 *   mode 0: p[e] = exp(l[e]) / sum_j exp(l[j])   (max subtracted first)
 *   mode 1: p[e] = 1 / (1 + exp(-l[e]))
 *   the pick key is l[e] without a bias (both scores keep the logits'
 *   order), or p[e] + bias[e] with one;
 *   ids: the k experts of largest key, largest first, equal keys by the
 *   lower index;
 *   w[r] = p[ids[r]], divided by their sum when renorm, then times w_scale.
 *
 * Readings: selection by the logit order without a bias (the order the
 * scores have in exact arithmetic); ties go to the lower index; the bias
 * never enters a weight.  Everything in double precision; the key used
 * for picking with a bias is the double p + bias.
 */
void orc_route(const float *logits, long S, long E, long k, int mode, int renorm,
               const float *bias, double w_scale, int32_t *ids, double *w, double *key_out)
{
    for (long t = 0; t < S; ++t) {
        const float *l = logits + t * E;
        double p[E > 0 ? E : 1], key[E > 0 ? E : 1];
        if (mode == 0) {
            double mx = l[0];
            for (long e = 1; e < E; ++e)
                if (l[e] > mx)
                    mx = l[e];
            double z = 0.0;
            for (long e = 0; e < E; ++e)
                z += exp((double)l[e] - mx);
            for (long e = 0; e < E; ++e)
                p[e] = exp((double)l[e] - mx) / z;
        } else {
            for (long e = 0; e < E; ++e)
                p[e] = 1.0 / (1.0 + exp(-(double)l[e]));
        }
        for (long e = 0; e < E; ++e)
            key[e] = bias ? p[e] + (double)bias[e] : (double)l[e];
        if (key_out)
            for (long e = 0; e < E; ++e)
                key_out[t * E + e] = key[e];
        /* selection: k passes, each taking the largest key not yet taken */
        char taken[E > 0 ? E : 1];
        for (long e = 0; e < E; ++e)
            taken[e] = 0;
        double sum = 0.0;
        for (long r = 0; r < k; ++r) {
            long best = -1;
            for (long e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || key[e] > key[best]))
                    best = e;
            taken[best] = 1;
            ids[t * k + r] = (int32_t)best;
            w[t * k + r] = p[best];
            sum += p[best];
        }
        for (long r = 0; r < k; ++r) {
            double v = w[t * k + r];
            if (renorm)
                v = v / sum;
            w[t * k + r] = v * w_scale;
        }
    }
}

void orc_set_threads(int n)
{
    if (n > 0)
        omp_set_num_threads(n);
}

int orc_get_threads(void)
{
    return omp_get_max_threads();
}
