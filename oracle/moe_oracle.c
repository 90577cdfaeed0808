/*
 * CPU oracle for the routed SwiGLU MoE forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's
 * cpu_baseline leg use it.  It shares no code, header or table with the HIP
 * library; it is written from the method's description, one step at a time,
 * in the order the sources give them.
 *
 * Sources (web pages):
 *   [MEGA]  Megatron-LM PR #7830, "flashinfer_mega" backend, section
 *           "1. Mega backend for generation" (canonical expert-id sort before
 *           the combine; gate/up interleaved in blocks of 32, K-major).
 *   [VALUE] Megatron-LM PR #7798, moe_training_matches_inference, sections
 *           "Background" (activation and FC2-input quantization fused into
 *           the FC1 epilogue, probabilities applied after FC2) and
 *           "What is changed" (finalize = fp32 fused multiply-adds of
 *           probability and row, from zero, in the listed order).
 *   [BOUND] Megatron-LM PR #8367, "bound the FlashInfer MoE expert kernels by
 *           token count", section "Problem" (device-side live token count;
 *           fp32 finalize output without a bf16 downcast).
 *   [API]   Megatron-Core API docs, core.transformer.moe.
 *           training_matches_inference, `_route` ([tokens, topk] probs and
 *           ids; the finalize sums routes in the order listed).
 *   [CUDNN] cudnn-frontend PR #448, MoeEp class docstring (rows grouped by
 *           expert ascending, token-major route order inside an expert) and
 *           the MXFP8 32-element scale block.
 *
 * Precision.  Where the sources fix a precision (the fp32 finalize) the
 * oracle uses it exactly (fmaf).  Where they fix only "fp32 accumulate"
 * without an order (the expert GEMMs) the oracle computes the exact dot
 * product in fp64 and rounds once to fp32: the plain definition that any
 * fp32 accumulation order approximates.  Values that decide an integer
 * (a bf16 rounding, an E4M3 code, an E8M0 exponent) are decided from an
 * fp32 value, the kernel's precision.  The router softmax (precision not
 * fixed) is fp64, rounded to fp32 at the end.
 *
 * Every function here is pinned by tests under tests/ against something
 * other than itself (library casts, brute force, closed forms, dense fp64
 * matmuls, hand-derived cases); see the test files for which pin covers which
 * function.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Flag added to a forward's combine: the probabilities are applied inside FC1. */
#define ORC_APPLY_TOPK_IN_FC1 0x100

#define ORC_ERR_BAD_ID 1u      /* an expert id outside [0, E) in a live token */
#define ORC_ERR_DUP_ID 2u      /* the same expert id twice in one live token  */
#define ORC_ERR_LIVE_HIGH 4u   /* live count above capacity: clamped           */
#define ORC_ERR_LIVE_NEG 8u    /* live count below zero: treated as zero       */

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float v) { uint32_t u; memcpy(&u, &v, 4); return u; }
static float bits_f32(uint32_t u) { float v; memcpy(&v, &u, 4); return v; }

/* bfloat16 = the top 16 bits of an fp32.  Round to nearest, ties to even
 * (RNE), written as: the kept part is rounded up when the dropped 16 bits
 * exceed half, or equal half and the kept part is odd.  NaN stays NaN. */
uint16_t orc_bf16_bits(float v)
{
    uint32_t u = f32_bits(v);
    if ((u & 0x7fffffffu) > 0x7f800000u)           /* NaN: keep sign, quiet */
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep = u >> 16;
    uint32_t drop = u & 0xffffu;
    if (drop > 0x8000u || (drop == 0x8000u && (keep & 1u)))
        keep += 1u;                                  /* may carry into inf */
    return (uint16_t)keep;
}

float orc_bf16_value(uint16_t b) { return bits_f32((uint32_t)b << 16); }

float orc_bf16_round(float v) { return orc_bf16_value(orc_bf16_bits(v)); }

void orc_bf16_round_array(const float* in, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_bits(in[i]);
}

/* E4M3FN (OCP 8-bit float, "fn" variant): 1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits; no infinities; S.1111.111 is NaN; largest finite
 * value 1.75 * 2^8 = 448; subnormals 0.mmm * 2^-6, the smallest 2^-9.
 * Decoding follows that definition. */
double orc_e4m3_decode(uint8_t c)
{
    int sign = (c >> 7) & 1;
    int ef = (c >> 3) & 15;
    int m = c & 7;
    double mag;
    if (ef == 15 && m == 7) return NAN;
    if (ef == 0) mag = ldexp((double)m, -9);           /* 0.mmm * 2^-6 */
    else mag = ldexp(8.0 + m, ef - 7 - 3);              /* 1.mmm * 2^(e-7) */
    return sign ? -mag : mag;
}

/* Encode a value whose magnitude is at most 448 (the caller's scale choice
 * guarantees it) to the nearest E4M3FN value, ties to the even code.  The
 * binade of |v| is found with frexp (exact); |v| is then expressed in units
 * of the binade's code spacing (an exact power-of-two scaling) and rounded
 * to an integer with nearbyint in the default round-to-nearest-even mode. */
uint8_t orc_e4m3_encode(double v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    if (isnan(v)) return (uint8_t)(sign | 0x7f);
    if (a == 0.0) return sign;
    int ex;
    frexp(a, &ex);                 /* a = f * 2^ex, f in [0.5, 1) => 2^(ex-1) <= a */
    int e = ex - 1;                /* unbiased exponent of the leading bit */
    if (e < -6) {                  /* subnormal range: spacing 2^-9 */
        double q = nearbyint(ldexp(a, 9));          /* 0..8 */
        return (uint8_t)(sign | (uint8_t)q);        /* q == 8 is the smallest normal */
    }
    double q = nearbyint(ldexp(a, 3 - e));          /* in [8, 16] */
    if (q == 16.0) { q = 8.0; e += 1; }
    /* |v| <= 448 keeps e <= 8 and the code below 0x7f. */
    return (uint8_t)(sign | (uint8_t)(((e + 7) << 3) | ((int)q - 8)));
}

/* E8M0 block exponent for one 32-element block: the smallest integer e in
 * [-127, 127] with amax <= 448 * 2^e (the power-of-two ceiling of
 * amax / 448).  amax == 0 gives -127.  Found by an exact search: the
 * comparisons are exact in fp64 because amax is an fp32 value and 448 * 2^e
 * is a power-of-two multiple of 448. */
int orc_e8m0_exponent(float amax)
{
    if (!(amax > 0.0f)) return -127;
    int ex;
    frexp((double)amax, &ex);
    int e = ex - 10;                                /* below the answer */
    while (!((double)amax <= ldexp(448.0, e))) e += 1;
    while (e > -127 && (double)amax <= ldexp(448.0, e - 1)) e -= 1;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* MXFP8 quantization of a [rows][cols] fp32 matrix along cols, one E8M0
 * scale per 32 consecutive elements: scale byte = e + 127, code =
 * E4M3(v / 2^e).  cols must be a multiple of 32. */
void orc_mx_quantize(const float* v, int64_t rows, int64_t cols, uint8_t* codes,
                     uint8_t* scales)
{
    int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const float* blk = v + r * cols + b * 32;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float a = fabsf(blk[i]);
                if (a > amax) amax = a;
            }
            int e = orc_e8m0_exponent(amax);
            scales[r * nb + b] = (uint8_t)(e + 127);
            for (int i = 0; i < 32; ++i)
                codes[r * cols + b * 32 + i] = orc_e4m3_encode(ldexp((double)blk[i], -e));
        }
    }
}

/* Value of an MXFP8 element: E4M3 value times 2^(scale - 127). */
void orc_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                       int64_t cols, double* out)
{
    int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = ldexp(orc_e4m3_decode(codes[r * cols + c]),
                                      (int)scales[r * nb + c / 32] - 127);
}

/* E2M1 (OCP MX 4-bit float): 1 sign bit, 2 exponent bits with bias 1, 1
 * mantissa bit; no infinities or NaN.  Exponent field 0 is subnormal
 * (0.m * 2^0); the magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4 and 6.  Decoding
 * follows that definition. */
double orc_e2m1_decode(uint8_t c)
{
    int sign = (c >> 3) & 1;
    int ef = (c >> 1) & 3;
    int m = c & 1;
    double mag = ef == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, ef - 1);
    return sign ? -mag : mag;
}

/* Encode a value whose magnitude is at most 6 (the caller's scale choice
 * guarantees it) to the nearest E2M1 value, ties to the even code, keeping
 * the sign (-0 and negatives that round to zero give code 8).  Exhaustive
 * search over the eight magnitudes. */
uint8_t orc_e2m1_encode(double v)
{
    uint8_t sign = signbit(v) ? 8 : 0;
    double a = fabs(v);
    int best = 0;
    double bd = INFINITY;
    for (int c = 0; c < 8; ++c) {
        double d = fabs(orc_e2m1_decode((uint8_t)c) - a);
        if (d < bd || (d == bd && (c & 1) == 0 && (best & 1))) { best = c; bd = d; }
    }
    return (uint8_t)(sign | best);
}

/* E8M0 block exponent for MXFP4: the smallest integer e in [-127, 127] with
 * amax <= 6 * 2^e (the power-of-two ceiling of amax / 6, the MXFP8 rule with
 * E2M1's largest value in place of E4M3's); amax == 0 gives -127.  Exact
 * search, as orc_e8m0_exponent. */
int orc_e8m0_exponent_fp4(float amax)
{
    if (!(amax > 0.0f)) return -127;
    int ex;
    frexp((double)amax, &ex);
    int e = ex - 4;                                 /* below the answer */
    while (!((double)amax <= ldexp(6.0, e))) e += 1;
    while (e > -127 && (double)amax <= ldexp(6.0, e - 1)) e -= 1;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* MXFP4 quantization of a [rows][cols] fp32 matrix along cols, one E8M0
 * scale per 32 consecutive elements: scale byte = e + 127, code (one per
 * byte here) = E2M1(v / 2^e).  cols must be a multiple of 32. */
void orc_mx4_quantize(const float* v, int64_t rows, int64_t cols, uint8_t* codes,
                      uint8_t* scales)
{
    int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const float* blk = v + r * cols + b * 32;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float a = fabsf(blk[i]);
                if (a > amax) amax = a;
            }
            int e = orc_e8m0_exponent_fp4(amax);
            scales[r * nb + b] = (uint8_t)(e + 127);
            for (int i = 0; i < 32; ++i)
                codes[r * cols + b * 32 + i] = orc_e2m1_encode(ldexp((double)blk[i], -e));
        }
    }
}

/* Value of an MXFP4 element: E2M1 value times 2^(scale - 127). */
void orc_mx4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                        int64_t cols, double* out)
{
    int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = ldexp(orc_e2m1_decode(codes[r * cols + c]),
                                      (int)scales[r * nb + c / 32] - 127);
}

/* ------------------------------------------------------------------------ */
/* Router ([API] `_route`; softmax, top-k, renormalize)                      */
/* ------------------------------------------------------------------------ */

static int32_t clamp_live(int32_t live, int64_t T_cap, uint32_t* err)
{
    if (live < 0) { *err |= ORC_ERR_LIVE_NEG; return 0; }
    if ((int64_t)live > T_cap) { *err |= ORC_ERR_LIVE_HIGH; return (int32_t)T_cap; }
    return live;
}

/* For each live token: softmax over the E logits, select the k experts with
 * the largest logits (ties to the lower id; selecting on the logits is the
 * same as selecting on the probabilities, which softmax orders the same way,
 * without ties that rounding could create), renormalize the selected
 * probabilities to sum to one, and emit them with ids ascending.  Softmax
 * and renormalization are fp64; the probabilities are rounded to fp32.
 * Rows at or beyond the live count are not written.  Returns error bits. */
uint32_t orc_route(const float* logits, int64_t T_cap, int32_t live, int E, int k,
                   int32_t* ids, float* probs)
{
    uint32_t err = 0;
    int32_t T = clamp_live(live, T_cap, &err);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const float* l = logits + t * E;
        double m = -INFINITY;
        for (int e = 0; e < E; ++e) if ((double)l[e] > m) m = l[e];
        double* p = (double*)malloc(sizeof(double) * E);
        char* taken = (char*)calloc(E, 1);
        double S = 0.0;
        for (int e = 0; e < E; ++e) { p[e] = exp((double)l[e] - m); S += p[e]; }
        for (int e = 0; e < E; ++e) p[e] /= S;
        int sel[64];
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;   /* strict: ties keep the lower id */
            }
            taken[best] = 1;
            sel[j] = best;
        }
        /* ascending id order */
        for (int a = 1; a < k; ++a)
            for (int b = a; b > 0 && sel[b - 1] > sel[b]; --b) {
                int tmp = sel[b]; sel[b] = sel[b - 1]; sel[b - 1] = tmp;
            }
        double Sk = 0.0;
        for (int j = 0; j < k; ++j) Sk += p[sel[j]];
        for (int j = 0; j < k; ++j) {
            ids[t * k + j] = sel[j];
            probs[t * k + j] = (float)(p[sel[j]] / Sk);
        }
        free(p);
        free(taken);
    }
    return err;
}

/* ------------------------------------------------------------------------ */
/* Permutation ([MEGA] canonical order; [CUDNN] row grouping)                */
/* ------------------------------------------------------------------------ */

/* Per live token, sort its k (id, prob) pairs by id ascending; equal ids
 * (a contract violation) keep their listed order.  Then a stable counting
 * sort of the routes r = t*k + j by expert: counts, exclusive offsets,
 * position of route r = offsets[e_r] + number of earlier routes (in r order)
 * to the same expert.  perm_src[pos] = r, dst[r] = pos.  A route whose id is
 * outside [0, E), or repeats the id of the route before it in canonical
 * order (the same expert listed twice for one token), is dropped: dst = -1,
 * not counted.  Outputs beyond the live routes are not written.  Returns
 * error bits. */
uint32_t orc_prepare(const int32_t* ids, const float* probs, int64_t T_cap, int32_t live,
                     int E, int k, int32_t* sorted_ids, float* sorted_probs,
                     int32_t* counts, int32_t* offsets, int32_t* perm_src, int32_t* dst,
                     int32_t* T_out)
{
    uint32_t err = 0;
    int32_t T = clamp_live(live, T_cap, &err);
    *T_out = T;
    for (int64_t t = 0; t < T; ++t) {
        int32_t id[64];
        float p[64];
        for (int j = 0; j < k; ++j) { id[j] = ids[t * k + j]; p[j] = probs[t * k + j]; }
        /* insertion sort: stable */
        for (int a = 1; a < k; ++a)
            for (int b = a; b > 0 && id[b - 1] > id[b]; --b) {
                int32_t ti = id[b]; id[b] = id[b - 1]; id[b - 1] = ti;
                float tp = p[b]; p[b] = p[b - 1]; p[b - 1] = tp;
            }
        for (int j = 0; j < k; ++j) {
            if (id[j] < 0 || id[j] >= E) err |= ORC_ERR_BAD_ID;
            if (j > 0 && id[j] == id[j - 1]) err |= ORC_ERR_DUP_ID;
            sorted_ids[t * k + j] = id[j];
            sorted_probs[t * k + j] = p[j];
        }
    }
    for (int e = 0; e < E; ++e) counts[e] = 0;
    int64_t R = (int64_t)T * k;
    char* drop = (char*)calloc((size_t)(R > 0 ? R : 1), 1);
    for (int64_t r = 0; r < R; ++r) {
        int32_t e = sorted_ids[r];
        if (e < 0 || e >= E || (r % k > 0 && sorted_ids[r - 1] == e)) { drop[r] = 1; continue; }
        counts[e] += 1;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t* fill = (int32_t*)calloc((size_t)(E > 0 ? E : 1), sizeof(int32_t));
    for (int64_t r = 0; r < R; ++r) {
        int32_t e = sorted_ids[r];
        if (drop[r]) { dst[r] = -1; continue; }
        int32_t pos = offsets[e] + fill[e]++;
        perm_src[pos] = (int32_t)r;
        dst[r] = pos;
    }
    free(fill);
    free(drop);
    return err;
}

/* ------------------------------------------------------------------------ */
/* Expert MLP and finalize                                                   */
/* ------------------------------------------------------------------------ */

/* Exact dot products of an operand row (fp64 values) with a weight row,
 * accumulated in fp64 and rounded once to fp32.  bf16 x bf16 and
 * MXFP8 x MXFP8 and MXFP8 x MXFP4 products are exact in fp64.  Weight rows are read either as
 * bf16 bit patterns or as fp32 values (the MXFP8 operand values, which fp32
 * holds exactly). */
static float dot_bf16(const double* a, const uint16_t* b, int64_t n)
{
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s += a[i] * (double)orc_bf16_value(b[i]);
    return (float)s;
}

static float dot_f32w(const double* a, const float* b, int64_t n)
{
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s += a[i] * (double)b[i];
    return (float)s;
}

/* SwiGLU of one (gate, up) pair, in fp64 from the fp32 accumulators, rounded
 * to fp32: silu(g) * u = g / (1 + exp(-g)) * u.  No clamp ([MEGA]: SwiGLU
 * only, no tanh clamp). */
static float swiglu_f32(float g, float u)
{
    double gd = g;
    return (float)(gd / (1.0 + exp(-gd)) * (double)u);
}

/* Weights of the oracle: the caller's bf16 bit patterns (bf16 path, not
 * copied) or fp32 operand values (MXFP8 path: the dequantized quantization). */
typedef struct {
    int E, H, F, k;
    int mx;                 /* 0: bf16 path, 1: MXFP8 path, 2: MXFP4 weights + MXFP8 activations */
    const uint16_t* w1b;    /* bf16 [E][2F][H] (gate rows 0..F-1, up rows F..2F-1) */
    const uint16_t* w2b;    /* bf16 [E][H][F] */
    const float* w1f;       /* MXFP8 / MXFP4 weight operand values, same shapes */
    const float* w2f;
} orc_model;

static float dot_w1(const orc_model* m, const double* xr, int64_t row)
{
    return m->mx ? dot_f32w(xr, m->w1f + row * m->H, m->H) : dot_bf16(xr, m->w1b + row * m->H, m->H);
}

static float dot_w2(const orc_model* m, const double* hr, int64_t row)
{
    return m->mx ? dot_f32w(hr, m->w2f + row * m->F, m->F) : dot_bf16(hr, m->w2b + row * m->F, m->F);
}

/* The expert MLP of one routed row: FC1 gate/up from the operand row xr
 * (length H), SwiGLU, the FC2-input rounding (bf16, or MXFP8 per 32-block),
 * then FC2 into o (length H, fp32).  Scratch a (F doubles) and hbuf (F).
 * With fc1_prob (the route's probability applied inside FC1, the MoeEp
 * apply_topk_in_fc1 option of cudnn-frontend PR #448), each SwiGLU value is
 * multiplied by p in fp32 before the FC2-input rounding, so FC2 returns the
 * weighted row; otherwise pass 1.0f (the product is then exact). */
static void expert_row_p(const orc_model* m, int e, const double* xr, float* o,
                         float* a32, double* hrow, float fc1_prob)
{
    const int64_t H = m->H, F = m->F;
    const int64_t r1 = (int64_t)e * 2 * F, r2 = (int64_t)e * H;
    for (int64_t n = 0; n < F; ++n) {
        float g = dot_w1(m, xr, r1 + n);
        float u = dot_w1(m, xr, r1 + F + n);
        a32[n] = swiglu_f32(g, u) * fc1_prob;
    }
    if (!m->mx) {
        for (int64_t n = 0; n < F; ++n) hrow[n] = orc_bf16_round(a32[n]);
    } else {
        for (int64_t b = 0; b < F / 32; ++b) {
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float a = fabsf(a32[b * 32 + i]);
                if (a > amax) amax = a;
            }
            int ex = orc_e8m0_exponent(amax);
            for (int i = 0; i < 32; ++i) {
                uint8_t c = orc_e4m3_encode(ldexp((double)a32[b * 32 + i], -ex));
                hrow[b * 32 + i] = ldexp(orc_e4m3_decode(c), ex);
            }
        }
    }
    for (int64_t mo = 0; mo < H; ++mo) o[mo] = dot_w2(m, hrow, r2 + mo);
}

static void expert_row(const orc_model* m, int e, const double* xr, float* o,
                       float* a32, double* hrow)
{
    expert_row_p(m, e, xr, o, a32, hrow, 1.0f);
}

/* Finalize ([VALUE] "What is changed"; [BOUND] "Problem"): for each live
 * token, acc = +0.0f, then for its routes in canonical order
 * acc = fmaf(p_j, O[dst[t*k+j]][m], acc); out[t][m] = acc in fp32.  A
 * dropped route (dst < 0) adds nothing.  Rows >= T are not written. */
void orc_finalize(const float* O, const int32_t* dst, const float* sorted_probs,
                  int32_t T, int k, int H, float* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t mo = 0; mo < H; ++mo) {
            float acc = 0.0f;
            for (int j = 0; j < k; ++j) {
                int32_t d = dst[t * k + j];
                if (d < 0) continue;
                acc = fmaf(sorted_probs[t * k + j], O[(int64_t)d * H + mo], acc);
            }
            out[t * H + mo] = acc;
        }
    }
}

/* BF16 combine ([VALUE] "What is changed", the BF16_RANK_PARTIALS unpermute,
 * which does what FlashInfer's finalize does): on one rank, a token's routes
 * are added as fp32 fused multiply-adds of probability and row from zero, in
 * the listed (canonical) order, and the sum is quantized to bf16 (round to
 * nearest even).  The fp32 sum is orc_finalize's. */
void orc_finalize_bf16(const float* O, const int32_t* dst, const float* sorted_probs,
                       int32_t T, int k, int H, uint16_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t mo = 0; mo < H; ++mo) {
            float acc = 0.0f;
            for (int j = 0; j < k; ++j) {
                int32_t d = dst[t * k + j];
                if (d < 0) continue;
                acc = fmaf(sorted_probs[t * k + j], O[(int64_t)d * H + mo], acc);
            }
            out[t * H + mo] = orc_bf16_bits(acc);
        }
    }
}

/* Finalize of the apply_topk_in_fc1 option (cudnn-frontend PR #448, MoeEp
 * constructor): the FC2 rows already carry their route's probability, so a
 * token's rows are added as an fp32 chain from +0.0f in canonical order,
 * acc = acc + O[dst[t*k+j]][m] (the fused multiply-add of [VALUE] with a
 * probability of 1, which is exact); to_bf16 rounds the sum to bf16 (nearest
 * even) as the bf16 combine does.  Dropped routes (dst < 0) add nothing. */
void orc_finalize_sum(const float* O, const int32_t* dst, int32_t T, int k, int H, int to_bf16,
                      void* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t mo = 0; mo < H; ++mo) {
            float acc = 0.0f;
            for (int j = 0; j < k; ++j) {
                int32_t d = dst[t * k + j];
                if (d < 0) continue;
                acc = acc + O[(int64_t)d * H + mo];
            }
            if (to_bf16) ((uint16_t*)out)[t * H + mo] = orc_bf16_bits(acc);
            else ((float*)out)[t * H + mo] = acc;
        }
}

/* Row mode ([VALUE] "What is changed", expert compute; [API]
 * expert_value_pass): every route goes through the finalize as a top-1 token
 * with probability 1.0, so the finalize returns the route's expert output
 * unscaled: rows[t][j][m] = fmaf(1.0f, O[dst[t*k+j]][m], +0.0f) for the j-th
 * route of token t in canonical order.  A dropped route (dst < 0) is a top-1
 * token with nothing to add: a row of +0.0.  Rows of tokens >= T are not
 * written. */
void orc_finalize_rows(const float* O, const int32_t* dst, int32_t T, int k, int H,
                       float* rows)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < (int64_t)T * k; ++r) {
        int32_t d = dst[r];
        for (int64_t mo = 0; mo < H; ++mo) {
            float acc = 0.0f;
            if (d >= 0) acc = fmaf(1.0f, O[(int64_t)d * H + mo], acc);
            rows[r * H + mo] = acc;
        }
    }
}

/* Operand values of x for the live tokens: bf16 values, or the MXFP8
 * quantization of those bf16 values (per token, per 32-block of H). */
static double* x_operands(const uint16_t* x, int64_t T, int H, int mx)
{
    double* xo = (double*)malloc(sizeof(double) * T * H);
    if (!mx) {
        for (int64_t i = 0; i < T * H; ++i) xo[i] = orc_bf16_value(x[i]);
    } else {
        float* xf = (float*)malloc(sizeof(float) * T * H);
        uint8_t* c = (uint8_t*)malloc(T * H);
        uint8_t* s = (uint8_t*)malloc(T * (H / 32));
        for (int64_t i = 0; i < T * H; ++i) xf[i] = orc_bf16_value(x[i]);
        orc_mx_quantize(xf, T, H, c, s);
        orc_mx_dequantize(c, s, T, H, xo);
        free(xf); free(c); free(s);
    }
    return xo;
}

/* MXFP8 weight operand values: the quantization of the bf16 values along K
 * (H for W1 rows, F for W2 rows), dequantized to fp32 (exact). */
static float* w_mx_operands(const uint16_t* w, int64_t rows, int64_t cols)
{
    float* wf = (float*)malloc(sizeof(float) * rows * cols);
    uint8_t* c = (uint8_t*)malloc(rows * cols);
    uint8_t* s = (uint8_t*)malloc(rows * (cols / 32));
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows * cols; ++i) wf[i] = orc_bf16_value(w[i]);
    orc_mx_quantize(wf, rows, cols, c, s);
    int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t q = 0; q < cols; ++q)
            wf[r * cols + q] = (float)ldexp(orc_e4m3_decode(c[r * cols + q]),
                                            (int)s[r * nb + q / 32] - 127);
    free(c); free(s);
    return wf;
}

/* MXFP4 weight operand values: the E2M1 quantization of the bf16 values
 * along K, dequantized to fp32 (exact). */
static float* w_mx4_operands(const uint16_t* w, int64_t rows, int64_t cols)
{
    float* wf = (float*)malloc(sizeof(float) * rows * cols);
    uint8_t* c = (uint8_t*)malloc(rows * cols);
    uint8_t* s = (uint8_t*)malloc(rows * (cols / 32));
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows * cols; ++i) wf[i] = orc_bf16_value(w[i]);
    orc_mx4_quantize(wf, rows, cols, c, s);
    int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t q = 0; q < cols; ++q)
            wf[r * cols + q] = (float)ldexp(orc_e2m1_decode(c[r * cols + q]),
                                            (int)s[r * nb + q / 32] - 127);
    free(c); free(s);
    return wf;
}

/* Opaque prepared weights, so that repeated oracle calls on the same model
 * (sampled tokens, timing) do not rebuild the operand values.  In the bf16
 * path the caller's arrays are read in place and must outlive the handle. */
typedef struct {
    orc_model m;
    float* w1f;
    float* w2f;
} orc_weights;

void* orc_weights_create(int E, int H, int F, int k, int mx, const uint16_t* w1,
                         const uint16_t* w2)
{
    orc_weights* w = (orc_weights*)calloc(1, sizeof(orc_weights));
    w->m.E = E; w->m.H = H; w->m.F = F; w->m.k = k; w->m.mx = mx;
    if (mx == 1) {
        w->w1f = w_mx_operands(w1, (int64_t)E * 2 * F, H);
        w->w2f = w_mx_operands(w2, (int64_t)E * H, F);
    } else if (mx == 2) {
        w->w1f = w_mx4_operands(w1, (int64_t)E * 2 * F, H);
        w->w2f = w_mx4_operands(w2, (int64_t)E * H, F);
    }
    w->m.w1b = w1; w->m.w2b = w2;
    w->m.w1f = w->w1f; w->m.w2f = w->w2f;
    return w;
}

void orc_weights_destroy(void* p)
{
    orc_weights* w = (orc_weights*)p;
    if (!w) return;
    free(w->w1f); free(w->w2f); free(w);
}

/* The whole forward, step by step: canonical sort and permutation
 * (orc_prepare), the expert MLP of every permuted row, in permuted order,
 * into O rows, then the finalize.  combine 0: out fp32 [T_cap][H] (orc_finalize);
 * 1: out bf16 bits [T_cap][H] (orc_finalize_bf16); 2: out fp32 [T_cap][k][H]
 * (orc_finalize_rows).  combine 0 or 1 with ORC_APPLY_TOPK_IN_FC1 added: the
 * probabilities multiply the SwiGLU rows (expert_row_p) and the finalize
 * sums the weighted rows (orc_finalize_sum).  Optional outputs: O_out [T*k][H] fp32 (permuted order)
 * and H_out [T*k][F] fp32 (the FC2 operand values).  Returns error bits. */
uint32_t orc_forward_ex(void* wp, const uint16_t* x, const int32_t* ids, const float* probs,
                        int64_t T_cap, int32_t live, int combine, void* out, float* O_out,
                        float* H_out)
{
    orc_weights* w = (orc_weights*)wp;
    const orc_model* m = &w->m;
    const int E = m->E, H = m->H, F = m->F, k = m->k;
    const int fc1_topk = (combine & ORC_APPLY_TOPK_IN_FC1) != 0;
    combine &= ~ORC_APPLY_TOPK_IN_FC1;
    int32_t T;
    int32_t* sorted_ids = (int32_t*)malloc(sizeof(int32_t) * (T_cap * k + 1));
    float* sorted_probs = (float*)malloc(sizeof(float) * (T_cap * k + 1));
    int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * E);
    int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (E + 1));
    int32_t* perm_src = (int32_t*)malloc(sizeof(int32_t) * (T_cap * k + 1));
    int32_t* dst = (int32_t*)malloc(sizeof(int32_t) * (T_cap * k + 1));
    uint32_t err = orc_prepare(ids, probs, T_cap, live, E, k, sorted_ids, sorted_probs,
                               counts, offsets, perm_src, dst, &T);
    int64_t nrows = offsets[E];
    double* xo = x_operands(x, T, H, m->mx);
    float* O = (float*)malloc(sizeof(float) * (nrows * H + 1));
#pragma omp parallel
    {
        float* a32 = (float*)malloc(sizeof(float) * F);
        double* hrow = (double*)malloc(sizeof(double) * F);
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < nrows; ++i) {
            int32_t r = perm_src[i];
            int32_t t = r / k;
            int32_t e = sorted_ids[r];
            expert_row_p(m, e, xo + (int64_t)t * H, O + i * H, a32, hrow,
                         fc1_topk ? sorted_probs[r] : 1.0f);
            if (H_out)
                for (int64_t n = 0; n < F; ++n) H_out[i * F + n] = (float)hrow[n];
        }
        free(a32); free(hrow);
    }
    if (fc1_topk)
        orc_finalize_sum(O, dst, T, k, H, combine == 1, out);
    else if (combine == 1)
        orc_finalize_bf16(O, dst, sorted_probs, T, k, H, (uint16_t*)out);
    else if (combine == 2)
        orc_finalize_rows(O, dst, T, k, H, (float*)out);
    else
        orc_finalize(O, dst, sorted_probs, T, k, H, (float*)out);
    if (O_out) memcpy(O_out, O, sizeof(float) * nrows * H);
    free(O); free(xo);
    free(sorted_ids); free(sorted_probs); free(counts); free(offsets); free(perm_src); free(dst);
    return err;
}

/* The forward with the fp32 combine (out fp32 [T_cap][H]). */
uint32_t orc_forward(void* wp, const uint16_t* x, const int32_t* ids, const float* probs,
                     int64_t T_cap, int32_t live, float* out, float* O_out, float* H_out)
{
    return orc_forward_ex(wp, x, ids, probs, T_cap, live, 0, out, O_out, H_out);
}

/* The naive per-token loop (no permutation): for each listed token, sort its
 * routes by id, run each route's expert MLP on the token's own row, and sum
 * the rows with the same fp32 fma chain.  out_rows is [n_tok][H].  Used to
 * pin the permutation bookkeeping of orc_forward, and to check sampled
 * tokens of large launches one by one. */
void orc_forward_tokens_ex(void* wp, const uint16_t* x, const int32_t* ids, const float* probs,
                           const int64_t* tokens, int64_t n_tok, int fc1_topk, float* out_rows);

void orc_forward_tokens(void* wp, const uint16_t* x, const int32_t* ids, const float* probs,
                        const int64_t* tokens, int64_t n_tok, float* out_rows)
{
    orc_forward_tokens_ex(wp, x, ids, probs, tokens, n_tok, 0, out_rows);
}

/* As orc_forward_tokens; with fc1_topk the probability is applied inside FC1
 * (expert_row_p) and the weighted rows are summed (orc_finalize_sum). */
void orc_forward_tokens_ex(void* wp, const uint16_t* x, const int32_t* ids, const float* probs,
                           const int64_t* tokens, int64_t n_tok, int fc1_topk, float* out_rows)
{
    orc_weights* w = (orc_weights*)wp;
    const orc_model* m = &w->m;
    const int E = m->E, H = m->H, F = m->F, k = m->k;
#pragma omp parallel
    {
        float* a32 = (float*)malloc(sizeof(float) * F);
        double* hrow = (double*)malloc(sizeof(double) * F);
        float* o = (float*)malloc(sizeof(float) * (int64_t)k * H);
        double* xr = (double*)malloc(sizeof(double) * H);
#pragma omp for schedule(dynamic, 1)
        for (int64_t q = 0; q < n_tok; ++q) {
            int64_t t = tokens[q];
            double* xo = x_operands(x + t * H, 1, H, m->mx);
            memcpy(xr, xo, sizeof(double) * H);
            free(xo);
            int32_t id[64];
            float p[64];
            for (int j = 0; j < k; ++j) { id[j] = ids[t * k + j]; p[j] = probs[t * k + j]; }
            for (int a = 1; a < k; ++a)
                for (int b = a; b > 0 && id[b - 1] > id[b]; --b) {
                    int32_t ti = id[b]; id[b] = id[b - 1]; id[b - 1] = ti;
                    float tp = p[b]; p[b] = p[b - 1]; p[b - 1] = tp;
                }
            int use[64];
            for (int j = 0; j < k; ++j)
                use[j] = id[j] >= 0 && id[j] < E && !(j > 0 && id[j] == id[j - 1]);
            for (int j = 0; j < k; ++j)
                if (use[j])
                    expert_row_p(m, id[j], xr, o + (int64_t)j * H, a32, hrow,
                                 fc1_topk ? p[j] : 1.0f);
            for (int64_t mo = 0; mo < H; ++mo) {
                float acc = 0.0f;
                for (int j = 0; j < k; ++j)
                    if (use[j])
                        acc = fc1_topk ? acc + o[(int64_t)j * H + mo]
                                       : fmaf(p[j], o[(int64_t)j * H + mo], acc);
                out_rows[q * H + mo] = acc;
            }
        }
        free(a32); free(hrow); free(o); free(xr);
    }
}

/* ------------------------------------------------------------------------ */
/* Kernel-weight buffer layout ([MEGA]: gate/up interleaved in blocks of 32, */
/* K-major), written from the layout's definition (see the C-ABI header):    */
/* rows interleaved, then tiled into MFMA operand blocks.                    */
/* ------------------------------------------------------------------------ */

/* Row order of the packed FC1 weight of one expert: packed row 64*b + i is
 * gate row 32*b + i for i < 32 and up row F + 32*b + (i - 32) for i >= 32.
 * FC2 rows keep their order. */
static int64_t fc1_logical_row(int64_t packed, int64_t F)
{
    int64_t b = packed / 64, i = packed % 64;
    return i < 32 ? 32 * b + i : F + 32 * b + (i - 32);
}

/* bf16 section of a weight with N rows of K elements per expert: 1 KB blocks
 * of 16 rows x 32 K; with c = n/16, s = k/32, KS = K/32, g = c/32 and
 * w = min(32, N/16 - 32g), element (e, n, k) sits at element index
 *   (e*(N/16)*KS + g*32*KS + s*w + c%32)*512 + ((k%32)/8)*128 + (n%16)*8 + k%8 . */
static int64_t bf16_index(int64_t e, int64_t n, int64_t k, int64_t N, int64_t K)
{
    const int64_t c = n / 16, s = k / 32, KS = K / 32, g = c / 32;
    const int64_t w = N / 16 - 32 * g < 32 ? N / 16 - 32 * g : 32;
    const int64_t block = e * (N / 16) * KS + g * 32 * KS + s * w + c % 32;
    return block * 512 + ((k % 32) / 8) * 128 + (n % 16) * 8 + k % 8;
}

static void pack_bf16_section(int E, int64_t N, int64_t K, int64_t F, int fc1,
                              const uint16_t* w, uint16_t* out)
{
    for (int64_t e = 0; e < E; ++e)
        for (int64_t n = 0; n < N; ++n) {
            int64_t src = fc1 ? fc1_logical_row(n, F) : n;
            for (int64_t k = 0; k < K; ++k)
                out[bf16_index(e, n, k, N, K)] = w[(e * N + src) * K + k];
        }
}

/* bf16 buffer: the FC1 section (N = 2F packed rows, K = H), then the FC2
 * section (N = H, K = F). */
void orc_pack_bf16(int E, int H, int F, const uint16_t* w1, const uint16_t* w2, uint8_t* kbuf)
{
    uint16_t* p1 = (uint16_t*)kbuf;
    uint16_t* p2 = p1 + (int64_t)E * 2 * F * H;
    pack_bf16_section(E, 2 * (int64_t)F, H, F, 1, w1, p1);
    pack_bf16_section(E, H, F, F, 0, w2, p2);
}

static int64_t up256(int64_t v) { return (v + 255) / 256 * 256; }
static int64_t ksteps(int64_t K) { return (K + 127) / 128; }
static int64_t code_bytes(int E, int64_t N, int64_t K) { return (int64_t)E * (N / 16) * ksteps(K) * 2048; }
static int64_t scale_bytes(int E, int64_t N, int64_t K) { return (int64_t)E * (N / 16) * ((ksteps(K) + 3) / 4) * 256; }

/* MXFP8 codes of a weight with N rows of K elements (KS = ceil(K/128)):
 *   (((e*(N/16) + n/16)*KS + k/128)*2 + (k%128)/64)*1024
 *     + ((k%64)/16*16 + n%16)*16 + k%16 ;
 * scales (KQ = ceil(KS/4)), for the 32-block b = k/32 of row n:
 *   ((e*(N/16) + n/16)*KQ + (b/4)/4)*256 + ((b%4)*16 + n%16)*4 + (b/4)%4 .
 * Bytes for k >= K are code 0 and scale 127 (2^0). */
static void pack_mx_section(int E, int64_t N, int64_t K, int64_t F, int fc1, const uint16_t* w,
                            uint8_t* codes, uint8_t* scales)
{
    int64_t KS = ksteps(K), KQ = (KS + 3) / 4;
    memset(codes, 0, code_bytes(E, N, K));
    memset(scales, 127, scale_bytes(E, N, K));
    float* row = (float*)malloc(sizeof(float) * K);
    uint8_t* c = (uint8_t*)malloc(K);
    uint8_t* sc = (uint8_t*)malloc(K / 32);
    for (int64_t e = 0; e < E; ++e)
        for (int64_t n = 0; n < N; ++n) {
            int64_t src = fc1 ? fc1_logical_row(n, F) : n;
            for (int64_t k = 0; k < K; ++k) row[k] = orc_bf16_value(w[(e * N + src) * K + k]);
            orc_mx_quantize(row, 1, K, c, sc);
            int64_t blk = e * (N / 16) + n / 16;
            for (int64_t k = 0; k < K; ++k)
                codes[((blk * KS + k / 128) * 2 + (k % 128) / 64) * 1024 +
                      ((k % 64) / 16 * 16 + n % 16) * 16 + k % 16] = c[k];
            for (int64_t b = 0; b < K / 32; ++b)
                scales[(blk * KQ + (b / 4) / 4) * 256 + ((b % 4) * 16 + n % 16) * 4 + (b / 4) % 4] =
                    sc[b];
        }
    free(row); free(c); free(sc);
}

/* MXFP8 buffer: FC1 codes, FC2 codes, FC1 scales, FC2 scales, each section
 * starting at a multiple of 256 bytes. */
void orc_pack_mxfp8(int E, int H, int F, const uint16_t* w1, const uint16_t* w2, uint8_t* kbuf)
{
    int64_t c1 = up256(code_bytes(E, 2 * (int64_t)F, H)), c2 = up256(code_bytes(E, H, F));
    int64_t s1 = up256(scale_bytes(E, 2 * (int64_t)F, H));
    pack_mx_section(E, 2 * (int64_t)F, H, F, 1, w1, kbuf, kbuf + c1 + c2);
    pack_mx_section(E, H, F, F, 0, w2, kbuf + c1, kbuf + c1 + c2 + s1);
}

/* MXFP4 codes of a weight with N rows of K elements: one 1 KB block per 16
 * rows x 128 K, lane (k%128)/32*16 + n%16 holding K (k%128)/32*32 + [0, 32)
 * of row n as 16 bytes, two codes per byte, the lower K in the low nibble.
 * The blocks of an expert are in 512-row groups: with c = n/16, g = c/32 and
 * w = min(32, N/16 - 32g) (the width of c's group), block (c, t = k/128) is
 * block number e*(N/16)*KS + g*32*KS + t*w + c%32, so code (e, n, k) is in
 *   byte (that block)*1024 + ((k%128)/32*16 + n%16)*16 + (k%32)/2, nibble k%2.
 * The 256-byte scale groups (4 K steps each, the MXFP8 arrangement inside)
 * follow the same grouping with KQ for KS and the group number Q = b/16 of
 * 32-block b for t: byte (e*(N/16)*KQ + g*32*KQ + Q*w + c%32)*256
 * + ((b%4)*16 + n%16)*4 + (b/4)%4.  Codes for k >= K are 0, scales 127. */
static int64_t code4_bytes(int E, int64_t N, int64_t K) { return (int64_t)E * (N / 16) * ksteps(K) * 1024; }

/* block number of column block c, step (or scale group) t in an expert's
 * section of nt column blocks and nsteps steps, 512-row grouping */
static int64_t mx4_block(int64_t e, int64_t c, int64_t t, int64_t nt, int64_t nsteps)
{
    const int64_t g = c / 32;
    const int64_t w = nt - 32 * g < 32 ? nt - 32 * g : 32;
    return e * nt * nsteps + g * 32 * nsteps + t * w + c % 32;
}

static void pack_mx4_section(int E, int64_t N, int64_t K, int64_t F, int fc1, const uint16_t* w,
                             uint8_t* codes, uint8_t* scales)
{
    int64_t KS = ksteps(K), KQ = (KS + 3) / 4;
    memset(codes, 0, code4_bytes(E, N, K));
    memset(scales, 127, scale_bytes(E, N, K));
    float* row = (float*)malloc(sizeof(float) * K);
    uint8_t* c = (uint8_t*)malloc(K);
    uint8_t* sc = (uint8_t*)malloc(K / 32);
    for (int64_t e = 0; e < E; ++e)
        for (int64_t n = 0; n < N; ++n) {
            int64_t src = fc1 ? fc1_logical_row(n, F) : n;
            for (int64_t k = 0; k < K; ++k) row[k] = orc_bf16_value(w[(e * N + src) * K + k]);
            orc_mx4_quantize(row, 1, K, c, sc);
            const int64_t nt = N / 16;
            for (int64_t k = 0; k < K; ++k)
                codes[mx4_block(e, n / 16, k / 128, nt, KS) * 1024 + ((k % 128) / 32 * 16 + n % 16) * 16 +
                      (k % 32) / 2] |= (uint8_t)(c[k] << (4 * (k % 2)));
            for (int64_t b = 0; b < K / 32; ++b)
                scales[mx4_block(e, n / 16, b / 16, nt, KQ) * 256 + ((b % 4) * 16 + n % 16) * 4 + (b / 4) % 4] =
                    sc[b];
        }
    free(row); free(c); free(sc);
}

/* MXFP4 buffer: FC1 codes, FC2 codes, FC1 scales, FC2 scales, each section
 * starting at a multiple of 256 bytes. */
void orc_pack_mxfp4(int E, int H, int F, const uint16_t* w1, const uint16_t* w2, uint8_t* kbuf)
{
    int64_t c1 = up256(code4_bytes(E, 2 * (int64_t)F, H)), c2 = up256(code4_bytes(E, H, F));
    int64_t s1 = up256(scale_bytes(E, 2 * (int64_t)F, H));
    pack_mx4_section(E, 2 * (int64_t)F, H, F, 1, w1, kbuf, kbuf + c1 + c2);
    pack_mx4_section(E, H, F, F, 0, w2, kbuf + c1, kbuf + c1 + c2 + s1);
}

int64_t orc_pack_bytes(int E, int H, int F, int mx)
{
    int64_t n1 = (int64_t)E * 2 * F * H, n2 = (int64_t)E * H * F;
    if (!mx) return 2 * (n1 + n2);
    if (mx == 2)
        return up256(code4_bytes(E, 2 * (int64_t)F, H)) + up256(code4_bytes(E, H, F)) +
               up256(scale_bytes(E, 2 * (int64_t)F, H)) + up256(scale_bytes(E, H, F));
    return up256(code_bytes(E, 2 * (int64_t)F, H)) + up256(code_bytes(E, H, F)) +
           up256(scale_bytes(E, 2 * (int64_t)F, H)) + up256(scale_bytes(E, H, F));
}

/* Section offsets of the MXFP8 buffer: FC1 codes, FC2 codes, FC1 scales,
 * FC2 scales, and the end. */
void orc_pack_mx4_offsets(int E, int H, int F, int64_t* off)
{
    off[0] = 0;
    off[1] = up256(code4_bytes(E, 2 * (int64_t)F, H));
    off[2] = off[1] + up256(code4_bytes(E, H, F));
    off[3] = off[2] + up256(scale_bytes(E, 2 * (int64_t)F, H));
    off[4] = off[3] + up256(scale_bytes(E, H, F));
}

void orc_pack_mx_offsets(int E, int H, int F, int64_t* off)
{
    off[0] = 0;
    off[1] = up256(code_bytes(E, 2 * (int64_t)F, H));
    off[2] = off[1] + up256(code_bytes(E, H, F));
    off[3] = off[2] + up256(scale_bytes(E, 2 * (int64_t)F, H));
    off[4] = off[3] + up256(scale_bytes(E, H, F));
}

/* Host threads of the OpenMP loops (timing aid for the CPU baseline, no part
 * of the method): n > 0 sets the count; returns the count in effect. */
int orc_set_threads(int n)
{
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
}
