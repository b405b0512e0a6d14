/*
 * ckv_oracle.c -- CPU oracle for certified quantized-KV decode attention.
 *
 * TEST INFRASTRUCTURE ONLY (see ckv_oracle.h).  Plain and slow on purpose:
 * each head is computed on its own, with full sorts where the method says
 * "order" and FP64 for every value; heads run on OpenMP threads, which
 * changes no result.  Built with -O2 -fno-fast-math -ffp-contract=off so
 * that every FP32 operation is the single IEEE operation written here.
 *
 * Section tags ([Meth-1] ...) refer to the page "Runtime-Certified
 * Bounded-Error Quantized Attention", technical summary; they are listed in
 * ckv_oracle.h.  Where the page leaves a step open, the reading taken is
 * stated at the step.
 */
#include "ckv_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_mutation = 0;

/* ------------------------------------------------------------------------ */
/* IEEE binary16 helpers                                                    */
/* ------------------------------------------------------------------------ */

/* binary16 -> binary32, exact (every half is a float). */
float orc_h2f(uint16_t h)
{
    int sign = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    float v;
    if (e == 0)
        v = ldexpf((float)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexpf((float)(m | 1024), e - 25);
    return sign ? -v : v;
}

/* Smallest non-negative binary16 that is >= x (x >= 0): rounding upward.
 * Positive halves are ordered like their bit patterns, so a bisection over
 * the patterns 0x0000..0x7C00 (the last is +inf) finds it. */
uint16_t orc_f2h_up(float x)
{
    if (!(x > 0.0f))
        return 0;
    unsigned lo = 0, hi = 0x7C00; /* orc_h2f(hi) >= x always */
    while (lo < hi) {
        unsigned mid = (lo + hi) / 2;
        if (orc_h2f((uint16_t)mid) >= x)
            hi = mid;
        else
            lo = mid + 1;
    }
    return (uint16_t)lo;
}

/* binary64 -> binary32 rounded upward. */
float orc_ru32(double x)
{
    float f = (float)x;
    if ((double)f < x)
        f = nextafterf(f, INFINITY);
    return f;
}

/* ------------------------------------------------------------------------ */
/* Canonical exponential used on every decision path.                       */
/* exp(x) for x <= 0: k = rint(x * log2(e)), r = x - k*ln2 in two steps     */
/* (Cody & Waite, "Software Manual for the Elementary Functions", 1980),    */
/* e^r by its degree-7 Taylor polynomial in Horner form, result r * 2^k.    */
/* Results below 2^-125 are flushed to 0 so that no subnormal is formed.    */
/* ------------------------------------------------------------------------ */
float orc_exp_c(float x)
{
    const float L2E = 0x1.715476p+0f;   /* log2(e) rounded to binary32 */
    const float LN2A = 0x1.62e4p-1f;    /* leading bits of ln 2        */
    const float LN2B = 0x1.7f7d1cp-20f; /* ln 2 - LN2A, rounded        */
    float y = x * L2E;
    float k = rintf(y);
    if (k < -125.0f)
        return 0.0f;
    float r = fmaf(-k, LN2A, x);
    r = fmaf(-k, LN2B, r);
    /* 1/j! for j = 7..0, each rounded to binary32 */
    float p = 0x1.a01a02p-13f;
    p = fmaf(p, r, 0x1.6c16c2p-10f);
    p = fmaf(p, r, 0x1.111112p-7f);
    p = fmaf(p, r, 0x1.555556p-5f);
    p = fmaf(p, r, 0x1.555556p-3f);
    p = fmaf(p, r, 0x1.0p-1f);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    return ldexpf(p, (int)k);
}

/* Halving-tree sum: for stride n/2, n/4, .., 1: a[i] += a[i + stride]. */
static float tree_f32(float *a, int n)
{
    for (int s = n / 2; s >= 1; s /= 2)
        for (int i = 0; i < s; i++)
            a[i] = a[i] + a[i + s];
    return a[0];
}

static double tree_f64(double *a, int n)
{
    for (int s = n / 2; s >= 1; s /= 2)
        for (int i = 0; i < s; i++)
            a[i] = a[i] + a[i + s];
    return a[0];
}

/* ------------------------------------------------------------------------ */
/* Upper bounds of e^x, e^x - 1 and tanh(x/2) for x >= 0, from +,-,*,/ only */
/* (so that every platform evaluates them to the same bits).                */
/* ------------------------------------------------------------------------ */

/* e^x <= expu(x).  x is halved j times (exactly) to r <= 1/16, e^r from its
 * Taylor series to degree 12 (remainder < 2^-60 relative), squared j times;
 * the factor (1 + 2^-36) covers the rounding of at most 10 squarings. */
double orc_expu(double x)
{
    if (!(x <= 64.0))
        return INFINITY;
    if (x <= 0.0)
        x = 0.0;
    int j = 0;
    double r = x;
    while (r > 0.0625) {
        r *= 0.5;
        j++;
    }
    double p = 1.0 / 479001600.0; /* 1/12! */
    double f = 479001600.0;
    for (int i = 11; i >= 0; i--) {
        f = f / (double)(i + 1); /* f = i! */
        p = fma(p, r, 1.0 / f);
    }
    for (int i = 0; i < j; i++)
        p = p * p;
    return p * (1.0 + 0x1p-36);
}

/* e^x - 1 <= em1u(x).  Series to degree 16 below 1/2, else expu(x) - 1. */
double orc_em1u(double x)
{
    if (!(x > 0.0))
        return 0.0;
    if (x > 64.0)
        return INFINITY;
    if (x <= 0.5) {
        /* x * sum_{i=0..15} x^i / (i+1)! */
        double c[16];
        double f = 1.0;
        for (int i = 0; i < 16; i++) {
            f = f * (double)(i + 1);
            c[i] = 1.0 / f;
        }
        double p = c[15];
        for (int i = 14; i >= 0; i--)
            p = fma(p, x, c[i]);
        return x * p * (1.0 + 0x1p-48);
    }
    return (orc_expu(x) - 1.0) * (1.0 + 0x1p-50);
}

/* tanh(x/2) = m / (m + 2) with m = e^x - 1, increasing in m. */
double orc_tanhu(double x)
{
    double m = orc_em1u(x);
    if (isinf(m))
        return 1.0;
    double t = m / (m + 2.0) * (1.0 + 0x1p-48);
    return t < 1.0 ? t : 1.0;
}

/* Bound terms in unsigned fixed point with 32 fraction bits, rounded up and
 * capped; a capped term makes the sum it enters "unbounded". */
#define FX_CAP ((uint64_t)1 << 46)
uint64_t orc_fx(double t)
{
    if (!(t < 16384.0))
        return FX_CAP;
    if (t <= 0.0)
        return 0;
    double v = ceil(t * 4294967296.0);
    uint64_t u = (uint64_t)v;
    return u < FX_CAP ? u : FX_CAP;
}

static double fx_to_bound(uint64_t sum, int saturated)
{
    if (saturated)
        return INFINITY;
    return (double)sum * 0x1p-32 * (1.0 + 0x1p-50);
}

/* ------------------------------------------------------------------------ */
/* Tier 1: quantization [Meth-1]                                            */
/* Reading: INT8 key scale/offset per channel per 64-token block; INT4      */
/* value scale/offset per token per 32-channel group; both affine with      */
/* offset = min (exact in FP16) and scale = (max - min)/levels rounded up   */
/* to FP16, so that no code is clamped and |x - x^| <= scale * (1/2 + eps). */
/* ------------------------------------------------------------------------ */
static uint16_t scale_for(float lo, float hi, float levels)
{
    float r = hi - lo;
    if (r == 0.0f)
        return 0;
    return orc_f2h_up(r / levels);
}

static int code_for(float x, float lo, float s, int maxcode)
{
    if (s == 0.0f)
        return 0;
    float c = rintf((x - lo) / s);
    if (c < 0.0f)
        c = 0.0f;
    if (c > (float)maxcode)
        c = (float)maxcode;
    return (int)c;
}

/* k: [64][d] FP16 of one block and one kv head. */
void orc_quant_k_block(int d, const uint16_t *k, uint8_t *code, uint16_t *s, uint16_t *z)
{
    for (int c = 0; c < d; c++) {
        float lo = orc_h2f(k[c]), hi = lo;
        for (int t = 1; t < ORC_BT; t++) {
            float x = orc_h2f(k[t * d + c]);
            if (x < lo)
                lo = x;
            if (x > hi)
                hi = x;
        }
        uint16_t sh = scale_for(lo, hi, 255.0f);
        /* the minimum is itself an FP16 value: store its bits */
        uint16_t zh = 0;
        for (int t = 0; t < ORC_BT; t++)
            if (orc_h2f(k[t * d + c]) == lo) {
                zh = k[t * d + c];
                break;
            }
        if (lo == 0.0f)
            zh = 0; /* +0 and -0 compare equal; store +0 */
        s[c] = sh;
        z[c] = zh;
        float sf = orc_h2f(sh);
        for (int t = 0; t < ORC_BT; t++)
            code[t * d + c] = (uint8_t)code_for(orc_h2f(k[t * d + c]), lo, sf, 255);
    }
}

/* v: [64][d] FP16.  eta = max |v - (z + s*code)| over the block, exact in
 * FP64 and rounded up to FP32 (reading of the per-block annotation).
 * bits = 4: the design's INT4 values, two codes per byte (low nibble = even
 * channel), [64][d/2]; bits = 8: the symmetric cache configuration of
 * [Results] (values at the keys' width; reading: the same per-token groups
 * of 32 channels, 255 levels), one code per byte, [64][d]. */
void orc_quant_v_block_bits(int d, int bits, const uint16_t *v, uint8_t *code, uint16_t *s, uint16_t *z,
                            float *eta)
{
    int ng = d / ORC_VG;
    const int levels = bits == 8 ? 255 : 15;
    double emax = 0.0;
    memset(code, 0, (size_t)ORC_BT * d * bits / 8);
    for (int t = 0; t < ORC_BT; t++) {
        for (int g = 0; g < ng; g++) {
            const uint16_t *row = v + (size_t)t * d + g * ORC_VG;
            float lo = orc_h2f(row[0]), hi = lo;
            uint16_t zh = row[0];
            for (int c = 1; c < ORC_VG; c++) {
                float x = orc_h2f(row[c]);
                if (x < lo) {
                    lo = x;
                    zh = row[c];
                }
                if (x > hi)
                    hi = x;
            }
            if (lo == 0.0f)
                zh = 0;
            uint16_t sh = scale_for(lo, hi, (float)levels);
            s[t * ng + g] = sh;
            z[t * ng + g] = zh;
            float sf = orc_h2f(sh);
            for (int c = 0; c < ORC_VG; c++) {
                float x = orc_h2f(row[c]);
                int q = code_for(x, lo, sf, levels);
                int ch = g * ORC_VG + c;
                if (bits == 8)
                    code[(size_t)t * d + ch] = (uint8_t)q;
                else
                    code[(size_t)t * (d / 2) + ch / 2] |= (uint8_t)((ch & 1) ? (q << 4) : q);
                double rec = (double)lo + (double)sf * (double)q;
                double e = fabs((double)x - rec);
                if (e > emax)
                    emax = e;
            }
        }
    }
    *eta = orc_ru32(emax);
}

void orc_quant_v_block(int d, const uint16_t *v, uint8_t *code, uint16_t *s, uint16_t *z, float *eta)
{
    orc_quant_v_block_bits(d, 4, v, code, s, z, eta);
}

/* ------------------------------------------------------------------------ */
/* INT8 scoring pass [Meth-3, adaptive top-K selection]                     */
/* Reading (the page gives no arithmetic for the cheap INT8 first pass):   */
/* an exact integer dot product of rounded weights.  w_c = q_c s_c is exact */
/* in FP32; with e = floor(log2 max_c |w_c|) the weights are rounded to     */
/* integers w~_c = rint(w_c 2^(20-e)), |w~_c| <= 2^21; S_t = sum_c w~_c     */
/* code_tc exactly; s^_t = fl32(fl64(C + S_t 2^(e-20)) * sm) with C the      */
/* halving-tree FP32 sum of q_c z_c.  No summation order enters S_t.        */
/* ------------------------------------------------------------------------ */

/* e = floor(log2 max_c |w_c|); returns 0 when every w_c is 0. */
static int weight_exponent(int d, const float *w, int *e)
{
    float W = 0.0f;
    for (int c = 0; c < d; c++)
        if (fabsf(w[c]) > W)
            W = fabsf(w[c]);
    if (W == 0.0f)
        return 0;
    *e = ilogbf(W);
    return 1;
}

void orc_score_q8(int d, const uint16_t *q, const uint8_t *code, const uint16_t *s,
                  const uint16_t *z, float sm, float *out)
{
    float w[256], cz[256];
    int64_t wt[256];
    for (int c = 0; c < d; c++) {
        w[c] = orc_h2f(q[c]) * orc_h2f(s[c]);
        cz[c] = orc_h2f(q[c]) * orc_h2f(z[c]);
    }
    float C = tree_f32(cz, d);
    int e = 0;
    int nz = weight_exponent(d, w, &e);
    for (int c = 0; c < d; c++)
        wt[c] = nz ? (int64_t)rintf(ldexpf(w[c], 20 - e)) : 0;
    for (int t = 0; t < ORC_BT; t++) {
        int64_t S = 0;
        for (int c = 0; c < d; c++)
            S += wt[c] * (int64_t)code[t * d + c];
        double x = (double)C + ldexp((double)S, e - 20);
        out[t] = (float)(x * (double)sm);
    }
}

/* FP16-key score: an FP64 fma chain over c of q_c * k_c (each product is
 * exact), times sm in FP64, rounded once to FP32. */
void orc_score_f16(int d, const uint16_t *q, const uint16_t *k, int n, float sm, float *out)
{
    for (int t = 0; t < n; t++) {
        double a = 0.0;
        for (int c = 0; c < d; c++)
            a = fma((double)orc_h2f(q[c]), (double)orc_h2f(k[t * d + c]), a);
        out[t] = (float)(a * (double)sm);
    }
}

/* ------------------------------------------------------------------------ */
/* Bound Delta on each token's INT8 score error [Meth-2, the E_key term]   */
/* from the query and the quantization scales (tracked quantities only).    */
/* With H = sum |q_c| s_c, A = sum |q_c| (|z_c| + 255 s_c) and              */
/* E_w = 2^(e-21) 255 d (the weight rounding: at most half a unit of         */
/* 2^(e-20) per channel, times codes <= 255; 0 when every w_c is 0):         */
/*   |s^ - s| <= Delta = sm (kappa H + E_w + (2^-20 + 2^-23) A + 2^-23 E_w)  */
/*   |s~ - s| <= rho   = sm 2^-23 A                   (FP16 key score)      */
/* kappa = 1/2 + 2^-14 covers the code rounding; 2^-20 A covers the tree    */
/* sum of C (depth <= 7, < 2^-20 relative); 2^-23 (A + E_w) the roundings    */
/* of the final FP64 sum, scale and FP32 conversion.  The FP16 chain runs   */
/* in FP64 and is rounded once to FP32 (2^-24 + (d+3) 2^-53 < 2^-23).        */
/* |k| <= |z| + 255 s for every key of the block, so A bounds sum |q_c k_c|. */
/* Sums are FP64 halving trees; (1 + 2^-20) covers the FP64 rounding;       */
/* results rounded up to FP32.                                              */
/* ------------------------------------------------------------------------ */
void orc_delta_rho(int d, const uint16_t *q, const uint16_t *s, const uint16_t *z, float sm,
                   float *delta, float *rho)
{
    double hv[256], av[256];
    float w[256];
    for (int c = 0; c < d; c++) {
        double aq = fabs((double)orc_h2f(q[c]));
        double sc = (double)orc_h2f(s[c]);
        double zc = fabs((double)orc_h2f(z[c]));
        hv[c] = aq * sc;
        av[c] = aq * (zc + 255.0 * sc);
        w[c] = orc_h2f(q[c]) * orc_h2f(s[c]);
    }
    double H = tree_f64(hv, d);
    double A = tree_f64(av, d);
    int e = 0;
    double Ew = weight_exponent(d, w, &e) ? ldexp(255.0 * (double)d, e - 21) : 0.0;
    double kappa = 0.5 + 0x1p-14;
    double dl = kappa * H + Ew;
    dl = dl + A * (0x1p-20 + 0x1p-23);
    dl = dl + Ew * 0x1p-23;
    dl = dl * (double)sm;
    dl = dl * (1.0 + 0x1p-20);
    double rh = A * 0x1p-23;
    rh = rh * (double)sm;
    rh = rh * (1.0 + 0x1p-20);
    if (orc_mutation & 2)
        dl *= 0.5;
    *delta = orc_ru32(dl);
    *rho = orc_ru32(rh);
}

/* rho for the FP16 tokens of a partial block: A = sum |q_c| max_t |k_tc|. */
static float rho_partial(int d, const uint16_t *q, const uint16_t *k, int n, float sm)
{
    double av[256];
    for (int c = 0; c < d; c++) {
        double m = 0.0;
        for (int t = 0; t < n; t++) {
            double x = (orc_mutation & 128) ? (double)orc_h2f(k[t * d + c]) : fabs((double)orc_h2f(k[t * d + c]));
            if (x > m)
                m = x;
        }
        av[c] = fabs((double)orc_h2f(q[c])) * m;
    }
    double A = tree_f64(av, d);
    double rh = A * 0x1p-23;
    rh = rh * (double)sm;
    rh = rh * (1.0 + 0x1p-20);
    return orc_ru32(rh);
}

/* Block estimate: max score and l = halving-tree sum over 64 slots of
 * exp_c(s_t - max); slots beyond n hold 0. */
void orc_block_est(const float *sc, int n, float *mx, float *l)
{
    float m = sc[0];
    for (int t = 1; t < n; t++)
        if (sc[t] > m)
            m = sc[t];
    float e[ORC_BT];
    for (int t = 0; t < ORC_BT; t++)
        e[t] = t < n ? orc_exp_c(sc[t] - m) : 0.0f;
    *mx = m;
    *l = tree_f32(e, ORC_BT);
}

/* ------------------------------------------------------------------------ */
/* Selection by order (value desc, index asc)                               */
/* ------------------------------------------------------------------------ */
typedef struct {
    uint64_t v;
    int b;
} vb_t;

static int cmp_vb_desc(const void *x, const void *y)
{
    const vb_t *a = (const vb_t *)x, *b = (const vb_t *)y;
    if (a->v != b->v)
        return a->v > b->v ? -1 : 1;
    return a->b < b->b ? -1 : (a->b > b->b);
}

/* value ascending, index ascending: only for the rung-2 order mutation */
static int cmp_vb_asc(const void *x, const void *y)
{
    const vb_t *a = (const vb_t *)x, *b = (const vb_t *)y;
    if (a->v != b->v)
        return a->v < b->v ? -1 : 1;
    return a->b < b->b ? -1 : (a->b > b->b);
}

int orc_select(int n, const uint64_t *m, uint64_t need, uint8_t *in_set)
{
    memset(in_set, 0, (size_t)n);
    if (need == 0)
        return 0;
    vb_t *o = (vb_t *)malloc(sizeof(vb_t) * (size_t)(n > 0 ? n : 1));
    for (int b = 0; b < n; b++) {
        o[b].v = m[b];
        o[b].b = b;
    }
    qsort(o, (size_t)n, sizeof(vb_t), cmp_vb_desc);
    uint64_t acc = 0;
    int k = 0;
    while (k < n && acc < need) {
        acc += o[k].v;
        in_set[o[k].b] = 1;
        k++;
    }
    free(o);
    return k;
}

int64_t orc_discordant(int n, const uint64_t *key_a, const uint64_t *key_b)
{
    int64_t D = 0;
    for (int i = 0; i < n; i++)
        for (int j = i + 1; j < n; j++)
            if ((key_a[i] > key_a[j]) != (key_b[i] > key_b[j]))
                D++;
    return D;
}

/* ------------------------------------------------------------------------ */
/* The plan of one q head: selection, the two-term bound and rungs 1-2,      */
/* computed before paging from INT8-side quantities only [Contrib].          */
/* ------------------------------------------------------------------------ */
typedef struct {
    int N, has_part;
    const float *bmax, *bl, *delta, *rho, *eta; /* [Np] (eta: [N]) */
    double R;                                   /* range of V */
    /* results */
    float mref;
    uint64_t *M; /* [Np] */
    uint64_t S;
    uint8_t *inP, *inVP; /* [N] */
    uint64_t *cval;      /* [N] E_val contribution of each block */
    int kstar, nvp, widened, cap_fail;
    double tau, mu, tv, ekey, eval;
} plan_t;

static double phat_up(uint64_t Mb, uint64_t S)
{
    return ((double)(Mb + 1) / (double)S) * (1.0 + 0x1p-16);
}

/* Bound on the mass of block b under the certified scores relative to its
 * INT8 estimate: p~_b <= phat_b * F * X_b, F = exp(max_{P} (Delta + rho)),
 * X_b = exp(Delta_b + rho_b) on P, 1 on the tail. */
static double factor_F(const plan_t *p)
{
    double mx = 0.0;
    for (int b = 0; b < p->N; b++)
        if (p->inP[b]) {
            double f = (double)p->delta[b] + (double)p->rho[b];
            if (f > mx)
                mx = f;
        }
    return orc_expu(mx);
}

static double factor_X(const plan_t *p, int b)
{
    return p->inP[b] ? orc_expu((double)p->delta[b] + (double)p->rho[b]) : 1.0;
}

/* E_key [Meth-2]: TV(p~, p) <= mu / (1 - mu), mu = sum_b p~_b (e^delta_b - 1),
 * and TV <= tanh(delta_max / 2); the output error is at most TV * range(V)
 * because sum (p~ - p) = 0.  delta_b = rho on P (FP16 keys), Delta on the
 * tail (INT8 keys). */
static void key_bound(plan_t *p)
{
    double F = factor_F(p);
    uint64_t sum = 0;
    int sat = 0;
    double dmax = 0.0;
    for (int b = 0; b < p->N; b++) {
        double dl = p->inP[b] ? (double)p->rho[b] : (double)p->delta[b];
        double t = phat_up(p->M[b], p->S) * F * factor_X(p, b) * orc_em1u(dl) * (1.0 + 0x1p-48);
        uint64_t u = orc_fx(t);
        sat |= (u == FX_CAP);
        sum += u;
        if (dl > dmax)
            dmax = dl;
    }
    if (p->has_part) {
        double dl = (double)p->rho[p->N];
        double t = phat_up(p->M[p->N], p->S) * F * 1.0 * orc_em1u(dl) * (1.0 + 0x1p-48);
        uint64_t u = orc_fx(t);
        sat |= (u == FX_CAP);
        sum += u;
        if (dl > dmax)
            dmax = dl;
    }
    double mu = fx_to_bound(sum, sat);
    double tv = 1.0;
    if (mu < 1.0)
        tv = mu / (1.0 - mu) * (1.0 + 0x1p-48);
    double th = orc_tanhu(dmax);
    if (th < tv)
        tv = th;
    if (tv > 1.0)
        tv = 1.0;
    p->mu = mu;
    p->tv = tv;
    p->ekey = tv * p->R * (1.0 + 0x1p-50);
}

/* E_val contribution of block b [Meth-2]: p~_b * eta_b, bounded by
 * phat_b * F * X_b * eta_b. */
static uint64_t val_term(const plan_t *p, double F, int b)
{
    double e = (double)p->eta[b];
    if (orc_mutation & 1)
        e = 0.0;
    double t = phat_up(p->M[b], p->S) * F * factor_X(p, b) * e * (1.0 + 0x1p-48);
    return orc_fx(t);
}

static void plan_head(plan_t *p, const orc_thresholds *th)
{
    int N = p->N, Np = N + p->has_part;
    /* estimated masses */
    float mref = p->bmax[0];
    for (int b = 1; b < Np; b++)
        if (p->bmax[b] > mref)
            mref = p->bmax[b];
    p->mref = mref;
    uint64_t S = 0;
    for (int b = 0; b < Np; b++) {
        float mh = p->bl[b] * orc_exp_c(p->bmax[b] - mref);
        p->M[b] = (uint64_t)((double)mh * 4294967296.0);
        S += p->M[b];
    }
    p->S = S;
    uint64_t Mpart = p->has_part ? p->M[N] : 0;

    /* top-K* covering tau of the estimated mass, rung 1 widening [Meth-3].
     * Reading: widen while E_key > k_tol by halving the uncovered target,
     * at most n_widen times; still above k_tol escalates to rung 4. */
    double tau = (double)th->tau_cov;
    p->widened = 0;
    p->cap_fail = 0;
    for (int w = 0;; w++) {
        uint64_t T = (uint64_t)ceil(tau * (double)S);
        uint64_t need = T > Mpart ? T - Mpart : 0;
        p->kstar = orc_select(N, p->M, need, p->inP);
        key_bound(p);
        if (!(p->ekey > (double)th->k_tol))
            break;
        if (w >= th->n_widen) {
            p->cap_fail = 1;
            break;
        }
        tau = 1.0 - (1.0 - tau) * ((orc_mutation & 64) ? (1.0 / 3.0) : 0.5);
        p->widened = 1;
    }
    p->tau = tau;

    /* E_val and rung 2: promote FP16 values of the blocks with the largest
     * bounded contribution (order: contribution desc, index asc) until
     * E_val <= v_tol.  Reading: no cap by default (promoting more values
     * always pages less than a dense recompute); a caller-set cap that is
     * too small escalates to rung 4. */
    double F = factor_F(p);
    uint64_t *cb = p->cval;
    for (int b = 0; b < N; b++)
        cb[b] = val_term(p, F, b);
    vb_t *o = (vb_t *)malloc(sizeof(vb_t) * (size_t)(N > 0 ? N : 1));
    for (int b = 0; b < N; b++) {
        o[b].v = cb[b];
        o[b].b = b;
    }
    qsort(o, (size_t)N, sizeof(vb_t), (orc_mutation & 32) ? cmp_vb_asc : cmp_vb_desc);
    /* suffix sums: rest[k] = sum of o[k..N) */
    memset(p->inVP, 0, (size_t)N);
    int k = 0;
    for (;; k++) {
        uint64_t rest = 0;
        int sat = 0;
        for (int i = k; i < N; i++) {
            rest += o[i].v;
            sat |= (o[i].v == FX_CAP);
        }
        double ev = fx_to_bound(rest, sat);
        if (!(ev > (double)th->v_tol) || k == N) {
            p->eval = ev;
            break;
        }
    }
    for (int i = 0; i < k; i++)
        p->inVP[o[i].b] = 1;
    p->nvp = k;
    int vcap = th->v_cap_blocks > 0 ? th->v_cap_blocks : N;
    if (k > vcap || p->eval > (double)th->v_tol)
        p->cap_fail = 1;
    free(o);
}

/* ------------------------------------------------------------------------ */
/* Exact dense attention (FP64) [Signif: "FP16 reference"; Meth-1 fallback]  */
/* ------------------------------------------------------------------------ */
void orc_dense_head(int T, int Hkv, int d, int g, const uint16_t *k, const uint16_t *v,
                    const uint16_t *q, double sm, double *out)
{
    double *s = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    double mx = -INFINITY;
    for (int t = 0; t < T; t++) {
        const uint16_t *kt = k + ((size_t)t * Hkv + g) * d;
        double a = 0.0;
        for (int c = 0; c < d; c++)
            a += (double)orc_h2f(q[c]) * (double)orc_h2f(kt[c]);
        s[t] = sm * a;
        if (s[t] > mx)
            mx = s[t];
    }
    double den = 0.0;
    for (int c = 0; c < d; c++)
        out[c] = 0.0;
    for (int t = 0; t < T; t++) {
        double p = exp(s[t] - mx);
        den += p;
        const uint16_t *vt = v + ((size_t)t * Hkv + g) * d;
        for (int c = 0; c < d; c++)
            out[c] += p * (double)orc_h2f(vt[c]);
    }
    for (int c = 0; c < d; c++)
        out[c] /= den;
    free(s);
}

/* ------------------------------------------------------------------------ */
/* The decode step                                                          */
/* The work of one sequence runs in phases, each a loop over kv heads or q  */
/* heads whose iterations touch disjoint outputs; with OpenMP the           */
/* iterations run on threads.  The arithmetic of each head is the same      */
/* sequence of operations whatever the thread count.                        */
/* ------------------------------------------------------------------------ */
void orc_set_threads(int n)
{
#ifdef _OPENMP
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}

int orc_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

int orc_certified_decode(int B, int T, int Hq, int Hkv, int d, const uint16_t *K,
                         const uint16_t *V, const uint16_t *q, const orc_thresholds *th,
                         double *out, orc_report *rep, orc_trace *tr)
{
    return orc_certified_decode_vb(B, T, Hq, Hkv, d, 4, K, V, q, th, out, rep, tr);
}

/* Sizes and per-sequence arrays shared by the phases of one sequence. */
typedef struct {
    int T, Hq, Hkv, d, G, N, np, has_part, Np, ng, v_bits;
    size_t vcb, nb;
    const uint16_t *Kn, *Vn; /* [T][Hkv][d] of the sequence */
    const orc_thresholds *th;
    /* tier 1 per kv head */
    uint8_t *kc, *vc;        /* [Hkv][nb][64][d], [Hkv][nb][64][vcb] */
    uint16_t *ks, *kz;       /* [Hkv][nb][d] */
    uint16_t *vs, *vz;       /* [Hkv][nb][64][ng] */
    float *eta, *vrange;     /* [Hkv][nb], [Hkv] */
    /* per q head */
    plan_t *plans;                        /* [Hq] */
    float *bmax, *bl, *dl, *rh, *sc;      /* [Hq][Np] ([Hq][Np*64] for sc) */
    uint64_t *M, *cval;                   /* [Hq][Np], [Hq][nb] */
    uint8_t *inP, *inVP;                  /* [Hq][nb] */
    float *smix;                          /* [Hq][Np*64] certified scores */
    double *odense, *ocert;               /* [Hq][d] */
    int64_t *D;                           /* [Hq] discordant pairs */
    int *rank_ok;                         /* [Hq] */
} seq_t;

/* Phase 1, per kv head g: quantize every full block [Meth-1] and take the
 * value range R_g over all tokens ("value ranges" of [Meth-2]). */
static void kv_head_tier1(const seq_t *S, int n, int g, orc_trace *tr)
{
    const int d = S->d, Hkv = S->Hkv, N = S->N, T = S->T, ng = S->ng;
    const size_t vcb = S->vcb, nb = S->nb;
    uint8_t *kc = S->kc + (size_t)g * nb * ORC_BT * d;
    uint16_t *ks = S->ks + (size_t)g * nb * d, *kz = S->kz + (size_t)g * nb * d;
    uint8_t *vc = S->vc + (size_t)g * nb * ORC_BT * vcb;
    uint16_t *vs = S->vs + (size_t)g * nb * ORC_BT * ng, *vz = S->vz + (size_t)g * nb * ORC_BT * ng;
    float *eta = S->eta + (size_t)g * nb;
    uint16_t *blk = (uint16_t *)malloc((size_t)ORC_BT * d * 2);
    uint16_t *blv = (uint16_t *)malloc((size_t)ORC_BT * d * 2);
    for (int b = 0; b < N; b++) {
        for (int t = 0; t < ORC_BT; t++)
            for (int c = 0; c < d; c++) {
                size_t src = ((size_t)(b * ORC_BT + t) * Hkv + g) * d + c;
                blk[t * d + c] = S->Kn[src];
                blv[t * d + c] = S->Vn[src];
            }
        orc_quant_k_block(d, blk, kc + (size_t)b * ORC_BT * d, ks + (size_t)b * d, kz + (size_t)b * d);
        orc_quant_v_block_bits(d, S->v_bits, blv, vc + (size_t)b * ORC_BT * vcb, vs + (size_t)b * ORC_BT * ng,
                               vz + (size_t)b * ORC_BT * ng, &eta[b]);
    }
    free(blk);
    free(blv);
    size_t gofs = ((size_t)n * Hkv + g) * N;
    if (tr->k_code)
        memcpy(tr->k_code + gofs * ORC_BT * d, kc, (size_t)N * ORC_BT * d);
    if (tr->k_s)
        memcpy(tr->k_s + gofs * d, ks, (size_t)N * d * 2);
    if (tr->k_z)
        memcpy(tr->k_z + gofs * d, kz, (size_t)N * d * 2);
    if (tr->v_code)
        memcpy(tr->v_code + gofs * ORC_BT * vcb, vc, (size_t)N * ORC_BT * vcb);
    if (tr->v_s)
        memcpy(tr->v_s + gofs * ORC_BT * ng, vs, (size_t)N * ORC_BT * ng * 2);
    if (tr->v_z)
        memcpy(tr->v_z + gofs * ORC_BT * ng, vz, (size_t)N * ORC_BT * ng * 2);
    if (tr->eta)
        memcpy(tr->eta + gofs, eta, (size_t)N * sizeof(float));

    double rmax = 0.0;
    for (int c = 0; c < d; c++) {
        double lo = INFINITY, hi = -INFINITY;
        for (int t = 0; t < T; t++) {
            double x = (double)orc_h2f(S->Vn[((size_t)t * Hkv + g) * d + c]);
            if (x < lo)
                lo = x;
            if (x > hi)
                hi = x;
        }
        if (hi - lo > rmax)
            rmax = hi - lo;
    }
    S->vrange[g] = orc_ru32(rmax);
    if (tr->vrange)
        tr->vrange[(size_t)n * Hkv + g] = S->vrange[g];
}

/* Phase 2, per q head h: the scoring pass over tier 1 (the partial block
 * from its FP16 keys), the plan (selection, bounds, rungs 1-2) from
 * INT8-side quantities only [Contrib], the certified scores (FP16 keys on
 * P, paged from tier 2 [Meth-3]) and exact dense attention.  Returns 1 when
 * a cap of rung 1 or 2 was exhausted. */
static int q_head_plan(const seq_t *S, int n, int h, const uint16_t *q, orc_trace *tr)
{
    const int d = S->d, Hkv = S->Hkv, N = S->N, np = S->np, Np = S->Np, G = S->G, g = h / G;
    const size_t nb = S->nb;
    const orc_thresholds *th = S->th;
    const uint8_t *kc = S->kc + (size_t)g * nb * ORC_BT * d;
    const uint16_t *ks = S->ks + (size_t)g * nb * d, *kz = S->kz + (size_t)g * nb * d;
    const uint16_t *qh = q + ((size_t)n * S->Hq + h) * d;
    float *sc = S->sc + (size_t)h * Np * ORC_BT;
    float *bmax = S->bmax + (size_t)h * Np, *bl = S->bl + (size_t)h * Np;
    float *dl = S->dl + (size_t)h * Np, *rh = S->rh + (size_t)h * Np;
    uint16_t *blk = (uint16_t *)malloc((size_t)ORC_BT * d * 2);

    for (int b = 0; b < N; b++) {
        orc_score_q8(d, qh, kc + (size_t)b * ORC_BT * d, ks + (size_t)b * d, kz + (size_t)b * d, th->sm_scale,
                     sc + (size_t)b * ORC_BT);
        orc_block_est(sc + (size_t)b * ORC_BT, ORC_BT, &bmax[b], &bl[b]);
        orc_delta_rho(d, qh, ks + (size_t)b * d, kz + (size_t)b * d, th->sm_scale, &dl[b], &rh[b]);
    }
    if (S->has_part) {
        for (int t = 0; t < np; t++)
            for (int c = 0; c < d; c++)
                blk[t * d + c] = S->Kn[((size_t)(N * ORC_BT + t) * Hkv + g) * d + c];
        float *sp = sc + (size_t)N * ORC_BT;
        orc_score_f16(d, qh, blk, np, th->sm_scale, sp);
        for (int t = np; t < ORC_BT; t++)
            sp[t] = 0.0f;
        orc_block_est(sp, np, &bmax[N], &bl[N]);
        rh[N] = rho_partial(d, qh, blk, np, th->sm_scale);
        dl[N] = rh[N];
    }
    plan_t *p = &S->plans[h];
    p->N = N;
    p->has_part = S->has_part;
    p->bmax = bmax;
    p->bl = bl;
    p->delta = dl;
    p->rho = rh;
    p->eta = S->eta + (size_t)g * nb;
    p->R = (double)S->vrange[g];
    p->M = S->M + (size_t)h * Np;
    p->inP = S->inP + (size_t)h * nb;
    p->inVP = S->inVP + (size_t)h * nb;
    p->cval = S->cval + (size_t)h * nb;
    plan_head(p, th);

    size_t ho = (size_t)n * S->Hq + h;
    if (tr->score)
        memcpy(tr->score + ho * Np * ORC_BT, sc, (size_t)Np * ORC_BT * sizeof(float));
    if (tr->bmax)
        memcpy(tr->bmax + ho * Np, bmax, (size_t)Np * sizeof(float));
    if (tr->bl)
        memcpy(tr->bl + ho * Np, bl, (size_t)Np * sizeof(float));
    if (tr->delta)
        memcpy(tr->delta + ho * Np, dl, (size_t)Np * sizeof(float));
    if (tr->rho)
        memcpy(tr->rho + ho * Np, rh, (size_t)Np * sizeof(float));
    if (tr->mref)
        tr->mref[ho] = p->mref;
    if (tr->mfx)
        memcpy(tr->mfx + ho * Np, p->M, (size_t)Np * sizeof(uint64_t));
    if (tr->cval)
        memcpy(tr->cval + ho * N, p->cval, (size_t)N * sizeof(uint64_t));
    if (tr->sel)
        for (int b = 0; b < N; b++)
            tr->sel[ho * N + b] = (uint8_t)(p->inP[b] | (p->inVP[b] << 1));
    if (tr->bounds) {
        tr->bounds[ho * 4 + 0] = p->mu;
        tr->bounds[ho * 4 + 1] = p->tv;
        tr->bounds[ho * 4 + 2] = p->ekey;
        tr->bounds[ho * 4 + 3] = p->eval;
    }

    /* certified scores: FP16 keys on P (paged from tier 2) and on the
     * partial block, INT8 scores on the tail [Meth-3] */
    float *smix = S->smix + (size_t)h * Np * ORC_BT;
    memcpy(smix, sc, (size_t)Np * ORC_BT * sizeof(float));
    for (int b = 0; b < N; b++) {
        if (!p->inP[b])
            continue;
        for (int t = 0; t < ORC_BT; t++)
            for (int c = 0; c < d; c++)
                blk[t * d + c] = S->Kn[((size_t)(b * ORC_BT + t) * Hkv + g) * d + c];
        orc_score_f16(d, qh, blk, ORC_BT, th->sm_scale, smix + (size_t)b * ORC_BT);
    }
    orc_dense_head(S->T, Hkv, d, g, S->Kn, S->Vn, qh, (double)th->sm_scale, S->odense + (size_t)h * d);
    free(blk);
    return p->cap_fail;
}

/* Phase 3, per q head h: the rank-consistency check on the promoted blocks
 * [Meth-3].  The INT8 order is (estimated mass M desc, index asc); the FP16
 * order is (M16 desc, index asc), M16 the fixed-point FP16-key block mass
 * relative to the largest FP16-key block max over P; D = Kendall discordant
 * pairs between the two orders; inconsistent iff D > floor(rank_tol *
 * K*(K*-1)/2). */
static void q_head_rank(const seq_t *S, int n, int h, orc_trace *tr)
{
    const int N = S->N, Np = S->Np;
    const plan_t *p = &S->plans[h];
    const float *sm16 = S->smix + (size_t)h * Np * ORC_BT;
    size_t nb = S->nb;
    float *b16max = (float *)malloc(nb * sizeof(float)), *b16l = (float *)malloc(nb * sizeof(float));
    uint64_t *keyI = (uint64_t *)malloc(nb * sizeof(uint64_t)), *key16 = (uint64_t *)malloc(nb * sizeof(uint64_t));
    int *plist = (int *)malloc(nb * sizeof(int));
    int kk = 0;
    for (int b = 0; b < N; b++)
        if (p->inP[b])
            plist[kk++] = b;
    float mr16 = -INFINITY;
    for (int i = 0; i < kk; i++) {
        int b = plist[i];
        orc_block_est(sm16 + (size_t)b * ORC_BT, ORC_BT, &b16max[i], &b16l[i]);
        if (b16max[i] > mr16)
            mr16 = b16max[i];
    }
    if (orc_mutation & 8)
        mr16 = p->mref;
    size_t ho = (size_t)n * S->Hq + h;
    if (tr->m16fx)
        memset(tr->m16fx + ho * N, 0, (size_t)N * sizeof(uint64_t));
    if (tr->score16) {
        memset(tr->score16 + ho * N * ORC_BT, 0, (size_t)N * ORC_BT * sizeof(float));
        for (int i = 0; i < kk; i++)
            memcpy(tr->score16 + ho * N * ORC_BT + (size_t)plist[i] * ORC_BT, sm16 + (size_t)plist[i] * ORC_BT,
                   ORC_BT * sizeof(float));
    }
    for (int i = 0; i < kk; i++) {
        int b = plist[i];
        float m = b16l[i] * orc_exp_c(b16max[i] - mr16);
        uint64_t M16 = (uint64_t)((double)m * 4294967296.0);
        if (tr->m16fx)
            tr->m16fx[ho * N + b] = M16;
        uint64_t tie = (orc_mutation & 4) ? (uint64_t)b : (uint64_t)(0xFFFF - b);
        keyI[i] = (p->M[b] << 16) | tie;
        key16[i] = (((orc_mutation & 16) ? p->M[b] : M16) << 16) | tie;
    }
    S->D[h] = orc_discordant(kk, keyI, key16);
    double pairs = (double)kk * (double)(kk - 1) / 2.0;
    double lim = floor((double)S->th->rank_tol * pairs);
    S->rank_ok[h] = !((double)S->D[h] > lim);
    free(b16max);
    free(b16l);
    free(keyI);
    free(key16);
    free(plist);
}

/* Phase 4, per q head h: the certified output, the measured key and value
 * errors against exact attention, and the ladder outcome [Meth-3,
 * four-rung fallback ladder]; heads at rung 3 or 4 return exact dense
 * attention [Contrib, deterministic recovery]. */
static void q_head_output(const seq_t *S, int n, int h, int rung4_pre, int rung4_post, const uint16_t *q,
                          double *out, orc_report *rep, orc_trace *tr)
{
    const int d = S->d, Hkv = S->Hkv, N = S->N, T = S->T, G = S->G, g = h / G, ng = S->ng, Np = S->Np;
    const size_t vcb = S->vcb, nb = S->nb;
    const double sm = (double)S->th->sm_scale;
    const plan_t *p = &S->plans[h];
    const uint16_t *Vg = S->Vn;
    const float *smh = S->smix + (size_t)h * Np * ORC_BT;
    const uint8_t *vcg = S->vc + (size_t)g * nb * ORC_BT * vcb;
    const uint16_t *vsg = S->vs + (size_t)g * nb * ORC_BT * ng;
    const uint16_t *vzg = S->vz + (size_t)g * nb * ORC_BT * ng;
    double *oc = S->ocert + (size_t)h * d;
    const double *od = S->odense + (size_t)h * d;
    double *ptil = (double *)malloc((size_t)T * sizeof(double));
    double *pex = (double *)malloc((size_t)T * sizeof(double));
    /* p~ over all T tokens */
    double mx = -INFINITY;
    for (int t = 0; t < T; t++)
        if ((double)smh[t] > mx)
            mx = (double)smh[t];
    double den = 0.0;
    for (int t = 0; t < T; t++) {
        ptil[t] = exp((double)smh[t] - mx);
        den += ptil[t];
    }
    for (int t = 0; t < T; t++)
        ptil[t] /= den;
    /* exact p */
    {
        const uint16_t *qh = q + ((size_t)n * S->Hq + h) * d;
        double m2 = -INFINITY;
        for (int t = 0; t < T; t++) {
            const uint16_t *kt = S->Kn + ((size_t)t * Hkv + g) * d;
            double a = 0.0;
            for (int c = 0; c < d; c++)
                a += (double)orc_h2f(qh[c]) * (double)orc_h2f(kt[c]);
            pex[t] = sm * a;
            if (pex[t] > m2)
                m2 = pex[t];
        }
        double dd = 0.0;
        for (int t = 0; t < T; t++) {
            pex[t] = exp(pex[t] - m2);
            dd += pex[t];
        }
        for (int t = 0; t < T; t++)
            pex[t] /= dd;
    }
    double ek = 0.0, ev = 0.0;
    for (int c = 0; c < d; c++) {
        double acc = 0.0, akey = 0.0, aval = 0.0;
        for (int t = 0; t < T; t++) {
            int b = t / ORC_BT, tt = t % ORC_BT;
            double v = (double)orc_h2f(Vg[((size_t)t * Hkv + g) * d + c]);
            double vu = v;
            if (b < N && !p->inVP[b]) {
                int code;
                if (S->v_bits == 8) {
                    code = vcg[((size_t)b * ORC_BT + tt) * d + c];
                } else {
                    uint8_t byte = vcg[((size_t)b * ORC_BT + tt) * (d / 2) + c / 2];
                    code = (c & 1) ? (byte >> 4) : (byte & 15);
                }
                size_t mi = ((size_t)b * ORC_BT + tt) * ng + c / ORC_VG;
                vu = (double)orc_h2f(vzg[mi]) + (double)orc_h2f(vsg[mi]) * (double)code;
            }
            acc += ptil[t] * vu;
            akey += (ptil[t] - pex[t]) * v;
            aval += ptil[t] * (vu - v);
        }
        oc[c] = acc;
        if (fabs(akey) > ek)
            ek = fabs(akey);
        if (fabs(aval) > ev)
            ev = fabs(aval);
    }
    free(ptil);
    free(pex);
    size_t ho = (size_t)n * S->Hq + h;
    if (tr->err_key)
        tr->err_key[ho] = ek;
    if (tr->err_val)
        tr->err_val[ho] = ev;
    if (tr->o_cert)
        memcpy(tr->o_cert + ho * d, oc, (size_t)d * sizeof(double));
    if (tr->o_dense)
        memcpy(tr->o_dense + ho * d, od, (size_t)d * sizeof(double));

    int mask = 0;
    if (p->widened)
        mask |= 2;
    if (p->nvp > 0)
        mask |= 4;
    int is3 = !rung4_pre && !S->rank_ok[h];
    if (is3)
        mask |= 8;
    int is4 = rung4_pre || rung4_post;
    if (is4)
        mask |= 16;
    int dense = is3 || is4;
    int rmax = 0;
    for (int r = 1; r <= 4; r++)
        if (mask & (1 << r))
            rmax = r;
    orc_report *R = &rep[ho];
    R->kstar = p->kstar;
    R->n_v_promoted = p->nvp;
    R->tau_final = (float)p->tau;
    R->rank_ok = rung4_pre ? -1 : S->rank_ok[h];
    R->n_discordant = rung4_pre ? 0 : (int)S->D[h];
    R->rung_mask = mask;
    R->rung_max = rmax;
    if (dense) {
        R->e_key = R->e_val = R->tv_bound = 0.0f;
        memcpy(out + ho * d, od, (size_t)d * sizeof(double));
    } else {
        R->e_key = orc_ru32(p->ekey);
        R->e_val = orc_ru32(p->eval);
        R->tv_bound = orc_ru32(p->tv);
        memcpy(out + ho * d, oc, (size_t)d * sizeof(double));
    }
}

int orc_certified_decode_vb(int B, int T, int Hq, int Hkv, int d, int v_bits, const uint16_t *K,
                            const uint16_t *V, const uint16_t *q, const orc_thresholds *th,
                            double *out, orc_report *rep, orc_trace *tr)
{
    if (B < 1 || T < 1 || Hkv < 1 || Hq < Hkv || Hq % Hkv || (d != 64 && d != 128) ||
        (v_bits != 4 && v_bits != 8))
        return -1;
    orc_trace empty;
    memset(&empty, 0, sizeof empty);
    if (!tr)
        tr = &empty;
    seq_t S;
    memset(&S, 0, sizeof S);
    S.T = T;
    S.Hq = Hq;
    S.Hkv = Hkv;
    S.d = d;
    S.G = Hq / Hkv;
    S.N = T / ORC_BT;
    S.np = T % ORC_BT;
    S.has_part = S.np > 0;
    S.Np = S.N + S.has_part;
    S.ng = d / ORC_VG;
    S.v_bits = v_bits;
    S.vcb = (size_t)d * v_bits / 8; /* bytes of value codes per token */
    S.nb = (size_t)(S.N > 0 ? S.N : 1);
    S.th = th;
    const size_t nb = S.nb, Np = (size_t)S.Np;
    S.kc = (uint8_t *)malloc((size_t)Hkv * nb * ORC_BT * d);
    S.ks = (uint16_t *)malloc((size_t)Hkv * nb * d * 2);
    S.kz = (uint16_t *)malloc((size_t)Hkv * nb * d * 2);
    S.vc = (uint8_t *)malloc((size_t)Hkv * nb * ORC_BT * S.vcb);
    S.vs = (uint16_t *)malloc((size_t)Hkv * nb * ORC_BT * S.ng * 2);
    S.vz = (uint16_t *)malloc((size_t)Hkv * nb * ORC_BT * S.ng * 2);
    S.eta = (float *)malloc((size_t)Hkv * nb * sizeof(float));
    S.vrange = (float *)malloc((size_t)Hkv * sizeof(float));
    S.plans = (plan_t *)calloc((size_t)Hq, sizeof(plan_t));
    S.bmax = (float *)malloc((size_t)Hq * Np * sizeof(float));
    S.bl = (float *)malloc((size_t)Hq * Np * sizeof(float));
    S.dl = (float *)malloc((size_t)Hq * Np * sizeof(float));
    S.rh = (float *)malloc((size_t)Hq * Np * sizeof(float));
    S.sc = (float *)malloc((size_t)Hq * Np * ORC_BT * sizeof(float));
    S.M = (uint64_t *)malloc((size_t)Hq * Np * sizeof(uint64_t));
    S.cval = (uint64_t *)malloc((size_t)Hq * nb * sizeof(uint64_t));
    S.inP = (uint8_t *)malloc((size_t)Hq * nb);
    S.inVP = (uint8_t *)malloc((size_t)Hq * nb);
    S.smix = (float *)malloc((size_t)Hq * Np * ORC_BT * sizeof(float));
    S.odense = (double *)malloc((size_t)Hq * d * sizeof(double));
    S.ocert = (double *)malloc((size_t)Hq * d * sizeof(double));
    S.D = (int64_t *)calloc((size_t)Hq, sizeof(int64_t));
    S.rank_ok = (int *)malloc((size_t)Hq * sizeof(int));

    for (int n = 0; n < B; n++) {
        S.Kn = K + (size_t)n * T * Hkv * d;
        S.Vn = V + (size_t)n * T * Hkv * d;
#pragma omp parallel for schedule(dynamic, 1)
        for (int g = 0; g < Hkv; g++)
            kv_head_tier1(&S, n, g, tr);
        /* rung 4 before paging: a cap exhausted on any head of (n, layer) */
        int rung4_pre = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : rung4_pre)
        for (int h = 0; h < Hq; h++)
            rung4_pre |= q_head_plan(&S, n, h, q, tr);
#pragma omp parallel for schedule(dynamic, 1)
        for (int h = 0; h < Hq; h++)
            q_head_rank(&S, n, h, tr);
        /* rung 4 after the rank check: more than f_layer of the q heads
         * at rung 3 */
        int n_rung3 = 0;
        for (int h = 0; h < Hq; h++)
            n_rung3 += !S.rank_ok[h];
        int rung4_post = !rung4_pre && ((double)n_rung3 > (double)th->f_layer * (double)Hq);
        if (tr->seq_flags)
            tr->seq_flags[n] = rung4_pre | (rung4_post << 1);
#pragma omp parallel for schedule(dynamic, 1)
        for (int h = 0; h < Hq; h++)
            q_head_output(&S, n, h, rung4_pre, rung4_post, q, out, rep, tr);
    }

    free(S.kc); free(S.ks); free(S.kz); free(S.vc); free(S.vs); free(S.vz); free(S.eta); free(S.vrange);
    free(S.plans); free(S.bmax); free(S.bl); free(S.dl); free(S.rh); free(S.sc); free(S.M); free(S.cval);
    free(S.inP); free(S.inVP); free(S.smix); free(S.odense); free(S.ocert); free(S.D); free(S.rank_ok);
    return 0;
}
