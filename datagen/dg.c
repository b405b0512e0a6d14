/*
 * dg.c -- seeded synthetic inputs (keys, values, queries) for the certified
 * quantized-KV decode step.  Shared by the oracle tests, the GPU tests and
 * the benchmark; it holds none of the method's arithmetic.
 *
 * Random numbers: Philox4x32-10, the counter-based generator of Salmon,
 * Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
 * (SC'11), written from its published round function.  Element i of a
 * tensor uses counter (i / 2, tag) and key (seed), so any slice can be
 * produced independently and in parallel.  Normals: Box-Muller.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

typedef struct {
    uint32_t v[4];
} p4;

static inline void mulhilo(uint32_t a, uint32_t b, uint32_t *hi, uint32_t *lo)
{
    uint64_t p = (uint64_t)a * (uint64_t)b;
    *hi = (uint32_t)(p >> 32);
    *lo = (uint32_t)p;
}

/* Philox4x32 with 10 rounds. */
p4 dg_philox(p4 ctr, uint32_t k0, uint32_t k1)
{
    for (int r = 0; r < 10; r++) {
        uint32_t hi0, lo0, hi1, lo1;
        mulhilo(0xD2511F53u, ctr.v[0], &hi0, &lo0);
        mulhilo(0xCD9E8D57u, ctr.v[2], &hi1, &lo1);
        p4 n;
        n.v[0] = hi1 ^ ctr.v[1] ^ k0;
        n.v[1] = lo1;
        n.v[2] = hi0 ^ ctr.v[3] ^ k1;
        n.v[3] = lo0;
        ctr = n;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return ctr;
}

void dg_philox_raw(const uint32_t *ctr, const uint32_t *key, uint32_t *out)
{
    p4 c;
    memcpy(c.v, ctr, 16);
    p4 r = dg_philox(c, key[0], key[1]);
    memcpy(out, r.v, 16);
}

static inline double u53(uint32_t a, uint32_t b)
{
    return ((double)(a >> 5) * 67108864.0 + (double)(b >> 6)) * (1.0 / 9007199254740992.0);
}

/* Standard normal number i of stream (seed, tag). */
static inline double normal_at(uint64_t seed, uint32_t tag, uint64_t i)
{
    p4 c;
    uint64_t j = i >> 1;
    c.v[0] = (uint32_t)j;
    c.v[1] = (uint32_t)(j >> 32);
    c.v[2] = tag;
    c.v[3] = 0x6b7a1d35u;
    p4 r = dg_philox(c, (uint32_t)seed, (uint32_t)(seed >> 32));
    double u1 = 1.0 - u53(r.v[0], r.v[1]); /* (0, 1] */
    double u2 = u53(r.v[2], r.v[3]);       /* [0, 1) */
    double rad = sqrt(-2.0 * log(u1));
    double ang = 6.283185307179586 * u2;
    return (i & 1) ? rad * sin(ang) : rad * cos(ang);
}

/* Uniform in [0, 1), number i of stream (seed, tag). */
static inline double uniform_at(uint64_t seed, uint32_t tag, uint64_t i)
{
    p4 c;
    c.v[0] = (uint32_t)i;
    c.v[1] = (uint32_t)(i >> 32);
    c.v[2] = tag;
    c.v[3] = 0x2c1b3c6du;
    p4 r = dg_philox(c, (uint32_t)seed, (uint32_t)(seed >> 32));
    return u53(r.v[0], r.v[1]);
}

/* Both normals of pair j (numbers 2j and 2j + 1 of the stream). */
static inline void normal_pair(uint64_t seed, uint32_t tag, uint64_t j, double *z0, double *z1)
{
    p4 c;
    c.v[0] = (uint32_t)j;
    c.v[1] = (uint32_t)(j >> 32);
    c.v[2] = tag;
    c.v[3] = 0x6b7a1d35u;
    p4 r = dg_philox(c, (uint32_t)seed, (uint32_t)(seed >> 32));
    double u1 = 1.0 - u53(r.v[0], r.v[1]);
    double u2 = u53(r.v[2], r.v[3]);
    double rad = sqrt(-2.0 * log(u1));
    double ang = 6.283185307179586 * u2;
    *z0 = rad * cos(ang);
    *z1 = rad * sin(ang);
}

void dg_normal(uint64_t seed, uint32_t tag, int64_t start, int64_t n, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = normal_at(seed, tag, (uint64_t)(start + i));
}

void dg_uniform(uint64_t seed, uint32_t tag, int64_t start, int64_t n, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = uniform_at(seed, tag, (uint64_t)(start + i));
}

/* binary64 -> binary16, round to nearest even (IEEE 754 conversion). */
static uint16_t f2h_rne(double x)
{
    uint16_t sign = 0;
    if (x < 0 || (x == 0 && signbit(x))) {
        sign = 0x8000;
        x = -x;
    }
    if (isnan(x))
        return 0x7E00;
    if (x >= 65520.0)
        return sign | 0x7C00; /* overflow (65520 is the rounding boundary) */
    int e;
    double m = frexp(x, &e); /* x = m 2^e, m in [0.5, 1) */
    if (x == 0.0)
        return sign;
    /* unit in the last place of the result */
    int ulp_exp = e - 11; /* normal: 11 significant bits */
    if (ulp_exp < -24)
        ulp_exp = -24; /* subnormal spacing 2^-24 */
    double scaled = ldexp(x, -ulp_exp);
    double r = nearbyint(scaled); /* ties to even in default mode */
    (void)m;
    double y = ldexp(r, ulp_exp);
    /* encode y */
    if (y >= 65520.0)
        return sign | 0x7C00;
    if (y < 0x1p-14) {
        return sign | (uint16_t)(int)ldexp(y, 24);
    }
    int ey;
    double my = frexp(y, &ey); /* y = my 2^ey */
    int exp16 = ey - 1 + 15;
    int man = (int)ldexp(my, 11) - 1024;
    return sign | (uint16_t)(exp16 << 10) | (uint16_t)man;
}

void dg_to_f16(const double *in, int64_t n, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = f2h_rne(in[i]);
}

/*
 * Keys of one layer, [B][T][Hkv][d] FP16:
 *   k = o_gc * (lowrank + noise_std * z) + amp[n][g][blk] * dir[n][g][c]
 * with lowrank = sum_r u[n][t][g][r] W[g][r][c] (rank may be 0).
 * tie_mode[g] (with tie_eps > 0) arranges near ties: 1 = in every odd
 * block the keys are the even block's values plus o_gc * tie_eps * (2U - 1)
 * (near-tie pairs); 2 = every block is block 0 plus such a perturbation.
 */
void dg_keys(uint64_t seed, int B, int T, int Hkv, int d, const float *chan_scale,
             int rank, const float *W, double noise_std, const float *amp, const float *dir,
             double tie_eps, const int *tie_mode, uint16_t *out)
{
    const int NB = (T + 63) / 64;
#pragma omp parallel for schedule(static) collapse(2)
    for (int n = 0; n < B; n++)
        for (int t = 0; t < T; t++) {
            int blk = t / 64;
            for (int g = 0; g < Hkv; g++) {
                int mode = tie_eps > 0.0 ? tie_mode[g] : 0;
                int src_t = t;
                if (mode == 1 && (blk & 1))
                    src_t = t - 64;
                if (mode == 2)
                    src_t = t % 64;
                int tie = src_t != t;
                double u[64];
                for (int r = 0; r < rank && r < 64; r++)
                    u[r] = normal_at(seed, 11u, (((uint64_t)n * T + src_t) * Hkv + g) * 64 + r);
                int pblk = src_t / 64;
                double zz[2] = {0.0, 0.0};
                for (int c = 0; c < d; c++) {
                    uint64_t e = (((uint64_t)n * T + src_t) * Hkv + g) * d + c;
                    if ((c & 1) == 0)
                        normal_pair(seed, 10u, e >> 1, &zz[0], &zz[1]);
                    double lr = 0.0;
                    for (int r = 0; r < rank; r++)
                        lr += u[r] * (double)W[((size_t)g * rank + r) * d + c];
                    double o = (double)chan_scale[g * d + c];
                    double x = o * (lr + noise_std * zz[c & 1]);
                    x += (double)amp[((size_t)n * Hkv + g) * NB + pblk] * (double)dir[((size_t)n * Hkv + g) * d + c];
                    if (tie) {
                        uint64_t e2 = (((uint64_t)n * T + t) * Hkv + g) * d + c;
                        x += o * tie_eps * (2.0 * uniform_at(seed, 12u, e2) - 1.0);
                        x += ((double)amp[((size_t)n * Hkv + g) * NB + blk] -
                              (double)amp[((size_t)n * Hkv + g) * NB + pblk]) *
                             (double)dir[((size_t)n * Hkv + g) * d + c];
                    }
                    out[(((size_t)n * T + t) * Hkv + g) * d + c] = f2h_rne(x);
                }
            }
        }
}

/* Values of one layer, [B][T][Hkv][d] FP16: N(0,1) (nu <= 0) or Student-t
 * with nu degrees of freedom (integer nu: z / sqrt(chi2_nu / nu)). */
void dg_values(uint64_t seed, int B, int T, int Hkv, int d, int nu, double scale, uint16_t *out)
{
    int64_t n_el = (int64_t)B * T * Hkv * d; /* even: d is */
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_el; i += 2) {
        double z[2];
        normal_pair(seed, 20u, (uint64_t)i >> 1, &z[0], &z[1]);
        if (nu > 0) {
            double chi[2] = {0.0, 0.0};
            for (int j = 0; j < nu; j++) {
                double w0, w1;
                normal_pair(seed, 21u + (uint32_t)j, (uint64_t)i >> 1, &w0, &w1);
                chi[0] += w0 * w0;
                chi[1] += w1 * w1;
            }
            z[0] = z[0] / sqrt(chi[0] / nu);
            z[1] = z[1] / sqrt(chi[1] / nu);
        }
        out[i] = f2h_rne(scale * z[0]);
        out[i + 1] = f2h_rne(scale * z[1]);
    }
}
