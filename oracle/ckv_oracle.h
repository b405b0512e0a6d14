/*
 * ckv_oracle.h -- CPU oracle for certified quantized-KV decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this code; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no source with the HIP library.
 *
 * Source of the method: the page "Runtime-Certified Bounded-Error Quantized
 * Attention" (gist.science paper 2605.20868, technical summary).  Comments
 * cite its sections as
 *   [Meth-1]  Methodology, pillar 1: tiered storage with deterministic fallback
 *   [Meth-2]  Methodology, pillar 2: two-term error decomposition
 *   [Meth-3]  Methodology, pillar 3: adaptive precision and fallback ladder
 *   [Contrib] Key contributions
 *   [Results] Experimental results
 *   [Signif]  Significance and claims
 *
 * Values (outputs, the dense reference, measured errors) are computed in
 * FP64.  Decisions (codes, scores, masses, selected sets, bounds compared
 * with thresholds, verdicts) use a fixed FP32 / FP64 / fixed-point operation
 * sequence, written out at each function below; it is the contract the
 * GPU path must meet bit for bit.
 */
#ifndef CKV_ORACLE_H
#define CKV_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_BT 64 /* tokens per KV block */
#define ORC_VG 32 /* channels per INT4 value group */

typedef struct {
    float tau_cov;   /* coverage target of the top-K* selection [Meth-3] */
    float k_tol;     /* tolerance on E_key (output units) */
    float v_tol;     /* tolerance on E_val (output units) [Results: v_tol] */
    float rank_tol;  /* allowed fraction of discordant block pairs */
    float sm_scale;  /* softmax scale applied to q.k */
    float f_layer;   /* fraction of q heads at rung 3 that escalates to rung 4 */
    int n_widen;     /* maximum number of rung-1 widenings */
    int v_cap_blocks;/* maximum |VP| per head; <= 0 means no cap (N) */
} orc_thresholds;

typedef struct {
    float e_key, e_val, tv_bound, tau_final;
    int kstar, n_v_promoted, rank_ok, rung_max, rung_mask, n_discordant;
} orc_report;

/* Optional intermediate results; every pointer may be NULL.
 * N = full blocks per sequence, Np = N + (T % 64 != 0). */
typedef struct {
    uint8_t *k_code;   /* [B][Hkv][N][64][d]    INT8 key codes, token-major   */
    uint16_t *k_s;     /* [B][Hkv][N][d]        FP16 key scale per channel    */
    uint16_t *k_z;     /* [B][Hkv][N][d]        FP16 key offset per channel   */
    uint8_t *v_code;   /* [B][Hkv][N][64][d*v_bits/8]  INT4 pairs (low nibble = even) or INT8 */
    uint16_t *v_s;     /* [B][Hkv][N][64][d/32] FP16 value scale per group    */
    uint16_t *v_z;     /* [B][Hkv][N][64][d/32] FP16 value offset per group   */
    float *eta;        /* [B][Hkv][N]           per-block value error eta_b   */
    float *vrange;     /* [B][Hkv]              R_g, range of V               */
    float *score;      /* [B][Hq][Np*64]  INT8 scores; FP16 scores on partial */
    float *bmax;       /* [B][Hq][Np] */
    float *bl;         /* [B][Hq][Np] */
    float *delta;      /* [B][Hq][Np] (partial block: its rho)                */
    float *rho;        /* [B][Hq][Np] */
    float *mref;       /* [B][Hq]   largest estimated score                   */
    uint64_t *mfx;     /* [B][Hq][Np] fixed-point estimated block masses      */
    uint8_t *sel;      /* [B][Hq][N] bit0: block in P, bit1: block in VP      */
    double *bounds;    /* [B][Hq][4] mu, TV, E_key, E_val (final plan)        */
    int *seq_flags;    /* [B] bit0: rung 4 before paging, bit1: after         */
    float *score16;    /* [B][Hq][N*64] FP16-key scores on P blocks, else 0   */
    uint64_t *m16fx;   /* [B][Hq][N] fixed-point FP16 masses on P, else 0     */
    double *err_key;   /* [B][Hq] measured |sum (p~ - p) v|_inf               */
    double *err_val;   /* [B][Hq] measured |sum p~ (v_used - v)|_inf          */
    double *o_cert;    /* [B][Hq][d] certified output before any fallback     */
    double *o_dense;   /* [B][Hq][d] exact dense attention                    */
    uint64_t *cval;    /* [B][Hq][N] fixed-point E_val contribution per block */
} orc_trace;

/* Deliberate mistakes, used only by tests that check that the pins can
 * fail: bit0 eta_b forced to 0; bit1 Delta halved; bit2 the rank keys'
 * tie-break reversed (index desc); bit3 the FP16-side masses of the rank
 * check taken relative to the INT8 reference max instead of the largest
 * FP16-key block max over P; bit4 the FP16-side rank key built from the
 * INT8 mass; bit5 rung-2 blocks taken in ascending contribution order;
 * bit6 rung-1 widening by 1 - tau <- (1 - tau) / 3; bit7 rho of the
 * unfinished block from the signed key maximum. */
extern int orc_mutation;

/* OpenMP threads of the decode step (heads run in parallel; the results
 * do not depend on it).  Without OpenMP both are no-ops returning 1. */
void orc_set_threads(int n);
int orc_get_threads(void);

/* Conversions and elementary pieces (exported for the oracle's own pins). */
float orc_h2f(uint16_t h);
uint16_t orc_f2h_up(float x);
float orc_ru32(double x);
float orc_exp_c(float x);
double orc_expu(double x);
double orc_em1u(double x);
double orc_tanhu(double x);
uint64_t orc_fx(double t);

void orc_quant_k_block(int d, const uint16_t *k, uint8_t *code, uint16_t *s, uint16_t *z);
void orc_quant_v_block(int d, const uint16_t *v, uint8_t *code, uint16_t *s, uint16_t *z, float *eta);
void orc_quant_v_block_bits(int d, int bits, const uint16_t *v, uint8_t *code, uint16_t *s, uint16_t *z,
                            float *eta);
void orc_score_q8(int d, const uint16_t *q, const uint8_t *code, const uint16_t *s,
                  const uint16_t *z, float sm, float *out);
void orc_score_f16(int d, const uint16_t *q, const uint16_t *k, int n, float sm, float *out);
void orc_delta_rho(int d, const uint16_t *q, const uint16_t *s, const uint16_t *z, float sm,
                   float *delta, float *rho);
void orc_block_est(const float *sc, int n, float *mx, float *l);

/* Top-K*: minimal prefix of the order (M desc, index asc) whose sum reaches
 * `need`.  Returns K* and sets in_set[b] = 1 for the chosen blocks. */
int orc_select(int n, const uint64_t *m, uint64_t need, uint8_t *in_set);

/* Kendall discordant-pair count between two orders of the same blocks,
 * each given as keys sorted descending (keys are unique). */
int64_t orc_discordant(int n, const uint64_t *key_a, const uint64_t *key_b);

/* The full decode step for one layer.
 * K, V: [B][T][Hkv][d] FP16 bit patterns, q: [B][Hq][d] FP16 bit patterns.
 * out: [B][Hq][d] FP64, rep: [B][Hq].  Returns 0, or -1 on bad arguments. */
int orc_certified_decode(int B, int T, int Hq, int Hkv, int d, const uint16_t *K,
                         const uint16_t *V, const uint16_t *q, const orc_thresholds *th,
                         double *out, orc_report *rep, orc_trace *tr);
/* The same with the values at v_bits = 4 (the design) or 8 (the symmetric
 * cache configuration of [Results]). */
int orc_certified_decode_vb(int B, int T, int Hq, int Hkv, int d, int v_bits, const uint16_t *K,
                            const uint16_t *V, const uint16_t *q, const orc_thresholds *th,
                            double *out, orc_report *rep, orc_trace *tr);

/* Exact softmax attention in FP64 for one (sequence, q head); the "FP16
 * reference" of [Signif].  k, v: [T][Hkv][d] of one sequence. */
void orc_dense_head(int T, int Hkv, int d, int g, const uint16_t *k, const uint16_t *v,
                    const uint16_t *q, double sm, double *out);

#ifdef __cplusplus
}
#endif
#endif
