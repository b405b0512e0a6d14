// ckv_decode.hip -- kernels of the certified decode step.
//
// Section tags refer to the page "Runtime-Certified Bounded-Error Quantized
// Attention" (technical summary): [Meth-2] two-term error decomposition,
// [Meth-3] adaptive top-K selection, rank-consistency check and the
// four-rung fallback ladder, [Contrib] bounds computable without the FP16
// originals during the main pass.
//
//   k_score     INT8 scoring pass: one wave per (seq, kv head, block); lane =
//               token; 16-byte coalesced code loads; per-block weights
//               w_c = q_c s_c staged in LDS.  Block max / mass / Delta / rho.
//   k_select    per (seq, q head): estimated masses, top-K* by radix select,
//               E_key / E_val, rung 1 (widen), rung 2 (FP16 values).
//   k_tail      split-K flash decoding over the blocks outside P and VP:
//   k_promoted  INT4 values (tail), and over the promoted blocks: FP16-key
//               scores on P, FP16 values on VP; values unpacked in registers
//               and contracted with the softmax weights on the matrix cores.
//   k_keys16    FP16-key scores of the P blocks (staging area), FP64 chain;
//               FP16-side block max / mass for the rank check.
//   k_merge     rank-consistency check + merge of all partials -> output.
//   k_dense     exact attention on FP16 blocks (rungs 3 / 4, and the dense
//               comparator), split-K partials; k_merge_dense -> output.
#include <type_traits>

#include "ckv_device.hpp"
#include "ckv_internal.hpp"

namespace ckv {

template <class F>
static hipError_t dispatch(int d, int G, F f) {
#define CKV_CASE(DD, GG) \
    if (d == DD && G == GG) return f(std::integral_constant<int, DD>{}, std::integral_constant<int, GG>{});
    CKV_CASE(64, 1) CKV_CASE(64, 2) CKV_CASE(64, 4) CKV_CASE(64, 8)
    CKV_CASE(128, 1) CKV_CASE(128, 2) CKV_CASE(128, 4) CKV_CASE(128, 8)
#undef CKV_CASE
    return hipErrorInvalidValue;
}

// ===========================================================================
// K1: INT8 scoring pass [Meth-3: scores from the INT8 keys give an estimate
// of each block's attention mass] and the per-token bound on the score
// error from quantization [Meth-2: E_key follows from it].
//
// Score of token t for q head h in block b, as an exact integer dot product:
//   w_c = q_c s_c (exact in FP32), e = floor(log2 max_c |w_c|),
//   w~_c = rint(w_c 2^(20-e)) in [-2^21, 2^21],
//   S_t = sum_c w~_c code_tc (exact), s^_t = fl32(fl64(C + S_t 2^(e-20)) sm),
//   C = halving-tree FP32 sum of q_c z_c.
// S_t is formed on the matrix cores: w~ = 2^16 d2 + 2^8 d1 + d0 with signed
// byte digits, codes stored as code - 128, one v_mfma_i32_16x16x64_i8 per
// (16 tokens, 64 channels) with rows = (head, digit); int32 accumulation is
// exact, so the result does not depend on the order of the sums.
//   Delta = sm (kappa H + E_w + (2^-20 + 2^-23) A + 2^-23 E_w) (1 + 2^-20),
//   rho = sm 2^-23 A (1 + 2^-20), E_w = 2^(e-21) 255 d,
// with H = sum |q_c| s_c, A = sum |q_c| (|z_c| + 255 s_c) as FP64 trees.
// A workgroup holds SCORE_W waves on consecutive block slots of a (kv head,
// sequence), SCORE_BPW slots per wave, and shares q through LDS.  Each wave
// requests the codes and scales of all its slots when it starts, then scores
// them in turn: the later slots' data arrive while the first is computed,
// and many short waves keep the memory system full.  Nothing waits on a
// workgroup barrier after the q set-up.
typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int SCORE_W = 4;  // waves per workgroup of the scoring pass
#ifndef SCORE_BPW
#define SCORE_BPW 1
#endif
constexpr int SCORE_BPW_ = SCORE_BPW;  // block slots per wave

template <int D, int G>
__global__ __launch_bounds__(64 * SCORE_W) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 5 : 4))) void k_score(Layout Ly, Step St) {
    KernelClock kc(St.clk);
    constexpr int CPL = D / 64;           // channels per lane (meta, trees)
    constexpr int KS = D / 64;            // MFMA k-steps of 64 channels
    constexpr int RT = (4 * G + 15) / 16; // MFMA row tiles of 4 heads x 4 digits
    constexpr int CPR = D / 16;           // channels per lane in the set-up rows
    constexpr int BPW = SCORE_BPW_;
    const int g = blockIdx.y, n = blockIdx.z;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int l = St.layer;
    const int len = __builtin_amdgcn_readfirstlane(Ly.len[l * Ly.B + n]);
    const int N = len / 64, np = len % 64;
    const int nslot = N + (np ? 1 : 0);
    const int slot0 = (blockIdx.x * SCORE_W + wave) * BPW;
    __shared__ float qs[G][D];
    __shared__ __attribute__((aligned(16))) int8_t dig[SCORE_W][G][4][D];
    __shared__ uint32_t kms[SCORE_W][D];
    __shared__ double hd_C[SCORE_W][G];
    __shared__ int hd_e[SCORE_W][G], hd_W[SCORE_W][G];
    __shared__ float hd_dl[SCORE_W][G], hd_rh[SCORE_W][G];
    const int i16 = lane % 16;
    // the operands of the wave's full blocks, requested first: codes (MFMA B
    // operands) and the scale | offset words (D / 64 per lane, spread
    // through LDS below).  The requests do not wait for the sequence's
    // length: they cover the slots below the batch's largest full-block
    // count (within the sequence's capacity), and only the sequence's own
    // full blocks are scored (0.7 us less per launch at 32K and 128K tokens)
    v4i bq[BPW][4][KS];
    uint32_t kmw[BPW][CPL];
#pragma unroll
    for (int u = 0; u < BPW; ++u) {
        const int slot = slot0 + u;
        if (slot < St.nb) {
            const size_t bi = Ly.blk(l, n, g, slot);
            const uint8_t *kb = Ly.kq + bi * 64 * D;
#pragma unroll
            for (int tile = 0; tile < 4; ++tile)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    bq[u][tile][ks] = *reinterpret_cast<const v4i *>(kb + (ks * 4 + lane / 16) * 1024 +
                                                                     (tile * 16 + lane % 16) * 16);
            if constexpr (CPL == 2) {
                const uint2 w = reinterpret_cast<const uint2 *>(Ly.kmeta + bi * D)[lane];
                kmw[u][0] = w.x;
                kmw[u][CPL - 1] = w.y;
            } else {
                kmw[u][0] = Ly.kmeta[bi * D + lane];
            }
        }
    }
    for (int i = threadIdx.x; i < G * D; i += 64 * SCORE_W)
        qs[i / D][i % D] = h2f(St.q[((size_t)n * Ly.Hq + g * G + i / D) * D + (i % D)]);
    __syncthreads();
    if (blockIdx.x == 0 && wave == 0)  // q in FP64, [D][G] per (seq, kv head), for the FP16-key pass
        for (int i = lane; i < G * D; i += 64)
            St.qd[((size_t)n * Ly.Hkv + g) * D * G + i] = (double)qs[i % G][i / G];
    if (slot0 >= nslot) return;  // no workgroup barrier follows
    const float sm = St.sm;
    const size_t NS64 = (size_t)St.NS * 64;

    // unfinished block: FP16 keys on the device, FP64 chain, one rounding
    auto partial = [&](int slot) {
        const uint16_t *kp = Ly.kpart + Ly.seqg(l, n, g) * 64 * D;
        const bool valid = lane < np;
        double a[G];
#pragma unroll
        for (int j = 0; j < G; ++j) a[j] = 0.0;
        for (int ch = 0; ch < D / 8; ++ch) {
            const uint4 v = *reinterpret_cast<const uint4 *>(kp + ch * 512 + lane * 8);
            const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const double kc = (double)h2f((uint16_t)(wd[i / 2] >> (16 * (i & 1))));
#pragma unroll
                for (int j = 0; j < G; ++j) a[j] = fma((double)qs[j][ch * 8 + i], kc, a[j]);
            }
            // one chunk at a time (bounds the registers holding q)
#pragma unroll
            for (int j = 0; j < G; ++j) asm volatile("" : "+v"(a[j])::"memory");
        }
        // rho of the unfinished block: A = sum |q_c| max_t |k_tc|
        double kmax[CPL];
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            const int c = lane + 64 * k;
            double m = 0.0;
            for (int t = 0; t < np; ++t) m = fmax(m, fabs((double)h2f(kp[(c / 8) * 512 + t * 8 + (c % 8)])));
            kmax[k] = m;
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const int h = g * G + j;
            const float s = valid ? (float)(a[j] * (double)sm) : 0.0f;
            St.score[(size_t)(n * Ly.Hq + h) * NS64 + (size_t)slot * 64 + lane] = s;
            const float mx = wave_max_dpp(valid ? s : -INFINITY);
            const float l_ = tree64_f32_dpp(valid ? exp_c(s - mx) : 0.0f);
            double av = fabs((double)qs[j][lane]) * kmax[0];
            if (CPL == 2) av = av + fabs((double)qs[j][lane + 64]) * kmax[CPL - 1];
            const double A = tree64_f64(av);
            if (lane == 0) {
                double rh = A * 0x1p-23;
                rh = rh * (double)sm;
                rh = rh * (1.0 + 0x1p-20);
                const float r = ru32(rh);
                St.bstat[(size_t)(n * Ly.Hq + h) * St.NS + slot] = make_float4(mx, l_, r, r);
            }
        }
    };

    // a full block: per-head weights, digits and bounds, then the exact
    // integer dot products on the matrix cores and the block estimate
    auto full = [&](int slot, const v4i (&bqu)[4][KS], const uint32_t (&kmwu)[CPL]) {
        // the scale | offset words of channels i16 + 16 k, k < D / 16; the
        // wave's previous block has finished reading kms, dig and hd_*
        wave_sync();
        if constexpr (CPL == 2) {
            kms[wave][2 * lane] = kmwu[0];
            kms[wave][2 * lane + 1] = kmwu[CPL - 1];
        } else {
            kms[wave][lane] = kmwu[0];
        }
        for (int i = lane; i < G * D; i += 64) dig[wave][i / D][3][i % D] = 0;  // the unused digit row
        wave_sync();
        uint32_t km[CPR];
#pragma unroll
        for (int k = 0; k < CPR; ++k) km[k] = kms[wave][i16 + 16 * k];
        if (lane == 0) St.sel[((size_t)n * Ly.Hkv + g) * Ly.Nmax + slot] = 0u;
        // set-up per head: row r of the wave takes head r (+4 on a second
        // pass); lane i of the row holds channels c = i + 16 k, k < D/16, so
        // the halving tree over the channels runs in-lane for strides >= 16
        // and across the row (DPP) for strides 8..1.
        const int r = lane / 16;
        float sc[CPR], zc[CPR];
#pragma unroll
        for (int k = 0; k < CPR; ++k) {
            sc[k] = h2f((uint16_t)(km[k] & 0xFFFFu));
            zc[k] = h2f((uint16_t)(km[k] >> 16));
        }
        const double kappa = 0.5 + 0x1p-14;
#pragma unroll
        for (int pass = 0; pass < (G + 3) / 4; ++pass) {
            const int j = pass * 4 + r;
            if (j < G) {
                float w[CPR], cz[CPR];
                double hv[CPR], av[CPR];
                float wm = 0.0f;
#pragma unroll
                for (int k = 0; k < CPR; ++k) {
                    const float q = qs[j][i16 + 16 * k];
                    w[k] = q * sc[k];
                    cz[k] = q * zc[k];
                    hv[k] = fabs((double)q) * (double)sc[k];
                    av[k] = fabs((double)q) * (fabs((double)zc[k]) + 255.0 * (double)sc[k]);
                    wm = fmaxf(wm, fabsf(w[k]));
                }
                // in-lane tree levels (channel strides D/2 .. 16)
#pragma unroll
                for (int st = CPR / 2; st >= 1; st >>= 1)
#pragma unroll
                    for (int k = 0; k < st; ++k) {
                        cz[k] = cz[k] + cz[k + st];
                        hv[k] = hv[k] + hv[k + st];
                        av[k] = av[k] + av[k + st];
                    }
                const float C = row_tree_f32(cz[0]);
                const double H = row_tree_f64(hv[0]);
                const double A = row_tree_f64(av[0]);
                wm = row_max_f32(wm);
                const bool nz = wm > 0.0f;
                const int e = nz ? (int)((__float_as_uint(wm) >> 23) & 0xFFu) - 127 : 0;
                int wsum = 0;
#pragma unroll
                for (int k = 0; k < CPR; ++k) {
                    const int wt = nz ? (int)rintf(ldexpf(w[k], 20 - e)) : 0;
                    wsum += wt;
                    const int d0 = (int8_t)wt;  // balanced base-256 digits
                    const int r1 = (wt - d0) >> 8;
                    const int d1 = (int8_t)r1;
                    const int d2 = (r1 - d1) >> 8;
                    const int c = i16 + 16 * k;
                    dig[wave][j][0][c] = (int8_t)d0;
                    dig[wave][j][1][c] = (int8_t)d1;
                    dig[wave][j][2][c] = (int8_t)d2;
                }
                wsum = row_sum_i32(wsum);
                if (i16 == 0) {
                    const double Ew = nz ? ldexp(255.0 * (double)D, e - 21) : 0.0;
                    double dl = kappa * H + Ew;
                    dl = dl + A * (0x1p-20 + 0x1p-23);
                    dl = dl + Ew * 0x1p-23;
                    dl = dl * (double)sm;
                    dl = dl * (1.0 + 0x1p-20);
                    double rh = A * 0x1p-23;
                    rh = rh * (double)sm;
                    rh = rh * (1.0 + 0x1p-20);
                    hd_C[wave][j] = (double)C;
                    hd_e[wave][j] = e;
                    hd_W[wave][j] = wsum;
                    hd_dl[wave][j] = ru32(dl);
                    hd_rh[wave][j] = ru32(rh);
                }
            }
        }
        wave_sync();

        // matrix cores: rows = (head, digit), columns = tokens, k = channels
        const int row = lane % 16, hrow = row / 4, drow = row % 4;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int ha = rt * 4 + hrow;  // head of this lane's A row
            v4i a[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ha < G)
                    a[ks] = *reinterpret_cast<const v4i *>(&dig[wave][ha][drow][ks * 64 + (lane / 16) * 16]);
                else
                    a[ks] = v4i{0, 0, 0, 0};
            }
            const int hh = rt * 4 + lane / 16;  // head of this lane's output rows
            float sv[4];
#pragma unroll
            for (int tile = 0; tile < 4; ++tile) {
                v4i acc = {0, 0, 0, 0};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[ks], bqu[tile][ks], acc, 0, 0, 0);
                sv[tile] = 0.0f;
                if (hh < G) {
                    // S = 2^16 acc2 + 2^8 acc1 + acc0 + 128 W: an integer below
                    // 2^53 in magnitude, formed exactly in FP64
                    const double S = fma((double)acc[2], 65536.0,
                                         fma((double)acc[1], 256.0, (double)acc[0] + 128.0 * (double)hd_W[wave][hh]));
                    const double x = hd_C[wave][hh] + ldexp(S, hd_e[wave][hh] - 20);
                    sv[tile] = (float)(x * (double)sm);
                    St.score[(size_t)(n * Ly.Hq + g * G + hh) * NS64 + (size_t)slot * 64 + tile * 16 + row] =
                        sv[tile];
                }
            }
            // block estimate of head hh: tokens tile*16 + row live in the 16
            // lanes of the group; the halving tree over the 64 tokens is the
            // in-lane steps of stride 32 and 16, then strides 8..1 across lanes
            float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
            mx = row_max_f32(mx);
            float e4[4];
#pragma unroll
            for (int tile = 0; tile < 4; ++tile) e4[tile] = exp_c(sv[tile] - mx);
            const float u0 = e4[0] + e4[2], u1 = e4[1] + e4[3];
            const float v = row_tree_f32(u0 + u1);
            if (hh < G && row == 0)
                St.bstat[(size_t)(n * Ly.Hq + g * G + hh) * St.NS + slot] =
                    make_float4(mx, v, hd_dl[wave][hh], hd_rh[wave][hh]);
        }
    };

#pragma unroll
    for (int u = 0; u < BPW; ++u) {
        const int slot = slot0 + u;
        if (slot < N)
            full(slot, bq[u], kmw[u]);
        else if (slot == N && np)
            partial(slot);
    }
}

// ===========================================================================
// K2: selection, bounds, rungs 1-2 [Meth-2, Meth-3, Contrib].
// One SEL_T-thread workgroup per (q head, sequence).
// ===========================================================================
constexpr int SEL_T = 1024;
constexpr int MAX_BPS = 64;
constexpr int SEL_LDS = 2048;  // blocks per head whose selection keys stay in LDS  // blocks per split, at most (the host keeps bps in [4, 64])

struct SelShared {
    uint64_t hsum[64];
    uint64_t hkey[64];
    uint32_t hsat[64];
    uint32_t hcnt[64];
    uint64_t red_u[SEL_T / 64];
    double red_d[SEL_T / 64];
    float red_f[SEL_T / 64];
    int red_i[SEL_T / 64];
    uint64_t bc_u[4];
    int bc_i[4];
};

__device__ __forceinline__ float block_max_f(float v, SelShared &sh) {
    v = wave_max_dpp(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh.red_f[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = sh.red_f[0];
    for (int i = 1; i < SEL_T / 64; ++i) r = fmaxf(r, sh.red_f[i]);
    return r;
}
__device__ __forceinline__ double block_max_d(double v, SelShared &sh) {
    v = wave_max_f64_dpp(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh.red_d[threadIdx.x >> 6] = v;
    __syncthreads();
    double r = sh.red_d[0];
    for (int i = 1; i < SEL_T / 64; ++i) r = fmax(r, sh.red_d[i]);
    return r;
}
__device__ __forceinline__ uint64_t block_sum_u(uint64_t v, SelShared &sh) {
    v = wave_sum_u64_dpp(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh.red_u[threadIdx.x >> 6] = v;
    __syncthreads();
    uint64_t r = 0;
    for (int i = 0; i < SEL_T / 64; ++i) r += sh.red_u[i];
    return r;
}
__device__ __forceinline__ int block_sum_i(int v, SelShared &sh) {
    v = wave_sum_i32_dpp(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh.red_i[threadIdx.x >> 6] = v;
    __syncthreads();
    int r = 0;
    for (int i = 0; i < SEL_T / 64; ++i) r += sh.red_i[i];
    return r;
}

// Threshold selection over the keys key(b) = (val_b << 16) | (0xFFFF - b),
// unique per block, so "key desc" is the order (value desc, index asc).
// TOP: the largest threshold t with sum_{key >= t} val >= need (the fewest
// blocks reaching `need`).  REST: the largest t whose rest sum_{key < t} val
// satisfies E <= tol with no capped term left (the fewest blocks to
// promote).  Returns t; the chosen set is {key >= t}.
// Bucket passes over the current key range [lo, hi]: 64 buckets of width
// 2^shift spanning the range, per-bucket value sums, counts and largest key
// by LDS atomics; the bucket holding the threshold becomes the next range.
// A bucket with a single key whose exclusion was tested (not the last
// bucket) ends the search: that key is the threshold.
template <bool TOP, class P>
__device__ __forceinline__ uint64_t radix_select(P val, int N, uint64_t need, double tol, SelShared &sh) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // key range and total (REST: the empty set may already satisfy)
    uint64_t kmin = ~0ull, kmax = 0, tot = 0;
    uint32_t tsat = 0;
    for (int b = tid; b < N; b += SEL_T) {
        const uint64_t v = val[b];
        const uint64_t key = (v << 16) | (uint64_t)(0xFFFF - b);
        kmin = key < kmin ? key : kmin;
        kmax = key > kmax ? key : kmax;
        tot += v;
        tsat += (!TOP && v >= FXCAP);
    }
    kmin = wave_min_u64_dpp(kmin);
    kmax = wave_max_u64_dpp(kmax);
    tot = wave_sum_u64_dpp(tot);
    tsat = (uint32_t)wave_sum_i32_dpp((int)tsat);
    __syncthreads();
    if (lane == 0) {
        sh.red_u[wave] = kmin;
        sh.hkey[wave] = kmax;
        sh.hsum[wave] = tot;
        sh.hsat[wave] = tsat;
    }
    __syncthreads();
    kmin = ~0ull;
    kmax = 0;
    tot = 0;
    tsat = 0;
    for (int w = 0; w < SEL_T / 64; ++w) {
        kmin = sh.red_u[w] < kmin ? sh.red_u[w] : kmin;
        kmax = sh.hkey[w] > kmax ? sh.hkey[w] : kmax;
        tot += sh.hsum[w];
        tsat += sh.hsat[w];
    }
    // the empty set already satisfies: threshold above every key
    if (N == 0 || (TOP ? need == 0 : !(fx_bound(tot, tsat != 0) > tol))) return ~0ull;
    uint64_t lo = kmin, hi = kmax;
    uint64_t outside = 0;  // TOP: sum above [lo, hi]; REST: sum below
    uint32_t sat_out = 0;
    // the first pass buckets by value octave when the values span more than
    // 64x (linear buckets would put nearly every key in the lowest bucket)
    bool logp = ((kmax >> 16) >> 6) > (kmin >> 16);
    for (;;) {
        const uint64_t span = hi - lo;  // >= 0
        const int shift = span >> 6 ? 58 - __builtin_clzll(span) : 0;  // (span >> shift) < 64
        __syncthreads();
        if (tid < 64) {
            sh.hsum[tid] = 0;
            sh.hkey[tid] = 0;
            sh.hsat[tid] = 0;
            sh.hcnt[tid] = 0;
        }
        __syncthreads();
        for (int r0 = 0; r0 < N; r0 += SEL_T) {
            const int b = r0 + tid;
            uint64_t v = 0, key = 0;
            bool act = false;
            int dg = 0;
            if (b < N) {
                v = val[b];
                key = (v << 16) | (uint64_t)(0xFFFF - b);
                act = key >= lo && key <= hi;
                dg = logp ? (v ? 64 - __builtin_clzll(v) : 0) : (int)((key - lo) >> shift);
            }
            const uint64_t am = __ballot(act);
            if (!am) continue;
            const int first = __builtin_ctzll(am);
            const int d0 = __builtin_amdgcn_readlane(dg, first);
            if (__ballot(act && dg != d0) == 0) {
                // the wave's keys share one bucket: one update for the wave
                // (same-address atomics from every lane would serialize)
                const uint64_t sw = wave_sum_u64_dpp(act ? v : 0);
                const uint32_t ns = (uint32_t)__popcll(__ballot(act && !TOP && v >= FXCAP));
                if (lane == first) {
                    atomicAdd((unsigned long long *)&sh.hsum[d0], (unsigned long long)sw);
                    atomicAdd(&sh.hcnt[d0], (uint32_t)__popcll(am));
                    if (ns) atomicAdd(&sh.hsat[d0], ns);
                    sh.hkey[d0] = key;  // read only when the bucket holds one key
                }
            } else if (act) {
                atomicAdd((unsigned long long *)&sh.hsum[dg], (unsigned long long)v);
                atomicAdd(&sh.hcnt[dg], 1u);
                if (!TOP && v >= FXCAP) atomicAdd(&sh.hsat[dg], 1u);
                sh.hkey[dg] = key;
            }
        }
        __syncthreads();
        if (tid < 64) {
            const int dg = tid;
            const uint64_t s = sh.hsum[dg];
            const uint32_t cs = sh.hsat[dg];
            bool pred;
            uint64_t add = 0;
            uint32_t addc = 0;
            if (TOP) {
                // suffix sum over buckets >= dg
                const uint64_t suf = wave_suffix_u64(s, dg);
                pred = (outside + suf >= need) || dg == 0;
                add = suf - s;  // sum over buckets > dg
            } else {
                // exclusive prefix over buckets < dg
                const uint64_t pre = wave_prefix_excl_u64(s, dg);
                const uint32_t pc = wave_prefix_excl_u32(cs, dg);
                const uint64_t rem = outside + pre;
                const bool satr = (sat_out + pc) != 0;
                pred = !(fx_bound(rem, satr) > tol) || dg == 0;
                add = pre;
                addc = pc;
            }
            const uint64_t bal = __ballot(pred);
            const int best = 63 - __builtin_clzll(bal);  // largest bucket with pred
            if (dg == best) {
                sh.bc_u[0] = outside + add;
                sh.bc_u[2] = sh.hkey[best];
                sh.bc_i[0] = (int)(sat_out + addc);
                sh.bc_i[1] = (int)sh.hcnt[best];
                sh.bc_i[2] = best;
            }
        }
        __syncthreads();
        outside = sh.bc_u[0];
        sat_out = (uint32_t)sh.bc_i[0];
        const int cnt = sh.bc_i[1], best = sh.bc_i[2];
        const uint64_t kk = sh.bc_u[2];
        // the threshold: a single key in the chosen bucket whose exclusion was
        // tested, or the key value itself once buckets are single values
        if (cnt == 1 && best < 63) return kk;
        if (logp) {
            // octave `best` holds the values [2^(best-1), 2^best) (0: value 0)
            const uint64_t olo = best ? (1ull << (best - 1)) << 16 : 0;
            const uint64_t ohi = best ? ((1ull << best) << 16) - 1 : 0xFFFFull;
            lo = olo > lo ? olo : lo;
            hi = ohi < hi ? ohi : hi;
            logp = false;
            continue;
        }
        if (shift == 0) return lo + (uint64_t)best;
        const uint64_t nlo = lo + ((uint64_t)best << shift);
        const uint64_t nhi = nlo + ((1ull << shift) - 1);
        lo = nlo;
        hi = nhi < hi ? nhi : hi;
    }
}

// Delta and rho of a block from its statistics (max, l, Delta, rho) or from
// the LDS copy (Delta, rho).
__device__ __forceinline__ float sel_delta(const float4 &v) { return v.z; }
__device__ __forceinline__ float sel_rho(const float4 &v) { return v.w; }
__device__ __forceinline__ float sel_delta(const float2 &v) { return v.x; }
__device__ __forceinline__ float sel_rho(const float2 &v) { return v.y; }

template <class P>
__device__ __forceinline__ bool in_set(P val, int b, uint64_t thr) {
    return ((val[b] << 16) | (uint64_t)(0xFFFF - b)) >= thr;
}

template <int D, int G>
__global__ __launch_bounds__(SEL_T) void k_select(Layout Ly, Step St, Th th) {
    KernelClock kc(St.clk);
    __shared__ SelShared sh;
    const int h = blockIdx.x, n = blockIdx.y, tid = threadIdx.x;
    const int g = h / G, j = h % G, l = St.layer;
    const int len = __builtin_amdgcn_readfirstlane(Ly.len[l * Ly.B + n]);
    const int N = len / 64, has_part = (len % 64) != 0, Np = N + has_part;
    const size_t hs = (size_t)n * Ly.Hq + h;
    const float4 *bs = St.bstat + hs * St.NS;
    uint64_t *M = St.mfx + hs * St.NS;
    uint64_t *cv = St.cval + hs * St.NS;
    // the block statistics, annotations, fixed-point masses and E_val
    // contributions stay in LDS while the selections read them (global
    // memory beyond SEL_LDS blocks); their loads are issued together
    __shared__ uint64_t sM[SEL_LDS], sC[SEL_LDS];
    __shared__ float2 sDR[SEL_LDS];  // Delta, rho
    __shared__ float sEta[SEL_LDS];
    const bool in_lds = Np <= SEL_LDS;
    const float *etag = Ly.eta + Ly.blk(l, n, g, 0);
    constexpr int SPT = SEL_LDS / SEL_T;
    float4 stv[SPT];
    float etv[SPT];

    // estimated masses in fixed point
    float m = -INFINITY;
    if (in_lds) {
#pragma unroll
        for (int k = 0; k < SPT; ++k) {
            const int b = tid + k * SEL_T;
            if (b < Np) stv[k] = bs[b];
            if (b < N) etv[k] = etag[b];
        }
#pragma unroll
        for (int k = 0; k < SPT; ++k)
            if (tid + k * SEL_T < Np) m = fmaxf(m, stv[k].x);
    } else {
        for (int b = tid; b < Np; b += SEL_T) m = fmaxf(m, bs[b].x);
    }
    const float mref = block_max_f(m, sh);
    uint64_t s = 0;
    auto mass = [&](const float4 &st) {
        const float mh = st.y * exp_c(st.x - mref);
        return (uint64_t)((double)mh * 4294967296.0);
    };
    if (in_lds) {
#pragma unroll
        for (int k = 0; k < SPT; ++k) {
            const int b = tid + k * SEL_T;
            if (b < Np) {
                const uint64_t Mb = mass(stv[k]);
                M[b] = Mb;
                sM[b] = Mb;
                sDR[b] = make_float2(stv[k].z, stv[k].w);
                s += Mb;
            }
            if (b < N) sEta[b] = etv[k];
        }
    } else {
        for (int b = tid; b < Np; b += SEL_T) {
            const uint64_t Mb = mass(bs[b]);
            M[b] = Mb;
            s += Mb;
        }
    }
    const uint64_t S = block_sum_u(s, sh);
    const uint64_t Mpart = has_part ? M[N] : 0;

    // range of V for this kv head: R = max_c (max - min), rounded up
    double rr = 0.0;
    for (int c = tid; c < D; c += SEL_T) {
        const size_t vi = Ly.seqg(l, n, g) * D + c;
        rr = fmax(rr, (double)ord2f(Ly.vmax[vi]) - (double)ord2f(Ly.vmin[vi]));
    }
    const double R = (double)ru32(block_max_d(rr, sh));

    const double Sd = (double)S;
    auto phat = [&](uint64_t Mb) { return ((double)(Mb + 1) / Sd) * (1.0 + 0x1p-16); };

    auto body = [&](auto *Mv, auto *Cv, auto *DRv, auto *Ev) {
        double tau = (double)th.tau;
        int widened = 0, cap_fail = 0;
        uint64_t thrP = ~0ull;
        double F = 1.0, mu = 0.0, tv = 1.0, ekey = 0.0;
        for (int wv = 0;; ++wv) {
            const uint64_t T = (uint64_t)ceil(tau * Sd);
            const uint64_t need = T > Mpart ? T - Mpart : 0;
            thrP = radix_select<true>(Mv, N, need, 0.0, sh);
            // F = exp(max over P of (Delta + rho))
            double fm = 0.0;
            for (int b = tid; b < N; b += SEL_T)
                if (in_set(Mv, b, thrP)) fm = fmax(fm, (double)sel_delta(DRv[b]) + (double)sel_rho(DRv[b]));
            F = expu(block_max_d(fm, sh));
            uint64_t sum = 0;
            int sat = 0;
            double dmax = 0.0;
            for (int b = tid; b < N; b += SEL_T) {
                const double dz = (double)sel_delta(DRv[b]), rh = (double)sel_rho(DRv[b]);
                const bool p = in_set(Mv, b, thrP);
                const double dl = p ? rh : dz;
                const double X = p ? expu(dz + rh) : 1.0;
                const uint64_t u = fx(phat(Mv[b]) * F * X * em1u(dl) * (1.0 + 0x1p-48));
                sat |= (u == FXCAP);
                sum += u;
                dmax = fmax(dmax, dl);
            }
            if (has_part && tid == 0) {
                const double dl = (double)bs[N].w;
                const uint64_t u = fx(phat(M[N]) * F * 1.0 * em1u(dl) * (1.0 + 0x1p-48));
                sat |= (u == FXCAP);
                sum += u;
                dmax = fmax(dmax, dl);
            }
            sum = block_sum_u(sum, sh);
            sat = block_sum_i(sat, sh);
            dmax = block_max_d(dmax, sh);
            mu = fx_bound(sum, sat != 0);
            tv = 1.0;
            if (mu < 1.0) tv = mu / (1.0 - mu) * (1.0 + 0x1p-48);
            const double thb = tanhu(dmax);
            if (thb < tv) tv = thb;
            if (tv > 1.0) tv = 1.0;
            ekey = tv * R * (1.0 + 0x1p-50);
            if (!(ekey > (double)th.k_tol)) break;
            if (wv >= th.n_widen) {
                cap_fail = 1;
                break;
            }
            tau = 1.0 - (1.0 - tau) * 0.5;
            widened = 1;
        }

        // E_val contributions with the final P; rung 2 by radix select
        uint64_t tot = 0;
        int satv = 0;
        for (int b = tid; b < N; b += SEL_T) {
            const bool p = in_set(Mv, b, thrP);
            const double X = p ? expu((double)sel_delta(DRv[b]) + (double)sel_rho(DRv[b])) : 1.0;
            const double e = (double)Ev[b];
            const uint64_t u = fx(phat(Mv[b]) * F * X * e * (1.0 + 0x1p-48));
            Cv[b] = u;
            tot += u;
            satv |= (u == FXCAP);
        }
        __syncthreads();
        const uint64_t thrV = radix_select<false>(Cv, N, 0, (double)th.v_tol, sh);
        uint64_t rest = 0;
        int nvp = 0, kst = 0, satr = 0;
        for (int b = tid; b < N; b += SEL_T) {
            const bool v = in_set(Cv, b, thrV);
            const bool p = in_set(Mv, b, thrP);
            nvp += v;
            kst += p;
            if (!v) {
                rest += Cv[b];
                satr |= (Cv[b] == FXCAP);
            }
            const uint32_t bits = (p ? (1u << j) : 0u) | (v ? (1u << (8 + j)) : 0u);
            if (bits) atomicOr(&St.sel[((size_t)n * Ly.Hkv + g) * Ly.Nmax + b], bits);
        }
        rest = block_sum_u(rest, sh);
        nvp = block_sum_i(nvp, sh);
        kst = block_sum_i(kst, sh);
        satr = block_sum_i(satr, sh);
        const double eval = fx_bound(rest, satr != 0);
        if ((th.vcap > 0 && nvp > th.vcap) || eval > (double)th.v_tol) cap_fail = 1;
        (void)tot;
        (void)satv;
        if (tid == 0) {
            HeadPlan P;
            P.mu = mu;
            P.tv = tv;
            P.ekey = ekey;
            P.eval = eval;
            P.tau = tau;
            P.mref = mref;
            P.mref16 = mref;
            P.kstar = kst;
            P.nvp = nvp;
            P.flags = widened | (cap_fail << 1);
            P.rank_ok = -1;
            P.ndisc = 0;
            P.S = S;
            St.plan[hs] = P;
        }
    };
    __syncthreads();
    if (in_lds) body(sM, sC, sDR, sEta); else body(M, cv, bs, etag);
}

// ===========================================================================
// Value passes (tail, promoted, dense): a wave covers one 64-token block and
// contracts the softmax weights with the values on the matrix cores
// (v_mfma_f32_16x16x32_f16; output path only, FP32 accumulation).
//
// Rows r = gv * G + h (value group gv of 32 channels, q head h), columns =
// channels, k = tokens.  Lane l holds, for k-step ks, 8 tokens of
// 16 (l / 16) + 8 ks + (0 .. 7) of A row / B column l % 16; accumulator
// tile (rt, nt) holds rows 16 rt + 4 (l / 16) + i, i < 4, of column
// 16 nt + l % 16.  Only rows whose group is the column's group are kept.
//
// The online softmax runs in the A layout: lane l holds the scores of the
// row's head for its 16 tokens, so the weights never leave the registers.
//
// INT4 values: an INT4 code n taken as FP16 bits is the subnormal n 2^-24,
// exact; masking a word of eight codes (token i at bits 4i) with 0x000F000F
// gives tokens (0, 4), with 0x00F000F0 tokens (1, 5) as 16 n 2^-24, and the
// same on the word shifted by 8 gives (2, 6), (3, 7).  The A weight is
// a = p s K (the odd registers a / 16), K = 2^k a per-group power of two
// that keeps a below 2^15 (from the running value range, which bounds every
// INT4 scale of the group); acc then holds sum p s n K 2^-24, and the
// offsets enter through z-sums sum_t p_t z_t kept per A row.
// FP16 values: B is the value itself and a = p K16, K16 = 2^14, in acc16.
// Weights are split into FP16 hi + lo parts (relative error <= 2^-20 above
// 2^-14, absolute <= 2^-24 below).
// A workgroup has four waves on four blocks; their states are combined
// through LDS at the end.
// ===========================================================================
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// 8 FP16 values (one 16-byte load) as FP32.
__device__ __forceinline__ void unpack_fp16x8(const uint4 &u, float (&v)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = h2f((uint16_t)(w[i / 2] >> (16 * (i & 1))));
}

// Eight INT4 codes of one word as an FP16 operand of subnormals: register r
// holds tokens (r, r + 4), scaled by 16 for odd r.
__device__ __forceinline__ v8h int4_operand(uint32_t w) {
    const uint32_t w8 = w >> 8;
    const v4u r = {w & 0x000F000Fu, w & 0x00F000F0u, w8 & 0x000F000Fu, w8 & 0x00F000F0u};
    return __builtin_bit_cast(v8h, r);
}

// Eight INT8 codes (tokens 0-3 in lo, 4-7 in hi, one byte each) as an FP16
// operand of subnormals in the same token order as int4_operand: register r
// holds tokens (r, r + 4), unscaled.
__device__ __forceinline__ v8h int8_operand(uint32_t lo, uint32_t hi) {
    const v4u r = {__builtin_amdgcn_perm(hi, lo, 0x0C040C00u), __builtin_amdgcn_perm(hi, lo, 0x0C050C01u),
                   __builtin_amdgcn_perm(hi, lo, 0x0C060C02u), __builtin_amdgcn_perm(hi, lo, 0x0C070C03u)};
    return __builtin_bit_cast(v8h, r);
}

// Value codes of one channel for a lane's 16 tokens: INT4 (8 bytes) or
// INT8 (16 bytes).
template <bool V8>
using CodeWord = typename std::conditional<V8, uint4, uint2>::type;

// x = hi + lo + err with FP16 hi, lo (round toward zero);
// |err| <= max(2^-20 |x|, 2^-24).
__device__ __forceinline__ void split_pair(float x, float y, uint32_t &hi, uint32_t &lo) {
    const auto h = __builtin_amdgcn_cvt_pkrtz(x, y);
    const auto w = __builtin_amdgcn_cvt_pkrtz(fmaf((float)h[0], -1.0f, x), fmaf((float)h[1], -1.0f, y));
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, w);
}

constexpr float K16 = 0x1p14f;  // weight scale of FP16 values

template <int D, int G, bool F16ACC>
struct VAcc {
    static constexpr int NG = D / 32;         // value groups
    static constexpr int R = NG * G;          // rows (group, head)
    static constexpr int RT = (R + 15) / 16;  // row tiles
    static constexpr int NT = D / 16;         // column tiles
    static constexpr int RT16 = F16ACC ? RT : 1;
    v4f acc[RT][NT];      // INT4 values (FP16 values when !F16ACC)
    v4f acc16[RT16][NT];  // FP16 values (F16ACC)
    float zacc[RT];       // sum p z of the A row
    float mrow[RT], lrow[RT];  // online softmax of the A row's head

    __device__ __forceinline__ void init() {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            zacc[rt] = 0.0f;
            mrow[rt] = -INFINITY;
            lrow[rt] = 0.0f;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[rt][nt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        }
#pragma unroll
        for (int rt = 0; rt < RT16; ++rt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc16[rt][nt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }
    static __device__ __forceinline__ int arow(int rt, int lane) { return 16 * rt + (lane & 15); }
    static __device__ __forceinline__ int ahead(int rt, int lane) { return arow(rt, lane) % G; }
    static __device__ __forceinline__ int agroup(int rt, int lane) { return min(arow(rt, lane) / G, NG - 1); }

    // Online softmax over one block.  sv[rt][i]: score of the A row's head
    // for token 16 (lane / 16) + i, -inf where the token is invalid or the
    // head takes no part; replaced by the weights.  Rescales the state.
    __device__ __forceinline__ void softmax(float (&sv)[RT][16], int lane) {
        float sc[RT];
        bool resc = false;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float bm = sv[rt][0];
#pragma unroll
            for (int i = 1; i < 16; ++i) bm = fmaxf(bm, sv[rt][i]);
            bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
            bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
            const float mn = fmaxf(mrow[rt], bm);
            sc[rt] = mn == mrow[rt] ? 1.0f : __expf(mrow[rt] - mn);
            resc |= sc[rt] != 1.0f;
            // p = 2^(s log2e - mn log2e); a row with no part has mn = -inf and
            // only -inf scores, which give 0 against a finite offset
            const float off = mn == -INFINITY ? 0.0f : -mn * 1.44269504088896341f;
            float ls = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = __builtin_amdgcn_exp2f(fmaf(sv[rt][i], 1.44269504088896341f, off));
                sv[rt][i] = p;
                ls += p;
            }
            ls += __shfl_xor(ls, 16, 64);
            ls += __shfl_xor(ls, 32, 64);
            lrow[rt] = fmaf(lrow[rt], sc[rt], ls);
            mrow[rt] = mn;
            zacc[rt] *= sc[rt];
        }
        if (__builtin_amdgcn_ballot_w64(resc)) {
            // factor of head h: lane h (row h of the first tile) holds it
            float scH[G];
#pragma unroll
            for (int h = 0; h < G; ++h) scH[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc[0]), h));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float f = G <= 4 ? scH[i % G] : ((lane >> 4) & 1 ? scH[(4 + i) % G] : scH[i % G]);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) acc[rt][nt][i] *= f;
#pragma unroll
                for (int rt = 0; rt < RT16; ++rt)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        if (F16ACC) acc16[rt][nt][i] *= f;
            }
        }
    }
    // INT4 (INT8 if V8) values for the heads in `mask`.  p: weights (A
    // layout); cw[nt]: the codes of channel 16 nt + lane % 16 for tokens
    // 16 (lane / 16) + 0..15; mt[rt]: scale | offset words of the A row's
    // group for the same tokens.
    template <bool V8>
    __device__ __forceinline__ void int4_block(uint32_t mask, const float (&p)[RT][16], const v4u (&mt)[RT][4],
                                               const CodeWord<V8> (&cw)[NT], const float *ksg, int lane) {
        v8h ahi[RT][2], alo[RT][2];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const bool on = arow(rt, lane) < R && (mask & (1u << ahead(rt, lane)));
            const float K = on ? ksg[agroup(rt, lane)] : 0.0f;
            float a[16];
            float z = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint32_t mw = mt[rt][i / 4][i % 4];
                const float s = h2f((uint16_t)(mw & 0xFFFFu)), zz = h2f((uint16_t)(mw >> 16));
                // INT4: odd registers of the operand (tokens 1, 3, 5, 7 of
                // each 8) carry codes scaled by 16
                a[i] = (p[rt][i] * s) * ((!V8 && (i & 1)) ? K * 0.0625f : K);
                z = fmaf(p[rt][i], zz, z);
            }
            zacc[rt] += on ? z : 0.0f;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                v4u hi, lo;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    uint32_t x, y;
                    split_pair(a[8 * ks + r], a[8 * ks + r + 4], x, y);
                    hi[r] = x;
                    lo[r] = y;
                }
                ahi[rt][ks] = __builtin_bit_cast(v8h, hi);
                alo[rt][ks] = __builtin_bit_cast(v8h, lo);
            }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            v8h b0, b1;
            if constexpr (V8) {
                b0 = int8_operand(cw[nt].x, cw[nt].y);
                b1 = int8_operand(cw[nt].z, cw[nt].w);
            } else {
                b0 = int4_operand(cw[nt].x);
                b1 = int4_operand(cw[nt].y);
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                v4f c = acc[rt][nt];
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[rt][0], b0, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[rt][0], b0, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[rt][1], b1, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[rt][1], b1, c, 0, 0, 0);
                acc[rt][nt] = c;
            }
        }
    }
    // FP16 values for the heads in `mask`.  vv[nt][ks]: tokens
    // 16 (lane / 16) + 8 ks + (0 .. 7) of channel 16 nt + lane % 16.
    __device__ __forceinline__ void fp16_block(uint32_t mask, const float (&p)[RT][16], const uint4 (&vv)[NT][2],
                                               int lane) {
        v8h ahi[RT][2], alo[RT][2];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const bool on = arow(rt, lane) < R && (mask & (1u << ahead(rt, lane)));
            const float K = on ? K16 : 0.0f;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                v4u hi, lo;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    uint32_t x, y;
                    split_pair(p[rt][8 * ks + 2 * r] * K, p[rt][8 * ks + 2 * r + 1] * K, x, y);
                    hi[r] = x;
                    lo[r] = y;
                }
                ahi[rt][ks] = __builtin_bit_cast(v8h, hi);
                alo[rt][ks] = __builtin_bit_cast(v8h, lo);
            }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const v8h b0 = __builtin_bit_cast(v8h, vv[nt][0]), b1 = __builtin_bit_cast(v8h, vv[nt][1]);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                v4f c = F16ACC ? acc16[F16ACC ? rt : 0][nt] : acc[rt][nt];
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[rt][0], b0, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[rt][0], b0, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[rt][1], b1, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[rt][1], b1, c, 0, 0, 0);
                if (F16ACC) acc16[F16ACC ? rt : 0][nt] = c; else acc[rt][nt] = c;
            }
        }
    }
};

// A lane's share of a block's value scale | offset words: D / 32 words
// (the block holds 2 D words).
template <int D>
using MetaWord = typename std::conditional<D == 128, v4u, uint2>::type;

// Tier-1 value operands of one block for this lane, through buffer
// resources over the (sequence, kv head)'s blocks (rq: codes, rm: scale |
// offset words) at block offsets cb, mb (RSRC_OOB: loads zeros from
// nowhere): INT4 codes (channel-major, 32 bytes per channel; INT8 if V8: 64
// bytes per channel) and this lane's share of the scale | offset words
// (group-major, 64 words per group), one load per lane; the words reach the
// lanes that use them through LDS (vmeta_rows).
template <int D, int G, bool F, bool V8>
__device__ __forceinline__ void load_int4(__amdgpu_buffer_rsrc_t rq, __amdgpu_buffer_rsrc_t rm, uint32_t cb,
                                          uint32_t mb, int lane, CodeWord<V8> (&cw)[D / 16], MetaWord<D> &mw) {
    using VA = VAcc<D, G, F>;
    if constexpr (V8) {
        // [d][64]: channel 16 nt + lane % 16, tokens 16 (lane / 16) .. + 15
#pragma unroll
        for (int nt = 0; nt < VA::NT; ++nt)
            cw[nt] = rsrc_load16(rq, cb + (uint32_t)((16 * nt + (lane & 15)) * 64 + 16 * (lane >> 4)));
    } else {
        // [d/32][64][16]: one 16-byte load per lane and channel pair gives
        // the codes of column tiles 2 p and 2 p + 1 for the lane's tokens
#pragma unroll
        for (int p = 0; p < VA::NT / 2; ++p) {
            const uint4 w = rsrc_load16(rq, cb + (uint32_t)(p * 1024 + lane * 16));
            cw[2 * p] = make_uint2(w.x, w.y);
            cw[2 * p + 1] = make_uint2(w.z, w.w);
        }
    }
    if constexpr (D == 128) {
        const uint4 w = rsrc_load16(rm, mb + lane * 16);
        mw = v4u{w.x, w.y, w.z, w.w};
    } else {
        mw = rsrc_load8(rm, mb + lane * 8);
    }
}

// The scale | offset words of the A rows' groups for this lane's 16 tokens,
// from the block's words in LDS (vms: 2 D words).
template <int D, int G, bool F>
__device__ __forceinline__ void vmeta_rows(const uint32_t *vms, int lane, v4u (&mt)[VAcc<D, G, F>::RT][4]) {
    using VA = VAcc<D, G, F>;
#pragma unroll
    for (int rt = 0; rt < VA::RT; ++rt) {
        const v4u *src = reinterpret_cast<const v4u *>(vms + VA::agroup(rt, lane) * 64 + 16 * (lane >> 4));
#pragma unroll
        for (int i = 0; i < 4; ++i) mt[rt][i] = src[i];
    }
}

// FP16 value operands of a channel-major block [D][64].
template <int D>
__device__ __forceinline__ void load_fp16v(const uint16_t *vb, int lane, uint4 (&vv)[D / 16][2]) {
#pragma unroll
    for (int nt = 0; nt < D / 16; ++nt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            vv[nt][ks] = *reinterpret_cast<const uint4 *>(vb + (16 * nt + (lane & 15)) * 64 +
                                                          16 * (lane >> 4) + 8 * ks);
}
// The same through a buffer resource at byte offset vb (RSRC_OOB: zeros).
template <int D>
__device__ __forceinline__ void load_fp16v(__amdgpu_buffer_rsrc_t r, uint32_t vb, int lane, uint4 (&vv)[D / 16][2]) {
#pragma unroll
    for (int nt = 0; nt < D / 16; ++nt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            vv[nt][ks] = rsrc_load16(r, vb + (uint32_t)(((16 * nt + (lane & 15)) * 64 + 16 * (lane >> 4) + 8 * ks) * 2));
}

// Scores of the A rows' heads for this lane's 16 tokens (four 16-byte reads
// per row tile) from a per-head array with stride hstride floats (base1 for
// the heads in sel1, base0 for the others).
template <int D, int G, bool F>
__device__ __forceinline__ void load_scores(const float *base0, const float *base1, uint32_t sel1,
                                            size_t hstride, int lane, float (&sv)[VAcc<D, G, F>::RT][16]) {
    using VA = VAcc<D, G, F>;
#pragma unroll
    for (int rt = 0; rt < VA::RT; ++rt) {
        const int h = VA::ahead(rt, lane);
        const float *src = ((sel1 >> h) & 1 ? base1 : base0) + h * hstride + 16 * (lane >> 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 x = reinterpret_cast<const float4 *>(src)[i];
            sv[rt][4 * i] = x.x;
            sv[rt][4 * i + 1] = x.y;
            sv[rt][4 * i + 2] = x.z;
            sv[rt][4 * i + 3] = x.w;
        }
    }
}

// Marks the tokens >= np (an unfinished block) and the rows whose head is
// not in `use` as taking no part.
template <int D, int G, bool F>
__device__ __forceinline__ void mask_scores(uint32_t use, int np, int lane, float (&sv)[VAcc<D, G, F>::RT][16]) {
    using VA = VAcc<D, G, F>;
#pragma unroll
    for (int rt = 0; rt < VA::RT; ++rt) {
        const bool on = VA::arow(rt, lane) < VA::R && (use & (1u << VA::ahead(rt, lane)));
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (!on || 16 * (lane >> 4) + i >= np) sv[rt][i] = -INFINITY;
    }
}

// Write one partial (m, l, acc[D]) per head of the group to
// part + (head * pstride + sp) * (D + 2), combining the four waves.
template <int D, int G, bool F>
__device__ __forceinline__ void write_partials(VAcc<D, G, F> &va, const float *ksg, float *part,
                                               size_t hbase, size_t pstride, int sp,
                                               uint32_t heads_mask, bool int4) {
    using VA = VAcc<D, G, F>;
    __shared__ float sm_m[4][G], sm_l[4][G];
    __shared__ float sm_acc[4][G][D];
    __shared__ float sm_z[4][VA::RT * 16];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, kg = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < VA::RT; ++rt) {
        float z = va.zacc[rt];
        z += __shfl_xor(z, 16, 64);
        z += __shfl_xor(z, 32, 64);
        if (lane < 16) sm_z[wave][16 * rt + lane] = z;
    }
    wave_sync();
    // column tile nt belongs to value group nt / 2; the rows of that group
    // hold its heads (accumulator indices stay compile-time constants)
#pragma unroll
    for (int nt = 0; nt < VA::NT; ++nt) {
        // INT4 values are in units of 2^-24 / K, FP16 values in units of 1 / K16
        const float inv = int4 ? 0x1p24f / ksg[nt / 2] : 1.0f / ksg[nt / 2];
#pragma unroll
        for (int rt = 0; rt < VA::RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * rt + 4 * kg + i;
                if (r < VA::R && r / G == nt / 2) {
                    float v = fmaf(va.acc[rt][nt][i], inv, sm_z[wave][r]);
                    if (F) v = fmaf(va.acc16[F ? rt : 0][nt][i], 1.0f / K16, v);
                    sm_acc[wave][r % G][16 * nt + (lane & 15)] = v;
                }
            }
    }
    // the softmax state of head h sits in lane h (row h of the first tile)
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(va.mrow[0]), h));
        const float l = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(va.lrow[0]), h));
        if (lane == 0) {
            sm_m[wave][h] = m;
            sm_l[wave][h] = l;
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < G * (D + 2); e += 256) {
        const int j = e / (D + 2), c = e % (D + 2);
        if (!(heads_mask & (1u << j))) continue;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][j]);
        float r;
        if (c == 0) {
            r = M;
        } else {
            r = 0.0f;
            if (M != -INFINITY) {
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    if (sm_m[w][j] == -INFINITY) continue;
                    const float e_ = __expf(sm_m[w][j] - M);
                    r = fmaf(e_, c == 1 ? sm_l[w][j] : sm_acc[w][j][c - 2], r);
                }
            }
        }
        part[((hbase + j) * pstride + sp) * (D + 2) + c] = r;
    }
}

// ===========================================================================
// K3 (k_tail) / K4a values (k_promoted4, k_promoted16): split-K flash
// decoding over one split of blocks of a (kv head, sequence); 256 threads,
// one wave per block, two blocks in flight per wave.
//   VP_TAIL   heads outside P and VP [Meth-3: the blocks not promoted keep
//             their INT8 keys]: INT8 scores, INT4 values.
//   VP_INT4   heads of P without FP16 values: FP16-key scores (k_keys16),
//             INT4 values.
//   VP_FP16   heads of VP (FP16-key scores on P, else INT8 scores) and every
//             head of the unfinished block (FP16 scores from the scoring
//             pass): FP16 values from the staging area / the device.
// Output path only: hardware exp and any summation order are allowed here.
// ===========================================================================
enum { VP_TAIL = 0, VP_INT4 = 1, VP_FP16 = 2 };

template <int D, int G, int MODE, bool V8>
__device__ __forceinline__ void values_pass(const Layout &Ly, const Step &St, const int *skip_seq) {
    constexpr bool F16 = MODE == VP_FP16;
    using VA = VAcc<D, G, false>;
    const int sp = blockIdx.x, g = blockIdx.y, n = blockIdx.z;
    // wave index as a uniform value: the block loop below branches uniformly
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int l = St.layer;
    // uniform words through the constant address space (scalar loads,
    // requested together; none is written during this kernel)
    typedef const __attribute__((address_space(4))) int cint;
    if (MODE != VP_TAIL && ((cint *)skip_seq)[n]) return;
    if (F16 && (n * Ly.Hkv + g < St.p16_lo || n * Ly.Hkv + g >= St.p16_hi)) return;  // another launch's pair
    const int len = ((cint *)Ly.len)[l * Ly.B + n];
    const int N = len / 64, np = len % 64;
    const int nslot = F16 ? N + (np ? 1 : 0) : N;
    constexpr uint32_t ALL = (1u << G) - 1u;
    __shared__ float ksg[VA::NG];
    __shared__ uint32_t sbits[MAX_BPS], sblk[MAX_BPS];
    __shared__ __attribute__((aligned(16))) float st[4][G][64];
    __shared__ __attribute__((aligned(16))) uint32_t vms[F16 ? 1 : 4][F16 ? 4 : 2 * D];
    const size_t selbase = ((size_t)n * Ly.Hkv + g) * Ly.Nmax;
    // The blocks of this split: an equal share of the pass's block list, over
    // as many splits as the block range [0, nslot) has of bps blocks (the
    // partials the merge reads); every listed block serves some head here.
    int ne, e0;
    {
        const size_t ng = (size_t)n * Ly.Hkv + g, nk = (size_t)Ly.B * Ly.Hkv;
        const int kind = MODE == VP_TAIL ? WL_TAIL : F16 ? WL_FP16 : WL_INT4;
        const int cnt = ((cint *)St.wcnt)[kind * nk + ng];
        // the tail: splits of bps blocks of the context; the promoted passes:
        // splits by the length of the pair's list (the merge reads as many)
        const int tpe = F16 ? St.t16 : St.t4;
        const int nsp = MODE == VP_TAIL ? (nslot + St.bps - 1) / St.bps : (cnt + tpe - 1) / tpe;
        if (MODE != VP_TAIL && sp >= nsp) return;  // the whole workgroup; no partial is read for it
        e0 = sp < nsp ? (int)((long long)sp * cnt / nsp) : cnt;
        const int e1 = sp < nsp ? (int)((long long)(sp + 1) * cnt / nsp) : cnt;
        ne = min(e1 - e0, MAX_BPS);
        const uint32_t *lst = St.wl + (kind * nk + ng) * (size_t)(Ly.Nmax + 1);
        // block indices and selection bits of the split, one load each
        for (int i = threadIdx.x; i < ne; i += 256) {
            const uint32_t e = lst[e0 + i];
            sblk[i] = e & 0xFFFFu;
            sbits[i] = e >> 16;
        }
    }
    if (threadIdx.x < VA::NG) ksg[threadIdx.x] = F16 ? K16 : Ly.vscale[Ly.seqg(l, n, g) * VA::NG + threadIdx.x];
    __syncthreads();
    const size_t NS64 = (size_t)St.NS * 64;
    VA va;
    va.init();
    struct Blk {
        uint32_t pm, use;
        int b, li;  // block, index in the pass's list of the pair
        bool part, valid;
    };
    struct Opd {
        uint4 vv[F16 ? VA::NT : 1][2];
        CodeWord<V8> cw[F16 ? 1 : VA::NT];
        MetaWord<D> mw;
        float s[G];  // scores, lane = token
    };
    // entry i of the split: block, heads of P, heads whose values it serves;
    // past the split's entries: no block (its loads read nothing)
    auto plan = [&](int i) {
        Blk k;
        k.valid = i < ne;
        k.b = k.valid ? (int)__builtin_amdgcn_readfirstlane(sblk[i]) : 0;
        k.li = e0 + (k.valid ? i : 0);
        k.part = F16 && k.valid && k.b == N;
        k.pm = 0;
        k.use = k.valid ? ALL : 0u;
        if (k.valid && !k.part) {
            const uint32_t bits = __builtin_amdgcn_readfirstlane(sbits[i]);
            k.pm = bits & ALL;
            const uint32_t vm = (bits >> 8) & ALL;
            k.use = MODE == VP_TAIL ? (~(k.pm | vm) & ALL) : MODE == VP_INT4 ? (k.pm & ~vm) : vm;
        }
        return k;
    };
    // the scores of the group's heads as buffer resources (uniform bases, a
    // 32-bit offset per lane)
    const size_t srow = (size_t)(n * Ly.Hq + g * G) * NS64;
    const uint32_t sbytes = (uint32_t)(G * NS64 * 4);
    const __amdgpu_buffer_rsrc_t rs8 = make_rsrc(St.score + srow, sbytes);
    const __amdgpu_buffer_rsrc_t rs16 = make_rsrc(St.score16 + srow, sbytes);
    // the block operands of the (sequence, kv head) as buffer resources
    constexpr uint32_t CBLK = D * (V8 ? 64 : 32), MBLK = 64 * (D / 32) * 4, FBLK = 64 * D * 2;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Ly.vq + Ly.blk(l, n, g, 0) * CBLK, (uint32_t)Ly.Nmax * CBLK);
    const __amdgpu_buffer_rsrc_t rm = make_rsrc(Ly.vmeta + Ly.blk(l, n, g, 0) * (MBLK / 4), (uint32_t)Ly.Nmax * MBLK);
    // FP16 values: packed slot vpref + list index, or (pair, block)
    const size_t vbase = St.packed && F16 ? (size_t)((cint *)St.vpref)[selbase / Ly.Nmax] : 0;
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(Ly.vpart + Ly.seqg(l, n, g) * 64 * D, FBLK);
    auto issue = [&](const Blk &k, Opd &o) {
        const int b = k.b;
        if constexpr (F16) {
            const size_t slot = St.packed ? vbase + (size_t)k.li : selbase + (size_t)b;
            const __amdgpu_buffer_rsrc_t rv = make_rsrc(St.stage_v + slot * 64 * D, FBLK);
            load_fp16v<D>(k.part ? rp : rv, !k.valid ? RSRC_OOB : 0u, lane, o.vv);
        }
        else
            load_int4<D, G, false, V8>(rq, rm, k.valid ? (uint32_t)b * CBLK : RSRC_OOB,
                                       k.valid ? (uint32_t)b * MBLK : RSRC_OOB, lane, o.cw, o.mw);
        // scores of the group's heads: the FP16-key ones on P (promoted
        // passes), the INT8 ones elsewhere, zero for heads not served here
        // (an offset past the range: no memory access)
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const bool f16 = MODE != VP_TAIL && (k.pm & (1u << j));
            const uint32_t off = (k.use & (1u << j)) ? (uint32_t)j * (uint32_t)(NS64 * 4) + (uint32_t)b * 256u : RSRC_OOB;
            o.s[j] = rsrc_load_f32(f16 ? rs16 : rs8, off + lane * 4);
        }
    };
    // Softmax weights against a fixed reference per head, at least every
    // score the pass uses: the largest INT8 block estimate M^ (INT8 scores,
    // and the unfinished block's FP16 scores, are <= M^) for the tail; for
    // the promoted passes also the largest FP16-key block max over P (from
    // the rank check).  So p = e^(s - m) <= 1: the weights never overflow
    // (the weight scales of the matrix-core operands assume p <= 1) and
    // need no rescaling.  The merge rescales partials of different m.  The
    // sum of the weights accumulates per lane (token) and is reduced once
    // at the end.
    float mh[G], lt[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const HeadPlan &P = St.plan[(size_t)n * Ly.Hq + g * G + j];
        mh[j] = MODE == VP_TAIL ? P.mref : P.mref16;
        lt[j] = 0.0f;
    }
    auto consume = [&](const Blk &k, Opd &o) {
        // weights (lane = token) of the heads this block serves, 0 for the
        // others and past an unfinished block's end; to the A layout
        // through LDS, with the block's value scales and offsets
        const bool tok = !k.part || lane < np;
        wave_sync();  // the wave's previous block has read st and vms
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const float e = __builtin_amdgcn_exp2f((o.s[j] - mh[j]) * 1.44269504088896341f);
            const float w = tok && ((k.use >> j) & 1u) ? e : 0.0f;
            lt[j] += w;
            st[wave][j][lane] = w;
        }
        if constexpr (!F16) *reinterpret_cast<MetaWord<D> *>(&vms[wave][lane * (D / 32)]) = o.mw;
        wave_sync();
        float sv[VA::RT][16];
        load_scores<D, G, false>(&st[wave][0][0], &st[wave][0][0], 0u, 64, lane, sv);
        if constexpr (F16)
            va.fp16_block(k.use, sv, o.vv, lane);
        else
        {
            v4u mt[VA::RT][4];
            vmeta_rows<D, G, false>(&vms[wave][0], lane, mt);
            va.template int4_block<V8>(k.use, sv, mt, o.cw, ksg, lane);
        }
    };
    // entries wave, wave + 4, ...: the next entry's operands in flight
    // while the current one is used.  Every path makes the same requests
    // (entries past the wave's share load zeros from nowhere) and consume
    // makes none, so the wait before each use covers exactly its block.
    const int nw = ne > wave ? (ne - wave + 3) / 4 : 0;
    Opd o0, o1;
    Blk k0 = plan(wave), k1;
    issue(k0, o0);
    for (int t = 0; t < nw; t += 2) {
        k1 = plan(wave + 4 * (t + 1));
        issue(k1, o1);
        consume(k0, o0);
        k0 = plan(wave + 4 * (t + 2));
        issue(k0, o0);
        if (t + 1 < nw) consume(k1, o1);
    }
    // the fixed max and the weight sums of the A rows' heads, for the
    // partials (row h of the first tile lies in lane h)
    {
        float L[G];
#pragma unroll
        for (int j = 0; j < G; ++j) L[j] = wave_sum_dpp(lt[j]);
#pragma unroll
        for (int rt = 0; rt < VA::RT; ++rt) {
            const int h = VA::ahead(rt, lane);
            float m = mh[0], l_ = L[0];
#pragma unroll
            for (int j = 1; j < G; ++j) {
                m = h == j ? mh[j] : m;
                l_ = h == j ? L[j] : l_;
            }
            va.mrow[rt] = m;
            va.lrow[rt] = l_;
        }
    }
    float *part = MODE == VP_TAIL ? St.part_tail : MODE == VP_INT4 ? St.part_blk : St.part_blk16;
    write_partials<D, G, false>(va, ksg, part, (size_t)n * Ly.Hq + g * G, St.nsplit_cap, sp, ALL, !F16);
}

// Three waves per SIMD where the registers allow (INT4 codes, G d <= 512).
template <int D, int G, bool V8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(!V8 && G * D <= 512 ? 3 : 2))) void k_tail(Layout Ly, Step St) {
    KernelClock kc(St.clk);
    values_pass<D, G, VP_TAIL, V8>(Ly, St, nullptr);
}

template <int D, int G, bool V8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(!V8 && G * D <= 512 ? 3 : 2))) void k_promoted4(Layout Ly, Step St, const int *skip_seq) {
    KernelClock kc(St.clk);
    values_pass<D, G, VP_INT4, V8>(Ly, St, skip_seq);
}

template <int D, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_promoted16(Layout Ly, Step St, const int *skip_seq) {
    KernelClock kc(St.clk);
    values_pass<D, G, VP_FP16, false>(Ly, St, skip_seq);
}

// ===========================================================================
// K4a (keys): FP16-key scores of the P blocks from the staging area [Meth-3
// rank-consistency check], one wave per block, lane = token: FP64 fma chain
// over c = 0 .. D-1 with one rounding to FP32 after the scale (the decision
// arithmetic of the rank check), the block's FP16-side max and mass (64-leaf
// tree of exp_c), and the scores for the value pass.  q in FP64 comes from qd
// through uniform scalar loads.  Wave w of workgroup x takes entry 4x + w of
// the step's flat P list; it requests the entry and the list's count
// together (the entry through a buffer resource, so an index past the list
// reads zeros), then both halves of its block (D/2 channels each) before
// any arithmetic: many short waves that ask for all their data at once keep
// the memory system full, and the registers (two halves) allow five waves
// per SIMD.  The results are stored after the last load.
// ===========================================================================
template <int D, int G>
__global__ __launch_bounds__(256) void k_keys16(Layout Ly, Step St, const int *skip_seq,
                                                const double *qd) {
    KernelClock kc(St.clk);
    (void)skip_seq;  // skipped sequences are not in the flat list
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    constexpr uint32_t ALL = (1u << G) - 1u;
    const int e = blockIdx.x * 4 + wave;
    const size_t cap = (size_t)Ly.B * Ly.Hkv * Ly.Nmax;  // entries the list can hold
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(St.klist, (uint32_t)min(cap * 8, (size_t)0xFFFFFFF0u));
    const uint2 ent = rsrc_load8(rl, (uint32_t)e * 8u);
    const int total = __builtin_amdgcn_readfirstlane(*St.kcount);
    if (e >= total) return;  // no barrier follows
    const int ng = (int)__builtin_amdgcn_readfirstlane(ent.x);
    const int b = (int)(__builtin_amdgcn_readfirstlane(ent.y) & 0xFFFFFFu);
    const uint32_t pm = (__builtin_amdgcn_readfirstlane(ent.y) >> 24) & ALL;
    // q as [D][G] FP64, read through the constant address space (qd is not
    // written during this kernel): the loads are scalar
    typedef const __attribute__((address_space(4))) double cdouble;
    const size_t NS64 = (size_t)St.NS * 64;
    constexpr uint32_t BLKB = 64 * D * 2;
    constexpr int HC = D / 16;  // 16-byte chunks per lane in half a block
    using Half = uint4[HC];
    // the block's K: packed slot e (the list is in packed order), or (pair,
    // block) in the staging area
    const size_t slot = St.packed ? (size_t)e : (size_t)ng * Ly.Nmax + (size_t)b;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(St.stage_k + slot * 64 * D, BLKB);
    auto issue = [&](int h, Half &kr) {
#pragma unroll
        for (int ch = 0; ch < HC; ++ch) kr[ch] = rsrc_load16(rs, lane * 16 + h * HC * 1024 + ch * 1024);
    };
    // FP64 chain over the channels of half h for the G heads
    auto chain = [&](const Half &kr, int h, double (&a)[G]) {
        int qoff = 0;
        asm volatile("" : "+s"(qoff));  // opaque zero: keeps the q loads in the loop
        // q in groups of 16 doubles (CS channels x G heads, two scalar loads);
        // the next group is requested before the current one is used
        constexpr int QN = 16, CS = QN / G, NQ = D / 2 / CS;
        cdouble *qb = (cdouble *)qd + __builtin_amdgcn_readfirstlane(ng * D * G + h * (D / 2) * G + qoff);
        double qc[QN], qn[QN];
#pragma unroll
        for (int i = 0; i < QN; ++i) qc[i] = qb[i];
        float kf[8];
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
            if (qi + 1 < NQ)
#pragma unroll
                for (int i = 0; i < QN; ++i) qn[i] = qb[(qi + 1) * QN + i];
            // the next group's loads are issued here, before this group's FMAs
#pragma unroll
            for (int jj = 0; jj < G; ++jj) asm volatile("" : "+v"(a[jj])::"memory");
#pragma unroll
            for (int cc = 0; cc < CS; ++cc) {
                const int c = qi * CS + cc;  // channel within the half
                if (c % 8 == 0) unpack_fp16x8(kr[c / 8], kf);
                const double kc = (double)kf[c % 8];
#pragma unroll
                for (int jj = 0; jj < G; ++jj) a[jj] = fma(qc[cc * G + jj], kc, a[jj]);
            }
            // and the loads after them wait for these FMAs (bounds the
            // scalar registers holding q)
#pragma unroll
            for (int jj = 0; jj < G; ++jj) asm volatile("" : "+v"(a[jj])::"memory");
#pragma unroll
            for (int i = 0; i < QN; ++i) qc[i] = qn[i];
        }
    };
    Half X, Y;
    issue(0, X);
    __builtin_amdgcn_sched_barrier(0);  // requests in this order (the waits count on it)
    issue(1, Y);
    __builtin_amdgcn_sched_barrier(0);
    double a[G];
#pragma unroll
    for (int jj = 0; jj < G; ++jj) a[jj] = 0.0;
    chain(X, 0, a);
    chain(Y, 1, a);
    // scores, block max and mass of the heads of P
    const int n = ng / Ly.Hkv, g = ng - n * Ly.Hkv;
#pragma unroll
    for (int jj = 0; jj < G; ++jj) {
        if (!(pm & (1u << jj))) continue;
        const int h = g * G + jj;
        const float sc = (float)(a[jj] * (double)St.sm);
        St.score16[(size_t)(n * Ly.Hq + h) * NS64 + (size_t)b * 64 + lane] = sc;
        const float mx = wave_max_dpp(sc);
        const float l_ = tree64_f32_dpp(exp_c(sc - mx));
        if (lane == 0) St.st16[((size_t)n * Ly.Hq + h) * Ly.Nmax + b] = make_float2(mx, l_);
    }
}

// ===========================================================================
// Device-initiated paging (a measured alternative to host-issued copies):
// the FP16 K blocks of the P lists and the FP16 V blocks of the VP lists,
// read from tier 2 (pinned host memory mapped into the device's address
// space) over the host link and written to the staging area, only the
// listed blocks (no gap fill) and no per-copy overhead; `kinds`: bit 0 the
// K blocks, bit 1 the V blocks.  One workgroup per
// (slice, kv head, sequence); wave w of slice x takes list entries
// 4x + w, 4x + w + 4*GATHER_X, ...; a wave moves a 64-token block as D/8
// 16-byte loads per lane.  Skipped sequences (rung 4 before paging) are left
// to the host's copies.
// ===========================================================================
constexpr int GATHER_X = 32;

template <int D>
__global__ __launch_bounds__(256) void k_gather(Layout Ly, Step St, const int *skip_seq, const uint16_t *t2k,
                                                const uint16_t *t2v, uint16_t *stk, uint16_t *stv, int kinds) {
    KernelClock kc(St.clk);
    const int x = blockIdx.x, g = blockIdx.y, n = blockIdx.z;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (skip_seq[n]) return;
    const int l = St.layer;
    const int N = __builtin_amdgcn_readfirstlane(Ly.len[l * Ly.B + n]) / 64;
    const size_t ng = (size_t)n * Ly.Hkv + g, nk = (size_t)Ly.B * Ly.Hkv;
    const int W = GATHER_X * 4;
    constexpr int NL = D / 8;  // 16-byte loads per lane per block
#pragma unroll
    for (int kind = 0; kind < 2; ++kind) {
        if (!(kinds & (1 << kind))) continue;
        const int lk = kind == 0 ? WL_KEYS : WL_FP16;
        const int cnt = __builtin_amdgcn_readfirstlane(St.wcnt[lk * nk + ng]);
        const uint32_t *lst = St.wl + (lk * nk + ng) * (size_t)(Ly.Nmax + 1);
        const uint16_t *src = kind == 0 ? t2k : t2v;
        uint16_t *dst = kind == 0 ? stk : stv;
        for (int i = x * 4 + wave; i < cnt; i += W) {
            const int b = __builtin_amdgcn_readfirstlane(lst[i]) & 0xFFFF;
            if (b >= N) continue;  // the unfinished block stays on the device
            const uint4 *sp = reinterpret_cast<const uint4 *>(src + Ly.blk(l, n, g, b) * 64 * D);
            uint4 *dp = reinterpret_cast<uint4 *>(dst + (ng * Ly.Nmax + b) * 64 * D);
            // streaming loads (not kept in the caches: a reset sequence's
            // tier-2 blocks get new contents later)
            v4u32 r[NL];
#pragma unroll
            for (int c = 0; c < NL; ++c) r[c] = __builtin_nontemporal_load(reinterpret_cast<const v4u32 *>(sp) + c * 64 + lane);
#pragma unroll
            for (int c = 0; c < NL; ++c) dp[c * 64 + lane] = make_uint4(r[c].x, r[c].y, r[c].z, r[c].w);
        }
    }
}

// ===========================================================================
// Block lists of the value and FP16-key passes, two kernels of one
// workgroup per (kv head, sequence).
//
// k_wlcount: the sequence's skip flag (rung 4 before paging: a cap of rung
// 1 or 2 exhausted on some head; written by the workgroup of kv head 0), and
// the pair's counts of blocks in P of some head and of blocks with FP16
// values for some head (0 for a skipped sequence).  These counts order the
// packed staging areas of staged paging: the K (V) blocks of the pairs not
// skipped, pair by pair and ascending, then those of the skipped pairs.
//
// k_worklist: the blocks of the sequence in ascending order (an entry is
// the block index | its selection bits << 16) whose selection
// bits put them in P of some head (FP16 keys), in P without FP16 values for
// some head (INT4 values at FP16-key weights), give FP16 values to some head
// (the unfinished block, when there is one, ends this list), or leave some
// head's block outside P and VP (the tail); the prefix of the earlier
// pairs' counts (the pair's first packed V slot, kept for the FP16 value
// pass); and the pair's P blocks in the step's flat FP16-key list at the
// prefix of the earlier pairs' P counts, so that the list is in the packed
// K order and an entry's index is its block's packed K slot.  Skipped
// sequences are left out of the flat list; the passes and the
// device-initiated paging read the skip flags without the host's round trip.
// ===========================================================================
template <int G>
__global__ __launch_bounds__(256) void k_wlcount(Layout Ly, Step St, int *skip_seq) {
    const int g = blockIdx.x, n = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    __shared__ int sh_skip, kc[4], vc[4];
    if (wave == 0) {
        int sk = 0;
        for (int h = lane; h < Ly.Hq; h += 64) sk |= (St.plan[(size_t)n * Ly.Hq + h].flags >> 1) & 1;
        const bool any = __ballot(sk != 0) != 0;
        if (lane == 0) {
            sh_skip = any ? 1 : 0;
            if (g == 0) skip_seq[n] = any ? 1 : 0;
        }
    }
    const int N = __builtin_amdgcn_readfirstlane(Ly.len[St.layer * Ly.B + n]) / 64;
    constexpr uint32_t ALL = (1u << G) - 1u;
    const size_t ng = (size_t)n * Ly.Hkv + g, nk = (size_t)Ly.B * Ly.Hkv;
    const uint32_t *sel = St.sel + ng * Ly.Nmax;
    int ck = 0, cv = 0;
    for (int r0 = 0; r0 < N; r0 += 256) {
        const int b = r0 + tid;
        const uint32_t bits = b < N ? sel[b] : 0u;
        ck += __popcll(__ballot((bits & ALL) != 0));
        cv += __popcll(__ballot(((bits >> 8) & ALL) != 0));
    }
    if (lane == 0) {
        kc[wave] = ck;
        vc[wave] = cv;
    }
    __syncthreads();
    if (tid == 0) {
        St.pcnt[ng] = sh_skip ? 0 : kc[0] + kc[1] + kc[2] + kc[3];
        St.pcnt[nk + ng] = sh_skip ? 0 : vc[0] + vc[1] + vc[2] + vc[3];
    }
}

template <int G>
__global__ __launch_bounds__(256) void k_worklist(Layout Ly, Step St, const int *skip_seq) {
    const int g = blockIdx.x, n = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int len = __builtin_amdgcn_readfirstlane(Ly.len[St.layer * Ly.B + n]);
    const int N = len / 64;
    constexpr uint32_t ALL = (1u << G) - 1u;
    const size_t ng = (size_t)n * Ly.Hkv + g, nk = (size_t)Ly.B * Ly.Hkv;
    const int npair = St.batch * Ly.Hkv;
    const uint32_t *sel = St.sel + ng * Ly.Nmax;
    uint32_t *lst[WL_KINDS];
#pragma unroll
    for (int k = 0; k < WL_KINDS; ++k) lst[k] = St.wl + (k * nk + ng) * (size_t)(Ly.Nmax + 1);
    __shared__ int wc[WL_KINDS][4];
    __shared__ int pk[4], pv[4], tk[4];
    // prefixes of the earlier pairs' counts, and the total of P blocks
    {
        int ak = 0, av = 0, at = 0;
        for (int i = tid; i < npair; i += 256) {
            const int c = St.pcnt[i];
            at += c;
            if (i < (int)ng) {
                ak += c;
                av += St.pcnt[nk + i];
            }
        }
        ak = wave_sum_i32_dpp(ak);
        av = wave_sum_i32_dpp(av);
        at = wave_sum_i32_dpp(at);
        if (lane == 0) {
            pk[wave] = ak;
            pv[wave] = av;
            tk[wave] = at;
        }
        __syncthreads();
    }
    const int kpref = pk[0] + pk[1] + pk[2] + pk[3];
    if (tid == 0) {
        St.vpref[ng] = pv[0] + pv[1] + pv[2] + pv[3];
        if (ng == 0) *St.kcount = tk[0] + tk[1] + tk[2] + tk[3];
    }
    const bool kflat = skip_seq[n] == 0;
    int base[WL_KINDS] = {};
    const uint64_t below = (1ull << lane) - 1ull;
    for (int r0 = 0; r0 < N; r0 += 256) {
        const int b = r0 + tid;
        const uint32_t bits = b < N ? sel[b] : 0u;
        const uint32_t pm = bits & ALL, vm = (bits >> 8) & ALL;
        const bool f[WL_KINDS] = {pm != 0, (pm & ~vm) != 0, vm != 0, b < N && (pm | vm) != ALL};
        uint64_t bal[WL_KINDS];
#pragma unroll
        for (int k = 0; k < WL_KINDS; ++k) {
            bal[k] = __ballot(f[k]);
            if (lane == 0) wc[k][wave] = __popcll(bal[k]);
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < WL_KINDS; ++k) {
            int off = base[k], tot = 0;
            for (int w = 0; w < 4; ++w) {
                off += w < wave ? wc[k][w] : 0;
                tot += wc[k][w];
            }
            const int pos = off + __popcll(bal[k] & below);
            // entry: block | selection bits << 16 (P heads, then VP heads)
            if (f[k]) lst[k][pos] = (uint32_t)b | ((pm | (vm << 8)) << 16);
            if (k == WL_KEYS && kflat && f[k])
                St.klist[kpref + pos] = make_uint2((uint32_t)ng, (uint32_t)b | (pm << 24));
            base[k] += tot;
        }
        __syncthreads();
    }
    if (tid == 0) {
        if (len % 64) lst[WL_FP16][base[WL_FP16]++] = (uint32_t)N;  // the unfinished block, no bits
#pragma unroll
        for (int k = 0; k < WL_KINDS; ++k) St.wcnt[k * nk + ng] = base[k];
    }
}

// ===========================================================================
// K4b: rank-consistency check [Meth-3] + merge of the partials -> output.
// One MERGE_T-thread workgroup per (q head, sequence).  Fixed-point FP16 masses M16 on P relative
// to the largest FP16 block max of P; Kendall discordant pairs against the
// INT8 order; inconsistent iff D > floor(rank_tol * K*(K*-1)/2).
// ===========================================================================
constexpr int RANK_LDS = 2048;
constexpr int RANK_PAIRS = 512;  // up to this K the pairs are counted directly
constexpr int MERGE_T = 1024;

// Number of elements of the descending run r[0..n) greater than x
// (keys are unique).
__device__ __forceinline__ int count_greater(const uint64_t *r, int n, uint64_t x) {
    int lo = 0, hi = n;  // r[0..lo) > x, r[hi..n) < x
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (r[mid] > x) lo = mid + 1; else hi = mid;
    }
    return lo;
}

// Kendall discordant pairs between two orders of the same K <= RANK_LDS items
// given as unique keys (kI[i], k16[i]) whose low 16 bits are 0xFFFF - i:
// sort kI descending (bitonic, in LDS), gather the k16 keys in that order,
// then merge-sort them descending, counting for every element of a right run
// the elements of the left run smaller than it.  Exact integer result,
// independent of the thread count.  Wave w owns elements [128w, 128w + 128):
// sort stages with stride <= 64 and merge passes with runs <= 64 stay inside
// a wave (no workgroup barrier).  Uses and overwrites kI, k16, tmp (RANK_LDS
// entries each).  All threads call it.
__device__ __forceinline__ long long discordant_sorted(uint64_t *kI, uint64_t *k16, uint64_t *tmp, int K) {
    const int tid = threadIdx.x;
    int Kp = 1, lgKp = 0;
    while (Kp < K) {
        Kp <<= 1;
        ++lgKp;
    }
    for (int i = K + tid; i < Kp; i += MERGE_T) kI[i] = 0;  // padding sorts last (real keys are > 0 after +1)
    for (int i = tid; i < K; i += MERGE_T) kI[i] += 1;
    __syncthreads();
    // one compare-exchange per thread and stage (Kp / 2 <= MERGE_T)
    auto stage = [&](int lgs, int size) {
        const int t = tid;
        if (t < (Kp >> 1)) {
            const int stride = 1 << lgs;
            const int i = ((t >> lgs) << (lgs + 1)) | (t & (stride - 1));
            const int jx = i + stride;
            const bool desc = (i & size) == 0;
            const uint64_t a = kI[i], b = kI[jx];
            if ((a < b) == desc) {
                kI[i] = b;
                kI[jx] = a;
            }
        }
    };
    for (int lsz = 1; lsz <= lgKp; ++lsz) {
        const int size = 1 << lsz;
        int lgs = lsz - 1;
        for (; lgs >= 7; --lgs) {  // stride >= 128: across waves
            stage(lgs, size);
            __syncthreads();
        }
        for (; lgs >= 0; --lgs) {  // inside the wave's 128 elements
            stage(lgs, size);
            wave_sync();
        }
        __syncthreads();
    }
    // the FP16-side keys in INT8 order
    for (int e = tid; e < K; e += MERGE_T) tmp[e] = k16[0xFFFF - (int)((kI[e] - 1) & 0xFFFF)];
    __syncthreads();
    long long D = 0;
    uint64_t *src = tmp, *dst = k16;
    const int wv = tid >> 6, lane = tid & 63;
    for (int lw = 0; (1 << lw) < K; ++lw) {
        const int w = 1 << lw;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int e = 128 * wv + 64 * half + lane;
            if (e < K) {
                const int s0 = (e >> (lw + 1)) << (lw + 1);
                const int lw_ = min(w, K - s0);
                const int rw = max(0, min(w, K - s0 - w));
                const uint64_t x = src[e];
                int pos;
                if (e < s0 + lw_) {
                    pos = (e - s0) + count_greater(src + s0 + lw_, rw, x);
                } else {
                    const int gg = count_greater(src + s0, lw_, x);
                    D += lw_ - gg;  // left elements smaller than x: discordant
                    pos = (e - s0 - lw_) + gg;
                }
                dst[s0 + pos] = x;
            }
        }
        if (w >= 64) __syncthreads(); else wave_sync();
        uint64_t *t_ = src;
        src = dst;
        dst = t_;
    }
    return D;
}

template <int D, int G>
// part: bit 0 the rank check (needs the FP16-key pass only, so it can run
// while the FP16 values are still being paged), bit 1 the merge.
__global__ __launch_bounds__(MERGE_T) void k_merge(Layout Ly, Step St, Th th, const int *skip_seq,
                                                   uint32_t *plist_g, uint64_t *keys_g, int part) {
    KernelClock kc(St.clk);
    constexpr int CPL = D / 64;
    const int h = blockIdx.x, n = blockIdx.y, tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int g = h / G, j = h % G, l = St.layer;
    // the uniform words through the constant address space, requested
    // together (scalar loads; none is written during this kernel): the
    // skip flag, the length and the promoted passes' list lengths
    typedef const __attribute__((address_space(4))) int cint;
    const size_t ngp = (size_t)n * Ly.Hkv + g, nkp = (size_t)Ly.B * Ly.Hkv;
    const int skip = ((cint *)skip_seq)[n];
    const int len = ((cint *)Ly.len)[l * Ly.B + n];
    const int cnt4 = ((cint *)St.wcnt)[WL_INT4 * nkp + ngp], cnt16 = ((cint *)St.wcnt)[WL_FP16 * nkp + ngp];
    if (skip) return;
    const int N = len / 64, np = len % 64;
    const size_t hs = (size_t)n * Ly.Hq + h;
    const uint32_t *sel = St.sel + ((size_t)n * Ly.Hkv + g) * Ly.Nmax;
    __shared__ uint32_t lds_list[RANK_LDS];
    __shared__ uint64_t lds_kI[RANK_LDS], lds_k16[RANK_LDS], lds_tmp[RANK_LDS];
    __shared__ long long red_ll[MERGE_T / 64];
    __shared__ float red_f[MERGE_T / 64];
    __shared__ float w_m[MERGE_T / 64], w_l[MERGE_T / 64], w_acc[MERGE_T / 64][D];
    if (part & 1) {

    // compact list of P blocks (ascending index): one block per thread and
    // round, per-wave counts combined through LDS
    const uint32_t bitP = 1u << j;
    uint32_t *plist = plist_g + hs * Ly.Nmax;
    __shared__ int wcnt[MERGE_T / 64];
    int K = 0;
    for (int r0 = 0; r0 < N; r0 += MERGE_T) {
        const int b = r0 + tid;
        const bool inP = b < N && (sel[b] & bitP);
        const uint64_t bal = __ballot(inP);
        if (lane == 0) wcnt[wave] = __popcll(bal);
        __syncthreads();
        int off = K, tot = 0;
        for (int w = 0; w < MERGE_T / 64; ++w) {
            off += w < wave ? wcnt[w] : 0;
            tot += wcnt[w];
        }
        const int pos = off + __popcll(bal & ((1ull << lane) - 1ull));
        if (inP) {
            plist[pos] = (uint32_t)b;
            if (pos < RANK_LDS) lds_list[pos] = (uint32_t)b;
        }
        K += tot;
        __syncthreads();
    }
    const bool use_lds = K <= RANK_LDS;
    const float2 *st16 = St.st16 + hs * Ly.Nmax;
    const uint64_t *M = St.mfx + hs * St.NS;
    // block b's fixed-point FP16 mass M16 (relative to the largest FP16 block
    // max mr over P) and the two keys (mass desc, index asc)
    // ties broken by `tie`, ascending: the block index, or its position in
    // the (ascending) P list, which orders the same way
    auto keys = [&](uint32_t b, uint32_t tie, float mr, uint64_t &ki, uint64_t &k16) {
        const float2 s = st16[b];
        const float m16 = s.y * exp_c(s.x - mr);
        const uint64_t M16 = (uint64_t)((double)m16 * 4294967296.0);
        St.m16[hs * Ly.Nmax + b] = M16;
        ki = (M[b] << 16) | (uint64_t)(0xFFFF - tie);
        k16 = (M16 << 16) | (uint64_t)(0xFFFF - tie);
    };
    auto block_max = [&](float v) {
        v = wave_max_f32(v);
        if (lane == 0) red_f[wave] = v;
        __syncthreads();
        float r = red_f[0];
        for (int w = 1; w < MERGE_T / 64; ++w) r = fmaxf(r, red_f[w]);
        return r;
    };
    // Kendall discordant pairs; the LDS path names the shared arrays
    // directly (LDS instructions, not generic addresses)
    long long D_ = 0;
    float mrP = -INFINITY;  // largest FP16-key block max over P
    if (use_lds) {
        float mr = -INFINITY;
        for (int i = tid; i < K; i += MERGE_T) mr = fmaxf(mr, st16[lds_list[i]].x);
        mr = block_max(mr);
        mrP = mr;
        for (int i = tid; i < K; i += MERGE_T) keys(lds_list[i], (uint32_t)i, mr, lds_kI[i], lds_k16[i]);
        __syncthreads();
        if (K <= RANK_PAIRS) {
            // all pairs (i, q > i) from LDS: RANK_SUB threads per row, rows
            // i and K-1-i on the same thread group (equal work)
            constexpr int RANK_SUB = 8;
            const int sub = tid % RANK_SUB;
            int d = 0;
            for (int i = tid / RANK_SUB; i < (K + 1) / 2; i += MERGE_T / RANK_SUB) {
                const int rows[2] = {i, K - 1 - i};
                for (int r = 0; r < (rows[0] == rows[1] ? 1 : 2); ++r) {
                    const int a_ = rows[r];
                    const uint64_t a = lds_kI[a_], c = lds_k16[a_];
#pragma unroll 4
                    for (int q = a_ + 1 + sub; q < K; q += RANK_SUB) d += ((a > lds_kI[q]) != (c > lds_k16[q]));
                }
            }
            D_ = d;
        } else {
            D_ = discordant_sorted(lds_kI, lds_k16, lds_tmp, K);
        }
    } else {
        uint64_t *kI = keys_g + hs * 2 * Ly.Nmax;
        uint64_t *k16 = kI + Ly.Nmax;
        float mr = -INFINITY;
        for (int i = tid; i < K; i += MERGE_T) mr = fmaxf(mr, st16[plist[i]].x);
        mr = block_max(mr);
        mrP = mr;
        for (int i = tid; i < K; i += MERGE_T) keys(plist[i], plist[i], mr, kI[i], k16[i]);
        __syncthreads();
        // rows i and K-1-i go to the same thread (equal work per thread)
        for (int i = tid; i < (K + 1) / 2; i += MERGE_T) {
            const int rows[2] = {i, K - 1 - i};
            for (int r = 0; r < (rows[0] == rows[1] ? 1 : 2); ++r) {
                const int a_ = rows[r];
                const uint64_t a = kI[a_], c = k16[a_];
                for (int q = a_ + 1; q < K; ++q) D_ += ((a > kI[q]) != (c > k16[q]));
            }
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) D_ += __shfl_xor(D_, o, 64);
    if (lane == 0) red_ll[wave] = D_;
    __syncthreads();
    if (tid == 0) {
        long long Dt = 0;
        for (int w = 0; w < MERGE_T / 64; ++w) Dt += red_ll[w];
        const double pairs = (double)K * (double)(K - 1) / 2.0;
        const double lim = floor((double)th.rank_tol * pairs);
        St.plan[hs].rank_ok = !((double)Dt > lim);
        St.plan[hs].ndisc = (int)Dt;
        // the softmax reference of the promoted value passes
        St.plan[hs].mref16 = fmaxf(St.plan[hs].mref, mrP);
    }
    }  // rank check
    if (!(part & 2)) return;

    // merge: tail partials then promoted partials; each wave merges a
    // contiguous share in one pass (eight partials in flight, the running
    // maximum raised batch by batch and the sums rescaled to it), the
    // shares are combined in wave order
    // the splits each pass wrote for this pair: the tail's by context, the
    // promoted passes' by the length of their lists
    const int nsp_t = (N + St.bps - 1) / St.bps;
    const int nsp_4 = (cnt4 + St.t4 - 1) / St.t4;
    const int nsp_f = (cnt16 + St.t16 - 1) / St.t16;
    const float *pt = St.part_tail + hs * St.nsplit_cap * (D + 2);
    const float *p4 = St.part_blk + hs * St.nsplit_cap * (D + 2);
    const float *pf = St.part_blk16 + hs * St.nsplit_cap * (D + 2);
    auto part_ptr = [&](int i) {
        return i < nsp_t ? pt + (size_t)i * (D + 2)
             : i < nsp_t + nsp_4 ? p4 + (size_t)(i - nsp_t) * (D + 2) : pf + (size_t)(i - nsp_t - nsp_4) * (D + 2);
    };
    const int ntot = nsp_t + nsp_4 + nsp_f;
    const int per = (ntot + MERGE_T / 64 - 1) / (MERGE_T / 64);
    const int i_lo = wave * per, i_hi = min(ntot, i_lo + per);
    constexpr int BATCH = 8;
    float mx = -INFINITY, den = 0.0f, num[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) num[k] = 0.0f;
    for (int i0 = i_lo; i0 < i_hi; i0 += BATCH) {
        float m[BATCH], l_[BATCH], a[BATCH][CPL];
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            m[i] = -INFINITY;
            if (i0 + i < i_hi) {
                const float *p = part_ptr(i0 + i);
                m[i] = p[0];
                l_[i] = p[1];
#pragma unroll
                for (int k = 0; k < CPL; ++k) a[i][k] = p[2 + lane + 64 * k];
            }
        }
        float bm = mx;
#pragma unroll
        for (int i = 0; i < BATCH; ++i) bm = fmaxf(bm, m[i]);
        if (bm == -INFINITY) continue;  // nothing yet (empty partials)
        if (bm != mx) {
            // a larger maximum: the sums so far to its scale (0 before any)
            const float sc = __expf(mx - bm);
            den *= sc;
#pragma unroll
            for (int k = 0; k < CPL; ++k) num[k] *= sc;
            mx = bm;
        }
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            if (m[i] != -INFINITY) {
                const float e = __expf(m[i] - mx);
                den = fmaf(e, l_[i], den);
#pragma unroll
                for (int k = 0; k < CPL; ++k) num[k] = fmaf(e, a[i][k], num[k]);
            }
        }
    }
    if (lane == 0) {
        w_m[wave] = mx;
        w_l[wave] = den;
    }
#pragma unroll
    for (int k = 0; k < CPL; ++k) w_acc[wave][lane + 64 * k] = num[k];
    __syncthreads();
    if (wave == 0) {
        float Mx = -INFINITY;
        for (int w = 0; w < MERGE_T / 64; ++w) Mx = fmaxf(Mx, w_m[w]);
        float dd = 0.0f, nn[CPL];
#pragma unroll
        for (int k = 0; k < CPL; ++k) nn[k] = 0.0f;
        for (int w = 0; w < MERGE_T / 64; ++w) {
            if (w_m[w] == -INFINITY) continue;
            const float e = __expf(w_m[w] - Mx);
            dd = fmaf(e, w_l[w], dd);
#pragma unroll
            for (int k = 0; k < CPL; ++k) nn[k] = fmaf(e, w_acc[w][lane + 64 * k], nn[k]);
        }
#pragma unroll
        for (int k = 0; k < CPL; ++k) St.out[hs * D + lane + 64 * k] = nn[k] / dd;
    }
}

// ===========================================================================
// K5: exact attention on FP16 blocks (rungs 3 / 4 [Meth-1 fallback, Meth-3]
// and the dense comparator).  Blocks of (seq, kv head) are at
// kbase + ((n * Hkv + g) * nstride + b) * 64 * D (K chunk-interleaved, V
// channel-major); `nfull[n]` full blocks, then an optional unfinished block.
// Scores in FP32 on the vector units (lane = token), moved to the A layout
// through LDS; values on the matrix cores.
// ===========================================================================
template <int D, int G>
__global__ __launch_bounds__(256) void k_dense(DenseSrc S) {
    using VA = VAcc<D, G, false>;
    const int sp = blockIdx.x, g = blockIdx.y, n = blockIdx.z;
    // wave index as a uniform value: the block loops below branch uniformly
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const uint32_t mask = S.mask ? S.mask[n * S.Hkv + g] : ((1u << G) - 1u);
    if (!mask) return;
    const int len = S.len ? __builtin_amdgcn_readfirstlane(S.len[n]) : S.len_all;
    const int N = len / 64, np = len % 64;
    const int nslot = N + (np ? 1 : 0);
    const int b0 = sp * S.bps, b1 = min(nslot, b0 + S.bps);
    __shared__ float qs[G][D];
    __shared__ __attribute__((aligned(16))) float st[4][G][64];  // scores, lane = token -> A layout
    __shared__ float ksg[VA::NG];
    for (int i = threadIdx.x; i < G * D; i += 256)
        qs[i / D][i % D] = h2f(S.q[((size_t)n * S.Hq + g * G + i / D) * D + (i % D)]);
    if (threadIdx.x < VA::NG) ksg[threadIdx.x] = K16;  // FP16 values only
    __syncthreads();
    VA va;
    va.init();
    for (int b = b0 + wave; b < b1; b += 4) {
        const bool part = b == N;
        const uint16_t *kb, *vb;
        if (part) {
            kb = S.kp + ((size_t)n * S.Hkv + g) * 64 * D;
            vb = S.vp + ((size_t)n * S.Hkv + g) * 64 * D;
        } else {
            const size_t ix = ((size_t)n * S.Hkv + g) * S.nstride + b;
            kb = S.k + (S.kmap ? (size_t)S.kmap[ix] : ix) * 64 * D;
            vb = S.v + (S.vmap ? (size_t)S.vmap[ix] : ix) * 64 * D;
        }
        uint4 kv[D / 8];
#pragma unroll
        for (int ch = 0; ch < D / 8; ++ch) kv[ch] = *reinterpret_cast<const uint4 *>(kb + ch * 512 + lane * 8);
        uint4 vv[VA::NT][2];
        // opaque zero offset: keeps the q reads inside the loop
        int qoff = 0;
        asm volatile("" : "+s"(qoff));
        const float *qsp = &qs[0][0] + qoff;
        float a[G];
#pragma unroll
        for (int jj = 0; jj < G; ++jj) a[jj] = 0.0f;
#pragma unroll
        for (int ch = 0; ch < D / 8; ++ch) {
            if (ch == D / 16) load_fp16v<D>(vb, lane, vv);  // values halfway through the keys
            float kf[8];
            unpack_fp16x8(kv[ch], kf);
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int jj = 0; jj < G; ++jj) a[jj] = fmaf(qsp[jj * D + ch * 8 + i], kf[i], a[jj]);
#pragma unroll
            for (int jj = 0; jj < G; ++jj) asm volatile("" : "+v"(a[jj])::"memory");
        }
#pragma unroll
        for (int jj = 0; jj < G; ++jj) st[wave][jj][lane] = a[jj] * S.sm;
        wave_sync();
        float sv[VA::RT][16];
#pragma unroll
        for (int rt = 0; rt < VA::RT; ++rt) {
            const float4 *src = reinterpret_cast<const float4 *>(&st[wave][VA::ahead(rt, lane)][16 * (lane >> 4)]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 x = src[i];
                sv[rt][4 * i] = x.x;
                sv[rt][4 * i + 1] = x.y;
                sv[rt][4 * i + 2] = x.z;
                sv[rt][4 * i + 3] = x.w;
            }
        }
        wave_sync();
        mask_scores<D, G, false>(mask, part ? np : 64, lane, sv);
        va.softmax(sv, lane);
        va.fp16_block(mask, sv, vv, lane);
    }
    write_partials<D, G, false>(va, ksg, S.part, (size_t)n * S.Hq + g * G, S.nsplit_cap, sp, mask, false);
}

template <int D, int G>
__global__ __launch_bounds__(64) void k_merge_dense(DenseSrc S) {
    constexpr int CPL = D / 64;
    const int h = blockIdx.x, n = blockIdx.y, lane = threadIdx.x;
    const int g = h / G, j = h % G;
    const uint32_t mask = S.mask ? S.mask[n * S.Hkv + g] : ((1u << G) - 1u);
    if (!(mask & (1u << j))) return;
    const int len = S.len ? __builtin_amdgcn_readfirstlane(S.len[n]) : S.len_all;
    const int nslot = len / 64 + ((len % 64) ? 1 : 0);
    const int nsp = (nslot + S.bps - 1) / S.bps;
    const float *pt = S.part + (size_t)(n * S.Hq + h) * S.nsplit_cap * (D + 2);
    float mx = -INFINITY;
    for (int s = 0; s < nsp; ++s) mx = fmaxf(mx, pt[(size_t)s * (D + 2)]);
    float den = 0.0f, num[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) num[k] = 0.0f;
    for (int s = 0; s < nsp; ++s) {
        const float *p = pt + (size_t)s * (D + 2);
        if (p[0] == -INFINITY) continue;
        const float e = __expf(p[0] - mx);
        den = fmaf(e, p[1], den);
#pragma unroll
        for (int k = 0; k < CPL; ++k) num[k] = fmaf(e, p[2 + lane + 64 * k], num[k]);
    }
#pragma unroll
    for (int k = 0; k < CPL; ++k) S.out[((size_t)n * S.Hq + h) * D + lane + 64 * k] = num[k] / den;
}

// ---- launchers -------------------------------------------------------------

hipError_t launch_score(const Layout &Ly, const Step &St, hipStream_t s) {
    return dispatch(Ly.d, Ly.G, [&](auto D, auto G) {
        hipLaunchKernelGGL((k_score<decltype(D)::value, decltype(G)::value>),
                           dim3((St.nb + 1 + SCORE_W * SCORE_BPW_ - 1) / (SCORE_W * SCORE_BPW_), Ly.Hkv, St.batch),
                           dim3(64 * SCORE_W), 0, s,
                           Ly, St);
        return hipGetLastError();
    });
}

hipError_t launch_select(const Layout &Ly, const Step &St, const Th &th, hipStream_t s) {
    return dispatch(Ly.d, Ly.G, [&](auto D, auto G) {
        hipLaunchKernelGGL((k_select<decltype(D)::value, decltype(G)::value>),
                           dim3(Ly.Hq, St.batch), dim3(SEL_T), 0, s, Ly, St, th);
        return hipGetLastError();
    });
}

hipError_t launch_tail(const Layout &Ly, const Step &St, hipStream_t s) {
    return dispatch(Ly.d, Ly.G, [&](auto D, auto G) {
        if (Ly.vb == 8)
            hipLaunchKernelGGL((k_tail<decltype(D)::value, decltype(G)::value, true>),
                               dim3(St.nsplit, Ly.Hkv, St.batch), dim3(256), 0, s, Ly, St);
        else
            hipLaunchKernelGGL((k_tail<decltype(D)::value, decltype(G)::value, false>),
                               dim3(St.nsplit, Ly.Hkv, St.batch), dim3(256), 0, s, Ly, St);
        return hipGetLastError();
    });
}

hipError_t launch_gather(const Layout &Ly, const Step &St, const int *skip_seq, const uint16_t *t2k,
                         const uint16_t *t2v, uint16_t *stk, uint16_t *stv, int kinds, hipStream_t s) {
    return dispatch(Ly.d, Ly.G, [&](auto D, auto G) {
        (void)G;
        hipLaunchKernelGGL((k_gather<decltype(D)::value>), dim3(GATHER_X, Ly.Hkv, St.batch), dim3(256), 0, s,
                           Ly, St, skip_seq, t2k, t2v, stk, stv, kinds);
        return hipGetLastError();
    });
}
hipError_t launch_worklist(const Layout &Ly, const Step &St, int *skip_seq, hipStream_t s) {
    return dispatch(Ly.d, Ly.G, [&](auto D, auto G) {
        (void)D;
        hipLaunchKernelGGL((k_wlcount<decltype(G)::value>), dim3(Ly.Hkv, St.batch), dim3(256), 0, s, Ly, St,
                           skip_seq);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((k_worklist<decltype(G)::value>), dim3(Ly.Hkv, St.batch), dim3(256), 0, s, Ly, St,
                           (const int *)skip_seq);
        return hipGetLastError();
    });
}
hipError_t launch_keys16(const Layout &Ly, const Step &St, const int *skip_seq, hipStream_t s) {
    return dispatch(Ly.d, Ly.G, [&](auto D, auto G) {
        // one wave per entry of the flat list, which holds at most nb
        // blocks per sequence and kv head
        const long long bound = (long long)St.nb * Ly.Hkv * St.batch;
        if (bound == 0) return hipSuccess;
        const int nsp = (int)((bound + 3) / 4);
        hipLaunchKernelGGL((k_keys16<decltype(D)::value, decltype(G)::value>), dim3(nsp), dim3(256), 0, s, Ly, St,
                           skip_seq, (const double *)St.qd);
        return hipGetLastError();
    });
}

hipError_t launch_promoted4(const Layout &Ly, const Step &St, const int *skip_seq, hipStream_t s) {
    return dispatch(Ly.d, Ly.G, [&](auto D, auto G) {
        const int nsp4 = St.nsp4;
        if (nsp4 > 0 && Ly.vb == 8)
            hipLaunchKernelGGL((k_promoted4<decltype(D)::value, decltype(G)::value, true>),
                               dim3(nsp4, Ly.Hkv, St.batch), dim3(256), 0, s, Ly, St, skip_seq);
        else if (nsp4 > 0)
            hipLaunchKernelGGL((k_promoted4<decltype(D)::value, decltype(G)::value, false>),
                               dim3(nsp4, Ly.Hkv, St.batch), dim3(256), 0, s, Ly, St, skip_seq);
        return hipGetLastError();
    });
}
hipError_t launch_promoted16(const Layout &Ly, const Step &St, const int *skip_seq, hipStream_t s) {
    return dispatch(Ly.d, Ly.G, [&](auto D, auto G) {
        const int nsp = St.nsp16;
        if (nsp <= 0) return hipSuccess;
        hipLaunchKernelGGL((k_promoted16<decltype(D)::value, decltype(G)::value>),
                           dim3(nsp, Ly.Hkv, St.batch), dim3(256), 0, s, Ly, St, skip_seq);
        return hipGetLastError();
    });
}

hipError_t launch_merge_impl(const Layout &Ly, const Step &St, const Th &th, const int *skip_seq,
                             uint32_t *plist, uint64_t *keys, int part, hipStream_t s) {
    if (part < 1 || part > 3) return hipErrorInvalidValue;
    return dispatch(Ly.d, Ly.G, [&](auto D, auto G) {
        hipLaunchKernelGGL((k_merge<decltype(D)::value, decltype(G)::value>),
                           dim3(Ly.Hq, St.batch), dim3(MERGE_T), 0, s, Ly, St, th, skip_seq, plist, keys, part);
        return hipGetLastError();
    });
}

hipError_t launch_dense_src(int d, int G, const DenseSrc &S, int nsplit, int batch, hipStream_t s) {
    return dispatch(d, G, [&](auto D, auto GG) {
        hipLaunchKernelGGL((k_dense<decltype(D)::value, decltype(GG)::value>),
                           dim3(nsplit, S.Hkv, batch), dim3(256), 0, s, S);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((k_merge_dense<decltype(D)::value, decltype(GG)::value>),
                           dim3(S.Hq, batch), dim3(64), 0, s, S);
        return hipGetLastError();
    });
}

}  // namespace ckv
