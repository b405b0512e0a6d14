// ckv_internal.hpp -- layouts shared by the kernels and the host runtime.
//
// HBM layout of tier 1 (device), per (layer l, sequence n, kv head g,
// block b), blocks of 64 tokens, d = head_dim:
//   kq    u8  [d/16][64][16]   INT8 key codes stored as code ^ 0x80 (= code -
//                              128 as a signed byte), chunk-interleaved: one 16-byte
//                              load per lane covers 16 channels of one token
//                              and a wave's load covers 1 KiB contiguous
//   kmeta u32 [d]              binary16 scale | binary16 offset << 16
//   vq    u8  [d/32][64][16]   INT4 value codes by channel pair p = c / 32
//                              and lane l = 16 (t / 16) + c % 16: 8 bytes of
//                              channel 32 p + c % 16, then 8 of channel
//                              32 p + 16 + c % 16, for tokens 16 (t / 16) ..
//                              + 15 (byte j: tokens 2 j, 2 j + 1, low nibble
//                              = even); one 16-byte load per lane and pair,
//                              1 KiB per wave (vb = 8: u8 [d][64], byte
//                              c * 64 + t)
//   vmeta u32 [d/32][64]       per (group, token): binary16 scale |
//                              binary16 offset << 16
//   eta   f32                  value-error annotation of the block
// Unfinished block (device, FP16): kpart [d/8][64][8], vpart [d][64].
// Tier 2 (pinned host) and the device staging area hold FP16 blocks in the
// same per-block layout: K [d/8][64][8] (one 16-byte load = 8 channels of a
// token), V [d][64] (channel-major: a 16-byte load = 8 tokens of a channel,
// the k-operand order of the value contraction).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ckv {

struct Layout {
    int L, B, Hq, Hkv, d, G, Nmax;  // Nmax: full-block capacity per sequence
    int vb;                         // value code width, 4 or 8
    uint8_t *kq;
    uint32_t *kmeta;
    uint8_t *vq;
    uint32_t *vmeta;
    float *eta;
    uint32_t *vmin, *vmax;  // [L][B][Hkv][d] order-preserving encodings of FP32
    float *vscale;          // [L][B][Hkv][d/32] power-of-two weight scale per value group
    uint16_t *kpart, *vpart;
    int *len;               // [L][B] tokens per sequence (device mirror)

    __host__ __device__ size_t blk(int l, int n, int g, int b) const {
        return (((size_t)l * B + n) * Hkv + g) * Nmax + b;
    }
    __host__ __device__ size_t seqg(int l, int n, int g) const {
        return ((size_t)l * B + n) * Hkv + g;
    }
};

// Order-preserving u32 encoding of an FP32 value (for atomic min / max).
__host__ __device__ inline uint32_t f2ord(float f) {
    uint32_t u;
    __builtin_memcpy(&u, &f, 4);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__host__ __device__ inline float ord2f(uint32_t u) {
    uint32_t v = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
    float f;
    __builtin_memcpy(&f, &v, 4);
    return f;
}

// Plan of one (sequence, q head), written by the selection kernel and
// completed by the rank-check kernel.
struct HeadPlan {
    double mu, tv, ekey, eval, tau;
    float mref;    // largest INT8 block estimate M^ (the selection's reference)
    float mref16;  // max(M^, largest FP16-key block max over P): rank check
    int kstar, nvp, flags;  // flags: bit0 widened, bit1 a cap was exhausted
    int rank_ok, ndisc;
    uint64_t S;
};
static_assert(sizeof(HeadPlan) % 4 == 0, "plans reach the host as 4-byte words");

// Scratch of one decode step; strides use the cache capacity so that any
// batch size fits.  NS = Nmax + 1 slots per head (the extra one is the
// unfinished block).
struct Step {
    int layer, batch, nb;   // nb: max full blocks over the batch
    int NS;                 // slot stride
    int nsplit, bps;        // tail splits per (seq, kv head), blocks per split
    int ncu;                // compute units of the device
    float sm;
    const uint16_t *q;      // [batch][Hq][d]
    float *score;           // [B][Hq][NS*64]  INT8 scores (unfinished block: FP16)
    float *score16;         // [B][Hq][NS*64]  FP16-key scores on P
    float4 *bstat;          // [B][Hq][NS]  max, l, Delta, rho
    uint64_t *mfx;          // [B][Hq][NS]
    uint64_t *cval;         // [B][Hq][NS]  E_val contribution per block
    uint32_t *sel;          // [B][Hkv][Nmax]
    HeadPlan *plan;         // [B][Hq]
    float2 *st16;           // [B][Hq][Nmax] FP16-key block max, l on P
    uint64_t *m16;          // [B][Hq][Nmax]
    float *part_tail;       // [B][Hq][nsplit_cap][d+2]  m, l, acc
    float *part_blk;        // [B][Hq][NS][d+2]  promoted blocks, INT4 values
    float *part_blk16;      // [B][Hq][NS][d+2]  promoted blocks, FP16 values
    int nsplit_cap;
    const uint16_t *stage_k, *stage_v;  // [B][Hkv][Nmax][64*d]
    double *qd;             // [B][Hkv][d][G] q in FP64 (written by the scoring pass)
    // Block lists per (seq, kv head), ascending block index, WL_KINDS kinds
    // at a stride of B*Hkv*(Nmax+1) entries: WL_KEYS blocks in P of some head
    // (FP16 keys), WL_INT4 blocks in P of some head without FP16 values,
    // WL_FP16 blocks with FP16 values for some head, then the unfinished
    // block (index N) when there is one, WL_TAIL blocks outside P and VP for
    // some head.  wcnt[kind][B][Hkv] = lengths.
    uint32_t *wl;
    int *wcnt;
    // The FP16-key pass's entries of the whole step as one list: (pair
    // n * Hkv + g, block | P heads << 24), pair by pair, a pair's entries
    // ascending (the packed K order), kcount entries; skipped sequences are
    // left out.  pcnt: [2][B * Hkv] the pairs' P and FP16-value block counts
    // (0 when skipped); vpref: [B * Hkv] a pair's first packed V slot.
    uint2 *klist;
    int *kcount;
    int *pcnt, *vpref;
    // 1: the step's FP16 blocks are in the packed staging areas (staged
    // paging of a layer without the persistent FP16 cache): a P block's K
    // is at packed slot = its index in klist, a VP block's V at vpref of
    // its pair + its index in the pair's FP16-value list.  0: the staging
    // areas are indexed by (pair, block).
    int packed;
    // the promoted passes' entries per split (t4: INT4 values, t16: FP16
    // values) and grid widths (the largest split count over the pairs not
    // skipped), host-computed from the selection
    int t4, t16, nsp4, nsp16;
    // the FP16 value pass serves the pairs n * Hkv + g in [p16_lo, p16_hi)
    // (packed staging runs it in two launches: the pairs whose FP16 values
    // have landed while the last chunk is still being copied, then the rest)
    int p16_lo, p16_hi;
    float *out;             // [batch][Hq][d]
    // profiling: when not null, the kernel launched with this step stamps
    // its execution span here (KernelClock: CLK_SLOTS start slots, then
    // CLK_SLOTS end slots, in ticks of the device's constant-rate clock)
    unsigned long long *clk;
};
enum { WL_KEYS = 0, WL_INT4 = 1, WL_FP16 = 2, WL_TAIL = 3, WL_KINDS = 4 };

// Source of an exact dense attention: FP16 blocks of (seq n, kv head g) at
// k + ((n * Hkv + g) * nstride + b) * 64 * D (K chunk-interleaved, V
// channel-major), len[n] tokens (len_all for every sequence when len is
// null), the unfinished block (if any) at kp / vp + (n * Hkv + g) * 64 * D.
struct DenseSrc {
    const uint16_t *k, *v;
    const uint16_t *kp, *vp;
    const int *len;
    int len_all;
    size_t nstride;
    // packed staging: block (pair, b) at slot kmap / vmap[pair * nstride + b]
    // of k / v (null: at pair * nstride + b)
    const uint32_t *kmap, *vmap;
    const uint32_t *mask;       // [B][Hkv] q heads of the group to compute (null: all)
    const uint16_t *q;
    float sm;
    float *part;                // [B][Hq][nsplit_cap][D+2]
    int nsplit_cap, bps, Hq, Hkv;
    float *out;
};

// Decision thresholds as the kernels see them.
struct Th {
    float tau, k_tol, v_tol, rank_tol, f_layer;
    int n_widen, vcap;  // vcap <= 0: no cap
};

// Blocks per split of the value passes and the dense pass (ckv_api.cpp).
int split_blocks(int nb, int Hkv, int batch);
// The calling thread's last-error message (ckv_api.cpp); returns st.
int set_error(int st, const char *msg);

// Promoted value passes: a (sequence, kv head) pair with c entries in the
// pass's list takes ceil(c / t) splits, so a pair's split count follows its
// list, not its context (the partial buffers hold one split per block).
// The host picks t per step so that a pass has about VP_WG4 (INT4 values)
// or VP_WG16 (FP16 values) workgroups over the whole batch (measured best on
// the 32K x 4 and 128K x 1 layers), t in [VP_TMIN, VP_TMAX].
constexpr int VP_WG4 = 352, VP_WG16 = 384, VP_TMIN = 4, VP_TMAX = 64;

// Spread slots of the kernel clock: workgroup w stamps slot w % CLK_SLOTS;
// a slot is one word at the start of its own 128-byte line (CLK_PAD words),
// since atomics on one line are serialized where they are performed.
constexpr int CLK_SLOTS = 64;
constexpr int CLK_PAD = 16;
constexpr int CLK_WORDS = 2 * CLK_SLOTS * CLK_PAD;  // per timed kernel: starts, then ends

// ---- launchers (defined in the .hip files) ---------------------------------
// header bytes of a staged-paging chunk: up to 512 block addresses
constexpr int PAGE_HDR = 4096;
hipError_t launch_page_scatter(const uint8_t *chunk, int nblk, int blk_bytes, hipStream_t s);
// Copy two device buffers (sizes multiples of 4 bytes) into pinned host
// memory mapped into the device's address space (device addresses ha, hb).
hipError_t launch_to_host(const void *a, void *ha, size_t abytes, const void *b, void *hb, size_t bbytes,
                          hipStream_t s);
hipError_t launch_append_token(const Layout &Ly, int l, int batch, const uint16_t *kin, const uint16_t *vin,
                               hipStream_t s);
hipError_t launch_pack(const Layout &Ly, int l, int n, const uint16_t *kin, const uint16_t *vin,
                       int len0, int ntok, int b0, int nblk, uint16_t *pk, uint16_t *pv,
                       hipStream_t s);
hipError_t launch_quant(const Layout &Ly, int l, int n, int b0, int nfull, int nblk,
                        const uint16_t *pk, const uint16_t *pv, hipStream_t s);
hipError_t launch_set_partial(const Layout &Ly, int l, int n, int slot, int nblk,
                              const uint16_t *pk, const uint16_t *pv, hipStream_t s);
hipError_t launch_vrange(const Layout &Ly, int l, int n, const uint16_t *vin, int ntok,
                         int reset, hipStream_t s);

hipError_t launch_score(const Layout &Ly, const Step &St, hipStream_t s);
hipError_t launch_select(const Layout &Ly, const Step &St, const Th &th, hipStream_t s);
hipError_t launch_tail(const Layout &Ly, const Step &St, hipStream_t s);
hipError_t launch_worklist(const Layout &Ly, const Step &St, int *skip_seq, hipStream_t s);
hipError_t launch_gather(const Layout &Ly, const Step &St, const int *skip_seq, const uint16_t *t2k,
                         const uint16_t *t2v, uint16_t *stk, uint16_t *stv, int kinds, hipStream_t s);
hipError_t launch_keys16(const Layout &Ly, const Step &St, const int *skip_seq, hipStream_t s);
hipError_t launch_promoted4(const Layout &Ly, const Step &St, const int *skip_seq, hipStream_t s);
hipError_t launch_promoted16(const Layout &Ly, const Step &St, const int *skip_seq, hipStream_t s);
// part: 1 the rank check, 2 the merge of the partials, 3 both
hipError_t launch_merge_impl(const Layout &Ly, const Step &St, const Th &th, const int *skip_seq,
                             uint32_t *plist, uint64_t *keys, int part, hipStream_t s);
hipError_t launch_dense_src(int d, int G, const DenseSrc &S, int nsplit, int batch,
                            hipStream_t s);
// profiling: folds the clock slots of nk timed kernels into 2 nk words and
// re-arms the slots
hipError_t launch_clock_fold(unsigned long long *clk, unsigned long long *out, int nk, hipStream_t s);

}  // namespace ckv
