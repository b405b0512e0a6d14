// ckv_api.cpp -- host runtime and C ABI of the certified quantized-KV
// library: cache allocation (tier 1 in HBM, tier 2 FP16 originals in pinned
// host memory, staging and scratch), the append path, and the orchestration
// of a decode step with its host round trips (page lists after selection,
// rank verdicts after the promoted pass).
//
// Section tags refer to the page "Runtime-Certified Bounded-Error Quantized
// Attention" (technical summary): [Meth-1] tiered storage, [Meth-3] the
// adaptive selection and the fallback ladder.
#include <hip/hip_runtime.h>
#include <immintrin.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <climits>
#include <condition_variable>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <memory>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "../../include/ckv.h"
#include "ckv_internal.hpp"

using namespace ckv;

namespace {

thread_local std::string g_err;

ckv_status fail(ckv_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

}  // namespace

// Sets the calling thread's last-error message (for the other translation
// units of the library) and returns `st`.
int ckv::set_error(int st, const char *msg) {
    g_err = msg;
    return st;
}

namespace {

#define HIPCHK(expr)                                                                        \
    do {                                                                                    \
        hipError_t e_ = (expr);                                                             \
        if (e_ != hipSuccess)                                                               \
            return fail(CKV_EHIP, "%s failed: %s (%s:%d)", #expr, hipGetErrorString(e_),    \
                        __FILE__, __LINE__);                                                \
    } while (0)

enum { PH_SCORE, PH_SELECT, PH_TAIL, PH_PAGE, PH_PROMO4, PH_FALLBACK, PH_STEP, PH_MERGE, PH_KEYS, PH_PROMO16, PH_N = 10 };
enum { KEV_SCORE, KEV_SELECT, KEV_TAIL, KEV_KEYS, KEV_PROMO4, KEV_PROMO16, KEV_RANK, KEV_MERGE, KEV_GATHER, KEV_PROMO16B,
       KEV_N };

}  // namespace

// Paging streams.  A host-to-device copy costs about 10 us of its stream's
// time beyond the bytes on the link; copies on two streams overlap that
// latency (measured: 2 streams beat 1 by 11-16% per layer-step, 4 streams
// share hardware queues with the compute stream and do slightly worse).
constexpr int NSIDE = 2;

// Staged paging: host threads pack the listed FP16 blocks of a step into a
// ring of pinned chunks; each chunk crosses the host link in one copy and a
// kernel moves its blocks to their staging slots.  Only listed blocks cross
// the link, and the per-copy cost is paid once per chunk, not per run.
constexpr int PAGE_SLOTS = 16;                   // ring chunks, a multiple of NSIDE
constexpr size_t PAGE_CHUNK = (size_t)4 << 20;  // block bytes per chunk (4 MiB: 3% faster than 2)
static_assert(PAGE_SLOTS % NSIDE == 0, "a ring slot must stay on one stream");

struct Stager {
    int device = 0, nthreads = 0;
    uint8_t *hring = nullptr, *dring = nullptr;  // pinned ring, its device twin
    size_t stride = 0;                           // bytes per chunk slot
    int per_chunk = 0, blk_bytes = 0;
    hipEvent_t ev[PAGE_SLOTS] = {};  // the last copy + scatter out of each slot
    // the current job: blocks in copy order (K first), chunk bounds
    std::vector<const void *> src, vsrc;
    std::vector<uint64_t> dst, vdst;
    std::vector<int> cstart;
    int nchunk = 0;
    std::unique_ptr<std::atomic<int>[]> ready;
    size_t ready_cap = 0;
    std::atomic<int> next{0}, issued{0}, busy{0}, err{0};
    std::vector<std::thread> th;
    std::mutex m;
    std::condition_variable cv;
    uint64_t gen = 0;
    bool quit = false;
};

// Pack one block into the ring with streaming (non-temporal) stores: the
// chunk goes to memory, not into the CPU's caches, so that the copy engine's
// reads of it do not have to pull dirty lines out of them.  `n` is a
// multiple of 64 bytes and `dst` 16-byte aligned.
static void pack_block(void *dst, const void *src, size_t n) {
    const __m128i *s = static_cast<const __m128i *>(src);
    __m128i *d = static_cast<__m128i *>(dst);
    for (size_t i = 0; i < n / 16; i += 4) {
        const __m128i a = _mm_loadu_si128(s + i), b = _mm_loadu_si128(s + i + 1);
        const __m128i x = _mm_loadu_si128(s + i + 2), y = _mm_loadu_si128(s + i + 3);
        _mm_stream_si128(d + i, a);
        _mm_stream_si128(d + i + 1, b);
        _mm_stream_si128(d + i + 2, x);
        _mm_stream_si128(d + i + 3, y);
    }
}

// Read one byte of every page of [p, p + bytes) on `threads` threads, each a
// contiguous share.  Pinned host memory written only by the device is mapped
// into the process page by page on its first CPU access; the faults contend
// on one lock, and taken during packing they cut the packing rate about
// tenfold, so staged paging takes them all up front.
static void touch_pages(const void *p, size_t bytes, int threads) {
    const size_t pg = 4096, n = bytes / pg;
    std::atomic<uint64_t> sink{0};
    std::vector<std::thread> th;
    for (int t = 0; t < threads; ++t)
        th.emplace_back([=, &sink] {
            const volatile uint8_t *b = static_cast<const volatile uint8_t *>(p);
            uint64_t acc = 0;
            for (size_t i = n * t / threads; i < n * (t + 1) / threads; ++i) acc += b[i * pg];
            sink += acc;
        });
    for (auto &x : th) x.join();
}

// A worker: take chunks in order of a shared counter; wait until the copy
// that last left the chunk's slot has finished, then pack the blocks behind
// the header of their destination addresses.
static void pack_chunk(Stager *S, int ci) {
    const int slot = ci % PAGE_SLOTS;
    while (S->issued.load(std::memory_order_acquire) <= ci - PAGE_SLOTS) std::this_thread::yield();
    // polled: the wait is at most one chunk's copy
    hipError_t qe;
    while ((qe = hipEventQuery(S->ev[slot])) == hipErrorNotReady) std::this_thread::yield();
    if (qe != hipSuccess) S->err.store(1);
    uint8_t *hc = S->hring + (size_t)slot * S->stride;
    uint64_t *hdr = reinterpret_cast<uint64_t *>(hc);
    for (int i = S->cstart[ci], j = 0; i < S->cstart[ci + 1]; ++i, ++j) {
        hdr[j] = S->dst[i];
        pack_block(hc + PAGE_HDR + (size_t)j * S->blk_bytes, S->src[i], S->blk_bytes);
    }
    _mm_sfence();  // the streaming stores are globally visible before the flag
    S->ready[ci].store(1, std::memory_order_release);
}

static void stager_work(Stager *S) {
    for (;;) {
        const int ci = S->next.fetch_add(1, std::memory_order_relaxed);
        if (ci >= S->nchunk) return;
        pack_chunk(S, ci);
    }
}

// `seen`: the generation current when the thread was started; the thread
// works only for later ones (a generation issued before it started belongs
// to the threads that were running then).
static void stager_thread(Stager *S, uint64_t seen) {
    (void)hipSetDevice(S->device);
    for (;;) {
        {
            std::unique_lock<std::mutex> lk(S->m);
            S->cv.wait(lk, [&] { return S->quit || S->gen != seen; });
            if (S->quit) return;
            seen = S->gen;
        }
        stager_work(S);
        S->busy.fetch_sub(1, std::memory_order_acq_rel);
    }
}

static void stager_stop(Stager *S) {
    {
        std::lock_guard<std::mutex> lk(S->m);
        S->quit = true;
    }
    S->cv.notify_all();
    for (auto &t : S->th) t.join();
    S->th.clear();
}

struct ckv_cache {
    ckv_config cfg{};
    Layout Ly{};
    int G = 0, d = 0, Nmax = 0, NS = 0, nsplit_cap = 0;
    int ncu = 0;  // compute units of the device
    size_t blk_fp16 = 0;  // elements of one FP16 block
    std::vector<void *> dev_allocs;
    size_t dev_bytes = 0, host_bytes = 0, tier1_bytes = 0;
    // tier 2 (pinned host)
    uint16_t *t2k = nullptr, *t2v = nullptr;
    size_t t2_bytes = 0;  // of each of t2k, t2v
    // staging and scratch (device)
    uint16_t *stage_k = nullptr, *stage_v = nullptr;
    float *score = nullptr, *score16 = nullptr, *part_tail = nullptr, *part_blk = nullptr, *part_blk16 = nullptr;
    double *qd = nullptr;
    float4 *bstat = nullptr;
    uint64_t *mfx = nullptr, *cval = nullptr, *m16 = nullptr, *keys = nullptr;
    uint32_t *sel = nullptr, *plist = nullptr, *dmask = nullptr, *wl = nullptr;
    int *wcnt = nullptr;
    uint2 *klist = nullptr;
    int *kcount = nullptr;
    int *pcnt = nullptr, *vpref = nullptr;
    // packed staging (staged paging without the persistent FP16 cache): the
    // packed K / V slot of each listed block, for the dense fallback, which
    // reads every block of a pair (pinned host copy, device copy)
    uint32_t *h_kmap = nullptr, *h_vmap = nullptr, *kmap = nullptr, *vmap = nullptr;
    HeadPlan *plan = nullptr;
    float2 *st16 = nullptr;
    int *dskip = nullptr;
    // pinned host mirrors
    uint32_t *h_sel = nullptr, *h_mask = nullptr;
    HeadPlan *h_plan = nullptr;
    int *h_skip = nullptr, *h_len = nullptr;
    std::vector<int> len;  // [L][B]
    // append staging (device, grown on demand)
    uint16_t *ain_k = nullptr, *ain_v = nullptr, *pk = nullptr, *pv = nullptr;
    size_t ain_cap = 0, pk_cap = 0;
    // paging streams: host-issued copies spread over several streams so that
    // the per-copy latency of one stream overlaps the others'
    hipStream_t side[NSIDE] = {};
    hipEvent_t ev_side[NSIDE] = {}, ev_kside[NSIDE] = {};
    // packed staging: the paging streams after the step's second-to-last
    // chunk (the FP16 value pass starts on the pairs complete by then)
    hipEvent_t ev_vsplit[NSIDE] = {};
    hipEvent_t ev_sel = nullptr, ev_paged = nullptr, ev_done = nullptr;
    // h_sel and h_plan as device addresses: the selection kernel's words and
    // plans are stored there by the device (mapped, coherent pinned memory)
    void *h_sel_dev = nullptr, *h_plan_dev = nullptr;
    hipEvent_t pev[15] = {};
    // profiling: the execution span of each timed kernel (scoring,
    // selection, tail, FP16 keys, INT4 promoted, FP16 promoted, rank check,
    // merge, the K gather of device paging) stamped by the kernel itself on the device's constant-rate
    // clock: KEV_N x CLK_WORDS (CLK_SLOTS start slots, then CLK_SLOTS end
    // slots, CLK_PAD words apart), armed from h_clk_init at creation, when
    // profiling is switched on and after a failed step; a profiled step
    // ends with a fold of each kernel's slots into its first start and last
    // end (dclkf, 2 words a kernel, read back into h_clkf), which re-arms them
    unsigned long long *dclk = nullptr, *h_clk_init = nullptr, *dclkf = nullptr, *h_clkf = nullptr;
    double clk_khz = 0.0;
    std::vector<uint8_t> staged_k, staged_v;  // [B][Hkv][Nmax] of the last step
    // persistent FP16 mirror of layers 0 .. pcache_layers-1: blocks paged in
    // once stay in HBM across steps (complete blocks never change)
    int pcache_layers = 0;
    // paging by the device (a kernel reading tier 2 over the host link)
    // instead of host-issued copies; the device addresses of tier 2
    bool device_gather = false;
    const uint16_t *t2k_dev = nullptr, *t2v_dev = nullptr;
    hipEvent_t ev_wl = nullptr;
    // device paging: the gather kernels' stream, and the ends of its K and
    // V gathers
    hipStream_t gstream = nullptr;
    hipEvent_t ev_gk = nullptr, ev_gv = nullptr;
    // the plans to the host right after the rank check (the fallback's
    // decisions), on a stream of their own: the paging streams are busy
    hipStream_t pstream = nullptr;
    hipEvent_t ev_rank = nullptr, ev_plan = nullptr;
    std::vector<uint16_t *> pstage_k, pstage_v;
    std::vector<std::vector<uint8_t>> pstaged_k, pstaged_v;
    std::vector<int> seq_flags;               // [B] of the last step
    bool have_step = false;
    int last_batch = 0, last_np = 0, last_nb = 0;
    bool prof = false;
    ckv_profile pf{};
    Stager *stager = nullptr;  // staged paging when set
    // ckv_inject_paging_fault: paging copies still to issue before the one
    // that reports failure (-1: none)
    long fault_after = -1;
};

namespace {

template <class T>
ckv_status dalloc(ckv_cache *c, T **p, size_t count) {
    void *ptr = nullptr;
    size_t bytes = std::max<size_t>(count * sizeof(T), 256);
    hipError_t e = hipMalloc(&ptr, bytes);
    if (e != hipSuccess) return fail(CKV_ENOMEM, "hipMalloc(%zu) failed: %s", bytes, hipGetErrorString(e));
    c->dev_allocs.push_back(ptr);
    c->dev_bytes += bytes;
    *p = static_cast<T *>(ptr);
    return CKV_OK;
}

template <class T>
ckv_status halloc(ckv_cache *c, T **p, size_t count, bool tier2 = false, bool dev_written = false) {
    void *ptr = nullptr;
    size_t bytes = std::max<size_t>(count * sizeof(T), 64);
    // tier 2 is also mapped into the device's address space (read by the
    // device-initiated paging kernel); buffers the device writes for the
    // host are mapped and coherent (the device's stores reach host memory)
    const unsigned flags = dev_written ? (hipHostMallocMapped | hipHostMallocCoherent)
                           : tier2     ? hipHostMallocMapped
                                       : hipHostMallocDefault;
    hipError_t e = hipHostMalloc(&ptr, bytes, flags);
    if (e != hipSuccess)
        return fail(CKV_ENOMEM, "hipHostMalloc(%zu) failed: %s", bytes, hipGetErrorString(e));
    if (tier2) c->host_bytes += bytes;
    *p = static_cast<T *>(ptr);
    return CKV_OK;
}

#define TRY(expr)                          \
    do {                                   \
        ckv_status s_ = (expr);            \
        if (s_ != CKV_OK) return s_;       \
    } while (0)

ckv_status grow(ckv_cache *c, uint16_t **a, uint16_t **b, size_t *cap, size_t need) {
    if (need <= *cap) return CKV_OK;
    if (*a) (void)hipFree(*a);
    if (*b) (void)hipFree(*b);
    *a = *b = nullptr;
    *cap = 0;
    HIPCHK(hipMalloc((void **)a, need * 2));
    HIPCHK(hipMalloc((void **)b, need * 2));
    *cap = need;
    return CKV_OK;
}

void fill_failed_reports(ckv_head_report *r, int n) {
    if (!r) return;
    for (int i = 0; i < n; ++i) {
        std::memset(&r[i], 0, sizeof r[i]);
        r[i].rung_max = -1;
    }
}

}  // namespace

// Blocks per split of the value passes: about 768 four-wave workgroups, so
// that the grid is resident in one round at three waves per SIMD (256 CUs x
// 4 SIMDs x 3 = 3072 waves) and every CU holds three of them (704, rounded to
// a multiple of 4 blocks, left a quarter of the CUs with two: the tail took
// 0.6 us longer at 32K x 4 and 128K); in [4, 64].
int ckv::split_blocks(int nb, int Hkv, int batch) {
    const long units = (long)nb * Hkv * batch;
    int bps = (int)((units + 767) / 768);
    bps = std::max(4, std::min(64, bps));
    return bps;
}

namespace {

float ru32h(double x) {
    float f = (float)x;
    if ((double)f < x) f = std::nextafter(f, INFINITY);
    return f;
}

}  // namespace

extern "C" {

const char *ckv_last_error(void) { return g_err.c_str(); }

void ckv_destroy(ckv_cache *c) {
    if (!c) return;
    (void)hipSetDevice(c->cfg.device);
    (void)hipDeviceSynchronize();
    for (void *p : c->dev_allocs) (void)hipFree(p);
    for (void *p : {(void *)c->ain_k, (void *)c->ain_v, (void *)c->pk, (void *)c->pv})
        if (p) (void)hipFree(p);
    for (void *p : {(void *)c->t2k, (void *)c->t2v, (void *)c->h_sel, (void *)c->h_mask,
                    (void *)c->h_plan, (void *)c->h_skip, (void *)c->h_len, (void *)c->h_clkf,
                    (void *)c->h_clk_init, (void *)c->h_kmap, (void *)c->h_vmap})
        if (p) (void)hipHostFree(p);
    for (hipStream_t st : c->side)
        if (st) (void)hipStreamDestroy(st);
    for (hipEvent_t e : c->ev_side)
        if (e) (void)hipEventDestroy(e);
    for (hipEvent_t e : c->ev_kside)
        if (e) (void)hipEventDestroy(e);
    for (hipEvent_t e : c->ev_vsplit)
        if (e) (void)hipEventDestroy(e);
    for (hipEvent_t e : {c->ev_sel, c->ev_paged, c->ev_done, c->ev_wl, c->ev_gk, c->ev_gv, c->ev_rank,
                         c->ev_plan})
        if (e) (void)hipEventDestroy(e);
    if (c->gstream) (void)hipStreamDestroy(c->gstream);
    if (c->pstream) (void)hipStreamDestroy(c->pstream);
    for (hipEvent_t e : c->pev)
        if (e) (void)hipEventDestroy(e);
    if (Stager *S = c->stager) {
        stager_stop(S);
        for (hipEvent_t e : S->ev)
            if (e) (void)hipEventDestroy(e);
        if (S->hring) (void)hipHostFree(S->hring);
        delete S;
    }
    delete c;
}

ckv_status ckv_create(const ckv_config *cfg, ckv_cache **out) {
    if (!cfg || !out) return fail(CKV_EINVAL, "null argument");
    *out = nullptr;
    const ckv_config &k = *cfg;
    if (k.n_layers < 1 || k.max_batch < 1 || k.n_kv_heads < 1 || k.n_q_heads < k.n_kv_heads ||
        k.n_q_heads % k.n_kv_heads || (k.head_dim != 64 && k.head_dim != 128) || k.max_context < 1)
        return fail(CKV_EINVAL, "bad cache shape");
    const int G = k.n_q_heads / k.n_kv_heads;
    const int vbits = k.v_bits == 0 ? 4 : k.v_bits;
    if (vbits != 4 && vbits != 8) return fail(CKV_EINVAL, "v_bits must be 4 or 8");
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(CKV_EINVAL, "n_q_heads / n_kv_heads must be 1, 2, 4 or 8");
    const int Nmax = (k.max_context + 63) / 64;
    // the FP16 staging area of one (sequence, kv head) is addressed with
    // 32-bit byte offsets (up to 1 GiB: 4M tokens at head_dim 128)
    if ((size_t)Nmax * 64 * k.head_dim * 2 > ((size_t)1 << 30))
        return fail(CKV_EINVAL, "max_context %d too large for head_dim %d", k.max_context, k.head_dim);
    if (Nmax > 65536) return fail(CKV_EINVAL, "max_context above 4M tokens");
    HIPCHK(hipSetDevice(k.device));
    int ncu = 0;
    HIPCHK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, k.device));
    ckv_cache *c = new ckv_cache();
    c->cfg = k;
    c->G = G;
    c->d = k.head_dim;
    c->Nmax = Nmax;
    c->NS = Nmax + 1;
    c->nsplit_cap = c->NS;
    c->blk_fp16 = (size_t)64 * k.head_dim;
    c->ncu = ncu;
    const int L = k.n_layers, B = k.max_batch, Hq = k.n_q_heads, Hkv = k.n_kv_heads, d = k.head_dim;
    const size_t nblk = (size_t)L * B * Hkv * Nmax;
    auto cleanup = [&](ckv_status s) {
        std::string msg = g_err;
        ckv_destroy(c);
        g_err = msg;
        return s;
    };
#define CTRY(expr)                     \
    do {                               \
        ckv_status s_ = (expr);        \
        if (s_ != CKV_OK) return cleanup(s_); \
    } while (0)
    Layout &Ly = c->Ly;
    Ly.L = L; Ly.B = B; Ly.Hq = Hq; Ly.Hkv = Hkv; Ly.d = d; Ly.G = G; Ly.Nmax = Nmax;
    Ly.vb = vbits;
    // tier 1 [Meth-1]
    size_t before = c->dev_bytes;
    CTRY(dalloc(c, &Ly.kq, nblk * 64 * d));
    CTRY(dalloc(c, &Ly.kmeta, nblk * d));
    CTRY(dalloc(c, &Ly.vq, nblk * 64 * d * vbits / 8));
    CTRY(dalloc(c, &Ly.vmeta, nblk * 64 * (d / 32)));
    CTRY(dalloc(c, &Ly.eta, nblk));
    c->tier1_bytes = c->dev_bytes - before;
    CTRY(dalloc(c, &Ly.vmin, (size_t)L * B * Hkv * d));
    CTRY(dalloc(c, &Ly.vmax, (size_t)L * B * Hkv * d));
    CTRY(dalloc(c, &Ly.vscale, (size_t)L * B * Hkv * (d / 32)));
    CTRY(dalloc(c, &Ly.kpart, (size_t)L * B * Hkv * 64 * d));
    CTRY(dalloc(c, &Ly.vpart, (size_t)L * B * Hkv * 64 * d));
    CTRY(dalloc(c, &Ly.len, (size_t)L * B));
    HIPCHK(hipMemset(Ly.len, 0, sizeof(int) * L * B));
    // tier 2: FP16 originals in pinned host memory [Meth-1]
    c->t2_bytes = nblk * 64 * d * sizeof(uint16_t);
    CTRY(halloc(c, &c->t2k, nblk * 64 * d, true));
    CTRY(halloc(c, &c->t2v, nblk * 64 * d, true));
    // staging for one layer-step and scratch
    const size_t sblk = (size_t)B * Hkv * Nmax;
    CTRY(dalloc(c, &c->stage_k, sblk * 64 * d));
    CTRY(dalloc(c, &c->stage_v, sblk * 64 * d));
    const size_t hsl = (size_t)B * Hq * c->NS;
    CTRY(dalloc(c, &c->score, hsl * 64));
    CTRY(dalloc(c, &c->score16, hsl * 64));
    CTRY(dalloc(c, &c->bstat, hsl));
    CTRY(dalloc(c, &c->mfx, hsl));
    CTRY(dalloc(c, &c->cval, hsl));
    CTRY(dalloc(c, &c->sel, sblk));
    CTRY(dalloc(c, &c->plan, (size_t)B * Hq));
    CTRY(dalloc(c, &c->st16, (size_t)B * Hq * Nmax));
    CTRY(dalloc(c, &c->m16, (size_t)B * Hq * Nmax));
    CTRY(dalloc(c, &c->part_tail, (size_t)B * Hq * c->nsplit_cap * (d + 2)));
    CTRY(dalloc(c, &c->part_blk, hsl * (d + 2)));
    CTRY(dalloc(c, &c->part_blk16, hsl * (d + 2)));
    CTRY(dalloc(c, &c->qd, (size_t)B * Hq * d));
    CTRY(dalloc(c, &c->plist, (size_t)B * Hq * Nmax));
    CTRY(dalloc(c, &c->wl, (size_t)WL_KINDS * B * Hkv * (Nmax + 1)));
    CTRY(dalloc(c, &c->wcnt, (size_t)WL_KINDS * B * Hkv));
    CTRY(dalloc(c, &c->klist, (size_t)B * Hkv * Nmax));
    CTRY(dalloc(c, &c->kcount, 1));
    CTRY(dalloc(c, &c->pcnt, (size_t)2 * B * Hkv));
    CTRY(dalloc(c, &c->vpref, (size_t)B * Hkv));
    CTRY(dalloc(c, &c->kmap, sblk));
    CTRY(dalloc(c, &c->vmap, sblk));
    CTRY(halloc(c, &c->h_kmap, sblk));
    CTRY(halloc(c, &c->h_vmap, sblk));
    CTRY(dalloc(c, &c->keys, (size_t)B * Hq * 2 * Nmax));
    CTRY(dalloc(c, &c->dskip, (size_t)B));
    CTRY(dalloc(c, &c->dmask, (size_t)B * Hkv));
    CTRY(halloc(c, &c->h_sel, sblk, false, true));
    CTRY(halloc(c, &c->h_mask, (size_t)B * Hkv));
    CTRY(halloc(c, &c->h_plan, (size_t)B * Hq, false, true));
    CTRY(halloc(c, &c->h_skip, (size_t)B));
    CTRY(halloc(c, &c->h_len, (size_t)L * B));
    c->len.assign((size_t)L * B, 0);
    c->staged_k.assign(sblk, 0);
    c->staged_v.assign(sblk, 0);
    for (int k = 0; k < NSIDE; ++k) {
        HIPCHK(hipStreamCreateWithFlags(&c->side[k], hipStreamNonBlocking));
        HIPCHK(hipEventCreateWithFlags(&c->ev_side[k], hipEventDisableTiming));
        HIPCHK(hipEventCreateWithFlags(&c->ev_kside[k], hipEventDisableTiming));
        HIPCHK(hipEventCreateWithFlags(&c->ev_vsplit[k], hipEventDisableTiming));
    }
    HIPCHK(hipEventCreateWithFlags(&c->ev_sel, hipEventDisableTiming));
    HIPCHK(hipEventCreateWithFlags(&c->ev_wl, hipEventDisableTiming));
    HIPCHK(hipStreamCreateWithFlags(&c->gstream, hipStreamNonBlocking));
    HIPCHK(hipStreamCreateWithFlags(&c->pstream, hipStreamNonBlocking));
    HIPCHK(hipEventCreateWithFlags(&c->ev_rank, hipEventDisableTiming));
    HIPCHK(hipEventCreateWithFlags(&c->ev_plan, hipEventDisableTiming));
    HIPCHK(hipEventCreateWithFlags(&c->ev_gk, hipEventDisableTiming));
    HIPCHK(hipEventCreateWithFlags(&c->ev_gv, hipEventDisableTiming));
    {
        void *pk = nullptr, *pv = nullptr;
        HIPCHK(hipHostGetDevicePointer(&pk, c->t2k, 0));
        HIPCHK(hipHostGetDevicePointer(&pv, c->t2v, 0));
        c->t2k_dev = static_cast<const uint16_t *>(pk);
        c->t2v_dev = static_cast<const uint16_t *>(pv);
        HIPCHK(hipHostGetDevicePointer(&c->h_sel_dev, c->h_sel, 0));
        HIPCHK(hipHostGetDevicePointer(&c->h_plan_dev, c->h_plan, 0));
    }
    HIPCHK(hipEventCreateWithFlags(&c->ev_paged, hipEventDisableTiming));
    HIPCHK(hipEventCreateWithFlags(&c->ev_done, hipEventDisableTiming));
    for (auto &e : c->pev) HIPCHK(hipEventCreate(&e));
    {
        const size_t nclk = (size_t)KEV_N * CLK_WORDS;
        CTRY(dalloc(c, &c->dclk, nclk));
        CTRY(dalloc(c, &c->dclkf, (size_t)2 * KEV_N));
        CTRY(halloc(c, &c->h_clkf, (size_t)2 * KEV_N));
        CTRY(halloc(c, &c->h_clk_init, nclk));
        // start slots at the largest value, end slots (and the padding) at 0
        for (size_t i = 0; i < nclk; ++i)
            c->h_clk_init[i] = (i % CLK_WORDS) < (size_t)CLK_SLOTS * CLK_PAD ? ~0ull : 0ull;
        HIPCHK(hipMemcpy(c->dclk, c->h_clk_init, nclk * sizeof(unsigned long long), hipMemcpyHostToDevice));
        int khz = 0;
        HIPCHK(hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, cfg->device));
        c->clk_khz = khz;
    }
    {
        // staged paging on by default with min(8, half the host's CPUs)
        // packing threads: four kept up with the link on 4 GiB of tier 2 but
        // not on 16 GiB of it at 128K (scattered blocks: 4.07 ms per
        // layer-step with four, 3.69 with eight, 3.71 with twelve)
        const unsigned hw = std::thread::hardware_concurrency();
        const ckv_status st = ckv_set_staged_paging(c, (int)std::max(1u, std::min(8u, hw / 2)));
        if (st != CKV_OK) return cleanup(st);
    }
    *out = c;
    return CKV_OK;
#undef CTRY
}

ckv_status ckv_reset_sequence(ckv_cache *c, int seq) {
    if (!c || seq < 0 || seq >= c->cfg.max_batch) return fail(CKV_EINVAL, "bad sequence");
    HIPCHK(hipSetDevice(c->cfg.device));
    for (int l = 0; l < c->cfg.n_layers; ++l) {
        c->len[(size_t)l * c->cfg.max_batch + seq] = 0;
        c->h_len[(size_t)l * c->cfg.max_batch + seq] = 0;
    }
    // the sequence's mirrored blocks are stale from now on
    const size_t per_seq = (size_t)c->Ly.Hkv * c->Ly.Nmax;
    for (int l = 0; l < c->pcache_layers; ++l) {
        std::fill(c->pstaged_k[l].begin() + seq * per_seq, c->pstaged_k[l].begin() + (seq + 1) * per_seq, 0);
        std::fill(c->pstaged_v[l].begin() + seq * per_seq, c->pstaged_v[l].begin() + (seq + 1) * per_seq, 0);
    }
    HIPCHK(hipMemcpy(c->Ly.len, c->h_len, sizeof(int) * c->cfg.n_layers * c->cfg.max_batch,
                     hipMemcpyHostToDevice));
    return CKV_OK;
}

ckv_status ckv_enable_fp16_cache(ckv_cache *c, size_t max_bytes, int *layers) {
    if (!c) return fail(CKV_EINVAL, "null cache");
    if (c->pcache_layers) return fail(CKV_ESTATE, "the FP16 cache is already enabled");
    HIPCHK(hipSetDevice(c->cfg.device));
    const size_t sblk = (size_t)c->Ly.B * c->Ly.Hkv * c->Ly.Nmax;
    const size_t per_layer = 2 * sblk * 64 * c->d * sizeof(uint16_t);
    const int m = (int)std::min<size_t>((size_t)c->cfg.n_layers, max_bytes / per_layer);
    // on an allocation failure the layers mirrored so far stay in use
    for (int l = 0; l < m; ++l) {
        uint16_t *k = nullptr, *v = nullptr;
        ckv_status st = dalloc(c, &k, sblk * 64 * c->d);
        if (st == CKV_OK) st = dalloc(c, &v, sblk * 64 * c->d);
        if (st != CKV_OK) {
            c->pcache_layers = l;
            if (layers) *layers = l;
            return st;
        }
        c->pstage_k.push_back(k);
        c->pstage_v.push_back(v);
        c->pstaged_k.emplace_back(sblk, 0);
        c->pstaged_v.emplace_back(sblk, 0);
    }
    c->pcache_layers = m;
    if (layers) *layers = m;
    return CKV_OK;
}

ckv_status ckv_set_device_paging(ckv_cache *c, int enable) {
    if (!c) return fail(CKV_EINVAL, "null cache");
    c->device_gather = enable != 0;
    return CKV_OK;
}

ckv_status ckv_set_staged_paging(ckv_cache *c, int threads) {
    if (!c) return fail(CKV_EINVAL, "null cache");
    if (threads < 0 || threads > 64) return fail(CKV_EINVAL, "threads must be 0 .. 64");
    HIPCHK(hipSetDevice(c->cfg.device));
    HIPCHK(hipDeviceSynchronize());
    if (c->stager) {
        // the ring stays allocated for a later switch back
        stager_stop(c->stager);
        c->stager->nthreads = 0;
    }
    if (threads == 0) return CKV_OK;
    if (!c->stager) {
        Stager *S = new Stager();
        S->device = c->cfg.device;
        S->blk_bytes = (int)(c->blk_fp16 * 2);
        S->per_chunk = (int)std::min<size_t>(PAGE_HDR / 8, std::max<size_t>(1, PAGE_CHUNK / S->blk_bytes));
        S->stride = PAGE_HDR + (size_t)S->per_chunk * S->blk_bytes;
        ckv_status st = halloc(c, &S->hring, (size_t)PAGE_SLOTS * S->stride);
        if (st == CKV_OK) st = dalloc(c, &S->dring, (size_t)PAGE_SLOTS * S->stride);
        for (int i = 0; i < PAGE_SLOTS && st == CKV_OK; ++i)
            if (hipEventCreateWithFlags(&S->ev[i], hipEventDisableTiming) != hipSuccess)
                st = fail(CKV_EHIP, "hipEventCreate failed");
        if (st != CKV_OK) {
            for (hipEvent_t e : S->ev)
                if (e) (void)hipEventDestroy(e);
            if (S->hring) (void)hipHostFree(S->hring);
            delete S;  // dring stays in the cache's device allocations
            return st;
        }
        c->stager = S;
        try {
            touch_pages(c->t2k, c->t2_bytes, threads);
            touch_pages(c->t2v, c->t2_bytes, threads);
            touch_pages(S->hring, (size_t)PAGE_SLOTS * S->stride, 1);
        } catch (...) {
            return fail(CKV_ENOMEM, "cannot start paging threads");
        }
    }
    Stager *S = c->stager;
    S->quit = false;
    S->nthreads = threads;
    uint64_t gen0;
    {
        std::lock_guard<std::mutex> lk(S->m);
        gen0 = S->gen;
    }
    try {
        for (int i = 0; i < threads; ++i) S->th.emplace_back(stager_thread, S, gen0);
    } catch (...) {
        stager_stop(S);
        S->nthreads = 0;  // staged paging stays off: no thread would pack
        return fail(CKV_ENOMEM, "cannot start paging threads");
    }
    return CKV_OK;
}

ckv_status ckv_seq_length(const ckv_cache *c, int layer, int seq, int *n) {
    if (!c || !n || layer < 0 || layer >= c->cfg.n_layers || seq < 0 || seq >= c->cfg.max_batch)
        return fail(CKV_EINVAL, "bad layer or sequence");
    *n = c->len[(size_t)layer * c->cfg.max_batch + seq];
    return CKV_OK;
}

ckv_status ckv_footprint(const ckv_cache *c, size_t *dev, size_t *host, size_t *tier1) {
    if (!c) return fail(CKV_EINVAL, "null cache");
    if (dev) *dev = c->dev_bytes;
    if (host) *host = c->host_bytes;
    if (tier1) *tier1 = c->tier1_bytes;
    return CKV_OK;
}

// Append [Meth-1]: pack the new tokens (with the unfinished block's earlier
// tokens) into whole FP16 blocks, quantize the completed blocks, keep the
// unfinished block FP16 on the device, update the value range, and copy
// the FP16 blocks to tier 2.
ckv_status ckv_append_kv(ckv_cache *c, int layer, int seq, const void *k, const void *v,
                         int ntok, int src_on_device, void *stream) {
    if (!c) return fail(CKV_EINVAL, "null cache");
    const ckv_config &cf = c->cfg;
    if (layer < 0 || layer >= cf.n_layers || seq < 0 || seq >= cf.max_batch || ntok < 0)
        return fail(CKV_EINVAL, "bad layer, sequence or token count");
    if (ntok == 0) return CKV_OK;
    if (!k || !v) return fail(CKV_EINVAL, "null K or V");
    const size_t li = (size_t)layer * cf.max_batch + seq;
    const int len0 = c->len[li];
    if ((long)len0 + ntok > cf.max_context)
        return fail(CKV_ERANGE, "append of %d tokens to %d exceeds max_context %d", ntok, len0,
                    cf.max_context);
    HIPCHK(hipSetDevice(cf.device));
    hipStream_t s = (hipStream_t)stream;
    const int d = c->d, Hkv = cf.n_kv_heads;
    const size_t tokel = (size_t)Hkv * d;
    const uint16_t *kin = (const uint16_t *)k, *vin = (const uint16_t *)v;
    if (!src_on_device) {
        TRY(grow(c, &c->ain_k, &c->ain_v, &c->ain_cap, (size_t)ntok * tokel));
        HIPCHK(hipMemcpyAsync(c->ain_k, k, (size_t)ntok * tokel * 2, hipMemcpyHostToDevice, s));
        HIPCHK(hipMemcpyAsync(c->ain_v, v, (size_t)ntok * tokel * 2, hipMemcpyHostToDevice, s));
        kin = c->ain_k;
        vin = c->ain_v;
    }
    const int b0 = len0 / 64;
    const int new_len = len0 + ntok;
    const int b_end = (new_len - 1) / 64;
    const int nblk = b_end - b0 + 1;
    TRY(grow(c, &c->pk, &c->pv, &c->pk_cap, (size_t)Hkv * nblk * c->blk_fp16));
    const Layout &Ly = c->Ly;
    HIPCHK(launch_pack(Ly, layer, seq, kin, vin, len0, ntok, b0, nblk, c->pk, c->pv, s));
    const int nfull = new_len / 64 - b0;
    HIPCHK(launch_quant(Ly, layer, seq, b0, nfull, nblk, c->pk, c->pv, s));
    if (new_len % 64) HIPCHK(launch_set_partial(Ly, layer, seq, nblk - 1, nblk, c->pk, c->pv, s));
    HIPCHK(launch_vrange(Ly, layer, seq, vin, ntok, len0 == 0, s));
    // tier 2 receives the blocks this append completed; the unfinished block
    // is read from its device copy until it completes
    for (int g = 0; g < Hkv && nfull > 0; ++g) {
        const size_t dst = Ly.blk(layer, seq, g, b0) * c->blk_fp16;
        const size_t src = (size_t)g * nblk * c->blk_fp16;
        HIPCHK(hipMemcpyAsync(c->t2k + dst, c->pk + src, (size_t)nfull * c->blk_fp16 * 2,
                              hipMemcpyDeviceToHost, s));
        HIPCHK(hipMemcpyAsync(c->t2v + dst, c->pv + src, (size_t)nfull * c->blk_fp16 * 2,
                              hipMemcpyDeviceToHost, s));
    }
    c->h_len[li] = new_len;
    HIPCHK(hipMemcpyAsync(c->Ly.len + li, c->h_len + li, sizeof(int), hipMemcpyHostToDevice, s));
    HIPCHK(hipStreamSynchronize(s));
    c->len[li] = new_len;
    return CKV_OK;
}

// Decode append [Meth-1]: one token for each of sequences 0 .. batch-1 of a
// layer in one pass (the unfinished blocks' device copies, the value ranges
// and weight scales), then the blocks this token completed: quantized, and
// written to tier 2.
ckv_status ckv_append_token(ckv_cache *c, int layer, int batch, const void *k, const void *v,
                            int src_on_device, void *stream) {
    if (!c) return fail(CKV_EINVAL, "null cache");
    const ckv_config &cf = c->cfg;
    if (layer < 0 || layer >= cf.n_layers || batch < 0 || batch > cf.max_batch)
        return fail(CKV_EINVAL, "bad layer or batch");
    if (batch == 0) return CKV_OK;
    if (!k || !v) return fail(CKV_EINVAL, "null K or V");
    const size_t l0 = (size_t)layer * cf.max_batch;
    for (int n = 0; n < batch; ++n)
        if (c->len[l0 + n] + 1 > cf.max_context)
            return fail(CKV_ERANGE, "append to sequence %d exceeds max_context %d", n, cf.max_context);
    HIPCHK(hipSetDevice(cf.device));
    hipStream_t s = (hipStream_t)stream;
    const int d = c->d, Hkv = cf.n_kv_heads;
    const size_t tokel = (size_t)Hkv * d;
    const uint16_t *kin = (const uint16_t *)k, *vin = (const uint16_t *)v;
    if (!src_on_device) {
        TRY(grow(c, &c->ain_k, &c->ain_v, &c->ain_cap, (size_t)batch * tokel));
        HIPCHK(hipMemcpyAsync(c->ain_k, k, (size_t)batch * tokel * 2, hipMemcpyHostToDevice, s));
        HIPCHK(hipMemcpyAsync(c->ain_v, v, (size_t)batch * tokel * 2, hipMemcpyHostToDevice, s));
        kin = c->ain_k;
        vin = c->ain_v;
    }
    const Layout &Ly = c->Ly;
    HIPCHK(launch_append_token(Ly, layer, batch, kin, vin, s));
    const size_t bb = c->blk_fp16 * 2;  // bytes of one FP16 block
    for (int n = 0; n < batch; ++n) {
        const int nl = c->len[l0 + n] + 1;
        if (nl % 64) continue;
        // block b of (layer, n) is complete: quantize it from the device
        // copy ([Hkv] consecutive blocks) and write it to tier 2
        const int b = nl / 64 - 1;
        const uint16_t *kp = Ly.kpart + Ly.seqg(layer, n, 0) * c->blk_fp16;
        const uint16_t *vp = Ly.vpart + Ly.seqg(layer, n, 0) * c->blk_fp16;
        HIPCHK(launch_quant(Ly, layer, n, b, 1, 1, kp, vp, s));
        HIPCHK(hipMemcpy2DAsync(c->t2k + Ly.blk(layer, n, 0, b) * c->blk_fp16, (size_t)Ly.Nmax * bb, kp, bb, bb, Hkv,
                                hipMemcpyDeviceToHost, s));
        HIPCHK(hipMemcpy2DAsync(c->t2v + Ly.blk(layer, n, 0, b) * c->blk_fp16, (size_t)Ly.Nmax * bb, vp, bb, bb, Hkv,
                                hipMemcpyDeviceToHost, s));
    }
    for (int n = 0; n < batch; ++n) c->h_len[l0 + n] = c->len[l0 + n] + 1;
    HIPCHK(hipMemcpyAsync(c->Ly.len + l0, c->h_len + l0, sizeof(int) * batch, hipMemcpyHostToDevice, s));
    HIPCHK(hipStreamSynchronize(s));
    for (int n = 0; n < batch; ++n) c->len[l0 + n] += 1;
    return CKV_OK;
}

namespace {

// Copies of one paging round: tier 2 -> staging.
struct CopyList {
    std::vector<void *> dst, src;
    std::vector<size_t> size;
    size_t bytes = 0;
    void clear() {
        dst.clear();
        src.clear();
        size.clear();
        bytes = 0;
    }
};

// Largest run of unwanted blocks that is copied anyway to join two runs:
// a 16 KiB block costs ~0.3 us on the host link, a separate copy ~10 us of
// one stream's time, shared by the paging streams (12 was the best of
// 3, 6, 12, 24 at 32K and 128K contexts with two streams).
constexpr int PAGE_GAP = 12;
// per-copy cost, in bytes of link time, when spreading runs over the streams
constexpr size_t COPY_COST_BYTES = (size_t)512 << 10;

// Queue the FP16 blocks of (seq n, kv head g) whose flag is set (and not
// already staged) as runs of consecutive blocks, small gaps filled.
// First block at or after b that is wanted and not staged (N if none);
// both flag arrays hold 0 / 1 bytes, scanned eight at a time.
static int next_needed(const uint8_t *want, const uint8_t *staged, int b, int N) {
    for (; b + 8 <= N; b += 8) {
        uint64_t w, s;
        std::memcpy(&w, want + b, 8);
        std::memcpy(&s, staged + b, 8);
        const uint64_t need = w & ~s;
        if (need) return b + (__builtin_ctzll(need) >> 3);
    }
    while (b < N && (!want[b] || staged[b])) ++b;
    return b;
}

static void page_runs(ckv_cache *c, int layer, int n, int g, int N, const uint8_t *want,
               std::vector<uint8_t> &staged, const uint16_t *t2, uint16_t *stage, CopyList &cl) {
    const Layout &Ly = c->Ly;
    const size_t sb = ((size_t)n * Ly.Hkv + g) * Ly.Nmax;
    int b = 0;
    while (b < N) {
        b = next_needed(want, staged.data() + sb, b, N);
        if (b >= N) break;
        int e = b + 1, last = b;
        while (e < N && !staged[sb + e] && e - last <= PAGE_GAP) {
            if (want[e]) last = e;
            ++e;
        }
        e = last + 1;
        const size_t nbytes = (size_t)(e - b) * c->blk_fp16 * 2;
        cl.dst.push_back(stage + (sb + b) * c->blk_fp16);
        cl.src.push_back((void *)(t2 + Ly.blk(layer, n, g, b) * c->blk_fp16));
        cl.size.push_back(nbytes);
        cl.bytes += nbytes;
        for (int i = b; i < e; ++i) staged[sb + i] = 1;
        b = e;
    }
}

// One host-to-device paging copy on stream `st`.  With a fault injected by
// ckv_inject_paging_fault, the chosen copy is not issued and reports
// failure, as a failed hipMemcpyAsync would.
static hipError_t page_copy(ckv_cache *c, void *dst, const void *src, size_t bytes, hipStream_t st) {
    if (c->fault_after >= 0) {
        if (c->fault_after == 0) {
            c->fault_after = -1;
            return hipErrorUnknown;
        }
        --c->fault_after;
    }
    return hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, st);
}

// Issue a paging round over the paging streams (each run to the stream with
// the fewest bytes so far, one hipMemcpyAsync per run), then, if `join`,
// join them on side[0].
static ckv_status issue_copies(ckv_cache *c, CopyList &cl, bool join = true) {
    if (cl.size.empty()) return CKV_OK;
    CopyList per[NSIDE];
    size_t load[NSIDE] = {};
    for (size_t i = 0; i < cl.size.size(); ++i) {
        int k = 0;
        for (int j = 1; j < NSIDE; ++j)
            if (load[j] < load[k]) k = j;
        load[k] += cl.size[i] + COPY_COST_BYTES;
        per[k].dst.push_back(cl.dst[i]);
        per[k].src.push_back(cl.src[i]);
        per[k].size.push_back(cl.size[i]);
    }
    for (int k = 0; k < NSIDE; ++k) {
        CopyList &q = per[k];
        if (q.size.empty()) continue;
        for (size_t i = 0; i < q.size.size(); ++i) HIPCHK(page_copy(c, q.dst[i], q.src[i], q.size[i], c->side[k]));
        if (k > 0 && join) {
            HIPCHK(hipEventRecord(c->ev_side[k], c->side[k]));
            HIPCHK(hipStreamWaitEvent(c->side[0], c->ev_side[k], 0));
        }
    }
    return CKV_OK;
}

// Staged paging.  The FP16 blocks of (seq n, kv head g) whose flag is set
// and that are not staged yet, no gaps filled: runs of consecutive blocks of
// at least a chunk's bytes to `direct` (one copy each, as efficient as a
// chunk), the other blocks to the packing list.
// Next free slot of the packed K and V staging areas (the step's listed
// blocks in listing order).
struct Slots {
    uint32_t k = 0, v = 0;
};

// 16 flag bytes (0 or 1 each) as 16 bits.
static inline uint32_t flag_bits16(const uint8_t *p) {
    const __m128i v = _mm_loadu_si128(reinterpret_cast<const __m128i *>(p));
    return (uint32_t)_mm_movemask_epi8(_mm_sub_epi8(_mm_setzero_si128(), v));
}

// List the blocks of (n, g) that `want` asks for and are not staged yet:
// runs of at least a chunk's size as direct copies, the rest for packing.
// Block-indexed staging (`slot` null): a block's destination is its (pair,
// block) place, kept in `dst` as an address.  Packed staging: it is the
// next slot of the area, kept in `dst` as the slot number (and in `map`),
// so a run takes consecutive slots and packed blocks keep listing order.
// `want`: bit masks, 64 blocks a word, (N + 63) / 64 words, no bit at or
// past N; `need`: scratch of as many words.  The runs are found with bit
// operations (first set bit, then the first clear one after it), so the
// cost is a few operations per run plus the stores of each listed block.
static void list_blocks(ckv_cache *c, int layer, int n, int g, int N, const uint64_t *want,
                        std::vector<uint8_t> &staged, const uint16_t *t2, uint16_t *stage,
                        std::vector<const void *> &src, std::vector<uint64_t> &dst, CopyList &direct,
                        uint32_t *slot, uint32_t *map, uint64_t *need) {
    const Layout &Ly = c->Ly;
    const size_t sb = ((size_t)n * Ly.Hkv + g) * Ly.Nmax, bb = c->blk_fp16 * 2;
    const int min_run = (int)((PAGE_CHUNK + bb - 1) / bb);
    uint8_t *st = staged.data() + sb;
    const int nw = (N + 63) / 64;
    int cnt = 0;
    for (int w = 0; w < nw; ++w) {
        const int b0 = 64 * w;
        uint64_t sm = 0;
        if (b0 + 64 <= N) {
            for (int k = 0; k < 4; ++k) sm |= (uint64_t)flag_bits16(st + b0 + 16 * k) << (16 * k);
        } else {
            for (int b = b0; b < N; ++b) sm |= (uint64_t)(st[b] != 0) << (b - b0);
        }
        need[w] = want[w] & ~sm;
        cnt += __builtin_popcountll(need[w]);
    }
    if (!cnt) return;
    const size_t k0 = src.size();
    src.resize(k0 + cnt);
    dst.resize(k0 + cnt);
    const void **ps = src.data() + k0;
    uint64_t *pd = dst.data() + k0;
    const uint16_t *from = t2 + Ly.blk(layer, n, g, 0) * c->blk_fp16;
    uint32_t sl = slot ? *slot : 0;
    int w = 0;
    uint64_t m = need[0];
    for (;;) {
        while (!m && ++w < nw) m = need[w];
        if (!m) break;
        const int b = 64 * w + __builtin_ctzll(m);
        // the run's end: the first block at or after b not needed
        int we = w;
        uint64_t x = ~need[w] & (~0ull << (b - 64 * w));
        while (!x && ++we < nw) x = ~need[we];
        const int e = x ? std::min(N, 64 * we + __builtin_ctzll(x)) : N;
        if (e - b >= min_run) {
            direct.dst.push_back(stage + (slot ? (size_t)sl : sb + b) * c->blk_fp16);
            direct.src.push_back((void *)(from + (size_t)b * c->blk_fp16));
            direct.size.push_back((size_t)(e - b) * bb);
            direct.bytes += (size_t)(e - b) * bb;
            for (int i = b; i < e; ++i) {
                if (slot) map[sb + i] = sl++;
                st[i] = 1;
            }
        } else {
            for (int i = b; i < e; ++i) {
                *ps++ = from + (size_t)i * c->blk_fp16;
                if (slot) {
                    map[sb + i] = sl;
                    *pd++ = sl++;
                } else {
                    *pd++ = (uint64_t)(uintptr_t)(stage + (sb + i) * c->blk_fp16);
                }
                st[i] = 1;
            }
        }
        if (e >= N) break;
        w = e / 64;
        m = need[w] & (~0ull << (e % 64));
    }
    src.resize((size_t)(ps - src.data()));
    dst.resize((size_t)(pd - dst.data()));
    if (slot) *slot = sl;
}

// The selection words of one (sequence, kv head), sl[0 .. N), as bit masks
// of (N + 63) / 64 words (no bit at or past N), four words per SSE step:
// km blocks in P of some head, vm blocks with FP16 values for some head, im
// blocks in P of some head that has no FP16 values there, tm blocks with
// some head outside P and VP (the tail's).
static void sel_masks(const uint32_t *sl, int N, uint32_t allg, uint64_t *km, uint64_t *vm, uint64_t *im,
                      uint64_t *tm) {
    const int nw = (N + 63) / 64;
    for (int w = 0; w < nw; ++w) km[w] = vm[w] = im[w] = tm[w] = 0;
    const __m128i A = _mm_set1_epi32((int)allg), Z = _mm_setzero_si128();
    auto nz4 = [&](__m128i x) {  // lanes not equal to Z, as 4 bits
        return (uint64_t)(~_mm_movemask_ps(_mm_castsi128_ps(_mm_cmpeq_epi32(x, Z))) & 0xF);
    };
    int b = 0;
    for (; b + 4 <= N; b += 4) {
        const __m128i x = _mm_loadu_si128(reinterpret_cast<const __m128i *>(sl + b));
        const __m128i p = _mm_and_si128(x, A), v = _mm_and_si128(_mm_srli_epi32(x, 8), A);
        const int w = b >> 6, sh = b & 63;
        km[w] |= nz4(p) << sh;
        vm[w] |= nz4(v) << sh;
        im[w] |= nz4(_mm_andnot_si128(v, p)) << sh;
        tm[w] |= (uint64_t)(~_mm_movemask_ps(_mm_castsi128_ps(_mm_cmpeq_epi32(_mm_or_si128(p, v), A))) & 0xF) << sh;
    }
    for (; b < N; ++b) {
        const uint32_t p = sl[b] & allg, v = (sl[b] >> 8) & allg;
        const int w = b >> 6, sh = b & 63;
        km[w] |= (uint64_t)(p != 0) << sh;
        vm[w] |= (uint64_t)(v != 0) << sh;
        im[w] |= (uint64_t)((p & ~v) != 0) << sh;
        tm[w] |= (uint64_t)((p | v) != allg) << sh;
    }
}

// Blocks [0, N) as a bit mask.
static void ones_mask(uint64_t *m, int N) {
    const int nw = (N + 63) / 64;
    for (int w = 0; w < nw; ++w) m[w] = 64 * (w + 1) <= N ? ~0ull : (1ull << (N - 64 * w)) - 1ull;
}

static int popcount_mask(const uint64_t *m, int N) {
    int c = 0;
    for (int w = 0; w < (N + 63) / 64; ++w) c += __builtin_popcountll(m[w]);
    return c;
}

// A mask as 0 / 1 bytes (the run copies' lists take bytes).
static void mask_bytes(const uint64_t *m, int N, uint8_t *out) {
    for (int b = 0; b < N; ++b) out[b] = (uint8_t)((m[b >> 6] >> (b & 63)) & 1);
}

// Copy the listed blocks: the long K runs and chunks of packed K blocks, then
// the long V runs and chunks of packed V blocks.  Block-indexed staging
// (pk null): a chunk is one copy into its device ring slot and one scatter
// to the blocks' places.  Packed staging (pk, pv: the K and V areas): a
// chunk holds consecutive slots and is one copy straight to them.  Once the
// K side is issued, `s` waits for it (the FP16-key pass needs only K); at
// the end the paging streams are joined on side[0].  `vsplit` (packed
// staging, may be null): with two V chunks or more, ev_vsplit is recorded
// on every paging stream after the second-to-last chunk and *vsplit set to
// the V slot below which every slot is then issued (0: no such point).
static ckv_status stage_and_copy(ckv_cache *c, Stager &S, CopyList &kruns, CopyList &vruns, hipStream_t s,
                                 size_t &bytes, uint16_t *pk, uint16_t *pv, uint32_t *vsplit = nullptr) {
    const size_t nk = S.src.size();
    S.src.insert(S.src.end(), S.vsrc.begin(), S.vsrc.end());
    S.dst.insert(S.dst.end(), S.vdst.begin(), S.vdst.end());
    S.vsrc.clear();
    S.vdst.clear();
    const size_t nblk = S.src.size();
    S.cstart.clear();
    // the step's first chunk is 1/8 of a full one and each next one 1.25x
    // the last, up to full size: the first copy starts after a short packing
    // time, and the chunks that the threads start on together become ready
    // one after another rather than all at once (measured: 2% off the
    // 128K-token step against 1/8, 1/4, 1/2, then full chunks); packed
    // staging also starts a chunk wherever the slots stop being consecutive
    // (around a direct run)
    const bool packed = pk != nullptr;
    auto cut = [&](size_t i0, size_t i1, size_t i, int cap) {
        size_t e = std::min(i1, i + (size_t)cap);
        if (packed)
            for (size_t j = i + 1; j < e; ++j)
                if (S.dst[j] != S.dst[j - 1] + 1) {
                    e = j;
                    break;
                }
        (void)i0;
        return e;
    };
    double frac = 0.125;
    for (size_t i = 0; i < nk; frac *= 1.25) {
        S.cstart.push_back((int)i);
        i = cut(0, nk, i, std::max(1, (int)(S.per_chunk * std::min(1.0, frac))));
    }
    const int nkc = (int)S.cstart.size();
    for (size_t i = nk; i < nblk;) {
        S.cstart.push_back((int)i);
        i = cut(nk, nblk, i, S.per_chunk);
    }
    S.nchunk = (int)S.cstart.size();
    S.cstart.push_back((int)nblk);
    const int csplit = vsplit && packed && S.nchunk - 2 >= nkc ? S.nchunk - 2 : -1;
    if (vsplit) *vsplit = 0;
    auto kjoin = [&]() -> hipError_t {
        for (int k = 0; k < NSIDE; ++k) {
            hipError_t e = hipEventRecord(c->ev_kside[k], c->side[k]);
            if (e == hipSuccess) e = hipStreamWaitEvent(s, c->ev_kside[k], 0);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    };
    hipError_t e = hipSuccess;
    S.err.store(0);
    ckv_status runs_st = CKV_OK;  // a failed run copy (its message already set)
    // the long runs go first: the copy engines work on them while the
    // threads pack the first chunks
    if ((runs_st = issue_copies(c, kruns, false)) != CKV_OK) e = hipErrorUnknown;
    bytes += kruns.bytes;
    if (nkc == 0 && e == hipSuccess) {
        e = kjoin();
        if (e == hipSuccess && (runs_st = issue_copies(c, vruns, false)) != CKV_OK) e = hipErrorUnknown;
        bytes += vruns.bytes;
    }
    if (S.nchunk > 0 && e == hipSuccess) {
        // the threads start on chunks 1, 2, ... (waking them before the long
        // runs are issued made the 32K-token step 1% slower)
        if ((size_t)S.nchunk > S.ready_cap) {
            S.ready_cap = std::max<size_t>(S.nchunk, 2 * S.ready_cap);
            S.ready.reset(new std::atomic<int>[S.ready_cap]);
        }
        for (int i = 0; i < S.nchunk; ++i) S.ready[i].store(0, std::memory_order_relaxed);
        S.next.store(1);  // chunk 0 is packed here while the threads wake
        S.issued.store(0);
        S.err.store(0);
        S.busy.store(S.nthreads);
        {
            std::lock_guard<std::mutex> lk(S.m);
            ++S.gen;
        }
        S.cv.notify_all();
        pack_chunk(&S, 0);
        for (int ci = 0; ci < S.nchunk && e == hipSuccess; ++ci) {
            while (!S.ready[ci].load(std::memory_order_acquire)) std::this_thread::yield();
            if (S.err.load()) {
                e = hipErrorUnknown;
                break;
            }
            const int slot = ci % PAGE_SLOTS, nb = S.cstart[ci + 1] - S.cstart[ci];
            hipStream_t st = c->side[slot % NSIDE];
            uint8_t *hc = S.hring + (size_t)slot * S.stride;
            size_t cb;
            if (packed) {
                // the blocks straight to their consecutive slots
                uint16_t *area = ci < nkc ? pk : pv;
                uint8_t *dst = reinterpret_cast<uint8_t *>(area) + (size_t)S.dst[S.cstart[ci]] * S.blk_bytes;
                cb = (size_t)nb * S.blk_bytes;
                e = page_copy(c, dst, hc + PAGE_HDR, cb, st);
            } else {
                uint8_t *dc = S.dring + (size_t)slot * S.stride;
                cb = PAGE_HDR + (size_t)nb * S.blk_bytes;
                e = page_copy(c, dc, hc, cb, st);
                if (e == hipSuccess) e = launch_page_scatter(dc, nb, S.blk_bytes, st);
            }
            if (e == hipSuccess) e = hipEventRecord(S.ev[slot], st);
            if (e != hipSuccess) break;
            bytes += cb;
            S.issued.store(ci + 1, std::memory_order_release);
            if (ci == csplit) {
                for (int k = 0; k < NSIDE && e == hipSuccess; ++k) e = hipEventRecord(c->ev_vsplit[k], c->side[k]);
                if (e != hipSuccess) break;
                *vsplit = (uint32_t)S.dst[S.cstart[ci + 1] - 1] + 1;
            }
            if (ci + 1 == nkc) {
                e = kjoin();
                if (e == hipSuccess && (runs_st = issue_copies(c, vruns, false)) != CKV_OK) e = hipErrorUnknown;
                bytes += vruns.bytes;
            }
        }
        if (e != hipSuccess) {
            // let the workers drain without packing further chunks
            S.next.store(INT_MAX / 2);
            S.issued.store(INT_MAX / 2);
        }
        while (S.busy.load(std::memory_order_acquire) > 0) std::this_thread::yield();
    }
    for (int k = 1; k < NSIDE && e == hipSuccess; ++k) {
        e = hipEventRecord(c->ev_side[k], c->side[k]);
        if (e == hipSuccess) e = hipStreamWaitEvent(c->side[0], c->ev_side[k], 0);
    }
    if (c->prof) c->pf.copies += S.nchunk + kruns.size.size() + vruns.size.size();
    S.src.clear();
    S.dst.clear();
    if (runs_st != CKV_OK) return runs_st;
    if (S.err.load()) return fail(CKV_EHIP, "staged paging: a ring slot's event failed");
    if (e != hipSuccess) return fail(CKV_EHIP, "staged paging: %s", hipGetErrorString(e));
    return CKV_OK;
}

}  // namespace

namespace {

ckv_status certified_step(ckv_cache *c, int layer, const void *q, int batch, const ckv_thresholds *th,
                          float *out, ckv_head_report *report, void *stream) {
    auto t_start = std::chrono::steady_clock::now();
    if (!c) return fail(CKV_EINVAL, "null cache");
    const ckv_config &cf = c->cfg;
    const int Hq = cf.n_q_heads, Hkv = cf.n_kv_heads, G = c->G, d = c->d;
    if (report && batch > 0 && batch <= cf.max_batch) fill_failed_reports(report, batch * Hq);
    if (layer < 0 || layer >= cf.n_layers || batch < 1 || batch > cf.max_batch || !q || !th || !out ||
        !report)
        return fail(CKV_EINVAL, "bad layer, batch or null pointer");
    if (!(th->tau_cov >= 0.0f && th->tau_cov <= 1.0f) || !(th->sm_scale > 0.0f) ||
        !std::isfinite(th->sm_scale) || th->n_widen < 0 || std::isnan(th->k_tol) ||
        std::isnan(th->v_tol) || std::isnan(th->rank_tol) || std::isnan(th->f_layer))
        return fail(CKV_EINVAL, "bad thresholds");
    int nb = 0, np_any = 0;
    for (int n = 0; n < batch; ++n) {
        const int L_ = c->len[(size_t)layer * cf.max_batch + n];
        if (L_ < 1) return fail(CKV_ESTATE, "sequence %d of layer %d is empty", n, layer);
        nb = std::max(nb, L_ / 64);
        np_any |= (L_ % 64) != 0;
    }
    HIPCHK(hipSetDevice(cf.device));
    hipStream_t s = (hipStream_t)stream;
    const Layout &Ly = c->Ly;

    Step St{};
    St.layer = layer;
    St.batch = batch;
    St.nb = nb;
    St.p16_lo = 0;
    St.p16_hi = INT_MAX;
    St.NS = c->NS;
    St.bps = split_blocks(nb, Hkv, batch);
    St.ncu = c->ncu;
    St.nsplit = (nb + St.bps - 1) / St.bps;
    St.nsplit_cap = c->nsplit_cap;
    St.sm = th->sm_scale;
    St.q = (const uint16_t *)q;
    St.score = c->score;
    St.score16 = c->score16;
    St.bstat = c->bstat;
    St.mfx = c->mfx;
    St.cval = c->cval;
    St.sel = c->sel;
    St.plan = c->plan;
    St.st16 = c->st16;
    St.m16 = c->m16;
    St.part_tail = c->part_tail;
    St.part_blk = c->part_blk;
    St.part_blk16 = c->part_blk16;
    // staging of this layer: its persistent mirror, or the shared area
    const bool pers = layer < c->pcache_layers;
    uint16_t *stage_k = pers ? c->pstage_k[layer] : c->stage_k;
    uint16_t *stage_v = pers ? c->pstage_v[layer] : c->stage_v;
    std::vector<uint8_t> &staged_k = pers ? c->pstaged_k[layer] : c->staged_k;
    std::vector<uint8_t> &staged_v = pers ? c->pstaged_v[layer] : c->staged_v;
    const bool gather = c->device_gather && !pers;
    // staged paging (host-packed chunks) for the host-issued copies
    const bool staged = !gather && c->stager && c->stager->nthreads > 0;
    // staged paging into the packed areas (the persistent FP16 cache keeps
    // block-indexed staging: its blocks stay across steps)
    const bool packed = staged && !pers;
    if (staged) {
        c->stager->src.clear();
        c->stager->dst.clear();
        c->stager->vsrc.clear();
        c->stager->vdst.clear();
    }
    St.stage_k = stage_k;
    St.stage_v = stage_v;
    St.qd = c->qd;
    St.wl = c->wl;
    St.wcnt = c->wcnt;
    St.klist = c->klist;
    St.kcount = c->kcount;
    St.pcnt = c->pcnt;
    St.vpref = c->vpref;
    St.packed = packed ? 1 : 0;
    St.out = out;
    Th T{};
    T.tau = th->tau_cov;
    T.k_tol = th->k_tol;
    T.v_tol = th->v_tol;
    T.rank_tol = th->rank_tol;
    T.f_layer = th->f_layer;
    T.n_widen = th->n_widen;
    T.vcap = th->v_cap_blocks;

    hipEvent_t *E = c->pev;
    const bool prof = c->prof;
    // the next kernel launched with St stamps its span in slot k (profiling)
    auto kev = [&](int k) { St.clk = prof ? c->dclk + (size_t)k * CLK_WORDS : nullptr; };
    // K1: INT8 scoring pass; K2: selection, bounds, rungs 1-2
    kev(KEV_SCORE);
    HIPCHK(launch_score(Ly, St, s));
    kev(KEV_SELECT);
    HIPCHK(launch_select(Ly, St, T, s));
    St.clk = nullptr;
    // page lists and plans to the host (the round trip of the selection): a
    // small kernel right behind the selection stores them into mapped host
    // memory, so the host's wait has no copy on another stream to wait for
    // (a cross-stream wait and two runtime copies had started ~17 us after
    // the selection ended); the passes below follow it by a few us
    const size_t selbytes = (size_t)batch * Hkv * Ly.Nmax * sizeof(uint32_t);
    HIPCHK(launch_to_host(c->sel, c->h_sel_dev, selbytes, c->plan, c->h_plan_dev,
                          sizeof(HeadPlan) * batch * Hq, s));
    HIPCHK(hipEventRecord(c->ev_sel, s));
    // block lists of the value passes and the sequences' skip flags; K3:
    // tail blocks; both overlap the host's page lists and the paging below
    HIPCHK(launch_worklist(Ly, St, c->dskip, s));
    HIPCHK(hipEventRecord(c->ev_wl, s));
    if (gather) {
        // device-initiated paging starts from the device's own block lists
        // and skip flags, before the host has seen the selection: K blocks,
        // then V blocks, on a stream of their own (skipped sequences are
        // left to the host's copies below)
        HIPCHK(hipStreamWaitEvent(c->gstream, c->ev_wl, 0));
        if (prof) HIPCHK(hipEventRecord(E[5], c->gstream));
        kev(KEV_GATHER);
        HIPCHK(launch_gather(Ly, St, c->dskip, c->t2k_dev, c->t2v_dev, stage_k, stage_v, 1, c->gstream));
        St.clk = nullptr;
        HIPCHK(hipEventRecord(c->ev_gk, c->gstream));
        HIPCHK(launch_gather(Ly, St, c->dskip, c->t2k_dev, c->t2v_dev, stage_k, stage_v, 2, c->gstream));
        HIPCHK(hipEventRecord(c->ev_gv, c->gstream));
    }
    kev(KEV_TAIL);
    if (St.nsplit > 0) HIPCHK(launch_tail(Ly, St, s));
    St.clk = nullptr;
    HIPCHK(hipEventSynchronize(c->ev_sel));

    // rung 4 before paging: a cap exhausted on any head of the sequence
    std::vector<uint8_t> wantk(Ly.Nmax), wantv(Ly.Nmax);
    const int mw = (Ly.Nmax + 63) / 64;
    std::vector<uint64_t> needw(mw), kmask(mw), vmask(mw), imask(mw), tmask(mw);
    if (!pers) {
        std::fill(c->staged_k.begin(), c->staged_k.end(), 0);
        std::fill(c->staged_v.begin(), c->staged_v.end(), 0);
    }
    size_t paged = 0;
    CopyList cl, clk;  // V runs (and the fallback's), K runs
    if (prof && !gather) HIPCHK(hipEventRecord(E[5], c->side[0]));
    const uint32_t allg = (1u << G) - 1u;
    for (int n = 0; n < batch; ++n) {
        int skip = 0;
        for (int h = 0; h < Hq; ++h) skip |= (c->h_plan[(size_t)n * Hq + h].flags >> 1) & 1;
        c->h_skip[n] = skip;
    }
    // packed slots, in the order the worklist kernel assumes: the pairs not
    // skipped, pair by pair, then the skipped ones (all their blocks)
    Slots slots;
    std::vector<int> pc4, pc16;  // the promoted passes' list lengths per pair
    std::vector<uint32_t> vend((size_t)batch * Hkv, 0);  // packed: a pair's V slots end here
    for (int pass = 0; pass < 2; ++pass)
        for (int n = 0; n < batch; ++n) {
            const int skip = c->h_skip[n];
            if (skip != pass) continue;
            const int N = c->len[(size_t)layer * cf.max_batch + n] / 64;
            for (int g = 0; g < Hkv; ++g) {
                const uint32_t *sl = c->h_sel + ((size_t)n * Hkv + g) * Ly.Nmax;
                sel_masks(sl, N, allg, kmask.data(), vmask.data(), imask.data(), tmask.data());
                if (!skip) {
                    // this pair's entries in the worklist kernel's
                    // INT4-promoted and FP16-value lists
                    pc4.push_back(popcount_mask(imask.data(), N));
                    pc16.push_back(popcount_mask(vmask.data(), N) +
                                   ((c->len[(size_t)layer * cf.max_batch + n] % 64) ? 1 : 0));
                }
                if (prof) {
                    c->pf.tail_blocks += popcount_mask(tmask.data(), N);
                    if (!skip) {
                        c->pf.k16_blocks += popcount_mask(kmask.data(), N);
                        c->pf.v16_blocks += popcount_mask(vmask.data(), N);
                        c->pf.int4p_blocks += popcount_mask(imask.data(), N);
                    }
                    c->pf.q8_blocks += N;
                }
                if (skip) {
                    // every block of a skipped sequence (the dense pass)
                    ones_mask(kmask.data(), N);
                    ones_mask(vmask.data(), N);
                }
                if (gather && !skip) {
                    // the device copies this (seq, kv head)'s listed blocks itself
                    paged += (size_t)(popcount_mask(kmask.data(), N) + popcount_mask(vmask.data(), N)) *
                             c->blk_fp16 * 2;
                    continue;
                }
                if (staged) {
                    Stager &S = *c->stager;
                    list_blocks(c, layer, n, g, N, kmask.data(), staged_k, c->t2k, stage_k, S.src, S.dst, clk,
                                packed ? &slots.k : nullptr, c->h_kmap, needw.data());
                    list_blocks(c, layer, n, g, N, vmask.data(), staged_v, c->t2v, stage_v, S.vsrc, S.vdst, cl,
                                packed ? &slots.v : nullptr, c->h_vmap, needw.data());
                    if (!skip) vend[(size_t)n * Hkv + g] = slots.v;
                    continue;
                }
                mask_bytes(kmask.data(), N, wantk.data());
                mask_bytes(vmask.data(), N, wantv.data());
                page_runs(c, layer, n, g, N, wantk.data(), staged_k, c->t2k, stage_k, clk);
                page_runs(c, layer, n, g, N, wantv.data(), staged_v, c->t2v, stage_v, cl);
            }
        }
    {
        // the promoted passes' entries per split and grid widths
        long long t4 = 0, t16 = 0;
        for (int x : pc4) t4 += x;
        for (int x : pc16) t16 += x;
        St.t4 = (int)std::min<long long>(VP_TMAX, std::max<long long>(VP_TMIN, (t4 + VP_WG4 - 1) / VP_WG4));
        St.t16 = (int)std::min<long long>(VP_TMAX, std::max<long long>(VP_TMIN, (t16 + VP_WG16 - 1) / VP_WG16));
        St.nsp4 = St.nsp16 = 0;
        for (int x : pc4) St.nsp4 = std::max(St.nsp4, (x + St.t4 - 1) / St.t4);
        for (int x : pc16) St.nsp16 = std::max(St.nsp16, (x + St.t16 - 1) / St.t16);
    }
    uint32_t vsplit = 0;
    if (staged) {
        TRY(stage_and_copy(c, *c->stager, clk, cl, s, paged, packed ? stage_k : nullptr, stage_v,
                           packed ? &vsplit : nullptr));
    } else {
        // K runs first: the FP16-key pass and the INT4 promoted pass need
        // only them and run while the V runs are copied
        TRY(issue_copies(c, clk, false));
        for (int k = 0; k < NSIDE; ++k) {
            HIPCHK(hipEventRecord(c->ev_kside[k], c->side[k]));
            HIPCHK(hipStreamWaitEvent(s, c->ev_kside[k], 0));
        }
        if (gather) {
            // the FP16-key pass also waits for the K gather; the end of the
            // paging (below) for the V gather
            HIPCHK(hipStreamWaitEvent(s, c->ev_gk, 0));
            HIPCHK(hipStreamWaitEvent(c->side[0], c->ev_gv, 0));
        }
        TRY(issue_copies(c, cl));
        paged += cl.bytes + clk.bytes;
        if (prof) c->pf.copies += cl.size.size() + clk.size.size();
    }
    if (prof) HIPCHK(hipEventRecord(E[6], c->side[0]));
    HIPCHK(hipEventRecord(c->ev_paged, c->side[0]));
    // K4: promoted blocks, rank check, merge
    kev(KEV_KEYS);
    HIPCHK(launch_keys16(Ly, St, c->dskip, s));
    // the rank check needs only the FP16-key pass: it runs while the FP16
    // values are still being paged, and sets the promoted passes' softmax
    // reference
    kev(KEV_RANK);
    HIPCHK(launch_merge_impl(Ly, St, T, c->dskip, c->plist, c->keys, 1, s));
    // the plans (the rank check's verdicts) to the host now: the fallback
    // below pages its blocks while the promoted passes and the merge run
    HIPCHK(hipEventRecord(c->ev_rank, s));
    HIPCHK(hipStreamWaitEvent(c->pstream, c->ev_rank, 0));
    HIPCHK(hipMemcpyAsync(c->h_plan, c->plan, sizeof(HeadPlan) * batch * Hq, hipMemcpyDeviceToHost, c->pstream));
    HIPCHK(hipEventRecord(c->ev_plan, c->pstream));
    kev(KEV_PROMO4);
    HIPCHK(launch_promoted4(Ly, St, c->dskip, s));
    // the FP16 value pass: with packed staging, first the pairs (in listing
    // order, a prefix of n * Hkv + g) whose V slots were all issued by the
    // second-to-last chunk, as soon as it has landed; the rest after the
    // paging (only the last chunk's pairs wait for it)
    int p16_split = 0;
    if (vsplit > 0) {
        p16_split = batch * Hkv;
        for (int pr = 0; pr < batch * Hkv; ++pr)
            if (!c->h_skip[pr / Hkv] && vend[pr] > vsplit) {
                p16_split = pr;
                break;
            }
    }
    if (p16_split > 0) {
        for (int k = 0; k < NSIDE; ++k) HIPCHK(hipStreamWaitEvent(s, c->ev_vsplit[k], 0));
        St.p16_lo = 0;
        St.p16_hi = p16_split;
        kev(KEV_PROMO16);
        HIPCHK(launch_promoted16(Ly, St, c->dskip, s));
    }
    HIPCHK(hipStreamWaitEvent(s, c->ev_paged, 0));
    if (p16_split < batch * Hkv) {
        St.p16_lo = p16_split;
        St.p16_hi = INT_MAX;
        kev(p16_split > 0 ? KEV_PROMO16B : KEV_PROMO16);
        HIPCHK(launch_promoted16(Ly, St, c->dskip, s));
    }
    kev(KEV_MERGE);
    HIPCHK(launch_merge_impl(Ly, St, T, c->dskip, c->plist, c->keys, 2, s));
    St.clk = nullptr;
    HIPCHK(hipEventSynchronize(c->ev_plan));

    // rungs 3 and 4 [Meth-3]: per-head dense on an inconsistent ranking;
    // the whole layer (per sequence) when more than f_layer of the heads
    // fell back, or when a cap was exhausted before paging.  The missing
    // blocks of the groups concerned are paged behind the step's own (the
    // link stays busy) and the dense pass runs after the merge, whose
    // outputs it replaces for those heads.
    std::vector<int> dense((size_t)batch * Hq, 0), r4post(batch, 0);
    bool any_dense = false;
    for (int n = 0; n < batch; ++n) {
        int n3 = 0;
        for (int h = 0; h < Hq; ++h) n3 += !c->h_skip[n] && c->h_plan[(size_t)n * Hq + h].rank_ok == 0;
        r4post[n] = !c->h_skip[n] && ((double)n3 > (double)th->f_layer * (double)Hq);
        for (int h = 0; h < Hq; ++h) {
            const HeadPlan &P = c->h_plan[(size_t)n * Hq + h];
            dense[(size_t)n * Hq + h] = c->h_skip[n] || r4post[n] || P.rank_ok == 0;
            any_dense |= dense[(size_t)n * Hq + h] != 0;
        }
    }
    if (any_dense) {
        // timed from where the step's own paging ends on side[0]
        if (prof) HIPCHK(hipEventRecord(E[9], c->side[0]));
        std::vector<uint8_t> all(Ly.Nmax, 1);
        cl.clear();
        CopyList clv;  // V runs (staged paging)
        for (int n = 0; n < batch; ++n) {
            const int N = c->len[(size_t)layer * cf.max_batch + n] / 64;
            for (int g = 0; g < Hkv; ++g) {
                uint32_t m = 0;
                for (int j = 0; j < G; ++j) m |= (uint32_t)dense[(size_t)n * Hq + g * G + j] << j;
                c->h_mask[n * Hkv + g] = m;
                if (m && staged) {
                    // the blocks between those already staged: packed
                    Stager &SG = *c->stager;
                    ones_mask(vmask.data(), N);
                    list_blocks(c, layer, n, g, N, vmask.data(), staged_k, c->t2k, stage_k, SG.src, SG.dst, cl,
                                packed ? &slots.k : nullptr, c->h_kmap, needw.data());
                    list_blocks(c, layer, n, g, N, vmask.data(), staged_v, c->t2v, stage_v, SG.vsrc, SG.vdst, clv,
                                packed ? &slots.v : nullptr, c->h_vmap, needw.data());
                } else if (m) {
                    page_runs(c, layer, n, g, N, all.data(), staged_k, c->t2k, stage_k, cl);
                    page_runs(c, layer, n, g, N, all.data(), staged_v, c->t2v, stage_v, cl);
                }
                if (m && prof) c->pf.dense_blocks += N;
            }
        }
        if (gather) {
            // the device's gathers write the staging area too: these copies
            // (of the same blocks or others) start after them
            for (int k = 0; k < NSIDE; ++k) HIPCHK(hipStreamWaitEvent(c->side[k], c->ev_gv, 0));
        }
        if (staged) {
            TRY(stage_and_copy(c, *c->stager, cl, clv, s, paged, packed ? stage_k : nullptr, stage_v));
            if (packed) {
                // where the dense pass finds each block of its pairs
                const size_t mb = (size_t)batch * Hkv * Ly.Nmax * sizeof(uint32_t);
                HIPCHK(hipMemcpyAsync(c->kmap, c->h_kmap, mb, hipMemcpyHostToDevice, c->side[0]));
                HIPCHK(hipMemcpyAsync(c->vmap, c->h_vmap, mb, hipMemcpyHostToDevice, c->side[0]));
            }
        } else {
            TRY(issue_copies(c, cl));
            paged += cl.bytes;
            if (prof) c->pf.copies += cl.size.size();
        }
        HIPCHK(hipMemcpyAsync(c->dmask, c->h_mask, sizeof(uint32_t) * batch * Hkv, hipMemcpyHostToDevice,
                              c->side[0]));
        HIPCHK(hipEventRecord(c->ev_paged, c->side[0]));
        HIPCHK(hipStreamWaitEvent(s, c->ev_paged, 0));
        DenseSrc S{};
        S.k = stage_k;
        S.v = stage_v;
        S.kmap = packed ? c->kmap : nullptr;
        S.vmap = packed ? c->vmap : nullptr;
        S.kp = Ly.kpart + Ly.seqg(layer, 0, 0) * c->blk_fp16;
        S.vp = Ly.vpart + Ly.seqg(layer, 0, 0) * c->blk_fp16;
        S.len = Ly.len + (size_t)layer * cf.max_batch;
        S.nstride = Ly.Nmax;
        S.mask = c->dmask;
        S.q = (const uint16_t *)q;
        S.sm = th->sm_scale;
        S.part = c->part_tail;
        S.nsplit_cap = c->nsplit_cap;
        S.bps = St.bps;
        S.Hq = Hq;
        S.Hkv = Hkv;
        S.out = out;
        const int nsl = nb + np_any;
        HIPCHK(launch_dense_src(d, G, S, (nsl + S.bps - 1) / S.bps, batch, s));
        if (prof) HIPCHK(hipEventRecord(E[10], s));
    }
    if (prof) {
        HIPCHK(launch_clock_fold(c->dclk, c->dclkf, KEV_N, s));
        HIPCHK(hipMemcpyAsync(c->h_clkf, c->dclkf, sizeof(unsigned long long) * 2 * KEV_N, hipMemcpyDeviceToHost,
                              s));
    }
    HIPCHK(hipEventRecord(c->ev_done, s));
    HIPCHK(hipEventSynchronize(c->ev_done));

    // report [Meth-2 bounds per head and step; Meth-3 ladder]
    for (int n = 0; n < batch; ++n)
        for (int h = 0; h < Hq; ++h) {
            const size_t i = (size_t)n * Hq + h;
            const HeadPlan &P = c->h_plan[i];
            ckv_head_report &R = report[i];
            int mask = 0;
            if (P.flags & 1) mask |= 2;
            if (P.nvp > 0) mask |= 4;
            const bool r3 = !c->h_skip[n] && P.rank_ok == 0;
            if (r3) mask |= 8;
            if (c->h_skip[n] || r4post[n]) mask |= 16;
            int rmax = 0;
            for (int r = 1; r <= 4; ++r)
                if (mask & (1 << r)) rmax = r;
            R.kstar = P.kstar;
            R.n_v_promoted = P.nvp;
            R.tau_final = (float)P.tau;
            R.rank_ok = c->h_skip[n] ? -1 : P.rank_ok;
            R.n_discordant = c->h_skip[n] ? 0 : P.ndisc;
            R.rung_mask = mask;
            R.rung_max = rmax;
            if (dense[i]) {
                R.e_key = R.e_val = R.tv_bound = 0.0f;
            } else {
                R.e_key = ru32h(P.ekey);
                R.e_val = ru32h(P.eval);
                R.tv_bound = ru32h(P.tv);
            }
        }
    c->seq_flags.assign(batch, 0);
    for (int n = 0; n < batch; ++n) c->seq_flags[n] = c->h_skip[n] | (r4post[n] << 1);
    c->have_step = true;
    c->last_batch = batch;
    c->last_nb = nb;
    c->last_np = nb + np_any;
    if (prof) {
        c->pf.bytes_paged += paged;
        c->pf.steps += 1;
        float t;
        auto acc = [&](int ph, int a, int b) -> ckv_status {
            HIPCHK(hipEventElapsedTime(&t, E[a], E[b]));
            c->pf.ms[ph] += t;
            c->pf.counts[ph] += 1;
            return CKV_OK;
        };
        // kernel phases: each kernel's own execution span, first wave's
        // start to last wave's end (the tail, FP16-key and INT4 promoted
        // passes launch only when the batch has a full block)
        auto kacc = [&](int ph, int k) -> ckv_status {
            const unsigned long long t0 = c->h_clkf[2 * k], t1 = c->h_clkf[2 * k + 1];
            if (t0 == ~0ull && t1 == 0) return CKV_OK;  // not launched this step (nothing to do)
            if (t0 == ~0ull || t1 < t0 || !(c->clk_khz > 0.0))
                return fail(CKV_EHIP, "kernel clock of a profiled kernel stamped incompletely");
            c->pf.ms[ph] += (double)(t1 - t0) / c->clk_khz;
            c->pf.counts[ph] += 1;
            return CKV_OK;
        };
        TRY(kacc(PH_SCORE, KEV_SCORE));
        TRY(kacc(PH_SELECT, KEV_SELECT));
        if (nb > 0) {
            TRY(kacc(PH_TAIL, KEV_TAIL));
            TRY(kacc(PH_KEYS, KEV_KEYS));
            TRY(kacc(PH_PROMO4, KEV_PROMO4));
        }
        TRY(acc(PH_PAGE, 5, 6));
        {
            // one phase per step, one or two launches (their spans added)
            const int before = c->pf.counts[PH_PROMO16];
            TRY(kacc(PH_PROMO16, KEV_PROMO16));
            TRY(kacc(PH_PROMO16, KEV_PROMO16B));
            if (c->pf.counts[PH_PROMO16] - before == 2) c->pf.counts[PH_PROMO16] -= 1;
        }
        TRY(kacc(PH_MERGE, KEV_RANK));
        TRY(kacc(PH_MERGE, KEV_MERGE));
        c->pf.counts[PH_MERGE] -= 1;  // one merge phase per step, two launches
        if (gather) {
            // when the device paging started, after the selection ended
            const unsigned long long sel_end = c->h_clkf[2 * KEV_SELECT + 1], g0 = c->h_clkf[2 * KEV_GATHER];
            if (g0 != ~0ull && sel_end != 0) {
                c->pf.gather_lead_ms += ((double)g0 - (double)sel_end) / c->clk_khz;
                c->pf.gather_steps += 1;
            }
        }
        if (any_dense) TRY(acc(PH_FALLBACK, 9, 10));
        c->pf.ms[PH_STEP] += std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t_start).count();
        c->pf.counts[PH_STEP] += 1;
    }
    return CKV_OK;
}

}  // namespace

ckv_status ckv_certified_decode_attention(ckv_cache *c, int layer, const void *q, int batch,
                                          const ckv_thresholds *th, float *out,
                                          ckv_head_report *report, void *stream) {
    const ckv_status st = certified_step(c, layer, q, batch, th, out, report, stream);
    if (st != CKV_OK && c && layer >= 0 && layer < c->cfg.n_layers) {
        // paging already issued by the failed step (copies, gathers) ends
        // before the next step reuses the staging area
        for (hipStream_t ps : c->side)
            if (ps) (void)hipStreamSynchronize(ps);
        if (c->gstream) (void)hipStreamSynchronize(c->gstream);
        if (c->pstream) (void)hipStreamSynchronize(c->pstream);
        if (c->prof) {
            // the step's kernels may have stamped the clock slots without
            // the fold that re-arms them
            (void)hipStreamSynchronize((hipStream_t)stream);
            (void)hipMemcpy(c->dclk, c->h_clk_init, sizeof(unsigned long long) * KEV_N * CLK_WORDS,
                            hipMemcpyHostToDevice);
        }
        // blocks listed for paging are marked staged before their copies
        // are issued; after a failed step none of them can be trusted, so
        // the layer's next step pages them again
        std::fill(c->staged_k.begin(), c->staged_k.end(), 0);
        std::fill(c->staged_v.begin(), c->staged_v.end(), 0);
        if (layer < c->pcache_layers) {
            std::fill(c->pstaged_k[layer].begin(), c->pstaged_k[layer].end(), 0);
            std::fill(c->pstaged_v[layer].begin(), c->pstaged_v[layer].end(), 0);
        }
    }
    return st;
}

ckv_status ckv_inject_paging_fault(ckv_cache *c, int after_copies) {
    if (!c) return fail(CKV_EINVAL, "null cache");
    c->fault_after = after_copies < 0 ? -1 : after_copies;
    return CKV_OK;
}

ckv_status ckv_dense_decode_attention(ckv_cache *c, const void *k, const void *v, int ntok,
                                      const void *q, int batch, float sm, float *out, void *stream) {
    if (!c || !k || !v || !q || !out) return fail(CKV_EINVAL, "null argument");
    const ckv_config &cf = c->cfg;
    if (batch < 1 || batch > cf.max_batch || ntok < 64 || ntok % 64 || ntok > c->Nmax * 64 || !(sm > 0))
        return fail(CKV_EINVAL, "bad batch, token count (multiple of 64) or scale");
    HIPCHK(hipSetDevice(cf.device));
    hipStream_t s = (hipStream_t)stream;
    DenseSrc S{};
    S.k = (const uint16_t *)k;
    S.v = (const uint16_t *)v;
    S.kp = S.vp = nullptr;
    S.len = nullptr;  // every sequence holds ntok tokens
    S.len_all = ntok;
    S.nstride = (size_t)ntok / 64;
    S.mask = nullptr;
    S.q = (const uint16_t *)q;
    S.sm = sm;
    S.part = c->part_tail;
    S.nsplit_cap = c->nsplit_cap;
    const int nb = ntok / 64;
    S.bps = split_blocks(nb, cf.n_kv_heads, batch);
    S.Hq = cf.n_q_heads;
    S.Hkv = cf.n_kv_heads;
    S.out = out;
    HIPCHK(launch_dense_src(c->d, c->G, S, (nb + S.bps - 1) / S.bps, batch, s));
    return CKV_OK;
}

ckv_status ckv_export_block(ckv_cache *c, int layer, int seq, int g, int b, uint8_t *k_code,
                            uint16_t *k_s, uint16_t *k_z, uint8_t *v_code, uint16_t *v_s,
                            uint16_t *v_z, float *eta) {
    if (!c) return fail(CKV_EINVAL, "null cache");
    const ckv_config &cf = c->cfg;
    if (layer < 0 || layer >= cf.n_layers || seq < 0 || seq >= cf.max_batch || g < 0 ||
        g >= cf.n_kv_heads || b < 0 || (long)(b + 1) * 64 > c->len[(size_t)layer * cf.max_batch + seq])
        return fail(CKV_EINVAL, "block not complete or out of range");
    HIPCHK(hipSetDevice(cf.device));
    const Layout &Ly = c->Ly;
    const int d = c->d;
    const size_t bi = Ly.blk(layer, seq, g, b);
    if (k_code) {
        std::vector<uint8_t> raw((size_t)64 * d);
        HIPCHK(hipMemcpy(raw.data(), Ly.kq + bi * 64 * d, raw.size(), hipMemcpyDeviceToHost));
        for (int t = 0; t < 64; ++t)
            for (int ch = 0; ch < d; ++ch) k_code[t * d + ch] = raw[(ch / 16) * 1024 + t * 16 + ch % 16] ^ 0x80;
    }
    if (k_s || k_z) {
        std::vector<uint32_t> m(d);
        HIPCHK(hipMemcpy(m.data(), Ly.kmeta + bi * d, d * 4, hipMemcpyDeviceToHost));
        for (int ch = 0; ch < d; ++ch) {
            if (k_s) k_s[ch] = (uint16_t)(m[ch] & 0xFFFFu);
            if (k_z) k_z[ch] = (uint16_t)(m[ch] >> 16);
        }
    }
    if (v_code && Ly.vb == 8) {
        // stored channel-major (byte c * 64 + t)
        std::vector<uint8_t> raw((size_t)64 * d);
        HIPCHK(hipMemcpy(raw.data(), Ly.vq + bi * 64 * d, raw.size(), hipMemcpyDeviceToHost));
        for (int t = 0; t < 64; ++t)
            for (int ch = 0; ch < d; ++ch) v_code[t * d + ch] = raw[ch * 64 + t];
    } else if (v_code) {
        // stored [d/32][64][16] (see the tier-1 layout): channel c, token t
        // at byte (c/32)*1024 + ((t/16)*16 + c%16)*16 + ((c/16)%2)*8 +
        // (t%16)/2, low nibble = even t
        std::vector<uint8_t> raw((size_t)64 * (d / 2));
        HIPCHK(hipMemcpy(raw.data(), Ly.vq + bi * 64 * (d / 2), raw.size(), hipMemcpyDeviceToHost));
        auto code = [&](int ch, int t) {
            const size_t at = (size_t)(ch / 32) * 1024 + (size_t)((t / 16) * 16 + ch % 16) * 16 +
                              (size_t)((ch / 16) % 2) * 8 + (size_t)((t % 16) / 2);
            return (raw[at] >> (4 * (t & 1))) & 15;
        };
        for (int t = 0; t < 64; ++t)
            for (int ch = 0; ch < d; ch += 2)
                v_code[t * (d / 2) + ch / 2] = (uint8_t)(code(ch, t) | (code(ch + 1, t) << 4));
    }
    if (v_s || v_z) {
        // stored group-major [d/32][64]
        const int ng = d / 32;
        std::vector<uint32_t> m((size_t)64 * ng);
        HIPCHK(hipMemcpy(m.data(), Ly.vmeta + bi * 64 * ng, m.size() * 4, hipMemcpyDeviceToHost));
        for (int t = 0; t < 64; ++t)
            for (int gr = 0; gr < ng; ++gr) {
                const uint32_t w = m[(size_t)gr * 64 + t];
                if (v_s) v_s[t * ng + gr] = (uint16_t)(w & 0xFFFFu);
                if (v_z) v_z[t * ng + gr] = (uint16_t)(w >> 16);
            }
    }
    if (eta) HIPCHK(hipMemcpy(eta, Ly.eta + bi, 4, hipMemcpyDeviceToHost));
    return CKV_OK;
}

ckv_status ckv_export_step(ckv_cache *c, int batch, int *np_out, float *score, float *bstat,
                           float *mref, uint64_t *mfx, uint32_t *sel, uint64_t *m16fx, double *bounds,
                           int *seq_flags) {
    if (!c) return fail(CKV_EINVAL, "null cache");
    if (!c->have_step) return fail(CKV_ESTATE, "no decode step yet");
    if (batch < 1 || batch > c->last_batch) return fail(CKV_EINVAL, "bad batch");
    HIPCHK(hipSetDevice(c->cfg.device));
    const int Hq = c->cfg.n_q_heads, Hkv = c->cfg.n_kv_heads, NS = c->NS, Np = c->last_np,
              N = c->last_nb, Nmax = c->Nmax;
    if (np_out) *np_out = Np;
    for (int n = 0; n < batch; ++n)
        for (int h = 0; h < Hq; ++h) {
            const size_t hs = (size_t)n * Hq + h, ho = hs;
            if (score)
                HIPCHK(hipMemcpy(score + ho * Np * 64, c->score + hs * NS * 64, (size_t)Np * 64 * 4,
                                 hipMemcpyDeviceToHost));
            if (bstat)
                HIPCHK(hipMemcpy(bstat + ho * Np * 4, c->bstat + hs * NS, (size_t)Np * 16, hipMemcpyDeviceToHost));
            if (mfx)
                HIPCHK(hipMemcpy(mfx + ho * Np, c->mfx + hs * NS, (size_t)Np * 8, hipMemcpyDeviceToHost));
            if (m16fx && N)
                HIPCHK(hipMemcpy(m16fx + ho * Np, c->m16 + hs * Nmax, (size_t)N * 8, hipMemcpyDeviceToHost));
        }
    if (sel && N)
        for (int n = 0; n < batch; ++n)
            for (int g = 0; g < Hkv; ++g)
                HIPCHK(hipMemcpy(sel + ((size_t)n * Hkv + g) * Np, c->sel + ((size_t)n * Hkv + g) * Nmax,
                                 (size_t)N * 4, hipMemcpyDeviceToHost));
    if (mref || bounds) {
        std::vector<HeadPlan> P((size_t)batch * Hq);
        HIPCHK(hipMemcpy(P.data(), c->plan, sizeof(HeadPlan) * P.size(), hipMemcpyDeviceToHost));
        for (size_t i = 0; i < P.size(); ++i) {
            if (mref) mref[i] = P[i].mref;
            if (bounds) {
                bounds[i * 4 + 0] = P[i].mu;
                bounds[i * 4 + 1] = P[i].tv;
                bounds[i * 4 + 2] = P[i].ekey;
                bounds[i * 4 + 3] = P[i].eval;
            }
        }
    }
    if (seq_flags)
        for (int n = 0; n < batch; ++n) seq_flags[n] = c->seq_flags[n];
    return CKV_OK;
}

ckv_status ckv_set_profiling(ckv_cache *c, int enable) {
    if (!c) return fail(CKV_EINVAL, "null cache");
    if (enable) {
        // the clock slots armed (a failed step may have left stamps)
        HIPCHK(hipSetDevice(c->cfg.device));
        HIPCHK(hipMemcpy(c->dclk, c->h_clk_init, sizeof(unsigned long long) * KEV_N * CLK_WORDS,
                         hipMemcpyHostToDevice));
    }
    c->prof = enable != 0;
    c->pf = ckv_profile{};
    return CKV_OK;
}

ckv_status ckv_get_profile(const ckv_cache *c, ckv_profile *p) {
    if (!c || !p) return fail(CKV_EINVAL, "null argument");
    *p = c->pf;
    p->staged_threads = c->stager ? c->stager->nthreads : 0;
    return CKV_OK;
}

}  // extern "C"
