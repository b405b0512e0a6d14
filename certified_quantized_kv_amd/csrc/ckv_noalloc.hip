// ckv_noalloc.hip -- exact dense decode attention that allocates nothing.
//
// The same computation as ckv_dense_decode_attention (the split-K dense pass
// k_dense and its merge k_merge_dense), for callers that cannot allocate
// device memory: code under HIP graph capture, serving loops and harnesses
// that forbid hipMalloc.  Instead of a cache's scratch, the split partials
// (m, l, acc[d]) per (sequence, q head, split) live in `scratch`, a static
// device array of NOALLOC_SCRATCH_BYTES that every GPU the library runs on
// holds until the process ends.  Each call writes every partial it reads, so
// nothing has to start at zero; calls that overlap on one GPU (two streams,
// two threads) share the array and race.
#include <mutex>

#include "../../include/ckv.h"
#include "ckv_internal.hpp"

namespace ckv {

constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)4 << 20;
constexpr int NOALLOC_MAX_DEVICES = 64;

static __device__ __align__(256) float scratch[NOALLOC_SCRATCH_BYTES / sizeof(float)];

// Device address of `scratch` on each device (taken once per device with the
// device current; the array's name in host code is not a device address).
static std::mutex g_scratch_mutex;
static float *g_scratch[NOALLOC_MAX_DEVICES] = {};

static hipError_t scratch_on(int dev, float **p) {
    std::lock_guard<std::mutex> lk(g_scratch_mutex);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = static_cast<float *>(ptr);
    }
    *p = g_scratch[dev];
    return hipSuccess;
}

}  // namespace ckv

using namespace ckv;

extern "C" ckv_status ckv_dense_decode_attention_noalloc(const void *k, const void *v, int n_tokens,
                                                         const void *q_fp16, int batch, int n_q_heads,
                                                         int n_kv_heads, int head_dim, float sm_scale,
                                                         float *out, void *stream) {
    if (!k || !v || !q_fp16 || !out) return (ckv_status)set_error(CKV_EINVAL, "null argument");
    if (batch < 1 || n_kv_heads < 1 || n_q_heads < n_kv_heads || n_q_heads % n_kv_heads ||
        (head_dim != 64 && head_dim != 128))
        return (ckv_status)set_error(CKV_EINVAL, "bad batch or head shape");
    const int G = n_q_heads / n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return (ckv_status)set_error(CKV_EINVAL, "n_q_heads / n_kv_heads must be 1, 2, 4 or 8");
    if (n_tokens < 64 || n_tokens % 64 || !(sm_scale > 0.0f))
        return (ckv_status)set_error(CKV_EINVAL, "bad token count (a multiple of 64) or scale");
    // the partials of one split for every (sequence, q head) must fit
    const size_t per_split = (size_t)batch * n_q_heads * (head_dim + 2) * sizeof(float);
    const long long max_splits = (long long)(NOALLOC_SCRATCH_BYTES / per_split);
    if (max_splits < 1)
        return (ckv_status)set_error(CKV_EINVAL,
                                     "batch x n_q_heads too large for the 4 MiB scratch of the "
                                     "allocation-free dense pass");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess && (dev < 0 || dev >= NOALLOC_MAX_DEVICES)) e = hipErrorInvalidDevice;
    float *part = nullptr;
    if (e == hipSuccess) e = scratch_on(dev, &part);
    if (e != hipSuccess) return (ckv_status)set_error(CKV_EHIP, hipGetErrorString(e));
    // splits as the cached entry point takes them, fewer when the scratch
    // would not hold them (longer splits: the result differs only in the
    // rounding of the merge)
    const int nb = n_tokens / 64;
    int bps = split_blocks(nb, n_kv_heads, batch);
    if ((nb + bps - 1) / bps > max_splits) bps = (int)((nb + max_splits - 1) / max_splits);
    const int nsplit = (nb + bps - 1) / bps;
    DenseSrc S{};
    S.k = static_cast<const uint16_t *>(k);
    S.v = static_cast<const uint16_t *>(v);
    S.kp = S.vp = nullptr;
    S.len = nullptr;
    S.len_all = n_tokens;
    S.nstride = (size_t)nb;
    S.mask = nullptr;
    S.q = static_cast<const uint16_t *>(q_fp16);
    S.sm = sm_scale;
    S.part = part;
    S.nsplit_cap = nsplit;
    S.bps = bps;
    S.Hq = n_q_heads;
    S.Hkv = n_kv_heads;
    S.out = out;
    e = launch_dense_src(head_dim, G, S, nsplit, batch, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return (ckv_status)set_error(CKV_EHIP, hipGetErrorString(e));
    return CKV_OK;
}
