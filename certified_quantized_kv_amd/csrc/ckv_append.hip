// ckv_append.hip -- tier-1 construction [Meth-1 of the page "Runtime-
// Certified Bounded-Error Quantized Attention": INT8 per-channel keys, INT4
// per-group values, scales/offsets and per-block error annotations].
//
// Readings (where the page is silent): the key scale/offset is per channel
// per 64-token block; the value scale/offset per token per 32-channel group;
// both affine with offset = the exact FP16 minimum and scale = range /
// levels rounded up to FP16, so no code is clamped; eta_b = the largest
// absolute value-reconstruction error of the block, exact in FP64, rounded
// up to FP32.
#include "ckv_device.hpp"
#include "ckv_internal.hpp"

namespace ckv {

// Pack tokens [len0, len0 + ntok) of (l, n), plus the unfinished block's
// earlier tokens, into whole FP16 blocks b0 .. b0 + nblk - 1 in the tier-2
// layout.  kin / vin: [ntok][Hkv][d].  Slots past the last token are 0.
__global__ __launch_bounds__(256) void k_pack(Layout Ly, int l, int n, const uint16_t *kin,
                                              const uint16_t *vin, int len0, int ntok, int b0,
                                              int nblk, uint16_t *pk, uint16_t *pv) {
    const int bi = blockIdx.x, g = blockIdx.y, d = Ly.d;
    const size_t sg = Ly.seqg(l, n, g);
    const uint16_t *kp = Ly.kpart + sg * 64 * d;
    const uint16_t *vp = Ly.vpart + sg * 64 * d;
    uint16_t *ok = pk + ((size_t)g * nblk + bi) * 64 * d;
    uint16_t *ov = pv + ((size_t)g * nblk + bi) * 64 * d;
    for (int e = threadIdx.x; e < 64 * d; e += blockDim.x) {
        const int t = e / d, c = e % d;
        const long i = (long)(b0 + bi) * 64 + t;
        uint16_t kv = 0, vv = 0;
        if (i < len0) {
            kv = kp[(c / 8) * 512 + t * 8 + (c % 8)];
            vv = vp[c * 64 + t];
        } else if (i < (long)len0 + ntok) {
            const size_t src = ((size_t)(i - len0) * Ly.Hkv + g) * d + c;
            kv = kin[src];
            vv = vin[src];
        }
        ok[(c / 8) * 512 + t * 8 + (c % 8)] = kv;
        ov[c * 64 + t] = vv;
    }
}

__device__ __forceinline__ int quant_code(float x, float lo, float s, float maxc) {
    if (s == 0.0f) return 0;
    float c = rintf((x - lo) / s);
    c = c < 0.0f ? 0.0f : c;
    c = c > maxc ? maxc : c;
    return (int)c;
}

// Quantize full packed blocks 0 .. nfull-1 (block b0 + bi of the sequence).
template <int D>
__global__ __launch_bounds__(128) void k_quant(Layout Ly, int l, int n, int b0, int nblk,
                                               const uint16_t *pk, const uint16_t *pv) {
    const int bi = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
    const size_t blk = Ly.blk(l, n, g, b0 + bi);
    const uint16_t *kb = pk + ((size_t)g * nblk + bi) * 64 * D;
    const uint16_t *vb = pv + ((size_t)g * nblk + bi) * 64 * D;
    __shared__ double emax_s[128];

    // keys: one thread per channel
    if (tid < D) {
        const int c = tid;
        const uint16_t *col = kb + (c / 8) * 512 + (c % 8);
        float lo = h2f(col[0]), hi = lo;
        for (int t = 1; t < 64; ++t) {
            float x = h2f(col[t * 8]);
            lo = fminf(lo, x);
            hi = fmaxf(hi, x);
        }
        const float r = hi - lo;
        const uint16_t sb = r == 0.0f ? (uint16_t)0 : f2h_up(r / 255.0f);
        const uint16_t zb = lo == 0.0f ? (uint16_t)0 : __half_as_ushort(__float2half_rn(lo));
        const float sf = h2f(sb);
        Ly.kmeta[blk * D + c] = (uint32_t)sb | ((uint32_t)zb << 16);
        uint8_t *kq = Ly.kq + blk * 64 * D + (c / 16) * 1024 + (c % 16);
        // stored as code - 128 (two's complement byte): the signed operand
        // of the scoring pass's integer matrix product
        for (int t = 0; t < 64; ++t) kq[t * 16] = (uint8_t)(quant_code(h2f(col[t * 8]), lo, sf, 255.0f) ^ 0x80);
    }
    // values: one thread per token; the codes are staged in LDS and stored
    // channel-major, two tokens per byte (INT4) or one (INT8)
    __shared__ uint8_t cq[D][64];
    const float levels = Ly.vb == 8 ? 255.0f : 15.0f;
    double emax = 0.0;
    if (tid < 64) {
        const int t = tid;
        uint32_t *vm = Ly.vmeta + blk * 64 * (D / 32);
        for (int gr = 0; gr < D / 32; ++gr) {
            const uint16_t *col = vb + (size_t)gr * 32 * 64 + t;  // channel gr*32 + c at col[c * 64]
            float lo = h2f(col[0]), hi = lo;
            for (int c = 1; c < 32; ++c) {
                const float x = h2f(col[c * 64]);
                lo = fminf(lo, x);
                hi = fmaxf(hi, x);
            }
            const float r = hi - lo;
            const uint16_t sb = r == 0.0f ? (uint16_t)0 : f2h_up(r / levels);
            const uint16_t zb = lo == 0.0f ? (uint16_t)0 : __half_as_ushort(__float2half_rn(lo));
            const float sf = h2f(sb);
            vm[gr * 64 + t] = (uint32_t)sb | ((uint32_t)zb << 16);
            for (int c = 0; c < 32; ++c) {
                const float x = h2f(col[c * 64]);
                const int q = quant_code(x, lo, sf, levels);
                cq[gr * 32 + c][t] = (uint8_t)q;
                const double rec = (double)lo + (double)sf * (double)q;
                emax = fmax(emax, fabs((double)x - rec));
            }
        }
    }
    emax_s[tid] = emax;
    __syncthreads();
    if (Ly.vb == 8) {
        uint8_t *vq = Ly.vq + blk * 64 * D;
        for (int e = tid; e < D * 64; e += 128) vq[e] = cq[e / 64][e % 64];
    } else {
        // [d/32][64][16]: lane l = 16 tg + i of a channel pair p holds the 8
        // bytes of channel 32 p + i, then of channel 32 p + 16 + i, for
        // tokens 16 tg .. 16 tg + 15 (byte j: tokens 2 j, 2 j + 1)
        uint8_t *vq = Ly.vq + blk * 64 * (D / 2);
        for (int e = tid; e < D * 32; e += 128) {
            const int c = e / 32, j = e % 32;
            const int pr = c >> 5, hf = (c >> 4) & 1, i = c & 15, tg = j >> 3, jj = j & 7;
            vq[pr * 1024 + (tg * 16 + i) * 16 + hf * 8 + jj] = (uint8_t)(cq[c][2 * j] | (cq[c][2 * j + 1] << 4));
        }
    }
    if (tid == 0) {
        double m = 0.0;
        for (int i = 0; i < 64; ++i) m = fmax(m, emax_s[i]);
        Ly.eta[blk] = ru32(m);
    }
}

// Copy packed block `bi` (the unfinished one) into the device FP16 slot.
__global__ __launch_bounds__(256) void k_set_partial(Layout Ly, int l, int n, int bi, int nblk,
                                                     const uint16_t *pk, const uint16_t *pv) {
    const int g = blockIdx.x, d = Ly.d;
    const size_t sg = Ly.seqg(l, n, g);
    const uint16_t *sk = pk + ((size_t)g * nblk + bi) * 64 * d;
    const uint16_t *sv = pv + ((size_t)g * nblk + bi) * 64 * d;
    for (int e = threadIdx.x; e < 64 * d; e += blockDim.x) {
        Ly.kpart[sg * 64 * d + e] = sk[e];
        Ly.vpart[sg * 64 * d + e] = sv[e];
    }
}

__global__ void k_vrange_init(Layout Ly, int l, int n) {
    const int g = blockIdx.x, c = threadIdx.x;
    if (c < Ly.d) {
        Ly.vmin[Ly.seqg(l, n, g) * Ly.d + c] = 0xFFFFFFFFu;
        Ly.vmax[Ly.seqg(l, n, g) * Ly.d + c] = 0u;
    }
}

// Running per-channel min / max of V ("value ranges" of [Meth-2]).
__global__ __launch_bounds__(128) void k_vrange(Layout Ly, int l, int n, const uint16_t *vin,
                                                int ntok, int chunk) {
    const int g = blockIdx.x, c = threadIdx.x, d = Ly.d;
    if (c >= d) return;
    const int t0 = blockIdx.y * chunk, t1 = min(ntok, t0 + chunk);
    if (t0 >= t1) return;
    float lo = h2f(vin[((size_t)t0 * Ly.Hkv + g) * d + c]), hi = lo;
    for (int t = t0 + 1; t < t1; ++t) {
        const float x = h2f(vin[((size_t)t * Ly.Hkv + g) * d + c]);
        lo = fminf(lo, x);
        hi = fmaxf(hi, x);
    }
    atomicMin(&Ly.vmin[Ly.seqg(l, n, g) * d + c], f2ord(lo));
    atomicMax(&Ly.vmax[Ly.seqg(l, n, g) * d + c], f2ord(hi));
}

// K of a value group from its range R (largest max minus smallest min over
// the group's channels): the smallest power of two P >= R / lv (1 + 2^-8)
// bounds every scale of the group (lv = 15 levels for INT4, 255 for INT8;
// scale = range / lv rounded up to FP16, so scale <= R / lv (1 + 2^-10)
// (1 + 2^-23)), and K = 2^14 / P, kept in [1, 2^15].  The value passes
// weight the codes by p s K and FP16 values by p K, both below 2^15, before
// splitting the weights into FP16 parts.
__device__ __forceinline__ float value_scale(double R, double lv) {
    const double x = R / lv * (1.0 + 0x1p-8);
    if (!(x > 0.0)) return 0x1p15f;
    int e;
    (void)frexp(x, &e);  // x < 2^e
    const int k = min(15, max(0, 14 - e));
    return ldexpf(1.0f, k);
}

// One thread per (kv head, value group) of (l, n), after the range update.
__global__ void k_vscale(Layout Ly, int l, int n) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x, ng = Ly.d / 32;
    if (t >= Ly.Hkv * ng) return;
    const int g = t / ng, gr = t % ng;
    const size_t base = Ly.seqg(l, n, g) * Ly.d + gr * 32;
    float lo = INFINITY, hi = -INFINITY;
    for (int c = 0; c < 32; ++c) {
        lo = fminf(lo, ord2f(Ly.vmin[base + c]));
        hi = fmaxf(hi, ord2f(Ly.vmax[base + c]));
    }
    Ly.vscale[Ly.seqg(l, n, g) * ng + gr] = value_scale((double)hi - (double)lo, Ly.vb == 8 ? 255.0 : 15.0);
}

// One decode token for each sequence n < batch of layer l (kin, vin:
// [batch][Hkv][d]): written into the unfinished block's device copy at
// position len % 64, the running value range updated (set, for a sequence's
// first token) and the weight scales of the value groups recomputed; the
// same state as an append of that token alone.  One workgroup per (kv head,
// sequence), a thread per channel; len is read before the host updates it.
__global__ __launch_bounds__(128) void k_append_token(Layout Ly, int l, const uint16_t *kin, const uint16_t *vin) {
    const int g = blockIdx.x, n = blockIdx.y, c = threadIdx.x, d = Ly.d;
    const int len = Ly.len[l * Ly.B + n];
    const int t = len % 64;
    const size_t sg = Ly.seqg(l, n, g);
    __shared__ float lo_s[128], hi_s[128];
    if (c < d) {
        const size_t src = ((size_t)n * Ly.Hkv + g) * d + c;
        const uint16_t kv = kin[src], vv = vin[src];
        uint16_t *kp = Ly.kpart + sg * 64 * d, *vp = Ly.vpart + sg * 64 * d;
        if (t == 0)  // a new block: the slots past the token hold 0 (as after a pack)
            for (int u = 1; u < 64; ++u) {
                kp[(c / 8) * 512 + u * 8 + (c % 8)] = 0;
                vp[c * 64 + u] = 0;
            }
        kp[(c / 8) * 512 + t * 8 + (c % 8)] = kv;
        vp[c * 64 + t] = vv;
        // this workgroup alone touches the range of (l, n, g)
        const uint32_t o = f2ord(h2f(vv));
        uint32_t *mn = &Ly.vmin[sg * d + c], *mx = &Ly.vmax[sg * d + c];
        const uint32_t nmn = len == 0 ? o : min(*mn, o), nmx = len == 0 ? o : max(*mx, o);
        *mn = nmn;
        *mx = nmx;
        lo_s[c] = ord2f(nmn);
        hi_s[c] = ord2f(nmx);
    }
    __syncthreads();
    if (c < d / 32) {
        float lo = INFINITY, hi = -INFINITY;
        for (int i = 0; i < 32; ++i) {
            lo = fminf(lo, lo_s[c * 32 + i]);
            hi = fmaxf(hi, hi_s[c * 32 + i]);
        }
        Ly.vscale[sg * (d / 32) + c] = value_scale((double)hi - (double)lo, Ly.vb == 8 ? 255.0 : 15.0);
    }
}

hipError_t launch_append_token(const Layout &Ly, int l, int batch, const uint16_t *kin, const uint16_t *vin,
                               hipStream_t s) {
    hipLaunchKernelGGL(k_append_token, dim3(Ly.Hkv, batch), dim3(128), 0, s, Ly, l, kin, vin);
    return hipGetLastError();
}

hipError_t launch_pack(const Layout &Ly, int l, int n, const uint16_t *kin, const uint16_t *vin,
                       int len0, int ntok, int b0, int nblk, uint16_t *pk, uint16_t *pv,
                       hipStream_t s) {
    hipLaunchKernelGGL(k_pack, dim3(nblk, Ly.Hkv), dim3(256), 0, s, Ly, l, n, kin, vin, len0, ntok,
                       b0, nblk, pk, pv);
    return hipGetLastError();
}

hipError_t launch_quant(const Layout &Ly, int l, int n, int b0, int nfull, int nblk,
                        const uint16_t *pk, const uint16_t *pv, hipStream_t s) {
    if (nfull <= 0) return hipSuccess;
    if (Ly.d == 64)
        hipLaunchKernelGGL(k_quant<64>, dim3(nfull, Ly.Hkv), dim3(128), 0, s, Ly, l, n, b0, nblk, pk, pv);
    else
        hipLaunchKernelGGL(k_quant<128>, dim3(nfull, Ly.Hkv), dim3(128), 0, s, Ly, l, n, b0, nblk, pk, pv);
    return hipGetLastError();
}

hipError_t launch_set_partial(const Layout &Ly, int l, int n, int slot, int nblk,
                              const uint16_t *pk, const uint16_t *pv, hipStream_t s) {
    hipLaunchKernelGGL(k_set_partial, dim3(Ly.Hkv), dim3(256), 0, s, Ly, l, n, slot, nblk, pk, pv);
    return hipGetLastError();
}

hipError_t launch_vrange(const Layout &Ly, int l, int n, const uint16_t *vin, int ntok, int reset,
                         hipStream_t s) {
    if (reset) hipLaunchKernelGGL(k_vrange_init, dim3(Ly.Hkv), dim3(128), 0, s, Ly, l, n);
    const int chunk = 256;
    const int nch = (ntok + chunk - 1) / chunk;
    hipLaunchKernelGGL(k_vrange, dim3(Ly.Hkv, nch), dim3(128), 0, s, Ly, l, n, vin, ntok, chunk);
    hipLaunchKernelGGL(k_vscale, dim3((Ly.Hkv * (Ly.d / 32) + 255) / 256), dim3(256), 0, s, Ly, l, n);
    return hipGetLastError();
}

// Staged paging: a chunk is a header of destination addresses (one 64-bit
// device address per block, PAGE_HDR bytes) followed by the blocks packed
// back to back; workgroup i moves block i of the chunk to its staging slot.
__global__ __launch_bounds__(256) void k_page_scatter(const uint8_t *__restrict__ chunk, int blk_bytes) {
    const uint64_t dst = reinterpret_cast<const uint64_t *>(chunk)[blockIdx.x];
    const uint4 *src = reinterpret_cast<const uint4 *>(chunk + PAGE_HDR + (size_t)blockIdx.x * blk_bytes);
    uint4 *out = reinterpret_cast<uint4 *>(dst);
    const int n = blk_bytes / 16;
    for (int i = threadIdx.x; i < n; i += 256) out[i] = src[i];
}

hipError_t launch_page_scatter(const uint8_t *chunk, int nblk, int blk_bytes, hipStream_t s) {
    if (nblk <= 0) return hipSuccess;
    if (nblk > PAGE_HDR / 8 || blk_bytes % 16) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_page_scatter, dim3(nblk), dim3(256), 0, s, chunk, blk_bytes);
    return hipGetLastError();
}

// The selection's words and plans to the host: device stores straight into
// mapped, coherent pinned memory, on the stream of the kernel that wrote
// them (the host waits on an event recorded right after this kernel).  One
// 4-byte word per thread per pass over the two buffers.
__global__ __launch_bounds__(256) void k_to_host(const uint32_t *__restrict__ a, uint32_t *ha, size_t na,
                                                 const uint32_t *__restrict__ b, uint32_t *hb, size_t nb) {
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < na + nb; i += stride) {
        if (i < na)
            ha[i] = a[i];
        else
            hb[i - na] = b[i - na];
    }
}

hipError_t launch_to_host(const void *a, void *ha, size_t abytes, const void *b, void *hb, size_t bbytes,
                          hipStream_t s) {
    if (abytes % 4 || bbytes % 4) return hipErrorInvalidValue;
    const size_t na = abytes / 4, nb = bbytes / 4;
    if (na + nb == 0) return hipSuccess;
    const unsigned grid = (unsigned)std::min<size_t>(64, (na + nb + 255) / 256);
    hipLaunchKernelGGL(k_to_host, dim3(grid), dim3(256), 0, s, static_cast<const uint32_t *>(a),
                       static_cast<uint32_t *>(ha), na, static_cast<const uint32_t *>(b),
                       static_cast<uint32_t *>(hb), nb);
    return hipGetLastError();
}

}  // namespace ckv
