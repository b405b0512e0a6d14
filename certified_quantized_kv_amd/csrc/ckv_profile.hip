// ckv_profile.hip -- the kernel clock of profiled decode steps: folding the
// timed kernels' clock slots into one start and one end per kernel; and a
// streaming-read probe that measures what the device's memory delivers to
// loads shaped like the decode passes' (the ceiling their rates are read
// against).
#include "../../include/ckv.h"
#include "ckv_device.hpp"
#include "ckv_internal.hpp"

namespace ckv {

// The execution spans of the timed kernels of a profiled step: wave k
// folds kernel k's start slots (min) and end slots (max) into out[2 k] and
// out[2 k + 1], and sets the slots back (starts to the largest value, ends
// to 0) for the next profiled step.  Each lane reads, then writes, its own
// slot pair only.
static_assert(CLK_SLOTS == 64, "one lane per clock slot");
__global__ __launch_bounds__(64) void k_clock_fold(unsigned long long *clk, unsigned long long *out) {
    const int k = blockIdx.x, lane = threadIdx.x;
    unsigned long long *w = clk + (size_t)k * CLK_WORDS;
    unsigned long long t0 = w[lane * CLK_PAD], t1 = w[(CLK_SLOTS + lane) * CLK_PAD];
    w[lane * CLK_PAD] = ~0ull;
    w[(CLK_SLOTS + lane) * CLK_PAD] = 0ull;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const unsigned long long a = __shfl_xor(t0, o, 64), b = __shfl_xor(t1, o, 64);
        t0 = a < t0 ? a : t0;
        t1 = b > t1 ? b : t1;
    }
    if (lane == 0) {
        out[2 * k] = t0;
        out[2 * k + 1] = t1;
    }
}

hipError_t launch_clock_fold(unsigned long long *clk, unsigned long long *out, int nk, hipStream_t s) {
    hipLaunchKernelGGL(k_clock_fold, dim3(nk), dim3(64), 0, s, clk, out);
    return hipGetLastError();
}

// Streaming read: wave w reads KIB KiB at byte offset w * KIB KiB, as KIB
// 16-byte loads per lane (each load one contiguous KiB across the wave), all
// requested before any is used -- the shape of the scoring pass (8 KiB of
// key codes per wave) and of the FP16-key pass (16 KiB per block).  The
// loaded words are folded and written only if the fold hits one value, so
// the loads stay and (almost) nothing is written.
template <int KIB>
__global__ __launch_bounds__(256) void k_read_probe(const unsigned char *buf, unsigned long long nwaves,
                                                    unsigned *sink) {
    const unsigned long long w = (unsigned long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= nwaves) return;
    const int lane = threadIdx.x & 63;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(buf + w * (KIB * 1024ull), KIB * 1024u);
    uint4 x[KIB];
#pragma unroll
    for (int i = 0; i < KIB; ++i) x[i] = rsrc_load16(r, (uint32_t)(i * 1024 + lane * 16));
    unsigned f = 0;
#pragma unroll
    for (int i = 0; i < KIB; ++i) f ^= x[i].x ^ x[i].y ^ x[i].z ^ x[i].w;
    if (f == 0x9E3779B9u) sink[0] = (unsigned)w;
}

}  // namespace ckv

using namespace ckv;

extern "C" ckv_status ckv_read_probe(const void *dev_buf, size_t bytes, int wave_kib, unsigned *dev_sink,
                                     void *stream) {
    if (!dev_buf || !dev_sink) return (ckv_status)set_error(CKV_EINVAL, "null argument");
    if (wave_kib != 4 && wave_kib != 8 && wave_kib != 16)
        return (ckv_status)set_error(CKV_EINVAL, "wave_kib must be 4, 8 or 16");
    const size_t per = (size_t)wave_kib * 1024;
    if (bytes == 0 || bytes % per || bytes / per > (size_t)1 << 32)
        return (ckv_status)set_error(CKV_EINVAL, "bytes must be a positive multiple of wave_kib KiB, at most 2^32 waves");
    const unsigned long long nw = bytes / per;
    const dim3 grid((unsigned)((nw + 3) / 4));
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const unsigned char *b = static_cast<const unsigned char *>(dev_buf);
    if (wave_kib == 4) hipLaunchKernelGGL(k_read_probe<4>, grid, dim3(256), 0, s, b, nw, dev_sink);
    else if (wave_kib == 8) hipLaunchKernelGGL(k_read_probe<8>, grid, dim3(256), 0, s, b, nw, dev_sink);
    else hipLaunchKernelGGL(k_read_probe<16>, grid, dim3(256), 0, s, b, nw, dev_sink);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (ckv_status)set_error(CKV_EHIP, hipGetErrorString(e));
    return CKV_OK;
}
