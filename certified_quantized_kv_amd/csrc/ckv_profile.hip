// ckv_profile.hip -- the kernel clock of profiled decode steps: folding the
// timed kernels' clock slots into one start and one end per kernel.
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

}  // namespace ckv
