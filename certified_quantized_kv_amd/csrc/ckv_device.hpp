// ckv_device.hpp -- device helpers of the certified quantized-KV library.
//
// Decision arithmetic (codes, scores, masses, bounds, verdicts) must give the
// same bits on every run and every launch shape, so it is written here as a
// fixed sequence of single IEEE operations: FP32 fma chains in one lane,
// halving-tree sums whose pairing is fixed (lane i + lane i+stride), an
// exponential built from fma/rint/ldexp only, FP64 upper bounds built from
// + - * / only, and unsigned fixed-point sums (order-free).  The library is
// compiled with -ffp-contract=off so no other fusion happens.
#pragma once
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ckv_internal.hpp"

namespace ckv {

constexpr int BT = 64;       // tokens per block
constexpr int VG = 32;       // channels per INT4 value group
constexpr uint64_t FXCAP = 1ull << 46;

__device__ __forceinline__ float h2f(uint16_t b) { return __half2float(__ushort_as_half(b)); }

// Smallest binary16 >= x, for x >= 0 (scale rounding upward).
__device__ __forceinline__ uint16_t f2h_up(float x) {
    if (!(x > 0.0f)) return 0;
    uint16_t h = __half_as_ushort(__float2half_rn(x));
    if (h < 0x7C00u && h2f(h) < x) h = (uint16_t)(h + 1);
    return h;
}

// binary64 -> binary32 rounded upward, for x >= 0 (bounds and ranges).
__device__ __forceinline__ float ru32(double x) {
    float f = (float)x;
    if ((double)f < x) f = __int_as_float(__float_as_int(f) + 1);
    return f;
}

// exp(x) for x <= 0: k = rint(x log2 e); r = x - k ln2 with ln2 split in two
// parts (Cody-Waite); e^r by the degree-7 Taylor polynomial (Horner, fma);
// result r 2^k; 0 when k < -125 (no subnormal results).
__device__ __forceinline__ float exp_c(float x) {
    float y = x * 1.44269502f;           // log2(e) in binary32: 0x3FB8AA3B
    float k = rintf(y);
    // below 2^-125 the result is 0; selected at the end rather than branched
    // on, so that the caller's loop has no lane-divergent paths
    const bool under = k < -125.0f;
    float r = fmaf(-k, 0.693145751953125f, x);   // 0x3F317200
    r = fmaf(-k, 1.42860677e-06f, r);            // 0x35BFBE8E
    float p = 1.98412701e-04f;                   // 1/7!  0x39500D01
    p = fmaf(p, r, 1.38888892e-03f);             // 1/6!  0x3AB60B61
    p = fmaf(p, r, 8.33333377e-03f);             // 1/5!  0x3C088889
    p = fmaf(p, r, 4.16666679e-02f);             // 1/4!  0x3D2AAAAB
    p = fmaf(p, r, 1.66666672e-01f);             // 1/3!  0x3E2AAAAB
    p = fmaf(p, r, 0.5f);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    return under ? 0.0f : ldexpf(p, (int)k);
}

// Upper bound of e^x, x >= 0: halve to r <= 1/16, Taylor to degree 12,
// square back, times (1 + 2^-36).
__device__ __forceinline__ double expu(double x) {
    if (!(x <= 64.0)) return __longlong_as_double(0x7FF0000000000000ll);
    if (x <= 0.0) x = 0.0;
    int j = 0;
    double r = x;
    while (r > 0.0625) { r *= 0.5; ++j; }
    double f = 479001600.0;              // 12!
    double p = 1.0 / f;
    for (int i = 11; i >= 0; --i) {
        f = f / (double)(i + 1);         // i!
        p = fma(p, r, 1.0 / f);
    }
    for (int i = 0; i < j; ++i) p = p * p;
    return p * (1.0 + 0x1p-36);
}

// Upper bound of e^x - 1, x >= 0.
__device__ __forceinline__ double em1u(double x) {
    if (!(x > 0.0)) return 0.0;
    if (x > 64.0) return __longlong_as_double(0x7FF0000000000000ll);
    if (x <= 0.5) {
        double c[16];
        double f = 1.0;
        for (int i = 0; i < 16; ++i) { f = f * (double)(i + 1); c[i] = 1.0 / f; }
        double p = c[15];
        for (int i = 14; i >= 0; --i) p = fma(p, x, c[i]);
        return x * p * (1.0 + 0x1p-48);
    }
    return (expu(x) - 1.0) * (1.0 + 0x1p-50);
}

// Upper bound of tanh(x/2) = m / (m + 2), m = e^x - 1.
__device__ __forceinline__ double tanhu(double x) {
    double m = em1u(x);
    if (__isinf(m)) return 1.0;
    double t = m / (m + 2.0) * (1.0 + 0x1p-48);
    return t < 1.0 ? t : 1.0;
}

// Bound term -> fixed point with 32 fraction bits, rounded up, capped.
__device__ __forceinline__ uint64_t fx(double t) {
    if (!(t < 16384.0)) return FXCAP;
    if (t <= 0.0) return 0;
    uint64_t u = (uint64_t)ceil(t * 4294967296.0);
    return u < FXCAP ? u : FXCAP;
}

__device__ __forceinline__ double fx_bound(uint64_t sum, bool sat) {
    if (sat) return __longlong_as_double(0x7FF0000000000000ll);
    return (double)sum * 0x1p-32 * (1.0 + 0x1p-50);
}

// LDS writes of the wave's lanes visible to the wave's other lanes.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Execution span of one kernel launch, for profiling.  With a non-null
// clk, every wave reads the device's constant-rate wall clock when it starts
// and again when it ends; wave 0 of each workgroup takes the minimum of its
// start time into start slot w % CLK_SLOTS and every wave the maximum of its
// end time into the matching end slot (w = the linear workgroup index), so
// max(end) - min(start) over the slots is the span from the first wave's
// start to the last wave's end.  Both atomics are issued at the end, after
// the wave's last load: an atomic issued first would hold the wave's first
// load wait until it completed (memory counters retire in order).  The end
// is stamped when the object goes out of scope, so early returns are
// covered.  Spreading over slots on separate lines keeps the atomics from
// queueing on one line.
struct KernelClock {
    unsigned long long *clk;
    unsigned long long t0;
    __device__ __forceinline__ explicit KernelClock(unsigned long long *c) : clk(c), t0(0) {
        if (clk) t0 = (unsigned long long)wall_clock64();
    }
    __device__ __forceinline__ ~KernelClock() {
        if (clk && (threadIdx.x & 63) == 0) {
            const unsigned long long t1 = (unsigned long long)wall_clock64();
            const int slot = (int)((blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z)) % CLK_SLOTS);
            if (threadIdx.x == 0) atomicMin(clk + slot * CLK_PAD, t0);
            atomicMax(clk + (CLK_SLOTS + slot) * CLK_PAD, t1);
        }
    }
    KernelClock(const KernelClock &) = delete;
    KernelClock &operator=(const KernelClock &) = delete;
};

// ---- wave reductions (wave64) ---------------------------------------------

// Halving-tree sum: lane i adds lane i + stride for stride 32..1; the result
// is in lane 0 (other lanes hold partial sums).
__device__ __forceinline__ double tree64_f64(double v) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v = v + __shfl_down(v, s, 64);
    return v;
}

// Order-free reductions (every lane gets the result).
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v = fmaxf(v, __shfl_xor(v, s, 64));
    return v;
}

// ---- buffer-resource loads ---------------------------------------------------
// A buffer resource covers [base, base + bytes); a load at an offset past
// the range returns zeros and touches no memory, so a load instruction can be
// issued on every path (as a placeholder where there is nothing to load).
// Word 3 of the resource: 32-bit data format, no swizzle, no index stride.
typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));
constexpr uint32_t RSRC_OOB = 0x40000000u;  // an offset past every range used
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ float rsrc_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint4 rsrc_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const v4u32 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 rsrc_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    typedef uint32_t v2u32_ __attribute__((ext_vector_type(2)));
    const v2u32_ v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
    return make_uint2(v.x, v.y);
}

// ---- DPP row operations (16-lane rows of a wave64) --------------------------
// row_shl:n gives lane i the value of lane i + n of its row, row_shr:n the
// value of lane i - n; lanes whose source lies outside the row keep the
// `old` operand (their own value, or 0 in the zero-filling forms).  quad_perm / mirrors permute inside
// a row.  These run on the VALU without going through LDS.
enum : int {
    DPP_QP_1032 = 0xB1,        // quad_perm [1,0,3,2]
    DPP_QP_2301 = 0x4E,        // quad_perm [2,3,0,1]
    DPP_ROW_SL1 = 0x101,
    DPP_ROW_SL2 = 0x102,
    DPP_ROW_SL4 = 0x104,
    DPP_ROW_SL8 = 0x108,
    DPP_ROW_SR1 = 0x111,
    DPP_ROW_SR2 = 0x112,
    DPP_ROW_SR4 = 0x114,
    DPP_ROW_SR8 = 0x118,
    DPP_ROW_MIRROR = 0x140,
    DPP_ROW_HALF_MIRROR = 0x141,
};

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
    return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp((int)b, (int)b, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp((int)(b >> 32), (int)(b >> 32), CTRL, 0xF, 0xF, false);
    return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// Halving tree over the 16 lanes of a row (strides 8, 4, 2, 1: lane i adds
// lane i + stride); the row's sum ends in its lane 0.
__device__ __forceinline__ float row_tree_f32(float v) {
    v = v + dpp_f32<DPP_ROW_SL8>(v);
    v = v + dpp_f32<DPP_ROW_SL4>(v);
    v = v + dpp_f32<DPP_ROW_SL2>(v);
    v = v + dpp_f32<DPP_ROW_SL1>(v);
    return v;
}
__device__ __forceinline__ double row_tree_f64(double v) {
    v = v + dpp_f64<DPP_ROW_SL8>(v);
    v = v + dpp_f64<DPP_ROW_SL4>(v);
    v = v + dpp_f64<DPP_ROW_SL2>(v);
    v = v + dpp_f64<DPP_ROW_SL1>(v);
    return v;
}
// Order-free reductions over a row; every lane of the row gets the result.
__device__ __forceinline__ float row_max_f32(float v) {
    v = fmaxf(v, dpp_f32<DPP_QP_1032>(v));
    v = fmaxf(v, dpp_f32<DPP_QP_2301>(v));
    v = fmaxf(v, dpp_f32<DPP_ROW_HALF_MIRROR>(v));
    v = fmaxf(v, dpp_f32<DPP_ROW_MIRROR>(v));
    return v;
}
__device__ __forceinline__ int row_sum_i32(int v) {
    v = v + dpp_i32<DPP_QP_1032>(v);
    v = v + dpp_i32<DPP_QP_2301>(v);
    v = v + dpp_i32<DPP_ROW_HALF_MIRROR>(v);
    v = v + dpp_i32<DPP_ROW_MIRROR>(v);
    return v;
}

__device__ __forceinline__ float row_sum_f32(float v) {
    v = v + dpp_f32<DPP_QP_1032>(v);
    v = v + dpp_f32<DPP_QP_2301>(v);
    v = v + dpp_f32<DPP_ROW_HALF_MIRROR>(v);
    v = v + dpp_f32<DPP_ROW_MIRROR>(v);
    return v;
}

// Wave-wide max / sum: DPP inside the rows, then the four row results read
// as scalars.  Every lane gets the result.
__device__ __forceinline__ float wave_max_dpp(float v) {
    v = row_max_f32(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
    v = row_sum_f32(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

// The halving tree over 64 lanes (strides 32, 16 across rows, then 8..1
// inside row 0); the result is in lane 0.  Same pairing as tree64_f64.
__device__ __forceinline__ float tree64_f32_dpp(float v) {
    v = v + __shfl_down(v, 32, 64);
    v = v + __shfl_down(v, 16, 64);
    return row_tree_f32(v);
}

// ---- 64-bit DPP helpers and order-free wave reductions ---------------------
// (max, min, sum, or: any combination order gives the same result)
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const int lo = __builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp((int)(v >> 32), (int)(v >> 32), CTRL, 0xF, 0xF, false);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
// shifted copy inside the row with zero fill (row_shl / row_shr)
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64_z(uint64_t v) {
    const int lo = __builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(v >> 32), CTRL, 0xF, 0xF, false);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32_z(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
    const uint32_t lo = __builtin_amdgcn_readlane((int)v, l), hi = __builtin_amdgcn_readlane((int)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}
template <class Op>
__device__ __forceinline__ uint64_t wave_reduce_u64(uint64_t v, Op op) {
    v = op(v, dpp_u64<DPP_QP_1032>(v));
    v = op(v, dpp_u64<DPP_QP_2301>(v));
    v = op(v, dpp_u64<DPP_ROW_HALF_MIRROR>(v));
    v = op(v, dpp_u64<DPP_ROW_MIRROR>(v));
    return op(op(readlane_u64(v, 0), readlane_u64(v, 16)), op(readlane_u64(v, 32), readlane_u64(v, 48)));
}
__device__ __forceinline__ uint64_t wave_sum_u64_dpp(uint64_t v) {
    return wave_reduce_u64(v, [](uint64_t a, uint64_t b) { return a + b; });
}
__device__ __forceinline__ uint64_t wave_min_u64_dpp(uint64_t v) {
    return wave_reduce_u64(v, [](uint64_t a, uint64_t b) { return a < b ? a : b; });
}
__device__ __forceinline__ uint64_t wave_max_u64_dpp(uint64_t v) {
    return wave_reduce_u64(v, [](uint64_t a, uint64_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ double wave_max_f64_dpp(double v) {
    v = fmax(v, dpp_f64<DPP_QP_1032>(v));
    v = fmax(v, dpp_f64<DPP_QP_2301>(v));
    v = fmax(v, dpp_f64<DPP_ROW_HALF_MIRROR>(v));
    v = fmax(v, dpp_f64<DPP_ROW_MIRROR>(v));
    auto rl = [&](int l) { return __longlong_as_double((long long)readlane_u64((uint64_t)__double_as_longlong(v), l)); };
    return fmax(fmax(rl(0), rl(16)), fmax(rl(32), rl(48)));
}
__device__ __forceinline__ int wave_sum_i32_dpp(int v) {
    v = row_sum_i32(v);
    return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
           (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}

// Inclusive suffix sums over the 64 lanes (lane i gets sum of lanes >= i)
// and exclusive prefix sums (lane i gets sum of lanes < i), exact integers.
__device__ __forceinline__ uint64_t wave_suffix_u64(uint64_t v, int lane) {
    v += dpp_u64_z<DPP_ROW_SL1>(v);
    v += dpp_u64_z<DPP_ROW_SL2>(v);
    v += dpp_u64_z<DPP_ROW_SL4>(v);
    v += dpp_u64_z<DPP_ROW_SL8>(v);
    const uint64_t t1 = readlane_u64(v, 16), t2 = readlane_u64(v, 32), t3 = readlane_u64(v, 48);
    const int r = lane >> 4;
    return v + (r < 1 ? t1 : 0) + (r < 2 ? t2 : 0) + (r < 3 ? t3 : 0);
}
__device__ __forceinline__ uint64_t wave_prefix_excl_u64(uint64_t v, int lane) {
    const uint64_t x = v;
    v += dpp_u64_z<DPP_ROW_SR1>(v);
    v += dpp_u64_z<DPP_ROW_SR2>(v);
    v += dpp_u64_z<DPP_ROW_SR4>(v);
    v += dpp_u64_z<DPP_ROW_SR8>(v);
    const uint64_t t0 = readlane_u64(v, 15), t1 = readlane_u64(v, 31), t2 = readlane_u64(v, 47);
    const int r = lane >> 4;
    return v - x + (r > 0 ? t0 : 0) + (r > 1 ? t1 : 0) + (r > 2 ? t2 : 0);
}
__device__ __forceinline__ uint32_t wave_prefix_excl_u32(uint32_t v, int lane) {
    const uint32_t x = v;
    v += dpp_u32_z<DPP_ROW_SR1>(v);
    v += dpp_u32_z<DPP_ROW_SR2>(v);
    v += dpp_u32_z<DPP_ROW_SR4>(v);
    v += dpp_u32_z<DPP_ROW_SR8>(v);
    const uint32_t t0 = __builtin_amdgcn_readlane((int)v, 15), t1 = __builtin_amdgcn_readlane((int)v, 31),
                   t2 = __builtin_amdgcn_readlane((int)v, 47);
    const int r = lane >> 4;
    return v - x + (r > 0 ? t0 : 0) + (r > 1 ? t1 : 0) + (r > 2 ? t2 : 0);
}

}  // namespace ckv
