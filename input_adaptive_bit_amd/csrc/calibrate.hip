// Threshold calibration on the device (GRINQH note, key design 1: the
// thresholds theta_1..theta_P are fixed offline from the magnitudes of about
// 128 sample inputs of the layer).
//
// The thresholds are quantiles of the pooled magnitudes |x| of the samples:
// for a level q, with the n magnitudes sorted ascending (NaN after +Inf),
// h = (n - 1) * q, lo = floor(h), hi = min(lo + 1, n - 1), t = h - lo, the
// threshold is v[lo] + t * (v[hi] - v[lo]) in fp64 (v[lo] itself at t = 0),
// rounded once to fp32.  The host computes lo, hi and t; the device finds the
// order statistics v[lo] and v[hi] exactly and interpolates.
//
// Order statistics by radix selection on the magnitude key: the fp32 bit
// pattern of |x| with the sign cleared, whose integer order is the numeric
// order of the magnitudes (NaN patterns above +Inf).  Three passes fix the
// key bits 31..21, 20..10 and 9..0 of every target rank: a histogram of the
// pass's digit over the keys that share the bits fixed so far (one shared
// histogram in the first pass), then a scan of that histogram by one
// workgroup, which picks the digit holding the target's rank and moves the
// rank inside it.  Every count and rank fits 32 bits (n < 2^32).
#include <math.h>

#include "device_common.hpp"
#include "internal.h"

namespace grinqh {
namespace {

constexpr int kCalThreads = 256;
constexpr int kCalMaxLevels = 4;               // thresholds of b_max 8
constexpr int kCalTargets = 2 * kCalMaxLevels; // v[lo] and v[hi] of every level
constexpr int kCalBins = 2048;                 // widest digit: 11 bits
constexpr int kCalMaxBlocks = 1024;

__host__ __device__ constexpr int pass_shift(int d) { return d == 0 ? 21 : d == 1 ? 10 : 0; }
__host__ __device__ constexpr int pass_width(int d) { return d == 2 ? 10 : 11; }

struct CalWorkspace {
    uint32_t prefix[kCalTargets];              // key bits fixed so far, per target
    uint32_t rank[kCalTargets];                // rank among the keys sharing that prefix
    uint32_t hist[kCalTargets * kCalBins];     // this pass's histograms
};

struct CalRanks {
    uint32_t rank[kCalTargets];
    int n_targets;
};

struct CalLevels {
    double t[kCalMaxLevels];
    int n_levels;
};

__device__ __forceinline__ uint32_t magnitude_key(const void* x, int dtype, int64_t i) {
    if (dtype == GRINQH_BF16) return (static_cast<uint32_t>(static_cast<const uint16_t*>(x)[i]) << 16) & 0x7FFFFFFFu;
    return __float_as_uint(static_cast<const float*>(x)[i]) & 0x7FFFFFFFu;
}

__global__ __launch_bounds__(kCalThreads) void cal_init(CalWorkspace* ws, CalRanks r) {
    const int i = blockIdx.x * kCalThreads + threadIdx.x;
    if (i < kCalTargets * kCalBins) ws->hist[i] = 0u;
    if (i < kCalTargets) {
        ws->prefix[i] = 0u;
        ws->rank[i] = i < r.n_targets ? r.rank[i] : 0u;
    }
}

// Histogram of pass D's digit.  Pass 0 counts every key into one histogram;
// later passes count, for every target, the keys whose higher bits equal the
// target's prefix.  Per-workgroup counts in LDS, added to the workspace.
template <int D>
__global__ __launch_bounds__(kCalThreads) void cal_hist(const void* x, int dtype, int64_t n, CalWorkspace* ws,
                                                        int n_targets) {
    constexpr int SHIFT = pass_shift(D);
    constexpr int WIDTH = pass_width(D);
    constexpr int BINS = 1 << WIDTH;
    constexpr int NT = D == 0 ? 1 : kCalTargets;
    __shared__ uint32_t h[NT * BINS];
    __shared__ uint32_t pre[kCalTargets];
    for (int i = threadIdx.x; i < NT * BINS; i += kCalThreads) h[i] = 0u;
    if (D > 0 && threadIdx.x < kCalTargets) pre[threadIdx.x] = ws->prefix[threadIdx.x] >> (SHIFT + WIDTH);
    __syncthreads();
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kCalThreads;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kCalThreads + threadIdx.x; i < n; i += stride) {
        const uint32_t k = magnitude_key(x, dtype, i);
        const uint32_t digit = (k >> SHIFT) & (BINS - 1);
        if constexpr (D == 0) {
            atomicAdd(&h[digit], 1u);
        } else {
            const uint32_t high = k >> (SHIFT + WIDTH);
            for (int t = 0; t < n_targets; ++t)
                if (high == pre[t]) atomicAdd(&h[t * BINS + digit], 1u);
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < NT * BINS; i += kCalThreads) {
        const uint32_t c = h[i];
        if (c != 0u) atomicAdd(&ws->hist[i], c);
    }
}

// One workgroup: for every target, the digit of pass D whose keys hold the
// target's rank; the rank moves inside that digit.  Clears the histograms
// for the next pass.
template <int D>
__global__ __launch_bounds__(kCalThreads) void cal_select(CalWorkspace* ws, int n_targets) {
    constexpr int SHIFT = pass_shift(D);
    constexpr int BINS = 1 << pass_width(D);
    constexpr int PER = BINS / kCalThreads;     // bins per thread
    __shared__ uint32_t scan[kCalThreads];
    __shared__ uint32_t s_prefix[kCalTargets], s_rank[kCalTargets];
    const int tid = threadIdx.x;
    if (tid < kCalTargets) {
        s_prefix[tid] = ws->prefix[tid];
        s_rank[tid] = ws->rank[tid];
    }
    __syncthreads();
    for (int t = 0; t < n_targets; ++t) {
        const uint32_t* h = ws->hist + (D == 0 ? 0 : t * BINS);
        uint32_t local[PER];
        uint32_t sum = 0u;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            local[j] = h[tid * PER + j];
            sum += local[j];
        }
        // inclusive scan of the per-thread sums
        scan[tid] = sum;
        __syncthreads();
        for (int off = 1; off < kCalThreads; off <<= 1) {
            const uint32_t add = tid >= off ? scan[tid - off] : 0u;
            __syncthreads();
            scan[tid] += add;
            __syncthreads();
        }
        const uint32_t r = s_rank[t];
        const uint32_t before = scan[tid] - sum;
        __syncthreads();
        if (before <= r && r < before + sum) {
            uint32_t c = before;
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                if (r < c + local[j]) {
                    s_prefix[t] |= static_cast<uint32_t>(tid * PER + j) << SHIFT;
                    s_rank[t] = r - c;
                    break;
                }
                c += local[j];
            }
        }
        __syncthreads();
    }
    if (tid < kCalTargets) {
        ws->prefix[tid] = s_prefix[tid];
        ws->rank[tid] = s_rank[tid];
    }
    for (int i = tid; i < kCalTargets * kCalBins; i += kCalThreads) ws->hist[i] = 0u;
}

// The magnitude a key stands for, in fp64 (exact).  A subnormal key is
// widened by hand, so the result does not depend on the fp32 denormal mode.
__device__ __forceinline__ double key_value(uint32_t k) {
    if ((k >> 23) == 0u) return __dmul_rn(static_cast<double>(k), 0x1p-149);
    return static_cast<double>(__uint_as_float(k));
}

// theta_k = v[lo] + t * (v[hi] - v[lo]) in fp64 with separate roundings
// (v[lo] itself at t = 0), rounded to fp32.
__global__ void cal_finish(const CalWorkspace* ws, CalLevels lv, float* theta) {
    const int k = threadIdx.x;
    if (k >= lv.n_levels) return;
    const double a = key_value(ws->prefix[2 * k]);
    const double b = key_value(ws->prefix[2 * k + 1]);
    const double t = lv.t[k];
    const double v = t == 0.0 ? a : __dadd_rn(a, __dmul_rn(t, __dsub_rn(b, a)));
    theta[k] = static_cast<float>(v);
}

size_t cal_workspace_bytes() { return (sizeof(CalWorkspace) + 255) / 256 * 256; }

}  // namespace
}  // namespace grinqh

using namespace grinqh;

extern "C" size_t grinqh_calibrate_workspace_bytes(void) { return cal_workspace_bytes(); }

extern "C" grinqh_status grinqh_calibrate_thresholds(const void* x, grinqh_dtype x_dtype, int64_t count,
                                                     const double* levels, int32_t n_levels, float* theta,
                                                     void* workspace, size_t workspace_bytes, void* stream) {
    if (x == nullptr || levels == nullptr || theta == nullptr || workspace == nullptr) return GRINQH_EINVAL;
    if (x_dtype != GRINQH_BF16 && x_dtype != GRINQH_F32) return GRINQH_EINVAL;
    if (count < 1 || count > static_cast<int64_t>(UINT32_MAX)) return GRINQH_EINVAL;
    if (n_levels < 1 || n_levels > kCalMaxLevels) return GRINQH_EINVAL;
    for (int k = 0; k < n_levels; ++k)
        if (!(levels[k] >= 0.0 && levels[k] <= 1.0)) return GRINQH_EINVAL;      // NaN fails too
    const size_t xb = x_dtype == GRINQH_BF16 ? 2 : 4;
    if (reinterpret_cast<uintptr_t>(x) % xb != 0 || reinterpret_cast<uintptr_t>(theta) % 4 != 0 ||
        reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return GRINQH_EALIGN;
    if (workspace_bytes < cal_workspace_bytes()) return GRINQH_ENOSPACE;
    DeviceInfo dev;
    hipError_t e;
    if (!current_device_info(&dev, &e))
        return (e == hipErrorNoDevice || e == hipErrorInvalidDevice) ? GRINQH_ENODEV : GRINQH_EDEVICE;

    CalRanks ranks{};
    CalLevels lv{};
    ranks.n_targets = 2 * n_levels;
    lv.n_levels = n_levels;
    for (int k = 0; k < n_levels; ++k) {
        const double h = static_cast<double>(count - 1) * levels[k];
        const double lo = floor(h);
        const int64_t ilo = static_cast<int64_t>(lo);
        const int64_t ihi = ilo + 1 < count ? ilo + 1 : count - 1;
        ranks.rank[2 * k] = static_cast<uint32_t>(ilo);
        ranks.rank[2 * k + 1] = static_cast<uint32_t>(ihi);
        lv.t[k] = h - lo;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    auto* ws = static_cast<CalWorkspace*>(workspace);
    const int64_t want = (count + kCalThreads * 8 - 1) / (kCalThreads * 8);
    const unsigned blocks = static_cast<unsigned>(want < kCalMaxBlocks ? (want < 1 ? 1 : want) : kCalMaxBlocks);
    cal_init<<<(kCalTargets * kCalBins + kCalThreads - 1) / kCalThreads, kCalThreads, 0, s>>>(ws, ranks);
    cal_hist<0><<<blocks, kCalThreads, 0, s>>>(x, x_dtype, count, ws, ranks.n_targets);
    cal_select<0><<<1, kCalThreads, 0, s>>>(ws, ranks.n_targets);
    cal_hist<1><<<blocks, kCalThreads, 0, s>>>(x, x_dtype, count, ws, ranks.n_targets);
    cal_select<1><<<1, kCalThreads, 0, s>>>(ws, ranks.n_targets);
    cal_hist<2><<<blocks, kCalThreads, 0, s>>>(x, x_dtype, count, ws, ranks.n_targets);
    cal_select<2><<<1, kCalThreads, 0, s>>>(ws, ranks.n_targets);
    cal_finish<<<1, 64, 0, s>>>(ws, lv, theta);
    e = hipGetLastError();
    return e == hipSuccess ? GRINQH_OK : GRINQH_EDEVICE;
}
