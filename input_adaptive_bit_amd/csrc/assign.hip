// Runtime bit assignment (GRINQH note, key design 1): b_i from exact compares
// of |x_i| with the layer's thresholds, plus the ascending list of loaded
// channels (b_i > 0).  One workgroup walks the channels in blocks of 1024;
// a wave ballot gives each active lane its rank, so the list comes out in
// ascending order without atomics and is identical on every run.
#include "device_common.hpp"
#include "internal.h"

namespace grinqh {
namespace {

constexpr int kThreads = 1024;

template <int P>
__global__ __launch_bounds__(kThreads) void assign_kernel(const void* __restrict__ x, int x_dtype,
                                                          const float* __restrict__ theta,
                                                          uint8_t* __restrict__ bits,
                                                          int32_t* __restrict__ active_idx,
                                                          int32_t* __restrict__ n_active, int d_in) {
    __shared__ int wave_count[kThreads / kWave];
    float th[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < P; ++k) th[k] = theta[k];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    int base = 0;
    for (int i0 = 0; i0 < d_in; i0 += kThreads) {
        const int i = i0 + threadIdx.x;
        int b = 0;
        if (i < d_in) {
            b = bits_of<P>(load_x(x, x_dtype, i), th);
            bits[i] = static_cast<uint8_t>(b);
        }
        const unsigned long long m = __ballot(b > 0);
        const int rank = __popcll(m & ((1ull << lane) - 1ull));
        if (lane == 0) wave_count[wv] = __popcll(m);
        __syncthreads();
        int off = base, total = 0;
        for (int k = 0; k < kThreads / kWave; ++k) {
            if (k < wv) off += wave_count[k];
            total += wave_count[k];
        }
        if (b > 0 && active_idx != nullptr) active_idx[off + rank] = i;
        __syncthreads();
        base += total;
    }
    if (threadIdx.x == 0 && n_active != nullptr) *n_active = base;
}

}  // namespace

hipError_t launch_assign_bits(const grinqh_layout& L, const void* x, int x_dtype,
                              const float* theta, uint8_t* bits, int32_t* active_idx,
                              int32_t* n_active, hipStream_t stream) {
    dim3 grid(1), block(kThreads);
    switch (L.n_planes) {
        case 1: assign_kernel<1><<<grid, block, 0, stream>>>(x, x_dtype, theta, bits, active_idx, n_active, L.d_in); break;
        case 2: assign_kernel<2><<<grid, block, 0, stream>>>(x, x_dtype, theta, bits, active_idx, n_active, L.d_in); break;
        case 3: assign_kernel<3><<<grid, block, 0, stream>>>(x, x_dtype, theta, bits, active_idx, n_active, L.d_in); break;
        case 4: assign_kernel<4><<<grid, block, 0, stream>>>(x, x_dtype, theta, bits, active_idx, n_active, L.d_in); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace grinqh
