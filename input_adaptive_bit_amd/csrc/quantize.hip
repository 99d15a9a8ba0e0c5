// Offline front end: round-to-nearest (RTN) quantisation of a weight matrix
// onto the b_max-bit grid that the GRINQH dequantisation (note, key design 3)
// reconstructs at full width.  The note names RTN as a base the method can
// sit on without defining it; the reading here is per output channel and
// asymmetric:
//
//   lo_j, hi_j = min, max of row j (NaN ignored),
//   s_j = fp16((hi_j - lo_j) / 2^b_max),  z_j = fp16(lo_j)  (a zero stored as +0),
//   q = min(max(floor((w - z_j) / s_j), 0), 2^b_max - 1)   in fp32 with the stored
//       s_j and z_j (a NaN quotient gives 0; a row with s_j = 0 gets q = 0),
//
// so that s_j * (q + 1/2) + z_j, the key-design-3 value at b = b_max, is the
// midpoint of w's interval.  One workgroup per output row: a min/max pass,
// then the codes (the row is read again from L2).
#include <hip/hip_fp16.h>
#include <math.h>

#include "internal.h"

namespace grinqh {
namespace {

constexpr int kRtnThreads = 256;

__device__ __forceinline__ float bf16_value(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint8_t rtn_code(float w, float z, float s, float top) {
    float u = floorf(__fdiv_rn(w - z, s));
    u = fmaxf(u, 0.f);                         // a NaN quotient becomes 0 here
    u = fminf(u, top);
    return static_cast<uint8_t>(u);
}

__global__ __launch_bounds__(kRtnThreads) void rtn_kernel(const uint16_t* __restrict__ w, int d_in, int b_max,
                                                          uint8_t* __restrict__ q, uint16_t* __restrict__ s_out,
                                                          uint16_t* __restrict__ z_out) {
    const int j = blockIdx.x;
    const int tid = threadIdx.x;
    const uint16_t* row = w + static_cast<size_t>(j) * d_in;
    uint8_t* qrow = q + static_cast<size_t>(j) * d_in;
    // 16-byte loads when the row allows it
    const bool vec = (d_in % 8 == 0) && (reinterpret_cast<uintptr_t>(row) % 16 == 0) &&
                     (reinterpret_cast<uintptr_t>(qrow) % 8 == 0);
    float lo = __uint_as_float(0x7FC00000u), hi = lo;   // NaN: ignored by fminf / fmaxf
    if (vec) {
        for (int i = tid * 8; i < d_in; i += kRtnThreads * 8) {
            const uint4 v = *reinterpret_cast<const uint4*>(row + i);
            const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float a = bf16_value(p[k] & 0xFFFFu), b = bf16_value(p[k] >> 16);
                lo = fminf(lo, fminf(a, b));
                hi = fmaxf(hi, fmaxf(a, b));
            }
        }
    } else {
        for (int i = tid; i < d_in; i += kRtnThreads) {
            const float a = bf16_value(row[i]);
            lo = fminf(lo, a);
            hi = fmaxf(hi, a);
        }
    }
    __shared__ float red_lo[kRtnThreads], red_hi[kRtnThreads];
    __shared__ float sz[2];
    red_lo[tid] = lo;
    red_hi[tid] = hi;
    __syncthreads();
    for (int h = kRtnThreads / 2; h > 0; h >>= 1) {
        if (tid < h) {
            red_lo[tid] = fminf(red_lo[tid], red_lo[tid + h]);
            red_hi[tid] = fmaxf(red_hi[tid], red_hi[tid + h]);
        }
        __syncthreads();
    }
    if (tid == 0) {
        const float rlo = red_lo[0], rhi = red_hi[0];
        const __half sh = __float2half_rn((rhi - rlo) * __uint_as_float(static_cast<uint32_t>(127 - b_max) << 23) + 0.f);
        const __half zh = __float2half_rn(rlo + 0.f);
        s_out[j] = __half_as_ushort(sh);
        z_out[j] = __half_as_ushort(zh);
        sz[0] = __half2float(sh);
        sz[1] = __half2float(zh);
    }
    __syncthreads();
    const float s = sz[0], z = sz[1];
    const float top = static_cast<float>((1 << b_max) - 1);
    const bool zero_scale = s == 0.f;
    if (vec) {
        for (int i = tid * 8; i < d_in; i += kRtnThreads * 8) {
            const uint4 v = *reinterpret_cast<const uint4*>(row + i);
            const uint32_t p[4] = {v.x, v.y, v.z, v.w};
            uint32_t out[2] = {0u, 0u};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t c0 = zero_scale ? 0u : rtn_code(bf16_value(p[k] & 0xFFFFu), z, s, top);
                const uint32_t c1 = zero_scale ? 0u : rtn_code(bf16_value(p[k] >> 16), z, s, top);
                out[k >> 1] |= (c0 | (c1 << 8)) << (16 * (k & 1));
            }
            *reinterpret_cast<uint2*>(qrow + i) = make_uint2(out[0], out[1]);
        }
    } else {
        for (int i = tid; i < d_in; i += kRtnThreads)
            qrow[i] = zero_scale ? static_cast<uint8_t>(0) : rtn_code(bf16_value(row[i]), z, s, top);
    }
}

}  // namespace
}  // namespace grinqh

using namespace grinqh;

extern "C" grinqh_status grinqh_quantize_rtn(int32_t d_in, int32_t d_out, int32_t b_max, const uint16_t* w,
                                             uint8_t* q, uint16_t* s, uint16_t* z, void* stream) {
    if (w == nullptr || q == nullptr || s == nullptr || z == nullptr) return GRINQH_EINVAL;
    if (d_in < 1 || d_in > (1 << 30) || d_out < 1 || d_out > (1 << 30)) return GRINQH_EINVAL;
    if (b_max != 2 && b_max != 4 && b_max != 6 && b_max != 8) return GRINQH_EINVAL;
    if (reinterpret_cast<uintptr_t>(w) % 2 != 0 || reinterpret_cast<uintptr_t>(s) % 2 != 0 ||
        reinterpret_cast<uintptr_t>(z) % 2 != 0)
        return GRINQH_EALIGN;
    DeviceInfo dev;
    hipError_t e;
    if (!current_device_info(&dev, &e))
        return (e == hipErrorNoDevice || e == hipErrorInvalidDevice) ? GRINQH_ENODEV : GRINQH_EDEVICE;
    rtn_kernel<<<static_cast<unsigned>(d_out), kRtnThreads, 0, static_cast<hipStream_t>(stream)>>>(
        w, d_in, b_max, q, s, z);
    e = hipGetLastError();
    return e == hipSuccess ? GRINQH_OK : GRINQH_EDEVICE;
}
