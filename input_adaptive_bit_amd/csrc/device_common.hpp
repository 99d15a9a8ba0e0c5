// Device helpers shared by the GRINQH kernels (gfx950).
//
// Method source: "GRINQH: Graded Input-Based Quantization Hierarchy for
// Efficient LLM Generation" (papernotes.org note), key design (关键设计)
// items 1-3: KD1 bit assignment, KD2 bit-planar storage, KD3 midpoint dequant.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace grinqh {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// x_i as fp32 (bf16 widens exactly).  dtype: 0 = bf16, 1 = f32.
__device__ __forceinline__ float load_x(const void* x, int dtype, int i) {
    if (dtype == 0) return bf16_to_f32(static_cast<const uint16_t*>(x)[i]);
    return static_cast<const float*>(x)[i];
}

// KD1: b_i = 2 * #{k : theta_k <= |x_i|}.  Exact fp32 compares; a NaN |x|
// fails every compare and gets 0 bits.
template <int P>
__device__ __forceinline__ int bits_of(float x, const float (&theta)[4]) {
    float a = __builtin_fabsf(x);
    int level = 0;
#pragma unroll
    for (int k = 0; k < P; ++k) level += (theta[k] <= a) ? 1 : 0;
    return 2 * level;
}

__device__ __forceinline__ int bits_of_rt(float x, const float (&theta)[4], int P) {
    float a = __builtin_fabsf(x);
    int level = 0;
    for (int k = 0; k < P; ++k) level += (theta[k] <= a) ? 1 : 0;
    return 2 * level;
}

// KD3: phi = 2^(k-1) with k = b_max - b (1/2 at k = 0), as an exact float.
__device__ __forceinline__ float phi_of(int b_max, int b) {
    int k = b_max - b;
    // 2^(k-1) for k in 0..8: build the exponent field directly (always normal).
    return __builtin_bit_cast(float, static_cast<uint32_t>(127 + k - 1) << 23);
}

}  // namespace grinqh
