// Plane decoding shared by the GEMV kernel and the debug-codes kernel
// (GRINQH note, key design 2: fragment of output 16w+t at bits [2t, 2t+1] of
// word w; key design 3: the taken planes concatenate into the truncated code).
#pragma once

#include "device_common.hpp"

namespace grinqh {

// 2-bit fragment t (0..15) of a plane word.
__device__ __forceinline__ uint32_t fragment(uint32_t word, int t) {
    return (word >> (2 * t)) & 3u;
}

// Weight of plane p in a code of P planes: 4^(P-1-p) (plane 0 most significant).
template <int P>
__device__ __forceinline__ float plane_weight(int p) {
    return static_cast<float>(1u << (2 * (P - 1 - p)));
}

// Truncated code q_b * 2^(b_max-b) of output t from the first Pi plane words.
template <int P>
__device__ __forceinline__ uint32_t truncated_code(const uint32_t (&words)[4], int Pi, int t) {
    uint32_t c = 0;
#pragma unroll
    for (int p = 0; p < P; ++p)
        if (p < Pi) c |= fragment(words[p], t) << (2 * (P - 1 - p));
    return c;
}

}  // namespace grinqh
