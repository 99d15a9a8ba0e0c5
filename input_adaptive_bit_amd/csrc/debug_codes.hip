// Test and diagnostic kernel: the truncated codes q_b * 2^(b_max-b) for every
// loaded channel (GRINQH note, key designs 2-3), decoded by the same routine
// the GEMV kernel uses (decode_values in decode.hpp); skipped channels get 0.
#include "decode.hpp"
#include "internal.h"

namespace grinqh {
namespace {

// Codes of one word position as the GEMV kernel decodes them: the channel's
// Pb taken planes go through decode_values<Pb>; value * unit (exact) is the
// Pb-plane code, times 4^(P-Pb) at full width.
template <int P, int Pb>
__device__ __forceinline__ void decode16(const uint32_t* words, uint8_t (&out)[16]) {
    float val[16];
    decode_values<Pb>(words, val);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const uint32_t c = static_cast<uint32_t>(val[t] * decode_unit<Pb>(t & 3));
        out[t] = static_cast<uint8_t>(c << (2 * (P - Pb)));
    }
}

template <int P>
__global__ __launch_bounds__(256) void debug_codes_kernel(const uint8_t* __restrict__ bits,
                                                          const uint32_t* __restrict__ planes,
                                                          uint8_t* __restrict__ codes, int d_in,
                                                          int d_out, int row_words) {
    const int w = blockIdx.x * blockDim.x + threadIdx.x;   // word within the row
    if (w >= row_words) return;
    for (int i = blockIdx.y; i < d_in; i += gridDim.y) {
        const int Pi = bits[i] >> 1;
        uint32_t words[4] = {0u, 0u, 0u, 0u};
        for (int p = 0; p < Pi && p < P; ++p)
            words[p] = planes[(static_cast<size_t>(i) * P + p) * row_words + w];
        uint8_t c[16];
        switch (Pi < P ? Pi : P) {
            case 1: decode16<P, 1>(words, c); break;
            case 2: if constexpr (P >= 2) decode16<P, 2>(words, c); break;
            case 3: if constexpr (P >= 3) decode16<P, 3>(words, c); break;
            case 4: if constexpr (P >= 4) decode16<P, 4>(words, c); break;
            default:
#pragma unroll
                for (int t = 0; t < 16; ++t) c[t] = 0;
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int j = 16 * w + t;
            if (j < d_out) codes[static_cast<size_t>(i) * d_out + j] = c[t];
        }
    }
}

}  // namespace

hipError_t launch_debug_codes(const grinqh_layout& L, const uint8_t* bits,
                              const uint32_t* planes, uint8_t* codes, hipStream_t stream) {
    dim3 block(256);
    dim3 grid(static_cast<unsigned>((L.row_words + 255) / 256),
              static_cast<unsigned>(L.d_in < 65535 ? L.d_in : 65535));
    switch (L.n_planes) {
        case 1: debug_codes_kernel<1><<<grid, block, 0, stream>>>(bits, planes, codes, L.d_in, L.d_out, L.row_words); break;
        case 2: debug_codes_kernel<2><<<grid, block, 0, stream>>>(bits, planes, codes, L.d_in, L.d_out, L.row_words); break;
        case 3: debug_codes_kernel<3><<<grid, block, 0, stream>>>(bits, planes, codes, L.d_in, L.d_out, L.row_words); break;
        case 4: debug_codes_kernel<4><<<grid, block, 0, stream>>>(bits, planes, codes, L.d_in, L.d_out, L.row_words); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace grinqh
