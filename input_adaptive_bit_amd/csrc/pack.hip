// Offline bit-plane packing (GRINQH note, key design 2: 2-bit fragments
// stacked as planes from high to low significance, reduction dimension first,
// 16 fragments per uint32).
//
// One workgroup transposes a 64 (outputs) x 64 (input channels) tile of q
// through LDS: q rows are read as contiguous bytes, and each thread then
// writes the 4 consecutive words (64 outputs) of one (channel, plane) row
// segment, so stores go out 16 bytes at a time.
#include "device_common.hpp"
#include "internal.h"

namespace grinqh {
namespace {

constexpr int kTile = 64;

template <int P>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ q,
                                                   uint32_t* __restrict__ planes, int d_in,
                                                   int d_out, int row_words) {
    constexpr int b_max = 2 * P;
    __shared__ uint8_t tile[kTile][kTile + 4];   // [output][channel]
    const int j0 = blockIdx.x * kTile;           // first output of the tile
    const int i0 = blockIdx.y * kTile;           // first input channel of the tile
    const unsigned mask = (1u << b_max) - 1u;

    for (int idx = threadIdx.x; idx < kTile * kTile; idx += blockDim.x) {
        int jj = idx / kTile, ii = idx % kTile;
        int j = j0 + jj, i = i0 + ii;
        uint8_t v = 0;
        if (j < d_out && i < d_in) v = static_cast<uint8_t>(q[static_cast<size_t>(j) * d_in + i] & mask);
        tile[jj][ii] = v;                         // padding outputs get code 0
    }
    __syncthreads();

    // 64 channels x 4 words: thread -> (channel ii, word ww), words fastest.
    const int ww = threadIdx.x & 3;
    const int ii = threadIdx.x >> 2;
    const int i = i0 + ii;
    if (i >= d_in) return;
    const int w = (j0 >> 4) + ww;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int shift = b_max - 2 * p - 2;
        uint32_t word = 0;
#pragma unroll
        for (int t = 0; t < 16; ++t)
            word |= static_cast<uint32_t>((tile[ww * 16 + t][ii] >> shift) & 3u) << (2 * t);
        planes[(static_cast<size_t>(i) * P + p) * row_words + w] = word;
    }
}

}  // namespace

hipError_t launch_pack(const grinqh_layout& L, const uint8_t* q, uint32_t* planes,
                       hipStream_t stream) {
    // row_words * 16 (padded outputs) is a multiple of 64, so tiles cover rows exactly.
    dim3 grid(static_cast<unsigned>(L.row_words / 4), static_cast<unsigned>((L.d_in + kTile - 1) / kTile));
    dim3 block(256);
    switch (L.n_planes) {
        case 1: pack_kernel<1><<<grid, block, 0, stream>>>(q, planes, L.d_in, L.d_out, L.row_words); break;
        case 2: pack_kernel<2><<<grid, block, 0, stream>>>(q, planes, L.d_in, L.d_out, L.row_words); break;
        case 3: pack_kernel<3><<<grid, block, 0, stream>>>(q, planes, L.d_in, L.d_out, L.row_words); break;
        case 4: pack_kernel<4><<<grid, block, 0, stream>>>(q, planes, L.d_in, L.d_out, L.row_words); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace grinqh
