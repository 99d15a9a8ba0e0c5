// The decode GEMV (GRINQH note, key designs 1-3), first version.
//
//   kernel 1 (partial): workgroup = (output tile of 1024, slice of input
//     channels).  Each wave takes every 4th channel of the slice, assigns its
//     bit width from |x_i| and the thresholds, and for a loaded channel reads
//     only the first b_i/2 plane rows of the tile (one uint32 = 16 outputs
//     per lane), accumulating x_i * 4^(P-1-p) * fragment in fp32.  The four
//     waves are summed through LDS and the tile's partial sums are stored.
//     The tile-0 workgroup of each slice also stores S = sum x_i and
//     C = sum x_i * phi_i over the slice's loaded channels.
//   kernel 2 (epilogue): y_j = s_j * (A_j + C) + z_j * S with A_j the sum of
//     the slices' partials, in slice order.
//
// y_j = sum_i x_i * (s_j * (code_ij + phi_i) + z_j) regroups exactly into
// s_j * (A_j + C) + z_j * S, so the per-output work is one FMA per fragment.
#include "decode.hpp"
#include "internal.h"

namespace grinqh {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kTileOut = kWave * 16;      // 1024 outputs: one word per lane

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

template <int P>
__global__ __launch_bounds__(kThreads) void gemv_partial_kernel(
    const void* __restrict__ x, int x_dtype, const float* __restrict__ theta,
    const uint32_t* __restrict__ planes, int d_in, int row_words, int chunk, int padded_out,
    float* __restrict__ partials, float* __restrict__ sc) {
    constexpr int b_max = 2 * P;
    __shared__ float red[kWaves][kTileOut];
    __shared__ float sc_red[2][kWaves];

    const int tile = blockIdx.x;
    const int split = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    float th[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < P; ++k) th[k] = theta[k];

    const int i0 = split * chunk;
    const int i1 = min(d_in, i0 + chunk);
    const int word = tile * kWave + lane;
    const bool has_word = word < row_words;

    float acc[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) acc[t] = 0.f;

    for (int i = i0 + wv; i < i1; i += kWaves) {
        const float xv = load_x(x, x_dtype, i);
        const int Pi = bits_of<P>(xv, th) >> 1;            // planes to read
        const uint32_t* row = planes + static_cast<size_t>(i) * P * row_words + word;
        for (int p = 0; p < Pi; ++p) {
            const uint32_t wd = has_word ? row[static_cast<size_t>(p) * row_words] : 0u;
            const float alpha = xv * plane_weight<P>(p);
#pragma unroll
            for (int t = 0; t < 16; ++t) acc[t] += alpha * static_cast<float>(fragment(wd, t));
        }
    }

#pragma unroll
    for (int t = 0; t < 16; ++t) red[wv][lane * 16 + t] = acc[t];
    __syncthreads();
    for (int o = threadIdx.x; o < kTileOut; o += kThreads) {
        float v = red[0][o];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) v += red[w][o];
        partials[static_cast<size_t>(split) * padded_out + tile * kTileOut + o] = v;
    }

    if (tile == 0) {
        // S and C over this slice: fixed-order tree, so runs are identical.
        float S = 0.f, C = 0.f;
        for (int i = i0 + threadIdx.x; i < i1; i += kThreads) {
            const float xv = load_x(x, x_dtype, i);
            const int b = bits_of<P>(xv, th);
            if (b > 0) {
                S += xv;
                C += xv * phi_of(b_max, b);
            }
        }
#pragma unroll
        for (int off = kWave / 2; off > 0; off >>= 1) {
            S += __shfl_xor(S, off);
            C += __shfl_xor(C, off);
        }
        if (lane == 0) {
            sc_red[0][wv] = S;
            sc_red[1][wv] = C;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            float s_tot = sc_red[0][0], c_tot = sc_red[1][0];
            for (int w = 1; w < kWaves; ++w) {
                s_tot += sc_red[0][w];
                c_tot += sc_red[1][w];
            }
            sc[2 * split] = s_tot;
            sc[2 * split + 1] = c_tot;
        }
    }
}

__global__ __launch_bounds__(kThreads) void gemv_epilogue_kernel(
    const float* __restrict__ partials, const float* __restrict__ sc, int n_splits,
    int padded_out, const uint16_t* __restrict__ s, const uint16_t* __restrict__ z,
    void* __restrict__ y, int y_dtype, int d_out) {
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= d_out) return;
    float A = 0.f, S = 0.f, C = 0.f;
    for (int sp = 0; sp < n_splits; ++sp) {
        A += partials[static_cast<size_t>(sp) * padded_out + j];
        S += sc[2 * sp];
        C += sc[2 * sp + 1];
    }
    const float r = f16_to_f32(s[j]) * (A + C) + f16_to_f32(z[j]) * S;
    if (y_dtype == GRINQH_F32)
        static_cast<float*>(y)[j] = r;
    else
        static_cast<uint16_t*>(y)[j] = f32_to_bf16_rne(r);
}

}  // namespace

GemvPlan plan_gemv(const grinqh_layout& L, const DeviceInfo& dev) {
    GemvPlan pl{};
    pl.tile_outputs = kTileOut;
    pl.n_tiles = (L.row_words + kWave - 1) / kWave;
    // Aim for about 4 workgroups per CU, with at least 16 channels per slice.
    const int want_wg = 4 * dev.cu_count;
    int n_splits = (want_wg + pl.n_tiles - 1) / pl.n_tiles;
    const int max_splits = (L.d_in + 15) / 16;
    if (n_splits > max_splits) n_splits = max_splits;
    if (n_splits < 1) n_splits = 1;
    pl.chunk = (L.d_in + n_splits - 1) / n_splits;
    pl.n_splits = (L.d_in + pl.chunk - 1) / pl.chunk;
    const size_t padded_out = static_cast<size_t>(pl.n_tiles) * kTileOut;
    pl.ws_partials = 0;
    pl.ws_counters = align_up(static_cast<size_t>(pl.n_splits) * padded_out * sizeof(float), 256);
    pl.ws_bytes = align_up(pl.ws_counters + static_cast<size_t>(pl.n_splits) * 2 * sizeof(float), 256);
    return pl;
}

hipError_t launch_gemv(const grinqh_layout& L, const GemvPlan& plan, const void* x,
                       int x_dtype, const float* theta, const uint32_t* planes,
                       const uint16_t* s, const uint16_t* z, void* y, int y_dtype,
                       void* workspace, hipStream_t stream) {
    char* ws = static_cast<char*>(workspace);
    float* partials = reinterpret_cast<float*>(ws + plan.ws_partials);
    float* sc = reinterpret_cast<float*>(ws + plan.ws_counters);
    const int padded_out = plan.n_tiles * kTileOut;
    dim3 grid(static_cast<unsigned>(plan.n_tiles), static_cast<unsigned>(plan.n_splits));
    dim3 block(kThreads);
    switch (L.n_planes) {
        case 1: gemv_partial_kernel<1><<<grid, block, 0, stream>>>(x, x_dtype, theta, planes, L.d_in, L.row_words, plan.chunk, padded_out, partials, sc); break;
        case 2: gemv_partial_kernel<2><<<grid, block, 0, stream>>>(x, x_dtype, theta, planes, L.d_in, L.row_words, plan.chunk, padded_out, partials, sc); break;
        case 3: gemv_partial_kernel<3><<<grid, block, 0, stream>>>(x, x_dtype, theta, planes, L.d_in, L.row_words, plan.chunk, padded_out, partials, sc); break;
        case 4: gemv_partial_kernel<4><<<grid, block, 0, stream>>>(x, x_dtype, theta, planes, L.d_in, L.row_words, plan.chunk, padded_out, partials, sc); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid2(static_cast<unsigned>((L.d_out + kThreads - 1) / kThreads));
    gemv_epilogue_kernel<<<grid2, block, 0, stream>>>(partials, sc, plan.n_splits, padded_out, s, z,
                                                      y, y_dtype, L.d_out);
    return hipGetLastError();
}

}  // namespace grinqh
