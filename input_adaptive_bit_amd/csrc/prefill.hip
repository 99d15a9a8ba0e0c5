// Prefill-stage dense GEMM (GRINQH note, overview: the prefill stage keeps
// every weight at b_max precision in ordinary matrix products; key design 3
// at b = b_max gives k = 0 and phi = 1/2 for every channel).
//
//   Y[m][j] = sum_i X[m][i] * (s_j * (q_ji + 1/2) + z_j)
//           = s_j * A[m][j] + (s_j / 2 + z_j) * S_m,
//   A[m][j] = sum_i X[m][i] * q_ji,   S_m = sum_i X[m][i].
//
// A is a dense contraction of the bf16 activations with integer codes
// (q <= 255, exact in bf16), so it runs on the bf16 matrix cores with fp32
// accumulation (v_mfma_f32_32x32x16_bf16); S comes from a row-sum pass.
//
// Tiling.  A workgroup computes a 128-token x 128-output tile of Y and walks
// the input channels in stages of 64.  Its four waves own 64 x 64 quarters,
// each four 32 x 32 MFMA tiles.  Per stage every thread prefetches into
// registers four 16-byte chunks of X and, for two adjacent channels, the P
// plane words of one 16-output word position; while the matrix cores work on
// the current stage it decodes the prefetched words (merge_codes, shared with
// the decode GEMV) into bf16 channel pairs and writes both operands into the
// other half of a double-buffered LDS tile.
//
// LDS tiles are [128 rows][64 channels] of bf16, rows of 8 16-byte chunks,
// with chunk c of row r stored at chunk c ^ (r & 7) ^ ((r >> 4) & 7): the
// MFMA operand reads (8 consecutive rows, one chunk) and the transposing
// code writes (rows 16 apart, one chunk pair) both spread over all banks.
#include "decode.hpp"
#include "device_common.hpp"
#include "internal.h"

namespace grinqh {
namespace {

constexpr int kTM = 128;                 // tokens per workgroup tile
constexpr int kTN = 128;                 // outputs per workgroup tile
constexpr int kTK = 64;                  // input channels per stage
constexpr int kPThreads = 256;           // 4 waves, 2 x 2 quarters of 64 x 64
constexpr uint32_t kPlaneOutOfRange = 0x80000000u;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct PrefillArgs {
    const uint16_t* x;       // bf16 [M][d_in]
    const uint32_t* planes;  // [d_in][P][row_words]
    const uint16_t* s;       // fp16 [d_out]
    const uint16_t* z;       // fp16 [d_out]
    const float* rowsum;     // [M]
    void* y;                 // [M][d_out]
    int M, d_in, d_out, row_words, y_dtype, tiles_m;
    uint32_t plane_bytes;
};

__device__ __forceinline__ int tile_off(int r, int c) {
    return r * kTK + ((c ^ (r & 7) ^ ((r >> 4) & 7)) << 3);
}

// One stage's operands in flight: X chunks of rows (t / 8) + 32 i at chunk
// t % 8, and the plane words of channels k0 + 2 (t / 8) + {0, 1} at word
// position n0 / 16 + t % 8.
template <int P>
struct Stage {
    u32x4 xr[4];
    uint32_t w[2][P];
};

template <int P>
__device__ __forceinline__ void load_stage(Stage<P>& st, const PrefillArgs& a, int m0, int n0, int k0,
                                           __amdgpu_buffer_rsrc_t prs, uint32_t row_bytes) {
    const int t = threadIdx.x;
    const int c = t & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + (t >> 3) + 32 * i;
        const int k = k0 + 8 * c;
        if (m < a.M && k < a.d_in)   // d_in % 8 == 0: a chunk is all in or all out
            st.xr[i] = *reinterpret_cast<const u32x4*>(a.x + static_cast<size_t>(m) * a.d_in + k);
        else
            st.xr[i] = u32x4{0u, 0u, 0u, 0u};
    }
    const int word = (n0 >> 4) + (t & 7);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int ch = k0 + 2 * (t >> 3) + h;
        const bool ok = ch < a.d_in && word < a.row_words;
        // inside channel ch's P plane rows, so a plane offset keeps it in the buffer
        const uint32_t off = ok ? (static_cast<uint32_t>(ch) * P * static_cast<uint32_t>(a.row_words) +
                                   static_cast<uint32_t>(word)) * 4u
                                : kPlaneOutOfRange;
#pragma unroll
        for (int p = 0; p < P; ++p)
            st.w[h][p] = __builtin_amdgcn_raw_buffer_load_b32(prs, off, static_cast<uint32_t>(p) * row_bytes, 0);
    }
}

// Writes a prefetched stage into one LDS buffer: X chunks as they are, and
// the codes of both channels as bf16 pairs (channel 2 (t / 8) in the low
// half) at every output of the word position.  Code bytes carry the scale
// merge_codes leaves in byte lane k, undone in the epilogue.
template <int P>
__device__ __forceinline__ void store_stage(const Stage<P>& st, uint16_t* xs, uint16_t* ws) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4*>(xs + tile_off((t >> 3) + 32 * i, t & 7)) = st.xr[i];
    uint32_t E0[4], E1[4];
    merge_codes<P>(st.w[0], E0);
    merge_codes<P>(st.w[1], E1);
    // hide the known-zero bits so that each byte becomes one v_cvt_f32_ubyte
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        asm("" : "+v"(E0[k]));
        asm("" : "+v"(E1[k]));
    }
    const int cp = t >> 3;
    const int chunk = cp >> 2;
    const int elem = (2 * cp) & 7;
    const int row0 = 16 * (t & 7);
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float v0 = byte_f32(E0[k], b), v1 = byte_f32(E1[k], b);
            // integers <= 255: the bf16 is the upper half of the fp32, exactly
            const uint32_t pair = __builtin_amdgcn_perm(__float_as_uint(v1), __float_as_uint(v0), 0x07060302u);
            *reinterpret_cast<uint32_t*>(ws + tile_off(row0 + 4 * b + k, chunk) + elem) = pair;
        }
}

__device__ __forceinline__ void mma_stage(f32x16 (&acc)[2][2], const uint16_t* xs, const uint16_t* ws, int wm,
                                          int wn, int lane) {
#pragma unroll
    for (int kk = 0; kk < kTK / 16; ++kk) {
        const int c = 2 * kk + (lane >> 5);
        bf16x8 av[2], bv[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            av[i] = *reinterpret_cast<const bf16x8*>(xs + tile_off(64 * wm + 32 * i + (lane & 31), c));
            bv[i] = *reinterpret_cast<const bf16x8*>(ws + tile_off(64 * wn + 32 * i + (lane & 31), c));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
}

template <int P>
__global__ __launch_bounds__(kPThreads, 2) void prefill_kernel(PrefillArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][kTM * kTK];
    __shared__ __attribute__((aligned(16))) uint16_t wsh[2][kTN * kTK];
    __shared__ float srow[kTM];
    const int id = static_cast<int>(blockIdx.x);
    const int m0 = (id % a.tiles_m) * kTM;
    const int n0 = (id / a.tiles_m) * kTN;
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int wm = wv >> 1, wn = wv & 1;
    const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(a.planes), static_cast<short>(0), static_cast<int>(a.plane_bytes), 0x00020000);
    const uint32_t row_bytes = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a.row_words) * 4u);

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int n_stages = (a.d_in + kTK - 1) / kTK;
    Stage<P> st;
    load_stage<P>(st, a, m0, n0, 0, prs, row_bytes);
    store_stage<P>(st, xs[0], wsh[0]);
    __syncthreads();
    for (int s = 0; s < n_stages; ++s) {
        const int cur = s & 1;
        const bool more = s + 1 < n_stages;
        if (more) load_stage<P>(st, a, m0, n0, (s + 1) * kTK, prs, row_bytes);
        mma_stage(acc, xs[cur], wsh[cur], wm, wn, lane);
        if (more) store_stage<P>(st, xs[cur ^ 1], wsh[cur ^ 1]);
        __syncthreads();
    }

    if (threadIdx.x < kTM) {
        const int m = m0 + static_cast<int>(threadIdx.x);
        srow[threadIdx.x] = m < a.M ? a.rowsum[m] : 0.f;
    }
    __syncthreads();

    // y = s_j * u_j * acc + (s_j / 2 + z_j) * S_m, u_j undoing the byte scale
    // of output j's lane in merge_codes (outputs 4b + k sit in byte lane k)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int n = n0 + 64 * wn + 32 * j + (lane & 31);
        const bool n_ok = n < a.d_out;
        const int nc = n_ok ? n : a.d_out - 1;
        const float sj = f16_to_f32(a.s[nc]);
        const float zj = f16_to_f32(a.z[nc]);
        const float mul = sj * code_unscale<P>(lane & 3);
        const float add = 0.5f * sj + zj;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ml = 64 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int m = m0 + ml;
                if (!n_ok || m >= a.M) continue;
                const float yv = mul * acc[i][j][r] + add * srow[ml];
                const size_t o = static_cast<size_t>(m) * a.d_out + n;
                if (a.y_dtype == GRINQH_F32)
                    static_cast<float*>(a.y)[o] = yv;
                else
                    static_cast<uint16_t*>(a.y)[o] = f32_to_bf16_rne(yv);
            }
    }
}

// S_m = sum_i X[m][i] in fp32, one workgroup per token row, fixed order.
__global__ __launch_bounds__(256) void rowsum_kernel(const uint16_t* x, int d_in, float* out) {
    __shared__ float red[256];
    const uint16_t* row = x + static_cast<size_t>(blockIdx.x) * d_in;
    float acc = 0.f;
    for (int c = threadIdx.x; c < d_in / 8; c += 256) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(row + 8 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc += __uint_as_float(v[e] << 16);
            acc += __uint_as_float(v[e] & 0xFFFF0000u);
        }
    }
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if (static_cast<int>(threadIdx.x) < h) red[threadIdx.x] += red[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[blockIdx.x] = red[0];
}

template <int P>
hipError_t launch_p(const PrefillArgs& a, int tiles, hipStream_t stream) {
    prefill_kernel<P><<<dim3(static_cast<unsigned>(tiles)), dim3(kPThreads), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

size_t prefill_workspace_bytes(int M) {
    return M <= 0 ? 0 : (static_cast<size_t>(M) * sizeof(float) + 255) / 256 * 256;
}

long prefill_tiles(const grinqh_layout& L, int M) {
    return static_cast<long>((M + kTM - 1) / kTM) * ((L.d_out + kTN - 1) / kTN);
}

hipError_t launch_prefill(const grinqh_layout& L, const uint16_t* x, int M, const uint32_t* planes,
                          const uint16_t* s, const uint16_t* z, void* y, int y_dtype, float* rowsum,
                          hipStream_t stream) {
    rowsum_kernel<<<dim3(static_cast<unsigned>(M)), dim3(256), 0, stream>>>(x, L.d_in, rowsum);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    PrefillArgs a{};
    a.x = x;
    a.planes = planes;
    a.s = s;
    a.z = z;
    a.rowsum = rowsum;
    a.y = y;
    a.M = M;
    a.d_in = L.d_in;
    a.d_out = L.d_out;
    a.row_words = L.row_words;
    a.y_dtype = y_dtype;
    a.tiles_m = (M + kTM - 1) / kTM;
    a.plane_bytes = static_cast<uint32_t>(static_cast<size_t>(L.d_in) * L.n_planes * L.row_words * 4u);
    const int tiles = static_cast<int>(prefill_tiles(L, M));
    switch (L.n_planes) {
        case 1: return launch_p<1>(a, tiles, stream);
        case 2: return launch_p<2>(a, tiles, stream);
        case 3: return launch_p<3>(a, tiles, stream);
        case 4: return launch_p<4>(a, tiles, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace grinqh
