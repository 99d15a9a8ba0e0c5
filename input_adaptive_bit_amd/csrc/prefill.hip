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
// Tiling.  A workgroup of eight waves computes a TM x TN (tokens x outputs)
// tile of Y -- 256 x 256 or 256 x 128 with one workgroup per CU, 128 x 128
// with two -- and walks the input channels in stages of 64.  With at least
// two waves per SIMD, one wave's waits are covered by another's matrix work.
// The waves form a grid over the tile, each owning a block of 32 x 32 MFMA
// tiles (128 x 64, 64 x 64 and 32 x 64 tokens x outputs).  Every thread
// holds, two stages ahead, 16-byte chunks of X and, for one channel, 1, 2 or
// 4 plane words of consecutive word positions (one load per plane).  While
// the matrix cores work on stage s, the waves decode stage s + 1
// (merge_codes, shared with the decode GEMV, then one byte conversion per
// code, whose fp32 upper half is the code's bf16) into the other half of a
// double-buffered LDS tile: each MFMA is followed, in a fixed order, by its
// share of that work and of the loads.
//
// The X tile is [tokens][64 channels] of bf16 (rows of 8 16-byte chunks,
// permuted by tile_off); the code tile is [64 channels][TN outputs] (chunks
// permuted by code_off), written 8 outputs at a time and read into the B
// operand with transposing LDS reads (ds_read_b64_tr_b16).
#include "decode.hpp"
#include "device_common.hpp"
#include "internal.h"

namespace grinqh {
namespace {

constexpr int kTK = 64;                  // input channels per stage
// Eight waves per workgroup, at least two per SIMD, forming a WM x WN grid
// over the tile with WN = TN / 64: each wave owns TM / WM tokens x 64 outputs.
constexpr int kPWaves = 8;
__host__ __device__ constexpr int tile_wn(int TM, int TN) { return TN / 64; }
__host__ __device__ constexpr int tile_wm(int TM, int TN) { return kPWaves / tile_wn(TM, TN); }
// 32 x 32 MFMA tiles per wave along the tokens and the outputs
__host__ __device__ constexpr int tile_fm(int TM, int TN) { return TM / tile_wm(TM, TN) / 32; }
__host__ __device__ constexpr int tile_fn(int TM, int TN) { return TN / tile_wn(TM, TN) / 32; }
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
    int vec_y;
    int xcd_group;           // tile columns a multiple of 8: map columns to XCDs               // y 16-byte aligned and d_out a multiple of 16 bytes' worth of outputs
    uint32_t plane_bytes;
};

// Element offset of (row r, channel chunk c) in the [tokens][64] bf16 X
// tile.  Rows are 128 bytes; chunk c of row r sits at c ^ (r % 8) ^ (bit 3
// of r), so that 8 consecutive rows (an MFMA operand read, 8 lanes) fall on
// distinct chunks and 16 consecutive rows on distinct 16-byte bank groups
// of a 256-byte span.
__device__ __forceinline__ int tile_off(int r, int c) {
    return r * kTK + ((c ^ (r & 7) ^ ((r >> 3) & 1)) << 3);
}

// Element offset of (channel k, output n) in the [64][TN] bf16 code tile: one
// row per channel (a multiple of 256 bytes), outputs in 16-byte chunks.  With
// r = k % 4, chunk c sits at c ^ 4r ^ e, e = (bit 3 of c) + 2 par and par =
// parity of r ^ (bit 4 of c).  Both access patterns then touch every bank
// once per 128 bytes: the transposing reads of a 16-lane group (4 channels x
// 16 outputs) and the 16-byte code writes of 8 lanes (the eight threads of
// one channel).
template <int TN>
__device__ __forceinline__ int code_off(int k, int n) {
    const int c = n >> 3, r = k & 3;
    const int par = (r ^ (r >> 1) ^ (c >> 4)) & 1;
    const int e = ((c >> 3) & 1) | (par << 1);
    return k * TN + ((c ^ (r << 2) ^ e) << 3) + (n & 7);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// 4 consecutive channels for one output per lane (ds_read_b64_tr_b16): in each
// 16-lane group, lane i supplies the address of channel k0 + i / 4, outputs
// n0 + 4 (i % 4) .. + 3, and receives channels k0 .. k0 + 3 of output n0 + i.
template <int TN>
__device__ __forceinline__ s16x4 read_codes_tr(const uint16_t* ws, int k0, int n0, int i) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(ws + code_off<TN>(k0 + (i >> 2), n0 + 4 * (i & 3))));
}

// One stage's operands in flight.  X: chunk item i = t + NT u is row i / 8,
// chunk i % 8.  Planes: with TPC = NT / 64 threads per channel, thread t takes
// channel k0 + t / TPC and the WPT word positions from
// (n0 / 16) + (t % TPC) WPT, one 4 WPT-byte load per plane.
template <int P, int TM, int TN>
struct Stage {
    static constexpr int NT = 64 * kPWaves;             // threads
    static constexpr int WN = tile_wn(TM, TN), WM = tile_wm(TM, TN);  // wave grid
    static constexpr int FM = tile_fm(TM, TN), FN = tile_fn(TM, TN);
    static constexpr int TPC = NT / kTK;                // threads per input channel
    static constexpr int XI = TM * 8 / NT;              // X chunks per thread
    static constexpr int WPT = TN / 16 / TPC;           // plane words per thread and plane
    u32x4 xr[XI];
    uint32_t pw[P][WPT];
};

template <int P, int TM, int TN>
struct Merged {
    uint32_t E[Stage<P, TM, TN>::WPT][4];   // merge_codes words of each word position
};

template <int P, int TM, int TN, int L>
__device__ __forceinline__ void load_unit(Stage<P, TM, TN>& st, const PrefillArgs& a, int n0, int k0,
                                          __amdgpu_buffer_rsrc_t xrs, __amdgpu_buffer_rsrc_t prs,
                                          uint32_t row_bytes) {
    using St = Stage<P, TM, TN>;
    const int t = threadIdx.x;
    if constexpr (L < St::XI) {
        const int i = t + St::NT * L;
        const int k = k0 + 8 * (i & 7);
        // rows past M lie past the resource; d_in % 8 == 0, so a chunk is
        // all in or all out of the row
        const uint32_t off = k < a.d_in ? static_cast<uint32_t>((i >> 3) * a.d_in + k) * 2u : kPlaneOutOfRange;
        st.xr[L] = __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0);
    } else {
        constexpr int p = L - St::XI;
        const int ch = k0 + t / St::TPC;
        const int word = (n0 >> 4) + (t % St::TPC) * St::WPT;
        // row_words is a multiple of 4, so the WPT words are all in or all out;
        // inside channel ch's plane rows, a plane offset keeps it in the buffer
        const bool ok = ch < a.d_in && word < a.row_words;
        const uint32_t off = ok ? (static_cast<uint32_t>(ch) * P * static_cast<uint32_t>(a.row_words) +
                                   static_cast<uint32_t>(word)) * 4u
                                : kPlaneOutOfRange;
        if constexpr (St::WPT == 4) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(prs, off, static_cast<uint32_t>(p) * row_bytes, 0);
            st.pw[p][0] = v.x; st.pw[p][1] = v.y; st.pw[p][2] = v.z; st.pw[p][3] = v.w;
        } else if constexpr (St::WPT == 2) {
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(prs, off, static_cast<uint32_t>(p) * row_bytes, 0);
            st.pw[p][0] = v.x; st.pw[p][1] = v.y;
        } else {
            static_assert(St::WPT == 1, "one, two or four plane words per thread");
            st.pw[p][0] = __builtin_amdgcn_raw_buffer_load_b32(prs, off, static_cast<uint32_t>(p) * row_bytes, 0);
        }
    }
}

template <int P, int TM, int TN, int L0, int L1>
__device__ __forceinline__ void load_units(Stage<P, TM, TN>& st, const PrefillArgs& a, int n0, int k0,
                                           __amdgpu_buffer_rsrc_t xrs, __amdgpu_buffer_rsrc_t prs,
                                           uint32_t row_bytes) {
    if constexpr (L0 < L1) {
        load_unit<P, TM, TN, L0>(st, a, n0, k0, xrs, prs, row_bytes);
        load_units<P, TM, TN, L0 + 1, L1>(st, a, n0, k0, xrs, prs, row_bytes);
    }
}

// Byte codes of word position V (merge_codes: byte b of word k is the code
// of output 4b + k times the byte lane's power of two, undone in the
// epilogue).
template <int P, int TM, int TN, int V>
__device__ __forceinline__ void merge_unit(const Stage<P, TM, TN>& st, Merged<P, TM, TN>& mg) {
    uint32_t w[P];
#pragma unroll
    for (int p = 0; p < P; ++p) w[p] = st.pw[p][V];
    merge_codes<P>(w, mg.E[V]);
    // hide the known-zero bits so that each byte becomes one v_cvt_f32_ubyte
#pragma unroll
    for (int k = 0; k < 4; ++k) asm("" : "+v"(mg.E[V][k]));
}

// Code unit U: half h of word position v (outputs 8h .. 8h + 7 of the
// word), this thread's channel, one 16-byte write of four bf16 pairs (an
// integer up to 255 is the upper half of its fp32, exactly).
template <int P, int TM, int TN, int U>
__device__ __forceinline__ void code_unit(const Merged<P, TM, TN>& mg, uint16_t* ws) {
    constexpr int WPT = Stage<P, TM, TN>::WPT;
    constexpr int v = U / 2, h = U % 2;
    const int t = threadIdx.x;
    uint32_t d[4];
#pragma unroll
    for (int e = 0; e < 2; ++e)          // byte b = 2h + e: outputs 4b .. 4b + 3
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) { // outputs 4b + 2pr, 4b + 2pr + 1
            const float lo = byte_f32(mg.E[v][2 * pr], 2 * h + e);
            const float hi = byte_f32(mg.E[v][2 * pr + 1], 2 * h + e);
            d[2 * e + pr] = __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
        }
    constexpr int TPC = Stage<P, TM, TN>::TPC;
    const int n = 16 * ((t % TPC) * WPT + v) + 8 * h;
    *reinterpret_cast<u32x4*>(ws + code_off<TN>(t / TPC, n)) = u32x4{d[0], d[1], d[2], d[3]};
}

template <int P, int TM, int TN, int U0, int U1>
__device__ __forceinline__ void code_units(const Merged<P, TM, TN>& mg, uint16_t* ws) {
    if constexpr (U0 < U1) {
        code_unit<P, TM, TN, U0>(mg, ws);
        code_units<P, TM, TN, U0 + 1, U1>(mg, ws);
    }
}

template <int P, int TM, int TN, int V0, int V1>
__device__ __forceinline__ void merge_units(const Stage<P, TM, TN>& st, Merged<P, TM, TN>& mg) {
    if constexpr (V0 < V1) {
        merge_unit<P, TM, TN, V0>(st, mg);
        merge_units<P, TM, TN, V0 + 1, V1>(st, mg);
    }
}

template <int P, int TM, int TN, int X0, int X1>
__device__ __forceinline__ void x_units(const Stage<P, TM, TN>& st, uint16_t* xs) {
    if constexpr (X0 < X1) {
        const int i = static_cast<int>(threadIdx.x) + Stage<P, TM, TN>::NT * X0;
        *reinterpret_cast<u32x4*>(xs + tile_off(i >> 3, i & 7)) = st.xr[X0];
        x_units<P, TM, TN, X0 + 1, X1>(st, xs);
    }
}

// One wave's MFMA operands of a k-step: FM row fragments of X and FN of the
// codes, 8 consecutive channels per lane.
template <int FM, int FN>
struct Frag {
    bf16x8 a[FM];      // one set, each reloaded for the next k-step after its last use
    bf16x8 b[2][FN];   // two sets, by k-step parity
};

// Lane l takes channels 16 kk + 8 (l / 32) .. + 7 of token row + l % 32.
__device__ __forceinline__ bf16x8 read_a(const uint16_t* xs, int kk, int row, int lane) {
    return *reinterpret_cast<const bf16x8*>(xs + tile_off(row + (lane & 31), 2 * kk + (lane >> 5)));
}

// Lane l takes channels 16 kk + 8 (l / 32) .. + 7 of output col + l % 32.
template <int TN>
__device__ __forceinline__ bf16x8 read_b(const uint16_t* ws, int kk, int col, int lane) {
    const int k0 = 16 * kk + 8 * (lane >> 5);
    const int n0 = col + 16 * ((lane >> 4) & 1);
    const s16x4 r0 = read_codes_tr<TN>(ws, k0, n0, lane & 15);
    const s16x4 r1 = read_codes_tr<TN>(ws, k0 + 4, n0, lane & 15);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int FM, int FN, int TN>
__device__ __forceinline__ void read_frags(Frag<FM, FN>& f, int set, const uint16_t* xs, const uint16_t* ws,
                                           int kk, int row_a, int row_b, int lane) {
#pragma unroll
    for (int i = 0; i < FM; ++i) f.a[i] = read_a(xs, kk, row_a + 32 * i, lane);
#pragma unroll
    for (int j = 0; j < FN; ++j) f.b[set][j] = read_b<TN>(ws, kk, row_b + 32 * j, lane);
}

// One stage as a fixed sequence (scheduling fences between the steps): MFMA
// G of the current stage, then its share of the loads of the stage after next
// (phase 0: spread over the stage; phases 1 and 2: in one half), of the merges and code writes of the next stage and
// of its X writes.  Each A fragment is reloaded for the next k-step right
// after its last MFMA of this one; halfway through a k-step the next k-step's
// B fragments are read into the other B set.  Two MFMAs before the end come
// the stage barrier and the next stage's k-step 0 operand reads.
template <int G, int P, int TM, int TN, int PH>
__device__ __forceinline__ void body(f32x16 (&acc)[tile_fm(TM, TN)][tile_fn(TM, TN)],
                                     Frag<tile_fm(TM, TN), tile_fn(TM, TN)>& fr,
                                     const uint16_t* xs, const uint16_t* ws, const Stage<P, TM, TN>& cur,
                                     Stage<P, TM, TN>& nxt, Merged<P, TM, TN>& mg, uint16_t* xs_next,
                                     uint16_t* ws_next, const PrefillArgs& a, int n0, int k_load,
                                     __amdgpu_buffer_rsrc_t xrs, __amdgpu_buffer_rsrc_t prs, uint32_t row_bytes,
                                     int row_a, int row_b, int lane) {
    using St = Stage<P, TM, TN>;
    constexpr int FM = St::FM, FN = St::FN, PER = FM * FN, NM = PER * (kTK / 16);
    if constexpr (G < NM) {
        constexpr int kk = G / PER, mi = G % PER, i = mi / FN, j = mi % FN;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.a[i], fr.b[kk & 1][j], acc[i][j], 0, 0, 0);
        if constexpr (kk + 1 < kTK / 16) {
            if constexpr (j == FN - 1) fr.a[i] = read_a(xs, kk + 1, row_a + 32 * i, lane);
            if constexpr (mi == PER / 2) {
#pragma unroll
                for (int jj = 0; jj < FN; ++jj) fr.b[(kk + 1) & 1][jj] = read_b<TN>(ws, kk + 1, row_b + 32 * jj, lane);
            }
        }
        constexpr int NL = St::XI + P, WPT = St::WPT, NU = WPT * 2, NW = NM - 2;
        if constexpr (PH == 0) {
            // loads spread over the first three quarters of a stage (the first half
            // at 128 x 128), so the last has a quarter (a half) of one to arrive
            constexpr int NH = TM == 256 ? 3 * NM / 4 : NM / 2;
            if constexpr (G < NH) load_units<P, TM, TN, G * NL / NH, (G + 1) * NL / NH>(nxt, a, n0, k_load, xrs, prs, row_bytes);
            // merges in the first WPT slots, code and X writes over the rest but
            // the last two, which belong to the barrier and the next stage's
            // first operand reads
            static_assert(NW - WPT >= NU && NW >= St::XI, "a write slot for every unit");
            if constexpr (G < WPT) merge_units<P, TM, TN, G, G + 1>(cur, mg);
            if constexpr (G >= WPT && G < NW)
                code_units<P, TM, TN, (G - WPT) * NU / (NW - WPT), (G - WPT + 1) * NU / (NW - WPT)>(mg, ws_next);
            if constexpr (G < NW) x_units<P, TM, TN, G * St::XI / NW, (G + 1) * St::XI / NW>(cur, xs_next);
        } else {
            // The two waves of a SIMD take turns: phase 1 does all its loads and
            // decode in the first half of the stage, phase 2 in the second, so
            // each wave's plain run of MFMAs covers the other's vector work.
            constexpr int W0 = PH == 1 ? 0 : NM / 2, W1 = PH == 1 ? NM / 2 : NW, NS = W1 - W0;
            static_assert(NS - WPT >= NU && NS >= 2, "a work slot for every unit");
            if constexpr (G >= W0 && G < W1) {
                constexpr int g = G - W0, NLH = NS / 2;
                if constexpr (g < NLH) load_units<P, TM, TN, g * NL / NLH, (g + 1) * NL / NLH>(nxt, a, n0, k_load, xrs, prs, row_bytes);
                if constexpr (g < WPT) merge_units<P, TM, TN, g, g + 1>(cur, mg);
                if constexpr (g >= WPT)
                    code_units<P, TM, TN, (g - WPT) * NU / (NS - WPT), (g - WPT + 1) * NU / (NS - WPT)>(mg, ws_next);
                x_units<P, TM, TN, g * St::XI / NS, (g + 1) * St::XI / NS>(cur, xs_next);
            }
        }
        // Two MFMAs before the end every read of this stage's tiles has been
        // consumed and every write of the next stage's has been issued: the
        // barrier goes here, and the next stage's k-step 0 operands are read
        // while the last two MFMAs run (A row block FM - 1 after its last use).
        if constexpr (G == NW) {
            __syncthreads();
#pragma unroll
            for (int ii = 0; ii < FM - 1; ++ii) fr.a[ii] = read_a(xs_next, 0, row_a + 32 * ii, lane);
#pragma unroll
            for (int jj = 0; jj < FN; ++jj) fr.b[0][jj] = read_b<TN>(ws_next, 0, row_b + 32 * jj, lane);
        }
        if constexpr (G == NM - 1) fr.a[FM - 1] = read_a(xs_next, 0, row_a + 32 * (FM - 1), lane);
        __builtin_amdgcn_sched_barrier(0);
        body<G + 1, P, TM, TN, PH>(acc, fr, xs, ws, cur, nxt, mg, xs_next, ws_next, a, n0, k_load, xrs, prs, row_bytes,
                               row_a, row_b, lane);
    }
}

// The last stage's matrix work alone.
template <int FM, int FN, int TN>
__device__ __forceinline__ void mma_stage(f32x16 (&acc)[FM][FN], const uint16_t* xs, const uint16_t* ws,
                                          int row_a, int row_b, int lane) {
#pragma unroll
    for (int kk = 0; kk < kTK / 16; ++kk) {
        Frag<FM, FN> f;
        read_frags<FM, FN, TN>(f, 0, xs, ws, kk, row_a, row_b, lane);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[0][j], acc[i][j], 0, 0, 0);
    }
}

// One output in fp32, the same operations on either store path.
__device__ __forceinline__ float y_value(float mul, float acc, float add, float srow) {
    return __builtin_fmaf(mul, acc, add * srow);
}

// fp32 -> bf16, round to nearest even (one hardware conversion on gfx950).
__device__ __forceinline__ uint16_t y_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

template <int P, int TM, int TN>
__global__ __launch_bounds__(64 * kPWaves, (TM * TN > 128 * 128 ? 1 : 2)) void prefill_kernel(
    PrefillArgs a) {
    using St = Stage<P, TM, TN>;
    constexpr int FM = St::FM, FN = St::FN;
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][TM * kTK];
    __shared__ __attribute__((aligned(16))) uint16_t wsh[2][TN * kTK];
    __shared__ float srow[TM];
    const int id = static_cast<int>(blockIdx.x);
    // Workgroups go to the 8 XCDs in turn (id % 8).  When the tile columns
    // split evenly, XCD x takes the columns x, x + 8, ... whole, so the
    // workgroups that share an XCD's L2 share plane columns and X rows.
    int tm, tn;
    if (a.xcd_group) {
        const int k = id >> 3;
        tm = k % a.tiles_m;
        tn = (id & 7) + 8 * (k / a.tiles_m);
    } else {
        tm = id % a.tiles_m;
        tn = id / a.tiles_m;
    }
    const int m0 = tm * TM;
    const int n0 = tn * TN;
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int row_a = (wv / St::WN) * (TM / St::WM);   // this wave's first token row in the tile
    const int row_b = (wv % St::WN) * (TN / St::WN);   // and first output
    const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(a.planes), static_cast<short>(0), static_cast<int>(a.plane_bytes), 0x00020000);
    const uint32_t row_bytes = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a.row_words) * 4u);
    const int rows = min(TM, a.M - m0);
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.x + static_cast<size_t>(m0) * a.d_in), static_cast<short>(0),
        rows * a.d_in * 2, 0x00020000);

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int n_stages = (a.d_in + kTK - 1) / kTK;
    // Stage s is computed from LDS while stage s + 1, loaded one iteration
    // earlier, is decoded into the other LDS buffer and stage s + 2 is
    // loaded; stages past the last load nothing (out-of-range offsets).
    St sa, sb;
    Merged<P, TM, TN> mg;
    Frag<FM, FN> fr;
    load_units<P, TM, TN, 0, St::XI + P>(sa, a, n0, 0, xrs, prs, row_bytes);
    merge_units<P, TM, TN, 0, St::WPT>(sa, mg);
    code_units<P, TM, TN, 0, St::WPT * 2>(mg, wsh[0]);
    x_units<P, TM, TN, 0, St::XI>(sa, xs[0]);
    load_units<P, TM, TN, 0, St::XI + P>(sa, a, n0, kTK, xrs, prs, row_bytes);
    __syncthreads();
    // Each body ends with the barrier and the next stage's k-step 0 operands
    // in registers; the last one reads a stage past the end (zeros), unused.
    read_frags<FM, FN, TN>(fr, 0, xs[0], wsh[0], 0, row_a, row_b, lane);
    int s = 0;
    // Waves w and w + 4 share a SIMD: with at least 16 MFMAs per stage they take turns (phases 1 and 2).
    constexpr bool kTurns = FM * FN * (kTK / 16) >= 16;
    if (kTurns && wv < 4) {
        for (; s + 1 < n_stages; s += 2) {
            body<0, P, TM, TN, kTurns ? 1 : 0>(acc, fr, xs[0], wsh[0], sa, sb, mg, xs[1], wsh[1], a, n0, (s + 2) * kTK,
                                               xrs, prs, row_bytes, row_a, row_b, lane);
            body<0, P, TM, TN, kTurns ? 1 : 0>(acc, fr, xs[1], wsh[1], sb, sa, mg, xs[0], wsh[0], a, n0, (s + 3) * kTK,
                                               xrs, prs, row_bytes, row_a, row_b, lane);
        }
    } else {
        for (; s + 1 < n_stages; s += 2) {
            body<0, P, TM, TN, kTurns ? 2 : 0>(acc, fr, xs[0], wsh[0], sa, sb, mg, xs[1], wsh[1], a, n0, (s + 2) * kTK,
                                               xrs, prs, row_bytes, row_a, row_b, lane);
            body<0, P, TM, TN, kTurns ? 2 : 0>(acc, fr, xs[1], wsh[1], sb, sa, mg, xs[0], wsh[0], a, n0, (s + 3) * kTK,
                                               xrs, prs, row_bytes, row_a, row_b, lane);
        }
    }
    if (s < n_stages) mma_stage<FM, FN, TN>(acc, xs[0], wsh[0], row_a, row_b, lane);

    for (int r = threadIdx.x; r < TM; r += St::NT) {
        const int m = m0 + r;
        srow[r] = m < a.M ? a.rowsum[m] : 0.f;
    }
    __syncthreads();

    // y = s_j * u_j * acc + (s_j / 2 + z_j) * S_m, u_j undoing the byte scale
    // of output j's lane in merge_codes (outputs 4b + k sit in byte lane k)
    if (a.vec_y) {
        // Through LDS, so that y leaves in 128-byte row segments: each wave
        // stages its block of y 32 token rows at a time (bf16: 32 x 64; fp32:
        // 32 x 32 per pass) in the X tile's space, which the barrier above has
        // freed, and reads it back 16 bytes per lane.
        static_assert(FN * 32 == 64, "each wave owns 64 outputs");
        float mul[FN], add[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int nc = min(n0 + row_b + 32 * j + (lane & 31), a.d_out - 1);
            const float sj = f16_to_f32(a.s[nc]);
            mul[j] = sj * code_unscale<P>(lane & 3);
            add[j] = 0.5f * sj + f16_to_f32(a.z[nc]);
        }
        const int nb = n0 + row_b;   // the wave's first output
        if (a.y_dtype == GRINQH_F32) {
            float* stg = reinterpret_cast<float*>(&xs[0][0]) + wv * 1024;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int mb = row_a + 32 * i;   // the block's first token row in the tile
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int rl = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                        stg[rl * 32 + (lane & 31)] = y_value(mul[j], acc[i][j][r], add[j], srow[mb + rl]);
                    }
                    __syncthreads();
#pragma unroll
                    for (int q = 0; q < 4; ++q) {   // rows (lane / 8) + 8q, outputs 4 (lane % 8) .. + 3
                        const int rl = (lane >> 3) + 8 * q, cl = 4 * (lane & 7), c = 32 * j + cl;
                        const int m = m0 + mb + rl;
                        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + rl * 32 + cl);
                        if (m < a.M && nb + c < a.d_out)
                            *reinterpret_cast<u32x4*>(static_cast<float*>(a.y) + static_cast<size_t>(m) * a.d_out +
                                                      nb + c) = v;
                    }
                    __syncthreads();
                }
        } else {
            uint16_t* stg = reinterpret_cast<uint16_t*>(&xs[0][0]) + wv * 2048;
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int mb = row_a + 32 * i;
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int rl = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                        stg[rl * 64 + 32 * j + (lane & 31)] =
                            y_bf16(y_value(mul[j], acc[i][j][r], add[j], srow[mb + rl]));
                    }
                __syncthreads();
#pragma unroll
                for (int q = 0; q < 4; ++q) {   // rows (lane / 8) + 8q, outputs 8 (lane % 8) .. + 7
                    const int rl = (lane >> 3) + 8 * q, c = 8 * (lane & 7);
                    const int m = m0 + mb + rl;
                    const u32x4 w = *reinterpret_cast<const u32x4*>(stg + rl * 64 + c);
                    if (m < a.M && nb + c < a.d_out)
                        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.y) + static_cast<size_t>(m) * a.d_out +
                                                  nb + c) = w;
                }
                __syncthreads();
            }
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int n = n0 + row_b + 32 * j + (lane & 31);
        const bool n_ok = n < a.d_out;
        const int nc = n_ok ? n : a.d_out - 1;
        const float sj = f16_to_f32(a.s[nc]);
        const float zj = f16_to_f32(a.z[nc]);
        const float mul = sj * code_unscale<P>(lane & 3);
        const float add = 0.5f * sj + zj;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ml = row_a + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int m = m0 + ml;
                if (!n_ok || m >= a.M) continue;
                const float yv = y_value(mul, acc[i][j][r], add, srow[ml]);
                const size_t o = static_cast<size_t>(m) * a.d_out + n;
                if (a.y_dtype == GRINQH_F32)
                    static_cast<float*>(a.y)[o] = yv;
                else
                    static_cast<uint16_t*>(a.y)[o] = y_bf16(yv);
            }
    }
}

// S_m = sum_i X[m][i] in fp32: one wave per token row, in a fixed order
// (each lane adds its 16-byte chunks lane, lane + 64, ... in turn, then the
// 64 lane sums are added by xor butterfly, and lane 0's total is stored).
__global__ __launch_bounds__(256) void rowsum_kernel(const uint16_t* x, int M, int d_in, float* out) {
    const int row = static_cast<int>(blockIdx.x) * 4 + static_cast<int>(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= M) return;   // whole waves
    const uint16_t* xr = x + static_cast<size_t>(row) * d_in;
    float acc = 0.f;
#pragma unroll 4
    for (int c = lane; c < d_in / 8; c += 64) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(xr + 8 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc += __uint_as_float(v[e] << 16);
            acc += __uint_as_float(v[e] & 0xFFFF0000u);
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) out[row] = acc;
}

template <int P, int TM, int TN>
hipError_t launch_t(PrefillArgs a, hipStream_t stream) {
    a.tiles_m = (a.M + TM - 1) / TM;
    const int tiles_n = (a.d_out + TN - 1) / TN;
    a.xcd_group = tiles_n % 8 == 0;
    const long tiles = static_cast<long>(a.tiles_m) * tiles_n;
    prefill_kernel<P, TM, TN><<<dim3(static_cast<unsigned>(tiles)), dim3(Stage<P, TM, TN>::NT), 0, stream>>>(a);
    return hipGetLastError();
}

template <int P>
hipError_t launch_p(const PrefillArgs& a, int tile, hipStream_t stream) {
    if (tile == 2) return launch_t<P, 256, 256>(a, stream);
    if (tile == 1) return launch_t<P, 256, 128>(a, stream);
    return launch_t<P, 128, 128>(a, stream);
}

long tiles_of(int M, int d_out, int tm, int tn) {
    return static_cast<long>((M + tm - 1) / tm) * ((d_out + tn - 1) / tn);
}

}  // namespace

size_t prefill_workspace_bytes(int M) {
    return M <= 0 ? 0 : (static_cast<size_t>(M) * sizeof(float) + 255) / 256 * 256;
}

long prefill_tiles(const grinqh_layout& L, int M) { return tiles_of(M, L.d_out, 128, 128); }

// Tile shape (tokens x outputs): the least estimated time, counted as the
// waves of workgroups the CUs run (one 256-token workgroup per CU, two
// 128 x 128) times the time of one such wave relative to the others (34 : 20
// : 25 for 256 x 256, 256 x 128 and 128 x 128, and 16 for 128 x 128 tiles
// that leave each CU at most one, as measured at d_in 4096); up to 128
// tokens, 128 x 128, since a 256-token tile would be half empty.
hipError_t launch_prefill(const grinqh_layout& L, const uint16_t* x, int M, const uint32_t* planes,
                          const uint16_t* s, const uint16_t* z, void* y, int y_dtype, float* rowsum,
                          int cu_count, hipStream_t stream) {
    rowsum_kernel<<<dim3(static_cast<unsigned>((M + 3) / 4)), dim3(256), 0, stream>>>(x, M, L.d_in, rowsum);
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
    const int y_vec_outputs = y_dtype == GRINQH_F32 ? 4 : 8;   // outputs per 16 bytes
    a.vec_y = reinterpret_cast<uintptr_t>(y) % 16 == 0 && L.d_out % y_vec_outputs == 0;
    a.plane_bytes = static_cast<uint32_t>(static_cast<size_t>(L.d_in) * L.n_planes * L.row_words * 4u);
    const long cus = cu_count > 0 ? cu_count : 1;
    const long cost256 = 34 * ((tiles_of(M, L.d_out, 256, 256) + cus - 1) / cus);
    const long cost2561 = 20 * ((tiles_of(M, L.d_out, 256, 128) + cus - 1) / cus);
    const long t128 = tiles_of(M, L.d_out, 128, 128);
    const long cost128 = t128 <= cus ? 16 : 25 * ((t128 + 2 * cus - 1) / (2 * cus));
    int tile = 0;
    if (M > 128) tile = cost256 <= cost2561 && cost256 <= cost128 ? 2 : cost2561 <= cost128 ? 1 : 0;
    const int forced = launch_override().prefill_tile;   // 1: 128 x 128, 2: 256 x 128, 3: 256 x 256
    if (forced != 0) tile = forced - 1;
    switch (L.n_planes) {
        case 1: return launch_p<1>(a, tile, stream);
        case 2: return launch_p<2>(a, tile, stream);
        case 3: return launch_p<3>(a, tile, stream);
        case 4: return launch_p<4>(a, tile, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace grinqh
