// The decode GEMV of GRINQH (papernotes.org note, key designs 1-3) for gfx950.
//
// One launch computes one or several independent GEMVs (a "group", all with
// the same b_max).  Work item = (GEMV, output tile of T outputs, slice of up
// to 256 input channels); one 256-thread workgroup per item, all items
// resident at once (one generation of workgroups).  Slices are as long as
// the prologue allows, and the tile width (lane groups per wave) follows the
// launch's workgroup count (plan_gemv, choose_lane_groups).
//
// Prologue (key design 1).  The workgroup reads its slice of x, assigns
// b_i = 2 * #{k : theta_k <= |x_i|} with exact fp32 compares and bucket-sorts
// the loaded channels (b_i > 0) by plane count Pi = b_i / 2 into LDS, in
// ascending channel order inside each bucket (wave ballots; the bucket bounds
// are summed from per-wave counts on the scalar unit), so the order - and
// with it the fp32 summation order - is fixed.  It also forms the slice's
// S = sum x_i and C = sum x_i * phi_i over loaded channels.
//
// Main loop (key design 2).  A wave is split into G lane groups of 64/G
// lanes; lane r of a group owns 16*V consecutive outputs of the tile.  The
// 4G groups of the workgroup ("workers") take the channels of a bucket in
// turn and read only their first Pi plane rows: V words (4*V bytes) per lane
// per plane, so a group reads T/4 contiguous bytes per plane row, and
// untaken planes and skipped channels issue no memory request.  Every
// channel in a bucket has the same plane count, so the lanes of a wave never
// diverge.  Load batches are sized to hold a typical slice's share of a
// bucket, and two buckets are in flight at a time.
//
// Decode and accumulate (key design 3).  The Pi plane words of 16 outputs
// become 16 exact floats (decode.hpp: packed FP4 / FP8 conversions for one and
// two planes, a SWAR merge into byte codes and v_cvt_f32_ubyte for three and
// four), each accumulated with one fp32 FMA into acc_j += x_i * 4^(P-Pi) * code.
// With A_j = sum_i x_i * code_ij,
//   y_j = sum_i x_i * (s_j * (code_ij + phi_i) + z_j) = s_j * (A_j + C) + z_j * S.
//
// Reduction.  Every worker stores its partial row to LDS and each thread sums
// the workers' copies of its outputs in a fixed order; the tile's partial
// A_j + C_slice is added with fp32 atomics into a workspace row and S_slice
// into a per-tile slot.  A per-tile arrival counter elects the last
// workgroup, which applies the epilogue y_j = s_j * acc_j + z_j * S (bf16
// output rounded to nearest even) and clears its workspace row and counter
// for the next call.
#include <cstdlib>

#include "decode.hpp"
#include "internal.h"

namespace grinqh {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxChunk = kThreads;       // one channel per thread in the prologue
constexpr int kMinChunk = 64;             // shortest slice the launch shape picks by itself
constexpr int kWgPerCu = 4;               // resident workgroups per CU the kernel is sized for
constexpr int kV = 2;                     // plane words per lane per plane row (8-byte loads)

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Plane rows are read through a raw buffer resource covering the packed
// planes.  A lane with nothing to load uses an offset past the end: the
// load returns zeros without a memory request, so every load instruction is
// unconditional and the wait counters stay exact (no branches around loads).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t planes_rsrc(const uint32_t* planes, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(planes), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

constexpr int kNonTemporal = 2;   // plane rows are streamed once per call

// V words at byte offset voff + soff (soff: a wave-uniform plane offset).
template <int V>
__device__ __forceinline__ void load_words(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff,
                                           uint32_t (&w)[V]) {
    if constexpr (V == 4) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, soff, kNonTemporal);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rsrc, voff, soff, kNonTemporal);
        w[0] = v.x; w[1] = v.y;
    }
}

// acc[16 v + t] += x_scaled * code(t) for the 16 outputs t of each of the V
// word positions, code(t) = value(t) * decode_unit(t & 3) (decode.hpp).
template <int Pb, int V>
__device__ __forceinline__ void accumulate(float (&acc)[16 * V], const uint32_t (&w)[Pb][V], float xs) {
    float a[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] = xs * decode_unit<Pb>(k);
#pragma unroll
    for (int v = 0; v < V; ++v) {
        uint32_t pw[Pb];
#pragma unroll
        for (int p = 0; p < Pb; ++p) pw[p] = w[p][v];
        float val[16];
        decode_values<Pb>(pw, val);
#pragma unroll
        for (int t = 0; t < 16; ++t) acc[16 * v + t] = __builtin_fmaf(a[t & 3], val[t], acc[16 * v + t]);
    }
}

static_assert(kWaves == 4, "one count byte per wave in a word");

struct SliceLists {
    uint32_t off[kMaxChunk];   // byte offset of the channel's plane 0 row: i * P * row_bytes
    float xv[kMaxChunk];       // x_i * 4^(P - Pi): the multiplier of its Pi-plane code
    uint32_t cnt[4];           // word l, byte w: loaded channels of wave w with l + 1 planes
    float red_s[kWaves], red_c[kWaves];
    int is_last;
};

// Sum over the 64 lanes in a fixed order; every lane gets the total.  Lanes
// i and i ^ 32, then rows r and r ^ 1 are added with the swap instructions,
// then the 16 lanes of each row with DPP rotations and quad permutes.
__device__ __forceinline__ float wave_sum(float v) {
    {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        const uint32_t a = r[0], b = r[1];     // copied out before reinterpreting
        v = __uint_as_float(a) + __uint_as_float(b);
    }
    {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        const uint32_t a = r[0], b = r[1];
        v = __uint_as_float(a) + __uint_as_float(b);
    }
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false));  // row_ror:8
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xF, 0xF, false));  // row_ror:4
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));   // lane ^ 2
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));   // lane ^ 1
    return v;
}

// Plane words of U channels of one bucket (Pb planes each) of one worker.
// x_i stays in LDS until the decode, so a batch holds only plane words.
template <int Pb, int V, int U>
struct Batch {
    uint32_t w[U][Pb][V];
};

// Issues the plane loads of bucket entries e0, e0 + stride, ... (U of
// them).  Entries past the bucket end, and lanes whose words lie past the
// padded row (a tile wider than the layout), load from past the end of the
// buffer: zeros, no request.  Every other load lies inside its own plane row,
// so the wave-uniform plane offset never carries an access past the buffer,
// whether or not the hardware range check counts it.
struct PlaneSrc {
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t row_bytes;     // bytes per plane row
    uint32_t lane_bytes;    // byte offset of this lane's words within a row (kOutOfRange past it)
};

// Base offset of an entry past the bucket end, and the lane offset of a lane
// past the row: the planes are smaller than 2 GiB, so this offset plus a
// channel offset and a plane offset is past the end of the buffer and below
// 2^32.
constexpr uint32_t kOutOfRange = 0x80000000u;

template <int P, int Pb, int V, int U>
__device__ __forceinline__ void load_batch(Batch<Pb, V, U>& B, const SliceLists& L, int e0, int stride,
                                           int end, const PlaneSrc& src) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int e = e0 + u * stride;
        const bool ok = e < end;
        const uint32_t base = ok ? L.off[e] + src.lane_bytes : kOutOfRange;
#pragma unroll
        for (int p = 0; p < Pb; ++p)
            load_words<V>(src.rsrc, base, static_cast<uint32_t>(p) * src.row_bytes, B.w[u][p]);
    }
}

// Decodes the batch slot by slot; a slot that no lane group of the wave has a
// channel for is skipped as a whole (wave-uniform branch), so small buckets
// cost only the slots they fill.
template <int P, int Pb, int V, int U>
__device__ __forceinline__ void compute_batch(float (&acc)[16 * V], const Batch<Pb, V, U>& B,
                                              const SliceLists& L, int e0, int stride, int end) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int e = e0 + u * stride;
        const bool ok = e < end;
        if (__ballot(ok) == 0ull) continue;
        const float xe = L.xv[ok ? e : 0];      // in range either way: no branch
        accumulate<Pb, V>(acc, B.w[u], ok ? xe : 0.f);
    }
}

// Channels in flight per worker and bucket: the first batch of every bucket
// is issued before any decoding starts, and a batch holds a typical slice's
// share of its bucket, so a workgroup waits for about one memory round trip.
template <int Pb>
struct BatchSize { static constexpr int U = Pb == 4 ? 1 : Pb == 3 ? 3 : Pb == 2 ? 5 : 6; };

template <int P, int Pb, int V, int G>
struct Bucket {
    static constexpr int U = BatchSize<Pb>::U;
    static constexpr int stride = kWaves * G;
    Batch<Pb, V, U> B;
    int e, end;
    // begin, end: the bucket's entries (wave-uniform)
    __device__ __forceinline__ void first(const SliceLists& L, int begin, int end_, int worker,
                                          const PlaneSrc& src) {
        e = begin + worker;
        end = end_;
        load_batch<P, Pb, V, U>(B, L, e, stride, end, src);
    }
    __device__ __forceinline__ void finish(float (&acc)[16 * V], const SliceLists& L, const PlaneSrc& src) {
        compute_batch<P, Pb, V, U>(acc, B, L, e, stride, end);
        for (e += stride * U; e < end; e += stride * U) {
            load_batch<P, Pb, V, U>(B, L, e, stride, end, src);
            compute_batch<P, Pb, V, U>(acc, B, L, e, stride, end);
        }
    }
};

template <int P, int V, int G>
__global__ __launch_bounds__(kThreads, kWgPerCu) void gemv_kernel(GemvGroupArgs args) {
    constexpr int b_max = 2 * P;
    constexpr int LG = kWave / G;            // lanes per group
    constexpr int T = LG * 16 * V;           // outputs per tile
    constexpr int NW = kWaves * G;           // workers (lane groups) per workgroup
    __shared__ SliceLists L;
    __shared__ float red[NW][T];             // one partial row per worker

    // ---- locate the GEMV and the (tile, slice) of this workgroup
    int d = 0;
    while (d + 1 < args.n && static_cast<int>(blockIdx.x) >= args.g[d + 1].wg_begin) ++d;
    const GemvDesc& D = args.g[d];
    const int local = static_cast<int>(blockIdx.x) - D.wg_begin;
    const int tile = local % D.n_tiles;
    const int split = local / D.n_tiles;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);

    float th[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < P; ++k) th[k] = D.theta[k];

    // ---- prologue: bit assignment and bucket sort of the slice (key design 1)
    const int i0 = split * D.chunk;
    const int cnt = min(D.chunk, D.d_in - i0);
    float xv = 0.f;
    int pi = 0;
    if (tid < cnt) {
        xv = load_x(D.x, D.x_dtype, i0 + tid);
        pi = bits_of<P>(xv, th) >> 1;
    }
    int rank = 0;
#pragma unroll
    for (int l = 0; l < P; ++l) {
        const unsigned long long m = __ballot(pi == l + 1);
        if (pi == l + 1) rank = __popcll(m & ((1ull << lane) - 1ull));
        if (lane == 0) reinterpret_cast<uint8_t*>(L.cnt)[4 * l + wv] = static_cast<uint8_t>(__popcll(m));
    }
    __syncthreads();
    // Bucket bounds and this wave's place in each bucket, as wave-uniform
    // scalars: bucket Pi = 1 first, each in wave then lane order.
    int start[5];   // bucket Pi holds entries start[Pi - 1] .. start[Pi] - 1
    int below[4];   // first entry of bucket l + 1 written by this wave
    start[0] = 0;
#pragma unroll
    for (int l = 0; l < 4; ++l) {
        if (l < P) {
            const uint32_t c = __builtin_amdgcn_readfirstlane(L.cnt[l]);
            const int c0 = c & 255, c1 = (c >> 8) & 255, c2 = (c >> 16) & 255, c3 = c >> 24;
            below[l] = start[l] + (wv > 0 ? c0 : 0) + (wv > 1 ? c1 : 0) + (wv > 2 ? c2 : 0);
            start[l + 1] = start[l] + c0 + c1 + c2 + c3;
        } else {
            below[l] = start[l];
            start[l + 1] = start[l];
        }
    }
    if (pi > 0) {
        int pos = below[0];
#pragma unroll
        for (int l = 1; l < P; ++l) pos = pi == l + 1 ? below[l] : pos;
        pos += rank;
        L.off[pos] = static_cast<uint32_t>(i0 + tid) * (P * static_cast<uint32_t>(D.row_words) * 4u);
        L.xv[pos] = xv * static_cast<float>(1u << (2 * (P - pi)));
    }
    __syncthreads();

    // ---- main loop (key designs 2 and 3)
    const int group = lane / LG;
    const int r = lane % LG;
    const int word_off = tile * (T / 16) + r * V;      // first word of this lane in a plane row
    const int worker = wv * G + group;
    float acc[16 * V];
#pragma unroll
    for (int o = 0; o < 16 * V; ++o) acc[o] = 0.f;
    PlaneSrc src;
    // the row size is uniform; make that explicit so plane offsets stay scalar
    src.row_bytes = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(D.row_words) * 4u);
    src.rsrc = planes_rsrc(D.planes, src.row_bytes * static_cast<uint32_t>(P) * static_cast<uint32_t>(D.d_in));
    // lanes past the row get an offset that keeps every load out of range
    src.lane_bytes = word_off < D.row_words ? static_cast<uint32_t>(word_off) * 4u : kOutOfRange;
    Bucket<P, 1, V, G> k1;
    Bucket<P, (P >= 2 ? 2 : 1), V, G> k2;
    Bucket<P, (P >= 3 ? 3 : 1), V, G> k3;
    Bucket<P, (P >= 4 ? 4 : 1), V, G> k4;
    // Two buckets in flight at a time: the next bucket's first batch is
    // issued after the bucket two ahead is decoded.  Every workgroup on a CU
    // then keeps a part of its loads in the CU's queue instead of all of
    // them, so the resident workgroups are served side by side rather than
    // one after another.
    if constexpr (P >= 4) k4.first(L, start[3], start[4], worker, src);
    if constexpr (P >= 3) k3.first(L, start[2], start[3], worker, src);
    if constexpr (P <= 2) {
        if constexpr (P >= 2) k2.first(L, start[1], start[2], worker, src);
        k1.first(L, start[0], start[1], worker, src);
    }

    // slice sums S and C over loaded channels (fixed-order reduction), while
    // the first plane loads are in flight
    {
        const float s_w = wave_sum(pi > 0 ? xv : 0.f);
        const float c_w = wave_sum(pi > 0 ? xv * phi_of(b_max, 2 * pi) : 0.f);
        if (lane == 0) {
            L.red_s[wv] = s_w;
            L.red_c[wv] = c_w;
        }
    }
    if constexpr (P >= 4) k4.finish(acc, L, src);
    if constexpr (P >= 3) {
        k2.first(L, start[1], start[2], worker, src);
        k3.finish(acc, L, src);
        k1.first(L, start[0], start[1], worker, src);
    }
    if constexpr (P >= 2) k2.finish(acc, L, src);
    k1.finish(acc, L, src);


    // ---- reduction: every worker stores its partial row to LDS, then each
    // thread sums the NW copies of its outputs in worker order (fixed order)
#pragma unroll
    for (int o = 0; o < 16 * V; o += 4)
        *reinterpret_cast<float4*>(&red[worker][r * 16 * V + o]) =
            make_float4(acc[o], acc[o + 1], acc[o + 2], acc[o + 3]);
    __syncthreads();
    float s_slice = L.red_s[0], c_slice = L.red_c[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
        s_slice += L.red_s[w];
        c_slice += L.red_c[w];
    }
    float* ws_acc = D.acc + static_cast<size_t>(tile) * T;
    constexpr int OPT = T / kThreads;                   // outputs per thread
    // this thread's s_j and z_j, fetched now so that the epilogue, if this
    // workgroup runs it, does not wait for them
    float s_j[OPT], z_j[OPT];
#pragma unroll
    for (int k = 0; k < OPT; ++k) {
        const int j = tile * T + tid + k * kThreads;
        const int jc = j < D.d_out ? j : D.d_out - 1;
        s_j[k] = f16_to_f32(D.s[jc]);
        z_j[k] = f16_to_f32(D.z[jc]);
    }
#pragma unroll
    for (int k = 0; k < OPT; ++k) {
        const int o = tid + k * kThreads;
        // all NW partials first, then a fixed-order pairwise sum
        float v[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) v[w] = red[w][o];
#pragma unroll
        for (int h = NW / 2; h > 0; h /= 2)
#pragma unroll
            for (int w = 0; w < h; ++w) v[w] += v[w + h];
        unsafeAtomicAdd(ws_acc + o, v[0] + c_slice);
    }
    unsigned* ctrl = D.ctrl + static_cast<size_t>(tile) * kCtrlWords;   // own 256-byte line per tile
    float* ssum = reinterpret_cast<float*>(ctrl + 1);
    if (tid == 0) unsafeAtomicAdd(ssum, s_slice);

    // ---- last workgroup of the tile applies the epilogue.  No device-scope
    // fence: fp32 atomics are performed at the device coherence point, so each
    // thread waits until its own atomics have completed (s_waitcnt 0) before the
    // arrival count is taken, and the elected workgroup reads the row back with
    // agent-scope loads.  (A __threadfence here writes back and invalidates the
    // L2 for every workgroup, which serialises the whole grid.)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    if (tid == 0) {
        const unsigned prev = __hip_atomic_fetch_add(ctrl, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        L.is_last = (prev == static_cast<unsigned>(D.n_splits - 1)) ? 1 : 0;
    }
    __syncthreads();
    if (!L.is_last) return;
    const float S = __hip_atomic_load(ssum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int j0 = tile * T;
#pragma unroll
    for (int k = 0; k < OPT; ++k) {
        const int o = tid + k * kThreads;
        const int j = j0 + o;
        const float a = __hip_atomic_load(ws_acc + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ws_acc + o, 0.f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (j < D.d_out) {
            const float yv = s_j[k] * a + z_j[k] * S;
            if (D.y_dtype == GRINQH_F32)
                static_cast<float*>(D.y)[j] = yv;
            else
                static_cast<uint16_t*>(D.y)[j] = f32_to_bf16_rne(yv);
        }
    }
    if (tid == 0) {
        __hip_atomic_store(ssum, 0.f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ctrl, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int P, int V, int G>
hipError_t launch_t(const GemvGroupArgs& a, int total_wg, hipStream_t stream) {
    gemv_kernel<P, V, G><<<dim3(static_cast<unsigned>(total_wg)), dim3(kThreads), 0, stream>>>(a);
    return hipGetLastError();
}

template <int P>
hipError_t launch_p(const GemvGroupArgs& a, int G, int total_wg, hipStream_t stream) {
    switch (G) {
        case 1: return launch_t<P, kV, 1>(a, total_wg, stream);
        case 2: return launch_t<P, kV, 2>(a, total_wg, stream);
        case 4: return launch_t<P, kV, 4>(a, total_wg, stream);
        case 8: return launch_t<P, kV, 8>(a, total_wg, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int gemv_tile_outputs(int G) { return (kWave / G) * 16 * kV; }

// Optional launch-shape overrides for tuning on new shapes:
// GRINQH_LANE_GROUPS (1, 2, 4 or 8) and GRINQH_CHUNK (1 .. 256 channels per slice).
int env_int(const char* name) {
    const char* v = std::getenv(name);
    return v ? std::atoi(v) : 0;
}

GemvPlan plan_gemv(const grinqh_layout& L, const LaunchShape& shape) {
    GemvPlan pl{};
    const int padded = L.row_words * 16;
    const int G = shape.lane_groups;
    pl.lane_groups = G;
    pl.tile_outputs = gemv_tile_outputs(G);
    pl.n_tiles = (padded + pl.tile_outputs - 1) / pl.tile_outputs;
    const int chunk = shape.chunk < 1 ? 1 : shape.chunk > kMaxChunk ? kMaxChunk : shape.chunk;
    int n_splits = (L.d_in + chunk - 1) / chunk;
    if (n_splits < 1) n_splits = 1;
    pl.chunk = (L.d_in + n_splits - 1) / n_splits;       // balanced slices
    pl.n_splits = (L.d_in + pl.chunk - 1) / pl.chunk;
    const size_t acc_bytes = static_cast<size_t>(pl.n_tiles) * pl.tile_outputs * sizeof(float);
    pl.ws_acc = 0;
    pl.ws_ctrl = align_up(acc_bytes, 256);
    pl.ws_bytes = pl.ws_ctrl + static_cast<size_t>(pl.n_tiles) * kCtrlWords * sizeof(unsigned);
    return pl;
}

namespace {

// Workgroups of a launch of these GEMVs at a tile width and slice length.
long launch_workgroups(const grinqh_layout* layouts, int n, int G, int chunk) {
    long wg = 0;
    for (int k = 0; k < n; ++k) {
        const GemvPlan p = plan_gemv(layouts[k], LaunchShape{G, chunk});
        wg += static_cast<long>(p.n_tiles) * p.n_splits;
    }
    return wg;
}

}  // namespace

LaunchShape choose_launch(const grinqh_layout* layouts, int n, const DeviceInfo& dev) {
    const long cus = dev.cu_count > 0 ? dev.cu_count : 256;
    LaunchShape sh{4, kMaxChunk};
    // Tile width.  Every split of a tile adds one more row of atomics and one
    // more workgroup that the tile's last arriver waits for, and the main
    // loop of a slice is short next to that fixed chain: slices are as long
    // as the prologue allows (one channel per thread), and the tile width
    // keeps the launch within one generation of at most kWgPerCu workgroups
    // per CU (G = 2) or, for small launches, reaches more CUs (G = 8).
    const long wg4 = launch_workgroups(layouts, n, 4, kMaxChunk);
    if (wg4 > kWgPerCu * cus) sh.lane_groups = 2;
    else if (8 * wg4 < 5 * cus) sh.lane_groups = 8;
    const int env_groups = env_int("GRINQH_LANE_GROUPS");
    if (env_groups == 1 || env_groups == 2 || env_groups == 4 || env_groups == 8) sh.lane_groups = env_groups;
    // Slice length.  A launch of W workgroups leaves the CUs unevenly loaded
    // unless W is a multiple of the CU count; shorten the slices (not below
    // kMinChunk) until W reaches the next multiple, without passing it.
    const long wmin = launch_workgroups(layouts, n, sh.lane_groups, kMaxChunk);
    const long target = (wmin + cus - 1) / cus * cus;
    for (int c = kMaxChunk - 1; c >= kMinChunk; --c) {
        if (launch_workgroups(layouts, n, sh.lane_groups, c) > target) break;
        sh.chunk = c;
    }
    const int env_chunk = env_int("GRINQH_CHUNK");
    if (env_chunk >= 1 && env_chunk <= kMaxChunk) sh.chunk = env_chunk;
    return sh;
}

void fill_desc(GemvDesc* g, const grinqh_layout& L, const GemvPlan& plan, const void* x, int x_dtype,
               const float* theta, const uint32_t* planes, const uint16_t* s, const uint16_t* z,
               void* y, int y_dtype, void* workspace, int wg_begin) {
    char* ws = static_cast<char*>(workspace);
    g->x = x;
    g->theta = theta;
    g->planes = planes;
    g->s = s;
    g->z = z;
    g->y = y;
    g->acc = reinterpret_cast<float*>(ws + plan.ws_acc);
    g->ctrl = reinterpret_cast<unsigned*>(ws + plan.ws_ctrl);
    g->d_in = L.d_in;
    g->d_out = L.d_out;
    g->row_words = L.row_words;
    g->chunk = plan.chunk;
    g->n_splits = plan.n_splits;
    g->n_tiles = plan.n_tiles;
    g->wg_begin = wg_begin;
    g->x_dtype = x_dtype;
    g->y_dtype = y_dtype;
}

hipError_t launch_gemv_group(int n_planes, int lane_groups, const GemvGroupArgs& args, int total_wg,
                             hipStream_t stream) {
    switch (n_planes) {
        case 1: return launch_p<1>(args, lane_groups, total_wg, stream);
        case 2: return launch_p<2>(args, lane_groups, total_wg, stream);
        case 3: return launch_p<3>(args, lane_groups, total_wg, stream);
        case 4: return launch_p<4>(args, lane_groups, total_wg, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv(const grinqh_layout& L, const GemvPlan& plan, const void* x,
                       int x_dtype, const float* theta, const uint32_t* planes,
                       const uint16_t* s, const uint16_t* z, void* y, int y_dtype,
                       void* workspace, hipStream_t stream) {
    GemvGroupArgs a{};
    a.n = 1;
    fill_desc(&a.g[0], L, plan, x, x_dtype, theta, planes, s, z, y, y_dtype, workspace, 0);
    return launch_gemv_group(L.n_planes, plan.lane_groups, a, plan.n_tiles * plan.n_splits, stream);
}

}  // namespace grinqh
