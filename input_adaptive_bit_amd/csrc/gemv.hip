// The decode GEMV of GRINQH (papernotes.org note, key designs 1-3) for gfx950.
//
// One launch computes one or several independent GEMVs (a "group", all with
// the same b_max).  Work item = (GEMV, output tile of T outputs, slice of up
// to 256 input channels); one 256-thread workgroup per item, all items
// resident at once (one generation of workgroups).  Slices are as long as
// the prologue allows, and the tile width (lane groups per wave) follows the
// launch's workgroup count (plan_gemv, search_launch).
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
// bucket, and two buckets are in flight at a time.  A slice whose loaded
// channels all take every plane (dense mode) streams only the top bucket,
// two batches at a time; in other slices the first two batches skip their
// empty slots when their buckets are short.
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
#include <type_traits>

#include "decode.hpp"
#include "internal.h"

namespace grinqh {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxChunk = kThreads;       // one channel per thread in the prologue
constexpr int kMinChunk = 128;            // shortest slice the launch shape picks by itself
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

// Factor of decode_unit<Pb> that the slice list's multiplier already holds:
// all of it for one and two planes (one unit for every output), none for
// three and four (the unit depends on the byte lane).
template <int Pb>
__device__ __forceinline__ constexpr float folded_unit() {
    return Pb <= 2 ? decode_unit<Pb>(0) : 1.f;
}

// acc[16 v + t] += x_scaled * code(t) for the 16 outputs t of each of the V
// word positions, code(t) = value(t) * decode_unit(t & 3) (decode.hpp); xs
// is x_scaled * folded_unit<Pb>() (every factor a power of two, so the
// products are those of x_scaled * code).
template <int Pb, int V>
__device__ __forceinline__ void accumulate(float (&acc)[16 * V], const uint32_t (&w)[Pb][V], float xs) {
    float a[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] = Pb <= 2 ? xs : xs * decode_unit<Pb>(k);
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

static_assert(kWaves == 4, "the prologue sums the bucket counts of four waves");

// Exponents of the slice-list multipliers x_i * 4^(P - Pi) * folded_unit<Pi>(),
// one byte per plane count Pi = 1 .. 4 (byte Pi - 1).
template <int P>
constexpr uint32_t scale_exponents() {
    uint32_t e = 0;
    for (int pi = 1; pi <= 4; ++pi) {
        const int unit_exp = pi == 1 ? 1 : pi == 2 ? 9 : 0;   // log2 of folded_unit<Pi>()
        const int ex = pi <= P ? 2 * (P - pi) + unit_exp : 0;
        e |= static_cast<uint32_t>(ex) << (8 * (pi - 1));
    }
    return e;
}
static_assert(folded_unit<1>() == 2.f && folded_unit<2>() == 512.f && folded_unit<3>() == 1.f &&
                  folded_unit<4>() == 1.f,
              "scale_exponents matches the folded units");

// Entries read past a bucket's end: fewer than one batch (U * stride <= 192)
// beyond the last list entry.  The slice lists are padded so that those
// reads stay inside them; their values are discarded.
constexpr int kListPad = 192;

struct SliceLists {
    uint32_t off[kMaxChunk + kListPad];   // byte offset of the channel's plane 0 row: i * P * row_bytes
    float xv[kMaxChunk + kListPad];       // x_i * 4^(P - Pi) * folded_unit<Pi>(): multiplier of its Pi-plane code
    uint32_t cnt[kWaves];      // word w, byte l: loaded channels of wave w with l + 1 planes
    float red_s[kWaves], red_c[kWaves];
    int is_last;               // this workgroup arrived last at its tile
    float S;                   // the tile's sum of x over loaded channels (last arriver)
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

// Issues the plane loads of one batch.  Lane group g of a wave takes the
// bucket entries ew + g + u * stride (u < U), where ew is wave-uniform.
// Entries past the bucket end, and lanes whose words lie past the padded
// row (a tile wider than the layout), load from past the end of the buffer:
// zeros, no request.  Every other load lies inside its own plane row, so the
// wave-uniform plane offset never carries an access past the buffer, whether
// or not the hardware range check counts it.
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

// The lists are read at a per-lane base and compile-time offsets u * stride,
// so an entry costs no address arithmetic; validity is one compare of the
// lane group against the wave-uniform number of entries left.  All U list
// entries are read first, whether valid or not (the lists are padded), so
// that the reads are not put behind branches one by one, each waiting for
// its own LDS round trip; an invalid entry's base is then replaced by
// kOutOfRange with a select.  (An entry past the slice's last channel holds
// whatever the LDS held before, so its value must not reach the address.)
//
// With kSkipEmpty, slots that no lane group of the wave has an entry for
// issue nothing (a scalar test), instead of out-of-range loads, which cost
// the CU's address unit about as much as L2 hits.  The loads then sit behind
// branches, and the waits of every decode before the next unconditional load
// cover all of them; only batches issued together at the start use it.
template <int P, int Pb, int V, int U, int stride, bool kSkipEmpty = false>
__device__ __forceinline__ void load_batch(Batch<Pb, V, U>& B, const uint32_t* offp, int group, int left,
                                           const PlaneSrc& src) {
    uint32_t o[U];
#pragma unroll
    for (int u = 0; u < U; ++u) o[u] = offp[u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (kSkipEmpty && left - u * stride <= 0) break;
        const bool ok = group < left - u * stride;
        const uint32_t base = ok ? o[u] + src.lane_bytes : kOutOfRange;
#pragma unroll
        for (int p = 0; p < Pb; ++p)
            load_words<V>(src.rsrc, base, static_cast<uint32_t>(p) * src.row_bytes, B.w[u][p]);
    }
}

// Decodes the batch slot by slot.  With kSkip, a slot that no lane group of
// the wave has a channel for is skipped as a whole (a scalar test), so small
// buckets cost only the slots they fill.  A slot's words are then used only
// behind its test, and the compiler may sink the slot's loads past the decode
// of the slots before it: the batch is no longer in flight at once.
template <int P, int Pb, int V, int U, int stride, bool kSkip>
__device__ __forceinline__ void compute_batch(float (&acc)[16 * V], const Batch<Pb, V, U>& B, const float* xp,
                                              int group, int left) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (kSkip && left - u * stride <= 0) break;
        const bool ok = group < left - u * stride;
        const float xe = xp[u * stride];
        accumulate<Pb, V>(acc, B.w[u], ok ? xe : 0.f);
    }
}

// Channels in flight per worker and bucket: the first batch of every bucket
// is issued before any decoding starts, and a batch holds a typical slice's
// share of its bucket, so a workgroup waits for about one memory round trip.
// At b_max 2 (P = 1) every loaded channel is in the one bucket, whose later
// batches decode every slot; six channels there spill registers, four do not.
template <int P, int Pb>
struct BatchSize { static constexpr int U = P == 1 ? 4 : Pb == 4 ? 2 : Pb == 3 ? 3 : Pb == 2 ? 5 : 6; };

template <int P, int Pb, int V, int G>
struct Bucket {
    static constexpr int U = BatchSize<P, Pb>::U;
    static constexpr int stride = kWaves * G;
    static_assert(U * stride <= kListPad, "list padding covers a batch past the end");
    Batch<Pb, V, U> B;
    int ew, end;            // wave-uniform: lane group 0's entry in the batch, the bucket end
    // begin, end: the bucket's entries (wave-uniform).  Lane group g of wave
    // wv is worker wv * G + g; the wave that takes a bucket's uneven last
    // round rotates with the bucket: wave wv starts at entry
    // ((wv + Pb - 1) mod 4) * G.
    template <bool kSkipEmpty = false>
    __device__ __forceinline__ void first(const SliceLists& L, int begin, int end_, int wv, int group,
                                          const PlaneSrc& src) {
        ew = begin + ((wv + Pb - 1) & (kWaves - 1)) * G;
        end = end_;
        load_batch<P, Pb, V, U, stride, kSkipEmpty>(B, &L.off[ew + group], group, end - ew, src);
    }
    // The dense path's bucket (the only one loaded): the next batch is issued
    // before the current one is decoded, so two batches are in flight.  The
    // loop is unrolled by two so that each batch keeps its registers, and a
    // batch is issued only when it has entries, so nothing is loaded past the
    // bucket's end; each load sits in the block that decodes the batch before
    // it, which keeps the waits exact.
    __device__ __forceinline__ void finish_pipelined(float (&acc)[16 * V], const SliceLists& L, int group,
                                                     const PlaneSrc& src) {
        constexpr int S = stride * U;
        Batch<Pb, V, U> B2;
        int e = ew;
        while (true) {
            const int e2 = e + S;
            if (e2 >= end) {
                compute_batch<P, Pb, V, U, stride, true>(acc, B, &L.xv[e + group], group, end - e);
                break;
            }
            load_batch<P, Pb, V, U, stride>(B2, &L.off[e2 + group], group, end - e2, src);
            compute_batch<P, Pb, V, U, stride, false>(acc, B, &L.xv[e + group], group, end - e);
            const int e3 = e2 + S;
            if (e3 >= end) {
                compute_batch<P, Pb, V, U, stride, true>(acc, B2, &L.xv[e2 + group], group, end - e2);
                break;
            }
            load_batch<P, Pb, V, U, stride>(B, &L.off[e3 + group], group, end - e3, src);
            compute_batch<P, Pb, V, U, stride, false>(acc, B2, &L.xv[e2 + group], group, end - e2);
            e = e3;
        }
    }
    __device__ __forceinline__ void finish(float (&acc)[16 * V], const SliceLists& L, int group,
                                           const PlaneSrc& src) {
        compute_batch<P, Pb, V, U, stride, true>(acc, B, &L.xv[ew + group], group, end - ew);
        // Later batches exist only for buckets longer than one batch.  Those
        // of the top bucket (Pb = P: every channel in dense mode) decode every
        // slot, so that the channels of a batch stay in flight together; the
        // empty slots of a bucket's last batch cost little next to the rest.
        for (ew += stride * U; ew < end; ew += stride * U) {
            load_batch<P, Pb, V, U, stride>(B, &L.off[ew + group], group, end - ew, src);
            compute_batch<P, Pb, V, U, stride, (Pb < P)>(acc, B, &L.xv[ew + group], group, end - ew);
        }
    }
};

// Item number of this workgroup.  Workgroup b is dispatched to XCD b % 8.
// The items (GEMV, tile, slice) are numbered tile-major and each XCD takes a
// contiguous run of them, so the slices of a tile meet in one XCD's L2 (a
// tile may straddle two).
__device__ __forceinline__ int xcd_item() {
    const int W = static_cast<int>(gridDim.x);
    const int xq = W >> 3, xr = W & 7;
    const int bx = static_cast<int>(blockIdx.x) & 7, br = static_cast<int>(blockIdx.x) >> 3;
    return bx * xq + min(bx, xr) + br;
}

// The work of one workgroup: item `item` of the GEMV described by D.
template <int P, int V, int G>
__device__ __forceinline__ void gemv_item(const GemvDesc& D, int item) {
    constexpr int b_max = 2 * P;
    constexpr int LG = kWave / G;            // lanes per group
    constexpr int T = LG * 16 * V;           // outputs per tile
    constexpr int NW = kWaves * G;           // workers (lane groups) per workgroup
    __shared__ SliceLists L;
    // One partial row per worker; a lane's 16 * V outputs are stored with a
    // stride of 16 * V + 4 floats, so that the lanes of a wave's 16-byte
    // stores fall in different LDS banks.
    constexpr int RSTR = 16 * V + 4;
    __shared__ float red[NW][LG * RSTR];

    // Every field of the descriptor is loaded now, while x and theta are on
    // their way, rather than where the reduction and epilogue first use it
    // (a kernel-argument load there waits a whole memory round trip).
    asm volatile("" ::"s"(D.x), "s"(D.theta), "s"(D.planes), "s"(D.s), "s"(D.z), "s"(D.y), "s"(D.acc),
                 "s"(D.ctrl));
    asm volatile("" ::"s"(D.d_in), "s"(D.d_out), "s"(D.row_words), "s"(D.chunk), "s"(D.n_splits),
                 "s"(D.n_tiles), "s"(D.x_dtype), "s"(D.y_dtype));
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    float th[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < P; ++k) th[k] = D.theta[k];
    const int local = item - D.wg_begin;
    const int tile = D.split_magic ? static_cast<int>(__umulhi(static_cast<uint32_t>(local), D.split_magic))
                                   : local / D.n_splits;
    const int split = local - tile * D.n_splits;

    // ---- prologue: bit assignment and bucket sort of the slice (key design 1)
    // x is read through a buffer resource, threads past the slice from past
    // its end (zero, no request), so no branch holds the loads back.
    const int i0 = split * D.chunk;
    const int cnt = min(D.chunk, D.d_in - i0);
    const bool mine = tid < cnt;
    float xv;
    {
        const int esz = D.x_dtype == 0 ? 2 : 4;
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<void*>(D.x), static_cast<short>(0), D.d_in * esz, 0x00020000);
        const uint32_t xo = mine ? static_cast<uint32_t>(i0 + tid) * esz : kOutOfRange;
        if (D.x_dtype == 0)
            xv = bf16_to_f32(static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(xr, xo, 0, 0)));
        else
            xv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(xr, xo, 0, 0));
    }
    // (with theta_0 <= 0 a zero x would get bits: threads past the slice get none)
    const int pi = mine ? bits_of<P>(xv, th) >> 1 : 0;
    // Rank of the lane's channel among the wave's channels with the same
    // plane count (mbcnt: set bits of the ballot below this lane), and the
    // wave's counts per plane count, one byte each, in one LDS word.
    int rank = 0;
    uint32_t counts = 0;
#pragma unroll
    for (int l = 0; l < P; ++l) {
        const unsigned long long m = __ballot(pi == l + 1);
        const int below_lane = static_cast<int>(__builtin_amdgcn_mbcnt_hi(
            static_cast<uint32_t>(m >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
        rank = pi == l + 1 ? below_lane : rank;
        counts |= static_cast<uint32_t>(__popcll(m)) << (8 * l);
    }
    if (lane == 0) L.cnt[wv] = counts;
    __syncthreads();
    // Bucket bounds and this wave's place in each bucket, as wave-uniform
    // scalars: bucket Pi = 1 first, each in wave then lane order.
    int start[5];   // bucket Pi holds entries start[Pi - 1] .. start[Pi] - 1
    int below[4];   // first entry of bucket l + 1 written by this wave
    uint32_t cw[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) cw[w] = __builtin_amdgcn_readfirstlane(L.cnt[w]);
    start[0] = 0;
#pragma unroll
    for (int l = 0; l < 4; ++l) {
        if (l < P) {
            const int c0 = (cw[0] >> (8 * l)) & 255, c1 = (cw[1] >> (8 * l)) & 255;
            const int c2 = (cw[2] >> (8 * l)) & 255, c3 = (cw[3] >> (8 * l)) & 255;
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
        // x_i * 4^(P - Pi) * folded_unit<Pi>() as one exponent step: the
        // power of two for Pi = 1 .. 4 is byte Pi - 1 of kScaleExp.
        constexpr uint32_t kScaleExp = scale_exponents<P>();
        L.xv[pos] = __builtin_ldexpf(xv, static_cast<int>((kScaleExp >> (8 * (pi - 1))) & 255u));
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
    // slice sums S and C over loaded channels (fixed-order reduction), while
    // the first plane loads are in flight
    auto slice_sums = [&]() {
        const float s_w = wave_sum(pi > 0 ? xv : 0.f);
        const float c_w = wave_sum(pi > 0 ? xv * phi_of(b_max, 2 * pi) : 0.f);
        if (lane == 0) {
            L.red_s[wv] = s_w;
            L.red_c[wv] = c_w;
        }
    };
    if (P >= 3 && start[P - 1] == 0) {
        // Every loaded channel of the slice has all P planes (dense mode, or
        // thresholds that load no channel partially): only the top bucket is
        // streamed, and the empty buckets issue no loads at all.  (Their
        // out-of-range loads would cost the CU's address unit as much as L2
        // hits: 25 wave-loads per wave at b_max 8.)  A separate path keeps
        // the wait counts of both exact.  At b_max 4 the empty bucket costs
        // 6 wave-loads, and the second path would spill registers there.
        if constexpr (P == 4) {
            k4.first(L, start[3], start[4], wv, group, src);
            slice_sums();
            k4.finish_pipelined(acc, L, group, src);
        } else if constexpr (P == 3) {
            k3.first(L, start[2], start[3], wv, group, src);
            slice_sums();
            k3.finish_pipelined(acc, L, group, src);
        }
    } else {
        // Two buckets in flight at a time: the next bucket's first batch is
        // issued after the bucket two ahead is decoded.  Every workgroup on
        // a CU then keeps a part of its loads in the CU's queue instead of
        // all of them, so the resident workgroups are served side by side
        // rather than one after another.
        auto general = [&](auto skip_early) {
            constexpr bool kSkipEarly = decltype(skip_early)::value;
            if constexpr (P >= 4) k4.template first<kSkipEarly>(L, start[3], start[4], wv, group, src);
            if constexpr (P >= 3) k3.template first<kSkipEarly>(L, start[2], start[3], wv, group, src);
            if constexpr (P <= 2) {
                if constexpr (P >= 2) k2.first(L, start[1], start[2], wv, group, src);
                // the last batch issued: when its bucket is empty (dense mode
                // at b_max 4) it issues nothing, and the waits of the decode
                // before it only gain loads that left at the same time
                if (P == 1 || start[1] > start[0]) k1.first(L, start[0], start[1], wv, group, src);
            }
            slice_sums();
            if constexpr (P >= 4) k4.finish(acc, L, group, src);
            if constexpr (P >= 3) {
                k2.first(L, start[1], start[2], wv, group, src);
                k3.finish(acc, L, group, src);
                k1.first(L, start[0], start[1], wv, group, src);
            }
            if constexpr (P >= 2) k2.finish(acc, L, group, src);
            k1.finish(acc, L, group, src);
        };
        // When the four- and three-plane buckets each fit their first batch
        // (short buckets, as at about 3 effective bits), those two batches,
        // issued together, skip their empty slots and the first decode waits
        // for both.  Fuller buckets have no empty slots to skip and keep the
        // exact waits.  A launch of one workgroup per CU (G = 8) measured
        // faster with the exact form.
        bool skip_early = false;
        constexpr int stride = kWaves * G;
        if constexpr (P == 4 && G <= 4)
            skip_early = start[4] - start[3] < BatchSize<P, 4>::U * stride &&
                         start[3] - start[2] < BatchSize<P, 3>::U * stride;
        else if constexpr (P == 3 && G <= 4)
            skip_early = start[3] - start[2] < BatchSize<P, 3>::U * stride;
        if constexpr (P >= 3 && G <= 4) {
            if (skip_early) general(std::integral_constant<bool, true>{});
            else general(std::integral_constant<bool, false>{});
        } else {
            general(std::integral_constant<bool, false>{});
        }
    }


    // ---- reduction: every worker stores its partial row to LDS, then each
    // thread sums the NW copies of its outputs in worker order (fixed order)
#pragma unroll
    for (int o = 0; o < 16 * V; o += 4)
        *reinterpret_cast<float4*>(&red[worker][r * RSTR + o]) =
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
    // The tile's partial A_j + C_slice and S_slice go to the workspace with
    // agent-scope fp32 atomic adds.
    unsigned* ctrl = D.ctrl + static_cast<size_t>(tile) * kCtrlWords;   // own 256-byte line per tile
    float* ssum = reinterpret_cast<float*>(ctrl + 1);
#pragma unroll
    for (int k = 0; k < OPT; ++k) {
        const int o = tid + k * kThreads;
        // all NW partials first, then a fixed-order pairwise sum
        float v[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) v[w] = red[w][(o / (16 * V)) * RSTR + o % (16 * V)];
#pragma unroll
        for (int h = NW / 2; h > 0; h /= 2)
#pragma unroll
            for (int w = 0; w < h; ++w) v[w] += v[w + h];
        unsafeAtomicAdd(ws_acc + o, v[0] + c_slice);
    }
    if (tid == 0) unsafeAtomicAdd(ssum, s_slice);

    // ---- last workgroup of the tile applies the epilogue.
    //
    // Ordering.  Every access to the workspace row, the S slot and the
    // arrival counter is an agent-scope atomic read-modify-write, and such
    // atomics are performed at one point per address for the whole device
    // (every XCD's adds to an address combine there).  A wave's vector
    // memory counter counts its atomic adds until the memory system
    // acknowledges them as performed, so after s_waitcnt 0 each thread's
    // adds are done; the barrier then waits for every thread, and only
    // after it does thread 0 take the arrival count.  The workgroup that
    // sees n_splits - 1 earlier arrivals therefore finds every slice's adds
    // performed, and reads them with atomic exchanges against zero (read
    // and clear in one step) issued after it saw the count.  No release or acquire fence is used: at agent scope they
    // write back or invalidate the whole L2 of the XCD, which measured about
    // twice the time of a whole launch of this kernel.
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
    // The row and S are read back (and cleared) at the same time; thread 0
    // hands S to the other threads through LDS and resets the counter: every
    // arrival of this call has been counted.
    float a[OPT];
#pragma unroll
    for (int k = 0; k < OPT; ++k)
        a[k] = __hip_atomic_exchange(ws_acc + tid + k * kThreads, 0.f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) {
        L.S = __hip_atomic_exchange(ssum, 0.f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ctrl, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const float S = L.S;
    const int j0 = tile * T;
#pragma unroll
    for (int k = 0; k < OPT; ++k) {
        const int j = j0 + tid + k * kThreads;
        if (j < D.d_out) {
            const float yv = s_j[k] * a[k] + z_j[k] * S;
            if (D.y_dtype == GRINQH_F32)
                static_cast<float*>(D.y)[j] = yv;
            else
                static_cast<uint16_t*>(D.y)[j] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(yv));   // RNE
        }
    }
}

// A group of GEMVs: the workgroup finds its member from the item number.
template <int P, int V, int G>
__global__ __launch_bounds__(kThreads, kWgPerCu) void gemv_kernel(GemvGroupArgs args) {
    const int item = xcd_item();
    int d = 0;
    while (d + 1 < args.n && item >= args.g[d + 1].wg_begin) ++d;
    const GemvDesc D = args.g[d];
    gemv_item<P, V, G>(D, item);
}

// One GEMV (grinqh_gemv): the descriptor is the whole kernel argument.
template <int P, int V, int G>
__global__ __launch_bounds__(kThreads, kWgPerCu) void gemv_one_kernel(GemvDesc D) {
    gemv_item<P, V, G>(D, xcd_item());
}

template <int P, int V, int G>
hipError_t launch_t(const GemvGroupArgs& a, int total_wg, hipStream_t stream) {
    gemv_kernel<P, V, G><<<dim3(static_cast<unsigned>(total_wg)), dim3(kThreads), 0, stream>>>(a);
    return hipGetLastError();
}

template <int P, int V, int G>
hipError_t launch_one_t(const GemvDesc& d, int total_wg, hipStream_t stream) {
    gemv_one_kernel<P, V, G><<<dim3(static_cast<unsigned>(total_wg)), dim3(kThreads), 0, stream>>>(d);
    return hipGetLastError();
}

template <int P>
hipError_t launch_one_p(const GemvDesc& d, int G, int total_wg, hipStream_t stream) {
    switch (G) {
        case 1: return launch_one_t<P, kV, 1>(d, total_wg, stream);
        case 2: return launch_one_t<P, kV, 2>(d, total_wg, stream);
        case 4: return launch_one_t<P, kV, 4>(d, total_wg, stream);
        case 8: return launch_one_t<P, kV, 8>(d, total_wg, stream);
        default: return hipErrorInvalidValue;
    }
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

namespace {

// Launch shape for these GEMVs on a device with `cus` compute units.
LaunchShape search_launch(const grinqh_layout* layouts, int n, long cus) {
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
    // Slice length.  A launch of W workgroups leaves the CUs unevenly loaded
    // unless W is a multiple of the CU count; shorten the slices (not below
    // kMinChunk) until W reaches the next multiple, without passing it.  W
    // does not grow with the slice length, so the shortest slice that stays
    // within the target is found by bisection.  The floor matters only for
    // layouts with few tiles (d_out of a few thousand), where a slice of 64
    // channels streams too little to pay for its share of the tile's
    // hand-off: 4096->1024 took 6.3 us with 64-channel slices on every CU
    // and 5.8 us with 128-channel slices on half of them.
    const long wmin = launch_workgroups(layouts, n, sh.lane_groups, kMaxChunk);
    const long target = (wmin + cus - 1) / cus * cus;
    int lo = kMinChunk, hi = kMaxChunk;          // W(hi) <= target holds
    while (lo < hi) {
        const int mid = (lo + hi) / 2;
        if (launch_workgroups(layouts, n, sh.lane_groups, mid) <= target) hi = mid;
        else lo = mid + 1;
    }
    sh.chunk = hi;
    return sh;
}

// Launch shapes of recent calls, per host thread: an eager call with the same
// layouts on the same device pays no search.
struct PlanCacheEntry {
    int n, cus, force_groups, force_chunk;
    int dims[kMaxGroup][3];
    LaunchShape shape;
};
constexpr int kPlanCache = 16;
thread_local PlanCacheEntry t_plan_cache[kPlanCache];
thread_local int t_plan_cache_used = 0, t_plan_cache_next = 0;

bool same_key(const PlanCacheEntry& e, const grinqh_layout* layouts, int n, int cus, const LaunchOverride& ov) {
    if (e.n != n || e.cus != cus || e.force_groups != ov.lane_groups || e.force_chunk != ov.chunk) return false;
    for (int k = 0; k < n; ++k)
        if (e.dims[k][0] != layouts[k].d_in || e.dims[k][1] != layouts[k].d_out || e.dims[k][2] != layouts[k].b_max)
            return false;
    return true;
}

}  // namespace

LaunchShape choose_launch(const grinqh_layout* layouts, int n, const DeviceInfo& dev) {
    const int cus = dev.cu_count > 0 ? dev.cu_count : 256;
    const LaunchOverride ov = launch_override();
    for (int k = 0; k < t_plan_cache_used; ++k)
        if (same_key(t_plan_cache[k], layouts, n, cus, ov)) return t_plan_cache[k].shape;
    LaunchShape sh = search_launch(layouts, n, cus);
    if (ov.lane_groups != 0) sh.lane_groups = ov.lane_groups;
    if (ov.chunk != 0) sh.chunk = ov.chunk;
    if (n <= kMaxGroup) {
        PlanCacheEntry& e = t_plan_cache[t_plan_cache_next];
        t_plan_cache_next = (t_plan_cache_next + 1) % kPlanCache;
        if (t_plan_cache_used < kPlanCache) ++t_plan_cache_used;
        e.n = n;
        e.cus = cus;
        e.force_groups = ov.lane_groups;
        e.force_chunk = ov.chunk;
        for (int k = 0; k < n; ++k) {
            e.dims[k][0] = layouts[k].d_in;
            e.dims[k][1] = layouts[k].d_out;
            e.dims[k][2] = layouts[k].b_max;
        }
        e.shape = sh;
    }
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
    // The multiply-high quotient is exact while item * n_splits < 2^32; for
    // one split, or a launch too large for that, the kernel divides instead.
    const uint64_t items = static_cast<uint64_t>(plan.n_tiles) * static_cast<uint64_t>(plan.n_splits);
    g->split_magic = plan.n_splits > 1 && items * static_cast<uint64_t>(plan.n_splits) < (uint64_t{1} << 32)
                         ? static_cast<uint32_t>(((uint64_t{1} << 32) + plan.n_splits - 1) / plan.n_splits)
                         : 0u;
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
    GemvDesc d{};
    fill_desc(&d, L, plan, x, x_dtype, theta, planes, s, z, y, y_dtype, workspace, 0);
    const int wg = plan.n_tiles * plan.n_splits;
    switch (L.n_planes) {
        case 1: return launch_one_p<1>(d, plan.lane_groups, wg, stream);
        case 2: return launch_one_p<2>(d, plan.lane_groups, wg, stream);
        case 3: return launch_one_p<3>(d, plan.lane_groups, wg, stream);
        case 4: return launch_one_p<4>(d, plan.lane_groups, wg, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace grinqh
