/*
 * grinqh.h - C ABI of the MI355X (gfx950) decode-phase GEMV of GRINQH.
 *
 * Method source: the page "GRINQH: Graded Input-Based Quantization Hierarchy
 * for Efficient LLM Generation" (papernotes.org note on arXiv 2606.23419),
 * section 方法详解 / 关键设计 (key design) items 1-3, cited below as KD1
 * (bit assignment), KD2 (bit-planar storage) and KD3 (midpoint dequant).
 *
 * What the library computes, for one decode step (batch 1) of one linear:
 *
 *   b_i = 2 * #{k : theta_k <= |x_i|}                  KD1  (P = b_max/2 thresholds)
 *   w_hat_ij = s_j * (((q_ji >> k_i) << k_i) + phi_i) + z_j,
 *              k_i = b_max - b_i, phi_i = 2^(k_i - 1)   KD3  (phi = 1/2 at k_i = 0)
 *   y_j = sum over i with b_i > 0 of x_i * w_hat_ij      (channels with b_i = 0 are
 *                                                         never read, KD1/KD2)
 *
 * Only the top b_i/2 two-bit planes of each loaded channel are read (KD2).
 *
 * Packed layout (KD2).  planes is uint32 [d_in][P][W_row], W_row =
 * ceil(d_out/64)*4 words: for input channel i, plane p (p = 0 holds bits
 * [b_max-2, b_max-1] of the code, the most significant), the d_out fragments
 * are contiguous, 16 per word; the fragment of output 16w+t sits at bits
 * [2t, 2t+1] of word w.  Rows are padded to a multiple of 64 outputs with
 * zero fragments, so every plane row is a multiple of 16 bytes.
 *
 * Conventions shared by every call:
 *  - Every pointer argument is a device pointer unless marked "host".  The
 *    caller allocates and owns all memory; the library allocates nothing and
 *    keeps no state beyond a cached device-property query.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream) and never synchronise the host.  They are thread-safe; calls
 *    that share a workspace must be ordered on one stream.
 *  - Arguments are checked on the host before anything touches the device;
 *    a failed check returns an error code and launches nothing.  Nothing
 *    throws across the ABI.  Values inside device buffers are not checked:
 *    NaN activations get 0 bits (the channel is skipped), +-Inf gets b_max
 *    bits and makes y non-finite, codes above 2^b_max - 1 are masked by
 *    grinqh_pack, unsorted thresholds are used through the count formula.
 */
#ifndef GRINQH_H
#define GRINQH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GRINQH_OK = 0,
    GRINQH_EINVAL = 1,    /* NULL pointer, bad size, bad b_max, bad dtype, bad layout */
    GRINQH_EALIGN = 2,    /* a pointer is not aligned as documented */
    GRINQH_ENOSPACE = 3,  /* workspace smaller than grinqh_gemv_workspace_bytes() */
    GRINQH_ENODEV = 4,    /* no HIP device is visible */
    GRINQH_EDEVICE = 5    /* the HIP runtime reported an error (query or launch) */
} grinqh_status;

typedef enum {
    GRINQH_BF16 = 0,      /* bfloat16, 2 bytes, 2-byte aligned */
    GRINQH_F32 = 1        /* IEEE binary32, 4 bytes, 4-byte aligned */
} grinqh_dtype;

/* Shape of one packed linear layer (plain data; fill with grinqh_layout_init). */
typedef struct {
    int32_t d_in;         /* input channels (reduction dimension), 1 .. 2^20 */
    int32_t d_out;        /* output channels, 1 .. 2^20 */
    int32_t b_max;        /* 2, 4, 6 or 8: full code width */
    int32_t n_planes;     /* b_max / 2 */
    int32_t row_words;    /* ceil(d_out / 64) * 4 uint32 words per plane row */
} grinqh_layout;

/* Library version as major*10000 + minor*100 + patch. */
int32_t grinqh_version(void);

/* Short constant English text for a status code (host pointer, never NULL). */
const char* grinqh_status_string(grinqh_status status);

/* Fill *out (host pointer) for a layer.  EINVAL if out is NULL, a size is
 * outside 1 .. 2^20 or b_max is not 2, 4, 6 or 8.  Pure host function. */
grinqh_status grinqh_layout_init(int32_t d_in, int32_t d_out, int32_t b_max,
                                 grinqh_layout* out);

/* Bytes of the packed planes: d_in * n_planes * row_words * 4 (KD2: storage
 * stays at b_max bits per weight).  0 if L is NULL or invalid.  Host only. */
size_t grinqh_packed_bytes(const grinqh_layout* L);

/* Bytes of device workspace grinqh_gemv needs for this layout on the current
 * device (0 if L is NULL or invalid, or no device is visible).  Host only. */
size_t grinqh_gemv_workspace_bytes(const grinqh_layout* L);

/* Offline bit-plane packing (KD2).
 *   q       uint8 [d_out][d_in], row-major (nn.Linear orientation: q[j][i]
 *           is the code of output j, input i); codes are masked to b_max bits.
 *   planes  uint32 [d_in][n_planes][row_words], 16-byte aligned,
 *           grinqh_packed_bytes(L) bytes; fully overwritten, padding included.
 * q and planes must not overlap. */
grinqh_status grinqh_pack(const grinqh_layout* L, const uint8_t* q, uint32_t* planes,
                          void* stream);

/* Runtime bit assignment (KD1), on its own (grinqh_gemv does the same work
 * inside its own kernel and does not need this call).
 *   x           [d_in] of x_dtype.
 *   theta       float [n_planes], theta_1 .. theta_P (ascending for the
 *               interval reading; any order is defined by the count formula).
 *   bits        uint8 [d_in] out: b_i in {0, 2, .., b_max}.
 *   active_idx  int32 [d_in] out or NULL: the n_active indices with b_i > 0,
 *               ascending, in entries 0 .. n_active-1; later entries unwritten.
 *   n_active    int32 [1] out or NULL. */
grinqh_status grinqh_assign_bits(const grinqh_layout* L, const void* x, grinqh_dtype x_dtype,
                                 const float* theta, uint8_t* bits, int32_t* active_idx,
                                 int32_t* n_active, void* stream);

/* The decode GEMV: bit assignment, prefix-plane streaming, midpoint dequant
 * and the product, all in the library's kernels (KD1, KD2, KD3).
 *   x          [d_in] of x_dtype (GRINQH_BF16 or GRINQH_F32).
 *   theta      float [n_planes].
 *   planes     as written by grinqh_pack, 16-byte aligned.
 *   s, z       fp16 bit patterns [d_out]: per-output-channel scale and zero point.
 *   y          [d_out] of y_dtype, overwritten (not accumulated); bf16 output
 *              is the fp32 result rounded to nearest even.
 *   workspace  >= grinqh_gemv_workspace_bytes(L) bytes, 256-byte aligned.  It
 *              must be zero-filled before its first use; every call leaves it
 *              ready for the next call (no clearing between calls).  Calls
 *              sharing one workspace must not overlap in time.
 * The packed planes of L must be smaller than 2 GiB (EINVAL otherwise).
 * x and y must not overlap.  Accumulation is fp32; the partial sums of the
 * input-channel slices are combined with fp32 atomic adds, so repeated calls
 * may differ in the last bits of y (b_i, the loaded planes and the codes are
 * always identical).  The workspace must be device memory (hipMalloc). */
grinqh_status grinqh_gemv(const grinqh_layout* L, const void* x, grinqh_dtype x_dtype,
                          const float* theta, const uint32_t* planes, const uint16_t* s,
                          const uint16_t* z, void* y, grinqh_dtype y_dtype, void* workspace,
                          size_t workspace_bytes, void* stream);

/* grinqh_gemv without a workspace argument, for callers that cannot allocate
 * device memory: code under stream capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments (minus the workspace), checks,
 * kernels and results as grinqh_gemv.  The workspace is a static device
 * array of GRINQH_NOALLOC_SCRATCH_BYTES inside the library: every GPU the
 * library runs on holds its own copy until the process ends, and the call
 * allocates nothing.  The first call on a device also queues a kernel that
 * clears that device's copy, ahead of the GEMV on the same stream; every
 * call leaves it cleared for the next one.
 *   Returns ENOSPACE when this layout needs more workspace than the array
 *   holds (grinqh_gemv_workspace_bytes(L) > GRINQH_NOALLOC_SCRATCH_BYTES;
 *   about 230 thousand outputs), ENODEV beyond 64 devices.
 * All calls on one GPU share its array: calls that can overlap in time on
 * one GPU (other streams, other host threads) race and give wrong results;
 * order them on one stream. */
#define GRINQH_NOALLOC_SCRATCH_BYTES (1u << 20)
grinqh_status grinqh_gemv_noalloc(const grinqh_layout* L, const void* x, grinqh_dtype x_dtype,
                                  const float* theta, const uint32_t* planes, const uint16_t* s,
                                  const uint16_t* z, void* y, grinqh_dtype y_dtype, void* stream);

/* Operands of one GEMV in a group call (all device pointers, same meaning and
 * alignment as the grinqh_gemv arguments of the same names). */
typedef struct {
    const void* x;
    const float* theta;
    const uint32_t* planes;
    const uint16_t* s;
    const uint16_t* z;
    void* y;
} grinqh_gemv_operands;

#define GRINQH_MAX_GROUP 8

/* Workspace bytes for grinqh_gemv_group over these layouts (host arrays of n
 * entries); 0 if an argument is invalid or no device is visible. */
size_t grinqh_gemv_group_workspace_bytes(const grinqh_layout* layouts, int32_t n);

/* n (1 .. GRINQH_MAX_GROUP) independent decode GEMVs in one kernel launch,
 * e.g. the q/k/v or gate/up projections of a decoder layer, or any set of
 * linears whose inputs are ready.  Each member computes exactly what
 * grinqh_gemv computes for its own x, theta, planes, s, z and y (KD1-KD3);
 * one launch lets the members' memory latencies overlap.
 *   layouts    host array [n]; every layout must have the same b_max.
 *   ops        host array [n] of operands.
 *   x_dtype, y_dtype  shared by all members.
 *   workspace  >= grinqh_gemv_group_workspace_bytes(layouts, n) bytes,
 *              256-byte aligned, zero-filled before first use, self-clearing.
 * The members' outputs must not overlap each other or any member's input. */
grinqh_status grinqh_gemv_group(const grinqh_layout* layouts, const grinqh_gemv_operands* ops,
                                int32_t n, grinqh_dtype x_dtype, grinqh_dtype y_dtype,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Test and diagnostic call: the truncated codes q_b * 2^(b_max - b_i)
 * (KD3's spliced truncated integer, at full scale) that the GEMV kernel's own
 * plane decoder produces for every loaded channel, 0 for skipped channels.
 *   bits    uint8 [d_in], as written by grinqh_assign_bits.
 *   codes   uint8 [d_in][d_out] out. */
grinqh_status grinqh_debug_codes(const grinqh_layout* L, const uint8_t* bits,
                                 const uint32_t* planes, uint8_t* codes, void* stream);

/* Test and tuning call: force the launch shape of later GEMV and prefill
 * calls in this process (0 = the library's own choice, the default).
 *   lane_groups   0, 1, 2, 4 or 8 lane groups per wave: GEMV output tiles of
 *                 2048, 1024, 512 or 256 outputs.
 *   chunk         0 or 1 .. 256 input channels per GEMV slice.
 *   prefill_tile  0, or 1 (128 x 128), 2 (256 x 128), 3 (256 x 256) tokens
 *                 x outputs per prefill tile.
 * The GEMV workspace size depends on the shape: query it again after a
 * change.  EINVAL for any other value (nothing changes).  Host only. */
grinqh_status grinqh_debug_force_launch(int32_t lane_groups, int32_t chunk, int32_t prefill_tile);

/* ---- Threshold calibration (offline) ----------------------------------
 *
 * KD1 fixes the thresholds offline from the magnitudes of about 128 sample
 * inputs of a layer.  This call computes them as quantiles of the pooled
 * magnitudes: with the count magnitudes |x| sorted ascending (NaN after
 * +Inf), for each level q, h = (count - 1) * q, lo = floor(h),
 * hi = min(lo + 1, count - 1), t = h - lo,
 *   theta = v[lo] + t * (v[hi] - v[lo])      (fp64; v[lo] itself at t = 0),
 * rounded once to fp32.  The result is exact: order statistics by radix
 * selection, no sampling.
 *   x          count values (bf16 or fp32), e.g. n samples x d_in, any order.
 *   count      1 .. 2^32 - 1.
 *   levels     host array [n_levels] of quantile levels in [0, 1]; n_levels
 *              1 .. 4 (one per threshold, ascending levels give ascending
 *              thresholds).
 *   theta      fp32 [n_levels] out.
 *   workspace  >= grinqh_calibrate_workspace_bytes() bytes, 256-byte aligned;
 *              any contents (the call initialises it). */
size_t grinqh_calibrate_workspace_bytes(void);
grinqh_status grinqh_calibrate_thresholds(const void* x, grinqh_dtype x_dtype, int64_t count,
                                          const double* levels, int32_t n_levels, float* theta,
                                          void* workspace, size_t workspace_bytes, void* stream);

/* ---- Offline quantisation front end ("RTN") ----------------------------
 *
 * The note names round-to-nearest (RTN) as a base the method can sit on
 * without defining it.  This call quantises a bf16 weight matrix per output
 * channel onto the b_max-bit grid whose KD3 reconstruction at b = b_max,
 * s_j * (q + 1/2) + z_j, is the midpoint of each interval:
 *   lo_j, hi_j = min and max of row j (NaN ignored);
 *   s_j = fp16((hi_j - lo_j) / 2^b_max), z_j = fp16(lo_j) (zeros stored as +0);
 *   q = min(max(floor((w - z_j) / s_j), 0), 2^b_max - 1), in fp32 with the
 *       stored s_j and z_j (IEEE division; a NaN quotient gives 0, a row
 *       with s_j = 0 gets 0).
 * Every weight is then within s_j / 2 of its reconstruction, up to the fp16
 * rounding of s_j and z_j.  The outputs feed grinqh_pack and grinqh_gemv.
 *   w     bf16 [d_out][d_in]: row j holds output channel j's weights.
 *   q     uint8 [d_out][d_in] out.
 *   s, z  fp16 [d_out] out.
 * 1 <= d_in <= 2^30, 1 <= d_out <= 2^30, b_max in {2, 4, 6, 8}. */
grinqh_status grinqh_quantize_rtn(int32_t d_in, int32_t d_out, int32_t b_max, const uint16_t* w,
                                  uint8_t* q, uint16_t* s, uint16_t* z, void* stream);

/* ---- Prefill stage: dense b_max GEMM ----------------------------------
 *
 * The note's overview keeps the prefill stage dense: every weight at b_max
 * precision in ordinary matrix products, no thresholds.  For a block of M
 * prompt tokens this call computes, with every channel at b = b_max (KD3 at
 * k = 0, phi = 1/2),
 *   Y[m][j] = sum_i X[m][i] * (s_j * (q_ji + 1/2) + z_j)
 * from the same packed planes, s and z as grinqh_gemv.  The products of the
 * bf16 activations and the integer codes are exact; they are summed in fp32
 * on the bf16 matrix cores.
 *   L          layout of the planes (any b_max); d_in must be a multiple of 8.
 *   x          bf16 [M][d_in], row-major, 16-byte aligned (x_dtype must be
 *              GRINQH_BF16: the matrix cores take bf16 operands).
 *   M          1 .. 2^20 tokens.
 *   planes, s, z  as for grinqh_gemv.
 *   y          [M][d_out] of y_dtype, row-major, overwritten; bf16 output is
 *              the fp32 result rounded to nearest even.  A 16-byte aligned y
 *              with d_out a multiple of 8 (bf16) or 4 (fp32) is written in
 *              16-byte row segments, otherwise element by element (slower,
 *              same values).
 *   workspace  >= grinqh_prefill_workspace_bytes(M) bytes (the fp32 row sums
 *              of x), 256-byte aligned, any contents.
 * x and y must not overlap.  The planes must be smaller than 2 GiB. */
size_t grinqh_prefill_workspace_bytes(int32_t M);
grinqh_status grinqh_prefill_gemm(const grinqh_layout* L, const void* x, grinqh_dtype x_dtype, int32_t M,
                                  const uint32_t* planes, const uint16_t* s, const uint16_t* z, void* y,
                                  grinqh_dtype y_dtype, void* workspace, size_t workspace_bytes,
                                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GRINQH_H */
