// Plane decoding shared by the GEMV kernel and the debug-codes kernel.
//
// GRINQH note (papernotes.org), key design 2: the fragment of output 16w+t
// sits at bits [2t, 2t+1] of word w of a plane row, plane 0 most significant;
// key design 3: the taken planes concatenate into the truncated code.
//
// merge_codes<Pb>() turns the Pb plane words of one 16-output word position
// into four words E[0..3] whose bytes are the Pb-plane codes, using only
// shifts, masks and bit-field inserts (SWAR over 16 outputs at once):
//
//   byte b of E[k] holds the code of output 4b + k, multiplied by
//   code_scale<Pb>(k) (1 or 16 for Pb = 2, 1 or 4 for Pb = 3, 4^k for Pb = 1),
//
// so a consumer converts a byte with one v_cvt_f32_ubyte and folds the
// constant scale into its multiplier.  The merged value of a Pb-plane code
// is sum_{p<Pb} f_p * 4^(Pb-1-p); the truncated code at full width is that
// times 4^(P-Pb).  decode_values<Pb>() is the decode both kernels use: the
// 16 codes of a word position as exact floats (via packed FP4 / FP8
// conversions for one and two planes, via merge_codes otherwise).
#pragma once

#include "device_common.hpp"

namespace grinqh {

// 2-bit fragment t (0..15) of a plane word.
__device__ __forceinline__ uint32_t fragment(uint32_t word, int t) {
    return (word >> (2 * t)) & 3u;
}

// Inverse of the constant factor byte b of E[k] carries (see above).
template <int Pb>
__device__ __forceinline__ constexpr float code_unscale(int k) {
    if (Pb == 1) return k == 0 ? 1.f : k == 1 ? 0.25f : k == 2 ? 0.0625f : 0.015625f;
    if (Pb == 2) return (k & 2) ? 0.0625f : 1.f;
    if (Pb == 3) return (k & 2) ? 0.25f : 1.f;
    return 1.f;
}

template <int Pb>
__device__ __forceinline__ void merge_codes(const uint32_t* w, uint32_t (&E)[4]) {
    if constexpr (Pb == 1) {
        // no merge: mask fragment k of every byte in place (value f * 4^k)
        E[0] = w[0] & 0x03030303u;
        E[1] = w[0] & 0x0C0C0C0Cu;
        E[2] = w[0] & 0x30303030u;
        E[3] = w[0] & 0xC0C0C0C0u;
    } else {
        // nibble k of ne: (f0, f1) of output 2k; of no: of output 2k+1
        const uint32_t ne = ((w[0] << 2) & 0xCCCCCCCCu) | (w[1] & 0x33333333u);
        const uint32_t no = (w[0] & 0xCCCCCCCCu) | ((w[1] >> 2) & 0x33333333u);
        if constexpr (Pb == 2) {
            E[0] = ne & 0x0F0F0F0Fu;              // outputs 4b     (x1)
            E[1] = no & 0x0F0F0F0Fu;              // outputs 4b + 1 (x1)
            E[2] = ne & 0xF0F0F0F0u;              // outputs 4b + 2 (x16)
            E[3] = no & 0xF0F0F0F0u;              // outputs 4b + 3 (x16)
        } else if constexpr (Pb == 3) {
            const uint32_t f2 = w[2];
            E[0] = ((ne << 2) & 0x3C3C3C3Cu) | (f2 & 0x03030303u);          // 4b     (x1)
            E[1] = ((no << 2) & 0x3C3C3C3Cu) | ((f2 >> 2) & 0x03030303u);   // 4b + 1 (x1)
            E[2] = (ne & 0xF0F0F0F0u) | ((f2 >> 2) & 0x0C0C0C0Cu);          // 4b + 2 (x4)
            E[3] = (no & 0xF0F0F0F0u) | ((f2 >> 4) & 0x0C0C0C0Cu);          // 4b + 3 (x4)
        } else {
            const uint32_t me = ((w[2] << 2) & 0xCCCCCCCCu) | (w[3] & 0x33333333u);
            const uint32_t mo = (w[2] & 0xCCCCCCCCu) | ((w[3] >> 2) & 0x33333333u);
            E[0] = ((ne << 4) & 0xF0F0F0F0u) | (me & 0x0F0F0F0Fu);          // 4b
            E[1] = ((no << 4) & 0xF0F0F0F0u) | (mo & 0x0F0F0F0Fu);          // 4b + 1
            E[2] = (ne & 0xF0F0F0F0u) | ((me >> 4) & 0x0F0F0F0Fu);          // 4b + 2
            E[3] = (no & 0xF0F0F0F0u) | ((mo >> 4) & 0x0F0F0F0Fu);          // 4b + 3
        }
    }
}

// Byte b of a merged word as an exact float.
__device__ __forceinline__ float byte_f32(uint32_t e, int b) {
    return static_cast<float>((e >> (8 * b)) & 0xFFu);
}

// Decoded values of the 16 outputs of one word position for a Pb-plane
// code: code(t) = value[t] * decode_unit<Pb>(t & 3), where code(t) is the
// Pb-plane merged code sum_{p<Pb} f_p(t) * 4^(Pb-1-p).  Every value and unit
// is exact.  Per output this costs one conversion (or half of one):
//
//  * Pb = 1: w & 0x33333333 and (w >> 2) & 0x33333333 hold the even and the
//    odd fragments as 4-bit fields with the top two bits clear; such a field
//    read as an FP4 E2M1 number is f / 2, and one v_cvt_scalef32_pk_f32_fp4
//    converts the two fields of a byte (unit 2);
//  * Pb = 2: the 4-bit codes are spread to one per byte; a byte 0..15 read
//    as an FP8 E4M3 number is c * 2^-9 (exponent field 0 or 1: subnormal or
//    the first binade, evenly spaced), and one v_cvt_pk_f32_fp8 converts two
//    bytes (unit 2^9);
//  * Pb = 3, 4: the byte codes of merge_codes, one v_cvt_f32_ubyte each, with
//    the scale merge_codes leaves in byte lane k (unit code_unscale<Pb>(k)).
template <int Pb>
__device__ __forceinline__ constexpr float decode_unit(int k) {
    if (Pb == 1) return 2.0f;
    if (Pb == 2) return 512.0f;
    return code_unscale<Pb>(k);
}

typedef float decode_f2 __attribute__((ext_vector_type(2)));

// Byte B of the even-fragment and odd-fragment words: outputs 4B .. 4B+3.
template <int B>
__device__ __forceinline__ void fp4_byte(uint32_t ev, uint32_t od, float (&val)[16]) {
    const decode_f2 e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ev, 1.0f, B);   // outputs 4B, 4B+2
    const decode_f2 o = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(od, 1.0f, B);   // outputs 4B+1, 4B+3
    val[4 * B + 0] = e.x;
    val[4 * B + 2] = e.y;
    val[4 * B + 1] = o.x;
    val[4 * B + 3] = o.y;
}

template <int Pb>
__device__ __forceinline__ void decode_values(const uint32_t* w, float (&val)[16]) {
    if constexpr (Pb == 1) {
        const uint32_t ev = w[0] & 0x33333333u;            // nibble q: fragment 2q
        const uint32_t od = (w[0] >> 2) & 0x33333333u;     // nibble q: fragment 2q + 1
        fp4_byte<0>(ev, od, val);
        fp4_byte<1>(ev, od, val);
        fp4_byte<2>(ev, od, val);
        fp4_byte<3>(ev, od, val);
    } else if constexpr (Pb == 2) {
        // nibble k of ne: code of output 2k; of no: of output 2k+1
        const uint32_t ne = ((w[0] << 2) & 0xCCCCCCCCu) | (w[1] & 0x33333333u);
        const uint32_t no = (w[0] & 0xCCCCCCCCu) | ((w[1] >> 2) & 0x33333333u);
        uint32_t E[4];
        E[0] = ne & 0x0F0F0F0Fu;              // byte b: output 4b
        E[1] = no & 0x0F0F0F0Fu;              // 4b + 1
        E[2] = (ne >> 4) & 0x0F0F0F0Fu;       // 4b + 2
        E[3] = (no >> 4) & 0x0F0F0F0Fu;       // 4b + 3
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const decode_f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(E[k], false);   // bytes 0, 1
            const decode_f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(E[k], true);    // bytes 2, 3
            val[k] = lo.x;
            val[4 + k] = lo.y;
            val[8 + k] = hi.x;
            val[12 + k] = hi.y;
        }
    } else {
        uint32_t E[4];
        merge_codes<Pb>(w, E);
        // Hide the known-zero bits of E from the optimiser so that each byte
        // becomes one v_cvt_f32_ubyte{0..3} instead of a bit-field extract
        // followed by a conversion.
#pragma unroll
        for (int k = 0; k < 4; ++k) asm("" : "+v"(E[k]));
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int b = 0; b < 4; ++b) val[4 * b + k] = byte_f32(E[k], b);
    }
}

}  // namespace grinqh
