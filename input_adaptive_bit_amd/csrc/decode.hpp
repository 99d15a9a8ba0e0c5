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
// times 4^(P-Pb).
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

// Truncated full-width code of output t (0..15) from the merged words:
// the debug path decodes through the same merge the GEMV uses.
template <int P, int Pb>
__device__ __forceinline__ uint32_t code_from_merged(const uint32_t (&E)[4], int t) {
    const int k = t & 3, b = t >> 2;
    uint32_t v = (E[k] >> (8 * b)) & 0xFFu;
    if (Pb == 1) v >>= 2 * k;
    if (Pb == 2 && (k & 2)) v >>= 4;
    if (Pb == 3 && (k & 2)) v >>= 2;
    return v << (2 * (P - Pb));
}

}  // namespace grinqh
