// retro_decode.h - device decoders for the weight block formats (gfx950).
//
// Every kernel of the library (dequantize, tiled MFMA, skinny) turns stored
// bytes into float32 through the primitives below, so one bit-exact check of
// retro_dequantize covers the arithmetic of all of them.
//
// Exactness: a Q8_0/Q4_0/Q5_0 value d*(q - c) needs at most 11+8 significant
// bits (Q4_1/Q5_1 add the offset m with one rounding), a Q4_K product
// (d*sc)*q at most 11+6+4 = 21 (Q5_K: 22) and dmin*m at most 17, so every
// product below is exact in float32 and only the Q4_K/Q5_K subtraction rounds
// (once, to nearest-even); Q2_K (d*sc)*q needs at most 11+4+2 bits and rounds
// likewise only in its subtraction. A Q6_K value (d*sc)*(q - 32) and a Q3_K
// value (d*(sc - 32))*(q - 4) are exact. The formats that subtract a constant
// from the code (Q4_0, Q5_0, Q6_K, Q3_K) are decoded as scale times (q - c)
// in that order, never as scale*q - scale*c: the two agree on every finite
// value, but only the first gives the sign of a zero and an infinite scale's
// +-inf as the formats' own formulas do. Whether the compiler fuses a*q - b
// into an FMA changes no bit. An MXFP4 value, an E2M1 code times a power of
// two, is formed by the hardware's scaled FP4 conversion, which returns that
// product rounded once (exact unless it overflows to inf, subnormal scales
// and results included; NaN for the NaN scale).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace retro {

// GGUF tensor-type ids.
enum : int {
    kF32 = 0, kF16 = 1, kQ4_0 = 2, kQ4_1 = 3, kQ5_0 = 6, kQ5_1 = 7, kQ8_0 = 8, kQ2_K = 10, kQ3_K = 11, kQ4_K = 12,
    kQ5_K = 13, kQ6_K = 14, kBF16 = 30, kMXFP4 = 39, kNVFP4 = 40
};

// kBlock: elements per block; kBytes: bytes per block; kGroup: elements one
// thread decodes from one 16-byte code load in the tiled kernel.
template <int TYPE> struct Format;
template <> struct Format<kF32>  { static constexpr int kBlock = 1,   kBytes = 4,   kGroup = 4;  };
template <> struct Format<kF16>  { static constexpr int kBlock = 1,   kBytes = 2,   kGroup = 8;  };
template <> struct Format<kBF16> { static constexpr int kBlock = 1,   kBytes = 2,   kGroup = 8;  };
template <> struct Format<kQ8_0> { static constexpr int kBlock = 32,  kBytes = 34,  kGroup = 16; };
template <> struct Format<kQ4_0> { static constexpr int kBlock = 32,  kBytes = 18,  kGroup = 32; };
template <> struct Format<kQ4_1> { static constexpr int kBlock = 32,  kBytes = 20,  kGroup = 32; };
template <> struct Format<kQ5_0> { static constexpr int kBlock = 32,  kBytes = 22,  kGroup = 32; };
template <> struct Format<kQ5_1> { static constexpr int kBlock = 32,  kBytes = 24,  kGroup = 32; };
template <> struct Format<kMXFP4> { static constexpr int kBlock = 32, kBytes = 17,  kGroup = 32; };
// NVFP4: 64 elements in 36 bytes, four FP8 E4M3 sub-block scales then 32
// code bytes; sub-block s (elements 16s .. 16s + 15) takes code bytes
// 8s .. 8s + 7, element 16s + i (i < 8) the low nibble of byte 8s + i and
// element 16s + 8 + i its high nibble.
template <> struct Format<kNVFP4> { static constexpr int kBlock = 64, kBytes = 36,  kGroup = 32; };

// The 32-element nibble formats: element j < 16 is the low nibble of code
// byte j, element j + 16 its high nibble, after a header of kHeader bytes
// (fp16 d; Q4_1/Q5_1 an fp16 offset m; Q5_0/Q5_1 a 32-bit word of fifth
// bits, bit j for element j).
template <int TYPE> constexpr bool kNibble32 = TYPE == kQ4_0 || TYPE == kQ4_1 || TYPE == kQ5_0 || TYPE == kQ5_1;
template <int TYPE> constexpr bool kHasOffset = TYPE == kQ4_1 || TYPE == kQ5_1;
template <int TYPE> constexpr bool kHasFifth = TYPE == kQ5_0 || TYPE == kQ5_1;
template <int TYPE> constexpr int kHeader = Format<TYPE>::kBytes - 16;
// MXFP4 shares that code layout (after a one-byte E8M0 scale) but not the
// arithmetic.
template <int TYPE> constexpr bool kNibbleLayout = kNibble32<TYPE> || TYPE == kMXFP4;
template <> struct Format<kQ4_K> { static constexpr int kBlock = 256, kBytes = 144, kGroup = 32; };
template <> struct Format<kQ5_K> { static constexpr int kBlock = 256, kBytes = 176, kGroup = 32; };
template <> struct Format<kQ6_K> { static constexpr int kBlock = 256, kBytes = 210, kGroup = 32; };
template <> struct Format<kQ2_K> { static constexpr int kBlock = 256, kBytes = 84,  kGroup = 32; };
template <> struct Format<kQ3_K> { static constexpr int kBlock = 256, kBytes = 110, kGroup = 32; };

// The K-quant formats: 256-element super-blocks, so a tile of K holds whole
// super-blocks only when it is 256 columns wide.
template <int TYPE> constexpr bool kSuperBlock = Format<TYPE>::kBlock == 256;

// IEEE binary16 bits -> float32 (v_cvt_f32_f16; exact, subnormals included).
__device__ __forceinline__ float half_to_f32(uint32_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

// bfloat16 bits -> float32: the bits are the upper half of the binary32.
__device__ __forceinline__ float bf16_to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

// Two binary16 / bfloat16 values packed in one little-endian word.
__device__ __forceinline__ void f16x2(uint32_t w, float& lo, float& hi) {
    lo = half_to_f32(w & 0xFFFFu);
    hi = half_to_f32(w >> 16);
}
__device__ __forceinline__ void bf16x2(uint32_t w, float& lo, float& hi) {
    lo = __uint_as_float(w << 16);
    hi = __uint_as_float(w & 0xFFFF0000u);
}

// Q8_0: four int8 codes (one little-endian word) times the block scale d.
__device__ __forceinline__ void q8_0_x4(uint32_t w, float d, float out[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = static_cast<int>(static_cast<int8_t>((w >> (8 * i)) & 0xFFu));
        out[i] = d * static_cast<float>(q);
    }
}

// The four low (high = false) or high nibbles of a code word, one per byte.
// The mask is applied once per word by an instruction the compiler cannot
// see through, so that each byte is then converted by one byte-to-float
// instruction (v_cvt_f32_ubyte0..3) rather than a bit-field extract plus a
// conversion per element.
__device__ __forceinline__ uint32_t nibbles(uint32_t w, bool high) {
    const uint32_t x = high ? (w >> 4) : w;
    uint32_t m;
    asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(m) : "v"(x));
    return m;
}

// Bits first .. first + 3 of a 32-bit fifth-bit word, as bit 4 of the four
// bytes of a word (a multiply by 0x00204081 places bit i at bit 8i).
__device__ __forceinline__ uint32_t fifth_bits(uint32_t qh, int first) {
    return ((((qh >> first) & 15u) * 0x00204081u) & 0x01010101u) << 4;
}

// Four signed codes held in the top bits of the four bytes of `top`: byte i
// is (q_i - c) * 2^s as a signed 8-bit integer (the code's value q_i XOR c,
// c = 2^(b-1) for a b-bit code, placed at bits 8-b .. 7). Each element is
// one signed-byte conversion (exact) times as = a * 2^-s (exact: a power of
// two times a scale far above the subnormal range), so the result is
// a * (q_i - c) rounded once, which is exact.
__device__ __forceinline__ void signed_top_x4(uint32_t top, float as, float out[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = static_cast<float>(static_cast<int8_t>((top >> (8 * i)) & 0xFFu)) * as;
}

// The fifth bits first .. first + 3 of a 32-bit word, inverted, as bit 7 of
// the four bytes of a word (q XOR 16 for a 5-bit code).
__device__ __forceinline__ uint32_t fifth_bits_top(uint32_t qh, int first) {
    return (((((qh >> first) & 15u) * 0x00204081u) & 0x01010101u) << 7) ^ 0x80808080u;
}

// Q4_0: the low (high = false) or high nibbles of four code bytes, value
// d*(q - 8) = float(16*(q - 8)) * (d/16); ds = d/16.
__device__ __forceinline__ void q4_0_x4(uint32_t w, bool high, float ds, float out[4]) {
    const uint32_t x = w ^ 0x88888888u;  // every nibble q -> q XOR 8
    signed_top_x4((high ? x : (x << 4)) & 0xF0F0F0F0u, ds, out);
}

// Q5_0: the low or high nibbles of four code bytes plus their fifth bits
// `qh` bits first .. first + 3, value d*(q - 16) = float(8*(q - 16)) * (d/8);
// ds = d/8.
__device__ __forceinline__ void q5_0_x4(uint32_t w, bool high, uint32_t qh, int first, float ds, float out[4]) {
    signed_top_x4(((high ? (w >> 1) : (w << 3)) & 0x78787878u) | fifth_bits_top(qh, first), ds, out);
}

// Q4_1 / Q5_1: the low or high nibbles of four code bytes, plus the fifth
// bits `fifth` (fifth_bits; 0 for Q4_1); value d*q + m, m the block's offset.
__device__ __forceinline__ void q4_1_x4(uint32_t w, bool high, uint32_t fifth, float d, float m, float out[4]) {
    const uint32_t q = nibbles(w, high) | fifth;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = d * static_cast<float>((q >> (8 * i)) & 0xFFu) + m;
}

// MXFP4 scale from its E8M0 byte: 2^(e - 127) as float32 (e = 0 is the
// subnormal 2^-127, e = 255 NaN).
__device__ __forceinline__ float mx_scale(uint32_t e) {
    e &= 0xFFu;
    const uint32_t bits = e == 0u ? 0x00400000u : e == 255u ? 0x7FC00000u : (e << 23);
    return __uint_as_float(bits);
}

// MXFP4: the low (lo) and high (hi) nibbles of the four code bytes of w,
// each an E2M1 value times the scale s: one conversion per byte, which
// returns (low nibble, high nibble) of the selected byte.
__device__ __forceinline__ void mxfp4_x8(uint32_t w, float s, float lo[4], float hi[4]) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 0);
    const f2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 1);
    const f2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 2);
    const f2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 3);
    lo[0] = a.x; hi[0] = a.y;
    lo[1] = b.x; hi[1] = b.y;
    lo[2] = c.x; hi[2] = c.y;
    lo[3] = d.x; hi[3] = d.y;
}

// FP8 E4M3 byte -> float32, exactly (the NVFP4 sub-block scale): sign bit
// 7, exponent bits 6..3 (bias 7), mantissa bits 2..0; exponent 0 is the
// subnormal range m * 2^-9; exponent 15 with mantissa 7 is NaN (the format
// has no infinities). Branch-free: the normal pattern is built in the
// float32 fields (exponent + 120, mantissa at the top of the fraction).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    const float normal = __uint_as_float(((e + 120u) << 23) | (m << 20));
    const float sub = static_cast<float>(m) * 0x1p-9f;
    float mag = e == 0u ? sub : normal;
    mag = (b & 0x7Fu) == 0x7Fu ? __uint_as_float(0x7FC00000u) : mag;
    return (b & 0x80u) ? -mag : mag;
}

// NVFP4: the low (lo) and high (hi) nibbles of four code bytes of one
// sub-block, E2M1 values (the hardware conversion at scale 1, exact) times
// the sub-block scale s (exact: at most 2 + 4 significant bits, far from the
// subnormal range; NaN for the NaN scale).
__device__ __forceinline__ void nvfp4_x8(uint32_t w, float s, float lo[4], float hi[4]) {
    float l[4], h[4];
    mxfp4_x8(w, 1.0f, l, h);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lo[i] = l[i] * s;
        hi[i] = h[i] * s;
    }
}

// NVFP4: the low (high = false) or high nibbles of four code bytes.
__device__ __forceinline__ void nvfp4_x4(uint32_t w, bool high, float s, float out[4]) {
    float lo[4], hi[4];
    nvfp4_x8(w, s, lo, hi);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = high ? hi[i] : lo[i];
}

// MXFP4: the low (high = false) or high nibbles of four code bytes.
__device__ __forceinline__ void mxfp4_x4(uint32_t w, bool high, float s, float out[4]) {
    float lo[4], hi[4];
    mxfp4_x8(w, s, lo, hi);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = high ? hi[i] : lo[i];
}

// Scale, offset m and fifth-bit word qh of a 32-element nibble block whose
// first 8 bytes are the words h0, h1. Q4_1/Q5_1: d and the offset m
// (value d*q + m). Q4_0 and Q5_0 have no offset (m = 0) and give their scale
// d as d/16 and d/8, the factor of q4_0_x4 and q5_0_x4.
template <int TYPE>
__device__ __forceinline__ void nibble32_header(uint32_t h0, uint32_t h1, float& d, float& m, uint32_t& qh) {
    d = half_to_f32(h0 & 0xFFFFu);
    if constexpr (kHasOffset<TYPE>)
        m = half_to_f32(h0 >> 16);
    else
        m = 0.0f;
    if constexpr (TYPE == kQ4_0) d *= 0.0625f;
    if constexpr (TYPE == kQ5_0) d *= 0.125f;
    if constexpr (TYPE == kQ5_0)
        qh = (h0 >> 16) | (h1 << 16);
    else if constexpr (TYPE == kQ5_1)
        qh = h1;
    else
        qh = 0u;
}

// Elements first .. first + 3 (first % 4 == 0; the low nibbles of the code
// word w for first < 16, its high nibbles otherwise) of a 32-element nibble
// block with header values d, m, qh from nibble32_header.
template <int TYPE>
__device__ __forceinline__ void nibble32_x4(uint32_t w, uint32_t qh, int first, float d, float m, float out[4]) {
    const bool high = first >= 16;
    if constexpr (TYPE == kQ4_0)
        q4_0_x4(w, high, d, out);
    else if constexpr (TYPE == kQ5_0)
        q5_0_x4(w, high, qh, first, d, out);
    else
        q4_1_x4(w, high, fifth_bits(qh, first), d, m, out);
}

// Q4_K sub-scale and sub-min j (0..7) from the 12-byte field, given as its
// three little-endian words s0 (bytes 0-3), s1 (4-7), s2 (8-11). GGUF packing:
// j < 4: sc = low 6 bits of byte j, m = low 6 bits of byte j+4.
// j >= 4: sc = low nibble of byte j+4 | (top 2 bits of byte j-4) << 4,
//         m  = high nibble of byte j+4 | (top 2 bits of byte j) << 4.
__device__ __forceinline__ void q4_k_scale_min(uint32_t s0, uint32_t s1, uint32_t s2, int j,
                                               uint32_t& sc, uint32_t& m) {
    // both forms from byte j % 4 of each word, then a select (no branch: j
    // differs between lanes)
    const uint32_t sh = 8u * uint32_t(j & 3);
    const uint32_t b0 = (s0 >> sh) & 0xFFu, b1 = (s1 >> sh) & 0xFFu, b2 = (s2 >> sh) & 0xFFu;
    const bool low = j < 4;
    sc = low ? (b0 & 63u) : ((b2 & 15u) | ((b0 >> 6) << 4));
    m = low ? (b1 & 63u) : ((b2 >> 4) | ((b1 >> 6) << 4));
}

// Q4_K sub-block j of a super-block whose first 16 bytes are the words
// h0 (d | dmin << 16), s0, s1, s2: a = d*sc_j and b = dmin*m_j (both exact).
__device__ __forceinline__ void q4_k_coeffs(uint32_t h0, uint32_t s0, uint32_t s1, uint32_t s2, int j,
                                            float& a, float& b) {
    uint32_t sc, m;
    q4_k_scale_min(s0, s1, s2, j, sc, m);
    a = half_to_f32(h0 & 0xFFFFu) * static_cast<float>(sc);
    b = half_to_f32(h0 >> 16) * static_cast<float>(m);
}

// Q4_K: from four code bytes take the low or high nibbles; value a*q - b.
__device__ __forceinline__ void q4_k_x4(uint32_t w, bool high, float a, float b, float out[4]) {
    const uint32_t m = nibbles(w, high);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = a * static_cast<float>((m >> (8 * i)) & 0xFFu) - b;
}

// Q4_K with the nibbles selected by `mask`: 0x0F0F0F0F gives q (a = d*sc),
// 0xF0F0F0F0 leaves the high nibbles in place as 16 q, to be scaled by
// a = d*sc/16. Either way a times the byte is (d*sc)*q exactly, so the value
// is the same a*q - b rounded once as q4_k_x4's, with one AND per four
// elements instead of a shift and an AND.
__device__ __forceinline__ void q4_k_x4_masked(uint32_t w, uint32_t mask, float a, float b, float out[4]) {
    const uint32_t m = w & mask;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = a * static_cast<float>((m >> (8 * i)) & 0xFFu) - b;
}

// Q5_K: low (high = false) or high nibbles of four qs bytes, plus bit
// `bit` of the four qh bytes of the same elements as the fifth bit;
// value a*q - b with a = d*sc_j, b = dmin*m_j (q4_k_coeffs; same field).
__device__ __forceinline__ void q5_k_x4(uint32_t qs, uint32_t qh, int bit, bool high, float a, float b,
                                        float out[4]) {
    const uint32_t fifth = ((qh >> bit) & 0x01010101u) << 4;
    const uint32_t m = nibbles(qs, high) | fifth;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = a * static_cast<float>((m >> (8 * i)) & 0xFFu) - b;
}

// Q6_K: low or high nibbles of four ql bytes, plus bits 2p, 2p+1 of the four
// qh bytes of the same elements as bits 4-5 of q; value (d*sc)*(q - 32) =
// float(4*(q - 32)) * as with as = d*sc/4 (q6_k_coeffs).
__device__ __forceinline__ void q6_k_x4(uint32_t ql, bool high, uint32_t qh, int p, float as, float out[4]) {
    // q XOR 32 at bits 2..7: the nibble at bits 2-5, the two high bits at 6-7
    // with the upper one inverted
    const uint32_t lo4 = (high ? (ql >> 2) : (ql << 2)) & 0x3C3C3C3Cu;
    const uint32_t hi2 = (((qh >> (2 * p)) << 6) & 0xC0C0C0C0u) ^ 0x80808080u;
    signed_top_x4(lo4 | hi2, as, out);
}

// Signed 8-bit Q6_K sub-scale `i` (0..3) of a word, times d, over 4:
// as = d*sc/4 (exact), the factor of q6_k_x4.
__device__ __forceinline__ void q6_k_coeffs(uint32_t scales, int i, float d, float& as) {
    const int sc = static_cast<int>(static_cast<int8_t>((scales >> (8 * i)) & 0xFFu));
    as = d * static_cast<float>(sc) * 0.25f;
}

// Q2_K: the 2-bit codes at bits 2p, 2p+1 of four qs bytes; value a*q - b
// with a = d*sc, b = dmin*m of the element's pair byte.
__device__ __forceinline__ void q2_k_x4(uint32_t qs, int p, float a, float b, float out[4]) {
    const uint32_t m = (qs >> (2 * p)) & 0x03030303u;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = a * static_cast<float>((m >> (8 * i)) & 0xFFu) - b;
}

// Q2_K pair byte `i` (0..3) of a word (sub-scale low nibble, sub-min high).
__device__ __forceinline__ void q2_k_coeffs(uint32_t pairs, int i, float d, float dmin, float& a, float& b) {
    const uint32_t pr = (pairs >> (8 * i)) & 0xFFu;
    a = d * static_cast<float>(pr & 15u);
    b = dmin * static_cast<float>(pr >> 4);
}

// Q3_K sub-scale s (0..15, stored 0..63) from the 12-byte field given as
// its little-endian words f0, f1, f2. With i = s % 4, g = s / 4: low 4 bits
// are the low (g < 2) or high nibble of byte 4 (g % 2) + i, high 2 bits are
// bits 2g, 2g+1 of byte 8 + i.
__device__ __forceinline__ uint32_t q3_k_scale(uint32_t f0, uint32_t f1, uint32_t f2, int s) {
    const int i = s & 3, g = s >> 2;
    const uint32_t lo = (((g & 1) ? f1 : f0) >> (8 * i + 4 * (g >> 1))) & 15u;
    return lo | (((f2 >> (8 * i + 2 * g)) & 3u) << 4);
}

// Q3_K: low 2 bits at bits 2p, 2p+1 of four qs bytes, plus 4 where bit
// `hbit` of the four hmask bytes is set (q' = q + 4 in 0..7); value
// (d*(sc - 32))*(q' - 4) = float(32*(q' - 4)) * as with as = d*(sc - 32)/32
// (q3_k_coeffs).
__device__ __forceinline__ void q3_k_x4(uint32_t qs, uint32_t hm, int p, int hbit, float as, float out[4]) {
    // q' XOR 4 at bits 5..7: the low bits at 5-6, the mask bit inverted at 7
    const uint32_t lo2 = ((qs >> (2 * p)) & 0x03030303u) << 5;
    const uint32_t hi1 = (((hm >> hbit) & 0x01010101u) << 7) ^ 0x80808080u;
    signed_top_x4(lo2 | hi1, as, out);
}

__device__ __forceinline__ void q3_k_coeffs(uint32_t f0, uint32_t f1, uint32_t f2, int s, float d, float& as) {
    as = d * static_cast<float>(static_cast<int>(q3_k_scale(f0, f1, f2, s)) - 32) * 0.03125f;
}

}  // namespace retro
