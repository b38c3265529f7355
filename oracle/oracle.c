/*
 * oracle.c - plain CPU oracle for OUT_PROD through a block-quantized weight.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library. The HIP library never calls it and it
 * shares no code, header or table with the HIP library.
 *
 * What it computes. The llama.cpp PR "cuda: out_prod accepts a quantized
 * src0" (commit message and section "What") states that the backward of
 * mul_mat(W, x) with respect to x is out_prod(W, grad^T), and that OUT_PROD
 * now takes a quantized (or F16/BF16) src0 with F32 src1 and dst. Written
 * out, with W stored as N rows of K elements, G the F32 gradient (T x N) and
 * dst F32 (T x K):
 *
 *     dst[t][k] = sum_{n=0}^{N-1} W[n][k] * G[t][n]
 *
 * where W[n][k] is the value the stored block decodes to. The same page
 * (section "What") computes it as "decode W to F32, then an F32 GEMM", so the
 * plain definition above, with decoded values, is the whole method; this
 * file writes that definition out:
 *
 *   1. decode every row of W to F32 with a scalar block decoder;
 *   2. for every output, sum the N products in increasing n in double,
 *      also summing their absolute values (the error normaliser);
 *   3. round the double sum to F32 once.
 *
 * The only loop tiling is over blocks of t rows (several t rows share one
 * pass over W); it changes no output's summation order. Threads, when asked
 * for, split the t rows and likewise change no summation order.
 *
 * Block formats (GGUF; the pages only name them): fp16 fields are
 * little-endian binary16; see the decoder functions for each layout. Build
 * with -O2 -ffp-contract=off and no fast-math.
 *
 * Parity unpinned against the pages: the bit order of the Q4_K 12-byte
 * sub-scale/sub-min field. The pages print no Q4_K block; the order used is
 * the GGUF one, and the tests pin the decoder to hand-packed fixtures of that
 * reading and to a full pack bijection, not to values from the pages.
 *
 * Parity unpinned against the pages: the layouts of Q4_1, Q5_0 and Q5_1 (the
 * PR's commit message lists them among the swept types but prints no block),
 * the GGUF ones, pinned to hand-derived fixtures.
 *
 * Parity unpinned against the pages: MXFP4. The PR's type sweep names it
 * and prints no block; the element and scale encodings are those of the OCP
 * Microscaling (MX) specification (E2M1 elements, an E8M0 shared scale), in
 * the GGUF block order, pinned to hand-derived fixtures.
 *
 * Parity unpinned against the pages: NVFP4. The PR's type sweep names it and
 * prints no block. The element and scale encodings are those of NVIDIA's
 * NVFP4 format (E2M1 elements, one FP8 E4M3 scale per 16 elements; the
 * per-tensor F32 scale of that format is not part of a block and is taken
 * as 1). The block layout is this library's reading: 64 elements in 36
 * bytes, the four sub-block scales first, then 8 code bytes per sub-block in
 * the nibble order MXFP4 uses within its block. Pinned to hand-derived
 * fixtures, to the E4M3 decode of an independent library and to the pinned
 * E2M1 decode of MXFP4.
 *
 * Parity unpinned against the pages: Q2_K, Q3_K, Q5_K and Q6_K as a whole.
 * The pages name the K-quant family only through the Q4_K_M files it is
 * used in; these layouts are the GGUF ones, and the tests pin them to
 * hand-derived fixtures and to structural relations, not to values from the
 * pages.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum {
    T_F32 = 0, T_F16 = 1, T_Q4_0 = 2, T_Q4_1 = 3, T_Q5_0 = 6, T_Q5_1 = 7, T_Q8_0 = 8, T_Q2_K = 10, T_Q3_K = 11,
    T_Q4_K = 12, T_Q5_K = 13, T_Q6_K = 14, T_BF16 = 30, T_MXFP4 = 39, T_NVFP4 = 40
};

/* An E2M1 code (bit 3 sign, bits 2..1 exponent, bit 0 mantissa; exponent
 * bias 1, no infinities or NaNs): exponent field 0 is the subnormal range,
 * value m/2, otherwise (1 + m/2) * 2^(E - 1). */
static double e2m1_value(int code) {
    const int E = (code >> 1) & 3, m = code & 1;
    const double mag = E == 0 ? 0.5 * m : (1.0 + 0.5 * m) * ldexp(1.0, E - 1);
    return (code & 8) ? -mag : mag;
}

/* An FP8 E4M3 byte (the OCP 8-bit floating-point format E4M3, which NVFP4
 * uses for its block scales): bit 7 sign, bits 6..3 exponent E (bias 7),
 * bits 2..0 mantissa m. E = 0 is the subnormal range, value m/8 * 2^-6;
 * otherwise (1 + m/8) * 2^(E - 7). There are no infinities: E = 15 with
 * m = 7 is NaN (both signs), so the largest value is 1.75 * 2^8 = 448. */
static double e4m3_value(int byte) {
    const int E = (byte >> 3) & 15, m = byte & 7;
    if (E == 15 && m == 7) return NAN;
    const double mag = E == 0 ? ldexp((double)m, -9) : ldexp(8.0 + m, E - 10);
    return (byte & 0x80) ? -mag : mag;
}

/* IEEE-754 binary16 -> binary32: 1 sign bit, 5 exponent bits (bias 15), 10
 * fraction bits. Exponent 0: subnormal, value = frac * 2^-24. Exponent 31:
 * infinity (frac 0) or NaN. Otherwise (1024 + frac) * 2^(exp - 25). Every
 * binary16 value is exactly representable in binary32. */
float oracle_half_to_float(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25);
    }
    return (float)(sign ? -v : v);
}

/* bfloat16 -> binary32: the 16 bits are the upper half of the binary32. */
float oracle_bf16_to_float(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float x;
    memcpy(&x, &u, sizeof x);
    return x;
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* Q4_K sub-scale j and sub-min j (each 6 bits) from the 12-byte field s[].
 * GGUF layout: for j < 4 the sub-scale is the low 6 bits of s[j] and the
 * sub-min the low 6 bits of s[j+4]. For j >= 4 the low 4 bits of the
 * sub-scale are the low nibble of s[j+4] and its high 2 bits are the top 2
 * bits of s[j-4]; the low 4 bits of the sub-min are the high nibble of
 * s[j+4] and its high 2 bits the top 2 bits of s[j]. */
static void q4k_scale_min(const uint8_t *s, int j, int *sc, int *m) {
    if (j < 4) {
        *sc = s[j] & 63;
        *m = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

/* Decode one row of K elements. Returns 0, or -1 for an unknown type or a
 * K that is not a whole number of blocks. */
int oracle_decode_row(int type, const uint8_t *row, int64_t K, float *out) {
    int64_t k, b;
    switch (type) {
    case T_F32:
        memcpy(out, row, (size_t)K * 4);
        return 0;
    case T_F16:
        for (k = 0; k < K; k++) out[k] = oracle_half_to_float(rd16(row + 2 * k));
        return 0;
    case T_BF16:
        for (k = 0; k < K; k++) out[k] = oracle_bf16_to_float(rd16(row + 2 * k));
        return 0;
    case T_Q8_0:
        /* 34-byte block of 32 elements: fp16 scale d, then 32 int8 codes;
         * element j = d * code[j]. */
        if (K % 32) return -1;
        for (b = 0; b < K / 32; b++) {
            const uint8_t *blk = row + 34 * b;
            float d = oracle_half_to_float(rd16(blk));
            for (int j = 0; j < 32; j++) out[32 * b + j] = d * (float)(int8_t)blk[2 + j];
        }
        return 0;
    case T_Q4_0:
        /* 18-byte block of 32 elements: fp16 scale d, then 16 code bytes.
         * Element j < 16 is the low nibble of code byte j, element j + 16
         * its high nibble; value = d * (nibble - 8). */
        if (K % 32) return -1;
        for (b = 0; b < K / 32; b++) {
            const uint8_t *blk = row + 18 * b;
            float d = oracle_half_to_float(rd16(blk));
            for (int j = 0; j < 16; j++) {
                int lo = blk[2 + j] & 15, hi = blk[2 + j] >> 4;
                out[32 * b + j] = d * (float)(lo - 8);
                out[32 * b + j + 16] = d * (float)(hi - 8);
            }
        }
        return 0;
    case T_Q4_1:
    case T_Q5_0:
    case T_Q5_1: {
        /* 32-element blocks with an fp16 scale d, codes as in Q4_0 (element
         * j < 16 is the low nibble of code byte j, element j + 16 its high
         * nibble), and:
         *   Q4_1 (20 bytes): d, fp16 offset m, 16 code bytes; value d*q + m
         *   Q5_0 (22 bytes): d, 4 bytes qh, 16 code bytes; bit j of qh (a
         *     little-endian 32-bit word) is element j's fifth bit; value
         *     d*(q - 16)
         *   Q5_1 (24 bytes): d, m, qh, 16 code bytes; value d*q + m
         * d*q is exact in F32; the sum with m rounds once. */
        const int bytes = type == T_Q4_1 ? 20 : type == T_Q5_0 ? 22 : 24;
        const int has_m = type != T_Q5_0, has_qh = type != T_Q4_1;
        if (K % 32) return -1;
        for (b = 0; b < K / 32; b++) {
            const uint8_t *blk = row + bytes * b;
            float d = oracle_half_to_float(rd16(blk));
            float m = has_m ? oracle_half_to_float(rd16(blk + 2)) : 0.0f;
            const uint8_t *qhp = blk + (has_m ? 4 : 2);
            uint32_t qh = has_qh ? (uint32_t)qhp[0] | (uint32_t)qhp[1] << 8 | (uint32_t)qhp[2] << 16 |
                                       (uint32_t)qhp[3] << 24
                                 : 0;
            const uint8_t *qs = blk + bytes - 16;
            for (int j = 0; j < 32; j++) {
                int nib = j < 16 ? (qs[j] & 15) : (qs[j - 16] >> 4);
                int q = nib | (int)((qh >> j) & 1) << 4;
                if (type == T_Q5_0) {
                    out[32 * b + j] = d * (float)(q - 16);
                } else {
                    float v = d * (float)q;
                    out[32 * b + j] = v + m;
                }
            }
        }
        return 0;
    }
    case T_MXFP4:
        /* 17-byte block of 32 elements: an E8M0 scale byte e (the scale is
         * 2^(e - 127); e = 255 is NaN), then 16 code bytes. Element j < 16
         * is the low nibble of code byte j, element j + 16 its high nibble.
         * value = e2m1(code) * scale, formed exactly in double and rounded
         * once to F32 (exact unless it overflows). */
        if (K % 32) return -1;
        for (b = 0; b < K / 32; b++) {
            const uint8_t *blk = row + 17 * b;
            const double scale = blk[0] == 255 ? NAN : ldexp(1.0, (int)blk[0] - 127);
            for (int j = 0; j < 16; j++) {
                out[32 * b + j] = (float)(e2m1_value(blk[1 + j] & 15) * scale);
                out[32 * b + j + 16] = (float)(e2m1_value(blk[1 + j] >> 4) * scale);
            }
        }
        return 0;
    case T_NVFP4:
        /* 36-byte block of 64 elements: four E4M3 scale bytes, scale s for
         * the 16 elements 16s .. 16s + 15, then 32 code bytes, 8 per
         * sub-block: element 16s + i (i < 8) is the low nibble of code byte
         * 8s + i, element 16s + 8 + i its high nibble. value = e2m1(code) *
         * scale_s, exact in double (at most 2 + 4 significant bits) and
         * rounded once to F32, which is exact in range. */
        if (K % 64) return -1;
        for (b = 0; b < K / 64; b++) {
            const uint8_t *blk = row + 36 * b;
            for (int sb = 0; sb < 4; sb++) {
                const double scale = e4m3_value(blk[sb]);
                for (int i = 0; i < 8; i++) {
                    const int c = blk[4 + 8 * sb + i];
                    out[64 * b + 16 * sb + i] = (float)(e2m1_value(c & 15) * scale);
                    out[64 * b + 16 * sb + 8 + i] = (float)(e2m1_value(c >> 4) * scale);
                }
            }
        }
        return 0;
    case T_Q4_K:
        /* 144-byte super-block of 256 elements: fp16 d, fp16 dmin, 12 bytes
         * of sub-scales/sub-mins, 128 code bytes. Element e lies in 64-wide
         * chunk c = e / 64 at r = e % 64: for r < 32 its code is the low
         * nibble of code byte 32c + r and it uses sub-block 2c; otherwise
         * the high nibble of code byte 32c + r - 32, sub-block 2c + 1.
         * value = (d * sc_j) * q - (dmin * m_j), each product exact in F32,
         * one rounding in the subtraction. */
        if (K % 256) return -1;
        for (b = 0; b < K / 256; b++) {
            const uint8_t *blk = row + 144 * b;
            float d = oracle_half_to_float(rd16(blk));
            float dmin = oracle_half_to_float(rd16(blk + 2));
            const uint8_t *s = blk + 4;
            const uint8_t *qs = blk + 16;
            for (int e = 0; e < 256; e++) {
                int c = e / 64, r = e % 64, q, j, sc, m;
                if (r < 32) {
                    q = qs[32 * c + r] & 15;
                    j = 2 * c;
                } else {
                    q = qs[32 * c + r - 32] >> 4;
                    j = 2 * c + 1;
                }
                q4k_scale_min(s, j, &sc, &m);
                float a = d * (float)sc;
                float mm = dmin * (float)m;
                float v = a * (float)q;
                out[256 * b + e] = v - mm;
            }
        }
        return 0;
    case T_Q5_K:
        /* 176-byte super-block of 256 elements: fp16 d, fp16 dmin, the same
         * 12-byte sub-scale/sub-min field as Q4_K, 32 bytes qh holding each
         * element's fifth bit, 128 bytes qs of low nibbles. Element e lies
         * in chunk c = e / 64 at r = e % 64: for r < 32 its low 4 bits are
         * the low nibble of qs[32c + r], its fifth bit is bit 2c of qh[r],
         * and it uses sub-block 2c; otherwise the high nibble of
         * qs[32c + r - 32], bit 2c + 1 of qh[r - 32], sub-block 2c + 1.
         * value = (d * sc_j) * q - (dmin * m_j) with q in 0..31: each
         * product exact in F32, one rounding in the subtraction. */
        if (K % 256) return -1;
        for (b = 0; b < K / 256; b++) {
            const uint8_t *blk = row + 176 * b;
            float d = oracle_half_to_float(rd16(blk));
            float dmin = oracle_half_to_float(rd16(blk + 2));
            const uint8_t *s = blk + 4;
            const uint8_t *qh = blk + 16;
            const uint8_t *qs = blk + 48;
            for (int e = 0; e < 256; e++) {
                int c = e / 64, r = e % 64, q, j, sc, m;
                if (r < 32) {
                    q = (qs[32 * c + r] & 15) | (((qh[r] >> (2 * c)) & 1) << 4);
                    j = 2 * c;
                } else {
                    q = (qs[32 * c + r - 32] >> 4) | (((qh[r - 32] >> (2 * c + 1)) & 1) << 4);
                    j = 2 * c + 1;
                }
                q4k_scale_min(s, j, &sc, &m);
                float a = d * (float)sc;
                float mm = dmin * (float)m;
                float v = a * (float)q;
                out[256 * b + e] = v - mm;
            }
        }
        return 0;
    case T_Q6_K:
        /* 210-byte super-block of 256 elements: 128 bytes ql of low nibbles,
         * 64 bytes qh of 2-bit high parts, 16 signed 8-bit sub-scales (one
         * per 16 elements), fp16 d last. Element e lies in half h = e / 128,
         * quarter p = (e % 128) / 32, at l = e % 32: its low 4 bits are the
         * low (p < 2) or high (p >= 2) nibble of ql[64h + 32(p % 2) + l],
         * its high 2 bits are bits 2p and 2p + 1 of qh[32h + l], and its
         * sub-scale is scales[8h + 2p + l / 16]. value = (d * sc) * (q - 32)
         * with q in 0..63: the odd parts of d, sc and q - 32 have at most
         * 11, 7 and 5 bits, so the product is exact in F32. */
        if (K % 256) return -1;
        for (b = 0; b < K / 256; b++) {
            const uint8_t *blk = row + 210 * b;
            const uint8_t *ql = blk;
            const uint8_t *qh = blk + 128;
            const int8_t *sc = (const int8_t *)(blk + 192);
            float d = oracle_half_to_float(rd16(blk + 208));
            for (int e = 0; e < 256; e++) {
                int h = e / 128, p = (e % 128) / 32, l = e % 32;
                int lo = ql[64 * h + 32 * (p % 2) + l];
                lo = p < 2 ? (lo & 15) : (lo >> 4);
                int hi = (qh[32 * h + l] >> (2 * p)) & 3;
                int q = lo | (hi << 4);
                float a = d * (float)sc[8 * h + 2 * p + l / 16];
                out[256 * b + e] = a * (float)(q - 32);
            }
        }
        return 0;
    case T_Q2_K:
        /* 84-byte super-block of 256 elements: 16 bytes of 4-bit sub-scale
         * (low nibble) / sub-min (high nibble) pairs, 64 bytes qs of 2-bit
         * codes, fp16 d, fp16 dmin. Element e lies in half h = e / 128,
         * quarter p = (e % 128) / 32, at l = e % 32: its code is bits 2p and
         * 2p + 1 of qs[32h + l], its pair is byte 8h + 2p + l / 16.
         * value = (d * sc) * q - (dmin * m) with q in 0..3: each product
         * exact in F32, one rounding in the subtraction. */
        if (K % 256) return -1;
        for (b = 0; b < K / 256; b++) {
            const uint8_t *blk = row + 84 * b;
            const uint8_t *pairs = blk, *qs = blk + 16;
            float d = oracle_half_to_float(rd16(blk + 80));
            float dmin = oracle_half_to_float(rd16(blk + 82));
            for (int e = 0; e < 256; e++) {
                int h = e / 128, p = (e % 128) / 32, l = e % 32;
                int q = (qs[32 * h + l] >> (2 * p)) & 3;
                int pair = pairs[8 * h + 2 * p + l / 16];
                float a = d * (float)(pair & 15);
                float mm = dmin * (float)(pair >> 4);
                float v = a * (float)q;
                out[256 * b + e] = v - mm;
            }
        }
        return 0;
    case T_Q3_K:
        /* 110-byte super-block of 256 elements: 32 bytes hmask, 64 bytes qs
         * of 2-bit codes, 12 bytes of sixteen 6-bit sub-scales, fp16 d.
         * Element e lies in half h = e / 128, quarter p = (e % 128) / 32, at
         * l = e % 32: its low 2 bits are bits 2p, 2p + 1 of qs[32h + l]; bit
         * 4h + p of hmask[l] set means q = low, clear means q = low - 4 (q in
         * -4..3); its sub-scale is number 8h + 2p + l / 16. Sub-scale s
         * (0..15), with i = s % 4 and g = s / 4: low 4 bits are the low
         * (g < 2) or high (g >= 2) nibble of field byte 4 (g % 2) + i, high 2
         * bits are bits 2g, 2g + 1 of field byte 8 + i; it counts from -32.
         * value = (d * (sc - 32)) * q: at most 11 + 6 + 3 bits, exact. */
        if (K % 256) return -1;
        for (b = 0; b < K / 256; b++) {
            const uint8_t *blk = row + 110 * b;
            const uint8_t *hmask = blk, *qs = blk + 32, *f = blk + 96;
            float d = oracle_half_to_float(rd16(blk + 108));
            for (int e = 0; e < 256; e++) {
                int h = e / 128, p = (e % 128) / 32, l = e % 32;
                int low = (qs[32 * h + l] >> (2 * p)) & 3;
                int q = (hmask[l] >> (4 * h + p)) & 1 ? low : low - 4;
                int s = 8 * h + 2 * p + l / 16, i = s % 4, g = s / 4;
                int nib = f[4 * (g % 2) + i];
                nib = g < 2 ? (nib & 15) : (nib >> 4);
                int sc = nib | (((f[8 + i] >> (2 * g)) & 3) << 4);
                float a = d * (float)(sc - 32);
                out[256 * b + e] = a * (float)q;
            }
        }
        return 0;
    default:
        return -1;
    }
}

int64_t oracle_row_bytes(int type, int64_t K) {
    switch (type) {
    case T_F32: return 4 * K;
    case T_F16: case T_BF16: return 2 * K;
    case T_Q8_0: return K % 32 ? -1 : K / 32 * 34;
    case T_Q4_0: return K % 32 ? -1 : K / 32 * 18;
    case T_Q4_1: return K % 32 ? -1 : K / 32 * 20;
    case T_Q5_0: return K % 32 ? -1 : K / 32 * 22;
    case T_Q5_1: return K % 32 ? -1 : K / 32 * 24;
    case T_Q2_K: return K % 256 ? -1 : K / 256 * 84;
    case T_Q3_K: return K % 256 ? -1 : K / 256 * 110;
    case T_Q4_K: return K % 256 ? -1 : K / 256 * 144;
    case T_Q5_K: return K % 256 ? -1 : K / 256 * 176;
    case T_Q6_K: return K % 256 ? -1 : K / 256 * 210;
    case T_MXFP4: return K % 32 ? -1 : K / 32 * 17;
    case T_NVFP4: return K % 64 ? -1 : K / 64 * 36;
    default: return -1;
    }
}

/* Decode all N rows of W (row pitch = oracle_row_bytes) into out (N x K). */
int oracle_dequantize(int type, const uint8_t *W, int64_t K, int64_t N, float *out) {
    int64_t rb = oracle_row_bytes(type, K);
    if (rb < 0) return -1;
    for (int64_t n = 0; n < N; n++)
        if (oracle_decode_row(type, W + n * rb, K, out + n * K)) return -1;
    return 0;
}

enum { TBLOCK = 8 };

typedef struct {
    const float *w;        /* decoded W, N x K */
    const float *G;        /* T x N */
    const int64_t *rows;   /* which t rows to compute */
    int64_t nrows, K, N;
    float *dst;            /* nrows x K */
    double *acc, *abssum;  /* nrows x K */
    int tid, nthreads;
} job_t;

/* Rows [i0, i1) of the selected list: for n in increasing order, for each
 * row of the block and each k, add the double product w[n][k] * G[t][n]. */
static void contract_block(const job_t *j, int64_t i0, int64_t i1) {
    const int64_t K = j->K, N = j->N;
    for (int64_t i = i0; i < i1; i++) {
        memset(j->acc + i * K, 0, (size_t)K * sizeof(double));
        memset(j->abssum + i * K, 0, (size_t)K * sizeof(double));
    }
    for (int64_t n = 0; n < N; n++) {
        const float *wn = j->w + n * K;
        for (int64_t i = i0; i < i1; i++) {
            double g = (double)j->G[j->rows[i] * N + n];
            double *acc = j->acc + i * K;
            double *as = j->abssum + i * K;
            for (int64_t k = 0; k < K; k++) {
                double p = (double)wn[k] * g;
                acc[k] += p;
                as[k] += fabs(p);
            }
        }
    }
    for (int64_t i = i0; i < i1; i++)
        for (int64_t k = 0; k < K; k++) j->dst[i * K + k] = (float)j->acc[i * K + k];
}

static void *contract_worker(void *arg) {
    const job_t *j = (const job_t *)arg;
    int64_t nblocks = (j->nrows + TBLOCK - 1) / TBLOCK;
    for (int64_t blk = j->tid; blk < nblocks; blk += j->nthreads) {
        int64_t i0 = blk * TBLOCK;
        int64_t i1 = i0 + TBLOCK < j->nrows ? i0 + TBLOCK : j->nrows;
        contract_block(j, i0, i1);
    }
    return NULL;
}

/* dst[i][k] = sum_n W[n][k] * G[rows[i]][n] for the nrows selected t rows
 * (rows == NULL selects t = 0 .. nrows-1). acc receives the double sums,
 * abssum the double sums of |W[n][k] * G[t][n]|, dst the F32 rounding of
 * acc. Returns 0, or -1 on a bad type/K or an allocation failure. */
int oracle_out_prod(int type, const uint8_t *W, const float *G, int64_t K, int64_t N, int64_t T,
                    const int64_t *rows, int64_t nrows, float *dst, double *acc, double *abssum,
                    int nthreads) {
    if (oracle_row_bytes(type, K) < 0 || K < 0 || N < 0 || T < 0 || nrows < 0) return -1;
    if (K == 0 || nrows == 0) return 0;
    int64_t *own_rows = NULL;
    if (!rows) {
        if (nrows > T) return -1;
        own_rows = (int64_t *)malloc((size_t)nrows * sizeof(int64_t));
        if (!own_rows) return -1;
        for (int64_t i = 0; i < nrows; i++) own_rows[i] = i;
        rows = own_rows;
    }
    for (int64_t i = 0; i < nrows; i++)
        if (rows[i] < 0 || rows[i] >= T) { free(own_rows); return -1; }
    float *w = (float *)malloc((size_t)(N > 0 ? N : 1) * (size_t)K * sizeof(float));
    if (!w) { free(own_rows); return -1; }
    if (oracle_dequantize(type, W, K, N, w)) { free(w); free(own_rows); return -1; }

    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    job_t jobs[256];
    pthread_t th[256];
    for (int t = 0; t < nthreads; t++) {
        jobs[t] = (job_t){w, G, rows, nrows, K, N, dst, acc, abssum, t, nthreads};
    }
    int started = 0;
    for (int t = 1; t < nthreads; t++) {
        if (pthread_create(&th[t], NULL, contract_worker, &jobs[t]) != 0) break;
        started = t;
    }
    /* Any worker that failed to start has its blocks done here. */
    for (int t = started + 1; t < nthreads; t++) contract_worker(&jobs[t]);
    contract_worker(&jobs[0]);
    for (int t = 1; t <= started; t++) pthread_join(th[t], NULL);
    free(w);
    free(own_rows);
    return 0;
}

/* mul_mat, the forward of the layer whose input gradient out_prod computes
 * (the PR's commit message: the backward of mul_mat(W, x) with respect to x
 * is out_prod(W, grad^T)): y[t][n] = sum_k W[n][k] * x[t][k], with W[n][k]
 * the decoded value, for the nrows selected t rows (rows == NULL selects
 * t = 0 .. nrows-1). Products and sums in double, k increasing; acc gets the
 * sums, abssum the sums of |W[n][k] * x[t][k]|, y their F32 rounding, each
 * nrows x N. */
typedef struct {
    const float *w, *X;
    const int64_t *rows;
    int64_t nrows, K, N;
    float *y;
    double *acc, *abssum;
    int tid, nthreads;
} mm_job_t;

static void *mm_worker(void *arg) {
    const mm_job_t *j = (const mm_job_t *)arg;
    for (int64_t i = j->tid; i < j->nrows; i += j->nthreads) {
        const float *x = j->X + j->rows[i] * j->K;
        for (int64_t n = 0; n < j->N; n++) {
            const float *wn = j->w + n * j->K;
            double a = 0.0, s = 0.0;
            for (int64_t k = 0; k < j->K; k++) {
                double p = (double)wn[k] * (double)x[k];
                a += p;
                s += fabs(p);
            }
            j->acc[i * j->N + n] = a;
            j->abssum[i * j->N + n] = s;
            j->y[i * j->N + n] = (float)a;
        }
    }
    return NULL;
}

int oracle_mul_mat(int type, const uint8_t *W, const float *X, int64_t K, int64_t N, int64_t T,
                   const int64_t *rows, int64_t nrows, float *y, double *acc, double *abssum, int nthreads) {
    if (oracle_row_bytes(type, K) < 0 || K < 0 || N < 0 || T < 0 || nrows < 0) return -1;
    if (N == 0 || nrows == 0) return 0;
    int64_t *own_rows = NULL;
    if (!rows) {
        if (nrows > T) return -1;
        own_rows = (int64_t *)malloc((size_t)nrows * sizeof(int64_t));
        if (!own_rows) return -1;
        for (int64_t i = 0; i < nrows; i++) own_rows[i] = i;
        rows = own_rows;
    }
    for (int64_t i = 0; i < nrows; i++)
        if (rows[i] < 0 || rows[i] >= T) { free(own_rows); return -1; }
    float *w = (float *)malloc((size_t)N * (size_t)(K > 0 ? K : 1) * sizeof(float));
    if (!w) { free(own_rows); return -1; }
    if (oracle_dequantize(type, W, K, N, w)) { free(w); free(own_rows); return -1; }
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    mm_job_t jobs[256];
    pthread_t th[256];
    for (int t = 0; t < nthreads; t++) jobs[t] = (mm_job_t){w, X, rows, nrows, K, N, y, acc, abssum, t, nthreads};
    int started = 0;
    for (int t = 1; t < nthreads; t++) {
        if (pthread_create(&th[t], NULL, mm_worker, &jobs[t]) != 0) break;
        started = t;
    }
    for (int t = started + 1; t < nthreads; t++) mm_worker(&jobs[t]);
    mm_worker(&jobs[0]);
    for (int t = 1; t <= started; t++) pthread_join(th[t], NULL);
    free(w);
    free(own_rows);
    return 0;
}
