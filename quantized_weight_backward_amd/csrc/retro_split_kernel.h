// retro_split_kernel.h - OUT_PROD on bf16 MFMA with exact operands ("exact
// split"): a variant that trades the F32-input MFMA for the bf16
// matrix rate, keeping every product exact and every sum in F32. Written out
// below for Q4_K; Q5_K adds a fifth code bit (v < 2048), Q6_K has
// v = sc*(q - 32) and no min term, Q2_K has v = sc*q <= 45 (one bf16 part) and
// 16 sub-blocks of mins, Q3_K has v = (sc - 32)*q' with |v| <= 128 (one part)
// and no min term. For Q4_0, Q5_0, MXFP4, BF16 and F16 v is the decoded weight
// itself (at most 16 significant bits), A = G, on a 128-column tile.
//
// A Q4_K element of row n, sub-block j of a super-block is
// d*sc_j*q - dmin*m_j (q a nibble, sc_j and m_j 6-bit integers, d and dmin
// fp16). Over one super-block of columns the contraction splits as
//
//   dst[t][k] = sum_n (G[t][n]*d[n]) * v[n][k]  -  sum_n (G[t][n]*dmin[n]) * m_j(k)[n]
//
// with v = sc_j*q an integer below 1024. Each factor is made exact in bf16:
//   * v = hi + lo with hi its top 8 significant bits and lo the rest (at most
//     2 bits, as v < 1024);
//   * m_j, at most 6 bits, as it is;
//   * A = fl(G*d) and E = fl(G*dmin), single F32 roundings, each cut into
//     three bf16 parts (the top 8, the next 8 and the last 8 significant
//     bits: A = A0 + A1 + A2 exactly).
// The main term is then six bf16 MFMAs (A0, A1, A2 times hi and lo), the
// min term three (E0, E1, E2 times m). Products of bf16 values are exact;
// the matrix core adds them in F32 arithmetic (measured on gfx950: it keeps
// about F32 precision relative to the largest product of one instruction and
// truncates). Against the F32-input path the result differs by the two
// roundings of A and E and by that addition, all at F32 level.
//
// Organisation as in out_prod_ws_kernel (8 waves: 4 consumers, each 32 rows
// by all BK columns of a 128 x BK tile, BK = 256 for the K-quants and 128 for
// the others; 4 producers; G and the decoded W double buffered in LDS, one
// barrier per 32-row chunk). The producers write G (F32), d and dmin per row,
// the parts of v (bf16, k-major with the 32 rows of a column contiguous) and
// m (bf16); the consumers form the A and E parts in registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "retro_ws_kernel.h"

namespace retro {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// The weight types the exact split takes, and its tile width: whole
// super-blocks (256 columns) for the K-quants, 128 columns (four 32-element
// blocks, or dense columns) for the others.
template <int TYPE>
constexpr bool kSplitNarrow = TYPE == kQ4_0 || TYPE == kQ5_0 || TYPE == kMXFP4 || TYPE == kBF16 || TYPE == kF16;
template <int TYPE>
constexpr int kSplitBK = kSuperBlock<TYPE> ? 256 : 128;

template <int BK_>
struct SplitShape {
    static constexpr int kPThreads = 256;
    static constexpr int kThreads = 512;
    static constexpr int BT = 128, BK = BK_, BN = 32;
    static constexpr int GP = BN + 4;          // floats per t row of G
    static constexpr int G_FLOATS = BT * GP;   // 4608
    static constexpr int D_OFF = G_FLOATS;     // d of the chunk's 32 rows
    static constexpr int DM_OFF = D_OFF + BN;  // dmin
    // bf16 operands, counted in floats (two bf16 each)
    static constexpr int B_OFF = DM_OFF + BN;             // hi, lo: 2 x BK columns x 32 rows
    static constexpr int B_PART = BK * BN / 2;            // floats per part
    static constexpr int M_OFF = B_OFF + 2 * B_PART;      // m: 16 columns x 32 rows (8 used but for Q2_K)
    static constexpr int BUF_FLOATS = M_OFF + 16 * BN / 2;
    static constexpr int GSLOTS = BT * BN / 4 / kPThreads;  // 4
};

// Float offset, inside a part of the bf16 W operand, of the 8-byte group
// holding rows 4 r4 .. 4 r4 + 3 of column col. A column's 32 rows are four
// 16-byte units; unit u sits at position u ^ ((col >> 2) & 3), so that the
// 16 columns a quarter wave reads hit distinct banks.
__device__ __forceinline__ int split_b_index(int col, int r4) {
    return col * 16 + 4 * ((r4 >> 1) ^ ((col >> 2) & 3)) + 2 * (r4 & 1);
}

// The bf16 bits of an exactly representable float (its upper half).
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// x (8 floats) -> three bf16x8 parts with x = p0 + p1 + p2 exactly: p0 keeps
// the top 16 bits of x (sign, exponent, 7 fraction bits), p1 the same of the
// remainder, p2 the last remainder (at most 8 significant bits).
__device__ __forceinline__ void split3(const float (&x)[8], bf16x8& p0, bf16x8& p1, bf16x8& p2) {
    uint32_t w0[4], w1[4], w2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float h[2], m[2], r[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float v = x[2 * i + e];
            h[e] = __uint_as_float(__float_as_uint(v) & 0xFFFF0000u);
            const float r1 = v - h[e];
            m[e] = __uint_as_float(__float_as_uint(r1) & 0xFFFF0000u);
            r[e] = r1 - m[e];
        }
        w0[i] = bf16_pair(h[0], h[1]);
        w1[i] = bf16_pair(m[0], m[1]);
        w2[i] = bf16_pair(r[0], r[1]);
    }
    p0 = __builtin_bit_cast(bf16x8, u32x4{w0[0], w0[1], w0[2], w0[3]});
    p1 = __builtin_bit_cast(bf16x8, u32x4{w1[0], w1[1], w1[2], w1[3]});
    p2 = __builtin_bit_cast(bf16x8, u32x4{w2[0], w2[1], w2[2], w2[3]});
}

template <int TYPE>
// one 8-wave workgroup per CU: 2 waves per SIMD (amdgpu_waves_per_eu)
__global__ __launch_bounds__(512, 2) void out_prod_split_kernel(TileArgs args) {
    static_assert(kSuperBlock<TYPE> || kSplitNarrow<TYPE>, "no exact split for this type");
    constexpr bool kKQ = kSuperBlock<TYPE>;
    // sub-blocks of the min term per super-block (Q3_K and Q6_K values have none)
    constexpr int kMinCols = (TYPE == kQ4_K || TYPE == kQ5_K) ? 8 : TYPE == kQ2_K ? 16 : 0;
    constexpr bool kMin = kMinCols > 0;
    // bf16 parts of v: two for Q4_K, Q5_K (v < 2048) and Q6_K (|v| <= 4096),
    // one for Q2_K (v <= 45) and Q3_K (|v| <= 128). For the other types v is
    // the weight itself: one part for BF16 and MXFP4 (at most 2 significant
    // bits), two for F16 (11), Q4_0 (d (q - 8): 15) and Q5_0 (d (q - 16): 16).
    constexpr int kBParts = (TYPE == kQ2_K || TYPE == kQ3_K || TYPE == kBF16 || TYPE == kMXFP4) ? 1 : 2;
    // the K-quants take A = fl(G d) per super-block; the others A = G
    constexpr bool kScaleA = kKQ;
    constexpr bool kQ45 = TYPE == kQ4_K || TYPE == kQ5_K;
    constexpr uint32_t kCodes = TYPE == kQ5_K ? 48 : 16;  // first code byte of a super-block
    using S = SplitShape<kSplitBK<TYPE>>;
    using F = Format<TYPE>;
    constexpr int BT = S::BT, BK = S::BK, BN = S::BN, GP = S::GP;
    constexpr int NB = BK / 32;  // 32-column blocks of the tile

    __shared__ __attribute__((aligned(16))) float lds[2 * S::BUF_FLOATS];

    enter_batch(args);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tt, tk;
    tile_coords(blockIdx.x, args.tiles_t, args.tiles_k, args.group, tt, tk);
    const int t0 = tt * BT, k0 = tk * BK;
    const int K = args.K, N = args.N, T = args.T;
    const int nloc = (N + BN - 1) / BN;

    if (wave >= 4) {
        // ---------------- producer ----------------
        const int p = tid - S::kPThreads;
        // the m operand's unused columns 8..15 hold zeros (Q4_K, Q5_K; Q2_K
        // writes all 16 with each chunk)
        if (kMinCols == 8 && p < 2 * 8 * BN / 2) {
            const int b = p / (8 * BN / 2), o = p % (8 * BN / 2);
            lds[b * S::BUF_FLOATS + S::M_OFF + 8 * BN / 2 + o] = 0.f;
        }
        const long long kb0 = (long long)(k0 / F::kBlock) * F::kBytes;
        // G: slot s is t row id / 8, columns 4 (id % 8) .. + 3 (id = p + 256 s)
        uint32_t goff[S::GSLOTS];
#pragma unroll
        for (int s = 0; s < S::GSLOTS; ++s) {
            const int id = p + S::kPThreads * s;
            goff[s] = uint32_t(((id >> 3) * args.ldg + 4 * (id & 7)) * 4);
        }
        // W: rows 4 r4 .. 4 r4 + 3 of the chunk, code word w of each (bytes
        // 16 + 4w .. of the super-block: low nibbles are columns
        // 64 (w / 8) + 4 (w % 8) + 0..3 of sub-block 2 (w / 8), high nibbles
        // the same plus 32, of sub-block 2 (w / 8) + 1)
        // Q6_K instead: half h = w / 16 of the super-block, elements
        // l = 2 (w % 16) + e (e = 0, 1) of its four quarters qq: columns
        // 128 h + 32 qq + l.
        // The 128-column types: slot w = 2 u + f, the low (f = 0) or high
        // (f = 1) nibbles of code word u % 4 of block u / 4 (columns
        // 32 (u / 4) + 16 f + 4 (u % 4) + 0..3), or dense columns 4 w .. + 3.
        const int r4 = p >> 5, w = p & 31;
        uint32_t roff[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) roff[i] = uint32_t((4 * r4 + i) * args.pitch);
        // elements spanned by G (none when N = 0: G is empty and its pointer
        // may be null)
        const long long g_end = N == 0 ? 0 : (long long)(T - 1) * args.ldg + N;
        const long long w_end =
            N > 0 ? (long long)(N - 1) * args.pitch + (long long)(K / F::kBlock) * F::kBytes : 0;

        constexpr int R = 2;
        float4 gring[R][S::GSLOTS];
        uint32_t hring[R][4][4];  // Q4_K, Q5_K, per row: d | dmin << 16, the three scale words
        uint32_t cring[R][4];     // Q4_K, Q5_K, per row: the code word
        uint32_t fring[R][4];     // Q5_K, per row: the fifth-bit bytes of the code word's elements
        // Q6_K, per row: ql bytes (quarters 0, 2), (1, 3), qh bytes, 8 scales, d;
        // Q2_K: qs bytes, the 16 pair bytes, d | dmin << 16;
        // Q3_K: hmask bytes, qs bytes, the 12-byte scale field, d;
        // Q4_0, Q5_0, MXFP4: the code word, d or the scale byte, the fifth
        // bits; BF16, F16: the row's 8 columns
        uint32_t q6ring[R][4][6];

        auto load_chunk = [&](auto slot, int n0) __attribute__((always_inline)) {
            constexpr int I = decltype(slot)::value;
            n0 = __builtin_amdgcn_readfirstlane(n0);
            const long long gb = (long long)t0 * args.ldg + n0;
            const __amdgpu_buffer_rsrc_t gr =
                buffer_rsrc(args.G + gb, uint32_t(max(0ll, min(4 * (g_end - gb), (long long)0x7FFFFFFF))));
#pragma unroll
            for (int s = 0; s < S::GSLOTS; ++s) {
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(gr, goff[s], 0, 0);
                gring[I][s] = make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                                          __uint_as_float(v.w));
            }
            const long long wb = (long long)n0 * args.pitch + kb0;
            const __amdgpu_buffer_rsrc_t wr =
                buffer_rsrc(args.W + wb, uint32_t(max(0ll, min(w_end - wb, (long long)0x7FFFFFFF))));
            if constexpr (kQ45) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const u32x4 h = __builtin_amdgcn_raw_buffer_load_b128(wr, roff[i], 0, 0);
                    hring[I][i][0] = h.x;
                    hring[I][i][1] = h.y;
                    hring[I][i][2] = h.z;
                    hring[I][i][3] = h.w;
                    cring[I][i] = __builtin_amdgcn_raw_buffer_load_b32(wr, roff[i] + kCodes + 4 * w, 0, 0);
                    // qh bytes 4 (w % 8) .. + 3 hold the fifth bits of the word's bytes
                    if constexpr (TYPE == kQ5_K)
                        fring[I][i] = __builtin_amdgcn_raw_buffer_load_b32(wr, roff[i] + 16 + 4 * (w & 7), 0, 0);
                }
            } else if constexpr (TYPE == kQ6_K) {
                // super-blocks are 2-byte aligned; the 8-byte load of the
                // scales relies on the unaligned buffer access of gfx9-class GPUs
                const uint32_t hb = 64 * (w >> 4), lb = 2 * (w & 15);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    q6ring[I][i][0] = __builtin_amdgcn_raw_buffer_load_b16(wr, roff[i] + hb + lb, 0, 0);
                    q6ring[I][i][1] = __builtin_amdgcn_raw_buffer_load_b16(wr, roff[i] + hb + 32 + lb, 0, 0);
                    q6ring[I][i][2] = __builtin_amdgcn_raw_buffer_load_b16(wr, roff[i] + 128 + hb / 2 + lb, 0, 0);
                    const u32x2 sc = __builtin_amdgcn_raw_buffer_load_b64(wr, roff[i] + 192 + hb / 8, 0, 0);
                    q6ring[I][i][3] = sc.x;
                    q6ring[I][i][4] = sc.y;
                    q6ring[I][i][5] = __builtin_amdgcn_raw_buffer_load_b16(wr, roff[i] + 208, 0, 0);
                }
            } else if constexpr (TYPE == kQ2_K) {
                // 84-byte super-blocks: 16 pair bytes, 64 code bytes, d, dmin.
                // The lane's elements use pair bytes 8 h + w % 16 / 8 + 2 qq
                // (qq = 0..3): the 8 bytes from 8 h, shifted so that these are
                // bytes 0, 2, 4, 6; its sub-min is the high nibble of pair byte w.
                const uint32_t lb = 32 * (w >> 4) + 2 * (w & 15);
                const uint32_t sh = 8 * ((w >> 3) & 1);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    q6ring[I][i][0] = __builtin_amdgcn_raw_buffer_load_b16(wr, roff[i] + 16 + lb, 0, 0);
                    const u32x2 pr = __builtin_amdgcn_raw_buffer_load_b64(wr, roff[i] + 8 * (w >> 4), 0, 0);
                    const uint64_t p64 = ((uint64_t(pr.y) << 32) | pr.x) >> sh;
                    q6ring[I][i][1] = uint32_t(p64);
                    q6ring[I][i][2] = uint32_t(p64 >> 32);
                    q6ring[I][i][3] = __builtin_amdgcn_raw_buffer_load_b8(wr, roff[i] + (w & 15), 0, 0);
                    q6ring[I][i][5] = __builtin_amdgcn_raw_buffer_load_b32(wr, roff[i] + 80, 0, 0);
                }
            } else if constexpr (TYPE == kQ3_K) {
                // 110-byte super-blocks: 32 hmask bytes, 64 code bytes, the
                // 12-byte scale field, d (no load reaches past the block)
                const uint32_t lb = 2 * (w & 15);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    q6ring[I][i][0] = __builtin_amdgcn_raw_buffer_load_b16(wr, roff[i] + lb, 0, 0);
                    q6ring[I][i][1] = __builtin_amdgcn_raw_buffer_load_b16(wr, roff[i] + 32 + 32 * (w >> 4) + lb, 0, 0);
                    const u32x2 f = __builtin_amdgcn_raw_buffer_load_b64(wr, roff[i] + 96, 0, 0);
                    q6ring[I][i][2] = f.x;
                    q6ring[I][i][3] = f.y;
                    q6ring[I][i][4] = __builtin_amdgcn_raw_buffer_load_b32(wr, roff[i] + 104, 0, 0);
                    q6ring[I][i][5] = __builtin_amdgcn_raw_buffer_load_b16(wr, roff[i] + 108, 0, 0);
                }
            } else if constexpr (kNibbleLayout<TYPE>) {
                // Q4_0 (18-byte blocks: d, 16 code bytes), Q5_0 (22 bytes: d,
                // the 4 fifth-bit bytes, 16 code bytes), MXFP4 (17 bytes: the
                // scale byte, 16 code bytes): 2- or 1-byte aligned blocks,
                // read with unaligned buffer loads. Per row: the code word,
                // d (or the scale byte), the fifth bits.
                const int u = w >> 1;
                const uint32_t blk = uint32_t(F::kBytes) * uint32_t(u >> 2);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    q6ring[I][i][0] =
                        __builtin_amdgcn_raw_buffer_load_b32(wr, roff[i] + blk + kHeader<TYPE> + 4 * (u & 3), 0, 0);
                    if constexpr (TYPE == kMXFP4)
                        q6ring[I][i][1] = __builtin_amdgcn_raw_buffer_load_b8(wr, roff[i] + blk, 0, 0);
                    else
                        q6ring[I][i][1] = __builtin_amdgcn_raw_buffer_load_b16(wr, roff[i] + blk, 0, 0);
                    if constexpr (TYPE == kQ5_0)
                        q6ring[I][i][2] = __builtin_amdgcn_raw_buffer_load_b32(wr, roff[i] + blk + 2, 0, 0);
                }
            } else {
                // BF16, F16: columns 4 w .. 4 w + 3 of each row, one 8-byte load
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(wr, roff[i] + 8 * w, 0, 0);
                    q6ring[I][i][0] = v.x;
                    q6ring[I][i][1] = v.y;
                }
            }
        };

        auto store_chunk = [&](auto slot, auto buf, int n0) __attribute__((always_inline)) {
            constexpr int I = decltype(slot)::value;
            float* const base = lds + decltype(buf)::value * S::BUF_FLOATS;
            // G rows as loaded; columns at or past N (the next row's values in
            // the last chunk) zeroed
            if (n0 + BN > N) {
#pragma unroll
                for (int s = 0; s < S::GSLOTS; ++s) {
                    const int n = n0 + 4 * ((p + S::kPThreads * s) & 7);
                    if (n >= N) gring[I][s].x = 0.f;
                    if (n + 1 >= N) gring[I][s].y = 0.f;
                    if (n + 2 >= N) gring[I][s].z = 0.f;
                    if (n + 3 >= N) gring[I][s].w = 0.f;
                }
            }
#pragma unroll
            for (int s = 0; s < S::GSLOTS; ++s) {
                const int id = p + S::kPThreads * s;
                *reinterpret_cast<float4*>(base + (id >> 3) * GP + 4 * (id & 7)) = gring[I][s];
            }
            if constexpr (kQ45) {
                // d, dmin (words w = 8, 9) and m_w (w < 8) of the four rows
                if (w == 8 || w == 9) {
                    float4 v;
                    v.x = half_to_f32(w == 8 ? (hring[I][0][0] & 0xFFFFu) : (hring[I][0][0] >> 16));
                    v.y = half_to_f32(w == 8 ? (hring[I][1][0] & 0xFFFFu) : (hring[I][1][0] >> 16));
                    v.z = half_to_f32(w == 8 ? (hring[I][2][0] & 0xFFFFu) : (hring[I][2][0] >> 16));
                    v.w = half_to_f32(w == 8 ? (hring[I][3][0] & 0xFFFFu) : (hring[I][3][0] >> 16));
                    *reinterpret_cast<float4*>(base + (w == 8 ? S::D_OFF : S::DM_OFF) + 4 * r4) = v;
                } else if (w < 8) {
                    float m[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        uint32_t sc, mm;
                        q4_k_scale_min(hring[I][i][1], hring[I][i][2], hring[I][i][3], w, sc, mm);
                        m[i] = static_cast<float>(mm);
                    }
                    // column w, rows 4 r4 .. + 3 (plain k-major, 16 floats per column)
                    *reinterpret_cast<uint2*>(base + S::M_OFF + w * 16 + 2 * r4) =
                        make_uint2(bf16_pair(m[0], m[1]), bf16_pair(m[2], m[3]));
                }
                // v = sc * q of 8 columns x 4 rows (exact in F32: below 1024 for
                // Q4_K, 2048 for Q5_K), split as hi = its top 8 significant bits
                // and lo = v - hi (at most 3 bits), both exact in bf16
                const int c = w >> 3, j0 = 4 * (w & 7);
                float sc_lo[4], sc_hi[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    uint32_t sl, sh, mm;
                    q4_k_scale_min(hring[I][i][1], hring[I][i][2], hring[I][i][3], 2 * c, sl, mm);
                    q4_k_scale_min(hring[I][i][1], hring[I][i][2], hring[I][i][3], 2 * c + 1, sh, mm);
                    sc_lo[i] = static_cast<float>(sl);
                    sc_hi[i] = static_cast<float>(sh);
                }
                float* const hi_part = base + S::B_OFF;
                float* const lo_part = hi_part + S::B_PART;
#pragma unroll
                for (int half = 0; half < 2; ++half) {
#pragma unroll
                    for (int beta = 0; beta < 4; ++beta) {
                        // byte b of the code words; rotated by lane so that the 16
                        // lanes of a quarter wave write distinct banks
                        const int b = (beta + (w >> 2)) & 3;
                        float vh[4], vl[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            uint32_t qi = (cring[I][i] >> (8 * b + 4 * half)) & 15u;
                        if constexpr (TYPE == kQ5_K)  // bit 2c (low nibbles) or 2c + 1 (high) of qh byte
                            qi |= ((fring[I][i] >> (8 * b + 2 * c + half)) & 1u) << 4;
                        const float q = static_cast<float>(qi);
                            const float v = q * (half ? sc_hi[i] : sc_lo[i]);
                            vh[i] = __uint_as_float(__float_as_uint(v) & 0xFFFF0000u);
                            vl[i] = v - vh[i];
                        }
                        const int col = 64 * c + 32 * half + j0 + b;
                        const int o = split_b_index(col, r4);
                        *reinterpret_cast<uint2*>(hi_part + o) = make_uint2(bf16_pair(vh[0], vh[1]), bf16_pair(vh[2], vh[3]));
                        *reinterpret_cast<uint2*>(lo_part + o) = make_uint2(bf16_pair(vl[0], vl[1]), bf16_pair(vl[2], vl[3]));
                    }
                }
            } else if constexpr (TYPE == kQ6_K) {
                // d of the four rows (word w = 8)
                if (w == 8)
                    *reinterpret_cast<float4*>(base + S::D_OFF + 4 * r4) =
                        make_float4(half_to_f32(q6ring[I][0][5]), half_to_f32(q6ring[I][1][5]),
                                    half_to_f32(q6ring[I][2][5]), half_to_f32(q6ring[I][3][5]));
                // v = sc * (q - 32) of 8 columns x 4 rows (|v| <= 4096, exact in
                // F32), split as hi = its top 8 significant bits and lo = v - hi
                // (at most 5 bits), both exact in bf16. Element l = 2 (w % 16) + e
                // of quarter qq: ql byte l of quarter pair qq % 2 (high nibble for
                // qq >= 2), bits 2 qq .. of qh byte l, scale 2 qq + l / 16.
                const int h = w >> 4, jl = w & 15;
                float* const hi_part = base + S::B_OFF;
                float* const lo_part = hi_part + S::B_PART;
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        float vh[4], vl[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const uint32_t ql = q6ring[I][i][qq & 1] >> (8 * e + 4 * (qq >> 1));
                            const uint32_t qh = q6ring[I][i][2] >> (8 * e + 2 * qq);
                            const int q = int((ql & 15u) | ((qh & 3u) << 4)) - 32;
                            const int si = 2 * qq + (jl >> 3);  // scale byte within the half's 8
                            const int sc = int(int8_t((q6ring[I][i][3 + (si >> 2)] >> (8 * (si & 3))) & 0xFFu));
                            const float v = static_cast<float>(sc * q);
                            vh[i] = __uint_as_float(__float_as_uint(v) & 0xFFFF0000u);
                            vl[i] = v - vh[i];
                        }
                        const int col = 128 * h + 32 * qq + 2 * jl + e;
                        const int o = split_b_index(col, r4);
                        *reinterpret_cast<uint2*>(hi_part + o) =
                            make_uint2(bf16_pair(vh[0], vh[1]), bf16_pair(vh[2], vh[3]));
                        *reinterpret_cast<uint2*>(lo_part + o) =
                            make_uint2(bf16_pair(vl[0], vl[1]), bf16_pair(vl[2], vl[3]));
                    }
                }
            } else if constexpr (TYPE == kQ2_K || TYPE == kQ3_K) {
                // Q2_K and Q3_K: one bf16 part. Element l = 2 (w % 16) + e of
                // quarter qq of half h = w / 16: code bits 2 qq .. of code byte
                // 32 h + l, sub-scale 8 h + 2 qq + l / 16 (and, for Q3_K, bit
                // 4 h + qq of hmask byte l).
                const int h = w >> 4, jl = w & 15;
                if (w == 8 || (TYPE == kQ2_K && w == 9)) {
                    float4 v;
                    if constexpr (TYPE == kQ2_K) {
                        const int sh = w == 8 ? 0 : 16;
                        v = make_float4(half_to_f32((q6ring[I][0][5] >> sh) & 0xFFFFu),
                                        half_to_f32((q6ring[I][1][5] >> sh) & 0xFFFFu),
                                        half_to_f32((q6ring[I][2][5] >> sh) & 0xFFFFu),
                                        half_to_f32((q6ring[I][3][5] >> sh) & 0xFFFFu));
                    } else {
                        v = make_float4(half_to_f32(q6ring[I][0][5]), half_to_f32(q6ring[I][1][5]),
                                        half_to_f32(q6ring[I][2][5]), half_to_f32(q6ring[I][3][5]));
                    }
                    *reinterpret_cast<float4*>(base + (w == 8 ? S::D_OFF : S::DM_OFF) + 4 * r4) = v;
                }
                if constexpr (TYPE == kQ2_K) {
                    // sub-min m_w (high nibble of pair byte w) of the four rows
                    if (w < 16) {
                        float m[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) m[i] = static_cast<float>((q6ring[I][i][3] >> 4) & 15u);
                        *reinterpret_cast<uint2*>(base + S::M_OFF + w * 16 + 2 * r4) =
                            make_uint2(bf16_pair(m[0], m[1]), bf16_pair(m[2], m[3]));
                    }
                }
                float* const hi_part = base + S::B_OFF;
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        float v[4];
                        const int si = 8 * h + 2 * qq + (jl >> 3);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            if constexpr (TYPE == kQ2_K) {
                                const uint32_t q = (q6ring[I][i][0] >> (8 * e + 2 * qq)) & 3u;
                                const uint32_t sc = (q6ring[I][i][1 + (qq >> 1)] >> (16 * (qq & 1))) & 15u;
                                v[i] = static_cast<float>(sc * q);
                            } else {
                                const int q = int((q6ring[I][i][1] >> (8 * e + 2 * qq)) & 3u) - 4 +
                                              4 * int((q6ring[I][i][0] >> (8 * e + 4 * h + qq)) & 1u);
                                const int sc = int(q3_k_scale(q6ring[I][i][2], q6ring[I][i][3], q6ring[I][i][4], si)) - 32;
                                v[i] = static_cast<float>(sc * q);
                            }
                        }
                        const int col = 128 * h + 32 * qq + 2 * jl + e;
                        *reinterpret_cast<uint2*>(hi_part + split_b_index(col, r4)) =
                            make_uint2(bf16_pair(v[0], v[1]), bf16_pair(v[2], v[3]));
                    }
                }
            } else if constexpr (kNibbleLayout<TYPE>) {
                // v = d (q - 8) (Q4_0), d (q - 16) (Q5_0, q with its fifth bit)
                // or the E2M1 value times the scale (MXFP4), exact in F32;
                // byte e of the code word holds element 4 (u % 4) + e (low
                // nibble) or that plus 16 (high nibble) of block u / 4
                const int u = w >> 1, f = w & 1, blk = u >> 2, wb = u & 3;
                float* const hi_part = base + S::B_OFF;
                float* const lo_part = hi_part + S::B_PART;
                float val[4][4];  // [row][byte]: the value of this thread's nibble
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t cw = q6ring[I][i][0] >> (4 * f);  // the thread's nibbles in the low halves
                    if constexpr (TYPE == kMXFP4) {
                        float unused[4];
                        mxfp4_x8(cw, mx_scale(q6ring[I][i][1]), val[i], unused);
                    } else {
                        const float d = half_to_f32(q6ring[I][i][1] & 0xFFFFu);
                        constexpr int kOff = TYPE == kQ5_0 ? 16 : 8;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            int q = int((cw >> (8 * e)) & 15u);
                            if constexpr (TYPE == kQ5_0) q |= int((q6ring[I][i][2] >> (16 * f + 4 * wb + e)) & 1u) << 4;
                            val[i][e] = d * static_cast<float>(q - kOff);
                        }
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float vh[4], vl[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        vh[i] = __uint_as_float(__float_as_uint(val[i][e]) & 0xFFFF0000u);
                        vl[i] = val[i][e] - vh[i];
                    }
                    const int o = split_b_index(32 * blk + 16 * f + 4 * wb + e, r4);
                    *reinterpret_cast<uint2*>(hi_part + o) = make_uint2(bf16_pair(vh[0], vh[1]), bf16_pair(vh[2], vh[3]));
                    if constexpr (kBParts == 2)
                        *reinterpret_cast<uint2*>(lo_part + o) =
                            make_uint2(bf16_pair(vl[0], vl[1]), bf16_pair(vl[2], vl[3]));
                }
            } else {
                // BF16: the weights are the bf16 operand (halfword e % 2 of
                // word e / 2 of each row); F16: exact in F32, split as hi =
                // its top 8 significant bits and lo = the rest (at most 3)
                float* const hi_part = base + S::B_OFF;
                float* const lo_part = hi_part + S::B_PART;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int o = split_b_index(4 * w + e, r4);
                    const int wd = e >> 1;
                    if constexpr (TYPE == kBF16) {
                        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                        *reinterpret_cast<uint2*>(hi_part + o) =
                            make_uint2(__builtin_amdgcn_perm(q6ring[I][1][wd], q6ring[I][0][wd], sel),
                                       __builtin_amdgcn_perm(q6ring[I][3][wd], q6ring[I][2][wd], sel));
                    } else {
                        float vh[4], vl[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float v = half_to_f32((q6ring[I][i][wd] >> (16 * (e & 1))) & 0xFFFFu);
                            vh[i] = __uint_as_float(__float_as_uint(v) & 0xFFFF0000u);
                            vl[i] = v - vh[i];
                        }
                        *reinterpret_cast<uint2*>(hi_part + o) =
                            make_uint2(bf16_pair(vh[0], vh[1]), bf16_pair(vh[2], vh[3]));
                        *reinterpret_cast<uint2*>(lo_part + o) =
                            make_uint2(bf16_pair(vl[0], vl[1]), bf16_pair(vl[2], vl[3]));
                    }
                }
            }
        };

        using Zero = std::integral_constant<int, 0>;
        static_for<R>([&](auto i) { load_chunk(i, decltype(i)::value * BN); });
        store_chunk(Zero{}, Zero{}, 0);
        __syncthreads();
        auto step = [&](auto i, int c) __attribute__((always_inline)) {
            constexpr int I = decltype(i)::value;
            store_chunk(std::integral_constant<int, (I + 1) % R>{}, std::integral_constant<int, (I + 1) & 1>{},
                        (c + 1) * BN);
            load_chunk(i, (c + R) * BN);
            __syncthreads();
        };
        int c0 = 0;
        for (; c0 + R <= nloc; c0 += R) static_for<R>([&](auto i) { step(i, c0 + decltype(i)::value); });
        static_for<R>([&](auto i) {
            if (c0 + decltype(i)::value < nloc) step(i, c0 + decltype(i)::value);
        });
        __syncthreads();  // the consumers' exchange of the min term
        return;
    }

    // ---------------- consumer ----------------
    // wave w: tile rows 32 w .. 32 w + 31, all BK columns (NB blocks of 32)
    const int lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int wt = wave;
    f32x16 acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[b][v] = 0.f;
    f32x4 accm[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) accm[a] = f32x4{0.f, 0.f, 0.f, 0.f};

    // B operand offsets (floats) of the lane's columns, per k-step s
    int boff[2][NB];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int col = 32 * b + l32;
            boff[s][b] = S::B_OFF + col * 16 + 4 * ((2 * s + h) ^ ((col >> 2) & 3));
        }

    auto contract = [&](const float* base) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int n = 16 * s + 8 * h;
            bf16x8 ap[3];
            {
                const float* g = base + (32 * wt + l32) * GP + n;
                const f32x4 g0 = *reinterpret_cast<const f32x4*>(g);
                const f32x4 g1 = *reinterpret_cast<const f32x4*>(g + 4);
                float x[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[e] = g0[e];
                    x[4 + e] = g1[e];
                }
                if constexpr (kScaleA) {
                    const f32x4 d0 = *reinterpret_cast<const f32x4*>(base + S::D_OFF + n);
                    const f32x4 d1 = *reinterpret_cast<const f32x4*>(base + S::D_OFF + n + 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[e] *= d0[e];
                        x[4 + e] *= d1[e];
                    }
                }
                split3(x, ap[0], ap[1], ap[2]);
            }
            // the column blocks in groups of 4 (operands of one group live)
#pragma unroll
            for (int half = 0; half < NB / 4; ++half) {
                bf16x8 bp[4][kBParts];
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int q = 0; q < kBParts; ++q)
                        bp[b][q] = *reinterpret_cast<const bf16x8*>(base + boff[s][4 * half + b] + q * S::B_PART);
#pragma unroll
                for (int q = 0; q < kBParts; ++q)
#pragma unroll
                    for (int pa = 0; pa < 3; ++pa)
#pragma unroll
                        for (int b = 0; b < 4; ++b)
                            acc[4 * half + b] =
                                __builtin_amdgcn_mfma_f32_32x32x16_bf16(ap[pa], bp[b][q], acc[4 * half + b], 0, 0, 0);
            }
        }
        // min term: t rows 32 wt + 16 a + l % 16, all 32 rows n of the chunk
        // (n = 8 (l / 16) + 0..7), columns j = l % 16 (kMinCols used)
        if constexpr (kMin) {
            const int n = 8 * (lane >> 4);
            const f32x4 m0 = *reinterpret_cast<const f32x4*>(base + S::DM_OFF + n);
            const f32x4 m1 = *reinterpret_cast<const f32x4*>(base + S::DM_OFF + n + 4);
            const bf16x8 mb = *reinterpret_cast<const bf16x8*>(base + S::M_OFF + (lane & 15) * 16 + 4 * (lane >> 4));
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                const float* g = base + (32 * wt + 16 * a + (lane & 15)) * GP + n;
                const f32x4 g0 = *reinterpret_cast<const f32x4*>(g);
                const f32x4 g1 = *reinterpret_cast<const f32x4*>(g + 4);
                float x[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[e] = g0[e] * m0[e];
                    x[4 + e] = g1[e] * m1[e];
                }
                bf16x8 ep[3];
                split3(x, ep[0], ep[1], ep[2]);
#pragma unroll
                for (int pa = 0; pa < 3; ++pa)
                    accm[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ep[pa], mb, accm[a], 0, 0, 0);
            }
        }
    };

    __syncthreads();
    for (int c = 0; c < nloc; c += 2) {
        contract(lds);
        __syncthreads();
        if (c + 1 < nloc) {
            contract(lds + S::BUF_FLOATS);
            __syncthreads();
        }
    }

    // the min term of the wave's rows, columns (sub-blocks) 0 .. kMinCols - 1,
    // through LDS (D layout of the 16 x 16 product: lane l, register i holds
    // row 4 (l / 16) + i, column l % 16); each wave reads back its own rows
    float* const mins = lds + 32 * 16 * wt;
    if (kMin && (lane & 15) < kMinCols) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int i = 0; i < 4; ++i) mins[(16 * a + 4 * (lane >> 4) + i) * 16 + (lane & 15)] = accm[a][i];
    }
    __syncthreads();
    // D layout of the 32 x 32 product: lane l, register v holds row
    // 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32. Column block b is
    // sub-block b (32 columns) or, for Q2_K, sub-blocks 2b and 2b + 1.
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int k = k0 + 32 * b + l32;
        const int j = kMinCols == 16 ? 2 * b + (l32 >> 4) : b;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int tl = 8 * (v >> 2) + 4 * h + (v & 3);
            const int t = t0 + 32 * wt + tl;
            if (t < T && k < K) args.dst[(long long)t * args.ldd + k] = kMin ? acc[b][v] - mins[tl * 16 + j] : acc[b][v];
        }
    }
}

}  // namespace retro
