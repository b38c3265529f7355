// retro_mm_kernel.h - mul_mat, the forward y = x W^T of the layer whose
// input gradient OUT_PROD computes, through the same resident packed weight.
//
//     y[t][n] = sum_k W[n][k] * x[t][k]
//
// The reduction now runs along k, the direction the blocks are packed in,
// and the outputs are the rows of W. The kernel keeps the producer/consumer
// pipeline of out_prod_ws_kernel and its consumer waves unchanged (they see
// a t-major operand and a column-major operand of 32 reduction values per
// chunk, whatever the two indices mean); only the producers differ: per
// chunk of 32 k values they load x like G, and for each of the tile's W
// rows decode 32 consecutive elements of that row - one 32-element block,
// or one 32-element part of a 256-element super-block - writing each row's
// values as one column of the LDS operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "retro_ws_kernel.h"

namespace retro {

struct MmArgs {
    const uint8_t* W;
    const float* X;
    float* Y;
    int K, N, T;
    long long pitch;  // bytes between consecutive W rows
    long long ldx;    // floats between consecutive x rows (a multiple of 4)
    long long ldy;    // floats between consecutive y rows (>= N)
    int tiles_t, tiles_n, group;
};

// Loads and decode of 16 consecutive elements k .. k + 15 (k % 16 == 0) of
// one W row that starts at byte `ro` of buffer `wr`. All loads stay inside
// the row's blocks (dense rows: inside the row for k < K, and K % 4 == 0),
// so none straddles the end of W; rows at or past N read as zero.
template <int TYPE>
struct MmCodec;

template <>
struct MmCodec<kF32> {
    static constexpr int WORDS = 16;
    __device__ static void fetch(__amdgpu_buffer_rsrc_t wr, uint32_t ro, int k, uint32_t (&w)[WORDS]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(wr, ro + 4u * k + 16u * i, 0, 0);
            w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
        }
    }
    __device__ static void decode(const uint32_t (&w)[WORDS], int, float (&e)[16]) {
#pragma unroll
        for (int i = 0; i < 16; ++i) e[i] = __uint_as_float(w[i]);
    }
};

template <int TYPE>
struct MmCodecHalf {
    static constexpr int WORDS = 8;
    __device__ static void fetch(__amdgpu_buffer_rsrc_t wr, uint32_t ro, int k, uint32_t (&w)[WORDS]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(wr, ro + 2u * k + 16u * i, 0, 0);
            w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
        }
    }
    __device__ static void decode(const uint32_t (&w)[WORDS], int, float (&e)[16]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if constexpr (TYPE == kF16)
                f16x2(w[i], e[2 * i], e[2 * i + 1]);
            else
                bf16x2(w[i], e[2 * i], e[2 * i + 1]);
        }
    }
};
template <> struct MmCodec<kF16> : MmCodecHalf<kF16> {};
template <> struct MmCodec<kBF16> : MmCodecHalf<kBF16> {};

template <>
struct MmCodec<kQ8_0> {
    static constexpr int WORDS = 5;
    __device__ static void fetch(__amdgpu_buffer_rsrc_t wr, uint32_t ro, int k, uint32_t (&w)[WORDS]) {
        const uint32_t blk = ro + 34u * uint32_t(k >> 5);
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(wr, blk + 2u + 16u * ((k >> 4) & 1), 0, 0);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        w[4] = __builtin_amdgcn_raw_buffer_load_b16(wr, blk, 0, 0);
    }
    __device__ static void decode(const uint32_t (&w)[WORDS], int, float (&e)[16]) {
        const float d = half_to_f32(w[4] & 0xFFFFu);
#pragma unroll
        for (int i = 0; i < 4; ++i) q8_0_x4(w[i], d, e + 4 * i);
    }
};

// The 32-element nibble blocks and MXFP4: element j < 16 is the low nibble
// of code byte j, element j + 16 its high nibble.
template <int TYPE>
struct MmCodecNibble {
    static constexpr int HW = kHasFifth<TYPE> ? 2 : 1;
    static constexpr int WORDS = 4 + HW;
    __device__ static void fetch(__amdgpu_buffer_rsrc_t wr, uint32_t ro, int k, uint32_t (&w)[WORDS]) {
        const uint32_t blk = ro + uint32_t(Format<TYPE>::kBytes) * uint32_t(k >> 5);
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(wr, blk + kHeader<TYPE>, 0, 0);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        if constexpr (kHasFifth<TYPE>) {
            const u32x2 h = __builtin_amdgcn_raw_buffer_load_b64(wr, blk, 0, 0);
            w[4] = h.x;
            w[5] = h.y;
        } else if constexpr (TYPE == kQ4_1) {
            w[4] = __builtin_amdgcn_raw_buffer_load_b32(wr, blk, 0, 0);
        } else if constexpr (TYPE == kMXFP4) {
            w[4] = __builtin_amdgcn_raw_buffer_load_b8(wr, blk, 0, 0);
        } else {
            w[4] = __builtin_amdgcn_raw_buffer_load_b16(wr, blk, 0, 0);
        }
    }
    __device__ static void decode(const uint32_t (&w)[WORDS], int k, float (&e)[16]) {
        const bool high = ((k >> 4) & 1) != 0;  // elements 16 .. 31 of the block
        if constexpr (TYPE == kMXFP4) {
            const float s = mx_scale(w[4]);
#pragma unroll
            for (int i = 0; i < 4; ++i) mxfp4_x4(w[i], high, s, e + 4 * i);
        } else {
            float d, m;
            uint32_t qh;
            if constexpr (kHasFifth<TYPE>)
                nibble32_header<TYPE>(w[4], w[5], d, m, qh);
            else
                nibble32_header<TYPE>(w[4], 0u, d, m, qh);
            const int first = high ? 16 : 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) nibble32_x4<TYPE>(w[i], qh, first + 4 * i, d, m, e + 4 * i);
        }
    }
};
template <> struct MmCodec<kQ4_0> : MmCodecNibble<kQ4_0> {};
template <> struct MmCodec<kQ4_1> : MmCodecNibble<kQ4_1> {};
template <> struct MmCodec<kQ5_0> : MmCodecNibble<kQ5_0> {};
template <> struct MmCodec<kQ5_1> : MmCodecNibble<kQ5_1> {};
template <> struct MmCodec<kMXFP4> : MmCodecNibble<kMXFP4> {};

// NVFP4: a 16-element unit is one sub-block: its 8 code bytes (low nibbles
// are elements 0 .. 7, high nibbles 8 .. 15) and its E4M3 scale byte.
template <>
struct MmCodec<kNVFP4> {
    static constexpr int WORDS = 3;
    __device__ static void fetch(__amdgpu_buffer_rsrc_t wr, uint32_t ro, int k, uint32_t (&w)[WORDS]) {
        const uint32_t blk = ro + 36u * uint32_t(k >> 6);
        const uint32_t sb = uint32_t((k & 63) >> 4);
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(wr, blk + 4u + 8u * sb, 0, 0);
        w[0] = v.x;
        w[1] = v.y;
        w[2] = __builtin_amdgcn_raw_buffer_load_b8(wr, blk + sb, 0, 0);
    }
    __device__ static void decode(const uint32_t (&w)[WORDS], int, float (&e)[16]) {
        const float s = e4m3_to_f32(w[2]);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            float lo[4], hi[4];
            nvfp4_x8(w[i], s, lo, hi);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                e[4 * i + j] = lo[j];
                e[8 + 4 * i + j] = hi[j];
            }
        }
    }
};

// Q4_K / Q5_K: element e of a super-block lies in 64-element chunk c = e / 64
// at r = e % 64; its code is the low (r < 32) or high nibble of code byte
// 32c + r % 32, and it uses sub-block 2c + (r >= 32).
template <int TYPE>
struct MmCodecK45 {
    static constexpr bool kQ5 = TYPE == kQ5_K;
    static constexpr int WORDS = kQ5 ? 12 : 8;
    __device__ static void fetch(__amdgpu_buffer_rsrc_t wr, uint32_t ro, int k, uint32_t (&w)[WORDS]) {
        const uint32_t sb = ro + uint32_t(Format<TYPE>::kBytes) * uint32_t(k >> 8);
        const int e = k & 255, c = e >> 6, l = e & 31;
        const u32x4 cw = __builtin_amdgcn_raw_buffer_load_b128(wr, sb + (kQ5 ? 48u : 16u) + 32u * c + l, 0, 0);
        const u32x4 hd = __builtin_amdgcn_raw_buffer_load_b128(wr, sb, 0, 0);
        w[0] = cw.x; w[1] = cw.y; w[2] = cw.z; w[3] = cw.w;
        w[4] = hd.x; w[5] = hd.y; w[6] = hd.z; w[7] = hd.w;
        if constexpr (kQ5) {
            const u32x4 qh = __builtin_amdgcn_raw_buffer_load_b128(wr, sb + 16u + l, 0, 0);
            w[8] = qh.x; w[9] = qh.y; w[10] = qh.z; w[11] = qh.w;
        }
    }
    __device__ static void decode(const uint32_t (&w)[WORDS], int k, float (&e)[16]) {
        const int r = k & 63, c = (k & 255) >> 6;
        const bool high = r >= 32;
        const int j = 2 * c + (high ? 1 : 0);
        float a, b;
        q4_k_coeffs(w[4], w[5], w[6], w[7], j, a, b);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (kQ5)
                q5_k_x4(w[i], w[8 + i], j, high, a, b, e + 4 * i);
            else
                q4_k_x4(w[i], high, a, b, e + 4 * i);
        }
    }
};
template <> struct MmCodec<kQ4_K> : MmCodecK45<kQ4_K> {};
template <> struct MmCodec<kQ5_K> : MmCodecK45<kQ5_K> {};

// Q6_K, Q2_K, Q3_K: element e = 128 h + 32 p + l of a super-block, with
// sub-scale (Q2_K: pair) 8 h + 2 p + l / 16.
template <>
struct MmCodec<kQ6_K> {
    static constexpr int WORDS = 10;
    __device__ static void fetch(__amdgpu_buffer_rsrc_t wr, uint32_t ro, int k, uint32_t (&w)[WORDS]) {
        const uint32_t sb = ro + 210u * uint32_t(k >> 8);
        const int e = k & 255, h = e >> 7, p = (e >> 5) & 3, l = e & 31, si = 8 * h + 2 * p + (l >> 4);
        const u32x4 ql = __builtin_amdgcn_raw_buffer_load_b128(wr, sb + 64u * h + 32u * (p & 1) + l, 0, 0);
        const u32x4 qh = __builtin_amdgcn_raw_buffer_load_b128(wr, sb + 128u + 32u * h + l, 0, 0);
        w[0] = ql.x; w[1] = ql.y; w[2] = ql.z; w[3] = ql.w;
        w[4] = qh.x; w[5] = qh.y; w[6] = qh.z; w[7] = qh.w;
        w[8] = __builtin_amdgcn_raw_buffer_load_b32(wr, sb + 192u + uint32_t(si & ~3), 0, 0);
        w[9] = __builtin_amdgcn_raw_buffer_load_b16(wr, sb + 208u, 0, 0);
    }
    __device__ static void decode(const uint32_t (&w)[WORDS], int k, float (&e)[16]) {
        const int el = k & 255, h = el >> 7, p = (el >> 5) & 3, si = 8 * h + 2 * p + ((el & 31) >> 4);
        float a;
        q6_k_coeffs(w[8], si & 3, half_to_f32(w[9] & 0xFFFFu), a);
#pragma unroll
        for (int i = 0; i < 4; ++i) q6_k_x4(w[i], p >= 2, w[4 + i], p, a, e + 4 * i);
    }
};

template <>
struct MmCodec<kQ2_K> {
    static constexpr int WORDS = 6;
    __device__ static void fetch(__amdgpu_buffer_rsrc_t wr, uint32_t ro, int k, uint32_t (&w)[WORDS]) {
        const uint32_t sb = ro + 84u * uint32_t(k >> 8);
        const int e = k & 255, h = e >> 7, p = (e >> 5) & 3, l = e & 31, pi = 8 * h + 2 * p + (l >> 4);
        const u32x4 c = __builtin_amdgcn_raw_buffer_load_b128(wr, sb + 16u + 32u * h + l, 0, 0);
        w[0] = c.x; w[1] = c.y; w[2] = c.z; w[3] = c.w;
        w[4] = __builtin_amdgcn_raw_buffer_load_b32(wr, sb + uint32_t(pi & ~3), 0, 0);
        w[5] = __builtin_amdgcn_raw_buffer_load_b32(wr, sb + 80u, 0, 0);
    }
    __device__ static void decode(const uint32_t (&w)[WORDS], int k, float (&e)[16]) {
        const int el = k & 255, h = el >> 7, p = (el >> 5) & 3, pi = 8 * h + 2 * p + ((el & 31) >> 4);
        float a, b;
        q2_k_coeffs(w[4], pi & 3, half_to_f32(w[5] & 0xFFFFu), half_to_f32(w[5] >> 16), a, b);
#pragma unroll
        for (int i = 0; i < 4; ++i) q2_k_x4(w[i], p, a, b, e + 4 * i);
    }
};

template <>
struct MmCodec<kQ3_K> {
    static constexpr int WORDS = 12;
    __device__ static void fetch(__amdgpu_buffer_rsrc_t wr, uint32_t ro, int k, uint32_t (&w)[WORDS]) {
        const uint32_t sb = ro + 110u * uint32_t(k >> 8);
        const int e = k & 255, h = e >> 7, l = e & 31;
        const u32x4 qs = __builtin_amdgcn_raw_buffer_load_b128(wr, sb + 32u + 32u * h + l, 0, 0);
        const u32x4 hm = __builtin_amdgcn_raw_buffer_load_b128(wr, sb + l, 0, 0);
        const u32x2 f = __builtin_amdgcn_raw_buffer_load_b64(wr, sb + 96u, 0, 0);
        w[0] = qs.x; w[1] = qs.y; w[2] = qs.z; w[3] = qs.w;
        w[4] = hm.x; w[5] = hm.y; w[6] = hm.z; w[7] = hm.w;
        w[8] = f.x; w[9] = f.y;
        // field bytes 104 .. 107 and d at 108; nothing past the block
        w[10] = __builtin_amdgcn_raw_buffer_load_b32(wr, sb + 104u, 0, 0);
        w[11] = __builtin_amdgcn_raw_buffer_load_b16(wr, sb + 108u, 0, 0);
    }
    __device__ static void decode(const uint32_t (&w)[WORDS], int k, float (&e)[16]) {
        const int el = k & 255, h = el >> 7, p = (el >> 5) & 3, si = 8 * h + 2 * p + ((el & 31) >> 4);
        float a;
        q3_k_coeffs(w[8], w[9], w[10], si, half_to_f32(w[11] & 0xFFFFu), a);
#pragma unroll
        for (int i = 0; i < 4; ++i) q3_k_x4(w[i], w[4 + i], p, 4 * h + p, a, e + 4 * i);
    }
};

template <int TYPE, int WA, int WB, int CT, int NC_ = 4>
struct MmShape {
    using F = Format<TYPE>;
    static constexpr bool kDense = F::kBlock == 1;
    static constexpr int kPThreads = 256;
    // consumer waves: 4, or 8 for the 256 x 128 tile, whose producers' decode
    // then feeds twice the matrix work
    static constexpr int NC = NC_;
    static constexpr int kCThreads = 64 * NC;
    static constexpr int kThreads = kCThreads + kPThreads;
    static_assert((NC == 4 && (CT == 1 || CT == 2)) || (NC == 8 && CT == 4), "consumer grid 1x4, 2x2 or 4x2");
    static constexpr int CK = NC / CT;
    // consumers keep two operand sets (the next phase read during this one's
    // MFMAs) when the register budget allows
    static constexpr bool kPrefetch = NC == 4 || WA * WB <= 4;
    static constexpr int BT = 32 * WA * CT;  // rows of x per tile
    static constexpr int BK = 32 * WB * CK;  // rows of W (outputs) per tile
    // workgroups per CU the register budget is set for, and the same as waves
    // per SIMD for the launch bound (see WsShape)
    static constexpr int kWgPerCu = BT == 32 ? 2 : 1;
    static constexpr int kWavesPerSimd = kThreads / 64 / 4 * kWgPerCu;
    static constexpr int BN = 32;  // k values per chunk
    static constexpr int GP = BN + 4;
    static constexpr int WP = BN + 4;
    static constexpr int G_FLOATS = BT * GP;
    static constexpr int W_FLOATS = BK * WP;
    static constexpr int BUF_FLOATS = G_FLOATS + W_FLOATS;
    static constexpr int kResident = (160 * 1024) / (2 * BUF_FLOATS * 4) < 2 ? 1 : 2;
    static constexpr int GSLOTS = BT * BN / 4 / kPThreads;
    static_assert(GSLOTS * kPThreads * 4 == BT * BN, "x chunk splits evenly");
    // units of 16 elements of one W row per producer thread and chunk
    static constexpr int UNITS = BK * BN / 16 / kPThreads;
    static_assert(UNITS * kPThreads * 16 == BK * BN, "W chunk splits evenly");
    static constexpr int WWORDS = UNITS * MmCodec<TYPE>::WORDS;
    static constexpr int SLOT_REGS = 4 * GSLOTS + WWORDS;
    static constexpr int RING = SLOT_REGS <= 32 ? 4 : 2;
};

template <int TYPE, int WA, int WB, int CT, int NC>
__global__ __launch_bounds__((MmShape<TYPE, WA, WB, CT, NC>::kThreads),
                             (MmShape<TYPE, WA, WB, CT, NC>::kWavesPerSimd)) void mul_mat_ws_kernel(MmArgs args) {
    using S = MmShape<TYPE, WA, WB, CT, NC>;
    using C = MmCodec<TYPE>;
    constexpr int BT = S::BT, BK = S::BK, BN = S::BN, GP = S::GP, WP = S::WP;

    __shared__ __attribute__((aligned(16))) float lds_all[2 * S::BUF_FLOATS];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tt, tn;
    tile_coords(blockIdx.x, args.tiles_t, args.tiles_n, args.group, tt, tn);
    const int t0 = tt * BT, n0 = tn * BK;
    const int K = args.K, N = args.N, T = args.T;
    const int nloc = (K + BN - 1) / BN;

    if (wave >= NC) {
        // ---------------- producer ----------------
        const int p = tid - S::kCThreads;
        float* const lds = lds_all;
        constexpr int R = S::RING;
        float4 gring[R][S::GSLOTS];
        uint32_t wring[R][S::WWORDS];
        // x: slot s is t row id / 8, columns 4 (id % 8) .. + 3 of the chunk
        uint32_t goff[S::GSLOTS];
#pragma unroll
        for (int s = 0; s < S::GSLOTS; ++s) {
            const int id = p + S::kPThreads * s;
            goff[s] = uint32_t(((id >> 3) * args.ldx + 4 * (id & 7)) * 4);
        }
        // W: unit u is row id / 2 of the tile, elements 16 (id % 2) .. + 15
        // of the chunk, written as that row's column of the LDS operand
        uint32_t wro[S::UNITS];
        int wlds[S::UNITS][4], wk[S::UNITS];
#pragma unroll
        for (int u = 0; u < S::UNITS; ++u) {
            const int id = p + S::kPThreads * u, r = id >> 1, h = id & 1;
            wro[u] = uint32_t(r * args.pitch);
            wk[u] = 16 * h;
#pragma unroll
            for (int g = 0; g < 4; ++g) wlds[u][g] = ws_w_index<WP>(r, 16 * h + 4 * g);
        }
        const long long x_end = K == 0 ? 0 : (long long)(T - 1) * args.ldx + K;  // elements spanned by x
        const long long wb = (long long)n0 * args.pitch;
        const long long w_end =
            (long long)(N - 1) * args.pitch + (long long)(K / S::F::kBlock) * S::F::kBytes;
        const __amdgpu_buffer_rsrc_t wr =
            buffer_rsrc(args.W + wb, uint32_t(max(0ll, min(w_end - wb, (long long)0x7FFFFFFF))));

        // Chunk c covers k = 32 c .. 32 c + 31. Loads are issued the same way
        // for every chunk; x columns at or past K (the next row's values, or
        // a chunk past the last) are zeroed when written to LDS, and so are
        // the W values there (for dense rows they are the next row's; a
        // chunk past the last is never contracted).
        auto load_chunk = [&](auto slot, int c) {
            float4(&greg)[S::GSLOTS] = gring[decltype(slot)::value];
            uint32_t(&wreg)[S::WWORDS] = wring[decltype(slot)::value];
            const int k0 = __builtin_amdgcn_readfirstlane(c * BN);
            const long long xb = (long long)t0 * args.ldx + k0;
            const __amdgpu_buffer_rsrc_t xr =
                buffer_rsrc(args.X + xb, uint32_t(max(0ll, min(4 * (x_end - xb), (long long)0x7FFFFFFF))));
#pragma unroll
            for (int s = 0; s < S::GSLOTS; ++s) {
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(xr, goff[s], 0, 0);
                greg[s] = make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                                      __uint_as_float(v.w));
            }
            // a chunk past the last one reads the last chunk again (its
            // values are never used); no load leaves the row
            const int kc = max(0, min(k0, (nloc - 1) * BN));
#pragma unroll
            for (int u = 0; u < S::UNITS; ++u) {
                uint32_t(&w)[C::WORDS] = *reinterpret_cast<uint32_t(*)[C::WORDS]>(wreg + u * C::WORDS);
                C::fetch(wr, wro[u], kc + wk[u], w);
            }
        };

        auto store_chunk = [&](auto slot, auto buf, int c) {
            float4(&greg)[S::GSLOTS] = gring[decltype(slot)::value];
            const uint32_t(&wreg)[S::WWORDS] = wring[decltype(slot)::value];
            float* gs = lds + decltype(buf)::value * S::BUF_FLOATS;
            float* ws = gs + S::G_FLOATS;
            const int k0 = c * BN;
            if (k0 + BN > K) {
#pragma unroll
                for (int s = 0; s < S::GSLOTS; ++s) {
                    const int k = k0 + 4 * ((p + S::kPThreads * s) & 7);
                    if (k >= K) greg[s].x = 0.f;
                    if (k + 1 >= K) greg[s].y = 0.f;
                    if (k + 2 >= K) greg[s].z = 0.f;
                    if (k + 3 >= K) greg[s].w = 0.f;
                }
            }
#pragma unroll
            for (int s = 0; s < S::GSLOTS; ++s) {
                const int id = p + S::kPThreads * s;
                *reinterpret_cast<float4*>(gs + (id >> 3) * GP + 4 * (id & 7)) = greg[s];
            }
            const int kc = max(0, min(k0, (nloc - 1) * BN));
#pragma unroll
            for (int u = 0; u < S::UNITS; ++u) {
                const uint32_t(&w)[C::WORDS] = *reinterpret_cast<const uint32_t(*)[C::WORDS]>(wreg + u * C::WORDS);
                float e[16];
                C::decode(w, kc + wk[u], e);
                if (k0 + BN > K) {
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (k0 + wk[u] + i >= K) e[i] = 0.f;
                }
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *reinterpret_cast<float4*>(ws + wlds[u][g]) =
                        make_float4(e[4 * g], e[4 * g + 1], e[4 * g + 2], e[4 * g + 3]);
            }
        };

        using Zero = std::integral_constant<int, 0>;
        static_for<R>([&](auto i) { load_chunk(i, i); });
        store_chunk(Zero{}, Zero{}, 0);
        __syncthreads();
        auto step = [&](auto i, int c) {
            constexpr int I = decltype(i)::value;
            store_chunk(std::integral_constant<int, (I + 1) % R>{}, std::integral_constant<int, (I + 1) & 1>{},
                        c + 1);
            load_chunk(i, c + R);
            __syncthreads();
        };
        int c0 = 0;
        for (; c0 + R <= nloc; c0 += R) static_for<R>([&](auto i) { step(i, c0 + decltype(i)::value); });
        static_for<R>([&](auto i) {
            if (c0 + decltype(i)::value < nloc) step(i, c0 + decltype(i)::value);
        });
        return;
    }

    // ---------------- consumer ----------------
    ws_consume<S, WA, WB, 1>(lds_all, tid, wave, nloc, t0, n0, T, N, args.Y, args.ldy);
}

// mul_mat for T <= 16 TB a launch (the host runs one launch per 64 rows of
// x): one workgroup (NW = 8 or 16 waves) per 16 rows of W over all of k,
// v_mfma_f32_16x16x4_f32 with M = t, N = W row, K = 4 steps of k.
// Iteration g of a wave covers k = 64 g .. 64 g + 63: lane l decodes the 16
// elements 64 g + 16 (l / 16) .. + 15 of row n0 + l % 16 (one MmCodec unit,
// one header decode) and, for each block of 16 rows of x, takes the same 16
// x values of row t = 16 tb + l % 16, and round r, step s of the block's 16
// MFMAs uses element 4 r + s: the decode is shared by all TB blocks. x goes
// through a tile of the wave's own in LDS: loaded with 16 lanes per 256-byte
// row segment (the MFMA layout would give each lane its own 64-byte region
// and keep the address unit busy four times as long), then read back in the
// MFMA layout. The next iteration's loads are issued before the current one
// is decoded. Partial sums are added over waves in increasing wave order in
// LDS (the x tiles' space, once the loop is done).
template <int TYPE, int NW, int TB>
__global__ __launch_bounds__(NW * 64) void mul_mat_skinny_kernel(MmSimpleArgs a) {
    static_assert(NW >= 4, "the final sum uses 256 threads");
    using C = MmCodec<TYPE>;
    using F = Format<TYPE>;
    constexpr int XP = 68;  // floats per t row of a wave's x tile (64 + 4: conflict-free reads)
    constexpr int XT = NW * 16 * TB * XP, PT = NW * 256 * TB;
    __shared__ __attribute__((aligned(16))) float lds[XT > PT ? XT : PT];
    float* const part = lds;  // after the loop
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = blockIdx.x * 16;
    const int j = lane & 15, kk = lane >> 4;
    const int K = a.K;
    // W rows n0 .. n0 + 15 (rows at or past N read as zero); x rows t (t at
    // or past T read as zero: x rows are K floats apart)
    const long long wb = (long long)n0 * a.pitch;
    const long long w_end = (long long)(a.N - 1) * a.pitch + (long long)(K / F::kBlock) * F::kBytes;
    const __amdgpu_buffer_rsrc_t wr =
        buffer_rsrc(a.W + wb, uint32_t(max(0ll, min(w_end - wb, (long long)0x7FFFFFFF))));
    const long long x_end = K == 0 ? 0 : (long long)(a.T - 1) * a.ldx + K;
    const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(a.X, uint32_t(max(0ll, min(4 * x_end, (long long)0x7FFFFFFF))));
    const uint32_t ro = uint32_t(j * a.pitch);
    // x load i of an iteration: row 4 i + l / 16 of its block of 16, floats
    // 4 (l % 16) .. + 3 of the iteration's 64
    uint32_t xo[TB][4];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) xo[tb][i] = uint32_t(((16 * tb + 4 * i + kk) * a.ldx + 4 * j) * 4);
    float* const xt = lds + wave * 16 * TB * XP;
    const int groups = (K + 63) / 64;

    uint32_t wraw[2][C::WORDS];
    u32x4 xraw[2][TB][4];
    // Loads of group g into slot S: always issued (a group past the last
    // reads bytes it never uses), so that they stay in flight.
    auto fetch = [&](auto slot, int g) {
        constexpr int S = decltype(slot)::value;
        const int k = 64 * g + 16 * kk;
        C::fetch(wr, ro, k, wraw[S]);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                xraw[S][tb][i] = __builtin_amdgcn_raw_buffer_load_b128(xr, xo[tb][i] + 256u * g, 0, 0);
    };
    f32x4 acc[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](auto slot, int g) {
        constexpr int S = decltype(slot)::value;
        const int k = 64 * g + 16 * kk;
        float e[16];
        // the x tile through LDS; the fences keep the wave's LDS accesses in
        // program order (the previous iteration's reads before these writes,
        // these writes before the reads below)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<u32x4*>(xt + (16 * tb + 4 * i + kk) * XP + 4 * j) = xraw[S][tb][i];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // x of block tb, row t = 16 tb + l % 16, in the MFMA layout
        auto read_x = [&](int tb, float* xv) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(xt + (16 * tb + j) * XP + 16 * kk + 4 * i);
                xv[4 * i] = v[0];
                xv[4 * i + 1] = v[1];
                xv[4 * i + 2] = v[2];
                xv[4 * i + 3] = v[3];
            }
        };
        // the first block's x reads are in flight during the decode, each
        // later block's during the previous block's MFMAs
        float xv[2][16];
        read_x(0, xv[0]);
        C::decode(wraw[S], k, e);
        const bool tail = k + 16 > K;  // elements at or past K: zero on both sides
        if (tail) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (k + i >= K) e[i] = 0.f;
        }
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            float* cur = xv[tb & 1];
            if (tb + 1 < TB) read_x(tb + 1, xv[(tb + 1) & 1]);
            if (tail) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (k + i >= K) cur[i] = 0.f;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[tb] = __builtin_amdgcn_mfma_f32_16x16x4f32(cur[i], e[i], acc[tb], 0, 0, 0);
        }
    };
    using Slot0 = std::integral_constant<int, 0>;
    using Slot1 = std::integral_constant<int, 1>;
    int g = wave;
    if (g < groups) {
        fetch(Slot0{}, g);
        for (; g < groups; g += 2 * NW) {
            fetch(Slot1{}, g + NW);
            compute(Slot0{}, g);
            if (g + NW >= groups) break;
            fetch(Slot0{}, g + 2 * NW);
            compute(Slot1{}, g + NW);
        }
    }
    // D layout: lane l, register v holds t = 16 tb + 4 (l / 16) + v, row n0 + l % 16
    __syncthreads();  // every wave is done with its x tile
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int v = 0; v < 4; ++v) part[(wave * TB + tb) * 256 + (4 * kk + v) * 16 + j] = acc[tb][v];
    __syncthreads();
    for (int o = tid; o < 256 * TB; o += NW * 64) {
        const int tb = o >> 8, r = o & 255;
        const int t = 16 * tb + (r >> 4), nn = r & 15;
        float sum = part[tb * 256 + r];
#pragma unroll
        for (int w = 1; w < NW; ++w) sum += part[(w * TB + tb) * 256 + r];
        if (t < a.T && n0 + nn < a.N) a.Y[(long long)t * a.ldy + n0 + nn] = sum;
    }
}

}  // namespace retro
