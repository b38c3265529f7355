// retro_kernels.h - OUT_PROD kernels for gfx950 (MI355X).
//
//   dst[t][k] = sum_n W[n][k] * G[t][n]
//
// As a GEMM: M = T (rows of G), N_gemm = K (columns of W), and the reduction
// runs over n, across the rows of W. The block-quantized direction k is the
// output-column direction, so one decoded weight feeds T outputs.
//
// Four kernels:
//   tile     fused decode -> LDS -> v_mfma_f32_32x32x2_f32, one BT x BK tile of
//            dst per workgroup, loop over n in chunks of 32 rows of W.
//   skinny   T <= 64 a launch: v_mfma_f32_16x16x4_f32 with M = 16 rows of G
//            per block, one 64-column slab of dst per workgroup, all of n
//            inside the workgroup (waves split n and reduce through LDS in a
//            fixed order), one pass over W.
//   skinny split  the same, with n cut into one equal share per CU and the
//            parts of a slab added through a caller's workspace.
//   dequant  decode-only, for bit-exact checks of the decoders.
// None allocates memory and none materialises a decoded copy of W.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "retro_decode.h"

namespace retro {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Staging helpers
// ---------------------------------------------------------------------------

// Buffer resource over [base, base + bytes): gfx9 descriptor, raw 32-bit
// access, no stride. Loads at or past `bytes` return zero instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Four bytes starting at any LDS address: the two aligned words around
// them, funnel-shifted (reads at most 4 bytes past the last one).
__device__ __forceinline__ uint32_t lds_word_a1(const uint8_t* p) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    const uint32_t* q = reinterpret_cast<const uint32_t*>(a & ~uintptr_t(3));
    return __builtin_amdgcn_alignbyte(q[1], q[0], uint32_t(a & 3));
}

// Four code bytes starting at a 2-byte aligned LDS address.
__device__ __forceinline__ uint32_t lds_word_a2(const uint8_t* p) {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(p);
    return uint32_t(q[0]) | (uint32_t(q[1]) << 16);
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup b runs on
// XCD b % 8), and each XCD has its own L2. xcd_remap turns a workgroup id
// into a logical index such that every XCD owns one contiguous range of
// logical indices (a bijection on [0, n)), so neighbouring logical work items
// share their XCD's L2.
__device__ __forceinline__ int xcd_remap(int b, int n) {
    const int per = n >> 3, rem = n & 7;
    const int x = b & 7, i = b >> 3;
    return x * per + (x < rem ? x : rem) + i;
}

// Logical tile -> (row tile, column tile), in groups of `height` row tiles
// (row tile fastest), so that the tiles an XCD runs at once share rows of G
// and columns of W. The host picks the height that minimises the estimated
// fetch of G and W for the shape.
__device__ __forceinline__ void tile_coords(int b, int tiles_t, int tiles_k, int height, int& tt, int& tk) {
    const int lin = xcd_remap(b, tiles_t * tiles_k);
    const int span = height * tiles_k;
    const int group = lin / span;
    const int first = group * height;
    const int gsize = min(tiles_t - first, height);
    const int in = lin - group * span;
    tt = first + in % gsize;
    tk = in / gsize;
}

// ---------------------------------------------------------------------------
// Tiled kernel
// ---------------------------------------------------------------------------

// Batches over two outer dimensions (i2 < ne2, i3 < ne3 with ne2 * ne3 =
// gridDim.y): batch (i2, i3) reads W matrix (i2 / r2, i3 / r3), which
// broadcasts one W matrix over r2 x r3 batches, and G and dst matrix (i2, i3).
// Matrices are w2 / w3 bytes (W) and g2 / g3, d2 / d3 floats (G, dst) apart.
struct BatchArgs {
    int ne2, r2, r3;
    long long w2, w3, g2, g3, d2, d3;
};

// Moves the three base pointers to this workgroup's batch (blockIdx.y).
template <typename Args>
__device__ __forceinline__ void enter_batch(Args& a) {
    const int b = blockIdx.y;
    const int i2 = b % a.batch.ne2, i3 = b / a.batch.ne2;
    a.W += (long long)(i3 / a.batch.r3) * a.batch.w3 + (long long)(i2 / a.batch.r2) * a.batch.w2;
    a.G += (long long)i3 * a.batch.g3 + (long long)i2 * a.batch.g2;
    a.dst += (long long)i3 * a.batch.d3 + (long long)i2 * a.batch.d2;
}

struct TileArgs {
    const uint8_t* W;
    const float* G;
    float* dst;
    int K, N, T;
    long long pitch;  // bytes between consecutive W rows
    int wvec;         // W staging load width (16, 8, 4, 2)
    int gvec;         // 1: G rows take float4 loads (ldg % 4 == 0, not gcols)
    int gcols;        // 1: G is stored t-fastest (the columns of G are contiguous)
    int tiles_t, tiles_k;
    int group;        // row tiles per group of the tile order (tile_coords)
    long long ldg;    // G[t][n] at t * ldg + n (ldg >= N), or at n * ldg + t when gcols (ldg >= T)
    long long ldd;    // floats between consecutive dst rows (>= K)
    BatchArgs batch;
};

// Column swizzle of a decoded W tile in LDS: XOR column bits 2-4 with
// higher bits, chosen per format so that the decode stores of one wave (8
// lanes per LDS cycle, each writing a float4 at a format-specific stride) hit
// distinct banks. Bits 0-1 are untouched (float4 stores stay contiguous) and
// bits 5 and up are untouched (the 32 consecutive columns an MFMA operand
// read covers stay inside their 32-word group, so those reads stay
// conflict-free).
template <int TYPE>
__device__ __forceinline__ int lds_swizzle(int col) {
    if constexpr (TYPE == kQ4_K || TYPE == kQ5_K) return col ^ (((col >> 6) & 3) << 2);
    if constexpr (kNibbleLayout<TYPE> || TYPE == kNVFP4 || TYPE == kQ6_K || TYPE == kQ2_K || TYPE == kQ3_K)
        return col ^ (((col >> 5) & 7) << 2);
    if constexpr (TYPE == kQ8_0) return col ^ (((col >> 5) & 3) << 2);
    return col;
}

template <int TYPE, int WA, int WB, int WGT, int WGK>
struct TileShape {
    using F = Format<TYPE>;
    static constexpr int kThreads = 256;
    static_assert(WGT * WGK == 4, "four waves per workgroup");
    static constexpr int BT = 32 * WA * WGT;  // rows of T per tile
    static constexpr int BK = 32 * WB * WGK;  // columns of K per tile
    static constexpr int BN = 32;             // rows of W per chunk
    static_assert(BK % F::kBlock == 0, "a K tile holds whole blocks");
    static constexpr bool kDense = F::kBlock == 1;
    // G chunk in LDS: BT rows of 32 floats, reduction index permuted (see
    // kernel), row stride 36 floats: float4 fragment reads are conflict-free.
    static constexpr int GP = BN + 4;
    // Decoded W chunk in LDS: 32 rows of BK floats, row stride BK + 32 so the
    // two lane halves of an MFMA operand read (rows 2s and 2s+1) hit disjoint
    // banks.
    static constexpr int BP = BK + 32;
    // Packed W bytes of one full tile row, in 16-byte units.
    static constexpr int SPAN = BK / F::kBlock * F::kBytes;
    static constexpr int UPR = (SPAN + 15) / 16;
    static constexpr int RAWP = UPR * 16 + 16;  // raw row stride in LDS (bytes)
    static constexpr int WUNITS = BN * UPR;
    // Packed formats are staged through LDS as raw bytes (their blocks need
    // not be 16-byte aligned) and decoded from there.
    static constexpr bool kStaged = !kDense;
    static constexpr int WSLOTS = (WUNITS + kThreads - 1) / kThreads;
    static constexpr int GSLOTS = BT * BN / 4 / kThreads;
    static_assert(GSLOTS * kThreads * 4 == BT * BN, "G chunk splits evenly");
    static constexpr int GE = F::kGroup;
    static constexpr int GPR = BK / GE;  // decode groups per row
    static constexpr int DPASS = (BN * GPR + kThreads - 1) / kThreads;
    static __device__ __forceinline__ int swz(int col) { return lds_swizzle<TYPE>(col); }
    static constexpr int LDS_G = BT * GP * 4;
    static constexpr int LDS_B = BN * BP * 4;
    static constexpr int LDS_RAW = kStaged ? BN * RAWP : 0;
};

template <int TYPE, int WA, int WB, int WGT, int WGK>
// two 4-wave workgroups per CU: 2 waves per SIMD (amdgpu_waves_per_eu)
__global__ __launch_bounds__(256, 2) void out_prod_tile_kernel(TileArgs args) {
    using S = TileShape<TYPE, WA, WB, WGT, WGK>;
    using F = Format<TYPE>;
    constexpr int BT = S::BT, BK = S::BK, BN = S::BN, GP = S::GP, BP = S::BP;

    __shared__ __attribute__((aligned(16))) float Gs[BT * GP];
    __shared__ __attribute__((aligned(16))) float Bs[BN * BP];
    __shared__ __attribute__((aligned(16))) uint8_t Raw[S::kStaged ? S::LDS_RAW : 16];

    enter_batch(args);
    const int tid = threadIdx.x;
    int tt, tk;
    tile_coords(blockIdx.x, args.tiles_t, args.tiles_k, args.group, tt, tk);
    const int t0 = tt * BT, k0 = tk * BK;
    const int K = args.K, N = args.N, T = args.T;
    // Byte offset of this tile's k range inside one W row.
    const long long kb0 = (long long)(k0 / F::kBlock) * F::kBytes;

    float4 greg[S::GSLOTS];
    uint4 wreg[S::WSLOTS];

    // Byte offsets of this thread's staging loads from the chunk's buffer
    // bases (the same for every chunk and tile): G slot s covers tile row
    // r = id / 8, columns 4*(id % 8) .. +3 of the chunk (the four elements
    // gstep bytes apart); W slot s covers 16-byte unit u of tile row r.
    uint32_t goff[S::GSLOTS], woff[S::WSLOTS];
    const uint32_t gstep = args.gcols ? uint32_t(4 * args.ldg) : 4u;
#pragma unroll
    for (int s = 0; s < S::GSLOTS; ++s) {
        const int id = tid + S::kThreads * s;
        const long long r = id >> 3, c = 4 * (id & 7);
        goff[s] = uint32_t((args.gcols ? c * args.ldg + r : r * args.ldg + c) * 4);
    }
#pragma unroll
    for (int s = 0; s < S::WSLOTS; ++s) {
        const int id = min(tid + S::kThreads * s, S::WUNITS - 1);
        const int r = id / S::UPR, u = id - r * S::UPR;
        woff[s] = uint32_t(r * args.pitch + 16 * u);
    }
    // elements spanned by G (none when N = 0: G is empty and its pointer may
    // be null)
    const long long g_end =
        N == 0 ? 0 : args.gcols ? (long long)(N - 1) * args.ldg + T : (long long)(T - 1) * args.ldg + N;
    // bytes spanned by W: rows are `pitch` apart, the last one ends after
    // its K / block blocks
    const long long w_end = N > 0 ? (long long)(N - 1) * args.pitch + (long long)(K / F::kBlock) * F::kBytes : 0;

    // Global -> registers for the chunk of W rows [n0, n0 + 32). Both loads go
    // through buffer descriptors based at the chunk's first element, so what
    // lies past the end of G and of W (n >= N) reads as zero in hardware.
    // Bytes of a row past this tile's K range belong to the next row: they
    // only feed dst columns >= K, which are never stored; G rows t >= T (other
    // values when G is stored t-fastest) only feed dst rows that are never
    // stored. G columns >= N (possible only in the last chunk) are zeroed
    // explicitly.
    auto load_chunk = [&](int n0) {
        n0 = __builtin_amdgcn_readfirstlane(n0);
        const long long gb = args.gcols ? (long long)n0 * args.ldg + t0 : (long long)t0 * args.ldg + n0;
        const __amdgpu_buffer_rsrc_t gr =
            buffer_rsrc(args.G + gb, uint32_t(max(0ll, min(4 * (g_end - gb), (long long)0x7FFFFFFF))));
#pragma unroll
        for (int s = 0; s < S::GSLOTS; ++s) {
            if (args.gvec) {
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(gr, goff[s], 0, 0);
                greg[s] = make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                                      __uint_as_float(v.w));
            } else {
                greg[s].x = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(gr, goff[s], 0, 0));
                greg[s].y = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(gr, goff[s] + gstep, 0, 0));
                greg[s].z = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(gr, goff[s] + 2 * gstep, 0, 0));
                greg[s].w = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(gr, goff[s] + 3 * gstep, 0, 0));
            }
        }
        if (n0 + BN > N) {
#pragma unroll
            for (int s = 0; s < S::GSLOTS; ++s) {
                const int n = n0 + 4 * ((tid + S::kThreads * s) & 7);
                if (n >= N) greg[s].x = 0.f;
                if (n + 1 >= N) greg[s].y = 0.f;
                if (n + 2 >= N) greg[s].z = 0.f;
                if (n + 3 >= N) greg[s].w = 0.f;
            }
        }
        const long long wb = (long long)n0 * args.pitch + kb0;
        const uint32_t wrange = uint32_t(max(0ll, min(w_end - wb, (long long)0x7FFFFFFF)));
        const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(args.W + wb, wrange);
#pragma unroll
        for (int s = 0; s < S::WSLOTS; ++s) {
            if (S::WUNITS % S::kThreads != 0 && tid + S::kThreads * s >= S::WUNITS) continue;
            const uint32_t o = woff[s];
            uint4 v;
            if (args.wvec == 16) {
                const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(wr, o, 0, 0);
                v = make_uint4(x.x, x.y, x.z, x.w);
            } else if (args.wvec == 8) {
                const u32x2 x0 = __builtin_amdgcn_raw_buffer_load_b64(wr, o, 0, 0);
                const u32x2 x1 = __builtin_amdgcn_raw_buffer_load_b64(wr, o + 8, 0, 0);
                v = make_uint4(x0.x, x0.y, x1.x, x1.y);
            } else if (Format<TYPE>::kBytes % 2 != 0 && args.wvec == 1) {
                // rows of odd length: whole units inside W take one unaligned
                // load, the unit reaching past its end takes bytes (a word
                // straddling the end of a buffer range reads as zero)
                if (o + 16 <= wrange) {
                    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(wr, o, 0, 0);
                    v = make_uint4(x.x, x.y, x.z, x.w);
                } else {
                    uint32_t w4[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                    for (int q = 0; q < 16; ++q)
                        w4[q >> 2] |= uint32_t(__builtin_amdgcn_raw_buffer_load_b8(wr, o + q, 0, 0)) << (8 * (q & 3));
                    v = make_uint4(w4[0], w4[1], w4[2], w4[3]);
                }
            } else if (args.wvec == 4) {
                v = make_uint4(__builtin_amdgcn_raw_buffer_load_b32(wr, o, 0, 0),
                               __builtin_amdgcn_raw_buffer_load_b32(wr, o + 4, 0, 0),
                               __builtin_amdgcn_raw_buffer_load_b32(wr, o + 8, 0, 0),
                               __builtin_amdgcn_raw_buffer_load_b32(wr, o + 12, 0, 0));
            } else {
                uint32_t h[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) h[q] = __builtin_amdgcn_raw_buffer_load_b16(wr, o + 2 * q, 0, 0);
                v = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
            }
            wreg[s] = v;
        }
    };

    // Registers -> LDS. G goes to Gs with the reduction index permuted:
    // W row n0 + 2s + h of the chunk sits at column 16h + s, so that lane half
    // h of an MFMA operand finds its 16 steps contiguous. Dense W is decoded
    // straight into Bs; packed W goes to Raw first.
    auto store_chunk = [&]() {
#pragma unroll
        for (int s = 0; s < S::GSLOTS; ++s) {
            const int id = tid + S::kThreads * s;
            const int r = id >> 3, j = id & 7;
            float* row = Gs + r * GP;
            *reinterpret_cast<float2*>(row + 2 * j) = make_float2(greg[s].x, greg[s].z);
            *reinterpret_cast<float2*>(row + 16 + 2 * j) = make_float2(greg[s].y, greg[s].w);
        }
#pragma unroll
        for (int s = 0; s < S::WSLOTS; ++s) {
            const int id = tid + S::kThreads * s;
            if (S::WUNITS % S::kThreads == 0 || id < S::WUNITS) {
                const int r = id / S::UPR, u = id - r * S::UPR;
                const uint4 v = wreg[s];
                if constexpr (S::kDense) {
                    float* brow = Bs + r * BP;
                    if constexpr (TYPE == kF32) {
                        *reinterpret_cast<float4*>(brow + S::swz(4 * u)) =
                            make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                                        __uint_as_float(v.w));
                    } else {
                        float e[8];
                        if constexpr (TYPE == kF16) {
                            f16x2(v.x, e[0], e[1]);
                            f16x2(v.y, e[2], e[3]);
                            f16x2(v.z, e[4], e[5]);
                            f16x2(v.w, e[6], e[7]);
                        } else {
                            bf16x2(v.x, e[0], e[1]);
                            bf16x2(v.y, e[2], e[3]);
                            bf16x2(v.z, e[4], e[5]);
                            bf16x2(v.w, e[6], e[7]);
                        }
                        *reinterpret_cast<float4*>(brow + S::swz(8 * u)) = make_float4(e[0], e[1], e[2], e[3]);
                        *reinterpret_cast<float4*>(brow + S::swz(8 * u + 4)) = make_float4(e[4], e[5], e[6], e[7]);
                    }
                } else {
                    *reinterpret_cast<uint4*>(Raw + r * S::RAWP + 16 * u) = v;
                }
            }
        }
    };

    // Raw packed bytes in LDS -> decoded floats in Bs (Q8_0, Q4_0).
    auto decode_chunk = [&]() {
#pragma unroll
        for (int p = 0; p < S::DPASS; ++p) {
            const int id = tid + S::kThreads * p;
            if ((BN * S::GPR) % S::kThreads == 0 || id < BN * S::GPR) {
                const int r = id / S::GPR, g = id - r * S::GPR;
                const uint8_t* raw = Raw + r * S::RAWP;
                float* brow = Bs + r * BP;
                if constexpr (TYPE == kQ4_K) {
                    const int sb = g >> 3, c = (g >> 1) & 3, h = g & 1;
                    const uint4 hd = *reinterpret_cast<const uint4*>(raw + 144 * sb);
                    const uint4 cw = *reinterpret_cast<const uint4*>(raw + 144 * sb + 16 + 32 * c + 16 * h);
                    float a0, b0, a1, b1;
                    q4_k_coeffs(hd.x, hd.y, hd.z, hd.w, 2 * c, a0, b0);
                    q4_k_coeffs(hd.x, hd.y, hd.z, hd.w, 2 * c + 1, a1, b1);
                    const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
                    const int lo = 256 * sb + 64 * c + 16 * h, hi = lo + 32;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float e[4];
                        q4_k_x4(w[i], false, a0, b0, e);
                        *reinterpret_cast<float4*>(brow + S::swz(lo + 4 * i)) = make_float4(e[0], e[1], e[2], e[3]);
                        q4_k_x4(w[i], true, a1, b1, e);
                        *reinterpret_cast<float4*>(brow + S::swz(hi + 4 * i)) = make_float4(e[0], e[1], e[2], e[3]);
                    }
                } else if constexpr (TYPE == kQ5_K) {
                    // as Q4_K, plus the fifth bits: qh bytes 16h .. 16h + 15
                    // belong to the same elements as this code unit
                    const int sb = g >> 3, c = (g >> 1) & 3, h = g & 1;
                    const uint8_t* blk = raw + 176 * sb;
                    const uint4 hd = *reinterpret_cast<const uint4*>(blk);
                    const uint4 qh = *reinterpret_cast<const uint4*>(blk + 16 + 16 * h);
                    const uint4 cw = *reinterpret_cast<const uint4*>(blk + 48 + 32 * c + 16 * h);
                    float a0, b0, a1, b1;
                    q4_k_coeffs(hd.x, hd.y, hd.z, hd.w, 2 * c, a0, b0);
                    q4_k_coeffs(hd.x, hd.y, hd.z, hd.w, 2 * c + 1, a1, b1);
                    const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
                    const uint32_t hb[4] = {qh.x, qh.y, qh.z, qh.w};
                    const int lo = 256 * sb + 64 * c + 16 * h, hi = lo + 32;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float e[4];
                        q5_k_x4(w[i], hb[i], 2 * c, false, a0, b0, e);
                        *reinterpret_cast<float4*>(brow + S::swz(lo + 4 * i)) = make_float4(e[0], e[1], e[2], e[3]);
                        q5_k_x4(w[i], hb[i], 2 * c + 1, true, a1, b1, e);
                        *reinterpret_cast<float4*>(brow + S::swz(hi + 4 * i)) = make_float4(e[0], e[1], e[2], e[3]);
                    }
                } else if constexpr (TYPE == kQ6_K) {
                    // group (half hh, l range 8j .. 8j + 7) of super-block sb:
                    // the elements 128 hh + 32 p + 8j + 0..7 of all four
                    // quarters p; 2-byte aligned block, read in halfwords
                    const int sb = g >> 3, hh = (g >> 2) & 1, j = g & 3;
                    const uint8_t* blk = raw + 210 * sb;
                    const uint32_t qlw[2][2] = {{lds_word_a2(blk + 64 * hh + 8 * j), lds_word_a2(blk + 64 * hh + 8 * j + 4)},
                                                {lds_word_a2(blk + 64 * hh + 32 + 8 * j),
                                                 lds_word_a2(blk + 64 * hh + 32 + 8 * j + 4)}};
                    const uint32_t qhw[2] = {lds_word_a2(blk + 128 + 32 * hh + 8 * j),
                                             lds_word_a2(blk + 128 + 32 * hh + 8 * j + 4)};
                    const uint32_t scw[2] = {lds_word_a2(blk + 192 + 8 * hh), lds_word_a2(blk + 192 + 8 * hh + 4)};
                    const float d = half_to_f32(*reinterpret_cast<const uint16_t*>(blk + 208));
#pragma unroll
                    for (int qq = 0; qq < 4; ++qq) {
                        const int si = (j >> 1) + 2 * qq;  // sub-scale 8 hh + si
                        float a;
                        q6_k_coeffs(scw[si >> 2], si & 3, d, a);
                        const int col = 256 * sb + 128 * hh + 32 * qq + 8 * j;
#pragma unroll
                        for (int i = 0; i < 2; ++i) {
                            float e[4];
                            q6_k_x4(qlw[qq & 1][i], qq >= 2, qhw[i], qq, a, e);
                            *reinterpret_cast<float4*>(brow + S::swz(col + 4 * i)) =
                                make_float4(e[0], e[1], e[2], e[3]);
                        }
                    }
                } else if constexpr (TYPE == kQ2_K || TYPE == kQ3_K) {
                    // group (half hh, l range 8j .. 8j + 7) of super-block sb:
                    // elements 128 hh + 32 p + 8j + 0..7 of the four quarters p,
                    // whose 2-bit codes share the 8 qs bytes 32hh + 8j ..
                    const int sb = g >> 3, hh = (g >> 2) & 1, j = g & 3;
                    const uint8_t* blk = raw + Format<TYPE>::kBytes * sb;
                    constexpr int QS = (TYPE == kQ2_K) ? 16 : 32;
                    const uint32_t qw[2] = {lds_word_a2(blk + QS + 32 * hh + 8 * j),
                                            lds_word_a2(blk + QS + 32 * hh + 8 * j + 4)};
                    uint32_t aux[2] = {0u, 0u}, f0 = 0, f1 = 0, f2 = 0;
                    float d = 0.f, dmin = 0.f;
                    if constexpr (TYPE == kQ2_K) {
                        aux[0] = lds_word_a2(blk + 8 * hh);
                        aux[1] = lds_word_a2(blk + 8 * hh + 4);
                        const uint32_t dd = lds_word_a2(blk + 80);
                        d = half_to_f32(dd & 0xFFFFu);
                        dmin = half_to_f32(dd >> 16);
                    } else {
                        aux[0] = lds_word_a2(blk + 8 * j);  // hmask bytes 8j ..
                        aux[1] = lds_word_a2(blk + 8 * j + 4);
                        f0 = lds_word_a2(blk + 96);
                        f1 = lds_word_a2(blk + 100);
                        f2 = lds_word_a2(blk + 104);
                        d = half_to_f32(*reinterpret_cast<const uint16_t*>(blk + 108));
                    }
#pragma unroll
                    for (int qq = 0; qq < 4; ++qq) {
                        const int si = (j >> 1) + 2 * qq;  // pair / sub-scale 8 hh + si
                        float a, b = 0.f;
                        if constexpr (TYPE == kQ2_K)
                            q2_k_coeffs(aux[si >> 2], si & 3, d, dmin, a, b);
                        else
                            q3_k_coeffs(f0, f1, f2, 8 * hh + si, d, a);
                        const int col = 256 * sb + 128 * hh + 32 * qq + 8 * j;
#pragma unroll
                        for (int i = 0; i < 2; ++i) {
                            float e[4];
                            if constexpr (TYPE == kQ2_K)
                                q2_k_x4(qw[i], qq, a, b, e);
                            else
                                q3_k_x4(qw[i], aux[i], qq, 4 * hh + qq, a, e);
                            *reinterpret_cast<float4*>(brow + S::swz(col + 4 * i)) =
                                make_float4(e[0], e[1], e[2], e[3]);
                        }
                    }
                } else if constexpr (kNibble32<TYPE>) {
                    const uint8_t* blk = raw + Format<TYPE>::kBytes * g;
                    float d, m;
                    uint32_t qh;
                    nibble32_header<TYPE>(lds_word_a2(blk), lds_word_a2(blk + 4), d, m, qh);
                    const int lo = 32 * g;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t w = lds_word_a2(blk + kHeader<TYPE> + 4 * i);
                        float e[4];
                        nibble32_x4<TYPE>(w, qh, 4 * i, d, m, e);
                        *reinterpret_cast<float4*>(brow + S::swz(lo + 4 * i)) = make_float4(e[0], e[1], e[2], e[3]);
                        nibble32_x4<TYPE>(w, qh, 16 + 4 * i, d, m, e);
                        *reinterpret_cast<float4*>(brow + S::swz(lo + 16 + 4 * i)) =
                            make_float4(e[0], e[1], e[2], e[3]);
                    }
                } else if constexpr (TYPE == kMXFP4) {  // 17-byte blocks: any byte alignment
                    const uint8_t* blk = raw + 17 * g;
                    const float sc = mx_scale(blk[0]);
                    const int lo = 32 * g;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float el[4], eh[4];
                        mxfp4_x8(lds_word_a1(blk + 1 + 4 * i), sc, el, eh);
                        *reinterpret_cast<float4*>(brow + S::swz(lo + 4 * i)) = make_float4(el[0], el[1], el[2], el[3]);
                        *reinterpret_cast<float4*>(brow + S::swz(lo + 16 + 4 * i)) =
                            make_float4(eh[0], eh[1], eh[2], eh[3]);
                    }
                } else if constexpr (TYPE == kNVFP4) {  // 36-byte blocks, 4-byte aligned
                    // group g: sub-blocks 2h and 2h + 1 of block b
                    const int b = g >> 1, h = g & 1;
                    const uint8_t* blk = raw + 36 * b;
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const int sb = 2 * h + q;
                        const float sc = e4m3_to_f32(blk[sb]);
                        const int out = 64 * b + 16 * sb;
#pragma unroll
                        for (int i = 0; i < 2; ++i) {
                            float el[4], eh[4];
                            nvfp4_x8(*reinterpret_cast<const uint32_t*>(blk + 4 + 8 * sb + 4 * i), sc, el, eh);
                            *reinterpret_cast<float4*>(brow + S::swz(out + 4 * i)) =
                                make_float4(el[0], el[1], el[2], el[3]);
                            *reinterpret_cast<float4*>(brow + S::swz(out + 8 + 4 * i)) =
                                make_float4(eh[0], eh[1], eh[2], eh[3]);
                        }
                    }
                } else if constexpr (TYPE == kQ8_0) {
                    const int b = g >> 1, h = g & 1;
                    const uint8_t* blk = raw + 34 * b;
                    const float d = half_to_f32(*reinterpret_cast<const uint16_t*>(blk));
                    const int out = 32 * b + 16 * h;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t w = lds_word_a2(blk + 2 + 16 * h + 4 * i);
                        float e[4];
                        q8_0_x4(w, d, e);
                        *reinterpret_cast<float4*>(brow + S::swz(out + 4 * i)) = make_float4(e[0], e[1], e[2], e[3]);
                    }
                }
            }
        }
    };

    const int lane = tid & 63, wave = tid >> 6;
    const int wt = wave / WGK, wk = wave % WGK;
    const int h = lane >> 5, l32 = lane & 31;

    f32x16 acc[WA][WB];
#pragma unroll
    for (int a = 0; a < WA; ++a)
#pragma unroll
        for (int b = 0; b < WB; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

    const int nchunks = (N + BN - 1) / BN;
    if (nchunks > 0) load_chunk(0);
    for (int c = 0; c < nchunks; ++c) {
        store_chunk();
        __syncthreads();
        if (c + 1 < nchunks) load_chunk((c + 1) * BN);
        if constexpr (S::kStaged) {
            decode_chunk();
            __syncthreads();
        }
        // MFMA step s (0..15) contracts W rows n0 + 2s + h (lane half h):
        // A[i][h] = G[t_i][n0 + 2s + h], B[h][j] = W[n0 + 2s + h][k_j].
        const float* ga = Gs + (wt * 32 * WA + l32) * GP + 16 * h;
        const float* bb = Bs + h * BP;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f32x4 av[WA];
#pragma unroll
            for (int a = 0; a < WA; ++a) av[a] = *reinterpret_cast<const f32x4*>(ga + 32 * a * GP + 4 * q);
            float bv[4][WB];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int b = 0; b < WB; ++b) bv[r][b] = bb[(2 * (4 * q + r)) * BP + S::swz(wk * 32 * WB + 32 * b + l32)];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int a = 0; a < WA; ++a)
#pragma unroll
                    for (int b = 0; b < WB; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[a][r], bv[r][b], acc[a][b], 0, 0, 0);
        }
        __syncthreads();
    }

    // D layout of v_mfma_f32_32x32x2f32: lane l, register v holds
    // row 8*(v/4) + 4*(l/32) + v%4, column l%32.
#pragma unroll
    for (int a = 0; a < WA; ++a)
#pragma unroll
        for (int b = 0; b < WB; ++b) {
            const int k = k0 + wk * 32 * WB + 32 * b + l32;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int t = t0 + wt * 32 * WA + 32 * a + 8 * (v >> 2) + 4 * h + (v & 3);
                if (t < T && k < K) args.dst[(long long)t * args.ldd + k] = acc[a][b][v];
            }
        }
}

// ---------------------------------------------------------------------------
// Skinny kernel (up to T = 64 a launch)
// ---------------------------------------------------------------------------

struct SkinnyArgs {
    const uint8_t* W;
    const float* G;
    float* dst;
    int K, N, T;
    long long pitch;  // bytes between consecutive W rows
    long long ldg;    // G[t][n] at t * ldg + n (ldg >= N), or at n * ldg + t when gcols (ldg >= T)
    long long ldd;    // floats between consecutive dst rows (>= K)
    int wide;   // 1: W rows allow the widest load of 4 consecutive elements
    int gvec;   // 1: the fast path's G loads are aligned (G rows take float4 loads, or gcols)
    int gcols;  // 1: G is stored t-fastest (the columns of G are contiguous)
    BatchArgs batch;
};

// Four consecutive elements k, k+1, k+2, k+3 (k a multiple of 4) of W row
// `row`; elements at or beyond K read as zero.
template <int TYPE>
__device__ __forceinline__ void skinny_load4(const uint8_t* row, int k, int K, int wide, float e[4]) {
    if constexpr (TYPE == kF32) {
        const float* p = reinterpret_cast<const float*>(row) + k;
        if (wide && k + 4 <= K) {
            const float4 v = *reinterpret_cast<const float4*>(p);
            e[0] = v.x; e[1] = v.y; e[2] = v.z; e[3] = v.w;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) e[i] = (k + i < K) ? p[i] : 0.f;
        }
    } else if constexpr (TYPE == kF16 || TYPE == kBF16) {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(row) + k;
        uint32_t w0 = 0, w1 = 0;
        if (wide && k + 4 <= K) {
            const uint2 v = *reinterpret_cast<const uint2*>(p);
            w0 = v.x;
            w1 = v.y;
        } else {
            if (k < K) w0 |= p[0];
            if (k + 1 < K) w0 |= uint32_t(p[1]) << 16;
            if (k + 2 < K) w1 |= p[2];
            if (k + 3 < K) w1 |= uint32_t(p[3]) << 16;
        }
        if constexpr (TYPE == kF16) {
            f16x2(w0, e[0], e[1]);
            f16x2(w1, e[2], e[3]);
        } else {
            bf16x2(w0, e[0], e[1]);
            bf16x2(w1, e[2], e[3]);
        }
    } else if constexpr (TYPE == kQ8_0) {
        if (k >= K) { e[0] = e[1] = e[2] = e[3] = 0.f; return; }
        const uint8_t* blk = row + (k >> 5) * 34;
        const int r = k & 31;
        const float d = half_to_f32(*reinterpret_cast<const uint16_t*>(blk));
        const uint16_t* c = reinterpret_cast<const uint16_t*>(blk + 2 + r);
        q8_0_x4(uint32_t(c[0]) | (uint32_t(c[1]) << 16), d, e);
    } else if constexpr (TYPE == kNVFP4) {  // K is a multiple of 64, so k < K always
        const uint8_t* blk = row + (k >> 6) * 36;
        const int r = k & 63, sb = r >> 4, i = r & 15;
        const uint32_t w = *reinterpret_cast<const uint32_t*>(blk + 4 + 8 * sb + (i & 7));
        nvfp4_x4(w, i >= 8, e4m3_to_f32(blk[sb]), e);
    } else if constexpr (TYPE == kMXFP4) {  // 17-byte blocks: read bytewise
        if (k >= K) { e[0] = e[1] = e[2] = e[3] = 0.f; return; }
        const uint8_t* blk = row + (k >> 5) * 17;
        const int r = k & 31;
        const uint8_t* c = blk + 1 + (r & 15);
        const uint32_t w = uint32_t(c[0]) | (uint32_t(c[1]) << 8) | (uint32_t(c[2]) << 16) | (uint32_t(c[3]) << 24);
        mxfp4_x4(w, r >= 16, mx_scale(blk[0]), e);
    } else if constexpr (kNibble32<TYPE>) {  // 2-byte aligned blocks
        if (k >= K) { e[0] = e[1] = e[2] = e[3] = 0.f; return; }
        const uint8_t* blk = row + (k >> 5) * Format<TYPE>::kBytes;
        const int r = k & 31;
        const uint16_t* h = reinterpret_cast<const uint16_t*>(blk);
        float d, m;
        uint32_t qh;
        nibble32_header<TYPE>(uint32_t(h[0]) | (uint32_t(h[1]) << 16), uint32_t(h[2]) | (uint32_t(h[3]) << 16), d,
                              m, qh);
        const uint16_t* c = reinterpret_cast<const uint16_t*>(blk + kHeader<TYPE> + (r & 15));
        nibble32_x4<TYPE>(uint32_t(c[0]) | (uint32_t(c[1]) << 16), qh, r, d, m, e);
    } else if constexpr (TYPE == kQ4_K) {  // K is a multiple of 256, so k < K always
        const uint8_t* sbp = row + (k >> 8) * 144;
        const int e256 = k & 255, c = e256 >> 6, r = e256 & 63;
        const bool high = r >= 32;
        const uint32_t* hw = reinterpret_cast<const uint32_t*>(sbp);
        float a, b;
        q4_k_coeffs(hw[0], hw[1], hw[2], hw[3], 2 * c + (high ? 1 : 0), a, b);
        const uint32_t w = *reinterpret_cast<const uint32_t*>(sbp + 16 + 32 * c + (r & 31));
        q4_k_x4(w, high, a, b, e);
    } else if constexpr (TYPE == kQ5_K) {
        const uint8_t* sbp = row + (k >> 8) * 176;
        const int e256 = k & 255, c = e256 >> 6, r = e256 & 63;
        const bool high = r >= 32;
        const uint32_t* hw = reinterpret_cast<const uint32_t*>(sbp);
        float a, b;
        q4_k_coeffs(hw[0], hw[1], hw[2], hw[3], 2 * c + (high ? 1 : 0), a, b);
        const uint32_t qh = *reinterpret_cast<const uint32_t*>(sbp + 16 + (r & 31));
        const uint32_t qs = *reinterpret_cast<const uint32_t*>(sbp + 48 + 32 * c + (r & 31));
        q5_k_x4(qs, qh, 2 * c + (high ? 1 : 0), high, a, b, e);
    } else if constexpr (TYPE == kQ2_K) {  // 4-byte aligned super-blocks
        const uint8_t* sbp = row + (k >> 8) * 84;
        const int e256 = k & 255, h = e256 >> 7, p = (e256 >> 5) & 3, l = e256 & 31;
        const int pi = 8 * h + 2 * p + (l >> 4);
        const uint32_t dd = *reinterpret_cast<const uint32_t*>(sbp + 80);
        float a, b;
        q2_k_coeffs(*reinterpret_cast<const uint32_t*>(sbp + (pi & ~3)), pi & 3, half_to_f32(dd & 0xFFFFu),
                    half_to_f32(dd >> 16), a, b);
        q2_k_x4(*reinterpret_cast<const uint32_t*>(sbp + 16 + 32 * h + l), p, a, b, e);
    } else if constexpr (TYPE == kQ3_K) {  // 2-byte aligned super-blocks
        const uint8_t* sbp = row + (k >> 8) * 110;
        const int e256 = k & 255, h = e256 >> 7, p = (e256 >> 5) & 3, l = e256 & 31;
        const uint16_t* f = reinterpret_cast<const uint16_t*>(sbp + 96);
        const uint32_t f0 = f[0] | (uint32_t(f[1]) << 16), f1 = f[2] | (uint32_t(f[3]) << 16),
                       f2 = f[4] | (uint32_t(f[5]) << 16);
        float a;
        q3_k_coeffs(f0, f1, f2, 8 * h + 2 * p + (l >> 4), half_to_f32(f[6]), a);
        const uint16_t* qs = reinterpret_cast<const uint16_t*>(sbp + 32 + 32 * h + l);
        const uint16_t* hm = reinterpret_cast<const uint16_t*>(sbp + l);
        q3_k_x4(qs[0] | (uint32_t(qs[1]) << 16), hm[0] | (uint32_t(hm[1]) << 16), p, 4 * h + p, a, e);
    } else {  // kQ6_K: 2-byte aligned super-blocks
        const uint8_t* sbp = row + (k >> 8) * 210;
        const int e256 = k & 255, h = e256 >> 7, p = (e256 >> 5) & 3, l = e256 & 31;
        const uint16_t* ql = reinterpret_cast<const uint16_t*>(sbp + 64 * h + 32 * (p & 1) + l);
        const uint16_t* qh = reinterpret_cast<const uint16_t*>(sbp + 128 + 32 * h + l);
        const int si = 8 * h + 2 * p + (l >> 4);
        const uint32_t scw = *reinterpret_cast<const uint16_t*>(sbp + 192 + (si & ~1));
        float a;
        q6_k_coeffs(scw, si & 1, half_to_f32(*reinterpret_cast<const uint16_t*>(sbp + 208)), a);
        q6_k_x4(uint32_t(ql[0]) | (uint32_t(ql[1]) << 16), p >= 2, uint32_t(qh[0]) | (uint32_t(qh[1]) << 16), p, a, e);
    }
}

// Per-lane raw data of one 16-row group (see out_prod_skinny_kernel for the
// lane layout): the code words of the lane's 4 rows, the header words of the
// (row, block) scale this lane decodes for the whole wave, and 4 G values
// for each of the TB blocks of 16 rows of G.
template <int TYPE, int TB = 1>
struct SkinnyRaw {
    static constexpr int CW = (TYPE == kF32) ? 4
                              : (TYPE == kF16 || TYPE == kBF16 || TYPE == kQ5_K || TYPE == kQ6_K || TYPE == kQ3_K) ? 2
                                                                                                            : 1;
    static constexpr int HW = (TYPE == kQ4_K || TYPE == kQ5_K || TYPE == kQ3_K)    ? 4
                              : (TYPE == kQ6_K || TYPE == kQ2_K || kHasFifth<TYPE>) ? 2
                                                                                   : 1;
    uint32_t code[4][CW];
    uint32_t hdr[HW];
    float g[TB][4];
};

// Byte offsets, relative to the first W row / G column of a 16-row group,
// of everything one lane loads for that group on the fast path; they do not
// change from group to group, so each group costs one uniform base pointer.
struct SkinnyOffsets {
    uint32_t code[4];   // code words of rows 4*(l/16) + s, columns k0 + 4*(l%16) ..
    uint32_t code2[4];  // Q5_K fifth bits / Q6_K high parts of the same elements
    uint32_t hdr;       // header of the scale pair this lane decodes (Q6_K, Q2_K, Q3_K: see skinny_offsets)
    uint32_t hdr2;      // Q6_K, Q2_K: the scales of that row
    uint32_t g[4];      // G[min(16 tb + l%16, T-1)][n0 + 4*(l/16)] for t-block tb (bytes from G[0][n0])
};

// Fast path (K % 4 == 0, G rows 16-byte aligned or G stored t-fastest,
// whole group inside W). Columns at or beyond K and rows of G at or beyond T
// are clamped to valid addresses: they only feed dst columns and rows that
// are never stored.
template <int TYPE, int TB = 1>
__device__ __forceinline__ SkinnyOffsets skinny_offsets(const SkinnyArgs& a, int k0, int lane) {
    const int j = lane & 15, rq = lane >> 4;
    const int K = a.K;
    const int kl = min(k0 + 4 * j, K - 4);
    uint32_t col, col2 = 0;
    if constexpr (TYPE == kF32) {
        col = 4u * kl;
    } else if constexpr (TYPE == kF16 || TYPE == kBF16) {
        col = 2u * kl;
    } else if constexpr (TYPE == kQ8_0) {
        col = (kl >> 5) * 34 + 2 + (kl & 31);
    } else if constexpr (kNibbleLayout<TYPE>) {
        col = (kl >> 5) * Format<TYPE>::kBytes + kHeader<TYPE> + (kl & 15);
    } else if constexpr (TYPE == kNVFP4) {
        const int e = kl & 63;
        col = (kl >> 6) * 36 + 4 + 8 * (e >> 4) + (e & 7);
    } else if constexpr (TYPE == kQ4_K) {
        const int e = kl & 255;
        col = (kl >> 8) * 144 + 16 + 32 * (e >> 6) + (e & 31);
    } else if constexpr (TYPE == kQ5_K) {
        const int e = kl & 255;
        col = (kl >> 8) * 176 + 48 + 32 * (e >> 6) + (e & 31);
        col2 = (kl >> 8) * 176 + 16 + (e & 31);
    } else if constexpr (TYPE == kQ6_K) {
        const int e = kl & 255, h = e >> 7, p = (e >> 5) & 3, l = e & 31;
        col = (kl >> 8) * 210 + 64 * h + 32 * (p & 1) + l;
        col2 = (kl >> 8) * 210 + 128 + 32 * h + l;
    } else if constexpr (TYPE == kQ2_K) {
        const int e = kl & 255, h = e >> 7, l = e & 31;
        col = (kl >> 8) * 84 + 16 + 32 * h + l;
    } else {  // kQ3_K
        const int e = kl & 255, h = e >> 7, l = e & 31;
        col = (kl >> 8) * 110 + 32 + 32 * h + l;
        col2 = (kl >> 8) * 110 + l;
    }
    SkinnyOffsets o;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        o.code[s] = uint32_t((4 * rq + s) * a.pitch) + col;
        o.code2[s] = uint32_t((4 * rq + s) * a.pitch) + col2;
    }
    const int hr = (lane & 31) >> 1, sel = lane & 1;
    uint32_t hcol = 0;
    if constexpr (TYPE == kQ4_K) hcol = (k0 >> 8) * 144;
    if constexpr (TYPE == kQ5_K) hcol = (k0 >> 8) * 176;
    if constexpr (TYPE == kQ8_0 || kNibbleLayout<TYPE>)
        hcol = (min(k0 + 32 * sel, K - 32) >> 5) * Format<TYPE>::kBytes;
    o.hdr = uint32_t(hr * a.pitch) + hcol;
    o.hdr2 = 0;
    if constexpr (TYPE == kNVFP4)  // the scale byte of (row lane / 4, sub-block lane % 4)
        o.hdr = uint32_t((lane >> 2) * a.pitch) + uint32_t((k0 >> 6) * 36 + (lane & 3));
    if constexpr (TYPE == kQ6_K || TYPE == kQ2_K || TYPE == kQ3_K) {
        // lane -> (row lane / 4, sub-scale or pair 8h + 2(p0 + w / 2) + w % 2),
        // w = lane % 4, p0 the slab's first quarter. Q6_K: the halfword holding
        // that sub-scale and the row's d; Q2_K: the word holding the pair and
        // the row's d, dmin; Q3_K: the whole sub-scale field with d.
        const int e0 = k0 & 255, h = e0 >> 7, p0 = (e0 >> 5) & 3, w = lane & 3;
        const int si = 8 * h + 2 * (p0 + (w >> 1)) + (w & 1);
        const uint32_t rowb = uint32_t((lane >> 2) * a.pitch) + uint32_t((k0 >> 8) * Format<TYPE>::kBytes);
        if constexpr (TYPE == kQ6_K) {
            o.hdr = rowb + 192 + uint32_t(si & ~1);
            o.hdr2 = rowb + 208;
        } else if constexpr (TYPE == kQ2_K) {
            o.hdr = rowb + uint32_t(si & ~3);
            o.hdr2 = rowb + 80;
        } else {
            o.hdr = rowb + 96;
        }
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        const long long gt = min(16 * tb + j, a.T - 1);
        o.g[tb] = uint32_t((a.gcols ? 4 * rq * a.ldg + gt : gt * a.ldg + 4 * rq) * 4);
    }
    return o;
}

template <int TYPE, int TB>
__device__ __forceinline__ void skinny_fetch_fast(const SkinnyArgs& a, int n0, const SkinnyOffsets& o,
                                                  SkinnyRaw<TYPE, TB>& r) {
    // n0 is the same in every lane; readfirstlane makes that visible to the
    // compiler, so the two descriptors (this group's 16 W rows; the G columns
    // from n0 on) are built in scalar registers and every load is a fixed
    // per-lane offset from them.
    n0 = __builtin_amdgcn_readfirstlane(n0);
    const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(a.W + (long long)n0 * a.pitch, uint32_t(16 * a.pitch));
    if (a.gcols) {
        // G[t][n0 + 4(l/16) + q]: four words ldg apart (the 16 columns n0 ..
        // n0 + 15 span 15 ldg + T floats)
        const __amdgpu_buffer_rsrc_t gr =
            buffer_rsrc(a.G + (long long)n0 * a.ldg, uint32_t(4 * (15 * a.ldg + a.T)));
        const uint32_t step = uint32_t(4 * a.ldg);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                r.g[tb][q] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(gr, o.g[tb] + q * step, 0, 0));
    } else {
        const __amdgpu_buffer_rsrc_t gr = buffer_rsrc(a.G + n0, uint32_t(4 * ((long long)(a.T - 1) * a.ldg + 16)));
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const u32x4 gv = __builtin_amdgcn_raw_buffer_load_b128(gr, o.g[tb], 0, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q) r.g[tb][q] = __uint_as_float(gv[q]);
        }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        if constexpr (TYPE == kF32) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(wr, o.code[s], 0, 0);
            r.code[s][0] = v.x; r.code[s][1] = v.y; r.code[s][2] = v.z; r.code[s][3] = v.w;
        } else if constexpr (TYPE == kF16 || TYPE == kBF16) {
            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(wr, o.code[s], 0, 0);
            r.code[s][0] = v.x;
            r.code[s][1] = v.y;
        } else if constexpr (TYPE == kQ8_0 || kNibbleLayout<TYPE>) {
            // code bytes sit at 2-byte (MXFP4: any) alignment inside these blocks; the
            // dword load relies on the unaligned buffer access of gfx9-class GPUs
            r.code[s][0] = __builtin_amdgcn_raw_buffer_load_b32(wr, o.code[s], 0, 0);
        } else if constexpr (TYPE == kQ6_K || TYPE == kQ3_K) {
            // 2-byte aligned super-blocks (unaligned dword loads, as above)
            r.code[s][0] = __builtin_amdgcn_raw_buffer_load_b32(wr, o.code[s], 0, 0);
            r.code[s][1] = __builtin_amdgcn_raw_buffer_load_b32(wr, o.code2[s], 0, 0);
        } else {
            r.code[s][0] = __builtin_amdgcn_raw_buffer_load_b32(wr, o.code[s], 0, 0);
            if constexpr (TYPE == kQ5_K) r.code[s][1] = __builtin_amdgcn_raw_buffer_load_b32(wr, o.code2[s], 0, 0);
        }
    }
    if constexpr (TYPE == kQ4_K || TYPE == kQ5_K) {
        const u32x4 h = __builtin_amdgcn_raw_buffer_load_b128(wr, o.hdr, 0, 0);
        r.hdr[0] = h.x; r.hdr[1] = h.y; r.hdr[2] = h.z; r.hdr[3] = h.w;
    } else if constexpr (TYPE == kQ3_K) {
        // field bytes 96 .. 107 and d; no load reaches past the block, whose
        // end may be the end of this group's W range
        const u32x2 f = __builtin_amdgcn_raw_buffer_load_b64(wr, o.hdr, 0, 0);
        r.hdr[0] = f.x; r.hdr[1] = f.y;
        r.hdr[2] = __builtin_amdgcn_raw_buffer_load_b32(wr, o.hdr + 8, 0, 0);
        r.hdr[3] = __builtin_amdgcn_raw_buffer_load_b16(wr, o.hdr + 12, 0, 0);
    } else if constexpr (TYPE == kQ6_K) {
        r.hdr[0] = __builtin_amdgcn_raw_buffer_load_b16(wr, o.hdr, 0, 0);
        r.hdr[1] = __builtin_amdgcn_raw_buffer_load_b16(wr, o.hdr2, 0, 0);
    } else if constexpr (TYPE == kQ2_K) {
        r.hdr[0] = __builtin_amdgcn_raw_buffer_load_b32(wr, o.hdr, 0, 0);
        r.hdr[1] = __builtin_amdgcn_raw_buffer_load_b32(wr, o.hdr2, 0, 0);
    } else if constexpr (kHasFifth<TYPE>) {  // d, m, qh: the first 8 bytes of a 22- or 24-byte block
        const u32x2 h = __builtin_amdgcn_raw_buffer_load_b64(wr, o.hdr, 0, 0);
        r.hdr[0] = h.x;
        r.hdr[1] = h.y;
    } else if constexpr (TYPE == kQ4_1) {
        r.hdr[0] = __builtin_amdgcn_raw_buffer_load_b32(wr, o.hdr, 0, 0);
    } else if constexpr (TYPE == kQ8_0 || TYPE == kQ4_0) {
        r.hdr[0] = __builtin_amdgcn_raw_buffer_load_b16(wr, o.hdr, 0, 0);
    } else if constexpr (TYPE == kMXFP4 || TYPE == kNVFP4) {
        r.hdr[0] = __builtin_amdgcn_raw_buffer_load_b8(wr, o.hdr, 0, 0);
    } else {
        r.hdr[0] = 0u;
    }
}

// Any group and shape: out-of-range elements read as zero.
template <int TYPE, int TB>
__device__ __forceinline__ void skinny_fetch_masked(const SkinnyArgs& a, int n0, int k0, int lane,
                                                    SkinnyRaw<TYPE, TB>& r) {
    const int j = lane & 15, rq = lane >> 4;
    const int K = a.K, N = a.N;
    const int nq = n0 + 4 * rq;
    const int kl = k0 + 4 * j;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        const int t = 16 * tb + j;
#pragma unroll
        for (int s = 0; s < 4; ++s) r.g[tb][s] = 0.f;
        if (t < a.T) {
            // G[t][nq + s]
            const long long gs = a.gcols ? a.ldg : 1;
            const float* gp = a.G + (a.gcols ? (long long)nq * a.ldg + t : (long long)t * a.ldg + nq);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                if (nq + s < N) r.g[tb][s] = gp[s * gs];
        }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int w = 0; w < SkinnyRaw<TYPE, TB>::CW; ++w) r.code[s][w] = 0u;
        if (nq + s >= N) continue;
        const uint8_t* row = a.W + (long long)(nq + s) * a.pitch;
        if constexpr (TYPE == kF32) {
            const uint32_t* p = reinterpret_cast<const uint32_t*>(row) + kl;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (kl + i < K) r.code[s][i] = p[i];
        } else if constexpr (TYPE == kF16 || TYPE == kBF16) {
            const uint16_t* p = reinterpret_cast<const uint16_t*>(row) + kl;
            if (kl < K) r.code[s][0] |= p[0];
            if (kl + 1 < K) r.code[s][0] |= uint32_t(p[1]) << 16;
            if (kl + 2 < K) r.code[s][1] |= p[2];
            if (kl + 3 < K) r.code[s][1] |= uint32_t(p[3]) << 16;
        } else if constexpr (TYPE == kNVFP4) {  // K % 64 == 0, so kl < K
            const int e = kl & 63;
            r.code[s][0] = *reinterpret_cast<const uint32_t*>(row + (kl >> 6) * 36 + 4 + 8 * (e >> 4) + (e & 7));
        } else if constexpr (TYPE == kMXFP4) {
            if (kl < K) {
                const uint8_t* c = row + (kl >> 5) * 17 + 1 + (kl & 15);
                r.code[s][0] = uint32_t(c[0]) | (uint32_t(c[1]) << 8) | (uint32_t(c[2]) << 16) | (uint32_t(c[3]) << 24);
            }
        } else if constexpr (TYPE == kQ8_0 || kNibble32<TYPE>) {
            if (kl < K) {
                constexpr int BYTES = Format<TYPE>::kBytes;
                const int off = (TYPE == kQ8_0) ? 2 + (kl & 31) : kHeader<TYPE> + (kl & 15);
                const uint16_t* c = reinterpret_cast<const uint16_t*>(row + (kl >> 5) * BYTES + off);
                r.code[s][0] = uint32_t(c[0]) | (uint32_t(c[1]) << 16);
            }
        } else if constexpr (TYPE == kQ4_K) {  // K % 256 == 0, so kl < K
            const int e = kl & 255;
            r.code[s][0] = *reinterpret_cast<const uint32_t*>(row + (kl >> 8) * 144 + 16 + 32 * (e >> 6) + (e & 31));
        } else if constexpr (TYPE == kQ5_K) {
            const int e = kl & 255;
            const uint8_t* sb = row + (kl >> 8) * 176;
            r.code[s][0] = *reinterpret_cast<const uint32_t*>(sb + 48 + 32 * (e >> 6) + (e & 31));
            r.code[s][1] = *reinterpret_cast<const uint32_t*>(sb + 16 + (e & 31));
        } else if constexpr (TYPE == kQ2_K) {
            const int e = kl & 255, h = e >> 7, l = e & 31;
            r.code[s][0] = *reinterpret_cast<const uint32_t*>(row + (kl >> 8) * 84 + 16 + 32 * h + l);
        } else if constexpr (TYPE == kQ3_K) {
            const int e = kl & 255, h = e >> 7, l = e & 31;
            const uint8_t* sb = row + (kl >> 8) * 110;
            const uint16_t* qs = reinterpret_cast<const uint16_t*>(sb + 32 + 32 * h + l);
            const uint16_t* hm = reinterpret_cast<const uint16_t*>(sb + l);
            r.code[s][0] = uint32_t(qs[0]) | (uint32_t(qs[1]) << 16);
            r.code[s][1] = uint32_t(hm[0]) | (uint32_t(hm[1]) << 16);
        } else {  // kQ6_K
            const int e = kl & 255, h = e >> 7, p = (e >> 5) & 3, l = e & 31;
            const uint8_t* sb = row + (kl >> 8) * 210;
            const uint16_t* ql = reinterpret_cast<const uint16_t*>(sb + 64 * h + 32 * (p & 1) + l);
            const uint16_t* qh = reinterpret_cast<const uint16_t*>(sb + 128 + 32 * h + l);
            r.code[s][0] = uint32_t(ql[0]) | (uint32_t(ql[1]) << 16);
            r.code[s][1] = uint32_t(qh[0]) | (uint32_t(qh[1]) << 16);
        }
    }
    const int hr = (lane & 31) >> 1, sel = lane & 1;
    const bool hvalid = n0 + hr < N;
    const uint8_t* hrow = a.W + (long long)(n0 + hr) * a.pitch;
    if constexpr (TYPE == kQ4_K || TYPE == kQ5_K) {
        uint4 h = make_uint4(0u, 0u, 0u, 0u);
        if (hvalid) h = *reinterpret_cast<const uint4*>(hrow + (k0 >> 8) * Format<TYPE>::kBytes);
        r.hdr[0] = h.x; r.hdr[1] = h.y; r.hdr[2] = h.z; r.hdr[3] = h.w;
    } else if constexpr (TYPE == kQ6_K || TYPE == kQ2_K || TYPE == kQ3_K) {
        const int e0 = k0 & 255, h = e0 >> 7, p0 = (e0 >> 5) & 3, w = lane & 3;
        const int si = 8 * h + 2 * (p0 + (w >> 1)) + (w & 1);
#pragma unroll
        for (int i = 0; i < SkinnyRaw<TYPE, TB>::HW; ++i) r.hdr[i] = 0u;
        if (n0 + (lane >> 2) < N) {
            const uint8_t* sb = a.W + (long long)(n0 + (lane >> 2)) * a.pitch + (k0 >> 8) * Format<TYPE>::kBytes;
            if constexpr (TYPE == kQ6_K) {
                r.hdr[0] = *reinterpret_cast<const uint16_t*>(sb + 192 + (si & ~1));
                r.hdr[1] = *reinterpret_cast<const uint16_t*>(sb + 208);
            } else if constexpr (TYPE == kQ2_K) {
                r.hdr[0] = *reinterpret_cast<const uint32_t*>(sb + (si & ~3));
                r.hdr[1] = *reinterpret_cast<const uint32_t*>(sb + 80);
            } else {  // field bytes 96 .. 107 and d at 108 (inside the block)
                const uint16_t* f = reinterpret_cast<const uint16_t*>(sb + 96);
#pragma unroll
                for (int i = 0; i < 3; ++i) r.hdr[i] = uint32_t(f[2 * i]) | (uint32_t(f[2 * i + 1]) << 16);
                r.hdr[3] = f[6];
            }
        }
    } else if constexpr (TYPE == kNVFP4) {
        r.hdr[0] = 0u;
        if (n0 + (lane >> 2) < N) r.hdr[0] = a.W[(long long)(n0 + (lane >> 2)) * a.pitch + (k0 >> 6) * 36 + (lane & 3)];
    } else if constexpr (TYPE == kMXFP4) {
        const int kb = k0 + 32 * sel;
        r.hdr[0] = 0u;
        if (hvalid && kb < K) r.hdr[0] = hrow[(kb >> 5) * 17];
    } else if constexpr (TYPE == kQ8_0 || kNibble32<TYPE>) {
        // the header halfwords (d; m; qh), none past the header
        constexpr int HH = TYPE == kQ8_0 ? 1 : (kHeader<TYPE> / 2 < 4 ? kHeader<TYPE> / 2 : 4);
        const int kb = k0 + 32 * sel;
#pragma unroll
        for (int i = 0; i < SkinnyRaw<TYPE, TB>::HW; ++i) r.hdr[i] = 0u;
        if (hvalid && kb < K) {
            const uint16_t* h = reinterpret_cast<const uint16_t*>(hrow + (kb >> 5) * Format<TYPE>::kBytes);
#pragma unroll
            for (int i = 0; i < HH; ++i) r.hdr[i >> 1] |= uint32_t(h[i]) << (16 * (i & 1));
        }
    } else {
        r.hdr[0] = 0u;
    }
}

// Value of `v` held by lane `src` of this wave.
__device__ __forceinline__ float lane_value(float v, int src) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v)));
}

template <int TYPE, int TB>
__device__ __forceinline__ void skinny_decode(const SkinnyRaw<TYPE, TB>& r, int k0, int lane, float wv[4][4]) {
    const int j = lane & 15, rq = lane >> 4;
    const int hi = (j >= 8) ? 1 : 0;  // second block / sub-block of the 64-column slab
    if constexpr (TYPE == kF32) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) wv[s][i] = __uint_as_float(r.code[s][i]);
    } else if constexpr (TYPE == kF16) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            f16x2(r.code[s][0], wv[s][0], wv[s][1]);
            f16x2(r.code[s][1], wv[s][2], wv[s][3]);
        }
    } else if constexpr (TYPE == kBF16) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x2(r.code[s][0], wv[s][0], wv[s][1]);
            bf16x2(r.code[s][1], wv[s][2], wv[s][3]);
        }
    } else if constexpr (TYPE == kQ8_0) {
        const float dmine = half_to_f32(r.hdr[0]);
#pragma unroll
        for (int s = 0; s < 4; ++s) q8_0_x4(r.code[s][0], lane_value(dmine, 2 * (4 * rq + s) + hi), wv[s]);
    } else if constexpr (TYPE == kMXFP4) {
        // this lane decodes the scale of (row (lane % 32) / 2, block lane % 2)
        const float smine = mx_scale(r.hdr[0]);
        const int e = (4 * j) & 31;
#pragma unroll
        for (int s = 0; s < 4; ++s) mxfp4_x4(r.code[s][0], e >= 16, lane_value(smine, 2 * (4 * rq + s) + hi), wv[s]);
    } else if constexpr (TYPE == kNVFP4) {
        // this lane decodes the scale of (row lane / 4, sub-block lane % 4);
        // its own 4 columns 4j .. 4j + 3 lie in sub-block j / 4, the high
        // nibbles for j % 4 >= 2
        const float smine = e4m3_to_f32(r.hdr[0]);
        const bool high = (j & 2) != 0;
#pragma unroll
        for (int s = 0; s < 4; ++s) nvfp4_x4(r.code[s][0], high, lane_value(smine, 4 * (4 * rq + s) + (j >> 2)), wv[s]);
    } else if constexpr (kNibble32<TYPE>) {
        // this lane decodes the header of (row (lane % 32) / 2, block lane % 2)
        float dmine, mmine;
        uint32_t qhmine;
        if constexpr (kHasFifth<TYPE>)
            nibble32_header<TYPE>(r.hdr[0], r.hdr[1], dmine, mmine, qhmine);
        else
            nibble32_header<TYPE>(r.hdr[0], 0u, dmine, mmine, qhmine);
        const int e = (4 * j) & 31;  // element of the block this lane's 4 columns start at
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int src = 2 * (4 * rq + s) + hi;
            const float d = lane_value(dmine, src);
            float m = 0.f;
            if constexpr (kHasOffset<TYPE>) m = lane_value(mmine, src);
            uint32_t qh = 0u;
            if constexpr (kHasFifth<TYPE>) qh = uint32_t(__builtin_amdgcn_ds_bpermute(src << 2, int(qhmine)));
            nibble32_x4<TYPE>(r.code[s][0], qh, e, d, m, wv[s]);
        }
    } else if constexpr (TYPE == kQ4_K || TYPE == kQ5_K) {  // this lane's pair is sub-block 2c + (lane & 1)
        const int c = (k0 & 255) >> 6;
        float am, bm;
        q4_k_coeffs(r.hdr[0], r.hdr[1], r.hdr[2], r.hdr[3], 2 * c + (lane & 1), am, bm);
        // Q4_K: the odd sub-block's elements are the high nibbles, kept in
        // place as 16 q by the mask below, so their scale is d*sc/16 (exact)
        if constexpr (TYPE == kQ4_K) am *= (lane & 1) ? 0.0625f : 1.0f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int src = 2 * (4 * rq + s) + hi;
            if constexpr (TYPE == kQ4_K)
                q4_k_x4_masked(r.code[s][0], hi ? 0xF0F0F0F0u : 0x0F0F0F0Fu, lane_value(am, src), lane_value(bm, src),
                               wv[s]);
            else
                q5_k_x4(r.code[s][0], r.code[s][1], 2 * c + hi, hi != 0, lane_value(am, src), lane_value(bm, src),
                        wv[s]);
        }
    } else {  // Q6_K, Q2_K, Q3_K: this lane's pair is (row lane / 4, sub-scale slot lane % 4)
        const int e0 = k0 & 255, h = e0 >> 7, p0 = (e0 >> 5) & 3, p = p0 + hi, l16 = (j & 7) >> 2;
        const int w = lane & 3, si = 8 * h + 2 * (p0 + (w >> 1)) + (w & 1);
        float am, bm = 0.f;
        if constexpr (TYPE == kQ6_K)
            q6_k_coeffs(r.hdr[0], si & 1, half_to_f32(r.hdr[1]), am);
        else if constexpr (TYPE == kQ2_K)
            q2_k_coeffs(r.hdr[0], si & 3, half_to_f32(r.hdr[1] & 0xFFFFu), half_to_f32(r.hdr[1] >> 16), am, bm);
        else
            q3_k_coeffs(r.hdr[0], r.hdr[1], r.hdr[2], si, half_to_f32(r.hdr[3] & 0xFFFFu), am);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int src = 4 * (4 * rq + s) + 2 * hi + l16;
            const float a = lane_value(am, src);
            if constexpr (TYPE == kQ6_K)
                q6_k_x4(r.code[s][0], p >= 2, r.code[s][1], p, a, wv[s]);
            else if constexpr (TYPE == kQ2_K)
                q2_k_x4(r.code[s][0], p, a, lane_value(bm, src), wv[s]);
            else
                q3_k_x4(r.code[s][0], r.code[s][1], p, 4 * h + p, a, wv[s]);
        }
    }
}

// dst[t][k0 .. k0+63] for all t < T (T <= 16 TB <= 64). MFMA 16x16x4 operands:
// lane l supplies A[i = l%16][kk = l/16] and B[kk = l/16][j = l%16]. Step s
// of a 16-row group starting at n0 uses W row n0 + 4*(l/16) + s for lane l,
// so a lane reads G[t][n0 + 4*(l/16) .. +3] with one float4 per block of 16
// rows of G. Column j of accumulator block b is dst column k0 + 4*j + b, so a
// lane decodes 4 consecutive elements per row; each decoded element feeds
// one MFMA per block of 16 rows of G (TB of them), so the decode is shared
// by all of T. Each wave walks its own 16-row groups with the next group's
// loads in flight while the current one is decoded and contracted; the scale
// of each (row, block) is decoded by one lane and handed to the lanes that
// need it.
template <int TYPE, int NWAVES, bool FAST, int TB>
__global__ __launch_bounds__(NWAVES * 64) void out_prod_skinny_kernel(SkinnyArgs args) {
    constexpr int KS = 64;  // dst columns per workgroup
    __shared__ __attribute__((aligned(16))) float part[NWAVES * 16 * KS];

    enter_batch(args);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int K = args.K, N = args.N, T = args.T;
    // Consecutive 64-column slabs read the same 128-byte lines of every W row
    // (a Q4_K super-block spans four slabs): keep them on one XCD.
    const int k0 = xcd_remap(blockIdx.x, gridDim.x) * KS;
    const int j = lane & 15, rq = lane >> 4;

    f32x4 acc[TB][4];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[tb][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Decode a whole group, then issue its 16 TB MFMAs back to back (the
    // fences keep the compiler from interleaving each MFMA with the decode
    // of its own operand, which would stall on that dependency).
    auto contract = [&](const SkinnyRaw<TYPE, TB>& r) {
        float wv[4][4];
        skinny_decode<TYPE>(r, k0, lane, wv);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    acc[tb][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(r.g[tb][s], wv[s][b], acc[tb][b], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    // Full 16-row groups: group g goes to wave g % NWAVES. Loads run two
    // groups ahead of the contraction, rotating through three register
    // buffers; past the wave's last group the fetch repeats a valid group and
    // is not used.
    const int nfull = FAST ? N / 16 : 0;
    int g = wave;
    if (g < nfull) {
        const int last = nfull - 1;
        const int cnt = (nfull - wave + NWAVES - 1) / NWAVES;  // groups of this wave
        const SkinnyOffsets off = skinny_offsets<TYPE, TB>(args, k0, lane);
        auto row0 = [&](int i) { return 16 * min(wave + i * NWAVES, last); };
        SkinnyRaw<TYPE, TB> r0, r1, r2;
        skinny_fetch_fast(args, row0(0), off, r0);
        skinny_fetch_fast(args, row0(1), off, r1);
        // whole triples: no branch inside, so the loads of the next two groups
        // stay in flight while a group is contracted
        const int triples = cnt / 3;
        for (int t3 = 0, i = 0; t3 < triples; ++t3, i += 3) {
            skinny_fetch_fast(args, row0(i + 2), off, r2);
            contract(r0);
            skinny_fetch_fast(args, row0(i + 3), off, r0);
            contract(r1);
            skinny_fetch_fast(args, row0(i + 4), off, r1);
            contract(r2);
        }
        // 0, 1 or 2 groups left, already in r0 and r1
        const int left = cnt - 3 * triples;
        if (left >= 1) contract(r0);
        if (left >= 2) contract(r1);
        g = wave + cnt * NWAVES;
    }
    // Remaining (partial, or all groups of a shape off the fast path), masked.
    for (; 16 * g < N; g += NWAVES) {
        SkinnyRaw<TYPE, TB> r;
        skinny_fetch_masked(args, 16 * g, k0, lane, r);
        contract(r);
    }

    // D layout of v_mfma_f32_16x16x4f32: lane l, register v holds row
    // 4*(l/16) + v, column l%16. Partials of each wave go to LDS, then are
    // summed over waves in increasing wave order (deterministic), one block
    // of 16 rows of G at a time.
    float* mine = part + wave * 16 * KS;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        if (tb > 0) __syncthreads();  // the previous block's sums are read
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int v = 0; v < 4; ++v) mine[(4 * rq + v) * KS + 4 * j + b] = acc[tb][b][v];
        __syncthreads();
        for (int o = tid; o < 16 * KS; o += NWAVES * 64) {
            const int tr = 16 * tb + o / KS, kk = o % KS;
            float sum = part[o];
#pragma unroll
            for (int w = 1; w < NWAVES; ++w) sum += part[w * 16 * KS + o];
            if (tr < T && k0 + kk < K) args.dst[(long long)tr * args.ldd + k0 + kk] = sum;
        }
    }
}

// ---------------------------------------------------------------------------
// Skinny kernel with n split across workgroups (T <= 48 a launch, needs a
// workspace)
// ---------------------------------------------------------------------------
//
// The skinny kernel gives each 64-column slab of dst to one workgroup, so
// with fewer slabs than CUs part of the chip idles. Here the 16-row groups of
// all slabs, slab after slab, are cut into equal shares, one per workgroup
// (one per CU). A share covers the tail of one slab and the head of the next
// (or several whole slabs in between when shares are long). Each piece of a
// slab is summed as in the skinny kernel. A piece that is a whole slab is
// stored to dst; any other goes to its slot of the workspace, and the
// workgroup that finishes a slab's pieces last (a per-slab counter) adds the
// slab's slots in slot order and stores dst, so the result has the same bits
// whichever workgroup finishes last. Only a share's first and last piece can
// be part of a slab, so each workgroup owns two slots, and the counter of a
// split slab belongs to the workgroup holding its first group (no workgroup
// holds the first group of two split slabs): the workspace is 4 bytes plus
// two slots of 4 KiB per block of 16 rows of G per workgroup, whatever N and
// K. Slots and counters are read and written at device scope (the pieces of
// a slab may run on
// different XCDs); every counter is back at zero when the call ends. There is
// no waiting on other workgroups: each one runs to its end whatever the
// others do.
struct SkinnySplitArgs {
    unsigned* count;  // one word per workgroup: pieces of its counted slab finished so far
    float* slots;     // 16 TB x 64 floats per (workgroup, first or last piece)
    int ng;           // 16-row groups per slab (N / 16)
    long long share;  // groups per workgroup
};

template <int TYPE, int NWAVES, int TB>
__global__ __launch_bounds__(NWAVES * 64) void out_prod_skinny_split_kernel(SkinnyArgs args, SkinnySplitArgs sp) {
    constexpr int KS = 64;
    constexpr int SLOT = 16 * TB * KS;            // floats of a slot: all of T by the slab's columns
    constexpr int PER = SLOT / (NWAVES * 64);     // slab outputs per thread
    static_assert(PER * NWAVES * 64 == SLOT, "whole outputs per thread");
    __shared__ __attribute__((aligned(16))) float part[NWAVES * 16 * KS];
    __shared__ unsigned finisher[2];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int K = args.K, T = args.T, ng = sp.ng;
    const long long groups = (long long)((K + KS - 1) / KS) * ng;
    // consecutive shares (the two ends of a slab) on one XCD
    const int p = xcd_remap(blockIdx.x, gridDim.x);
    const long long begin = (long long)p * sp.share;
    const long long end = min(begin + sp.share, groups);
    if (begin >= end) return;
    const int j = lane & 15, rq = lane >> 4;

    // Piece [a, b) of slab s: the groups of this share inside that slab.
    struct Piece {
        int s, a, b;
    };
    auto piece_at = [&](long long at) {
        Piece pc;
        pc.s = int(at / ng);
        pc.a = int(at - (long long)pc.s * ng);
        pc.b = int(min(end - (long long)pc.s * ng, (long long)ng));
        return pc;
    };
    // Slabs this workgroup adds to without holding them whole: at most its
    // first piece and its last one.
    const int first_slab = int(begin / ng);
    int open0 = -1, open1 = -1;
    // the shares holding the first and the last group of slab s
    auto first_share = [&](int s) { return int((long long)s * ng / sp.share); };
    auto last_share = [&](int s) { return int(((long long)s * ng + ng - 1) / sp.share); };

    Piece cur = piece_at(begin);
    SkinnyOffsets off = skinny_offsets<TYPE, TB>(args, cur.s * KS, lane);
    SkinnyRaw<TYPE, TB> r0, r1, r2;
    // The first two groups of a piece for this wave, as the group loop
    // expects them (a repeat of a valid group past the wave's last one).
    auto prefetch = [&](const Piece& pc, const SkinnyOffsets& o) {
        const int g0 = min(pc.a + wave, pc.b - 1);
        skinny_fetch_fast(args, 16 * g0, o, r0);
        skinny_fetch_fast(args, 16 * min(g0 + NWAVES, pc.b - 1), o, r1);
    };
    prefetch(cur, off);

    for (;;) {
        const int k0 = cur.s * KS;
        f32x4 acc[TB][4];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[tb][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        auto contract = [&](const SkinnyRaw<TYPE, TB>& r) {
            float wv[4][4];
            skinny_decode<TYPE>(r, k0, lane, wv);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        acc[tb][c] = __builtin_amdgcn_mfma_f32_16x16x4f32(r.g[tb][q], wv[q][c], acc[tb][c], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        };
        // groups a + wave, a + wave + NWAVES, ... below b: the skinny
        // kernel's loop, two groups ahead
        const int g0 = cur.a + wave;
        if (g0 < cur.b) {
            const int last = cur.b - 1;
            const int cnt = (cur.b - g0 + NWAVES - 1) / NWAVES;
            auto row0 = [&](int i) { return 16 * min(g0 + i * NWAVES, last); };
            const int triples = cnt / 3;
            for (int t3 = 0, i = 0; t3 < triples; ++t3, i += 3) {
                skinny_fetch_fast(args, row0(i + 2), off, r2);
                contract(r0);
                skinny_fetch_fast(args, row0(i + 3), off, r0);
                contract(r1);
                skinny_fetch_fast(args, row0(i + 4), off, r1);
                contract(r2);
            }
            const int left = cnt - 3 * triples;
            if (left >= 1) contract(r0);
            if (left >= 2) contract(r1);
        }
        const long long next_at = (long long)cur.s * ng + cur.b;
        const Piece done = cur;
        // the next piece's first loads are in flight while this one is reduced
        if (next_at < end) {
            cur = piece_at(next_at);
            off = skinny_offsets<TYPE, TB>(args, cur.s * KS, lane);
            prefetch(cur, off);
        }

        // The skinny kernel's reduction over waves, in wave order, one block
        // of 16 rows of G at a time.
        const bool whole = (done.a == 0 && done.b == ng);
        // slot 2p for the share's first piece, 2p + 1 for its last
        float* slot = sp.slots + (2ll * p + (done.s != first_slab)) * SLOT;
        float* mine = part + wave * 16 * KS;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            if (tb > 0) __syncthreads();  // the previous block's sums are read
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int v = 0; v < 4; ++v) mine[(4 * rq + v) * KS + 4 * j + c] = acc[tb][c][v];
            __syncthreads();
            for (int o = tid; o < 16 * KS; o += NWAVES * 64) {
                const int tr = 16 * tb + o / KS, kk = o % KS;
                float sum = part[o];
#pragma unroll
                for (int w = 1; w < NWAVES; ++w) sum += part[w * 16 * KS + o];
                if (whole) {
                    if (tr < T && done.s * KS + kk < K) args.dst[(long long)tr * args.ldd + done.s * KS + kk] = sum;
                } else {
                    __hip_atomic_store(reinterpret_cast<unsigned*>(slot) + tb * 16 * KS + o, __float_as_uint(sum),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
        if (!whole) {
            if (open0 < 0)
                open0 = done.s;
            else
                open1 = done.s;
        }
        __syncthreads();  // part is rewritten by the next piece
        if (next_at >= end) break;
    }

    if (open0 < 0) return;
    // This workgroup's slots are complete at device scope before its counters
    // move; the last of a slab's pieces to arrive adds the slab's slots.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (tid == 0) {
        finisher[0] = __hip_atomic_fetch_add(sp.count + first_share(open0), 1u, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT) ==
                      unsigned(last_share(open0) - first_share(open0));
        finisher[1] = open1 >= 0 && __hip_atomic_fetch_add(sp.count + first_share(open1), 1u, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT) ==
                                        unsigned(last_share(open1) - first_share(open1));
    }
    __syncthreads();
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        if (!finisher[f]) continue;
        const int s = f ? open1 : open0, q0 = first_share(s), npieces = last_share(s) - q0 + 1;
        // Slot of share q0 + c: its first piece's (2q) unless slab s is not
        // where that share starts (2q + 1). Device-scope loads (sc1), a round
        // of four slots in flight at once.
        const __amdgpu_buffer_rsrc_t slots = buffer_rsrc(sp.slots + 2ll * q0 * SLOT, uint32_t(2 * npieces * SLOT * 4));
        auto slot_of = [&](int c) {
            const int q = q0 + c;
            return 2 * c + (int((long long)q * sp.share / ng) != s ? 1 : 0);
        };
        float sum[PER];
        for (int c0 = 0; c0 < npieces; c0 += 4) {
            float v[4][PER];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t base = uint32_t(slot_of(c0 + c) * SLOT * 4);
#pragma unroll
                for (int m = 0; m < PER; ++m)
                    v[c][m] = c0 + c < npieces
                                  ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                        slots, base + uint32_t((tid + m * NWAVES * 64) * 4), 0, 16))
                                  : 0.f;
            }
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int m = 0; m < PER; ++m) {
                    if (c0 + c == 0)
                        sum[m] = v[c][m];
                    else if (c0 + c < npieces)
                        sum[m] += v[c][m];
                }
        }
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int o = tid + m * NWAVES * 64, tr = o / KS, kk = o % KS;  // slot row tr = 16 tb + row of the block
            if (tr < T && s * KS + kk < K) args.dst[(long long)tr * args.ldd + s * KS + kk] = sum[m];
        }
        if (tid == 0) __hip_atomic_store(sp.count + q0, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---------------------------------------------------------------------------
// Dequantize kernel: out[n][k] = W[n][k]
// ---------------------------------------------------------------------------

struct DequantArgs {
    const uint8_t* W;
    float* out;
    int K, N;
    long long pitch;
    int wide;
    long long groups;  // N * groups_per_row
    int gpr;           // groups per row
};

// One thread decodes 4 consecutive elements (k = 4 * g within row n) with
// the same primitives the other kernels use.
template <int TYPE>
__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs args) {
    const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
    if (gid >= args.groups) return;
    const int n = (int)(gid / args.gpr);
    const int k = 4 * (int)(gid - (long long)n * args.gpr);
    float e[4];
    skinny_load4<TYPE>(args.W + (long long)n * args.pitch, k, args.K, args.wide, e);
    float* o = args.out + (long long)n * args.K + k;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (k + i < args.K) o[i] = e[i];
}

// ---------------------------------------------------------------------------
// mul_mat for shapes the tiled kernel refuses (dense rows with K % 4 != 0):
// one thread per output y[t][n], k increasing, decoded with the same
// primitives. A correctness path, not a fast one.
// ---------------------------------------------------------------------------

struct MmSimpleArgs {
    const uint8_t* W;
    const float* X;
    float* Y;
    int K, N, T;
    long long pitch, ldx, ldy;
    int wide;
};

template <int TYPE>
__global__ __launch_bounds__(256) void mul_mat_simple_kernel(MmSimpleArgs a) {
    const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
    if (gid >= (long long)a.T * a.N) return;
    const int t = (int)(gid / a.N), n = (int)(gid - (long long)t * a.N);
    const uint8_t* row = a.W + (long long)n * a.pitch;
    const float* x = a.X + (long long)t * a.ldx;
    float acc = 0.f;
    for (int k = 0; k < a.K; k += 4) {
        float e[4];
        skinny_load4<TYPE>(row, k, a.K, a.wide, e);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (k + i < a.K) acc = fmaf(e[i], x[k + i], acc);
    }
    a.Y[(long long)t * a.ldy + n] = acc;
}

}  // namespace retro
