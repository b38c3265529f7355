// retro_ws_kernel.h - OUT_PROD tile kernel with producer and consumer waves.
//
// Same contraction and tile mapping as out_prod_tile_kernel, organised so
// that the matrix pipe never waits on staging:
//   * NC + 4 waves per workgroup (NC = 4, or 8 for the 256 x 256 tile). Waves
//     0 .. NC - 1 (consumers, a CT x NC/CT grid over the tile) only read
//     operands from LDS and issue v_mfma_f32_32x32x2_f32. The last 4 waves
//     (producers) load G and packed W with buffer loads, decode W in
//     registers and write both into LDS.
//   * G and decoded W are double-buffered in LDS: while the consumers contract
//     chunk c from buffer c % 2, the producers fill buffer (c + 1) % 2 with
//     chunk c + 1, whose loads they issued one chunk earlier. One workgroup
//     barrier per 32-row chunk.
//   * With eight consumers (12 waves, three per SIMD) every decoded weight
//     feeds twice the matrix work of four, at the cost of one operand set per
//     consumer in the 168-register budget (see ws_consume).
//   * With NG = 2 the workgroup holds two such pipelines (16 waves) over the
//     same output tile, one for the even and one for the odd chunks, sharing
//     the barriers; their partial sums are added in LDS at the end. Each SIMD
//     then holds two consumer waves, whose MFMAs fill each other's waits, for
//     shapes with too few tiles for two workgroups per CU.
//   * Both operands are read as 16-byte vectors. G is kept t-major (a row of
//     32 reduction values per t) and decoded W k-major (a column of 32
//     reduction values per k), and MFMA step r of phase q contracts rows
//     8q + 4h + r in lane half h, so each lane's four steps of a phase sit in
//     one float4 of G and one float4 of W.
// On gfx950 VALU work and F32 MFMA work take turns on a SIMD (they do not
// overlap), so a SIMD holding one consumer and one producer wave spends its
// time on MFMA plus decode and little else.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "retro_kernels.h"

namespace retro {

template <int TYPE, int WA, int WB, int CT, int NG = 1, int NC_ = 4>
struct WsShape {
    using F = Format<TYPE>;
    static constexpr bool kDense = F::kBlock == 1;
    static_assert(NG == 1 || NG == 2, "one or two pipelines");
    // consumer waves per pipeline: 4, or 8 (one pipeline) for the 256 x 256
    // tile, whose producers' decode then feeds twice the matrix work
    static constexpr int NC = NC_;
    static_assert(NC == 4 || (NC == 8 && NG == 1), "4 consumer waves, or 8 with one pipeline");
    static constexpr int kPThreads = 256;                        // producer threads of one pipeline (4 waves)
    static constexpr int kCThreads = 64 * NC;                    // consumer threads of one pipeline
    static constexpr int kThreads = (kCThreads + kPThreads) * NG;
    // consumer waves CT x CK, each (32*WA) x (32*WB) outputs
    static_assert((NC == 4 && (CT == 1 || CT == 2)) || (NC == 8 && CT == 2), "consumer grid 1x4, 2x2 or 2x4");
    static constexpr int CK = NC / CT;
    // consumers keep two operand sets (the next phase read during this one's
    // MFMAs) when the register budget allows
    static constexpr bool kPrefetch = NC == 4 || WA * WB <= 4;
    static constexpr int BT = 32 * WA * CT;
    static constexpr int BK = 32 * WB * CK;
    static constexpr int BN = 32;
    static_assert(BK == 128 || BK == 256, "K tile of 128 or 256 columns");
    static_assert(!kSuperBlock<TYPE> || BK == 256, "K-quant tiles hold whole super-blocks");
    static constexpr int GP = BN + 4;  // floats per t row of G in LDS
    static constexpr int WP = BN + 4;  // floats per k column of W in LDS
    static constexpr int G_FLOATS = BT * GP;
    static constexpr int W_FLOATS = BK * WP;
    static constexpr int BUF_FLOATS = G_FLOATS + W_FLOATS;
    // workgroups that fit on a CU by LDS (160 KB), at most two (16 waves)
    static constexpr int kResident = (NG == 2 || (160 * 1024) / (2 * BUF_FLOATS * 4) < 2) ? 1 : 2;
    // Workgroups per CU the register budget is set for: two for the 32-row
    // tiles whose LDS allows it (32x128, 45 KB), whose second workgroup fills
    // the first one's barrier waits; one otherwise. The kernel's launch bound
    // states it as waves per SIMD (amdgpu_waves_per_eu): a workgroup's waves
    // spread over the CU's four SIMDs, so two 8-wave workgroups are 4 waves
    // per SIMD, a budget of 128 VGPRs each.
    static constexpr int kWgPerCu = (BT == 32 && kResident == 2) ? 2 : 1;
    static constexpr int kWavesPerSimd = kThreads / 64 / 4 * kWgPerCu;
    static_assert(kThreads % 256 == 0, "whole waves on each of the four SIMDs");
    static constexpr int GSLOTS = BT * BN / 4 / kPThreads;  // float4 of G per producer thread
    static_assert(GSLOTS * kPThreads * 4 == BT * BN, "G chunk splits evenly");
    // Dense W: units of 4 rows x 4 consecutive k (16 bytes of F32 or 8 of
    // F16/BF16 per row, DWPR words), so that each k column of a unit is one
    // float4 store into the k-major LDS layout.
    static constexpr int DWPR = F::kBytes;
    static constexpr int DUNITS = kDense ? (BN / 4) * (BK / 4) / kPThreads : 0;
    static_assert(!kDense || DUNITS * kPThreads * 16 == BN * BK, "dense chunk splits evenly");
    // Q8_0 and the 32-element nibble blocks: a block is split over QSPLIT
    // producer threads, each holding CB code bytes of it.
    static constexpr int QSPLIT = (TYPE == kQ8_0 || kNibbleLayout<TYPE>) ? kPThreads / (BN * BK / 32) : 1;
    static constexpr int CB = TYPE == kQ8_0 ? 32 / QSPLIT : 16 / QSPLIT;
    // NVFP4: each producer thread takes NV_SB consecutive 16-element
    // sub-blocks of one row (8 threads per row of the chunk).
    static constexpr int NV_SB = BK / 128;
    // words of W each producer thread holds between load and decode
    static constexpr int WWORDS = kDense ? 4 * DWPR * DUNITS
                                  : (TYPE == kQ4_K) ? 8
                                  : (TYPE == kQ5_K) ? 12
                                  : (TYPE == kQ6_K) ? 9
                                  : (TYPE == kQ2_K) ? 5
                                  : (TYPE == kQ3_K) ? 8
                                  : (TYPE == kNVFP4) ? 2 * NV_SB + 1
                                  : kHasFifth<TYPE> ? CB / 4 + 2
                                                    : CB / 4 + 1;
    // Chunks whose loads a producer thread keeps in registers: the chunk
    // being written to LDS plus RING - 1 in flight. Four when a chunk's
    // staging fits in 32 registers (small tiles, whose chunks are short next
    // to the global-load latency), else two. Even, so the LDS buffer of a
    // slot's chunk is fixed.
    static constexpr int SLOT_REGS = 4 * GSLOTS + WWORDS;
    static constexpr int RING = SLOT_REGS <= 32 ? 4 : 2;
};

// f(integral_constant<int, 0>{}), ..., f(integral_constant<int, COUNT - 1>{})
template <typename Fn, int... Is>
__device__ __forceinline__ void static_for_impl(Fn&& f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int COUNT, typename Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
    static_for_impl(f, std::make_integer_sequence<int, COUNT>{});
}

// Float index of W element (row n, column k) of a chunk inside the W part of
// an LDS buffer: column k holds its 32 rows with the aligned 4-row groups
// XOR-permuted by a 3-bit function of bits 3-7 of k (bit 0: k4 ^ k5, bit 1:
// k3 ^ k6, bit 2: k3 ^ k4 ^ k7). The permutation keeps every 4-row group
// together and in order, so a consumer still reads 4 rows as one float4; it
// is constant over each aligned group of 8 columns, so the 8 lanes of a
// float4 read (8 consecutive columns) still cover the 32 banks once; and it
// gives the lanes of every producer store pattern distinct banks: 4-byte
// stores of one row into 8 or 16 consecutive columns per lane (the lanes
// differing in row and in column bits 3-7 by the type's thread mapping) and
// float4 stores of 4 rows. A model of the 32-bank LDS counts no conflicts
// for any type or tile with it, against 128-768 extra cycles per chunk with
// bits 4-6 of k alone (which the conflict counters matched).
template <int WP>
__device__ __forceinline__ int ws_w_index(int k, int n) {
    const int v = (((k >> 4) ^ (k >> 5)) & 1) | ((((k >> 3) ^ (k >> 6)) & 1) << 1) |
                  ((((k >> 3) ^ (k >> 4) ^ (k >> 7)) & 1) << 2);
    return k * WP + (n ^ (v << 2));
}

// Consumer waves 0 .. NC NG - 1 of a producer/consumer tile kernel: contract
// the nloc chunks its pipeline's producers publish in LDS (shape S: BT x BK
// outputs, chunks of 32 reduction values; G-side operand t-major with pitch
// GP, W-side operand k-major through ws_w_index) and store the BT x BK tile
// at rows t0.., columns c0.. of dst (rows < T and columns < ncols only).
template <typename S, int WA, int WB, int NG>
__device__ __forceinline__ void ws_consume(float* lds_all, int tid, int wave, int nloc, int t0, int c0, int T,
                                           int ncols, float* dst, long long ldd) {
    const int lane = tid & 63;
    static_assert(NG == 1 || S::NC == 4, "two pipelines have four consumer waves each");
    const int cg = wave / S::NC, cw = wave % S::NC;  // pipeline, wave within it
    const int wt = cw / S::CK, wk = cw % S::CK;
    const float* const lds = lds_all + cg * 2 * S::BUF_FLOATS;
    constexpr int GP = S::GP, WP = S::WP;
    const int h = lane >> 5, l32 = lane & 31;
    f32x16 acc[WA][WB];
#pragma unroll
    for (int a = 0; a < WA; ++a)
#pragma unroll
        for (int b = 0; b < WB; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

    // Phase q reads G[t][8q + 4h .. + 3] for the lane's t rows and
    // W[8q + 4h .. + 3][k] for its k columns; the W index depends on q
    // through the group permutation, so it is kept per phase.
    const float* gbase = lds + (wt * 32 * WA + l32) * GP + 4 * h;
    int widx[4][WB];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int b = 0; b < WB; ++b)
            widx[q][b] = S::G_FLOATS + ws_w_index<WP>(wk * 32 * WB + 32 * b + l32, 8 * q + 4 * h);

    auto read_phase = [&](auto buf_tag, int q, f32x4 (&av)[WA], f32x4 (&bv)[WB]) {
        constexpr int off = decltype(buf_tag)::value * S::BUF_FLOATS;
#pragma unroll
        for (int a = 0; a < WA; ++a) av[a] = *reinterpret_cast<const f32x4*>(gbase + off + 32 * a * GP + 8 * q);
#pragma unroll
        for (int b = 0; b < WB; ++b) bv[b] = *reinterpret_cast<const f32x4*>(lds + off + widx[q][b]);
    };
    auto mfma_phase = [&](const f32x4 (&av)[WA], const f32x4 (&bv)[WB]) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int a = 0; a < WA; ++a)
#pragma unroll
                for (int b = 0; b < WB; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[a][r], bv[b][r], acc[a][b], 0, 0, 0);
    };
    // One chunk from buffer BUF. Phase q + 1 is read while phase q's MFMAs
    // run; phase 0 of the next chunk (buffer 1 - BUF) is read right after the
    // barrier that publishes it, ahead of this chunk's last MFMAs. After the
    // last chunk that read sees a stale buffer and its values are unused.
    // With eight consumer waves of 128 accumulators each (two per SIMD) the
    // register budget holds one operand set: each phase is read, then
    // contracted, and the SIMD's other consumer wave covers the read latency.
    constexpr bool kPrefetch = S::kPrefetch;
    f32x4 a0[WA], b0[WB];
    f32x4 a1[kPrefetch ? WA : 1], b1[kPrefetch ? WB : 1];
    auto chunk = [&](auto buf_tag) {
        using Next = std::integral_constant<int, 1 - decltype(buf_tag)::value>;
        if constexpr (kPrefetch) {
            read_phase(buf_tag, 1, a1, b1);
            mfma_phase(a0, b0);
            read_phase(buf_tag, 2, a0, b0);
            mfma_phase(a1, b1);
            read_phase(buf_tag, 3, a1, b1);
            mfma_phase(a0, b0);
            __syncthreads();
            read_phase(Next{}, 0, a0, b0);
            mfma_phase(a1, b1);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                read_phase(buf_tag, q, a0, b0);
                mfma_phase(a0, b0);
            }
            __syncthreads();
        }
    };
    using Buf0 = std::integral_constant<int, 0>;
    using Buf1 = std::integral_constant<int, 1>;
    __syncthreads();
    if constexpr (kPrefetch) read_phase(Buf0{}, 0, a0, b0);
    for (int c = 0; c < nloc; c += 2) {
        chunk(Buf0{});
        if (c + 1 < nloc) chunk(Buf1{});
    }
    if constexpr (NG == 2) {
        // pipeline 1's sums -> LDS (register r of lane l of wave w at
        // r * 256 + 64 w + l), added to pipeline 0's in that fixed order
        constexpr int NR = WA * WB * 16;
        static_assert(NR * 256 <= 2 * NG * S::BUF_FLOATS, "reduction fits in LDS");
        __syncthreads();
        float* red = lds_all + 64 * cw + lane;
        if (cg == 1) {
#pragma unroll
            for (int a = 0; a < WA; ++a)
#pragma unroll
                for (int b = 0; b < WB; ++b)
#pragma unroll
                    for (int v = 0; v < 16; ++v) red[((a * WB + b) * 16 + v) * 256] = acc[a][b][v];
        }
        __syncthreads();
        if (cg == 1) return;
#pragma unroll
        for (int a = 0; a < WA; ++a)
#pragma unroll
            for (int b = 0; b < WB; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[a][b][v] += red[((a * WB + b) * 16 + v) * 256];
    }

    // D layout of v_mfma_f32_32x32x2f32: lane l, register v holds
    // row 8*(v/4) + 4*(l/32) + v%4, column l%32.
#pragma unroll
    for (int a = 0; a < WA; ++a)
#pragma unroll
        for (int b = 0; b < WB; ++b) {
            const int k = c0 + wk * 32 * WB + 32 * b + l32;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int t = t0 + wt * 32 * WA + 32 * a + 8 * (v >> 2) + 4 * h + (v & 3);
                if (t < T && k < ncols) dst[(long long)t * ldd + k] = acc[a][b][v];
            }
        }
}

// GCOLS: G stored t-fastest (args.ldg floats between its columns); the
// consumers see the same LDS contents either way.
template <int TYPE, int WA, int WB, int CT, int NG, int NC, bool GCOLS>
__global__ __launch_bounds__((WsShape<TYPE, WA, WB, CT, NG, NC>::kThreads),
                             (WsShape<TYPE, WA, WB, CT, NG, NC>::kWavesPerSimd)) void out_prod_ws_kernel(TileArgs args) {
    using S = WsShape<TYPE, WA, WB, CT, NG, NC>;
    using F = Format<TYPE>;
    constexpr int BT = S::BT, BK = S::BK, BN = S::BN, GP = S::GP, WP = S::WP;

    __shared__ __attribute__((aligned(16))) float lds_all[2 * NG * S::BUF_FLOATS];

    enter_batch(args);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tt, tk;
    tile_coords(blockIdx.x, args.tiles_t, args.tiles_k, args.group, tt, tk);
    const int t0 = tt * BT, k0 = tk * BK;
    const int K = args.K, N = args.N, T = args.T;
    // pipeline g takes chunks g, g + NG, g + 2 NG, ...: nloc of them each (a
    // chunk past the last one reads and contracts zeros)
    const int nloc = ((N + BN - 1) / BN + NG - 1) / NG;

    // The two roles run separate loops with the same barrier sequence (one
    // after the prologue, one per chunk): the role test is uniform per wave,
    // and keeping the loops apart keeps the consumers' accumulators and the
    // producers' staging registers from being allocated side by side.
    if (wave >= NC * NG) {
        // ---------------- producer ----------------
        const int pg = (tid - NG * S::kCThreads) >> 8;  // pipeline
        const int p = (tid - NG * S::kCThreads) & (S::kPThreads - 1);
        float* const lds = lds_all + pg * 2 * S::BUF_FLOATS;
        auto chunk_n0 = [&](int c) { return (pg + NG * c) * BN; };
        const long long kb0 = (long long)(k0 / F::kBlock) * F::kBytes;
        constexpr int R = S::RING;
        float4 gring[R][S::GSLOTS];
        uint32_t wring[R][S::WWORDS];
        // Byte offsets of this thread's G loads from the chunk's base (the
        // same for every chunk): slot s is t row id / 8, columns
        // 4 (id % 8) .. + 3. With G stored t-fastest the thread holds a block
        // of GSLOTS columns by 4 t rows instead: slot s is column
        // GSLOTS (p % CG) + s, t rows 4 (p / CG) .. + 3 (CG = 32 / GSLOTS
        // column groups), so that each t row of the block is one LDS store.
        constexpr int CG = BN / S::GSLOTS;
        static_assert(CG * (BT / 4) == S::kPThreads, "column blocks cover the G chunk");
        uint32_t goff[S::GSLOTS];
#pragma unroll
        for (int s = 0; s < S::GSLOTS; ++s) {
            const int id = p + S::kPThreads * s;
            goff[s] = GCOLS ? uint32_t(((S::GSLOTS * (p % CG) + s) * args.ldg + 4 * (p / CG)) * 4)
                            : uint32_t(((id >> 3) * args.ldg + 4 * (id & 7)) * 4);
        }
        // W: byte offset of this thread's block in the chunk, and the LDS
        // float index of the first element it writes in each aligned group of
        // 8 columns (ws_w_index permutes rows per such group; the columns of
        // a group are then WP floats apart).
        uint32_t woff = 0;
        int wlds[S::kDense ? S::DUNITS : 4];
        if constexpr (S::kDense) {
            // unit id: rows 4 (id / (BK / 4)) .. + 3, columns 4 (id % (BK / 4)) .. + 3
#pragma unroll
            for (int s = 0; s < S::DUNITS; ++s) {
                const int id = p + S::kPThreads * s, rg = id / (BK / 4), u = id - rg * (BK / 4);
                wlds[s] = ws_w_index<WP>(4 * u, 4 * rg);
            }
        } else if constexpr (TYPE == kQ4_K || TYPE == kQ5_K) {
            // code unit p % 8 (16 bytes) of row p / 8: low nibbles are columns
            // 64c + 16h + 0..15, high nibbles 64c + 32 + 16h + 0..15
            const int r = p >> 3, u = p & 7, c = u >> 1, h = u & 1;
            woff = uint32_t(r * args.pitch);
            wlds[0] = ws_w_index<WP>(64 * c + 16 * h, r);
            wlds[1] = ws_w_index<WP>(64 * c + 16 * h + 8, r);
            wlds[2] = ws_w_index<WP>(64 * c + 32 + 16 * h, r);
            wlds[3] = ws_w_index<WP>(64 * c + 32 + 16 * h + 8, r);
        } else if constexpr (TYPE == kQ6_K || TYPE == kQ2_K || TYPE == kQ3_K) {
            // half hh, l range 8j .. 8j + 7 of row p / 8: columns
            // 128 hh + 32 qq + 8j + 0..7 of the four quarters qq
            const int r = p >> 3, hh = (p >> 2) & 1, j = p & 3;
            woff = uint32_t(r * args.pitch);
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) wlds[qq] = ws_w_index<WP>(128 * hh + 32 * qq + 8 * j, r);
        } else if constexpr (TYPE == kNVFP4) {
            // sub-blocks NV_SB u .. NV_SB u + NV_SB - 1 of row p / 8 (u = p % 8):
            // columns 16 NV_SB u .., one 16-column group each
            const int r = p >> 3, col = 16 * S::NV_SB * (p & 7);
            woff = uint32_t(r * args.pitch + (col >> 6) * 36);
#pragma unroll
            for (int i = 0; i < 2 * S::NV_SB; ++i) wlds[i] = ws_w_index<WP>(col + 8 * i, r);
        } else {
            // part s of block b of row r: code bytes CB s .. CB s + CB - 1
            const int id = p / S::QSPLIT, s = p - id * S::QSPLIT;
            const int r = id / (BK / 32), b = id - r * (BK / 32);
            woff = uint32_t(r * args.pitch + b * F::kBytes);
            if constexpr (TYPE == kQ8_0) {
                // columns 32b + CB s + 0 .. CB - 1: CB / 8 groups of 8
#pragma unroll
                for (int g = 0; g < S::CB / 8; ++g) wlds[g] = ws_w_index<WP>(32 * b + S::CB * s + 8 * g, r);
            } else {
                // byte j: low nibble is column 32b + j, high nibble 32b + 16 + j;
                // the thread's bytes CB s .. give CB / 8 groups of 8 in each half
#pragma unroll
                for (int g = 0; g < S::CB / 8; ++g) {
                    wlds[g] = ws_w_index<WP>(32 * b + S::CB * s + 8 * g, r);
                    wlds[2 + g] = ws_w_index<WP>(32 * b + 16 + S::CB * s + 8 * g, r);
                }
            }
        }
        // elements spanned by G (none when N = 0: G is empty and its pointer
        // may be null)
        const long long g_end =
            N == 0 ? 0 : GCOLS ? (long long)(N - 1) * args.ldg + T : (long long)(T - 1) * args.ldg + N;
        // bytes spanned by W: rows are `pitch` apart, the last one ends after
        // its K / block blocks
        const long long w_end =
            N > 0 ? (long long)(N - 1) * args.pitch + (long long)(K / F::kBlock) * F::kBytes : 0;

        // Loads of chunk rows [n0, n0 + 32) into registers, issued the same way
        // for every chunk (no branch), so that the loads of later chunks stay
        // in flight while an earlier slot is written to LDS. The buffer ranges
        // end at the end of G and of W: rows at or past N read as zero, and a
        // chunk past the last one reads zeros or rows it never uses. G columns
        // at or past N in the last chunk (the next t row's values) are zeroed
        // when the chunk is written to LDS. Columns past K in the last k tile
        // read bytes of the next row (or zero), and G rows past T (other values
        // when G is stored t-fastest) are read too: both only reach outputs
        // that are not stored. ldg % 4 == 0, so the G loads are 16-byte aligned.
        auto load_chunk = [&](auto slot, int n0) {
            float4(&greg)[S::GSLOTS] = gring[decltype(slot)::value];
            uint32_t(&wreg)[S::WWORDS] = wring[decltype(slot)::value];
            n0 = __builtin_amdgcn_readfirstlane(n0);
            const long long gb = GCOLS ? (long long)n0 * args.ldg + t0 : (long long)t0 * args.ldg + n0;
            const __amdgpu_buffer_rsrc_t gr =
                buffer_rsrc(args.G + gb, uint32_t(max(0ll, min(4 * (g_end - gb), (long long)0x7FFFFFFF))));
#pragma unroll
            for (int s = 0; s < S::GSLOTS; ++s) {
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(gr, goff[s], 0, 0);
                greg[s] = make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                                      __uint_as_float(v.w));
            }
            const long long wb = (long long)n0 * args.pitch + kb0;
            const __amdgpu_buffer_rsrc_t wr =
                buffer_rsrc(args.W + wb, uint32_t(max(0ll, min(w_end - wb, (long long)0x7FFFFFFF))));
            if constexpr (S::kDense) {
#pragma unroll
                for (int s = 0; s < S::DUNITS; ++s) {
                    const int id = p + S::kPThreads * s, rg = id / (BK / 4), u = id - rg * (BK / 4);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t o = uint32_t((4 * rg + j) * args.pitch + 4 * S::DWPR * u);
                        uint32_t* dstw = wreg + (4 * s + j) * S::DWPR;
                        if constexpr (S::DWPR == 4) {
                            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(wr, o, 0, 0);
                            dstw[0] = v.x; dstw[1] = v.y; dstw[2] = v.z; dstw[3] = v.w;
                        } else {
                            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(wr, o, 0, 0);
                            dstw[0] = v.x; dstw[1] = v.y;
                        }
                    }
                }
            } else if constexpr (TYPE == kQ4_K) {
                const u32x4 cw = __builtin_amdgcn_raw_buffer_load_b128(wr, woff + 16 + 16 * (p & 7), 0, 0);
                const u32x4 hd = __builtin_amdgcn_raw_buffer_load_b128(wr, woff, 0, 0);
                wreg[0] = cw.x; wreg[1] = cw.y; wreg[2] = cw.z; wreg[3] = cw.w;
                wreg[4] = hd.x; wreg[5] = hd.y; wreg[6] = hd.z; wreg[7] = hd.w;
            } else if constexpr (TYPE == kQ5_K) {
                // code unit, header, and the 16 fifth-bit bytes of the same elements
                const u32x4 cw = __builtin_amdgcn_raw_buffer_load_b128(wr, woff + 48 + 16 * (p & 7), 0, 0);
                const u32x4 hd = __builtin_amdgcn_raw_buffer_load_b128(wr, woff, 0, 0);
                const u32x4 qh = __builtin_amdgcn_raw_buffer_load_b128(wr, woff + 16 + 16 * (p & 1), 0, 0);
                wreg[0] = cw.x; wreg[1] = cw.y; wreg[2] = cw.z; wreg[3] = cw.w;
                wreg[4] = hd.x; wreg[5] = hd.y; wreg[6] = hd.z; wreg[7] = hd.w;
                wreg[8] = qh.x; wreg[9] = qh.y; wreg[10] = qh.z; wreg[11] = qh.w;
            } else if constexpr (TYPE == kQ6_K) {
                // ql bytes 64hh + 8j .. (quarters 0, 2) and 64hh + 32 + 8j ..
                // (1, 3), qh bytes 128 + 32hh + 8j .., the 8 sub-scales of half
                // hh, d. The super-blocks are only 2-byte aligned; the 8-byte
                // loads rely on the unaligned buffer access of gfx9-class GPUs.
                const int hh = (p >> 2) & 1, j = p & 3;
                const uint32_t at[4] = {woff + 64 * hh + 8 * j, woff + 64 * hh + 32 + 8 * j,
                                        woff + 128 + 32 * hh + 8 * j, woff + 192 + 8 * hh};
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(wr, at[f], 0, 0);
                    wreg[2 * f] = v.x;
                    wreg[2 * f + 1] = v.y;
                }
                wreg[8] = __builtin_amdgcn_raw_buffer_load_b16(wr, woff + 208, 0, 0);
            } else if constexpr (TYPE == kQ2_K) {
                // qs bytes 16 + 32hh + 8j .. (the 2-bit codes of all four
                // quarters), the 8 pair bytes of half hh, d and dmin
                const int hh = (p >> 2) & 1, j = p & 3;
                const u32x2 c = __builtin_amdgcn_raw_buffer_load_b64(wr, woff + 16 + 32 * hh + 8 * j, 0, 0);
                const u32x2 pr = __builtin_amdgcn_raw_buffer_load_b64(wr, woff + 8 * hh, 0, 0);
                wreg[0] = c.x; wreg[1] = c.y; wreg[2] = pr.x; wreg[3] = pr.y;
                wreg[4] = __builtin_amdgcn_raw_buffer_load_b32(wr, woff + 80, 0, 0);
            } else if constexpr (TYPE == kQ3_K) {
                // qs bytes 32 + 32hh + 8j .., hmask bytes 8j .., the 12-byte
                // sub-scale field and d (bytes 96 .. 109; no load reaches past
                // the block, whose end may be the end of W)
                const int hh = (p >> 2) & 1, j = p & 3;
                const u32x2 c = __builtin_amdgcn_raw_buffer_load_b64(wr, woff + 32 + 32 * hh + 8 * j, 0, 0);
                const u32x2 hm = __builtin_amdgcn_raw_buffer_load_b64(wr, woff + 8 * j, 0, 0);
                const u32x2 f = __builtin_amdgcn_raw_buffer_load_b64(wr, woff + 96, 0, 0);
                wreg[0] = c.x; wreg[1] = c.y; wreg[2] = hm.x; wreg[3] = hm.y;
                wreg[4] = f.x; wreg[5] = f.y;
                wreg[6] = __builtin_amdgcn_raw_buffer_load_b32(wr, woff + 104, 0, 0);
                wreg[7] = __builtin_amdgcn_raw_buffer_load_b16(wr, woff + 108, 0, 0);
            } else if constexpr (TYPE == kNVFP4) {
                // the code bytes of the thread's sub-blocks (8 each) and their
                // scale bytes; 36-byte blocks are 4-byte aligned
                const int sb0 = (S::NV_SB * (p & 7)) & 3;
                if constexpr (S::NV_SB == 1) {
                    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(wr, woff + 4 + 8 * sb0, 0, 0);
                    wreg[0] = v.x; wreg[1] = v.y;
                    wreg[2] = __builtin_amdgcn_raw_buffer_load_b8(wr, woff + sb0, 0, 0);
                } else {
                    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(wr, woff + 4 + 8 * sb0, 0, 0);
                    wreg[0] = v.x; wreg[1] = v.y; wreg[2] = v.z; wreg[3] = v.w;
                    wreg[4] = __builtin_amdgcn_raw_buffer_load_b16(wr, woff + sb0, 0, 0);
                }
            } else {  // Q8_0, nibble blocks: 2-byte (MXFP4: any) aligned blocks (unaligned buffer loads)
                constexpr int CW = S::CB / 4;
                constexpr int HDR = TYPE == kQ8_0 ? 2 : kHeader<TYPE>;
                const uint32_t codes = woff + HDR + S::CB * (p % S::QSPLIT);
                // header: d (and m), or its first 8 bytes (d, m, qh) for the
                // fifth-bit blocks, which are 22 or 24 bytes long
                if constexpr (kHasFifth<TYPE>) {
                    const u32x2 h = __builtin_amdgcn_raw_buffer_load_b64(wr, woff, 0, 0);
                    wreg[CW] = h.x;
                    wreg[CW + 1] = h.y;
                } else if constexpr (TYPE == kQ4_1) {
                    wreg[CW] = __builtin_amdgcn_raw_buffer_load_b32(wr, woff, 0, 0);
                } else if constexpr (TYPE == kMXFP4) {
                    wreg[CW] = __builtin_amdgcn_raw_buffer_load_b8(wr, woff, 0, 0);
                } else {
                    wreg[CW] = __builtin_amdgcn_raw_buffer_load_b16(wr, woff, 0, 0);
                }
                if constexpr (CW == 2) {
                    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(wr, codes, 0, 0);
                    wreg[0] = v.x; wreg[1] = v.y;
                } else {
#pragma unroll
                    for (int w = 0; w < CW; w += 4) {
                        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(wr, codes + 4 * w, 0, 0);
                        wreg[w] = v.x; wreg[w + 1] = v.y; wreg[w + 2] = v.z; wreg[w + 3] = v.w;
                    }
                }
            }
        };

        // Registers of `slot` -> LDS buffer `buf`: G rows as loaded, W decoded
        // to F32 into its k-major columns (element j of a 16-column group is
        // WP floats after element j - 1).
        auto store_chunk = [&](auto slot, auto buf, int n0) {
            float4(&greg)[S::GSLOTS] = gring[decltype(slot)::value];
            const uint32_t(&wreg)[S::WWORDS] = wring[decltype(slot)::value];
            float* gs = lds + decltype(buf)::value * S::BUF_FLOATS;
            float* ws = gs + S::G_FLOATS;
            if constexpr (GCOLS) {
                // the thread's block, transposed: t row j of it is element j
                // of every slot, stored as one vector of GSLOTS columns
                constexpr int GS = S::GSLOTS;
                const int c0 = GS * (p % CG);
                if (n0 + BN > N) {
#pragma unroll
                    for (int s = 0; s < GS; ++s)
                        if (n0 + c0 + s >= N) greg[s] = make_float4(0.f, 0.f, 0.f, 0.f);
                }
                auto elem = [](const float4& v, int j) { return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w; };
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float* row = gs + (4 * (p / CG) + j) * GP + c0;
                    if constexpr (GS % 4 == 0) {  // GS / 4 vectors of 4 columns
#pragma unroll
                        for (int v = 0; v < GS; v += 4)
                            *reinterpret_cast<float4*>(row + v) = make_float4(elem(greg[v], j), elem(greg[v + 1], j),
                                                                              elem(greg[v + 2], j), elem(greg[v + 3], j));
                    } else if constexpr (GS == 2) {
                        *reinterpret_cast<float2*>(row) = make_float2(elem(greg[0], j), elem(greg[1], j));
                    } else {
                        static_assert(GS == 1, "G slots per producer thread: 1, 2 or a multiple of 4");
                        row[0] = elem(greg[0], j);
                    }
                }
            } else {
                if (n0 + BN > N) {
#pragma unroll
                    for (int s = 0; s < S::GSLOTS; ++s) {
                        const int n = n0 + 4 * ((p + S::kPThreads * s) & 7);
                        if (n >= N) greg[s].x = 0.f;
                        if (n + 1 >= N) greg[s].y = 0.f;
                        if (n + 2 >= N) greg[s].z = 0.f;
                        if (n + 3 >= N) greg[s].w = 0.f;
                    }
                }
#pragma unroll
                for (int s = 0; s < S::GSLOTS; ++s) {
                    const int id = p + S::kPThreads * s;
                    *reinterpret_cast<float4*>(gs + (id >> 3) * GP + 4 * (id & 7)) = greg[s];
                }
            }
            if constexpr (S::kDense) {
#pragma unroll
                for (int s = 0; s < S::DUNITS; ++s) {
                    // v[j][e]: row j, column e of the unit
                    float v[4][4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t* w = wreg + (4 * s + j) * S::DWPR;
                        if constexpr (TYPE == kF32) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) v[j][e] = __uint_as_float(w[e]);
                        } else if constexpr (TYPE == kF16) {
                            f16x2(w[0], v[j][0], v[j][1]);
                            f16x2(w[1], v[j][2], v[j][3]);
                        } else {
                            bf16x2(w[0], v[j][0], v[j][1]);
                            bf16x2(w[1], v[j][2], v[j][3]);
                        }
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        *reinterpret_cast<float4*>(ws + wlds[s] + e * WP) = make_float4(v[0][e], v[1][e], v[2][e], v[3][e]);
                }
            } else if constexpr (TYPE == kQ4_K) {
                const int c = (p & 7) >> 1;
                float a0, b0, a1, b1;
                q4_k_coeffs(wreg[4], wreg[5], wreg[6], wreg[7], 2 * c, a0, b0);
                q4_k_coeffs(wreg[4], wreg[5], wreg[6], wreg[7], 2 * c + 1, a1, b1);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // columns 4i .. 4i + 3 of the 16: group i / 2 of the low and high halves
                    float* lo = ws + wlds[i >> 1] + 4 * (i & 1) * WP;
                    float* hi = ws + wlds[2 + (i >> 1)] + 4 * (i & 1) * WP;
                    float e[4];
                    q4_k_x4(wreg[i], false, a0, b0, e);
#pragma unroll
                    for (int j = 0; j < 4; ++j) lo[j * WP] = e[j];
                    q4_k_x4(wreg[i], true, a1, b1, e);
#pragma unroll
                    for (int j = 0; j < 4; ++j) hi[j * WP] = e[j];
                }
            } else if constexpr (TYPE == kQ5_K) {
                const int c = (p & 7) >> 1;
                float a0, b0, a1, b1;
                q4_k_coeffs(wreg[4], wreg[5], wreg[6], wreg[7], 2 * c, a0, b0);
                q4_k_coeffs(wreg[4], wreg[5], wreg[6], wreg[7], 2 * c + 1, a1, b1);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float* lo = ws + wlds[i >> 1] + 4 * (i & 1) * WP;
                    float* hi = ws + wlds[2 + (i >> 1)] + 4 * (i & 1) * WP;
                    float e[4];
                    q5_k_x4(wreg[i], wreg[8 + i], 2 * c, false, a0, b0, e);
#pragma unroll
                    for (int j = 0; j < 4; ++j) lo[j * WP] = e[j];
                    q5_k_x4(wreg[i], wreg[8 + i], 2 * c + 1, true, a1, b1, e);
#pragma unroll
                    for (int j = 0; j < 4; ++j) hi[j * WP] = e[j];
                }
            } else if constexpr (TYPE == kQ6_K) {
                const int j = p & 3;
                const float d = half_to_f32(wreg[8]);
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    const int si = (j >> 1) + 2 * qq;  // sub-scale 8hh + si
                    float a;
                    q6_k_coeffs(wreg[6 + (si >> 2)], si & 3, d, a);
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        float e[4];
                        q6_k_x4(wreg[2 * (qq & 1) + i], qq >= 2, wreg[4 + i], qq, a, e);
#pragma unroll
                        for (int t = 0; t < 4; ++t) ws[wlds[qq] + (4 * i + t) * WP] = e[t];
                    }
                }
            } else if constexpr (TYPE == kQ2_K || TYPE == kQ3_K) {
                const int hh = (p >> 2) & 1, j = p & 3;
                float d, dmin = 0.f;
                if constexpr (TYPE == kQ2_K) {
                    d = half_to_f32(wreg[4] & 0xFFFFu);
                    dmin = half_to_f32(wreg[4] >> 16);
                } else {
                    d = half_to_f32(wreg[7] & 0xFFFFu);
                }
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    const int si = (j >> 1) + 2 * qq;  // pair / sub-scale 8hh + si
                    float a, b = 0.f;
                    if constexpr (TYPE == kQ2_K)
                        q2_k_coeffs(wreg[2 + (si >> 2)], si & 3, d, dmin, a, b);
                    else
                        q3_k_coeffs(wreg[4], wreg[5], wreg[6], 8 * hh + si, d, a);
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        float e[4];
                        if constexpr (TYPE == kQ2_K)
                            q2_k_x4(wreg[i], qq, a, b, e);
                        else
                            q3_k_x4(wreg[i], wreg[2 + i], qq, 4 * hh + qq, a, e);
#pragma unroll
                        for (int t = 0; t < 4; ++t) ws[wlds[qq] + (4 * i + t) * WP] = e[t];
                    }
                }
            } else if constexpr (TYPE == kQ8_0) {
                constexpr int CW = S::CB / 4;
                const float d = half_to_f32(wreg[CW]);
#pragma unroll
                for (int w = 0; w < CW; ++w) {
                    float e[4];
                    q8_0_x4(wreg[w], d, e);
                    // columns CB s + 4w + j: group w / 2 of 8
                    float* col = ws + wlds[w >> 1] + 4 * (w & 1) * WP;
#pragma unroll
                    for (int j = 0; j < 4; ++j) col[j * WP] = e[j];
                }
            } else if constexpr (TYPE == kNVFP4) {
                // sub-block i: words 2i, 2i + 1 hold its 8 code bytes; low
                // nibbles are its columns 0 .. 7, high nibbles 8 .. 15
#pragma unroll
                for (int i = 0; i < S::NV_SB; ++i) {
                    const float sc = e4m3_to_f32((wreg[2 * S::NV_SB] >> (8 * i)) & 0xFFu);
#pragma unroll
                    for (int w = 0; w < 2; ++w) {
                        float el[4], eh[4];
                        nvfp4_x8(wreg[2 * i + w], sc, el, eh);
                        // each base's stores together, so that the compiler pairs
                        // them into two-address stores
#pragma unroll
                        for (int j = 0; j < 4; ++j) ws[wlds[2 * i] + (4 * w + j) * WP] = el[j];      // columns 0 .. 7
#pragma unroll
                        for (int j = 0; j < 4; ++j) ws[wlds[2 * i + 1] + (4 * w + j) * WP] = eh[j];  // columns 8 .. 15
                    }
                }
            } else if constexpr (TYPE == kMXFP4) {  // code bytes CB s .. of the block
                constexpr int CW = S::CB / 4;
                const float sc = mx_scale(wreg[CW]);
#pragma unroll
                for (int w = 0; w < CW; ++w) {
                    float el[4], eh[4];
                    mxfp4_x8(wreg[w], sc, el, eh);
                    // bytes 4w .. 4w + 3 of the thread's CB: group w / 2 of 8 in each half
#pragma unroll
                    for (int j = 0; j < 4; ++j) ws[wlds[w >> 1] + (4 * (w & 1) + j) * WP] = el[j];
#pragma unroll
                    for (int j = 0; j < 4; ++j) ws[wlds[2 + (w >> 1)] + (4 * (w & 1) + j) * WP] = eh[j];
                }
            } else {  // 32-element nibble blocks: code bytes CB s .. of the block
                constexpr int CW = S::CB / 4;
                float d, m;
                uint32_t qh;
                if constexpr (kHasFifth<TYPE>)
                    nibble32_header<TYPE>(wreg[CW], wreg[CW + 1], d, m, qh);
                else
                    nibble32_header<TYPE>(wreg[CW], 0u, d, m, qh);
                const int first = S::CB * (p % S::QSPLIT);
#pragma unroll
                for (int w = 0; w < CW; ++w) {
                    float e[4];
                    nibble32_x4<TYPE>(wreg[w], qh, first + 4 * w, d, m, e);
#pragma unroll
                    for (int j = 0; j < 4; ++j) ws[wlds[w >> 1] + (4 * (w & 1) + j) * WP] = e[j];
                    nibble32_x4<TYPE>(wreg[w], qh, 16 + first + 4 * w, d, m, e);
#pragma unroll
                    for (int j = 0; j < 4; ++j) ws[wlds[2 + (w >> 1)] + (4 * (w & 1) + j) * WP] = e[j];
                }
            }
        };

        // Chunk j is loaded into slot j % R and written to LDS buffer j % 2.
        // Prologue: start the loads of chunks 0 .. R - 1, fill buffer 0.
        using Zero = std::integral_constant<int, 0>;
        static_for<R>([&](auto i) { load_chunk(i, chunk_n0(i)); });
        store_chunk(Zero{}, Zero{}, chunk_n0(0));
        __syncthreads();
        // While the consumers contract chunk c: write chunk c + 1 to LDS, start
        // the loads of chunk c + R into the slot chunk c left, then the
        // barrier. Whole groups of R chunks run unguarded (a chunk past the end
        // is loaded and written but never read); the last partial group is
        // guarded per chunk.
        auto step = [&](auto i, int c) {
            constexpr int I = decltype(i)::value;
            store_chunk(std::integral_constant<int, (I + 1) % R>{}, std::integral_constant<int, (I + 1) & 1>{},
                        chunk_n0(c + 1));
            load_chunk(i, chunk_n0(c + R));
            __syncthreads();
        };
        int c0 = 0;
        for (; c0 + R <= nloc; c0 += R) static_for<R>([&](auto i) { step(i, c0 + decltype(i)::value); });
        static_for<R>([&](auto i) {
            if (c0 + decltype(i)::value < nloc) step(i, c0 + decltype(i)::value);
        });
        if constexpr (NG == 2) {  // the two barriers of the consumers' reduction
            __syncthreads();
            __syncthreads();
        }
        return;
    }

    // ---------------- consumer ----------------
    ws_consume<S, WA, WB, NG>(lds_all, tid, wave, nloc, t0, k0, T, K, args.dst, args.ldd);
}

}  // namespace retro
