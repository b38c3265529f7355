// retro_unit.hip - the kernels and launches of one weight type, chosen at
// compile time with -DRETRO_UNIT_TYPE=<GGUF type id>. The library links one
// such object per type; retro_api.hip validates arguments, picks the variant
// and calls the entry points declared in retro_host.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "retro_host.h"
#include "retro_kernels.h"
#include "retro_mm_kernel.h"
#include "retro_split_kernel.h"
#include "retro_ws_kernel.h"

#ifndef RETRO_UNIT_TYPE
#error "RETRO_UNIT_TYPE (a GGUF weight type id) must be defined"
#endif


namespace retro {
namespace host {

static_assert(kF32 == RETRO_F32 && kF16 == RETRO_F16 && kBF16 == RETRO_BF16 && kQ8_0 == RETRO_Q8_0 &&
                  kQ4_0 == RETRO_Q4_0 && kQ4_1 == RETRO_Q4_1 && kQ5_0 == RETRO_Q5_0 && kQ5_1 == RETRO_Q5_1 &&
                  kMXFP4 == RETRO_MXFP4 && kNVFP4 == RETRO_NVFP4 && kQ2_K == RETRO_Q2_K && kQ3_K == RETRO_Q3_K && kQ4_K == RETRO_Q4_K &&
                  kQ5_K == RETRO_Q5_K && kQ6_K == RETRO_Q6_K,
              "device and ABI type ids agree");

namespace {

BatchArgs batch_args(const Strides& s) {
    BatchArgs b;
    b.ne2 = int(s.ne2);
    b.r2 = int(s.ne2 / s.ne02);
    b.r3 = int(s.ne3 / s.ne03);
    b.w2 = s.sw2;
    b.w3 = s.sw3;
    b.g2 = s.sg2;
    b.g3 = s.sg3;
    b.d2 = s.sd2;
    b.d3 = s.sd3;
    return b;
}

template <int TYPE, int WA, int WB, int WGT, int WGK>
int launch_tile(const void* W, const float* G, float* dst, int64_t K, int64_t N, int64_t T, const Strides& s,
                hipStream_t st) {
    using S = TileShape<TYPE, WA, WB, WGT, WGK>;
    TileArgs a;
    a.W = static_cast<const uint8_t*>(W);
    a.G = G;
    a.dst = dst;
    a.K = int(K);
    a.N = int(N);
    a.T = int(T);
    a.pitch = s.ldw;
    a.ldg = s.ldg;
    a.ldd = s.ldd;
    // Widest staging load that the row pitch, the tile span and the row's
    // bytes are all multiples of (the base pointer is 16-byte aligned): then
    // no load straddles the end of W, where a buffer load reads zero for the
    // whole word.
    const int64_t rbytes = row_bytes_of(TYPE, K);
    int wvec = 16;
    while (wvec > 1 && ((a.pitch % wvec) != 0 || (S::SPAN % wvec) != 0 || (rbytes % wvec) != 0)) wvec >>= 1;
    a.wvec = wvec;
    a.gvec = (!s.gcols && s.ldg % 4 == 0) ? 1 : 0;
    a.gcols = s.gcols ? 1 : 0;
    a.tiles_t = int(cdiv(T, S::BT));
    a.tiles_k = int(cdiv(K, S::BK));
    a.group = group_height(a.tiles_t, a.tiles_k, 2, 4.0 * T * N, double(N) * rbytes);
    a.batch = batch_args(s);
    const unsigned nt = unsigned(a.tiles_t) * unsigned(a.tiles_k);
    clear_last_error();
    hipLaunchKernelGGL((out_prod_tile_kernel<TYPE, WA, WB, WGT, WGK>), dim3(nt, unsigned(s.batches())),
                       dim3(S::kThreads), 0, st, a);
    return launch_status();
}

template <int TYPE, int WA, int WB, int CT, int NG = 1, int NC = 4>
int launch_ws(const void* W, const float* G, float* dst, int64_t K, int64_t N, int64_t T, const Strides& s,
              hipStream_t st) {
    using S = WsShape<TYPE, WA, WB, CT, NG, NC>;
    TileArgs a;
    a.W = static_cast<const uint8_t*>(W);
    a.G = G;
    a.dst = dst;
    a.K = int(K);
    a.N = int(N);
    a.T = int(T);
    a.pitch = s.ldw;
    a.ldg = s.ldg;
    a.ldd = s.ldd;
    a.wvec = 16;
    a.gvec = 1;
    a.gcols = s.gcols ? 1 : 0;  // the kernel takes the layout as a template argument
    a.tiles_t = int(cdiv(T, S::BT));
    a.tiles_k = int(cdiv(K, S::BK));
    a.group = group_height(a.tiles_t, a.tiles_k, S::kResident, 4.0 * T * N, double(N) * row_bytes_of(TYPE, K));
    a.batch = batch_args(s);
    const unsigned nt = unsigned(a.tiles_t) * unsigned(a.tiles_k);
    clear_last_error();
    const dim3 grid(nt, unsigned(s.batches()));
    if (s.gcols)
        hipLaunchKernelGGL((out_prod_ws_kernel<TYPE, WA, WB, CT, NG, NC, true>), grid, dim3(S::kThreads), 0, st, a);
    else
        hipLaunchKernelGGL((out_prod_ws_kernel<TYPE, WA, WB, CT, NG, NC, false>), grid, dim3(S::kThreads), 0, st, a);
    return launch_status();
}

template <int TYPE>
int launch_split(const void* W, const float* G, float* dst, int64_t K, int64_t N, int64_t T, const Strides& s,
                 hipStream_t st) {
    using S = SplitShape<kSplitBK<TYPE>>;
    TileArgs a;
    a.W = static_cast<const uint8_t*>(W);
    a.G = G;
    a.dst = dst;
    a.K = int(K);
    a.N = int(N);
    a.T = int(T);
    a.pitch = s.ldw;
    a.ldg = s.ldg;
    a.ldd = s.ldd;
    a.wvec = 16;
    a.gvec = 1;
    a.gcols = 0;
    a.tiles_t = int(cdiv(T, S::BT));
    a.tiles_k = int(cdiv(K, S::BK));
    a.group = group_height(a.tiles_t, a.tiles_k, 1, 4.0 * T * N, double(N) * row_bytes_of(TYPE, K));
    a.batch = batch_args(s);
    const unsigned nt = unsigned(a.tiles_t) * unsigned(a.tiles_k);
    clear_last_error();
    hipLaunchKernelGGL((out_prod_split_kernel<TYPE>), dim3(nt, unsigned(s.batches())), dim3(S::kThreads), 0, st, a);
    return launch_status();
}

// Waves per skinny workgroup. Each CU runs one skinny workgroup (64 columns
// of dst over all of n), so this is the waves per SIMD, and 16 n rows per
// group go to the waves in turn. Measured on MI355X at N = 4096, K = 14336
// (interleaved in one process, 8 rounds of 40 launches): eight waves, each
// walking twice the groups, take 0.94-0.95x the time of sixteen at T = 16
// for Q4_0, Q4_1, Q5_0, MXFP4 and Q5_K, 0.96-0.98x for Q4_K, Q6_K, Q8_0,
// Q5_1, F16 and BF16, and the same for Q3_K and F32; at T = 8 and 4, 0.94-0.95x
// for Q4_0 and Q6_K and 0.98 for BF16. Sixteen stay faster for Q2_K and NVFP4
// (by 2-3%) and for Q4_K below T = 12 (1-4%). Above T = 16 the accumulators
// of the extra blocks of G take the registers of a 16-wave workgroup: eight.
int skinny_waves(int type, int64_t T) {
    if (T > 16) return 8;
    if (type == RETRO_Q2_K || type == RETRO_NVFP4) return 16;
    if (type == RETRO_Q4_K && T < 12) return 16;
    return 8;
}

template <int TYPE, int kWaves, int TB>
void launch_skinny_waves(const SkinnyArgs& a, dim3 grid, hipStream_t st) {
    const dim3 block(kWaves * 64);
    if (a.wide && a.gvec)
        hipLaunchKernelGGL((out_prod_skinny_kernel<TYPE, kWaves, true, TB>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((out_prod_skinny_kernel<TYPE, kWaves, false, TB>), grid, block, 0, st, a);
}

SkinnyArgs skinny_args(const void* W, const float* G, float* dst, int64_t K, int64_t N, int64_t T,
                       const Strides& s) {
    SkinnyArgs a;
    a.W = static_cast<const uint8_t*>(W);
    a.G = G;
    a.dst = dst;
    a.K = int(K);
    a.N = int(N);
    a.T = int(T);
    a.pitch = s.ldw;
    a.ldg = s.ldg;
    a.ldd = s.ldd;
    a.wide = (K % 4 == 0) ? 1 : 0;
    a.gvec = (s.gcols || s.ldg % 4 == 0) ? 1 : 0;
    a.gcols = s.gcols ? 1 : 0;
    a.batch = batch_args(s);
    return a;
}

// Offset of row t0 of G within each matrix: rows of ldg floats, or (G
// stored t-fastest) the t0-th float of every column.
int64_t g_row_offset(const Strides& s, int64_t t0) { return s.gcols ? t0 : t0 * s.ldg; }

// One pass over W per kSkinnyMaxT rows of G (the last pass takes the rest).
template <int TYPE>
int launch_skinny(const void* W, const float* G, float* dst, int64_t K, int64_t N, int64_t T, const Strides& s,
                  int waves, hipStream_t st) {
    const dim3 grid(unsigned(cdiv(K, 64)), unsigned(s.batches()));
    for (int64_t t0 = 0; t0 < T; t0 += kSkinnyMaxT) {
        const int64_t tc = T - t0 < kSkinnyMaxT ? T - t0 : kSkinnyMaxT;
        const SkinnyArgs a = skinny_args(W, G + g_row_offset(s, t0), dst + t0 * s.ldd, K, N, tc, s);
        clear_last_error();
        switch (skinny_blocks(tc)) {
            case 1:
                if (waves == 8)
                    launch_skinny_waves<TYPE, 8, 1>(a, grid, st);
                else
                    launch_skinny_waves<TYPE, 16, 1>(a, grid, st);
                break;
            case 2: launch_skinny_waves<TYPE, 8, 2>(a, grid, st); break;
            case 3: launch_skinny_waves<TYPE, 8, 3>(a, grid, st); break;
            default: launch_skinny_waves<TYPE, 8, 4>(a, grid, st); break;
        }
        const int rc = launch_status();
        if (rc != RETRO_OK) return rc;
    }
    return RETRO_OK;
}

template <int TYPE, int WA, int WB, int CT, int NC = 4>
int launch_mm(const void* W, const float* X, float* Y, int64_t K, int64_t N, int64_t T, int64_t ldy,
              hipStream_t st) {
    using S = MmShape<TYPE, WA, WB, CT, NC>;
    MmArgs a;
    a.W = static_cast<const uint8_t*>(W);
    a.X = X;
    a.Y = Y;
    a.K = int(K);
    a.N = int(N);
    a.T = int(T);
    a.pitch = row_bytes_of(TYPE, K);
    a.ldx = K;
    a.ldy = ldy;
    a.tiles_t = int(cdiv(T, S::BT));
    a.tiles_n = int(cdiv(N, S::BK));
    a.group = group_height(a.tiles_t, a.tiles_n, S::kResident, 4.0 * T * K, double(N) * a.pitch);
    const unsigned nt = unsigned(a.tiles_t) * unsigned(a.tiles_n);
    clear_last_error();
    hipLaunchKernelGGL((mul_mat_ws_kernel<TYPE, WA, WB, CT, NC>), dim3(nt), dim3(S::kThreads), 0, st, a);
    return launch_status();
}

MmSimpleArgs mm_simple_args(int type, const void* W, const float* X, float* Y, int64_t K, int64_t N, int64_t T,
                            int64_t ldy) {
    MmSimpleArgs a;
    a.W = static_cast<const uint8_t*>(W);
    a.X = X;
    a.Y = Y;
    a.K = int(K);
    a.N = int(N);
    a.T = int(T);
    a.pitch = row_bytes_of(type, K);
    a.ldx = K;
    a.ldy = ldy;
    a.wide = (K % 4 == 0) ? 1 : 0;
    return a;
}

}  // namespace

template <int TYPE>
int launch_out_prod(int variant, const void* W, const float* G, float* dst, int64_t K, int64_t N, int64_t T,
                    const Strides& s, hipStream_t st) {
    switch (variant) {
        case RETRO_VARIANT_SKINNY: return launch_skinny<TYPE>(W, G, dst, K, N, T, s, skinny_waves(TYPE, T), st);
        case RETRO_VARIANT_SKINNY_8: return launch_skinny<TYPE>(W, G, dst, K, N, T, s, 8, st);
        case RETRO_VARIANT_SKINNY_16: return launch_skinny<TYPE>(W, G, dst, K, N, T, s, 16, st);
        case RETRO_VARIANT_TILE_128x256: return launch_tile<TYPE, 2, 4, 2, 2>(W, G, dst, K, N, T, s, st);
        case RETRO_VARIANT_TILE_64x256: return launch_tile<TYPE, 1, 4, 2, 2>(W, G, dst, K, N, T, s, st);
        case RETRO_VARIANT_WS_256x256: return launch_ws<TYPE, 4, 2, 2, 1, 8>(W, G, dst, K, N, T, s, st);
        case RETRO_VARIANT_WS_128x256: return launch_ws<TYPE, 2, 4, 2>(W, G, dst, K, N, T, s, st);
        case RETRO_VARIANT_WS_64x256: return launch_ws<TYPE, 1, 4, 2>(W, G, dst, K, N, T, s, st);
        case RETRO_VARIANT_WS_32x256: return launch_ws<TYPE, 1, 2, 1>(W, G, dst, K, N, T, s, st);
        default: break;
    }
    if constexpr (kSuperBlock<TYPE>)
        if (variant == RETRO_VARIANT_SPLIT_128x256) return launch_split<TYPE>(W, G, dst, K, N, T, s, st);
    if constexpr (kSplitNarrow<TYPE>)
        if (variant == RETRO_VARIANT_SPLIT_128x128) return launch_split<TYPE>(W, G, dst, K, N, T, s, st);
    if constexpr (!kSuperBlock<TYPE>) {
        switch (variant) {
            case RETRO_VARIANT_TILE_128x128: return launch_tile<TYPE, 2, 2, 2, 2>(W, G, dst, K, N, T, s, st);
            case RETRO_VARIANT_TILE_64x128: return launch_tile<TYPE, 1, 2, 2, 2>(W, G, dst, K, N, T, s, st);
            case RETRO_VARIANT_TILE_64x64: return launch_tile<TYPE, 1, 1, 2, 2>(W, G, dst, K, N, T, s, st);
            case RETRO_VARIANT_WS_128x128: return launch_ws<TYPE, 2, 2, 2>(W, G, dst, K, N, T, s, st);
            case RETRO_VARIANT_WS_64x128: return launch_ws<TYPE, 1, 2, 2>(W, G, dst, K, N, T, s, st);
            case RETRO_VARIANT_WS2_64x128: return launch_ws<TYPE, 1, 2, 2, 2>(W, G, dst, K, N, T, s, st);
            case RETRO_VARIANT_WS_32x128: return launch_ws<TYPE, 1, 1, 1>(W, G, dst, K, N, T, s, st);
            default: break;
        }
    }
    return RETRO_E_VARIANT;
}

template <int TYPE>
int launch_mul_mat(int variant, const void* W, const float* X, float* Y, int64_t K, int64_t N, int64_t T,
                   int64_t ldy, hipStream_t st) {
    switch (variant) {
        case RETRO_VARIANT_WS_256x128: return launch_mm<TYPE, 2, 2, 4, 8>(W, X, Y, K, N, T, ldy, st);
        case RETRO_VARIANT_WS_128x128: return launch_mm<TYPE, 2, 2, 2>(W, X, Y, K, N, T, ldy, st);
        case RETRO_VARIANT_WS_64x128: return launch_mm<TYPE, 1, 2, 2>(W, X, Y, K, N, T, ldy, st);
        case RETRO_VARIANT_WS_32x128: return launch_mm<TYPE, 1, 1, 1>(W, X, Y, K, N, T, ldy, st);
        case RETRO_VARIANT_SIMPLE: {
            const MmSimpleArgs a = mm_simple_args(TYPE, W, X, Y, K, N, T, ldy);
            clear_last_error();
            hipLaunchKernelGGL((mul_mat_simple_kernel<TYPE>), dim3(unsigned(cdiv(T * N, 256))), dim3(256), 0, st,
                               a);
            return launch_status();
        }
        case RETRO_VARIANT_SKINNY: {
            // one pass over W per 64 rows of x and Y
            const dim3 grid(unsigned(cdiv(N, 16)));
            for (int64_t t0 = 0; t0 < T; t0 += kSkinnyMaxT) {
                const int64_t tc = T - t0 < kSkinnyMaxT ? T - t0 : kSkinnyMaxT;
                const MmSimpleArgs a = mm_simple_args(TYPE, W, X + t0 * K, Y + t0 * ldy, K, N, tc, ldy);
                clear_last_error();
                // the out_prod skinny kernel's wave rule; measured on the forward at
                // T = 16: eight waves 0.96-0.98x the time of sixteen for Q4_K, Q6_K,
                // Q4_0 and Q8_0 at N = 4096, K = 14336 (0.83x at N = 14336, K =
                // 4096), 1.007x for Q2_K, 1.025x for Q4_K at T = 4
                switch (skinny_blocks(tc)) {
                    case 1:
                        if (skinny_waves(TYPE, tc) == 8)
                            hipLaunchKernelGGL((mul_mat_skinny_kernel<TYPE, 8, 1>), grid, dim3(512), 0, st, a);
                        else
                            hipLaunchKernelGGL((mul_mat_skinny_kernel<TYPE, 16, 1>), grid, dim3(1024), 0, st, a);
                        break;
                    case 2: hipLaunchKernelGGL((mul_mat_skinny_kernel<TYPE, 8, 2>), grid, dim3(512), 0, st, a); break;
                    case 3: hipLaunchKernelGGL((mul_mat_skinny_kernel<TYPE, 8, 3>), grid, dim3(512), 0, st, a); break;
                    default: hipLaunchKernelGGL((mul_mat_skinny_kernel<TYPE, 8, 4>), grid, dim3(512), 0, st, a); break;
                }
                const int rc = launch_status();
                if (rc != RETRO_OK) return rc;
            }
            return RETRO_OK;
        }
        default: return RETRO_E_VARIANT;
    }
}

template <int TYPE>
int launch_dequant(const void* W, float* out, int64_t K, int64_t N, hipStream_t st) {
    DequantArgs a;
    a.W = static_cast<const uint8_t*>(W);
    a.out = out;
    a.K = int(K);
    a.N = int(N);
    a.pitch = row_bytes_of(TYPE, K);
    a.wide = (K % 4 == 0) ? 1 : 0;
    a.gpr = int(cdiv(K, 4));
    a.groups = N * int64_t(a.gpr);
    clear_last_error();
    hipLaunchKernelGGL((dequant_kernel<TYPE>), dim3(unsigned(cdiv(a.groups, 256))), dim3(256), 0, st, a);
    return launch_status();
}

template <int TYPE>
int launch_out_prod_split(const void* W, const float* G, float* dst, int64_t K, int64_t N, int64_t T,
                          const Strides& s, void* workspace, hipStream_t st) {
    // one pass over W per kSplitMaxT rows of G, in turn on the stream (each
    // leaves the workspace's counters at zero for the next)
    if (T > kSplitMaxT) {
        for (int64_t t0 = 0; t0 < T; t0 += kSplitMaxT) {
            const int64_t tc = T - t0 < kSplitMaxT ? T - t0 : kSplitMaxT;
            const int rc = launch_out_prod_split<TYPE>(W, G + g_row_offset(s, t0), dst + t0 * s.ldd, K, N, tc, s,
                                                       workspace, st);
            if (rc != RETRO_OK) return rc;
        }
        return RETRO_OK;
    }
    const SkinnyArgs a = skinny_args(W, G, dst, K, N, T, s);
    SkinnySplitArgs sp;
    sp.count = static_cast<unsigned*>(workspace);
    sp.slots = reinterpret_cast<float*>(static_cast<char*>(workspace) + kSplitCountBytes);
    sp.ng = int(N / 16);
    sp.share = cdiv(cdiv(K, 64) * (N / 16), kSplitGrid);
    clear_last_error();
    const dim3 grid(kSplitGrid), b8(512), b16(1024);
    switch (skinny_blocks(T)) {
        case 1:
            if (skinny_waves(TYPE, T) == 8)
                hipLaunchKernelGGL((out_prod_skinny_split_kernel<TYPE, 8, 1>), grid, b8, 0, st, a, sp);
            else
                hipLaunchKernelGGL((out_prod_skinny_split_kernel<TYPE, 16, 1>), grid, b16, 0, st, a, sp);
            break;
        case 2: hipLaunchKernelGGL((out_prod_skinny_split_kernel<TYPE, 8, 2>), grid, b8, 0, st, a, sp); break;
        case 3: hipLaunchKernelGGL((out_prod_skinny_split_kernel<TYPE, 8, 3>), grid, b8, 0, st, a, sp); break;
        default: return RETRO_E_VARIANT;  // not reached: T <= kSplitMaxT here
    }
    return launch_status();
}

template int launch_out_prod<RETRO_UNIT_TYPE>(int, const void*, const float*, float*, int64_t, int64_t, int64_t,
                                              const Strides&, hipStream_t);
template int launch_out_prod_split<RETRO_UNIT_TYPE>(const void*, const float*, float*, int64_t, int64_t, int64_t,
                                                    const Strides&, void*, hipStream_t);
template int launch_mul_mat<RETRO_UNIT_TYPE>(int, const void*, const float*, float*, int64_t, int64_t, int64_t, int64_t,
                                             hipStream_t);
template int launch_dequant<RETRO_UNIT_TYPE>(const void*, float*, int64_t, int64_t, hipStream_t);

}  // namespace host
}  // namespace retro

