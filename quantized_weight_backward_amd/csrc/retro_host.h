// retro_host.h - host-side pieces shared by the C ABI (retro_api.hip) and the
// per-type launch units (retro_unit.hip): block geometry, size limits, the
// operand layout, the tile-order heuristic and the launch entry points each
// unit defines for its one weight type. No device code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "retro_out_prod.h"

namespace retro {
namespace host {

constexpr int kNumCUs = 256;  // MI355X
constexpr int64_t kDimLimit = int64_t(1) << 31;
constexpr int64_t kByteLimit = int64_t(1) << 62;
constexpr int64_t kCountLimit = int64_t(1) << 60;  // float counts: 4 * count < 2^62
constexpr int64_t kGridLimit = int64_t(1) << 30;
constexpr int64_t kBatchLimit = 65535;  // workgroups along the grid's second dimension

struct Geometry {
    int block, bytes;
};

inline bool geometry(int type, Geometry& g) {
    switch (type) {
        case RETRO_F32: g = {1, 4}; return true;
        case RETRO_F16: g = {1, 2}; return true;
        case RETRO_BF16: g = {1, 2}; return true;
        case RETRO_Q8_0: g = {32, 34}; return true;
        case RETRO_Q4_0: g = {32, 18}; return true;
        case RETRO_Q4_1: g = {32, 20}; return true;
        case RETRO_Q5_0: g = {32, 22}; return true;
        case RETRO_Q5_1: g = {32, 24}; return true;
        case RETRO_MXFP4: g = {32, 17}; return true;
        case RETRO_NVFP4: g = {64, 36}; return true;
        case RETRO_Q4_K: g = {256, 144}; return true;
        case RETRO_Q5_K: g = {256, 176}; return true;
        case RETRO_Q2_K: g = {256, 84}; return true;
        case RETRO_Q3_K: g = {256, 110}; return true;
        case RETRO_Q6_K: g = {256, 210}; return true;
        default: return false;
    }
}

inline int64_t row_bytes_of(int type, int64_t K) {
    Geometry g;
    if (!geometry(type, g) || K < 0 || K % g.block) return -1;
    return K / g.block * g.bytes;
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Layout of the three operands: row strides, and the batches over two outer
// dimensions (ne2 x ne3 products; W has ne02 x ne03 matrices, each serving
// ne2 / ne02 x ne3 / ne03 consecutive batches).
struct Strides {
    int64_t ldw;  // bytes between consecutive W rows (>= the row's bytes)
    int64_t ldg;  // G[t][n] at float t * ldg + n (ldg >= N), or n * ldg + t when gcols (ldg >= T)
    int64_t ldd;  // floats between consecutive dst rows (>= K)
    bool gcols = false;  // G stored t-fastest: its columns are contiguous
    int64_t ne02 = 1, ne03 = 1, ne2 = 1, ne3 = 1;
    int64_t sw2 = 0, sw3 = 0;  // bytes between W matrices
    int64_t sg2 = 0, sg3 = 0;  // floats between G matrices
    int64_t sd2 = 0, sd3 = 0;  // floats between dst matrices
    int64_t batches() const { return ne2 * ne3; }
};

// Row tiles per group of the tile order. An XCD runs S = 32 CUs x wg_per_cu
// tiles at once, `height` row tiles by S / height column tiles of its range,
// so G is fetched about ceil(tiles_k / (S / height)) times and W about
// ceil(tiles_t / height) times; the height that minimises the sum wins.
inline int group_height(int64_t tiles_t, int64_t tiles_k, int wg_per_cu, double g_bytes, double w_bytes) {
    const int64_t S = 32 * int64_t(wg_per_cu);
    int best = 1;
    double best_cost = -1;
    for (int64_t h = 1; h <= S; h *= 2) {
        const double cost = g_bytes * double(cdiv(tiles_k, S / h)) + w_bytes * double(cdiv(tiles_t, h));
        if (best_cost < 0 || cost < best_cost) {
            best = int(h);
            best_cost = cost;
        }
        if (h >= tiles_t) break;
    }
    return best;
}

// hipGetLastError reports the last error of any runtime call on this thread,
// so it is cleared right before each launch (clear_last_error) and read right
// after it (launch_status): the result is this launch's status only.
inline void clear_last_error() { (void)hipGetLastError(); }
inline int launch_status() { return hipGetLastError() == hipSuccess ? RETRO_OK : RETRO_E_HIP; }

// Launches for one weight type, defined in retro_unit.hip (one object per
// type, built in parallel). Arguments are validated by the caller and the
// variant is one that applies.
template <int TYPE>
int launch_out_prod(int variant, const void* W, const float* G, float* dst, int64_t K, int64_t N, int64_t T,
                    const Strides& s, hipStream_t st);
// Y's rows are ldy floats apart (ldy >= N: a column range of a wider Y).
template <int TYPE>
int launch_mul_mat(int variant, const void* W, const float* X, float* Y, int64_t K, int64_t N, int64_t T,
                   int64_t ldy, hipStream_t st);
// The skinny kernels take T up to 64, in blocks of 16 rows of G.
constexpr int64_t kSkinnyMaxT = 64;
inline int skinny_blocks(int64_t T) { return int(cdiv(T, 16)); }

// The n-split skinny kernel's workspace: a counter word per workgroup
// (kSplitCountBytes in all), then two slots of 16 x 64 floats per block of
// 16 rows of G per workgroup. The counters must be zero before a call and
// are zero after it; the slots need no initial value. Its grid is one
// workgroup per CU.
constexpr int kSplitGrid = kNumCUs;
constexpr int64_t kSplitCountBytes = 4 * kSplitGrid;
constexpr int64_t kSplitSlotBytes = 16 * 64 * 4;  // per block of 16 rows of G
constexpr int64_t split_workspace_bytes(int blocks) {
    return kSplitCountBytes + 2 * kSplitGrid * kSplitSlotBytes * blocks;
}
// The n-split form takes T up to 48: at 64 its state would not fit the 256
// registers of a wave without spilling.
constexpr int64_t kSplitMaxT = 48;
constexpr int64_t kSplitWorkspaceMax = split_workspace_bytes(int(kSplitMaxT / 16));
static_assert(kSplitCountBytes % 256 == 0, "slots start 256-byte aligned");

// One launch of the n-split skinny kernel (one matrix; applicability checked
// by the caller), with a workspace of split_workspace_bytes(skinny_blocks(T)).
template <int TYPE>
int launch_out_prod_split(const void* W, const float* G, float* dst, int64_t K, int64_t N, int64_t T,
                          const Strides& s, void* workspace, hipStream_t st);
template <int TYPE>
int launch_dequant(const void* W, float* out, int64_t K, int64_t N, hipStream_t st);

}  // namespace host
}  // namespace retro
