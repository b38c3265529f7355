// retro_api.hip - the C ABI declared in include/retro_out_prod.h: argument
// validation and kernel choice. Host code only: the launches of each weight
// type are in its own object built from retro_unit.hip.
//
// The entry points follow the OUT_PROD admission rule of llama.cpp PR #3
// ("cuda: out_prod accepts a quantized src0", section "What": any contiguous
// src0 with an F32 converter, src1 and dst F32), but where that PR
// dequantizes into a pool copy and calls an F32 GEMM, every call here is one
// fused kernel with no allocation, and an unsupported call is an error, never
// a CPU fallback.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "retro_host.h"
#include "retro_out_prod.h"

// The workspace of retro_out_prod_noalloc, for callers that cannot allocate:
// one copy on every GPU the library runs on, held until the process ends,
// zero at load (the split kernel's counters must start at zero, and every
// call leaves them so). In host code `scratch` names a host-side stand-in,
// not device memory: kernels get the address hipGetSymbolAddress returns for
// the current device, never the name itself.
static __device__ __align__(256) unsigned char scratch[retro::host::kSplitWorkspaceMax];

namespace {

using namespace retro::host;

// a * b < limit for non-negative a, b.
bool product_below(int64_t a, int64_t b, int64_t limit) { return a == 0 || b < limit / a; }

int check_shape(int type, int64_t K, int64_t N, int64_t T) {
    Geometry g;
    if (!geometry(type, g)) return RETRO_E_TYPE;
    if (K < 0 || N < 0 || T < 0) return RETRO_E_SHAPE;
    if (K % g.block) return RETRO_E_SHAPE;
    if (K >= kDimLimit || N >= kDimLimit || T >= kDimLimit) return RETRO_E_SHAPE;
    const int64_t pitch = K / g.block * g.bytes;
    if (!product_below(T, K, kCountLimit) || !product_below(T, N, kCountLimit) ||
        !product_below(N, pitch, kByteLimit))
        return RETRO_E_SHAPE;
    return RETRO_OK;
}

Strides contiguous(int type, int64_t K, int64_t N) { return {row_bytes_of(type, K), N, K}; }

// Strides no shorter than the rows, and spans within the size limits (the
// shape itself already checked).
// Alignment of a block within a contiguous row: the largest power of two
// (at most 16) that divides the block's bytes. The kernels' loads assume it.
int64_t block_alignment(int type) {
    Geometry g;
    if (!geometry(type, g)) return 1;
    int64_t a = 1;
    while (a < 16 && g.bytes % (2 * a) == 0) a *= 2;
    return a;
}

int check_strides(int type, int64_t K, int64_t N, int64_t T, const Strides& s) {
    // G rows (or, stored t-fastest, columns) no shorter than they are long
    const int64_t g_len = s.gcols ? T : N, g_count = s.gcols ? N : T;
    if (s.ldw < row_bytes_of(type, K) || s.ldg < g_len || s.ldd < K) return RETRO_E_SHAPE;
    if (!product_below(N, s.ldw, kByteLimit) || !product_below(g_count, s.ldg, kCountLimit) ||
        !product_below(T, s.ldd, kCountLimit))
        return RETRO_E_SHAPE;
    // every row starts as aligned as a block of a contiguous row
    if (s.ldw % block_alignment(type)) return RETRO_E_ALIGN;
    // batches: W's counts divide the others', strides non-negative, spans
    // within the limits, every matrix starting as aligned as a single one
    if (s.ne02 < 1 || s.ne03 < 1 || s.ne2 < 0 || s.ne3 < 0 || s.ne2 % s.ne02 || s.ne3 % s.ne03)
        return RETRO_E_SHAPE;
    if (s.ne2 > kBatchLimit || s.ne3 > kBatchLimit || s.batches() > kBatchLimit) return RETRO_E_SHAPE;
    const int64_t st[6] = {s.sw2, s.sw3, s.sg2, s.sg3, s.sd2, s.sd3};
    for (int64_t v : st)
        if (v < 0 || v >= kCountLimit / kBatchLimit) return RETRO_E_SHAPE;
    if (s.sw2 % 16 || s.sw3 % 16 || s.sg2 % 4 || s.sg3 % 4 || s.sd2 % 4 || s.sd3 % 4) return RETRO_E_ALIGN;
    return RETRO_OK;
}

struct TileVariant {
    int id, bt, bk;
    double penalty;  // relative cost per output of the smaller tiles
    bool ws;         // producer/consumer kernel (else the single-role tile kernel)
};

constexpr TileVariant kTiles[] = {
    {RETRO_VARIANT_TILE_128x256, 128, 256, 1.00, false},
    {RETRO_VARIANT_TILE_128x128, 128, 128, 1.00, false},
    {RETRO_VARIANT_TILE_64x256, 64, 256, 1.05, false},
    {RETRO_VARIANT_TILE_64x128, 64, 128, 1.08, false},
    {RETRO_VARIANT_TILE_64x64, 64, 64, 1.20, false},
    {RETRO_VARIANT_WS_128x256, 128, 256, 1.00, true},
    // eight MFMA waves share the producers' decode: 0.88 against 0.84 of the
    // F32 peak for 128 x 256 at Q4_K 14336 x 4096, T = 4096 (equal rounds)
    {RETRO_VARIANT_WS_256x256, 256, 256, 0.95, true},
    {RETRO_VARIANT_WS_64x256, 64, 256, 1.04, true},
    {RETRO_VARIANT_WS_128x128, 128, 128, 1.00, true},
    {RETRO_VARIANT_WS_64x128, 64, 128, 1.02, true},
    {RETRO_VARIANT_WS_32x256, 32, 256, 1.06, true},
    {RETRO_VARIANT_WS_32x128, 32, 128, 1.04, true},
    // taken only through the rule at the end of choose()
    {RETRO_VARIANT_WS2_64x128, 64, 128, 1.50, true},
};

bool is_dense(int type) { return type == RETRO_F32 || type == RETRO_F16 || type == RETRO_BF16; }

// The producer/consumer kernel measures faster than the single-role kernel
// for every type on MI355X (Q4_K 0.84 vs 0.74 of the F32 peak at T = 4096,
// Q4_0 0.76 vs 0.66, Q8_0 0.73 vs 0.67, dense T = 512 0.61-0.68 vs 0.50),
// so it is preferred; the single-role kernel is the fallback for the shapes
// it does not take (G rows not in 16-byte units, or a dense K % 4 != 0).
bool prefers_ws(int) { return true; }
constexpr double kOtherFamily = 1.3;


const TileVariant* find_tile(int variant) {
    for (const auto& v : kTiles)
        if (v.id == variant) return &v;
    return nullptr;
}

// The tiled kernel addresses a tile's BT rows of G (with G stored t-fastest:
// a chunk's 32 columns) and a chunk's 32 rows of W with 32-bit offsets from
// per-chunk buffer bases.
bool tile_applies(const TileVariant& v, int type, int64_t K, int64_t N, int64_t T, const Strides& s) {
    Geometry geo;
    if (geometry(type, geo) && geo.block == 256 && v.bk % 256) return false;
    // the producer/consumer kernel loads G rows in 16-byte units and dense W
    // rows in 4-element units
    if (v.ws && (s.ldg % 4 || (is_dense(type) && K % 4))) return false;
    // chunk offsets run up to a few hundred rows past N in 32-bit arithmetic
    if (N >= kDimLimit - 4096) return false;
    const int64_t g_span = s.gcols ? 32 * s.ldg + v.bt : int64_t(v.bt) * s.ldg;
    return cdiv(T, v.bt) * cdiv(K, v.bk) < kGridLimit && g_span * 4 < (int64_t(1) << 31) &&
           33 * s.ldw < (int64_t(1) << 31);
}

// The skinny kernel runs one pass over W per 64 rows of G. A pass addresses
// one 16-row group of W, and the rows of G it reads (16 columns, when G is
// stored t-fastest: at most 16 ldg floats), through buffer descriptors whose
// sizes are signed 32-bit.
bool skinny_applies(int type, int64_t K, int64_t N, int64_t T, const Strides& s) {
    (void)type;
    (void)N;
    const int64_t tp = T < kSkinnyMaxT ? T : kSkinnyMaxT;  // rows of G per pass
    const int64_t g_span = s.gcols ? 16 * s.ldg + tp : (tp > 16 ? tp : 16) * s.ldg + 16;
    return cdiv(K, 64) < kGridLimit && 16 * s.ldw < (int64_t(1) << 31) && g_span * 4 < (int64_t(1) << 31);
}

// Estimated time (us) of the skinny kernel: per 16-row group and wave, 512
// cycles of MFMA per block of 16 rows of G plus about 300 of decode and
// waits, two waves per SIMD taking turns, one workgroup per CU per round,
// and about 4 us of launch and reduction plus 1.5 us per further block
// (fitted to Q4_K at N = 4096, K = 14336: 26.6, 44, 59 and 73 us for one to
// four blocks).
double skinny_pass_us(int64_t K, int64_t N, int64_t T, int64_t batches) {
    const double rounds = double(cdiv(cdiv(K, 64) * batches, kNumCUs)), per_wave = double(cdiv(cdiv(N, 16), 8));
    const double blocks = double(skinny_blocks(T));
    return 4.0 + 1.5 * (blocks - 1.0) + rounds * per_wave * 2.0 * (512.0 * blocks + 300.0) / 2400.0;
}

// Time of passes over rows of G, `per` rows a pass, the last one the rest.
template <typename Pass>
double passes_us(int64_t T, int64_t per, Pass pass) {
    const int64_t full = T / per, rest = T % per;
    return double(full) * pass(per) + (rest ? pass(rest) : 0.0);
}

double skinny_estimate_us(int64_t K, int64_t N, int64_t T, int64_t batches = 1) {
    return passes_us(T, kSkinnyMaxT, [&](int64_t t) { return skinny_pass_us(K, N, t, batches); });
}

// The n-split skinny kernel: the skinny kernel's fast path (whole 16-row
// groups, K in 4-element units, G rows in 16-byte units) over one matrix, in
// passes of up to 48 rows of G.
bool skinny_split_applies(int type, int64_t K, int64_t N, int64_t T, const Strides& s) {
    return skinny_applies(type, K, N, T, s) && T >= 1 && N >= 16 && N % 16 == 0 && K % 4 == 0 &&
           (s.gcols || s.ldg % 4 == 0) && s.batches() == 1;
}

// Estimated time (us) of the n-split skinny kernel: the skinny kernel's rate
// over one share per CU, plus about 5.6 us of launch, a second piece and the
// finishing sums (fitted to Q4_K at T = 16, K = 2048 .. 16384), and 1.5 us
// per further block of 16 rows of G.
double skinny_split_estimate_us(int64_t K, int64_t N, int64_t T) {
    const int64_t share = cdiv(cdiv(K, 64) * (N / 16), kSplitGrid);
    return passes_us(T, kSplitMaxT, [&](int64_t t) {
        const double blocks = double(skinny_blocks(t));
        return 5.6 + 1.5 * (blocks - 1.0) + double(cdiv(share, 8)) * 2.0 * (512.0 * blocks + 300.0) / 2400.0;
    });
}

// Whether the automatic choice may take tile v for this type. F32 rows spill
// registers in the 256 x 256 tile (their producers stage 16 bytes per
// element group): measured 0.99-1.04x the time of 128 x 256, where every
// other type gains 3-5%.
bool auto_takes(const TileVariant& v, int type) {
    return !(v.id == RETRO_VARIANT_WS_256x256 && type == RETRO_F32);
}

// Estimated cost of covering dst with tile v: (tiles per CU, rounded up) x
// tile area x relative cost. The rounding is the wave quantisation over 256
// CUs.
double tile_cost(const TileVariant& v, int type, int64_t K, int64_t T, const Strides& s) {
    const double weight = v.penalty * (v.ws == prefers_ws(type) ? 1.0 : kOtherFamily);
    const int64_t nt = cdiv(T, v.bt) * cdiv(K, v.bk) * s.batches();
    return double(cdiv(nt, kNumCUs)) * v.bt * v.bk * weight;
}

struct Choice {
    int id;       // variant, or RETRO_E_SHAPE when no tile applies
    double cost;  // tile_cost of the tile it was chosen by
};

// The tiled kernel of least cost (T > 16).
Choice choose_tile(int type, int64_t K, int64_t N, int64_t T, const Strides& s) {
    Choice best{-1, 0.0};
    for (const auto& v : kTiles) {
        if (!tile_applies(v, type, K, N, T, s) || !auto_takes(v, type)) continue;
        const double cost = tile_cost(v, type, K, T, s);
        if (best.id < 0 || cost < best.cost) best = {v.id, cost};
    }
    // 64 x 128 tiles in two pipelines per workgroup beat one pipeline per
    // workgroup when a CU gets at most one tile (one pipeline then leaves a
    // single MFMA wave per SIMD), and for F32 rows at any tile count
    // (measured: 0.64-0.70 vs 0.58-0.65 of the F32 peak at one tile per CU;
    // 0.75 vs 0.71 for F32 with several).
    if (best.id == RETRO_VARIANT_WS_64x128 &&
        (type == RETRO_F32 || cdiv(T, 64) * cdiv(K, 128) * s.batches() <= kNumCUs))
        best.id = RETRO_VARIANT_WS2_64x128;
    if (best.id < 0) best.id = RETRO_E_SHAPE;
    return best;
}

// Estimated time (us) of tile v over dst: rounds of one tile per CU, each
// tile a loop over 32-row chunks of W at 128 F32 MACs per cycle per CU, at
// the efficiency measured for the tile's rows of G with one tile per CU
// (Q4_K N = 4096, K = 14336 and F32 4096 x 4096: 32-row tiles 0.6, 64-row
// 0.72, larger 0.85).
double tile_estimate_us(int variant, int64_t K, int64_t N, int64_t T, const Strides& s) {
    const TileVariant* v = find_tile(variant);
    if (!v) return 1e30;
    const double rounds = double(cdiv(cdiv(T, v->bt) * cdiv(K, v->bk) * s.batches(), kNumCUs));
    const double eff = v->bt <= 32 ? 0.6 : v->bt <= 64 ? 0.72 : 0.85;
    return 4.0 + rounds * double(cdiv(N, 32)) * double(v->bt) * v->bk * 32.0 / 128.0 / eff / 2400.0;
}

// The kernel one launch over all of dst would use: the skinny kernel for
// T <= 16, and above that where its estimate (one pass over W per 64 rows of
// G) beats the best tile's (with few tiles per CU the tiled kernels leave
// most CUs idle: Q4_K N = 4096, K = 14336 at T = 17 .. 64 ran 183 us in
// 32 x 256 tiles).
int choose(int type, int64_t K, int64_t N, int64_t T, const Strides& s) {
    const bool skinny = skinny_applies(type, K, N, T, s);
    if (skinny && T <= 16) return RETRO_VARIANT_SKINNY;
    const Choice tile = choose_tile(type, K, N, T, s);
    // past one pass (T > 64) the skinny kernel must win by 10%: the
    // estimates are rougher there
    const double margin = T <= kSkinnyMaxT ? 1.0 : 0.9;
    if (skinny && (tile.id < 0 || skinny_estimate_us(K, N, T, s.batches()) <
                                      margin * tile_estimate_us(tile.id, K, N, T, s)))
        return RETRO_VARIANT_SKINNY;
    return tile.id;
}

// Whether the workspace calls take the split: an estimated gain of 10% or
// more over what retro_out_prod runs, and at most 192 slabs. From 224 slabs
// on (Q4_K, K = 14336) the split measured 1.04-1.24x the skinny kernel's
// time: it reads W without the L2 sharing that the skinny kernel's
// side-by-side slabs get.
bool skinny_split_pays(int type, int64_t K, int64_t N, int64_t T, const Strides& s) {
    if (cdiv(K, 64) > 192) return false;
    const int v = choose(type, K, N, T, s);
    const double one = v == RETRO_VARIANT_SKINNY ? skinny_estimate_us(K, N, T, s.batches())
                                                 : tile_estimate_us(v, K, N, T, s);
    return skinny_split_estimate_us(K, N, T) <= 0.9 * one;
}

// A launch plan: variant v0 over dst columns [0, k_split), then, when
// k_split < K, variant v1 over columns [k_split, K).
struct Plan {
    int v0;
    int64_t k_split;
    int v1;
};

// Byte offset of column k within a W row (k a whole number of blocks).
int64_t column_offset(int type, int64_t k) {
    Geometry g;
    return geometry(type, g) ? k / g.block * g.bytes : 0;
}

// A column split must start the second part on a whole block whose bytes,
// and whose dst column, keep the 16-byte alignment of the whole call.
bool split_point_ok(int type, int64_t k) {
    Geometry g;
    return geometry(type, g) && k % g.block == 0 && column_offset(type, k) % 16 == 0 && k % 4 == 0;
}

// Wave quantisation can leave the last round of tiles partly empty: Q4_0
// 17408 x 5120 at T = 2048 takes 1280 tiles of 64 x 128 (5 rounds of a
// small tile) or 320 of 128 x 256 (1.25 rounds). Two launches over disjoint
// column ranges of dst can do better: a larger tile over the columns whose
// tiles fill whole rounds, and the best tile over the rest (measured there:
// 128 x 256 over 4096 columns in 2.17 ms plus two-pipeline 64 x 128 over
// 1024 in 0.62 ms, against 2.99 ms for one launch). The plan is taken when
// its estimated cost is at least 1% lower and saves at least ~5 us of
// matrix time, which pays for the second launch.
// The smallest count c of column tiles for which tiles_t * c tiles fill
// whole rounds over the CUs: kNumCUs / gcd(tiles_t, kNumCUs).
int64_t whole_round_step(int64_t tiles_t) {
    int64_t g = kNumCUs, r = tiles_t % kNumCUs;
    while (r) {
        const int64_t t = g % r;
        g = r;
        r = t;
    }
    return kNumCUs / g;
}

constexpr double kPlanMargin = 0.99;
constexpr double kCuFlops = 157.3e12 / kNumCUs * 0.8;  // F32 FLOP/s of one CU at a typical tile efficiency
constexpr double kPlanMinSaving = 5e-6;                // seconds

Plan plan_for(int type, int64_t K, int64_t N, int64_t T, const Strides& s) {
    if (choose(type, K, N, T, s) == RETRO_VARIANT_SKINNY) return {RETRO_VARIANT_SKINNY, K, 0};
    const Choice single = choose_tile(type, K, N, T, s);
    Plan best{single.id, K, 0};
    if (single.id <= 0 || N == 0) return best;
    const double one = single.cost;
    double best_cost = one;
    for (const auto& v : kTiles) {
        // the two-pipeline tile is taken only through choose_tile's rule
        if (!v.ws || v.id == RETRO_VARIANT_WS2_64x128 || !auto_takes(v, type)) continue;
        if (!tile_applies(v, type, K, N, T, s)) continue;
        const int64_t tiles_t = cdiv(T, v.bt) * s.batches();
        const int64_t step = whole_round_step(tiles_t);
        for (int64_t c = step; c * v.bk < K; c += step) {
            const int64_t k1 = c * v.bk;
            if (!split_point_ok(type, k1)) continue;
            const Choice tail = choose_tile(type, K - k1, N, T, s);
            if (tail.id < 0) continue;
            const double cost = tile_cost(v, type, k1, T, s) + tail.cost;
            if (cost < best_cost) {
                best = {v.id, k1, tail.id};
                best_cost = cost;
            }
        }
    }
    if (best.k_split < K &&
        (best_cost > kPlanMargin * one || (one - best_cost) * 2.0 * double(N) / kCuFlops < kPlanMinSaving))
        return {single.id, K, 0};
    return best;
}

// The plan of the last few shapes seen on this thread. Automatic calls tend
// to repeat a shape, and a plan search costs a few microseconds of host time
// (about 20 tail choices over 13 tiles each), which a launch-bound call
// would feel. The plan depends on the type, the shape, W's and G's row
// strides, G's orientation and the number of matrices, nothing else.
struct PlanKey {
    int op;  // 0: out_prod, 1: mul_mat
    int type;
    int64_t K, N, T, ldw, ldg, batches;
    bool gcols;
    bool operator==(const PlanKey& o) const {
        return op == o.op && type == o.type && K == o.K && N == o.N && T == o.T && ldw == o.ldw &&
               ldg == o.ldg && batches == o.batches && gcols == o.gcols;
    }
};

template <typename Search>
Plan cached(const PlanKey& key, Search search) {
    constexpr int kSlots = 4;
    thread_local PlanKey keys[kSlots];
    thread_local Plan plans[kSlots];
    thread_local int used = 0, next = 0;
    for (int i = 0; i < used; ++i)
        if (keys[i] == key) return plans[i];
    const Plan p = search();
    keys[next] = key;
    plans[next] = p;
    next = (next + 1) % kSlots;
    if (used < kSlots) ++used;
    return p;
}

Plan cached_plan(int type, int64_t K, int64_t N, int64_t T, const Strides& s) {
    return cached(PlanKey{0, type, K, N, T, s.ldw, s.ldg, s.batches(), s.gcols},
                  [&] { return plan_for(type, K, N, T, s); });
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
    if (na <= 0 || nb <= 0) return false;
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + uint64_t(nb) && pb < pa + uint64_t(na);
}

// Whether a forced variant takes this type, shape and strides (all already
// checked).
bool variant_applies(int variant, int type, int64_t K, int64_t N, int64_t T, const Strides& s) {
    if (variant == RETRO_VARIANT_AUTO) return choose(type, K, N, T, s) > 0;
    if (variant == RETRO_VARIANT_SKINNY || variant == RETRO_VARIANT_SKINNY_8) return skinny_applies(type, K, N, T, s);
    if (variant == RETRO_VARIANT_SKINNY_16) return T <= 16 && skinny_applies(type, K, N, T, s);
    if (variant == RETRO_VARIANT_SPLIT_128x256) {
        // the 128 x 256 producer/consumer tile's limits, for G by rows
        constexpr TileVariant tile{RETRO_VARIANT_SPLIT_128x256, 128, 256, 1.0, true};
        Geometry g;
        return geometry(type, g) && g.block == 256 && !s.gcols && tile_applies(tile, type, K, N, T, s);
    }
    if (variant == RETRO_VARIANT_SPLIT_128x128) {
        // the 128 x 128 tile of the 32-element block types and the 16-bit
        // dense types, G by rows; dense rows are read in 16-byte units
        constexpr TileVariant tile{RETRO_VARIANT_SPLIT_128x128, 128, 128, 1.0, true};
        const bool typed = type == RETRO_Q4_0 || type == RETRO_Q5_0 || type == RETRO_MXFP4 ||
                           type == RETRO_BF16 || type == RETRO_F16;
        return typed && !s.gcols && (!is_dense(type) || s.ldw % 16 == 0) && tile_applies(tile, type, K, N, T, s);
    }
    const TileVariant* tv = find_tile(variant);
    return tv && tile_applies(*tv, type, K, N, T, s);
}

// G's layout from its two element strides: G[t][n] at t * sgt + n * sgn,
// with one of them 1 (rows contiguous: sgn = 1; columns contiguous, G stored
// t-fastest: sgt = 1, sgn > 1).
bool g_layout(int64_t sgt, int64_t sgn, Strides& s) {
    if (sgn == 1) {
        s.ldg = sgt;
        s.gcols = false;
        return true;
    }
    if (sgt == 1) {
        s.ldg = sgn;
        s.gcols = true;
        return true;
    }
    return false;
}

// Validation shared by the out_prod entry points: shape, strides, then (for
// a non-empty call) pointers, alignment and aliasing. `empty` is set when
// there is nothing to compute.
int check_call(int type, const void* W, const float* G, const float* dst, int64_t K, int64_t N, int64_t T,
               const Strides& s, bool& empty) {
    int rc = check_shape(type, K, N, T);
    if (rc != RETRO_OK) return rc;
    rc = check_strides(type, K, N, T, s);
    if (rc != RETRO_OK) return rc;
    empty = T == 0 || K == 0 || s.batches() == 0;
    if (empty) return RETRO_OK;
    // bytes each operand spans: one matrix, then all batches
    const int64_t w_bytes = N > 0 ? (N - 1) * s.ldw + row_bytes_of(type, K) : 0;
    const int64_t g_bytes = N > 0 ? (s.gcols ? (N - 1) * s.ldg + T : (T - 1) * s.ldg + N) * 4 : 0;
    const int64_t d_bytes = ((T - 1) * s.ldd + K) * 4;
    const int64_t w_all = N > 0 ? (s.ne03 - 1) * s.sw3 + (s.ne02 - 1) * s.sw2 + w_bytes : 0;
    const int64_t g_all = N > 0 ? ((s.ne3 - 1) * s.sg3 + (s.ne2 - 1) * s.sg2) * 4 + g_bytes : 0;
    const int64_t d_all = ((s.ne3 - 1) * s.sd3 + (s.ne2 - 1) * s.sd2) * 4 + d_bytes;
    if (!dst || (N > 0 && (!W || !G))) return RETRO_E_NULL;
    if (!aligned16(dst) || (N > 0 && (!aligned16(W) || !aligned16(G)))) return RETRO_E_ALIGN;
    if (overlap(dst, d_all, W, w_all) || overlap(dst, d_all, G, g_all)) return RETRO_E_ALIAS;
    // the dst matrices must not overlap one another: batch i2 after i2 - 1,
    // batch i3 after the whole of i3 - 1
    if ((s.ne2 > 1 && s.sd2 * 4 < d_bytes) || (s.ne3 > 1 && s.sd3 * 4 < (s.ne2 - 1) * s.sd2 * 4 + d_bytes))
        return RETRO_E_ALIAS;
    return RETRO_OK;
}

// One launch of `variant` (already checked to apply) over the call as given.
int launch_typed(int variant, int type, const void* W, const float* G, float* dst, int64_t K, int64_t N, int64_t T,
                 const Strides& s, hipStream_t st) {
    switch (type) {
        case RETRO_F32: return launch_out_prod<RETRO_F32>(variant, W, G, dst, K, N, T, s, st);
        case RETRO_F16: return launch_out_prod<RETRO_F16>(variant, W, G, dst, K, N, T, s, st);
        case RETRO_BF16: return launch_out_prod<RETRO_BF16>(variant, W, G, dst, K, N, T, s, st);
        case RETRO_Q8_0: return launch_out_prod<RETRO_Q8_0>(variant, W, G, dst, K, N, T, s, st);
        case RETRO_Q4_0: return launch_out_prod<RETRO_Q4_0>(variant, W, G, dst, K, N, T, s, st);
        case RETRO_Q4_1: return launch_out_prod<RETRO_Q4_1>(variant, W, G, dst, K, N, T, s, st);
        case RETRO_Q5_0: return launch_out_prod<RETRO_Q5_0>(variant, W, G, dst, K, N, T, s, st);
        case RETRO_Q5_1: return launch_out_prod<RETRO_Q5_1>(variant, W, G, dst, K, N, T, s, st);
        case RETRO_MXFP4: return launch_out_prod<RETRO_MXFP4>(variant, W, G, dst, K, N, T, s, st);
        case RETRO_NVFP4: return launch_out_prod<RETRO_NVFP4>(variant, W, G, dst, K, N, T, s, st);
        case RETRO_Q4_K: return launch_out_prod<RETRO_Q4_K>(variant, W, G, dst, K, N, T, s, st);
        case RETRO_Q5_K: return launch_out_prod<RETRO_Q5_K>(variant, W, G, dst, K, N, T, s, st);
        case RETRO_Q2_K: return launch_out_prod<RETRO_Q2_K>(variant, W, G, dst, K, N, T, s, st);
        case RETRO_Q3_K: return launch_out_prod<RETRO_Q3_K>(variant, W, G, dst, K, N, T, s, st);
        case RETRO_Q6_K: return launch_out_prod<RETRO_Q6_K>(variant, W, G, dst, K, N, T, s, st);
        default: return RETRO_E_TYPE;
    }
}

// The launches of a plan: the columns [0, k_split) of W and dst, then the
// rest. Each part reads all of G and writes only its own columns of dst.
int run_plan(const Plan& p, int type, const void* W, const float* G, float* dst, int64_t K, int64_t N, int64_t T,
             const Strides& s, hipStream_t st) {
    int rc = launch_typed(p.v0, type, W, G, dst, p.k_split, N, T, s, st);
    if (rc != RETRO_OK || p.k_split >= K) return rc;
    // with N = 0 there is no W to offset (it may be null, and is never read)
    const void* W1 = N > 0 ? static_cast<const void*>(static_cast<const char*>(W) + column_offset(type, p.k_split))
                           : W;
    return launch_typed(p.v1, type, W1, G, dst + p.k_split, K - p.k_split, N, T, s, st);
}

int out_prod_impl(int variant, int type, const void* W, const float* G, float* dst, int64_t K, int64_t N,
                  int64_t T, const Strides& s, void* stream) {
    bool empty = false;
    const int rc = check_call(type, W, G, dst, K, N, T, s, empty);
    if (rc != RETRO_OK || empty) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (variant == RETRO_VARIANT_AUTO) {
        const Plan p = cached_plan(type, K, N, T, s);
        if (p.v0 < 0) return p.v0;
        return run_plan(p, type, W, G, dst, K, N, T, s, st);
    }
    if (!variant_applies(variant, type, K, N, T, s)) return RETRO_E_VARIANT;
    return launch_typed(variant, type, W, G, dst, K, N, T, s, st);
}

// ---------------------------------------------------------------------------
// out_prod with a workspace: the n-split skinny kernel
// ---------------------------------------------------------------------------

int launch_split_typed(int type, const void* W, const float* G, float* dst, int64_t K, int64_t N, int64_t T,
                       const Strides& s, void* ws, hipStream_t st) {
    switch (type) {
        case RETRO_F32: return launch_out_prod_split<RETRO_F32>(W, G, dst, K, N, T, s, ws, st);
        case RETRO_F16: return launch_out_prod_split<RETRO_F16>(W, G, dst, K, N, T, s, ws, st);
        case RETRO_BF16: return launch_out_prod_split<RETRO_BF16>(W, G, dst, K, N, T, s, ws, st);
        case RETRO_Q8_0: return launch_out_prod_split<RETRO_Q8_0>(W, G, dst, K, N, T, s, ws, st);
        case RETRO_Q4_0: return launch_out_prod_split<RETRO_Q4_0>(W, G, dst, K, N, T, s, ws, st);
        case RETRO_Q4_1: return launch_out_prod_split<RETRO_Q4_1>(W, G, dst, K, N, T, s, ws, st);
        case RETRO_Q5_0: return launch_out_prod_split<RETRO_Q5_0>(W, G, dst, K, N, T, s, ws, st);
        case RETRO_Q5_1: return launch_out_prod_split<RETRO_Q5_1>(W, G, dst, K, N, T, s, ws, st);
        case RETRO_MXFP4: return launch_out_prod_split<RETRO_MXFP4>(W, G, dst, K, N, T, s, ws, st);
        case RETRO_NVFP4: return launch_out_prod_split<RETRO_NVFP4>(W, G, dst, K, N, T, s, ws, st);
        case RETRO_Q4_K: return launch_out_prod_split<RETRO_Q4_K>(W, G, dst, K, N, T, s, ws, st);
        case RETRO_Q5_K: return launch_out_prod_split<RETRO_Q5_K>(W, G, dst, K, N, T, s, ws, st);
        case RETRO_Q2_K: return launch_out_prod_split<RETRO_Q2_K>(W, G, dst, K, N, T, s, ws, st);
        case RETRO_Q3_K: return launch_out_prod_split<RETRO_Q3_K>(W, G, dst, K, N, T, s, ws, st);
        case RETRO_Q6_K: return launch_out_prod_split<RETRO_Q6_K>(W, G, dst, K, N, T, s, ws, st);
        default: return RETRO_E_TYPE;
    }
}

// Workspace bytes a call of `variant` uses for this (checked) shape: the
// split's fixed size, 0 for any other kernel, or RETRO_E_VARIANT.
int64_t workspace_need(int variant, int type, int64_t K, int64_t N, int64_t T, const Strides& s) {
    const int64_t bytes = split_workspace_bytes(skinny_blocks(T < kSplitMaxT ? T : kSplitMaxT));
    if (variant == RETRO_VARIANT_SKINNY_SPLIT) return skinny_split_applies(type, K, N, T, s) ? bytes : RETRO_E_VARIANT;
    if (variant == RETRO_VARIANT_AUTO)
        return skinny_split_applies(type, K, N, T, s) && skinny_split_pays(type, K, N, T, s) ? bytes : 0;
    return variant_applies(variant, type, K, N, T, s) ? 0 : RETRO_E_VARIANT;
}

int out_prod_ws_impl(int variant, int type, const void* W, const float* G, float* dst, int64_t K, int64_t N,
                     int64_t T, void* workspace, int64_t workspace_bytes, void* stream) {
    const Strides s = contiguous(type, K, N);
    bool empty = false;
    const int rc = check_call(type, W, G, dst, K, N, T, s, empty);
    if (rc != RETRO_OK) return rc;
    if (empty) return RETRO_OK;
    const int64_t need = workspace_need(variant, type, K, N, T, s);
    if (need < 0) return int(need);
    if (need == 0) return out_prod_impl(variant, type, W, G, dst, K, N, T, s, stream);
    if (!workspace || workspace_bytes < need) {
        if (variant == RETRO_VARIANT_SKINNY_SPLIT) return RETRO_E_WORKSPACE;
        return out_prod_impl(RETRO_VARIANT_AUTO, type, W, G, dst, K, N, T, s, stream);
    }
    if (!aligned16(workspace) || overlap(workspace, need, W, N * s.ldw) || overlap(workspace, need, G, T * N * 4) ||
        overlap(workspace, need, dst, T * K * 4))
        return RETRO_E_WORKSPACE;
    return launch_split_typed(type, W, G, dst, K, N, T, s, workspace, static_cast<hipStream_t>(stream));
}

// The device address of the current device's `scratch`, found once per
// device (with that device current) and kept; NULL if the runtime cannot
// give it.
constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_addr[kMaxDevices];
std::mutex scratch_mutex;

void* scratch_for_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void* p = scratch_addr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    p = scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        scratch_addr[dev].store(p, std::memory_order_release);
    }
    return p;
}

// retro_out_prod_ws with the static scratch as its workspace: validation
// first, and the scratch looked up only for a call that uses it.
int out_prod_noalloc_impl(int variant, int type, const void* W, const float* G, float* dst, int64_t K, int64_t N,
                          int64_t T, void* stream) {
    const Strides s = contiguous(type, K, N);
    bool empty = false;
    const int rc = check_call(type, W, G, dst, K, N, T, s, empty);
    if (rc != RETRO_OK || empty) return rc;
    const int64_t need = workspace_need(variant, type, K, N, T, s);
    if (need < 0) return int(need);
    if (need == 0) return out_prod_impl(variant, type, W, G, dst, K, N, T, s, stream);
    if (need > int64_t(sizeof(scratch))) return RETRO_E_WORKSPACE;
    void* ws = scratch_for_current_device();
    if (!ws) return RETRO_E_HIP;
    return out_prod_ws_impl(variant, type, W, G, dst, K, N, T, ws, int64_t(sizeof(scratch)), stream);
}

// ---------------------------------------------------------------------------
// mul_mat
// ---------------------------------------------------------------------------

struct MmTile {
    int id, bt, bn;
    double penalty;
};

constexpr MmTile kMmTiles[] = {
    {RETRO_VARIANT_WS_128x128, 128, 128, 1.00},
    // opt-in: measured slower than 128 x 128 (which runs two workgroups per
    // CU) on the quantized weights, faster only on dense rows (BF16 4096^3:
    // 1.02 against 1.06 ms)
    {RETRO_VARIANT_WS_256x128, 256, 128, 1.10},
    {RETRO_VARIANT_WS_64x128, 64, 128, 1.02},
    {RETRO_VARIANT_WS_32x128, 32, 128, 1.04},
};

// The tiled kernel loads x rows in 16-byte units and addresses a tile's W
// rows and x rows with 32-bit offsets.
bool mm_tile_applies(const MmTile& v, int type, int64_t K, int64_t N, int64_t T) {
    (void)N;
    if (is_dense(type) && K % 4) return false;
    return cdiv(T, v.bt) * cdiv(N, v.bn) < kGridLimit && int64_t(v.bn) * row_bytes_of(type, K) < (int64_t(1) << 31) &&
           int64_t(v.bt) * K * 4 < (int64_t(1) << 31);
}

bool mm_variant_applies(int variant, int type, int64_t K, int64_t N, int64_t T) {
    if (variant == RETRO_VARIANT_SIMPLE) return cdiv(T * N, 256) < kGridLimit;
    if (variant == RETRO_VARIANT_SKINNY)  // 16 rows of W and 64 of x (a pass) addressed with 32-bit offsets
        return cdiv(N, 16) < kGridLimit && !(is_dense(type) && K % 4) &&
               16 * row_bytes_of(type, K) < (int64_t(1) << 31) && kSkinnyMaxT * K * 4 < (int64_t(1) << 31);
    for (const auto& v : kMmTiles)
        if (v.id == variant) return mm_tile_applies(v, type, K, N, T);
    return false;
}

double mm_tile_cost(const MmTile& v, int64_t N, int64_t T) {
    return double(cdiv(cdiv(T, v.bt) * cdiv(N, v.bn), kNumCUs)) * v.bt * v.bn * v.penalty;
}

// The tiled forward kernel of least cost (wave quantisation over 256 CUs).
Choice mm_choose_tile(int type, int64_t K, int64_t N, int64_t T) {
    Choice best{-1, 0.0};
    for (const auto& v : kMmTiles) {
        if (!mm_tile_applies(v, type, K, N, T)) continue;
        const double cost = mm_tile_cost(v, N, T);
        if (best.id < 0 || cost < best.cost) best = {v.id, cost};
    }
    return best;
}

// Estimated times (us) for the forward. The skinny kernel, one pass per 64
// rows of x: about 4 us (and 1.5 per further block of 16 rows of x) plus, per
// 64-element k group of a wave, 0.88 us and 0.62 per further block (eight
// waves, one workgroup of 16 W rows per CU per round; fitted to Q4_K 4096 x
// 14336 and 14336 x 4096 and Q4_0 17408 x 5120: 28.8, 32.1 and 48.8 us at
// T = 16, 50.8 and 88 us at T = 32 and 64 on the first). A tile: rounds of one tile per CU, bt x bn x K MACs at 128 per
// cycle per CU and the efficiency of its rows of x (as for out_prod).
double mm_skinny_estimate_us(int64_t K, int64_t N, int64_t T) {
    const double rounds = double(cdiv(cdiv(N, 16), kNumCUs)), per_wave = double(cdiv(cdiv(K, 64), 8));
    auto pass = [&](int64_t t) {
        const double blocks = double(skinny_blocks(t));
        return 4.0 + 1.5 * (blocks - 1.0) + rounds * per_wave * (0.88 + 0.62 * (blocks - 1.0));
    };
    return passes_us(T, kSkinnyMaxT, pass);
}

double mm_tile_estimate_us(const MmTile& v, int64_t K, int64_t N, int64_t T) {
    const double rounds = double(cdiv(cdiv(T, v.bt) * cdiv(N, v.bn), kNumCUs));
    const double eff = v.bt <= 32 ? 0.6 : v.bt <= 64 ? 0.72 : 0.85;
    return 4.0 + rounds * double(v.bt) * v.bn * double(K) / 128.0 / eff / 2400.0;
}

// The skinny kernel for T <= 16, and above where its passes are estimated
// 10% faster than the best tile (with few tiles per CU the tiles leave most
// CUs idle: Q4_K 4096 x 14336 at T = 17 .. 128 ran 352 us in 32 x 128
// tiles, against 51 us for the skinny kernel at T = 32).
int mm_choose(int type, int64_t K, int64_t N, int64_t T) {
    const bool skinny = mm_variant_applies(RETRO_VARIANT_SKINNY, type, K, N, T);
    if (skinny && T <= 16) return RETRO_VARIANT_SKINNY;
    const Choice tile = mm_choose_tile(type, K, N, T);
    if (skinny) {
        const MmTile* v = nullptr;
        for (const auto& m : kMmTiles)
            if (m.id == tile.id) v = &m;
        if (!v || mm_skinny_estimate_us(K, N, T) < 0.9 * mm_tile_estimate_us(*v, K, N, T))
            return RETRO_VARIANT_SKINNY;
    }
    int best = tile.id;
    if (best < 0 && mm_variant_applies(RETRO_VARIANT_SIMPLE, type, K, N, T)) best = RETRO_VARIANT_SIMPLE;
    return best < 0 ? RETRO_E_SHAPE : best;
}

// The forward's plan: as for out_prod, but over W's rows (Y's columns),
// since Y[t][n] is complete in one tile. W rows [0, n_split) and the rest;
// every tile is 128 rows of W wide, so a split point is a multiple of 128
// and keeps the 16-byte alignment of W and Y. Measured on Q4_0 17408 x 5120,
// T = 2048: 128 x 128 tiles on 16384 rows plus one round of 64 x 128 on
// the last 1024 in 2.72 ms, against 2.85 ms for 17 rounds of 64 x 128.
Plan mm_plan_for(int type, int64_t K, int64_t N, int64_t T) {
    const int single = mm_choose(type, K, N, T);
    Plan best{single, N, 0};
    if (single <= 0 || single == RETRO_VARIANT_SKINNY || single == RETRO_VARIANT_SIMPLE || K == 0) return best;
    const double one = mm_choose_tile(type, K, N, T).cost;
    double best_cost = one;
    for (const auto& v : kMmTiles) {
        if (!mm_tile_applies(v, type, K, N, T)) continue;
        const int64_t tiles_t = cdiv(T, v.bt);
        const int64_t step = whole_round_step(tiles_t);
        for (int64_t c = step; c * v.bn < N; c += step) {
            const int64_t n1 = c * v.bn;
            const Choice tail = mm_choose_tile(type, K, N - n1, T);
            if (tail.id < 0) continue;
            const double cost = mm_tile_cost(v, n1, T) + tail.cost;
            if (cost < best_cost) {
                best = {v.id, n1, tail.id};
                best_cost = cost;
            }
        }
    }
    if (best.k_split < N &&
        (best_cost > kPlanMargin * one || (one - best_cost) * 2.0 * double(K) / kCuFlops < kPlanMinSaving))
        return {single, N, 0};
    return best;
}

Plan mm_cached_plan(int type, int64_t K, int64_t N, int64_t T) {
    return cached(PlanKey{1, type, K, N, T, 0, 0, 1, false}, [&] { return mm_plan_for(type, K, N, T); });
}

int launch_typed_mm(int variant, int type, const void* W, const float* X, float* Y, int64_t K, int64_t N, int64_t T,
                    int64_t ldy, hipStream_t st) {
    switch (type) {
        case RETRO_F32: return launch_mul_mat<RETRO_F32>(variant, W, X, Y, K, N, T, ldy, st);
        case RETRO_F16: return launch_mul_mat<RETRO_F16>(variant, W, X, Y, K, N, T, ldy, st);
        case RETRO_BF16: return launch_mul_mat<RETRO_BF16>(variant, W, X, Y, K, N, T, ldy, st);
        case RETRO_Q8_0: return launch_mul_mat<RETRO_Q8_0>(variant, W, X, Y, K, N, T, ldy, st);
        case RETRO_Q4_0: return launch_mul_mat<RETRO_Q4_0>(variant, W, X, Y, K, N, T, ldy, st);
        case RETRO_Q4_1: return launch_mul_mat<RETRO_Q4_1>(variant, W, X, Y, K, N, T, ldy, st);
        case RETRO_Q5_0: return launch_mul_mat<RETRO_Q5_0>(variant, W, X, Y, K, N, T, ldy, st);
        case RETRO_Q5_1: return launch_mul_mat<RETRO_Q5_1>(variant, W, X, Y, K, N, T, ldy, st);
        case RETRO_MXFP4: return launch_mul_mat<RETRO_MXFP4>(variant, W, X, Y, K, N, T, ldy, st);
        case RETRO_NVFP4: return launch_mul_mat<RETRO_NVFP4>(variant, W, X, Y, K, N, T, ldy, st);
        case RETRO_Q4_K: return launch_mul_mat<RETRO_Q4_K>(variant, W, X, Y, K, N, T, ldy, st);
        case RETRO_Q5_K: return launch_mul_mat<RETRO_Q5_K>(variant, W, X, Y, K, N, T, ldy, st);
        case RETRO_Q2_K: return launch_mul_mat<RETRO_Q2_K>(variant, W, X, Y, K, N, T, ldy, st);
        case RETRO_Q3_K: return launch_mul_mat<RETRO_Q3_K>(variant, W, X, Y, K, N, T, ldy, st);
        case RETRO_Q6_K: return launch_mul_mat<RETRO_Q6_K>(variant, W, X, Y, K, N, T, ldy, st);
        default: return RETRO_E_TYPE;
    }
}

// The launches of a forward plan: W rows and Y columns [0, n_split), then
// the rest (each reads all of X).
int run_mm_plan(const Plan& p, int type, const void* W, const float* X, float* Y, int64_t K, int64_t N, int64_t T,
                hipStream_t st) {
    const int64_t n1 = p.k_split;
    int rc = launch_typed_mm(p.v0, type, W, X, Y, K, n1, T, N, st);
    if (rc != RETRO_OK || n1 >= N) return rc;
    const void* W1 = static_cast<const char*>(W) + n1 * row_bytes_of(type, K);
    return launch_typed_mm(p.v1, type, W1, X, Y + n1, K, N - n1, T, N, st);
}

// Validation shared by the mul_mat entry points.
int check_mm_call(int type, const void* W, const float* X, const float* Y, int64_t K, int64_t N, int64_t T,
                  bool& empty) {
    const int rc = check_shape(type, K, N, T);
    if (rc != RETRO_OK) return rc;
    empty = T == 0 || N == 0;
    if (empty) return RETRO_OK;
    const int64_t w_bytes = N * row_bytes_of(type, K);
    const int64_t x_bytes = T * K * 4;
    const int64_t y_bytes = T * N * 4;
    if (!Y || (K > 0 && (!W || !X))) return RETRO_E_NULL;
    if (!aligned16(Y) || (K > 0 && (!aligned16(W) || !aligned16(X)))) return RETRO_E_ALIGN;
    if (overlap(Y, y_bytes, W, w_bytes) || overlap(Y, y_bytes, X, x_bytes)) return RETRO_E_ALIAS;
    return RETRO_OK;
}

int mul_mat_impl(int variant, int type, const void* W, const float* X, float* Y, int64_t K, int64_t N, int64_t T,
                 void* stream) {
    bool empty = false;
    const int rc = check_mm_call(type, W, X, Y, K, N, T, empty);
    if (rc != RETRO_OK || empty) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (variant == RETRO_VARIANT_AUTO) {
        const Plan p = mm_cached_plan(type, K, N, T);
        if (p.v0 < 0) return p.v0;
        return run_mm_plan(p, type, W, X, Y, K, N, T, st);
    }
    if (!mm_variant_applies(variant, type, K, N, T)) return RETRO_E_VARIANT;
    return launch_typed_mm(variant, type, W, X, Y, K, N, T, N, st);
}

}  // namespace

extern "C" {

int retro_mul_mat(int type, const void* W, const float* X, float* Y, int64_t K, int64_t N, int64_t T,
                  void* stream) {
    return mul_mat_impl(RETRO_VARIANT_AUTO, type, W, X, Y, K, N, T, stream);
}

int retro_mul_mat_variant(int variant, int type, const void* W, const float* X, float* Y, int64_t K, int64_t N,
                          int64_t T, void* stream) {
    return mul_mat_impl(variant, type, W, X, Y, K, N, T, stream);
}

int retro_mul_mat_choice(int type, int64_t K, int64_t N, int64_t T) {
    const int rc = check_shape(type, K, N, T);
    return rc != RETRO_OK ? rc : mm_cached_plan(type, K, N, T).v0;
}

int retro_mul_mat_plan(int type, int64_t K, int64_t N, int64_t T, int32_t* variant0, int64_t* n_split,
                       int32_t* variant1) {
    const int rc = check_shape(type, K, N, T);
    if (rc != RETRO_OK) return rc;
    if (!variant0 || !n_split || !variant1) return RETRO_E_NULL;
    const Plan p = mm_cached_plan(type, K, N, T);
    if (p.v0 < 0) return p.v0;
    *variant0 = p.v0;
    *n_split = p.k_split;
    *variant1 = p.k_split < N ? p.v1 : 0;
    return p.k_split < N ? 2 : 1;
}

int retro_mul_mat_row_split(int variant0, int64_t n_split, int variant1, int type, const void* W, const float* X,
                            float* Y, int64_t K, int64_t N, int64_t T, void* stream) {
    bool empty = false;
    const int rc = check_mm_call(type, W, X, Y, K, N, T, empty);
    if (rc != RETRO_OK) return rc;
    if (n_split <= 0 || n_split >= N) return RETRO_E_SHAPE;
    if (n_split % 4 || (n_split * row_bytes_of(type, K)) % 16) return RETRO_E_ALIGN;
    Plan p{variant0, n_split, variant1};
    if (p.v0 == RETRO_VARIANT_AUTO) p.v0 = mm_choose(type, K, n_split, T);
    if (p.v1 == RETRO_VARIANT_AUTO) p.v1 = mm_choose(type, K, N - n_split, T);
    if (p.v0 <= 0 || p.v1 <= 0 || !mm_variant_applies(p.v0, type, K, n_split, T) ||
        !mm_variant_applies(p.v1, type, K, N - n_split, T))
        return RETRO_E_VARIANT;
    if (empty) return RETRO_OK;
    return run_mm_plan(p, type, W, X, Y, K, N, T, static_cast<hipStream_t>(stream));
}

int retro_mul_mat_variant_applies(int variant, int type, int64_t K, int64_t N, int64_t T) {
    if (check_shape(type, K, N, T) != RETRO_OK) return 0;
    if (T == 0 || N == 0) return 1;
    if (variant == RETRO_VARIANT_AUTO) return mm_choose(type, K, N, T) > 0 ? 1 : 0;
    return mm_variant_applies(variant, type, K, N, T) ? 1 : 0;
}

int retro_out_prod(int type, const void* W, const float* G, float* dst, int64_t K, int64_t N, int64_t T,
                   void* stream) {
    return out_prod_impl(RETRO_VARIANT_AUTO, type, W, G, dst, K, N, T, contiguous(type, K, N), stream);
}

int retro_out_prod_ws(int variant, int type, const void* W, const float* G, float* dst, int64_t K, int64_t N,
                      int64_t T, void* workspace, int64_t workspace_bytes, void* stream) {
    return out_prod_ws_impl(variant, type, W, G, dst, K, N, T, workspace, workspace_bytes, stream);
}

int retro_out_prod_noalloc(int variant, int type, const void* W, const float* G, float* dst, int64_t K, int64_t N,
                           int64_t T, void* stream) {
    return out_prod_noalloc_impl(variant, type, W, G, dst, K, N, T, stream);
}

int64_t retro_out_prod_workspace_size(int variant, int type, int64_t K, int64_t N, int64_t T) {
    const int rc = check_shape(type, K, N, T);
    if (rc != RETRO_OK) return rc;
    return workspace_need(variant, type, K, N, T, contiguous(type, K, N));
}

int retro_out_prod_variant(int variant, int type, const void* W, const float* G, float* dst, int64_t K,
                           int64_t N, int64_t T, void* stream) {
    return out_prod_impl(variant, type, W, G, dst, K, N, T, contiguous(type, K, N), stream);
}

int retro_out_prod_strided(int type, const void* W, int64_t ldw, const float* G, int64_t ldg, float* dst,
                           int64_t ldd, int64_t K, int64_t N, int64_t T, void* stream) {
    return out_prod_impl(RETRO_VARIANT_AUTO, type, W, G, dst, K, N, T, Strides{ldw, ldg, ldd}, stream);
}

int retro_out_prod_strided_variant(int variant, int type, const void* W, int64_t ldw, const float* G,
                                   int64_t ldg, float* dst, int64_t ldd, int64_t K, int64_t N, int64_t T,
                                   void* stream) {
    return out_prod_impl(variant, type, W, G, dst, K, N, T, Strides{ldw, ldg, ldd}, stream);
}

int retro_out_prod_views_variant(int variant, int type, const void* W, int64_t ldw, int64_t sw2, int64_t sw3,
                                 const float* G, int64_t sgt, int64_t sgn, int64_t sg2, int64_t sg3, float* dst,
                                 int64_t ldd, int64_t sd2, int64_t sd3, int64_t K, int64_t N, int64_t T, int64_t ne02,
                                 int64_t ne03, int64_t ne2, int64_t ne3, void* stream) {
    Strides s{ldw, 0, ldd};
    if (!g_layout(sgt, sgn, s)) return RETRO_E_SHAPE;
    s.ne02 = ne02;
    s.ne03 = ne03;
    s.ne2 = ne2;
    s.ne3 = ne3;
    s.sw2 = sw2;
    s.sw3 = sw3;
    s.sg2 = sg2;
    s.sg3 = sg3;
    s.sd2 = sd2;
    s.sd3 = sd3;
    return out_prod_impl(variant, type, W, G, dst, K, N, T, s, stream);
}

int retro_out_prod_views(int type, const void* W, int64_t ldw, int64_t sw2, int64_t sw3, const float* G, int64_t sgt,
                         int64_t sgn, int64_t sg2, int64_t sg3, float* dst, int64_t ldd, int64_t sd2, int64_t sd3,
                         int64_t K, int64_t N, int64_t T, int64_t ne02, int64_t ne03, int64_t ne2, int64_t ne3,
                         void* stream) {
    return retro_out_prod_views_variant(RETRO_VARIANT_AUTO, type, W, ldw, sw2, sw3, G, sgt, sgn, sg2, sg3, dst, ldd,
                                        sd2, sd3, K, N, T, ne02, ne03, ne2, ne3, stream);
}

int retro_out_prod_batched_variant(int variant, int type, const void* W, int64_t ldw, int64_t sw2, int64_t sw3,
                                   const float* G, int64_t ldg, int64_t sg2, int64_t sg3, float* dst, int64_t ldd,
                                   int64_t sd2, int64_t sd3, int64_t K, int64_t N, int64_t T, int64_t ne02,
                                   int64_t ne03, int64_t ne2, int64_t ne3, void* stream) {
    return retro_out_prod_views_variant(variant, type, W, ldw, sw2, sw3, G, ldg, 1, sg2, sg3, dst, ldd, sd2, sd3, K,
                                        N, T, ne02, ne03, ne2, ne3, stream);
}

int retro_out_prod_batched(int type, const void* W, int64_t ldw, int64_t sw2, int64_t sw3, const float* G,
                           int64_t ldg, int64_t sg2, int64_t sg3, float* dst, int64_t ldd, int64_t sd2, int64_t sd3,
                           int64_t K, int64_t N, int64_t T, int64_t ne02, int64_t ne03, int64_t ne2, int64_t ne3,
                           void* stream) {
    return retro_out_prod_batched_variant(RETRO_VARIANT_AUTO, type, W, ldw, sw2, sw3, G, ldg, sg2, sg3, dst, ldd,
                                          sd2, sd3, K, N, T, ne02, ne03, ne2, ne3, stream);
}

int retro_dequantize(int type, const void* W, float* out, int64_t K, int64_t N, void* stream) {
    Geometry g;
    if (!geometry(type, g)) return RETRO_E_TYPE;
    if (K < 0 || N < 0 || K % g.block || K >= kDimLimit || N >= kDimLimit) return RETRO_E_SHAPE;
    if (!product_below(N, K, kCountLimit) || cdiv(N * cdiv(K, 4), 256) >= kGridLimit) return RETRO_E_SHAPE;
    if (K == 0 || N == 0) return RETRO_OK;
    if (!W || !out) return RETRO_E_NULL;
    if (!aligned16(W) || !aligned16(out)) return RETRO_E_ALIGN;
    if (overlap(out, N * K * 4, W, N * row_bytes_of(type, K))) return RETRO_E_ALIAS;
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (type) {
        case RETRO_F32: return launch_dequant<RETRO_F32>(W, out, K, N, st);
        case RETRO_F16: return launch_dequant<RETRO_F16>(W, out, K, N, st);
        case RETRO_BF16: return launch_dequant<RETRO_BF16>(W, out, K, N, st);
        case RETRO_Q8_0: return launch_dequant<RETRO_Q8_0>(W, out, K, N, st);
        case RETRO_Q4_0: return launch_dequant<RETRO_Q4_0>(W, out, K, N, st);
        case RETRO_Q4_1: return launch_dequant<RETRO_Q4_1>(W, out, K, N, st);
        case RETRO_Q5_0: return launch_dequant<RETRO_Q5_0>(W, out, K, N, st);
        case RETRO_Q5_1: return launch_dequant<RETRO_Q5_1>(W, out, K, N, st);
        case RETRO_MXFP4: return launch_dequant<RETRO_MXFP4>(W, out, K, N, st);
        case RETRO_NVFP4: return launch_dequant<RETRO_NVFP4>(W, out, K, N, st);
        case RETRO_Q4_K: return launch_dequant<RETRO_Q4_K>(W, out, K, N, st);
        case RETRO_Q5_K: return launch_dequant<RETRO_Q5_K>(W, out, K, N, st);
        case RETRO_Q2_K: return launch_dequant<RETRO_Q2_K>(W, out, K, N, st);
        case RETRO_Q3_K: return launch_dequant<RETRO_Q3_K>(W, out, K, N, st);
        case RETRO_Q6_K: return launch_dequant<RETRO_Q6_K>(W, out, K, N, st);
        default: return RETRO_E_TYPE;
    }
}

int retro_out_prod_supported(int type, int64_t K, int64_t N, int64_t T) {
    if (check_shape(type, K, N, T) != RETRO_OK) return 0;
    if (T == 0 || K == 0) return 1;
    return choose(type, K, N, T, contiguous(type, K, N)) > 0 ? 1 : 0;
}

int retro_out_prod_variant_applies(int variant, int type, int64_t K, int64_t N, int64_t T) {
    return retro_out_prod_strided_variant_applies(variant, type, K, N, T, row_bytes_of(type, K), N, K);
}

int retro_out_prod_strided_variant_applies(int variant, int type, int64_t K, int64_t N, int64_t T, int64_t ldw,
                                           int64_t ldg, int64_t ldd) {
    if (check_shape(type, K, N, T) != RETRO_OK) return 0;
    const Strides s{ldw, ldg, ldd};
    if (check_strides(type, K, N, T, s) != RETRO_OK) return 0;
    if (T == 0 || K == 0) return 1;
    return variant_applies(variant, type, K, N, T, s) ? 1 : 0;
}

int retro_out_prod_views_variant_applies(int variant, int type, int64_t K, int64_t N, int64_t T, int64_t ldw,
                                         int64_t sgt, int64_t sgn, int64_t ldd) {
    if (check_shape(type, K, N, T) != RETRO_OK) return 0;
    Strides s{ldw, 0, ldd};
    if (!g_layout(sgt, sgn, s) || check_strides(type, K, N, T, s) != RETRO_OK) return 0;
    if (T == 0 || K == 0) return 1;
    return variant_applies(variant, type, K, N, T, s) ? 1 : 0;
}

int retro_out_prod_views_choice(int type, int64_t K, int64_t N, int64_t T, int64_t ldw, int64_t sgt, int64_t sgn,
                                int64_t ldd, int64_t ne2, int64_t ne3) {
    int rc = check_shape(type, K, N, T);
    if (rc != RETRO_OK) return rc;
    Strides s{ldw, 0, ldd};
    if (!g_layout(sgt, sgn, s)) return RETRO_E_SHAPE;
    s.ne2 = ne2;
    s.ne3 = ne3;
    rc = check_strides(type, K, N, T, s);
    return rc != RETRO_OK ? rc : cached_plan(type, K, N, T, s).v0;
}

int retro_out_prod_choice(int type, int64_t K, int64_t N, int64_t T) {
    const int rc = check_shape(type, K, N, T);
    if (rc != RETRO_OK) return rc;
    return cached_plan(type, K, N, T, contiguous(type, K, N)).v0;
}

int retro_out_prod_plan(int type, int64_t K, int64_t N, int64_t T, int32_t* variant0, int64_t* k_split,
                        int32_t* variant1) {
    const int rc = check_shape(type, K, N, T);
    if (rc != RETRO_OK) return rc;
    if (!variant0 || !k_split || !variant1) return RETRO_E_NULL;
    const Plan p = cached_plan(type, K, N, T, contiguous(type, K, N));
    if (p.v0 < 0) return p.v0;
    *variant0 = p.v0;
    *k_split = p.k_split;
    *variant1 = p.k_split < K ? p.v1 : 0;
    return p.k_split < K ? 2 : 1;
}

int retro_out_prod_views_plan(int type, int64_t K, int64_t N, int64_t T, int64_t ldw, int64_t sgt, int64_t sgn,
                              int64_t ldd, int64_t ne2, int64_t ne3, int32_t* variant0, int64_t* k_split,
                              int32_t* variant1) {
    int rc = check_shape(type, K, N, T);
    if (rc != RETRO_OK) return rc;
    if (!variant0 || !k_split || !variant1) return RETRO_E_NULL;
    Strides s{ldw, 0, ldd};
    if (!g_layout(sgt, sgn, s)) return RETRO_E_SHAPE;
    s.ne2 = ne2;
    s.ne3 = ne3;
    rc = check_strides(type, K, N, T, s);
    if (rc != RETRO_OK) return rc;
    const Plan p = cached_plan(type, K, N, T, s);
    if (p.v0 < 0) return p.v0;
    *variant0 = p.v0;
    *k_split = p.k_split;
    *variant1 = p.k_split < K ? p.v1 : 0;
    return p.k_split < K ? 2 : 1;
}

int retro_out_prod_column_split(int variant0, int64_t k_split, int variant1, int type, const void* W,
                                const float* G, float* dst, int64_t K, int64_t N, int64_t T, void* stream) {
    const Strides s = contiguous(type, K, N);
    bool empty = false;
    const int rc = check_call(type, W, G, dst, K, N, T, s, empty);
    if (rc != RETRO_OK) return rc;
    Geometry g;
    geometry(type, g);  // known: check_call accepted the type
    if (k_split <= 0 || k_split >= K || k_split % g.block) return RETRO_E_SHAPE;
    if (!split_point_ok(type, k_split)) return RETRO_E_ALIGN;
    Plan p{variant0, k_split, variant1};
    if (p.v0 == RETRO_VARIANT_AUTO) p.v0 = choose(type, k_split, N, T, s);
    if (p.v1 == RETRO_VARIANT_AUTO) p.v1 = choose(type, K - k_split, N, T, s);
    if (p.v0 <= 0 || p.v1 <= 0 || !variant_applies(p.v0, type, k_split, N, T, s) ||
        !variant_applies(p.v1, type, K - k_split, N, T, s))
        return RETRO_E_VARIANT;
    if (empty) return RETRO_OK;
    return run_plan(p, type, W, G, dst, K, N, T, s, static_cast<hipStream_t>(stream));
}

int64_t retro_row_bytes(int type, int64_t K) { return row_bytes_of(type, K); }

const char* retro_strerror(int code) {
    switch (code) {
        case RETRO_OK: return "ok";
        case RETRO_E_TYPE: return "unknown or unsupported weight type";
        case RETRO_E_SHAPE: return "bad shape: negative size, K not a whole number of blocks, or size over the limits";
        case RETRO_E_NULL: return "NULL buffer";
        case RETRO_E_ALIGN: return "W, G and dst must be 16-byte aligned, and W rows as aligned as its blocks";
        case RETRO_E_ALIAS: return "dst overlaps W or G";
        case RETRO_E_HIP: return "HIP launch error";
        case RETRO_E_VARIANT: return "kernel variant unknown or not applicable to this type and shape";
        case RETRO_E_WORKSPACE: return "workspace missing, too small, misaligned or overlapping an operand";
        default: return "unknown error code";
    }
}

}  // extern "C"

