"""Parity of the HIP library against the CPU oracle, on cuda:0.

Bars (the project's acceptance criteria):
  * decoded values bit-exact (retro_dequantize, and the fused kernels'
    decode through an identity gradient);
  * the contraction within NMSE <= 1e-7 and max relative error <= 1e-5 per
    output, the error of an output taken relative to sum_n |W[n][k] G[t][n]|
    (the literal |y - r| / |r| is unattainable for any F32-accumulating
    contraction: outputs near zero by cancellation have unbounded relative
    error).
A tighter internal gate (max relative error <= 2e-6) catches a silent loss
of precision (for example a gradient rounded to fp16), which the contract
bars alone would let through.
"""

import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

NMSE_MAX = 1e-7
REL_MAX = 1e-5
REL_TIGHT = 2e-6
ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))

TYPES = [wl.F32, wl.F16, wl.BF16, wl.Q8_0, wl.Q4_0, wl.Q4_1, wl.Q5_0, wl.Q5_1, wl.MXFP4, wl.NVFP4, wl.Q2_K, wl.Q3_K,
         wl.Q4_K, wl.Q5_K, wl.Q6_K]
KQUANTS = (wl.Q2_K, wl.Q3_K, wl.Q4_K, wl.Q5_K, wl.Q6_K)
ALL_TILES = ["tile_128x128", "tile_128x256", "tile_64x128", "tile_64x64", "tile_64x256",
             "ws_256x256", "ws_128x256", "ws_64x256", "ws_128x128", "ws_64x128", "ws_32x256", "ws_32x128",
             "ws2_64x128"]


@pytest.fixture(scope="module")
def q():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import quantized_weight_backward_amd as q

    return q


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def variant_id(q, name):
    return {v: k for k, v in q.VARIANT_NAMES.items()}[name]


def tile_variants(wtype):
    if wtype in KQUANTS:
        return ["tile_128x256", "tile_64x256", "ws_256x256", "ws_128x256", "ws_64x256", "ws_32x256"]
    return ALL_TILES


def applies(q, c, variant):
    """Whether a forced variant takes this type and shape (host-only query)."""
    if variant == "auto":
        return True
    return q.variant_applies(variant_id(q, variant), c["type"], c["K"], c["N"], c["T"])


def run(q, c, variant="auto", prefill=float("nan")):
    W, G = dev(c["W"]), dev(c["G"])
    out = torch.full((c["T"], c["K"]), prefill, dtype=torch.float32, device="cuda")
    v = q.VARIANT_AUTO if variant == "auto" else variant_id(q, variant)
    q.out_prod(c["type"], W, G, c["K"], out=out, variant=v)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_close(y, acc, ab, label=""):
    e = oracle.errors(y, acc, ab)
    assert e["nonfinite"] == 0, (label, e)
    assert e["nmse"] <= NMSE_MAX, (label, e)
    assert e["max_rel"] <= REL_MAX, (label, e)
    assert e["max_rel"] <= REL_TIGHT, (label, e)
    return e


# Shapes spanning several tiles with ragged tails in T, N and K, and the
# alignment paths: (N % 4 != 0) -> scalar G loads; K chosen so that the W
# row pitch is 16-, 8-, 4- or only 2-byte aligned.
SMALL_K = {
    wl.F32: (300, 256, 301, 300),
    wl.F16: (301, 264, 296, 264),
    wl.BF16: (300, 520, 302, 520),
    wl.Q8_0: (416, 768, 352, 416),
    wl.Q4_0: (512, 352, 416, 352),
    wl.Q4_1: (512, 352, 192, 416),
    wl.Q5_0: (352, 416, 128, 352),
    wl.Q5_1: (512, 352, 416, 256),
    wl.MXFP4: (352, 416, 512, 128),   # 187-, 221-byte rows: odd pitches
    wl.NVFP4: (320, 448, 128, 384),   # 180-, 252-, 72-byte rows: 4-byte aligned pitches
    wl.Q4_K: (768, 512, 256, 768),
    wl.Q5_K: (512, 768, 256, 512),
    wl.Q6_K: (768, 256, 512, 768),
    wl.Q2_K: (512, 768, 256, 768),
    wl.Q3_K: (768, 512, 256, 512),
}
# (T, N): the last case has N % 4 == 0 (G rows 16-byte aligned, which the
# producer/consumer kernel needs) with a partial last chunk of 4 rows
SMALL_TN = ((200, 77), (130, 96), (67, 33), (150, 100))


def small_case(wtype, i, seed):
    T, N = SMALL_TN[i]
    return wl.make_case(wtype, N, SMALL_K[wtype][i], T, seed)


# --- decode ---------------------------------------------------------------------

def same_bits(a, b):
    """Bit-identical floats, the sign of every zero included (the decoders
    form a*(q - c) in that order, as the formats define it)."""
    a, b = np.asarray(a, np.float32), np.asarray(b, np.float32)
    return a.shape == b.shape and bool(np.all(a.view(np.uint32) == b.view(np.uint32)))


@pytest.mark.parametrize("wtype", TYPES)
@pytest.mark.parametrize("i", [0, 1, 2, 3])
def test_dequantize_bit_exact(q, wtype, i):
    c = small_case(wtype, i, 100 + i)
    ref = oracle.dequantize(wtype, c["W"], c["K"])
    got = q.dequantize(wtype, dev(c["W"]), c["K"], c["N"]).cpu().numpy()
    assert same_bits(got, ref)


def test_dequantize_hand_built_blocks(q, golden):
    for fixture, wtype in (("q8_0_blocks.txt", wl.Q8_0), ("q4_0_blocks.txt", wl.Q4_0)):
        g = golden(fixture)
        names = sorted(k[:-4] for k in g if k.endswith("_hex"))
        raw = np.stack([np.array([int(t, 16) for t in g[n + "_hex"]], dtype=np.uint8) for n in names])
        expected = np.stack([np.array([float(v) for v in g[n + "_expected"]], dtype=np.float32) for n in names])
        got = q.dequantize(wtype, dev(raw), 32, len(names)).cpu().numpy()
        assert np.array_equal(got.view(np.uint32), expected.view(np.uint32)), fixture


@pytest.mark.parametrize("wtype", TYPES)
def test_fused_decode_through_identity_gradient(q, wtype):
    """With T = N and G = I, out_prod(W, I) = decoded W exactly (every other
    term is w * 0); this checks every tile kernel's and the skinny kernel's
    decode without trusting retro_dequantize."""
    for K in (SMALL_K[wtype][0], SMALL_K[wtype][3]):
        for N, variants in ((48, tile_variants(wtype)), (16, ["skinny"] + tile_variants(wtype))):
            c = wl.make_case(wtype, N, K, N, seed=7)
            ref = oracle.dequantize(wtype, c["W"], c["K"])
            c["G"] = np.eye(N, dtype=np.float32)
            for v in variants:
                if not applies(q, c, v):
                    continue
                got = run(q, c, v)
                assert np.array_equal(got, ref), (v, N, K)


# --- contraction ----------------------------------------------------------------

def ws_expected(c):
    """Whether the producer/consumer variants should take a case: G rows in
    16-byte units, dense W rows in 4-element units."""
    dense = c["type"] in (wl.F32, wl.F16, wl.BF16)
    return c["N"] % 4 == 0 and (not dense or c["K"] % 4 == 0)


@pytest.mark.parametrize("wtype", TYPES)
@pytest.mark.parametrize("i", [0, 1, 2, 3])
def test_tile_variants_match_oracle(q, wtype, i):
    c = small_case(wtype, i, 200 + i)
    _, acc, ab = oracle.out_prod(wtype, c["W"], c["G"], c["K"], nthreads=ORACLE_THREADS)
    ran = []
    for v in ["auto"] + tile_variants(wtype):
        if applies(q, c, v):
            check_close(run(q, c, v), acc, ab, v)
            ran.append(v)
    expected = [v for v in tile_variants(wtype) if not v.startswith("ws") or ws_expected(c)]
    assert set(expected) <= set(ran), (expected, ran)


@pytest.mark.parametrize("wtype", TYPES)
@pytest.mark.parametrize("T,N", [(1, 77), (5, 96), (16, 300), (16, 33), (3, 1)])
def test_skinny_matches_oracle(q, wtype, T, N):
    c = wl.make_case(wtype, N, SMALL_K[wtype][0], T, seed=300 + T + N)
    _, acc, ab = oracle.out_prod(wtype, c["W"], c["G"], c["K"], nthreads=ORACLE_THREADS)
    assert q.choice(wtype, c["K"], N, T) == q.VARIANT_SKINNY
    for v in ("skinny", "skinny_8", "skinny_16", "auto"):
        check_close(run(q, c, v), acc, ab, v)
    small_tile = "tile_64x256" if wtype in KQUANTS else "tile_64x64"
    check_close(run(q, c, small_tile), acc, ab, "tile at small T")
    for v in tile_variants(wtype):
        if v.startswith("ws") and applies(q, c, v):
            check_close(run(q, c, v), acc, ab, v + " at small T")


@pytest.mark.parametrize("wtype", TYPES)
@pytest.mark.parametrize("T,N", [(17, 77), (33, 300), (48, 96), (64, 33), (40, 1), (130, 77), (200, 48)])
def test_skinny_blocks_of_t_match_oracle(q, wtype, T, N):
    """The skinny kernel feeds each decoded weight to every block of 16 rows
    of G, up to four blocks a pass over W (ragged last block, N ragged and
    below a group; T = 130 and 200 take three and four passes)."""
    c = wl.make_case(wtype, N, SMALL_K[wtype][1], T, seed=320 + T + N)
    _, acc, ab = oracle.out_prod(wtype, c["W"], c["G"], c["K"], nthreads=ORACLE_THREADS)
    assert applies(q, c, "skinny") and applies(q, c, "skinny_8") and not applies(q, c, "skinny_16")
    for v in ("skinny", "skinny_8", "auto"):
        check_close(run(q, c, v), acc, ab, v)
    # G stored t-fastest and a padded dst through the strided views
    W, G = dev(c["W"]), dev(c["G"])
    gt = torch.zeros((N, T + 5), device="cuda")
    gt[:, :T] = G.t()
    out = torch.full((T, c["K"] + 4), float("nan"), device="cuda")[:, 4:]
    q.out_prod(wtype, W, gt[:, :T].t(), c["K"], out=out, variant=q.VARIANT_SKINNY)
    torch.cuda.synchronize()
    check_close(out.cpu().numpy(), acc, ab, "skinny, G t-fastest")


@pytest.mark.parametrize("wtype,K", [(wl.F32, 301), (wl.F16, 301), (wl.BF16, 302)])
@pytest.mark.parametrize("T", [33, 70])
def test_skinny_blocks_of_t_dense_odd_k(q, wtype, K, T):
    """Dense rows whose K is not a multiple of 4 take the masked loads, also
    with several blocks of G and several passes over W."""
    c = wl.make_case(wtype, 96, K, T, seed=360 + T + K)
    _, acc, ab = oracle.out_prod(wtype, c["W"], c["G"], K, nthreads=ORACLE_THREADS)
    for v in ("skinny", "skinny_8"):
        check_close(run(q, c, v), acc, ab, v)


def test_q8_0_tiny_workload(q):
    c = wl.workload("q8_0_n128_k256_t64")
    dst, acc, ab = oracle.out_prod(c["type"], c["W"], c["G"], c["K"])
    y = run(q, c)
    check_close(y, acc, ab)


@pytest.mark.parametrize("wtype", [wl.Q8_0, wl.Q4_0, wl.Q4_1, wl.Q5_0, wl.Q5_1, wl.MXFP4, wl.NVFP4, wl.Q2_K, wl.Q3_K, wl.Q4_K,
                                   wl.Q5_K, wl.Q6_K, wl.F16, wl.BF16])
def test_f32_twin_on_device(q, wtype):
    """out_prod(Qx, W) and out_prod(F32, dequant(W)) run the same tile on
    identical B operands, so they agree bit for bit."""
    c = small_case(wtype, 1, 400)
    w32 = oracle.dequantize(wtype, c["W"], c["K"])
    twin = dict(c, type=wl.F32, W=w32.view(np.uint8))
    # the skinny kernel with its wave count pinned: the automatic count
    # depends on the type (and sets the order of the cross-wave sum)
    for v in tile_variants(wtype) + ["skinny_8", "skinny_16", "skinny_8_t40"]:
        if v == "skinny_8_t40":  # three blocks of 16 rows of G
            c2, t2 = dict(c, T=40, G=c["G"][:40]), dict(twin, T=40, G=c["G"][:40])
            v = "skinny_8"
        elif not applies(q, twin, v) or not applies(q, c, v):
            continue
        elif v.startswith("skinny"):
            c2, t2 = dict(c, T=16, G=c["G"][:16]), dict(twin, T=16, G=c["G"][:16])
        else:
            c2, t2 = c, twin
        a = run(q, c2, v)
        b = run(q, t2, v)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), v


# --- invariants -----------------------------------------------------------------

@pytest.mark.parametrize("wtype", [wl.Q2_K, wl.Q3_K, wl.Q4_K, wl.Q5_K, wl.Q6_K, wl.Q4_0, wl.Q5_1, wl.MXFP4, wl.NVFP4,
                                   wl.BF16])
@pytest.mark.parametrize("i", [0, 3])
def test_invariants(q, wtype, i):
    c = small_case(wtype, i, 500)
    base = run(q, c)
    # every output written (NaN prefill gone), two runs bitwise equal
    assert np.isfinite(base).all()
    assert np.array_equal(run(q, c, prefill=1e30).view(np.uint32), base.view(np.uint32))
    # scaling G by 2 scales every output by exactly 2
    two = run(q, dict(c, G=c["G"] * np.float32(2)))
    assert np.array_equal(two, 2 * base)
    # zero gradient
    assert not run(q, dict(c, G=np.zeros_like(c["G"]))).any()
    # permuting the rows of G permutes the rows of dst
    perm = np.random.default_rng(1).permutation(c["T"])
    pg = run(q, dict(c, G=c["G"][perm]))
    _, acc, ab = oracle.out_prod(wtype, c["W"], c["G"], c["K"], nthreads=ORACLE_THREADS)
    check_close(pg, acc[perm], ab[perm])


@pytest.mark.parametrize("wtype", TYPES)
def test_empty_reduction_fills_zeros(q, wtype):
    K = SMALL_K[wtype][0]
    for T in (7, 100):
        c = {"type": wtype, "K": K, "N": 0, "T": T, "W": np.zeros((0, wl.row_bytes(wtype, K)), np.uint8),
             "G": np.zeros((T, 0), np.float32)}
        y = run(q, c)
        assert np.array_equal(y, np.zeros((T, K), np.float32))


@pytest.mark.parametrize("wtype", [wl.Q4_K, wl.Q2_K, wl.Q3_K, wl.Q4_0, wl.F32, wl.MXFP4, wl.NVFP4])
def test_empty_reduction_with_a_row_stride(q, wtype):
    """N = 0 with G an empty view whose row stride is not 0 (torch hands over
    a null pointer for it): every kernel that takes the shape writes zeros and
    reads nothing of G or W."""
    K = SMALL_K[wtype][0]
    W = torch.zeros(0, dtype=torch.uint8, device="cuda")
    for T in (7, 100):
        G = torch.zeros((T, 8), device="cuda")[:, :0]
        for v in ["auto", "skinny"] + tile_variants(wtype) + ([SPLIT_VARIANT[wtype]] if wtype in SPLIT_VARIANT else []):
            vid = 0 if v == "auto" else variant_id(q, v)
            if v != "auto" and not q.variant_applies_strided(vid, wtype, K, 0, T, wl.row_bytes(wtype, K), 8, K):
                continue
            out = torch.full((T, K), float("nan"), device="cuda")
            q.out_prod(wtype, W, G, K, out=out, variant=vid)
            torch.cuda.synchronize()
            assert not out.any() and not out.isnan().any(), v


def test_zero_size_calls_touch_nothing(q):
    out = torch.full((0, 256), 1.0, device="cuda")
    q.out_prod(wl.Q4_K, torch.zeros(0, dtype=torch.uint8, device="cuda"),
               torch.zeros((0, 0), device="cuda"), 256, out=out)
    assert q.lib.retro_out_prod(wl.Q4_K, None, None, None, 0, 5, 5, None) == 0
    assert q.lib.retro_out_prod(wl.Q4_K, None, None, None, 256, 5, 0, None) == 0


@pytest.mark.parametrize("i", [0, 3])
def test_no_allocation_during_a_call(q, i):
    c = small_case(wl.Q4_K, i, 600)
    W, G = dev(c["W"]), dev(c["G"])
    out = torch.empty((c["T"], c["K"]), device="cuda")
    q.out_prod(wl.Q4_K, W, G, c["K"], out=out)  # warm (module load)
    torch.cuda.synchronize()
    before_alloc = torch.cuda.memory_allocated()
    free_before, _ = torch.cuda.mem_get_info()
    for _ in range(3):
        q.out_prod(wl.Q4_K, W, G, c["K"], out=out)
    torch.cuda.synchronize()
    free_after, _ = torch.cuda.mem_get_info()
    assert torch.cuda.memory_allocated() == before_alloc
    assert free_after == free_before


def test_device_side_argument_errors(q):
    c = small_case(wl.Q4_K, 1, 700)
    W, G = dev(c["W"]), dev(c["G"])
    T, N, K = c["T"], c["N"], c["K"]
    big = torch.empty(T * K + 64, device="cuda")
    out = big[:T * K]
    lib = q.lib
    args = lambda w, g, d: (wl.Q4_K, w, g, d, K, N, T, None)  # noqa: E731
    assert lib.retro_out_prod(*args(W.data_ptr(), G.data_ptr(), out.data_ptr())) == 0
    torch.cuda.synchronize()
    assert lib.retro_out_prod(*args(W.data_ptr() + 4, G.data_ptr(), out.data_ptr())) == q.E_ALIGN
    assert lib.retro_out_prod(*args(W.data_ptr(), G.data_ptr(), big.data_ptr() + 4)) == q.E_ALIGN
    assert lib.retro_out_prod(*args(W.data_ptr(), G.data_ptr(), G.data_ptr())) == q.E_ALIAS
    assert lib.retro_out_prod(*args(W.data_ptr(), G.data_ptr(), W.data_ptr())) == q.E_ALIAS
    assert lib.retro_out_prod(*args(None, G.data_ptr(), out.data_ptr())) == q.E_NULL
    assert lib.retro_out_prod_variant(q.VARIANT_TILE_128x128, *args(W.data_ptr(), G.data_ptr(),
                                                                   out.data_ptr())) == q.E_VARIANT
    with pytest.raises(q.RetroError):
        q.out_prod(wl.Q4_K, W, G, K, variant=q.VARIANT_SKINNY_16)  # T > 16


def test_runs_on_the_given_stream(q):
    c = small_case(wl.Q8_0, 1, 800)
    _, acc, ab = oracle.out_prod(c["type"], c["W"], c["G"], c["K"])
    W, G = dev(c["W"]), dev(c["G"])
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        out = q.out_prod(c["type"], W, G, c["K"])
    s.synchronize()
    check_close(out.cpu().numpy(), acc, ab)


# --- strided operands --------------------------------------------------------------

STRIDED = [(wl.Q4_K, 768, 96, 130), (wl.Q4_0, 512, 77, 200), (wl.F16, 264, 100, 150), (wl.Q6_K, 512, 60, 70),
           (wl.Q8_0, 416, 33, 16), (wl.Q2_K, 256, 40, 9), (wl.Q5_0, 352, 52, 90), (wl.Q5_1, 256, 44, 12),
           (wl.MXFP4, 352, 40, 70), (wl.NVFP4, 320, 40, 70)]


@pytest.mark.parametrize("wtype,K,N,T", STRIDED)
@pytest.mark.parametrize("gpad,wpad", [(4, "48"), (3, "48"), (4, "to16")])
def test_strided_operands_match_oracle(q, wtype, K, N, T, gpad, wpad):
    """G as a column slice of a wider buffer (row stride N + gpad + 4, first
    column 4), dst as a column block of a wider buffer, W rows padded by 48
    bytes or up to a multiple of 16 (a row pitch wider loads fit while the
    rows themselves end off that grid): every kernel that takes the strides
    matches the oracle on the contiguous data, and the rest of dst's buffer
    keeps its sentinel."""
    c = wl.make_case(wtype, N, K, T, seed=900 + N)
    _, acc, ab = oracle.out_prod(wtype, c["W"], c["G"], K, nthreads=ORACLE_THREADS)
    rb = wl.row_bytes(wtype, K)
    ldw = rb + 48 if wpad == "48" else (rb + 15) // 16 * 16
    wbig = torch.zeros((N, ldw), dtype=torch.uint8, device="cuda")
    wbig[:, :rb] = dev(c["W"])
    W = wbig[:, :rb]
    ldg = N + gpad + 4
    gbig = torch.full((T, ldg), float("nan"), device="cuda")
    gbig[:, 4:4 + N] = dev(c["G"])
    G = gbig[:, 4:4 + N]
    ldd = K + 12
    ran = []
    for v in ["auto", "skinny"] + tile_variants(wtype):
        if v != "auto" and not q.variant_applies_strided(variant_id(q, v), wtype, K, N, T, ldw, ldg, ldd):
            continue
        dbig = torch.full((T, ldd), 7.0, device="cuda")
        out = dbig[:, 8:8 + K]
        q.out_prod(wtype, W, G, K, out=out, variant=variant_id(q, v) if v != "auto" else 0)
        torch.cuda.synchronize()
        check_close(out.cpu().numpy(), acc, ab, f"strided {v}")
        rest = dbig.clone()
        rest[:, 8:8 + K] = 7.0
        assert bool((rest == 7.0).all()), v
        ran.append(v)
    families = {v.split("_")[0].rstrip("2") for v in ran if v != "auto"}
    assert "skinny" in families, ran  # the skinny kernel takes any T, in passes of 64 rows of G
    if T > 16:
        assert "tile" in families and (("ws" in families) == (ldg % 4 == 0)), ran


# --- G stored t-fastest (its columns contiguous) -------------------------------------

def g_columns(g, ldg):
    """A T x N view of g whose columns are contiguous: the transpose of an
    N x ldg buffer holding g^T in its first T columns and NaN after them."""
    T, N = g.shape
    big = torch.full((N, ldg), float("nan"), device="cuda")
    big[:, :T] = dev(np.ascontiguousarray(g.T))
    return big[:, :T].t()


GCOLS = [(wl.Q4_K, 768, 96, 130), (wl.Q4_0, 512, 77, 200), (wl.F16, 264, 100, 150), (wl.F32, 301, 64, 70),
         (wl.Q6_K, 512, 60, 70), (wl.Q8_0, 416, 33, 16), (wl.Q2_K, 256, 40, 9), (wl.Q5_1, 256, 44, 12),
         (wl.MXFP4, 352, 40, 70), (wl.NVFP4, 448, 36, 66), (wl.Q3_K, 512, 35, 100), (wl.BF16, 520, 50, 5), (wl.Q5_K, 256, 37, 67),
         (wl.Q4_1, 192, 64, 33), (wl.Q5_0, 352, 29, 16)]


@pytest.mark.parametrize("wtype,K,N,T", GCOLS)
@pytest.mark.parametrize("pad", ["none", "one", "to4"])
def test_g_columns_match_rows_and_oracle(q, wtype, K, N, T, pad):
    """G stored t-fastest (the transpose of an N x ldg buffer, NaN past its
    T values per column; ldg = T, T + 1, or a multiple of 4 past T): every
    kernel that takes the layout matches the oracle on the same G, and is
    bit-identical to the same kernel on G stored by rows (both layouts give
    the kernels the same values in the same order)."""
    c = wl.make_case(wtype, N, K, T, seed=1300 + N)
    _, acc, ab = oracle.out_prod(wtype, c["W"], c["G"], K, nthreads=ORACLE_THREADS)
    ldg = {"none": T, "one": T + 1, "to4": (T + 7) // 4 * 4}[pad]
    rb = wl.row_bytes(wtype, K)
    W, Gc = dev(c["W"]), g_columns(c["G"], ldg)
    assert Gc.stride() == (1, ldg)
    # G by rows, with the row stride rounded up to 4 floats (a layout every
    # kernel takes)
    gbig = torch.full((T, (N + 3) // 4 * 4), float("nan"), device="cuda")
    gbig[:, :N] = dev(c["G"])
    Gr = gbig[:, :N]
    ran = []
    for v in ["auto", "skinny"] + tile_variants(wtype):
        vid = 0 if v == "auto" else variant_id(q, v)
        if v != "auto" and not q.variant_applies_views(vid, wtype, K, N, T, rb, 1, ldg, K):
            continue
        out = torch.full((T, K), float("nan"), device="cuda")
        q.out_prod(wtype, W, Gc, K, out=out, variant=vid)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        check_close(got, acc, ab, f"g columns {v}")
        if v != "auto":
            ref = q.out_prod(wtype, W, Gr, K, variant=vid)
            torch.cuda.synchronize()
            assert np.array_equal(got.view(np.uint32), ref.cpu().numpy().view(np.uint32)), v
        ran.append(v)
    families = {v.split("_")[0].rstrip("2") for v in ran if v != "auto"}
    assert "skinny" in families, ran  # the skinny kernel takes any T, in passes of 64 rows of G
    dense_odd = wtype in (wl.F32, wl.F16, wl.BF16) and K % 4 != 0
    if T > 16:
        assert "tile" in families and (("ws" in families) == (ldg % 4 == 0 and not dense_odd)), ran


# --- exact split on bf16 MFMA (K-quants, opt-in) -------------------------------------

# the exact-split variant of each type it takes: 256-column tiles for the
# K-quants, 128-column tiles for the 32-element block types and 16-bit dense
SPLIT_VARIANT = {**{t: "split_128x256" for t in (wl.Q2_K, wl.Q3_K, wl.Q4_K, wl.Q5_K, wl.Q6_K)},
                 **{t: "split_128x128" for t in (wl.Q4_0, wl.Q5_0, wl.MXFP4, wl.BF16, wl.F16)}}
SPLIT_TYPES = tuple(SPLIT_VARIANT)
SPLIT_SHAPES = [(200, 76, 768), (130, 96, 512), (67, 36, 256), (150, 100, 768), (5, 40, 256), (129, 300, 512)]
# 128-column tiles: K a whole number of blocks but not of tiles (a partial last tile)
NARROW_SHAPES = [(140, 64, 352), (33, 100, 160)]


@pytest.mark.parametrize("T,N,K", SPLIT_SHAPES + NARROW_SHAPES)
@pytest.mark.parametrize("wtype", SPLIT_TYPES)
def test_split_matches_oracle(q, T, N, K, wtype):
    """The exact-split variant against the oracle at the same bars as the
    F32-input kernels, plus: deterministic, and exactly linear in G (G * 2
    doubles every output bit for bit: the parts of fl(2 G d) are twice those
    of fl(G d), and the matrix core's truncation scales with them)."""
    variant = SPLIT_VARIANT[wtype]
    if K % 256 and variant == "split_128x256":
        pytest.skip("K-quant rows are whole super-blocks")
    c = wl.make_case(wtype, N, K, T, seed=1400 + T)
    assert q.variant_applies(variant_id(q, variant), wtype, K, N, T)
    _, acc, ab = oracle.out_prod(wtype, c["W"], c["G"], K, nthreads=ORACLE_THREADS)
    y = run(q, c, variant)
    e = check_close(y, acc, ab, "split")
    assert np.array_equal(run(q, c, variant, prefill=1e30).view(np.uint32), y.view(np.uint32))
    two = run(q, dict(c, G=c["G"] * np.float32(2)), variant)
    assert np.array_equal(two, 2 * y)
    print(f"split {wl.TYPE_NAMES[wtype]} T={T} N={N} K={K}: nmse={e['nmse']:.3e} max_rel={e['max_rel']:.3e}")


@pytest.mark.parametrize("wtype", [wl.Q4_K, wl.Q4_0, wl.MXFP4, wl.BF16])
def test_split_strided_batched_and_empty(q, wtype):
    """Strided G and dst, batches with W broadcast, and N = 0 (the empty sum)."""
    variant = variant_id(q, SPLIT_VARIANT[wtype])
    K, N, T = 512, 70, 90
    cases = [wl.make_case(wtype, N, K, T, seed=1500 + i) for i in range(2)]
    rb = wl.row_bytes(wtype, K)
    W = torch.stack([dev(c["W"]).view(N, rb) for c in cases])          # [2, N, rb]
    g_host = np.stack([c["G"] for c in cases] * 2)                      # 4 batches, W i2 // 2
    gbig = torch.full((4, T, N + 6), float("nan"), device="cuda")
    gbig[:, :, 4:4 + N] = dev(g_host)
    G = gbig[:, :, 4:4 + N]
    dbig = torch.full((4, T, K + 8), 7.0, device="cuda")
    out = dbig[:, :, 4:4 + K]
    # W [1, 2, N, rb] broadcast over G [1, 4, T, N]: batch i2 takes W matrix i2 // 2
    q.out_prod_batched(wtype, W.unsqueeze(0), G.unsqueeze(0), K, out=out.unsqueeze(0), variant=variant)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for i in range(4):
        c = cases[i // 2]
        _, acc, ab = oracle.out_prod(wtype, c["W"], g_host[i], K)
        check_close(got[i], acc, ab, f"split batch {i}")
    rest = dbig.clone()
    rest[:, :, 4:4 + K] = 7.0
    assert bool((rest == 7.0).all())
    # N = 0
    g0 = torch.zeros((9, 4), device="cuda")[:, :0]  # row stride 4: 16-byte rows, as the variant needs
    empty = q.out_prod(wtype, torch.zeros(0, dtype=torch.uint8, device="cuda"), g0, 256, variant=variant)
    torch.cuda.synchronize()
    assert not empty.any()


@pytest.mark.parametrize("name,wtype", [(n, None) for n in (
    "q2_k_n14336_k4096_t4096", "q3_k_n14336_k4096_t4096", "q4_k_n14336_k4096_t4096", "q5_k_n14336_k4096_t4096",
    "q6_k_n14336_k4096_t4096", "q4_0_n17408_k5120_t2048", "q5_0_n17408_k5120_t2048", "mxfp4_n17408_k5120_t2048")] +
    [("dense_n4096_k4096_t512", wl.BF16), ("dense_n4096_k4096_t512", wl.F16)])
def test_split_full_size_sampled_rows(q, name, wtype):
    """The large workloads of every type the exact split takes, through it,
    on sampled rows the oracle computes one by one."""
    c = wl.workload(name, wtype)
    v = variant_id(q, SPLIT_VARIANT[c["type"]])
    W, G = dev(c["W"]), dev(c["G"])
    out = q.out_prod(c["type"], W, G, c["K"], variant=v)
    again = q.out_prod(c["type"], W, G, c["K"], variant=v)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item() and torch.equal(out, again)
    rows = np.unique(np.concatenate([[0, c["T"] - 1], np.random.default_rng(8).integers(0, c["T"], size=14)]))
    _, acc, ab = oracle.out_prod(c["type"], c["W"], c["G"], c["K"], rows=rows, nthreads=ORACLE_THREADS)
    e = check_close(out[torch.from_numpy(rows).cuda()].cpu().numpy(), acc, ab, "split full")
    print(f"split {name}: nmse={e['nmse']:.3e} max_rel={e['max_rel']:.3e}")


# --- batches over two outer dimensions, with W broadcast ------------------------------

BATCHED = [(wl.Q4_K, 512, 64, 40, ["auto", "ws_64x256", "ws_256x256", "tile_64x256"]),
           (wl.Q5_0, 352, 48, 12, ["auto", "skinny", "tile_64x64"]),
           (wl.BF16, 264, 40, 70, ["auto", "ws_32x128", "ws2_64x128", "tile_128x128"])]


def batched_operands(wtype, K, N, T, layout, ne03, ne02, ne3, ne2, seed):
    """W: ne03 x ne02 matrices with rows padded to 16-byte multiples; G: a
    permuted view of ne3 x ne2 matrices (its i3 batches closer than its i2
    ones), each stored by rows or t-fastest. Returns the cases, W, G, the
    host G values [i2][i3] and G's (t, n) strides."""
    rb = wl.row_bytes(wtype, K)
    ldw = (rb + 15) // 16 * 16
    cases = [wl.make_case(wtype, N, K, T, seed=seed + i) for i in range(ne03 * ne02)]
    wbig = torch.zeros((ne03, ne02, N, ldw), dtype=torch.uint8, device="cuda")
    for i, c in enumerate(cases):
        wbig[i // ne02, i % ne02, :, :rb] = dev(c["W"])
    rng = np.random.default_rng(seed + 77)
    g_host = rng.standard_normal((ne2, ne3, T, N)).astype(np.float32)
    if layout == "rows":
        G = dev(g_host).permute(1, 0, 2, 3)              # [ne3, ne2, T, N], not contiguous
    else:
        G = dev(np.ascontiguousarray(g_host.transpose(0, 1, 3, 2))).permute(1, 0, 3, 2)
        assert G.stride(2) == 1
    sgt, sgn = (N, 1) if layout == "rows" else (1, T)
    return cases, wbig, G, g_host, ldw, sgt, sgn


def check_batches(q, wtype, K, T, cases, wbig, G, g_host, ne03, ne02, ne3, ne2, variant, label):
    """Run out_prod_batched into dst matrices with gaps; every batch must
    match the oracle on its own pair of matrices, and the gaps keep their
    sentinel."""
    dbig = torch.full((ne3, ne2, T + 1, K + 4), 7.0, device="cuda")
    out = dbig[:, :, :T, :K]
    q.out_prod_batched(wtype, wbig, G, K, out=out, variant=variant)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for i3 in range(ne3):
        for i2 in range(ne2):
            c = cases[(i3 // (ne3 // ne03)) * ne02 + i2 // (ne2 // ne02)]
            _, acc, ab = oracle.out_prod(wtype, c["W"], g_host[i2, i3], K, nthreads=ORACLE_THREADS)
            check_close(got[i3, i2], acc, ab, f"batch {i3},{i2} {label}")
    rest = dbig.clone()
    rest[:, :, :T, :K] = 7.0
    assert bool((rest == 7.0).all()), label


@pytest.mark.parametrize("wtype,K,N,T,variants", BATCHED)
@pytest.mark.parametrize("layout", ["rows", "columns"])
def test_batched_broadcast_matches_oracle(q, wtype, K, N, T, variants, layout):
    """dst[i3][i2] = out_prod(W[i3 / 2][i2 / 2], G[i3][i2]) over 2 x 4 batches
    with 1 x 2 W matrices; W rows padded to 16-byte multiples, G a permuted
    view (its i3 batches closer than its i2 ones; each matrix stored by rows
    or t-fastest), dst matrices with gaps. Every batch matches the oracle on
    its own pair of matrices, and the gaps of dst keep their sentinel."""
    ne03, ne02, ne3, ne2 = 1, 2, 2, 4
    cases, wbig, G, g_host, ldw, sgt, sgn = batched_operands(wtype, K, N, T, layout, ne03, ne02, ne3, ne2, 1200)
    for v in variants:
        if v != "auto" and not q.variant_applies_views(variant_id(q, v), wtype, K, N, T, ldw, sgt, sgn, K):
            continue
        check_batches(q, wtype, K, T, cases, wbig, G, g_host, ne03, ne02, ne3, ne2,
                      variant_id(q, v) if v != "auto" else 0, v)


@pytest.mark.parametrize("wtype", [wl.Q4_0, wl.BF16, wl.MXFP4])
@pytest.mark.parametrize("layout", ["rows", "columns"])
def test_batched_two_launch_plan_matches_oracle(q, wtype, layout):
    """16 matrices of 200 x 1280 with N = 2048: their tiles fill whole rounds
    of 128 x 128 on 1024 columns, so the automatic choice runs two launches
    over column ranges of every dst matrix; W broadcast 2 x 4 times, G
    permuted, dst with gaps."""
    K, N, T = 1280, 2048, 200
    ne03, ne02, ne3, ne2 = 1, 2, 4, 4
    cases, wbig, G, g_host, ldw, sgt, sgn = batched_operands(wtype, K, N, T, layout, ne03, ne02, ne3, ne2, 1400)
    v0, ks, v1 = q.views_plan(wtype, K, N, T, ldw, sgt, sgn, K + 4, ne2, ne3)
    assert ks < K, (v0, ks, v1)
    print(f"plan {q.VARIANT_NAMES[v0]}[0:{ks}] + {q.VARIANT_NAMES[v1]}[{ks}:{K}]", flush=True)
    check_batches(q, wtype, K, T, cases, wbig, G, g_host, ne03, ne02, ne3, ne2, 0, "auto")


def test_batched_empty_and_single(q):
    """No batches is a no-op; one batch equals retro_out_prod."""
    c = wl.make_case(wl.Q4_0, 33, 256, 20, seed=5)
    W, G = dev(c["W"]).view(33, -1), dev(c["G"])
    ref = run(q, c)
    one = q.out_prod_batched(wl.Q4_0, W, G, 256)
    torch.cuda.synchronize()
    assert np.array_equal(one.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    empty = torch.zeros((0, 20, 256), device="cuda")
    q.out_prod_batched(wl.Q4_0, W, G.unsqueeze(0)[:0], 256, out=empty)


# --- two launches over column ranges of dst ---------------------------------------

# (type, K, N, T, k_split, variant0, variant1): ragged T, N and parts, both
# kernel families, the skinny kernel and the exact splits
COLUMN_SPLITS = [
    (wl.Q4_0, 640, 100, 200, 512, "ws_128x256", "ws2_64x128"),
    (wl.Q4_K, 768, 96, 130, 256, "ws_256x256", "ws_32x256"),
    (wl.Q4_K, 1024, 64, 67, 768, "ws_128x256", "tile_64x256"),
    (wl.F16, 520, 76, 150, 256, "ws_128x128", "tile_64x64"),
    (wl.MXFP4, 640, 36, 90, 512, "ws_64x256", "ws_32x128"),
    (wl.Q8_0, 512, 40, 16, 256, "skinny", "skinny"),
    (wl.F32, 300, 64, 70, 128, "auto", "auto"),
    (wl.NVFP4, 448, 48, 100, 256, "ws_128x256", "ws_64x128"),
    (wl.Q5_K, 768, 60, 70, 512, "split_128x256", "ws_32x256"),
    (wl.BF16, 520, 40, 33, 256, "split_128x128", "ws_32x128"),
]


@pytest.mark.parametrize("wtype,K,N,T,ks,v0,v1", COLUMN_SPLITS)
def test_column_split_matches_parts_and_oracle(q, wtype, K, N, T, ks, v0, v1):
    """retro_out_prod_column_split: the whole dst (NaN-prefilled) within the
    bars of the oracle, and each column range bit-identical to its variant
    run alone on those columns of W."""
    c = wl.make_case(wtype, N, K, T, seed=1300 + K + N)
    ids = [q.VARIANT_AUTO if v == "auto" else variant_id(q, v) for v in (v0, v1)]
    W, G = dev(c["W"]), dev(c["G"])
    out = torch.full((T, K), float("nan"), device="cuda")
    q.out_prod_column_split(wtype, W, G, K, ids[0], ks, ids[1], out=out)
    torch.cuda.synchronize()
    y = out.cpu().numpy()
    _, acc, ab = oracle.out_prod(wtype, c["W"], c["G"], K, nthreads=ORACLE_THREADS)
    check_close(y, acc, ab, f"{v0}+{v1}")
    rb, off = wl.row_bytes(wtype, K), wl.row_bytes(wtype, ks)
    rows = np.asarray(c["W"]).reshape(N, rb)
    parts = [dict(c, W=np.ascontiguousarray(rows[:, :off]), K=ks), dict(c, W=np.ascontiguousarray(rows[:, off:]),
                                                                      K=K - ks)]
    for part, v, cols in zip(parts, (v0, v1), (slice(0, ks), slice(ks, K))):
        assert applies(q, part, v), v
        assert same_bits(y[:, cols], run(q, part, v)), v


# --- full-size workloads ----------------------------------------------------------

# The five benchmarked workloads (the dense one in its three storage types):
# every output is compared with the oracle.
FIVE = [
    ("q8_0_n128_k256_t64", None),
    ("dense_n4096_k4096_t512", wl.F32),
    ("dense_n4096_k4096_t512", wl.F16),
    ("dense_n4096_k4096_t512", wl.BF16),
    ("q4_0_n17408_k5120_t2048", None),
    ("q4_k_n14336_k4096_t4096", None),
    ("q4_k_n4096_k14336_t16", None),
]
# The other types at the same shapes: sampled rows.
FULL = [
    ("q5_k_n14336_k4096_t4096", None),
    ("q6_k_n14336_k4096_t4096", None),
    ("q5_k_n4096_k14336_t16", None),
    ("q6_k_n4096_k14336_t16", None),
    ("q2_k_n14336_k4096_t4096", None),
    ("q3_k_n14336_k4096_t4096", None),
    ("q2_k_n4096_k14336_t16", None),
    ("q3_k_n4096_k14336_t16", None),
    ("q4_1_n17408_k5120_t2048", None),
    ("q5_0_n17408_k5120_t2048", None),
    ("q5_1_n17408_k5120_t2048", None),
    ("mxfp4_n17408_k5120_t2048", None),
    ("nvfp4_n17408_k5120_t2048", None),
    ("nvfp4_n4096_k14336_t16", None),
]


@pytest.mark.parametrize("name,wtype", FIVE)
def test_full_size_whole_output(q, name, wtype):
    """The launch configuration the benchmark times, every output compared
    with the oracle element by element (NMSE over the whole output, the
    relative error of each output), then determinism of a second call."""
    c = wl.workload(name, wtype)
    print(f"{name} {wl.TYPE_NAMES[c['type']]}: kernel {q.plan_names(c['type'], c['K'], c['N'], c['T'])}", flush=True)
    W, G = dev(c["W"]), dev(c["G"])
    out = torch.full((c["T"], c["K"]), float("nan"), device="cuda")
    q.out_prod(c["type"], W, G, c["K"], out=out)
    again = q.out_prod(c["type"], W, G, c["K"])
    torch.cuda.synchronize()
    assert torch.equal(out, again)
    y = out.cpu().numpy()
    del W, G, out, again
    _, acc, ab = oracle.out_prod(c["type"], c["W"], c["G"], c["K"], nthreads=ORACLE_THREADS)
    e = check_close(y, acc, ab, name)
    print(f"{name} {wl.TYPE_NAMES[c['type']]}: {y.size} outputs, nmse={e['nmse']:.3e} max_rel={e['max_rel']:.3e}")


@pytest.mark.parametrize("name,wtype", FULL)
def test_full_size_sampled_rows(q, name, wtype):
    """The other types at the benchmarked shapes, checked on sampled t rows
    that the oracle computes one by one (first, last and random rows), plus
    whole-output properties: all finite, deterministic."""
    c = wl.workload(name, wtype)
    W, G = dev(c["W"]), dev(c["G"])
    out = torch.full((c["T"], c["K"]), float("nan"), device="cuda")
    q.out_prod(c["type"], W, G, c["K"], out=out)
    again = q.out_prod(c["type"], W, G, c["K"])
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()
    assert torch.equal(out, again)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, c["T"] - 1], rng.integers(0, c["T"], size=14)]))
    _, acc, ab = oracle.out_prod(c["type"], c["W"], c["G"], c["K"], rows=rows, nthreads=ORACLE_THREADS)
    y = out[torch.from_numpy(rows).cuda()].cpu().numpy()
    e = check_close(y, acc, ab, name)
    print(f"{name} {wl.TYPE_NAMES[c['type']]}: nmse={e['nmse']:.3e} max_rel={e['max_rel']:.3e}")


@pytest.mark.parametrize("name,wtype", [("q4_k_n14336_k4096_t4096", None), ("q4_k_n4096_k14336_t16", None),
                                        ("q4_0_n17408_k5120_t2048", None), ("dense_n4096_k4096_t512", wl.BF16)])
def test_full_size_g_columns(q, name, wtype):
    """The benchmarked shapes with G stored t-fastest (the transpose of a
    contiguous N x T tensor, as ggml's OUT_PROD gets a contiguous src1): the
    same kernel is chosen and the whole output is bit-identical to the one
    from G stored by rows."""
    c = wl.workload(name, wtype)
    K, N, T = c["K"], c["N"], c["T"]
    rb = wl.row_bytes(c["type"], K)
    assert q.choice_views(c["type"], K, N, T, rb, 1, T, K) == q.choice(c["type"], K, N, T)
    W, Gr = dev(c["W"]), dev(c["G"])
    Gc = Gr.t().contiguous().t()
    a = q.out_prod(c["type"], W, Gr, K)
    b = q.out_prod(c["type"], W, Gc, K)
    torch.cuda.synchronize()
    assert torch.isfinite(b).all().item()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    del Gc


@pytest.mark.parametrize("name", ["q4_0_n17408_k5120_t2048", "q4_k_n14336_k4096_t4096", "q4_k_n4096_k14336_t16",
                                  "q5_k_n14336_k4096_t4096", "q6_k_n14336_k4096_t4096", "q6_k_n4096_k14336_t16",
                                  "q2_k_n14336_k4096_t4096", "q3_k_n14336_k4096_t4096", "q3_k_n4096_k14336_t16",
                                  "q5_0_n17408_k5120_t2048", "mxfp4_n17408_k5120_t2048"])
def test_full_size_decode_through_identity(q, name):
    """Full-size W through the benchmarked kernel with G = I (T = N): the
    output is the decoded W, bit for bit."""
    c = wl.workload(name)
    N, K = c["N"], c["K"]
    ref = oracle.dequantize(c["type"], c["W"], K)
    W = dev(c["W"])
    variant, ks, v1 = q.plan(c["type"], K, N, c["T"])
    if ks < K:
        # the two launches of the benchmarked call, each over its columns
        out = q.out_prod_column_split(c["type"], W, torch.eye(N, device="cuda"), K, variant, ks, v1)
        assert np.array_equal(out.cpu().numpy(), ref)
    elif variant == q.VARIANT_SKINNY:
        # T = N would leave the skinny range; check 16-row slices of W instead
        for n0 in range(0, N, N // 8):
            sl = slice(n0, n0 + 16)
            out = q.out_prod(c["type"], W[sl], torch.eye(16, device="cuda"), K, variant=variant)
            assert np.array_equal(out.cpu().numpy(), ref[sl]), n0
    else:
        out = q.out_prod(c["type"], W, torch.eye(N, device="cuda"), K, variant=variant)
        assert np.array_equal(out.cpu().numpy(), ref)
