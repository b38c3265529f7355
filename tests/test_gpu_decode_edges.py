"""Device decode of the hand-derived blocks and of the edge cases of every
block format, through retro_dequantize and through every kernel family.

The oracle's decoders are pinned by the fixtures in tests/golden (see
test_oracle_pins.py). Here the same blocks, and blocks whose scales sit at
the ends of their formats, go through the device:
  * retro_dequantize, compared element by element with the fixture values
    and with the oracle;
  * every out_prod kernel that takes the type (skinny, single-role tile,
    producer/consumer, exact split) and the forward mul_mat kernels, with a
    gradient that selects one row of W, so the output is that row's decoded
    values.
The bar is the decode contract: the same bits as the oracle, NaN compared
by class. Zeros are compared by value (+0 == -0) only because a kernel adds
zero products to the selected weight (-0 + 0 = +0); retro_dequantize keeps
the sign of every zero. The Retrograd "CUDA status" page sets
exact equality of device and CPU results as the bar for the base-weight
conversions (section "Base weights in F16 and BF16"); the llama.cpp PR
"cuda: out_prod accepts a quantized src0" checks OUT_PROD against the CPU
backend (section "Measured").

Selecting a row instead of using G = I keeps non-finite weights apart: with
G = I, the zero entries of G would meet an infinite weight of another row
and give 0 * inf = NaN. With a one-hot gradient row every other row of W is
finite and multiplied by zero, so each output is w * 1 plus zeros.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from blocks import golden_blocks

pytestmark = pytest.mark.gpu

TYPES = [wl.F32, wl.F16, wl.BF16, wl.Q8_0, wl.Q4_0, wl.Q4_1, wl.Q5_0, wl.Q5_1, wl.MXFP4, wl.NVFP4, wl.Q2_K, wl.Q3_K,
         wl.Q4_K, wl.Q5_K, wl.Q6_K]
KQUANTS = (wl.Q2_K, wl.Q3_K, wl.Q4_K, wl.Q5_K, wl.Q6_K)
OUT_PROD_VARIANTS = ["skinny", "skinny_8", "skinny_16", "tile_128x128", "tile_128x256", "tile_64x128", "tile_64x64", "tile_64x256",
                     "ws_256x256", "ws_128x256", "ws_64x256", "ws_128x128", "ws_64x128", "ws_32x256", "ws_32x128",
                     "ws2_64x128",
                     "split_128x256", "split_128x128"]
MUL_MAT_VARIANTS = ["skinny", "ws_256x128", "ws_128x128", "ws_64x128", "ws_32x128", "simple"]

# Byte offsets of the fp16 scale fields in one block (d first; then the
# second field: dmin for the K-quants with sub-mins, the offset m for Q4_1
# and Q5_1).
HALF_FIELDS = {
    wl.Q8_0: (0,), wl.Q4_0: (0,), wl.Q5_0: (0,), wl.Q4_1: (0, 2), wl.Q5_1: (0, 2),
    wl.Q2_K: (80, 82), wl.Q3_K: (108,), wl.Q4_K: (0, 2), wl.Q5_K: (0, 2), wl.Q6_K: (208,),
}
BLOCK = {wl.Q8_0: (32, 34), wl.Q4_0: (32, 18), wl.Q4_1: (32, 20), wl.Q5_0: (32, 22), wl.Q5_1: (32, 24),
         wl.MXFP4: (32, 17), wl.NVFP4: (64, 36), wl.Q2_K: (256, 84), wl.Q3_K: (256, 110), wl.Q4_K: (256, 144), wl.Q5_K: (256, 176),
         wl.Q6_K: (256, 210)}
# binary16 patterns at the ends of the format: the smallest and largest
# subnormals (both signs), zeros, the largest normal, infinities, NaNs
SPECIAL_HALVES = (0x0001, 0x8001, 0x03FF, 0x83FF, 0x0400, 0x0000, 0x8000, 0x7BFF, 0xFBFF, 0x7C00, 0xFC00, 0x7E00,
                  0xFE00, 0x7C01)
# E8M0 scales at the ends (e = 0: the subnormal 2^-127; e = 1: 2^-126, whose
# half-size codes are subnormal; 254: overflow of the larger codes; 255: NaN)
SPECIAL_E8M0 = (0, 1, 2, 126, 127, 128, 253, 254, 255)


@pytest.fixture(scope="module")
def q():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import quantized_weight_backward_amd as q

    return q


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def mismatches(got, want):
    """Indices where got and want differ under the decode contract: NaN by
    class, zeros by value, every other value by its bits."""
    got = np.asarray(got, np.float32).ravel()
    want = np.asarray(want, np.float32).ravel()
    gn, wn = np.isnan(got), np.isnan(want)
    same = np.where(wn | gn, gn == wn, (got.view(np.uint32) == want.view(np.uint32)) | ((got == 0) & (want == 0)))
    return np.nonzero(~same)[0]


def assert_decode(got, want, label, signed_zeros=False):
    bad = mismatches(got, want)
    if signed_zeros:
        g, w = np.asarray(got, np.float32).ravel(), np.asarray(want, np.float32).ravel()
        bad = np.union1d(bad, np.nonzero((g == 0) & (w == 0) & (np.signbit(g) != np.signbit(w)))[0])
    if len(bad):
        g = np.asarray(got, np.float32).ravel()
        w = np.asarray(want, np.float32).ravel()
        shown = ", ".join(f"[{i}] {g[i]!r} != {w[i]!r}" for i in bad[:6])
        raise AssertionError(f"{label}: {len(bad)} of {w.size} elements differ: {shown}")


def out_prod_variants(q, wtype, K, N, T):
    ids = {v: k for k, v in q.VARIANT_NAMES.items()}
    return [v for v in OUT_PROD_VARIANTS if q.variant_applies(ids[v], wtype, K, N, T)]


def mul_mat_variants(q, wtype, K, N, T):
    ids = {v: k for k, v in q.VARIANT_NAMES.items()}
    return [v for v in MUL_MAT_VARIANTS if q.mul_mat_variant_applies(ids[v], wtype, K, N, T)]


def filler_rows(wtype, K, n, seed):
    """n rows of finite random blocks (the workloads' own generator)."""
    return wl.make_case(wtype, n, K, 1, seed)["W"].reshape(n, -1)


def through_every_kernel(q, wtype, row, K, label, split=True):
    """Put `row` (one packed W row) at row 0 and at row 3 of a 4-row W with
    finite filler rows; a one-hot gradient row picks it out. Every out_prod
    kernel that takes the shape must return the oracle's decode of `row`."""
    want = oracle.dequantize(wtype, row, K)[0]
    fill = filler_rows(wtype, K, 3, seed=K + wtype)
    ids = {v: k for k, v in q.VARIANT_NAMES.items()}
    checked = []
    for pos in (0, 3):
        W = np.concatenate([fill[:pos], row.reshape(1, -1), fill[pos:]])
        G = np.zeros((1, 4), np.float32)
        G[0, pos] = 1.0
        Wd, Gd = dev(W), dev(G)
        for v in out_prod_variants(q, wtype, K, 4, 1):
            if v.startswith("split") and not split:
                continue
            out = torch.full((1, K), 12345.0, device="cuda")
            q.out_prod(wtype, Wd, Gd, K, out=out, variant=ids[v])
            torch.cuda.synchronize()
            assert_decode(out.cpu().numpy()[0], want, f"{label} out_prod {v} row {pos}")
            checked.append(v)
    return checked


# --- the golden blocks ------------------------------------------------------------

def test_golden_blocks_dequantize(q, golden):
    """Every hand-derived block of tests/golden decodes on the device to the
    fixture's values (with their signs, zeros included) and to the oracle's
    decode of every element."""
    blocks = golden_blocks(golden)
    assert {b[1] for b in blocks} == set(BLOCK)  # every block format has a fixture
    for label, wtype, K, raw, expected in blocks:
        got = q.dequantize(wtype, dev(raw), K, 1).cpu().numpy()[0]
        for e, v in expected.items():
            want = np.float32(v)
            if np.isnan(want):
                assert np.isnan(got[e]), (label, e)
            else:
                assert got[e] == want, (label, e, got[e], want)
        assert_decode(got, oracle.dequantize(wtype, raw, K)[0], label, signed_zeros=True)


def test_golden_blocks_through_every_kernel(q, golden):
    """The same blocks through every out_prod kernel and every mul_mat kernel
    that takes the type. Finite blocks also go through G = I (T = N = 16, and
    T = N = 48 for the tiled kernels), so that each block sits in several
    rows and lanes of a tile."""
    by_type = {}
    for label, wtype, K, raw, _ in golden_blocks(golden):
        by_type.setdefault(wtype, []).append((label, K, raw))
    ids = {v: k for k, v in q.VARIANT_NAMES.items()}
    for wtype, items in by_type.items():
        for label, K, raw in items:
            # the exact split (opt-in) takes finite weights only: its products
            # of operand parts meet an infinite weight with zero parts
            finite = bool(np.isfinite(oracle.dequantize(wtype, raw, K)).all())
            through_every_kernel(q, wtype, raw, K, label, split=finite)
        finite = [raw for label, K, raw in items if np.isfinite(oracle.dequantize(wtype, raw, K)).all()]
        K = items[0][1]
        for N in (16, 48):
            W = np.stack([finite[i % len(finite)] for i in range(N)])
            want = oracle.dequantize(wtype, W, K)
            Wd, I = dev(W), torch.eye(N, device="cuda")
            for v in out_prod_variants(q, wtype, K, N, N):
                out = q.out_prod(wtype, Wd, I, K, variant=ids[v])
                torch.cuda.synchronize()
                assert_decode(out.cpu().numpy(), want, f"{wl.TYPE_NAMES[wtype]} G=I N={N} {v}")
            # forward: Y = X W^T with X = I_K gives W^T
            X = torch.eye(K, device="cuda")
            for v in mul_mat_variants(q, wtype, K, N, K):
                y = q.mul_mat(wtype, Wd, X, N=N, variant=ids[v])
                torch.cuda.synchronize()
                assert_decode(y.cpu().numpy().T, want, f"{wl.TYPE_NAMES[wtype]} mul_mat X=I N={N} {v}")


# --- scales at the ends of their formats ---------------------------------------------

def special_scale_row(wtype, seed=11, halves=SPECIAL_HALVES):
    """One W row of blocks whose fp16 scale fields take the `halves`
    patterns: each field alone (the others random), then every field at once.
    The codes are random, so every code value meets every special scale."""
    blk_elems, blk_bytes = BLOCK[wtype]
    fields = HALF_FIELDS[wtype]
    combos = [(f,) for f in fields] + ([fields] if len(fields) > 1 else [])
    nblk = len(halves) * len(combos) * 2
    K = nblk * blk_elems
    row = wl.make_case(wtype, 1, K, 1, seed)["W"].reshape(-1, blk_bytes).copy()
    i = 0
    for fs in combos:
        for h in halves:
            for _rep in range(2):  # two blocks each: different random codes and other fields
                for f in fs:
                    row[i, f:f + 2] = [h & 255, h >> 8]
                i += 1
    assert i == nblk
    return row.reshape(-1), K


@pytest.mark.parametrize("wtype", sorted(HALF_FIELDS))
def test_special_fp16_scales(q, wtype):
    """fp16 scales and offsets that are subnormal, zero, the largest normal,
    infinite or NaN: the device decode follows the formats' formulas under
    IEEE arithmetic exactly as the oracle does (inf * 0 = NaN, inf - inf =
    NaN, subnormal scales exact), in retro_dequantize and in every kernel."""
    row, K = special_scale_row(wtype)
    want = oracle.dequantize(wtype, row, K)[0]
    assert np.isnan(want).any() and np.isinf(want).any()  # the row reaches the non-finite cases
    got = q.dequantize(wtype, dev(row), K, 1).cpu().numpy()[0]
    assert_decode(got, want, f"{wl.TYPE_NAMES[wtype]} dequantize", signed_zeros=True)
    checked = through_every_kernel(q, wtype, row, K, wl.TYPE_NAMES[wtype], split=False)
    assert "skinny" in checked and any(v.startswith("ws") for v in checked) and any(
        v.startswith("tile") for v in checked), checked


def mxfp4_scale_row():
    """For each E8M0 scale in SPECIAL_E8M0, 16 blocks whose 256 code bytes
    are 0..255: every nibble pair under every end of the scale range."""
    blocks = []
    for e in SPECIAL_E8M0:
        for b in range(16):
            blocks.append(np.concatenate([[e], np.arange(16 * b, 16 * b + 16)]).astype(np.uint8))
    return np.concatenate(blocks), 32 * len(blocks)


def test_mxfp4_scale_ends(q):
    """MXFP4 with E8M0 scales 2^-127 (a subnormal F32 scale), 2^-126, 2^127
    (the larger codes overflow to inf) and NaN, every code byte: the device
    decode (the hardware's scaled FP4 conversion) equals the oracle's E2M1
    times 2^(e - 127) with one IEEE rounding, in retro_dequantize and in
    every kernel."""
    row, K = mxfp4_scale_row()
    want = oracle.dequantize(wl.MXFP4, row, K)[0]
    assert np.isinf(want).any() and np.isnan(want).any()
    assert ((want != 0) & (np.abs(want) < np.float32(2.0 ** -126))).any()  # subnormal values present
    got = q.dequantize(wl.MXFP4, dev(row), K, 1).cpu().numpy()[0]
    assert_decode(got, want, "mxfp4 dequantize", signed_zeros=True)
    through_every_kernel(q, wl.MXFP4, row, K, "mxfp4", split=False)


def test_mxfp4_normal_scale_ends_through_split(q):
    """The exact split (opt-in) on MXFP4 takes the E2M1 value times its
    scale as one bf16 operand: exact for every scale whose values are finite
    (e <= 252; at e = 253 the code 6 overflows), subnormal values (e = 0, 1)
    included."""
    blocks = []
    for e in (0, 1, 2, 3, 126, 127, 128, 251, 252):
        for b in range(16):
            blocks.append(np.concatenate([[e], np.arange(16 * b, 16 * b + 16)]).astype(np.uint8))
    row = np.concatenate(blocks)
    K = 32 * len(blocks)
    want = oracle.dequantize(wl.MXFP4, row, K)[0]
    assert np.isfinite(want).all()
    fill = filler_rows(wl.MXFP4, K, 3, seed=5)
    ids = {v: k for k, v in q.VARIANT_NAMES.items()}
    W = dev(np.concatenate([row.reshape(1, -1), fill]))
    G = torch.zeros((1, 4), device="cuda")
    G[0, 0] = 1.0
    assert q.variant_applies(ids["split_128x128"], wl.MXFP4, K, 4, 1)
    out = q.out_prod(wl.MXFP4, W, G, K, variant=ids["split_128x128"])
    torch.cuda.synchronize()
    assert_decode(out.cpu().numpy()[0], want, "mxfp4 split_128x128")


def nvfp4_scale_row():
    """Every E4M3 scale byte (the four scales of a block take four of them)
    over code bytes that run through all 256 values: 64 blocks."""
    blocks = np.zeros((64, 36), dtype=np.uint8)
    blocks[:, 0:4] = np.arange(256, dtype=np.uint8).reshape(64, 4)
    blocks[:, 4:] = (np.arange(64 * 32) * 37 % 256).astype(np.uint8).reshape(64, 32)
    return blocks.reshape(-1), 64 * 64


def test_nvfp4_every_scale_byte(q):
    """NVFP4 with every E4M3 scale byte (zeros of either sign, subnormals, the
    largest, NaN) and every code: the device decode equals the oracle's E2M1
    times the E4M3 scale, in retro_dequantize and in every kernel."""
    row, K = nvfp4_scale_row()
    want = oracle.dequantize(wl.NVFP4, row, K)[0]
    assert np.isnan(want).any() and ((want != 0) & (np.abs(want) < 2.0 ** -6)).any()
    got = q.dequantize(wl.NVFP4, dev(row), K, 1).cpu().numpy()[0]
    assert_decode(got, want, "nvfp4 dequantize", signed_zeros=True)
    checked = through_every_kernel(q, wl.NVFP4, row, K, "nvfp4", split=False)
    assert "skinny" in checked and "ws_128x256" in checked and "tile_64x64" in checked, checked


@pytest.mark.parametrize("wtype", [wl.F16, wl.BF16])
def test_every_16_bit_pattern(q, wtype):
    """All 65536 binary16 / bfloat16 patterns in one row: subnormals, zeros,
    infinities and NaNs decode on the device as the oracle decodes them,
    through retro_dequantize and every kernel."""
    row = np.arange(65536, dtype=np.uint16).view(np.uint8)
    K = 65536
    want = oracle.dequantize(wtype, row, K)[0]
    got = q.dequantize(wtype, dev(row), K, 1).cpu().numpy()[0]
    assert_decode(got, want, f"{wl.TYPE_NAMES[wtype]} dequantize", signed_zeros=True)
    through_every_kernel(q, wtype, row, K, wl.TYPE_NAMES[wtype], split=False)


def test_f32_special_values(q):
    """F32 weights that are subnormal, zero, the largest finite, infinite or
    NaN pass through every kernel unchanged (times one, plus zeros)."""
    vals = np.array([2.0 ** -149, -2.0 ** -149, 2.0 ** -127, 3 * 2.0 ** -130, 2.0 ** -126, 0.0, -0.0,
                     np.finfo(np.float32).max, -np.finfo(np.float32).max, np.inf, -np.inf, np.nan, 1.0, -2.5],
                    dtype=np.float32)
    row = np.resize(vals, 1024).astype(np.float32)
    K = row.size
    want = oracle.dequantize(wl.F32, row.view(np.uint8), K)[0]
    got = q.dequantize(wl.F32, dev(row.view(np.uint8)), K, 1).cpu().numpy()[0]
    assert_decode(got, want, "f32 dequantize", signed_zeros=True)
    through_every_kernel(q, wl.F32, row.view(np.uint8), K, "f32", split=False)


SPLIT_TYPES = {wl.Q2_K: "split_128x256", wl.Q3_K: "split_128x256", wl.Q4_K: "split_128x256",
               wl.Q5_K: "split_128x256", wl.Q6_K: "split_128x256", wl.Q4_0: "split_128x128",
               wl.Q5_0: "split_128x128"}


@pytest.mark.parametrize("wtype", sorted(SPLIT_TYPES))
def test_finite_special_scales_through_split(q, wtype):
    """The exact split (opt-in) with the finite ends of the fp16 scales
    (subnormal, zero, the largest normal): its exact products give the
    decoded weight bit for bit, as the F32-input kernels do."""
    finite = tuple(h for h in SPECIAL_HALVES if (h & 0x7C00) != 0x7C00)
    row, K = special_scale_row(wtype, halves=finite)
    want = oracle.dequantize(wtype, row, K)[0]
    assert np.isfinite(want).all()
    fill = filler_rows(wtype, K, 3, seed=9)
    ids = {v: k for k, v in q.VARIANT_NAMES.items()}
    v = SPLIT_TYPES[wtype]
    assert q.variant_applies(ids[v], wtype, K, 4, 1)
    for pos in (0, 3):
        W = dev(np.concatenate([fill[:pos], row.reshape(1, -1), fill[pos:]]))
        G = torch.zeros((1, 4), device="cuda")
        G[0, pos] = 1.0
        out = q.out_prod(wtype, W, G, K, variant=ids[v])
        torch.cuda.synchronize()
        assert_decode(out.cpu().numpy()[0], want, f"{wl.TYPE_NAMES[wtype]} {v} row {pos}")
