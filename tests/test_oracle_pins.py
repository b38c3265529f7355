"""Pins of the CPU oracle to facts outside itself (no GPU).

Every check compares the oracle with something it does not compute: an
independent library routine (numpy binary16, torch bfloat16, numpy matmul,
torch autograd), hand-derived fixture values (tests/golden), closed forms,
or a brute force in a different loop order. Each is chosen so that a
plausible slip in the oracle (a swapped nibble, a dropped sub-scale bit, a
wrong sign, a transposed operand, a dropped term) fails at least one.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

TYPES = [wl.F32, wl.F16, wl.BF16, wl.Q8_0, wl.Q4_0, wl.Q4_K]


def hexbytes(tokens):
    return np.array([int(t, 16) for t in tokens], dtype=np.uint8)


# --- element decoders -------------------------------------------------------

def test_half_to_float_matches_numpy_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    mine = oracle.half_to_float(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan].view(np.uint32), ref[~nan].view(np.uint32))  # -0 and +0 distinct


def test_bf16_to_float_matches_torch_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    mine = oracle.bf16_to_float(bits)
    ref = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_dense_rows_decode_to_library_values():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(77) * 3).astype(np.float32)
    assert np.array_equal(oracle.dequantize(wl.F32, x.view(np.uint8), 77)[0].view(np.uint32), x.view(np.uint32))
    h = x.astype(np.float16)
    assert np.array_equal(oracle.dequantize(wl.F16, h.view(np.uint8), 77)[0], h.astype(np.float32))
    b = torch.from_numpy(x).bfloat16()
    got = oracle.dequantize(wl.BF16, b.view(torch.int16).numpy().view(np.uint8), 77)[0]
    assert np.array_equal(got, b.float().numpy())


# --- block decoders against hand-derived fixtures ---------------------------

@pytest.mark.parametrize("fixture,wtype", [("q8_0_blocks.txt", wl.Q8_0), ("q4_0_blocks.txt", wl.Q4_0)])
def test_hand_built_blocks(golden, fixture, wtype):
    g = golden(fixture)
    names = sorted(k[:-4] for k in g if k.endswith("_hex"))
    assert names
    for name in names:
        raw = hexbytes(g[name + "_hex"])
        expected = np.array([float(v) for v in g[name + "_expected"]], dtype=np.float32)
        got = oracle.dequantize(wtype, raw, 32)[0]
        assert np.array_equal(got, expected), name
        # signs of zero too (d < 0 times a zero code is -0)
        assert np.array_equal(np.signbit(got), np.signbit(expected)), name


def pack_q4_k_field(sc, m):
    """GGUF Q4_K sub-scale/sub-min packing, written for the tests (the oracle only unpacks)."""
    s = [0] * 12
    for j in range(4):
        s[j] = (sc[j] & 63) | ((sc[j + 4] >> 4) << 6)
        s[j + 4] = (m[j] & 63) | ((m[j + 4] >> 4) << 6)
        s[j + 8] = (sc[j + 4] & 15) | ((m[j + 4] & 15) << 4)
    return np.array(s, dtype=np.uint8)


def q4_k_superblock(d_bits, dmin_bits, field, codes):
    blk = np.zeros(144, dtype=np.uint8)
    blk[0:2] = np.array([d_bits & 255, d_bits >> 8], dtype=np.uint8)
    blk[2:4] = np.array([dmin_bits & 255, dmin_bits >> 8], dtype=np.uint8)
    blk[4:16] = field
    blk[16:144] = codes
    return blk


def test_q4_k_field_packer_matches_hand_packing(golden):
    g = golden("q4_k_pack.txt")
    sc = [int(v) for v in g["sc"]]
    m = [int(v) for v in g["m"]]
    assert np.array_equal(pack_q4_k_field(sc, m), hexbytes(g["field_hex"]))


def test_q4_k_hand_built_superblock(golden):
    g = golden("q4_k_pack.txt")
    sc = [int(v) for v in g["sc"]]
    m = [int(v) for v in g["m"]]
    i = np.arange(128)
    codes = (((i * 7 + 3) & 15) | (((i * 5 + 1) & 15) << 4)).astype(np.uint8)
    blk = q4_k_superblock(0x3C00, 0x3C00, hexbytes(g["field_hex"]), codes)
    got = oracle.dequantize(wl.Q4_K, blk, 256)[0]
    for item in g["spot_checks"]:
        e, v = item.split("=")
        assert got[int(e)] == float(v), item
    # every element: element e of chunk c at r uses sub-block 2c (r < 32, low
    # nibble of byte 32c + r) or 2c + 1 (high nibble of byte 32c + r - 32)
    for e in range(256):
        c, r = divmod(e, 64)
        if r < 32:
            q, j = int(codes[32 * c + r]) & 15, 2 * c
        else:
            q, j = int(codes[32 * c + r - 32]) >> 4, 2 * c + 1
        assert got[e] == sc[j] * q - m[j], e


def test_q4_k_non_integer_scales():
    # d = 2^-10 (0x1400), dmin = 0.5 (0x3800): value = 2^-10 * sc * q - 0.5 * m, exact
    sc = [5, 9, 33, 63, 1, 2, 40, 17]
    m = [7, 0, 63, 12, 31, 16, 1, 50]
    codes = (np.arange(128) * 37 % 256).astype(np.uint8)
    blk = q4_k_superblock(0x1400, 0x3800, pack_q4_k_field(sc, m), codes.astype(np.uint8))
    got = oracle.dequantize(wl.Q4_K, blk, 256)[0]
    for e in range(256):
        c, r = divmod(e, 64)
        q = int(codes[32 * c + r]) & 15 if r < 32 else int(codes[32 * c + r - 32]) >> 4
        j = 2 * c + (r >= 32)
        assert got[e] == np.float32(2.0 ** -10 * sc[j] * q - 0.5 * m[j]), e


@pytest.mark.parametrize("variant", ["same", "shifted"])
def test_q4_k_pack_bijection_every_pair_every_position(variant):
    """All 64 x 64 (sc, m) pairs at all eight positions: pack (test side),
    decode (oracle), read sc and m back from elements with q = 0 and q = 1."""
    nblk = 4096
    blocks = np.zeros((nblk, 144), dtype=np.uint8)
    expect_sc = np.zeros((nblk, 8), dtype=np.int64)
    expect_m = np.zeros((nblk, 8), dtype=np.int64)
    codes = np.zeros(128, dtype=np.uint8)
    for c in range(4):
        codes[32 * c + 0] = 0x00  # low q = 0 (sub-block 2c), high q = 0 (2c + 1)
        codes[32 * c + 1] = 0x11  # low q = 1, high q = 1
    for i in range(nblk):
        a, b = divmod(i, 64)
        if variant == "same":
            sc = [a] * 8
            m = [b] * 8
        else:
            sc = [(a + 11 * j) % 64 for j in range(8)]
            m = [(b + 5 * j + 3 * (j > 3)) % 64 for j in range(8)]
        expect_sc[i] = sc
        expect_m[i] = m
        blocks[i] = q4_k_superblock(0x3C00, 0x3C00, pack_q4_k_field(sc, m), codes)
    w = oracle.dequantize(wl.Q4_K, blocks, 256 * nblk)[0].reshape(nblk, 256).astype(np.int64)
    for j in range(8):
        c, hi = divmod(j, 2)
        e0 = 64 * c + 32 * hi  # q = 0
        assert np.array_equal(-w[:, e0], expect_m[:, j]), j
        assert np.array_equal(w[:, e0 + 1] + expect_m[:, j], expect_sc[:, j]), j


# --- the contraction ----------------------------------------------------------

def small_case(wtype, T, N, nblk, seed):
    blk, _ = wl.block_geometry(wtype)
    K = max(blk, 32) * nblk if blk > 1 else 37 * nblk
    return wl.make_case(wtype, N, K, T, seed)


@pytest.mark.parametrize("wtype", TYPES)
def test_brute_force_dot_products(wtype):
    c = small_case(wtype, T=5, N=7, nblk=2, seed=11)
    dst, acc, ab = oracle.out_prod(wtype, c["W"], c["G"], c["K"])
    w = oracle.dequantize(wtype, c["W"], c["K"])
    K = c["K"]
    for t in range(5):
        for k in range(0, K, max(1, K // 40)):
            # per-output dot product, summed from the last n down (another order)
            s = 0.0
            for n in reversed(range(7)):
                s += float(w[n, k]) * float(c["G"][t, n])
            assert abs(s - acc[t, k]) <= 1e-12 * ab[t, k]
            ulp = np.spacing(np.float32(abs(s)))
            assert abs(np.float32(s) - dst[t, k]) <= ulp


@pytest.mark.parametrize("wtype", TYPES)
def test_matches_numpy_matmul(wtype):
    c = small_case(wtype, T=33, N=65, nblk=3, seed=12)
    dst, acc, ab = oracle.out_prod(wtype, c["W"], c["G"], c["K"])
    w = oracle.dequantize(wtype, c["W"], c["K"]).astype(np.float64)
    ref = c["G"].astype(np.float64) @ w
    assert np.all(np.abs(ref - acc) <= 1e-12 * ab + 1e-300)
    assert np.allclose(ab, np.abs(c["G"].astype(np.float64)) @ np.abs(w), rtol=1e-12, atol=0)


def test_is_the_input_gradient_of_mul_mat():
    """x.grad for L = sum(mul_mat(W, x) * G) with mul_mat(W, x)[t][n] = sum_k W[n][k] x[t][k]."""
    c = small_case(wl.Q4_K, T=9, N=20, nblk=1, seed=13)
    w = torch.from_numpy(oracle.dequantize(wl.Q4_K, c["W"], c["K"]).astype(np.float64))
    x = torch.randn(9, c["K"], dtype=torch.float64, requires_grad=True)
    y = x @ w.T
    (y * torch.from_numpy(c["G"].astype(np.float64))).sum().backward()
    _, acc, ab = oracle.out_prod(wl.Q4_K, c["W"], c["G"], c["K"])
    assert np.all(np.abs(x.grad.numpy() - acc) <= 1e-12 * ab + 1e-300)


@pytest.mark.parametrize("wtype", [wl.Q8_0, wl.Q4_0, wl.Q4_K, wl.F16, wl.BF16])
def test_f32_twin_is_bit_identical(wtype):
    c = small_case(wtype, T=6, N=19, nblk=2, seed=14)
    w = oracle.dequantize(wtype, c["W"], c["K"])
    d1, a1, s1 = oracle.out_prod(wtype, c["W"], c["G"], c["K"])
    d2, a2, s2 = oracle.out_prod(wl.F32, w.view(np.uint8), c["G"], c["K"])
    assert np.array_equal(d1.view(np.uint32), d2.view(np.uint32))
    assert np.array_equal(a1, a2) and np.array_equal(s1, s2)


def test_closed_form_two_rows():
    # Q8_0, N = 2 rows: row 0 all codes 1 with d = 1, row 1 all codes 2 with d = 0.5
    # (value 1), row 1 block 1 codes -3 with d = 0.25 (value -0.75).
    W = np.zeros((2, 2, 34), dtype=np.uint8)
    W[0, :, 0:2] = [0x00, 0x3C]
    W[0, :, 2:] = 1
    W[1, 0, 0:2] = [0x00, 0x38]
    W[1, 0, 2:] = 2
    W[1, 1, 0:2] = [0x00, 0x34]
    W[1, 1, 2:] = np.uint8(256 - 3)
    G = np.array([[2.0, 3.0], [-1.0, 0.5]], dtype=np.float32)
    dst, _, _ = oracle.out_prod(wl.Q8_0, W.reshape(2, 68), G, 64)
    expect = np.empty((2, 64), dtype=np.float32)
    expect[:, :32] = (G[:, 0] * 1.0 + G[:, 1] * 1.0)[:, None]
    expect[:, 32:] = (G[:, 0] * 1.0 + G[:, 1] * -0.75)[:, None]
    assert np.array_equal(dst, expect)


def test_special_cases():
    c = small_case(wl.Q4_0, T=4, N=6, nblk=2, seed=15)
    # empty reduction
    d, a, s = oracle.out_prod(wl.Q4_0, c["W"][:0], c["G"][:, :0], c["K"])
    assert np.array_equal(d, np.zeros((4, c["K"]), dtype=np.float32))
    # zero gradient
    d, _, _ = oracle.out_prod(wl.Q4_0, c["W"], np.zeros_like(c["G"]), c["K"])
    assert not d.any()
    # identity gradient returns the decoded weight exactly
    eye = np.eye(6, dtype=np.float32)
    d, _, _ = oracle.out_prod(wl.Q4_0, c["W"], eye, c["K"])
    assert np.array_equal(d, oracle.dequantize(wl.Q4_0, c["W"], c["K"]))


def test_row_subset_and_threads_change_nothing():
    c = small_case(wl.Q4_K, T=21, N=40, nblk=2, seed=16)
    full, acc, ab = oracle.out_prod(wl.Q4_K, c["W"], c["G"], c["K"])
    rows = np.array([20, 3, 3, 0, 17])
    d2, a2, s2 = oracle.out_prod(wl.Q4_K, c["W"], c["G"], c["K"], rows=rows, nthreads=3)
    assert np.array_equal(d2, full[rows]) and np.array_equal(a2, acc[rows]) and np.array_equal(s2, ab[rows])


def test_row_bytes():
    assert oracle.row_bytes(wl.Q8_0, 256) == 272
    assert oracle.row_bytes(wl.Q4_0, 5120) == 2880
    assert oracle.row_bytes(wl.Q4_K, 4096) == 2304
    assert oracle.row_bytes(wl.Q4_K, 14336) == 8064
    assert oracle.row_bytes(wl.F16, 4096) == 8192
    assert oracle.row_bytes(wl.F32, 4096) == 16384
    assert oracle.row_bytes(wl.Q4_K, 100) == -1
    assert oracle.row_bytes(99, 32) == -1


def test_error_metrics_flag_a_planted_precision_loss():
    """The parity metrics separate F32 accumulation from a silently reduced
    precision (G rounded to fp16 before the product)."""
    c = small_case(wl.Q4_K, T=16, N=512, nblk=1, seed=17)
    _, acc, ab = oracle.out_prod(wl.Q4_K, c["W"], c["G"], c["K"])
    w = oracle.dequantize(wl.Q4_K, c["W"], c["K"])
    good = (c["G"] @ w).astype(np.float32)  # float32 accumulation
    bad = (c["G"].astype(np.float16).astype(np.float32) @ w).astype(np.float32)
    eg = oracle.errors(good, acc, ab)
    eb = oracle.errors(bad, acc, ab)
    assert eg["nmse"] < 1e-10 and eg["max_rel"] < 2e-6
    assert eb["max_rel"] > 2e-6
