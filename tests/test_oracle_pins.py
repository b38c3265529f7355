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
from blocks import (hexbytes, pack_q3_k_field, pack_q4_k_field, q2_k_superblock, q3_k_superblock,
                    q4_k_superblock, q5_k_superblock, q6_k_superblock, ramp_codes)
from blocks import fixture_value as _fixture_value

TYPES = [wl.F32, wl.F16, wl.BF16, wl.Q8_0, wl.Q4_0, wl.Q4_1, wl.Q5_0, wl.Q5_1, wl.MXFP4, wl.NVFP4, wl.Q2_K, wl.Q3_K,
         wl.Q4_K, wl.Q5_K, wl.Q6_K]




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


@pytest.mark.parametrize("name,wtype", [("q4_1_a", wl.Q4_1), ("q4_1_b", wl.Q4_1), ("q5_0_a", wl.Q5_0),
                                        ("q5_0_b", wl.Q5_0), ("q5_1_a", wl.Q5_1)])
def test_q4_1_q5_hand_built_blocks(golden, name, wtype):
    g = golden("q4_1_q5_blocks.txt")
    got = oracle.dequantize(wtype, hexbytes(g[name + "_hex"]), 32)[0]
    for item in g[name + "_expected"]:
        e, v = item.split("=")
        assert got[int(e)] == float(v), (name, item)




@pytest.mark.parametrize("name", ["mx_a", "mx_b", "mx_c", "mx_d", "mx_e"])
def test_mxfp4_hand_built_blocks(golden, name):
    g = golden("mxfp4_blocks.txt")
    got = oracle.dequantize(wl.MXFP4, hexbytes(g[name + "_hex"]), 32)[0]
    for item in g[name + "_expected"]:
        e, v = item.split("=")
        want = np.float32(_fixture_value(v))
        if np.isnan(want):
            assert np.isnan(got[int(e)]), (name, item)
        else:
            assert got[int(e)] == want and np.signbit(got[int(e)]) == np.signbit(want), (name, item)


@pytest.mark.parametrize("name", ["nv_a", "nv_b", "nv_c"])
def test_nvfp4_hand_built_blocks(golden, name):
    g = golden("nvfp4_blocks.txt")
    got = oracle.dequantize(wl.NVFP4, hexbytes(g[name + "_hex"]), 64)[0]
    for item in g[name + "_expected"]:
        e, v = item.split("=")
        want = np.float32(_fixture_value(v))
        if np.isnan(want):
            assert np.isnan(got[int(e)]), (name, item)
        else:
            assert got[int(e)] == want and np.signbit(got[int(e)]) == np.signbit(want), (name, item)


def test_nvfp4_scale_is_fp8_e4m3_of_an_independent_library():
    """Every one of the 256 scale bytes, under codes of value 1 (nibble 2):
    the decoded elements are the scale itself, which must be torch's
    float8_e4m3fn value of the byte (NaN for 0x7F and 0xFF, subnormals for
    exponent 0, signs and zeros included)."""
    blk = np.zeros((64, 36), dtype=np.uint8)
    blk[:, 0:4] = np.arange(256, dtype=np.uint8).reshape(64, 4)  # scale byte 4 i + s of block i
    blk[:, 4:] = 0x22
    got = oracle.dequantize(wl.NVFP4, blk, 64).reshape(64, 4, 16)
    ref = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn).float().numpy().reshape(64, 4)
    for i in range(16):
        col = got[:, :, i]
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(col), nan)
        assert np.array_equal(col[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_nvfp4_codes_are_the_pinned_e2m1():
    """Under scale 1 (E4M3 0x38) every code byte decodes, nibble for nibble,
    to the values MXFP4 gives the same byte under scale 1 (E8M0 127): the
    E2M1 decode pinned above. Element 16s + i takes the low nibble of code
    byte 8s + i and element 16s + 8 + i its high nibble."""
    codes = np.arange(256, dtype=np.uint8).reshape(8, 32)  # 8 NVFP4 blocks of 32 code bytes
    nv = np.zeros((8, 36), dtype=np.uint8)
    nv[:, 0:4] = 0x38
    nv[:, 4:] = codes
    got = oracle.dequantize(wl.NVFP4, nv, 64).reshape(8, 4, 2, 8)  # block, sub-block, half, i
    mx = np.zeros((16, 17), dtype=np.uint8)
    mx[:, 0] = 127
    mx[:, 1:] = np.arange(256, dtype=np.uint8).reshape(16, 16)
    ref = oracle.dequantize(wl.MXFP4, mx, 32)  # row r: byte 16 r + j -> lo at j, hi at j + 16
    lo_of = ref[:, :16].reshape(-1)
    hi_of = ref[:, 16:].reshape(-1)
    b = codes.reshape(8, 4, 8)  # the byte under (block, sub-block, i)
    for half, table in ((0, lo_of), (1, hi_of)):
        want = table[b]
        assert np.array_equal(got[:, :, half, :].view(np.uint32), want.view(np.uint32)), half


def test_mxfp4_structure():
    """Every code byte under several scales: a nibble decodes the same in
    either half of a byte, the sign bit negates (zero included), the eight
    magnitudes rise strictly from 0, and one more in the scale byte doubles
    every value."""
    blocks = np.zeros((16, 17), dtype=np.uint8)
    blocks[:, 1:] = np.arange(256, dtype=np.uint8).reshape(16, 16)   # code byte j of block i is 16 i + j
    vals = {}
    idx = np.arange(256)
    for e in (100, 101, 127, 200):
        blocks[:, 0] = e
        v = oracle.dequantize(wl.MXFP4, blocks, 32)
        lo, hi = v[:, :16].reshape(-1), v[:, 16:].reshape(-1)   # nibble values of byte b
        for a, b in ((lo, lo[idx & 15]), (hi, lo[idx >> 4])):
            assert np.array_equal(a, b) and np.array_equal(np.signbit(a), np.signbit(b))
        assert lo[0] == 0 and np.all(np.diff(lo[:8]) > 0)
        for c in range(8):
            assert lo[c | 8] == -lo[c] and np.signbit(lo[c | 8]) and not np.signbit(lo[c])
        vals[e] = v
    assert np.array_equal(vals[101], 2 * vals[100])
    assert np.array_equal(vals[127][0, :8], np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float32))


def test_q5_0_fifth_bits_one_to_one():
    """d = 1, all nibbles 0, qh = 1 << b: exactly element b becomes 0 (q = 16),
    the others stay -16; Q5_1 with m = 0 and the same bytes gives 16 there and
    0 elsewhere, and Q4_1 with qh's bytes removed matches Q5_1 with qh = 0."""
    for b in range(32):
        qh = (1 << b).to_bytes(4, "little")
        blk = np.frombuffer(bytes([0x00, 0x3C]) + qh + bytes(16), dtype=np.uint8)
        got = oracle.dequantize(wl.Q5_0, blk, 32)[0]
        assert got[b] == 0 and np.all(np.delete(got, b) == -16), b
        blk1 = np.frombuffer(bytes([0x00, 0x3C, 0x00, 0x00]) + qh + bytes(16), dtype=np.uint8)
        got1 = oracle.dequantize(wl.Q5_1, blk1, 32)[0]
        assert got1[b] == 16 and np.all(np.delete(got1, b) == 0), b
    rng = np.random.default_rng(5)
    for _ in range(20):
        d, m = (int(v) for v in rng.integers(0x0400, 0x4400, size=2))
        codes = rng.integers(0, 256, size=16, dtype=np.uint8).tobytes()
        head = bytes([d & 255, d >> 8, m & 255, m >> 8])
        a = oracle.dequantize(wl.Q5_1, np.frombuffer(head + bytes(4) + codes, np.uint8), 32)[0]
        b_ = oracle.dequantize(wl.Q4_1, np.frombuffer(head + codes, np.uint8), 32)[0]
        assert np.array_equal(a.view(np.uint32), b_.view(np.uint32))








def test_q5_k_hand_built_superblock(golden):
    g4, g5 = golden("q4_k_pack.txt"), golden("q5_k_block.txt")
    qh = ((np.arange(32) * 13 + 7) & 255).astype(np.uint8)
    blk = q5_k_superblock(0x3C00, 0x3C00, hexbytes(g4["field_hex"]), qh, ramp_codes(128))
    got = oracle.dequantize(wl.Q5_K, blk, 256)[0]
    for item in g5["spot_checks"]:
        e, v = item.split("=")
        assert got[int(e)] == float(v), item


def test_q5_k_without_fifth_bits_is_q4_k():
    """qh = 0: a Q5_K block decodes like the Q4_K block with the same scales,
    field and nibbles (the pinned Q4_K decoder), for random blocks and non-
    integer scales."""
    rng = np.random.default_rng(11)
    for _ in range(20):
        d, dmin = (int(v) for v in rng.integers(0x0400, 0x4400, size=2))
        field = rng.integers(0, 256, size=12, dtype=np.uint8)
        qs = rng.integers(0, 256, size=128, dtype=np.uint8)
        q5 = oracle.dequantize(wl.Q5_K, q5_k_superblock(d, dmin, field, np.zeros(32, np.uint8), qs), 256)[0]
        q4 = oracle.dequantize(wl.Q4_K, q4_k_superblock(d, dmin, field, qs), 256)[0]
        assert np.array_equal(q5.view(np.uint32), q4.view(np.uint32))


def test_q5_k_each_fifth_bit_moves_one_element_by_16_sub_scales(golden):
    """With d = dmin = 1 every value is the integer sc_j * q - m_j. Setting
    one bit of qh adds 16 * sc_j to exactly one element, and the 256 bits
    reach the 256 elements one to one: bit b of qh[r] belongs to element
    64 (b // 2) + 32 (b % 2) + r."""
    g4 = golden("q4_k_pack.txt")
    field = hexbytes(g4["field_hex"])
    sc = [int(v) for v in g4["sc"]]
    qs = ramp_codes(128)
    base = oracle.dequantize(wl.Q5_K, q5_k_superblock(0x3C00, 0x3C00, field, np.zeros(32, np.uint8), qs), 256)[0]
    seen = set()
    for r in range(32):
        for b in range(8):
            qh = np.zeros(32, np.uint8)
            qh[r] = 1 << b
            got = oracle.dequantize(wl.Q5_K, q5_k_superblock(0x3C00, 0x3C00, field, qh, qs), 256)[0]
            diff = np.nonzero(got != base)[0]
            assert len(diff) == 1, (r, b)
            e = int(diff[0])
            assert e == 64 * (b // 2) + 32 * (b % 2) + r, (r, b, e)
            assert got[e] - base[e] == 16 * sc[b], (r, b)
            seen.add(e)
    assert seen == set(range(256))


def test_q6_k_hand_built_superblock(golden):
    g = golden("q6_k_block.txt")
    scales = [int(v) for v in g["scales"]]
    qh = ((np.arange(64) * 13 + 7) & 255).astype(np.uint8)
    got = oracle.dequantize(wl.Q6_K, q6_k_superblock(0x3C00, scales, ramp_codes(128), qh), 256)[0]
    for item in g["spot_checks"]:
        e, v = item.split("=")
        assert got[int(e)] == float(v), item


def test_q6_k_structure():
    """d = 1, every sub-scale 1, qh = 0: element values are nibble - 32, and
    the 256 nibbles (low nibbles of ql, then high nibbles, by quarter and
    half) reach the 256 elements one to one. Then each of the 128 two-bit
    high parts, set to 1, adds 16 to exactly one element."""
    ql = np.zeros(128, np.uint8)
    seen = {}
    for i in range(128):
        for hi_nib in (0, 1):
            ql[:] = 0
            ql[i] = 0x10 if hi_nib else 0x01
            got = oracle.dequantize(wl.Q6_K, q6_k_superblock(0x3C00, [1] * 16, ql, np.zeros(64, np.uint8)), 256)[0]
            moved = np.nonzero(got != -32)[0]
            assert len(moved) == 1 and got[moved[0]] == -31, (i, hi_nib)
            seen[(i, hi_nib)] = int(moved[0])
    assert sorted(seen.values()) == list(range(256))
    # element 128h + 32p + l: nibble of ql[64h + 32(p % 2) + l], high half for p >= 2
    for (i, hi_nib), e in seen.items():
        h, p, l = e // 128, (e % 128) // 32, e % 32
        assert (i, hi_nib) == (64 * h + 32 * (p % 2) + l, int(p >= 2)), (i, hi_nib, e)
    moved_by_qh = set()
    for i in range(64):
        for p in range(4):
            qh = np.zeros(64, np.uint8)
            qh[i] = 1 << (2 * p)
            got = oracle.dequantize(wl.Q6_K, q6_k_superblock(0x3C00, [1] * 16, np.zeros(128, np.uint8), qh), 256)[0]
            moved = np.nonzero(got != -32)[0]
            assert len(moved) == 1 and got[moved[0]] == -16, (i, p)
            e = int(moved[0])
            assert e == 128 * (i // 32) + 32 * p + i % 32, (i, p, e)
            moved_by_qh.add(e)
    assert moved_by_qh == set(range(256))


def test_q6_k_sub_scale_index_and_sign():
    """One sub-scale at a time set to -3 (the rest 1): exactly the 16
    elements 128h + 32p + 16s + 0..15 of sub-scale 8h + 2p + s change, to
    -3 * (q - 32)."""
    ql = ramp_codes(128)
    qh = ((np.arange(64) * 13 + 7) & 255).astype(np.uint8)
    base = oracle.dequantize(wl.Q6_K, q6_k_superblock(0x3C00, [1] * 16, ql, qh), 256)[0]
    for i in range(16):
        scales = [1] * 16
        scales[i] = -3
        got = oracle.dequantize(wl.Q6_K, q6_k_superblock(0x3C00, scales, ql, qh), 256)[0]
        h, p, s_ = i // 8, (i % 8) // 2, i % 2
        idx = 128 * h + 32 * p + 16 * s_ + np.arange(16)
        assert np.array_equal(got[idx], -3 * base[idx])
        rest = np.setdiff1d(np.arange(256), idx)
        assert np.array_equal(got[rest], base[rest])


def test_q6_k_products_are_exact():
    """Largest odd parts of d, sub-scale and q - 32 (2047/1024, 127, 31): the
    oracle's F32 value equals the exact product."""
    ql = np.full(128, 0xFF, np.uint8)   # low nibbles 15
    qh = np.full(64, 0x55, np.uint8)    # every 2-bit high part 1 -> q = 31, q - 32 = -1
    got = oracle.dequantize(wl.Q6_K, q6_k_superblock(0x3FFF, [127] * 16, ql, qh), 256)[0]
    assert np.all(got == np.float32(-(2047 / 1024) * 127))
    qh = np.zeros(64, np.uint8)         # q = 15 -> q - 32 = -17
    ql = np.full(128, 0x11, np.uint8)   # q = 1 -> -31
    got = oracle.dequantize(wl.Q6_K, q6_k_superblock(0x3FFF, [127] * 16, ql, qh), 256)[0]
    assert np.all(got == np.float32(2047 * 127 * -31 / 1024))
    assert 2047 * 127 * 31 < 2 ** 24








def test_q2_k_hand_built_superblock(golden):
    g = golden("q2_k_block.txt")
    qs = ((np.arange(64) * 37 + 11) & 255).astype(np.uint8)
    got = oracle.dequantize(wl.Q2_K, q2_k_superblock(0x3C00, 0x3C00, hexbytes(g["pairs_hex"]), qs), 256)[0]
    for item in g["spot_checks"]:
        e, v = item.split("=")
        assert got[int(e)] == float(v), item


def test_q2_k_structure():
    """d = dmin = 1 and every pair (sc, m) = (1, 0): a code value v in bits
    2p, 2p + 1 of one qs byte makes exactly one element v, and the 256 (byte,
    p) positions reach the 256 elements one to one. Then each pair byte, set
    alone to (sc, m) = (3, 5), changes exactly its 16 elements to 3q - 5."""
    base_pairs = np.full(16, 0x01, np.uint8)
    zero = oracle.dequantize(wl.Q2_K, q2_k_superblock(0x3C00, 0x3C00, base_pairs, np.zeros(64, np.uint8)), 256)[0]
    assert np.all(zero == 0)
    seen = set()
    for i in range(64):
        for p in range(4):
            for v in (1, 2, 3):
                qs = np.zeros(64, np.uint8)
                qs[i] = v << (2 * p)
                got = oracle.dequantize(wl.Q2_K, q2_k_superblock(0x3C00, 0x3C00, base_pairs, qs), 256)[0]
                moved = np.nonzero(got)[0]
                assert len(moved) == 1 and got[moved[0]] == v, (i, p, v)
            seen.add(int(moved[0]))
    assert seen == set(range(256))
    qs = ((np.arange(64) * 37 + 11) & 255).astype(np.uint8)
    base = oracle.dequantize(wl.Q2_K, q2_k_superblock(0x3C00, 0x3C00, base_pairs, qs), 256)[0]
    for j in range(16):
        pairs = base_pairs.copy()
        pairs[j] = 3 | (5 << 4)
        got = oracle.dequantize(wl.Q2_K, q2_k_superblock(0x3C00, 0x3C00, pairs, qs), 256)[0]
        h, p, s_ = j // 8, (j % 8) // 2, j % 2
        idx = 128 * h + 32 * p + 16 * s_ + np.arange(16)
        assert np.array_equal(got[idx], 3 * base[idx] - 5)
        rest = np.setdiff1d(np.arange(256), idx)
        assert np.array_equal(got[rest], base[rest])


def test_q3_k_field_packer_matches_hand_packing(golden):
    g = golden("q3_k_block.txt")
    assert np.array_equal(pack_q3_k_field([int(v) for v in g["sc"]]), hexbytes(g["field_hex"]))


def test_q3_k_hand_built_superblock(golden):
    g = golden("q3_k_block.txt")
    hmask = ((np.arange(32) * 29 + 5) & 255).astype(np.uint8)
    qs = ((np.arange(64) * 37 + 11) & 255).astype(np.uint8)
    got = oracle.dequantize(wl.Q3_K, q3_k_superblock(0x3C00, hmask, qs, hexbytes(g["field_hex"])), 256)[0]
    for item in g["spot_checks"]:
        e, v = item.split("=")
        assert got[int(e)] == float(v), item


def test_q3_k_sub_scale_bijection_every_value_every_position():
    """Every 6-bit value at each of the 16 positions, the other 15 positions
    holding other values: packed (test side), decoded (oracle) with every
    code 1 (low = 1, mask bit set), so element values are sc - 32."""
    hmask = np.full(32, 0xFF, np.uint8)
    qs = np.full(64, 0x55, np.uint8)
    for pos in range(16):
        for v in range(64):
            sc = [(v + 7 * k + 1) % 64 for k in range(16)]
            sc[pos] = v
            got = oracle.dequantize(wl.Q3_K, q3_k_superblock(0x3C00, hmask, qs, pack_q3_k_field(sc)), 256)[0]
            for k in range(16):
                h, p, s_ = k // 8, (k % 8) // 2, k % 2
                idx = 128 * h + 32 * p + 16 * s_ + np.arange(16)
                assert np.all(got[idx] == sc[k] - 32), (pos, v, k)


def test_q3_k_mask_bits_and_codes():
    """Sub-scales all 33 (factor 1), codes 0: every element is -4 with an
    empty mask. Each mask bit b of hmask[l], set alone, lifts exactly one
    element to 0: element 128 (b // 4) + 32 (b % 4) + l; each 2-bit code,
    with the full mask, adds its value to exactly one element."""
    field = pack_q3_k_field([33] * 16)
    got = oracle.dequantize(wl.Q3_K, q3_k_superblock(0x3C00, np.zeros(32, np.uint8), np.zeros(64, np.uint8), field),
                            256)[0]
    assert np.all(got == -4)
    seen = set()
    for l in range(32):
        for b in range(8):
            hm = np.zeros(32, np.uint8)
            hm[l] = 1 << b
            got = oracle.dequantize(wl.Q3_K, q3_k_superblock(0x3C00, hm, np.zeros(64, np.uint8), field), 256)[0]
            moved = np.nonzero(got != -4)[0]
            assert len(moved) == 1 and got[moved[0]] == 0, (l, b)
            assert moved[0] == 128 * (b // 4) + 32 * (b % 4) + l, (l, b)
            seen.add(int(moved[0]))
    assert seen == set(range(256))
    full = np.full(32, 0xFF, np.uint8)
    seen = set()
    for i in range(64):
        for p in range(4):
            qs = np.zeros(64, np.uint8)
            qs[i] = 3 << (2 * p)
            got = oracle.dequantize(wl.Q3_K, q3_k_superblock(0x3C00, full, qs, field), 256)[0]
            moved = np.nonzero(got)[0]
            assert len(moved) == 1 and got[moved[0]] == 3, (i, p)
            seen.add(int(moved[0]))
    assert seen == set(range(256))


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


# --- mul_mat (the forward) ----------------------------------------------------

@pytest.mark.parametrize("wtype", TYPES)
def test_mul_mat_matches_numpy_and_torch(wtype):
    """y = x W^T with the decoded W: numpy float64 matmul and torch's
    float64 linear layer agree with the oracle's double sums."""
    K = 2 * max(wl.block_geometry(wtype)[0], 32)
    c = wl.make_case(wtype, 7, K, 5, seed=31)
    x = np.random.default_rng(3).standard_normal((5, K)).astype(np.float32)
    w = oracle.dequantize(wtype, c["W"], K).astype(np.float64)
    y, acc, ab = oracle.mul_mat(wtype, c["W"], x, K)
    ref = x.astype(np.float64) @ w.T
    assert np.allclose(acc, ref, rtol=1e-12, atol=1e-12)
    lin = torch.nn.functional.linear(torch.from_numpy(x).double(), torch.from_numpy(w)).numpy()
    assert np.allclose(acc, lin, rtol=1e-12, atol=1e-12)
    assert np.array_equal(y, acc.astype(np.float32))
    assert np.allclose(ab, np.abs(x.astype(np.float64)) @ np.abs(w).T, rtol=1e-12, atol=1e-12)


def test_mul_mat_brute_force_reverse_order():
    c = wl.make_case(wl.Q4_K, 3, 256, 2, seed=8)
    x = np.random.default_rng(4).standard_normal((2, 256)).astype(np.float32)
    w = oracle.dequantize(wl.Q4_K, c["W"], 256)
    _, acc, _ = oracle.mul_mat(wl.Q4_K, c["W"], x, 256)
    for t in range(2):
        for n in range(3):
            s = 0.0
            for k in reversed(range(256)):
                s += float(w[n, k]) * float(x[t, k])
            assert abs(s - acc[t, n]) <= 1e-12 * max(1.0, abs(s))


@pytest.mark.parametrize("wtype", [wl.Q8_0, wl.Q6_K, wl.MXFP4, wl.BF16])
def test_mul_mat_and_out_prod_are_adjoint(wtype):
    """<G, mul_mat(W, x)> = <out_prod(W, G), x>: the two oracle functions
    contract the same W along its two different directions."""
    K = 2 * max(wl.block_geometry(wtype)[0], 32)
    c = wl.make_case(wtype, 9, K, 4, seed=12)
    x = np.random.default_rng(5).standard_normal((4, K)).astype(np.float32)
    _, y, _ = oracle.mul_mat(wtype, c["W"], x, K)
    _, d, _ = oracle.out_prod(wtype, c["W"], c["G"], K)
    lhs = float((c["G"].astype(np.float64) * y).sum())
    rhs = float((d * x.astype(np.float64)).sum())
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))


def test_mul_mat_f32_twin_and_row_subset():
    c = wl.make_case(wl.Q5_K, 6, 512, 9, seed=14)
    x = np.random.default_rng(6).standard_normal((9, 512)).astype(np.float32)
    w32 = oracle.dequantize(wl.Q5_K, c["W"], 512)
    a, _, _ = oracle.mul_mat(wl.Q5_K, c["W"], x, 512)
    b, _, _ = oracle.mul_mat(wl.F32, w32.view(np.uint8), x, 512)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    rows = np.array([8, 0, 3])
    s, _, _ = oracle.mul_mat(wl.Q5_K, c["W"], x, 512, rows=rows, nthreads=3)
    assert np.array_equal(s, a[rows])


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
    assert oracle.row_bytes(wl.MXFP4, 5120) == 2720
    assert oracle.row_bytes(wl.MXFP4, 48) == -1
    assert oracle.row_bytes(wl.NVFP4, 5120) == 2880
    assert oracle.row_bytes(wl.NVFP4, 96) == -1
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


def test_golden_block_reader_matches_every_fixture(golden):
    """The block list the device tests read (tests/blocks.py) holds every
    fixture file, and the oracle decodes each of its blocks to the fixture's
    values, signs included."""
    import os

    from blocks import golden_blocks

    blocks = golden_blocks(golden)
    files = {label.split(":")[0] for label, *_ in blocks}
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    assert files == {f for f in os.listdir(here) if f.endswith(".txt")}
    for label, wtype, K, raw, expected in blocks:
        got = oracle.dequantize(wtype, raw, K)[0]
        for e, v in expected.items():
            want = np.float32(v)
            if np.isnan(want):
                assert np.isnan(got[e]), (label, e)
            else:
                assert got[e] == want and np.signbit(got[e]) == np.signbit(want), (label, e)
