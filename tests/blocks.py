"""Test-side block packers and the golden-fixture readers built on them.

These write weight blocks byte by byte from the GGUF layout descriptions
(the oracle and the HIP library only unpack), so that a test can state a
block by its fields: scales, sub-scale fields, code bytes. They hold none of
the decode arithmetic. Both the oracle pins (no GPU) and the device decode
tests use them, so that the device sees exactly the blocks the oracle's
fixtures pin.
"""

from __future__ import annotations

import numpy as np

import workloads as wl


def hexbytes(tokens):
    return np.array([int(t, 16) for t in tokens], dtype=np.uint8)


def fixture_value(v: str) -> float:
    """A fixture's expected value: decimal, C99 hex float (0x1p-128), inf, nan."""
    return float.fromhex(v) if "p" in v else float(v)


def pack_q4_k_field(sc, m):
    """GGUF Q4_K sub-scale/sub-min packing, written for the tests (the oracle only unpacks)."""
    s = [0] * 12
    for j in range(4):
        s[j] = (sc[j] & 63) | ((sc[j + 4] >> 4) << 6)
        s[j + 4] = (m[j] & 63) | ((m[j + 4] >> 4) << 6)
        s[j + 8] = (sc[j + 4] & 15) | ((m[j + 4] & 15) << 4)
    return np.array(s, dtype=np.uint8)


def _le16(bits):
    return np.array([bits & 255, (bits >> 8) & 255], dtype=np.uint8)


def q4_k_superblock(d_bits, dmin_bits, field, codes):
    blk = np.zeros(144, dtype=np.uint8)
    blk[0:2] = _le16(d_bits)
    blk[2:4] = _le16(dmin_bits)
    blk[4:16] = field
    blk[16:144] = codes
    return blk


def q5_k_superblock(d_bits, dmin_bits, field, qh, qs):
    blk = np.zeros(176, dtype=np.uint8)
    blk[0:2] = _le16(d_bits)
    blk[2:4] = _le16(dmin_bits)
    blk[4:16] = field
    blk[16:48] = qh
    blk[48:176] = qs
    return blk


def q6_k_superblock(d_bits, scales, ql, qh):
    blk = np.zeros(210, dtype=np.uint8)
    blk[0:128] = ql
    blk[128:192] = qh
    blk[192:208] = np.asarray(scales, dtype=np.int8).view(np.uint8)
    blk[208:210] = _le16(d_bits)
    return blk


def q2_k_superblock(d_bits, dmin_bits, pairs, qs):
    blk = np.zeros(84, dtype=np.uint8)
    blk[0:16] = pairs
    blk[16:80] = qs
    blk[80:82] = _le16(d_bits)
    blk[82:84] = _le16(dmin_bits)
    return blk


def pack_q3_k_field(sc):
    """Sixteen 6-bit Q3_K sub-scales into the 12-byte field, written for the
    tests from the layout description (the oracle only unpacks)."""
    f = [0] * 12
    for s_, v in enumerate(sc):
        i, g = s_ % 4, s_ // 4
        f[4 * (g % 2) + i] |= (v & 15) << (4 * (g // 2))
        f[8 + i] |= ((v >> 4) & 3) << (2 * g)
    return np.array(f, dtype=np.uint8)


def q3_k_superblock(d_bits, hmask, qs, field):
    blk = np.zeros(110, dtype=np.uint8)
    blk[0:32] = hmask
    blk[32:96] = qs
    blk[96:108] = field
    blk[108:110] = _le16(d_bits)
    return blk


def ramp_codes(n):
    i = np.arange(n)
    return (((i * 7 + 3) & 15) | (((i * 5 + 1) & 15) << 4)).astype(np.uint8)


# The code patterns the K-quant fixtures are stated for (see each fixture's
# comments).
def q5_k_fixture_qh():
    return ((np.arange(32) * 13 + 7) & 255).astype(np.uint8)


def q6_k_fixture_qh():
    return ((np.arange(64) * 13 + 7) & 255).astype(np.uint8)


def q2_k_fixture_qs():
    return ((np.arange(64) * 37 + 11) & 255).astype(np.uint8)


def q3_k_fixture_hmask():
    return ((np.arange(32) * 29 + 5) & 255).astype(np.uint8)


def q3_k_fixture_qs():
    return ((np.arange(64) * 37 + 11) & 255).astype(np.uint8)


def golden_blocks(read):
    """Every block of tests/golden as (label, type, K, block bytes,
    {element: expected value}), read through `read` (the conftest reader).
    Fixtures that list a whole block give every element; the others give
    their spot checks."""
    out = []
    for fixture, wtype in (("q8_0_blocks.txt", wl.Q8_0), ("q4_0_blocks.txt", wl.Q4_0)):
        g = read(fixture)
        for name in sorted(k[:-4] for k in g if k.endswith("_hex")):
            exp = {i: fixture_value(v) for i, v in enumerate(g[name + "_expected"])}
            out.append((f"{fixture}:{name}", wtype, 32, hexbytes(g[name + "_hex"]), exp))
    spot = lambda items: {int(e): fixture_value(v) for e, v in (s.split("=") for s in items)}  # noqa: E731
    g = read("q4_1_q5_blocks.txt")
    for name, wtype in (("q4_1_a", wl.Q4_1), ("q4_1_b", wl.Q4_1), ("q5_0_a", wl.Q5_0), ("q5_0_b", wl.Q5_0),
                        ("q5_1_a", wl.Q5_1)):
        out.append((f"q4_1_q5_blocks.txt:{name}", wtype, 32, hexbytes(g[name + "_hex"]), spot(g[name + "_expected"])))
    g = read("mxfp4_blocks.txt")
    for name in ("mx_a", "mx_b", "mx_c", "mx_d", "mx_e"):
        out.append((f"mxfp4_blocks.txt:{name}", wl.MXFP4, 32, hexbytes(g[name + "_hex"]),
                    spot(g[name + "_expected"])))
    g = read("nvfp4_blocks.txt")
    for name in ("nv_a", "nv_b", "nv_c"):
        out.append((f"nvfp4_blocks.txt:{name}", wl.NVFP4, 64, hexbytes(g[name + "_hex"]),
                    spot(g[name + "_expected"])))
    g4 = read("q4_k_pack.txt")
    field = hexbytes(g4["field_hex"])
    out.append(("q4_k_pack.txt", wl.Q4_K, 256, q4_k_superblock(0x3C00, 0x3C00, field, ramp_codes(128)),
                spot(g4["spot_checks"])))
    g = read("q5_k_block.txt")
    out.append(("q5_k_block.txt", wl.Q5_K, 256,
                q5_k_superblock(0x3C00, 0x3C00, field, q5_k_fixture_qh(), ramp_codes(128)), spot(g["spot_checks"])))
    g = read("q6_k_block.txt")
    out.append(("q6_k_block.txt", wl.Q6_K, 256,
                q6_k_superblock(0x3C00, [int(v) for v in g["scales"]], ramp_codes(128), q6_k_fixture_qh()),
                spot(g["spot_checks"])))
    g = read("q2_k_block.txt")
    out.append(("q2_k_block.txt", wl.Q2_K, 256,
                q2_k_superblock(0x3C00, 0x3C00, hexbytes(g["pairs_hex"]), q2_k_fixture_qs()), spot(g["spot_checks"])))
    g = read("q3_k_block.txt")
    out.append(("q3_k_block.txt", wl.Q3_K, 256,
                q3_k_superblock(0x3C00, q3_k_fixture_hmask(), q3_k_fixture_qs(), hexbytes(g["field_hex"])),
                spot(g["spot_checks"])))
    return out
