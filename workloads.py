"""Seeded synthetic inputs for OUT_PROD through a block-quantized weight.

This module only draws random numbers and lays them out as bytes. It holds
none of the method's arithmetic: no decoding, no scaling, no contraction.
Both the HIP path and the CPU oracle consume what it produces, and neither
is imported here.

Weight storage (one row of W = K elements along k, stored as consecutive
blocks; fp16 fields are little-endian; GGUF block formats):

  F32   4 bytes per element
  F16   2 bytes per element (IEEE binary16)
  BF16  2 bytes per element (upper half of a binary32)
  Q8_0  34 bytes per 32 elements: fp16 scale, then 32 signed 8-bit codes
  Q4_0  18 bytes per 32 elements: fp16 scale, then 16 bytes of 4-bit codes
  Q4_1  20 bytes per 32 elements: fp16 scale, fp16 offset, 16 bytes of codes
  Q5_0  22 bytes per 32 elements: fp16 scale, 4 bytes of fifth bits, 16
        bytes of 4-bit codes
  Q5_1  24 bytes per 32 elements: fp16 scale, fp16 offset, 4 bytes of fifth
        bits, 16 bytes of 4-bit codes
  MXFP4 17 bytes per 32 elements: an E8M0 scale byte, then 16 bytes of
        E2M1 codes
  NVFP4 36 bytes per 64 elements: four FP8 E4M3 scale bytes (one per 16
        elements), then 32 bytes of E2M1 codes
  Q4_K  144 bytes per 256 elements: fp16 scale, fp16 min-scale, 12 bytes
        holding eight 6-bit sub-scales and eight 6-bit sub-mins, then 128
        bytes of 4-bit codes
  Q5_K  176 bytes per 256 elements: as Q4_K, with 32 bytes of fifth code
        bits between the 12-byte field and the 128 bytes of low nibbles
  Q6_K  210 bytes per 256 elements: 128 bytes of low nibbles, 64 bytes of
        2-bit high parts, 16 signed 8-bit sub-scales, fp16 scale
  Q2_K  84 bytes per 256 elements: 16 bytes of 4-bit sub-scale/sub-min
        pairs, 64 bytes of 2-bit codes, fp16 scale, fp16 min-scale
  Q3_K  110 bytes per 256 elements: 32 bytes of high-bit masks, 64 bytes of
        2-bit codes, 12 bytes of sixteen 6-bit sub-scales, fp16 scale

Distributions (uniform ranges are [lo, hi) for floats and inclusive for
integers; N(0, s) takes s as the standard deviation):

  Q8_0  scale U[1e-3, 1e-2) rounded to fp16 (nearest-even), codes U{-127..127}
  Q4_0  scale U[1e-3, 1e-2) rounded to fp16, codes U{0..15}
  Q4_1, Q5_1  scale U[1e-3, 1e-2) and offset U[-0.1, 0) rounded to fp16,
        codes U{0..15} / U{0..31}
  Q5_0  scale U[1e-3, 1e-2) rounded to fp16, codes U{0..31}
  MXFP4 scale byte U{117..120} (scales 2^-10 .. 2^-7), codes U{0..15}
  NVFP4 scale bytes U{0x08..0x37} (positive normal E4M3 values 2^-6 ..
        1.875 * 2^-1), codes U{0..15}
  Q4_K  scale and min-scale U[1e-4, 1e-3) rounded to fp16, sub-scales and
        sub-mins U{0..63}, codes U{0..15}
  Q5_K  as Q4_K, codes U{0..31}
  Q6_K  scale U[1e-4, 1e-3) rounded to fp16, sub-scales U{-128..127},
        codes U{0..63}
  Q2_K  scale and min-scale U[1e-3, 1e-2) rounded to fp16, sub-scales and
        sub-mins U{0..15}, codes U{0..3}
  Q3_K  scale U[1e-3, 1e-2) rounded to fp16, sub-scales U{0..63} (-32
        offset applied in decoding), codes U{-4..3}
  dense W ~ N(0, 0.02) in F32, then rounded to F16 or BF16 (nearest-even)
  G     ~ N(0, sigma) in F32

Uniform 4-bit codes are drawn as uniform bytes (each byte is two independent
uniform nibbles). The Q4_K 12-byte scale field is drawn as 12 uniform bytes:
the field packs exactly 16 x 6 = 96 bits, every bit belongs to exactly one
sub-scale or sub-min, so uniform bytes are uniform 6-bit values for every
sub-scale and sub-min whatever the bit order of the pack.

Draw order for one case, from numpy Generator(PCG64(seed)): scales (the
scale, then the K-quant min-scale), then the sub-scale field, then codes
(Q5_K: fifth bits, then low nibbles; Q6_K: low nibbles, then high parts;
Q2_K: codes after its 16 pair bytes; Q3_K: high-bit masks, then low bits) or
the dense values, then G. Codes of several bits are drawn as uniform bytes
of their bit fields, which makes every code uniform over its range.
"""

from __future__ import annotations

import numpy as np

# GGUF tensor-type ids
F32, F16, Q4_0, Q4_1, Q5_0, Q5_1, Q8_0, Q2_K, Q3_K, Q4_K, Q5_K, Q6_K, BF16 = 0, 1, 2, 3, 6, 7, 8, 10, 11, 12, 13, 14, 30
MXFP4 = 39
NVFP4 = 40  # this library's id for it (the pages give no number)

TYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16", Q8_0: "q8_0", Q4_0: "q4_0", Q4_1: "q4_1", Q5_0: "q5_0",
              Q5_1: "q5_1", MXFP4: "mxfp4", NVFP4: "nvfp4", Q2_K: "q2_k", Q3_K: "q3_k", Q4_K: "q4_k", Q5_K: "q5_k", Q6_K: "q6_k"}
TYPE_IDS = {v: k for k, v in TYPE_NAMES.items()}

# (elements per block, bytes per block)
_GEOMETRY = {F32: (1, 4), F16: (1, 2), BF16: (1, 2), Q8_0: (32, 34), Q4_0: (32, 18), Q4_K: (256, 144),
             Q5_K: (256, 176), Q6_K: (256, 210), Q2_K: (256, 84), Q3_K: (256, 110), Q4_1: (32, 20),
             Q5_0: (32, 22), Q5_1: (32, 24), MXFP4: (32, 17),
             NVFP4: (64, 36)}


def block_geometry(wtype: int) -> tuple[int, int]:
    return _GEOMETRY[wtype]


def row_bytes(wtype: int, K: int) -> int:
    blk, nbytes = _GEOMETRY[wtype]
    if K % blk:
        raise ValueError(f"K={K} is not a multiple of the {TYPE_NAMES[wtype]} block ({blk})")
    return K // blk * nbytes


def _fp16_uniform(rng, lo, hi, shape):
    return rng.uniform(lo, hi, size=shape).astype(np.float16)  # numpy rounds to nearest-even


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite F32 values to the nearest BF16, ties to even; returns uint16 bits."""
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def make_weight(wtype: int, N: int, K: int, rng: np.random.Generator) -> np.ndarray:
    """Draw a W of N rows x K elements; returns uint8 bytes shaped (N, row_bytes)."""
    rb = row_bytes(wtype, K)
    if wtype in (F32, F16, BF16):
        w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
        if wtype == F32:
            raw = w.view(np.uint8)
        elif wtype == F16:
            raw = w.astype(np.float16).view(np.uint8)
        else:
            raw = _f32_to_bf16_bits(w).view(np.uint8)
        return np.ascontiguousarray(raw.reshape(N, rb))
    blk, nbytes = _GEOMETRY[wtype]
    nb = K // blk
    out = np.zeros((N, nb, nbytes), dtype=np.uint8)
    if wtype == Q8_0:
        d = _fp16_uniform(rng, 1e-3, 1e-2, (N, nb))
        q = rng.integers(-127, 128, size=(N, nb, 32), dtype=np.int8)
        out[:, :, 0:2] = d.view(np.uint8).reshape(N, nb, 2)
        out[:, :, 2:34] = q.view(np.uint8)
    elif wtype == Q4_0:
        d = _fp16_uniform(rng, 1e-3, 1e-2, (N, nb))
        qs = rng.integers(0, 256, size=(N, nb, 16), dtype=np.uint8)
        out[:, :, 0:2] = d.view(np.uint8).reshape(N, nb, 2)
        out[:, :, 2:18] = qs
    elif wtype in (Q4_1, Q5_0, Q5_1):
        d = _fp16_uniform(rng, 1e-3, 1e-2, (N, nb))
        out[:, :, 0:2] = d.view(np.uint8).reshape(N, nb, 2)
        at = 2
        if wtype != Q5_0:
            m = _fp16_uniform(rng, -0.1, 0.0, (N, nb))
            out[:, :, 2:4] = m.view(np.uint8).reshape(N, nb, 2)
            at = 4
        if wtype != Q4_1:
            out[:, :, at:at + 4] = rng.integers(0, 256, size=(N, nb, 4), dtype=np.uint8)
        out[:, :, nbytes - 16:nbytes] = rng.integers(0, 256, size=(N, nb, 16), dtype=np.uint8)
    elif wtype == MXFP4:
        out[:, :, 0] = rng.integers(117, 121, size=(N, nb), dtype=np.uint8)
        out[:, :, 1:17] = rng.integers(0, 256, size=(N, nb, 16), dtype=np.uint8)
    elif wtype == NVFP4:
        out[:, :, 0:4] = rng.integers(0x08, 0x38, size=(N, nb, 4), dtype=np.uint8)
        out[:, :, 4:36] = rng.integers(0, 256, size=(N, nb, 32), dtype=np.uint8)
    elif wtype == Q4_K:
        d = _fp16_uniform(rng, 1e-4, 1e-3, (N, nb))
        dmin = _fp16_uniform(rng, 1e-4, 1e-3, (N, nb))
        scales = rng.integers(0, 256, size=(N, nb, 12), dtype=np.uint8)
        qs = rng.integers(0, 256, size=(N, nb, 128), dtype=np.uint8)
        out[:, :, 0:2] = d.view(np.uint8).reshape(N, nb, 2)
        out[:, :, 2:4] = dmin.view(np.uint8).reshape(N, nb, 2)
        out[:, :, 4:16] = scales
        out[:, :, 16:144] = qs
    elif wtype == Q5_K:
        d = _fp16_uniform(rng, 1e-4, 1e-3, (N, nb))
        dmin = _fp16_uniform(rng, 1e-4, 1e-3, (N, nb))
        scales = rng.integers(0, 256, size=(N, nb, 12), dtype=np.uint8)
        qh = rng.integers(0, 256, size=(N, nb, 32), dtype=np.uint8)
        qs = rng.integers(0, 256, size=(N, nb, 128), dtype=np.uint8)
        out[:, :, 0:2] = d.view(np.uint8).reshape(N, nb, 2)
        out[:, :, 2:4] = dmin.view(np.uint8).reshape(N, nb, 2)
        out[:, :, 4:16] = scales
        out[:, :, 16:48] = qh
        out[:, :, 48:176] = qs
    elif wtype == Q6_K:
        d = _fp16_uniform(rng, 1e-4, 1e-3, (N, nb))
        scales = rng.integers(0, 256, size=(N, nb, 16), dtype=np.uint8)
        ql = rng.integers(0, 256, size=(N, nb, 128), dtype=np.uint8)
        qh = rng.integers(0, 256, size=(N, nb, 64), dtype=np.uint8)
        out[:, :, 0:128] = ql
        out[:, :, 128:192] = qh
        out[:, :, 192:208] = scales
        out[:, :, 208:210] = d.view(np.uint8).reshape(N, nb, 2)
    elif wtype == Q2_K:
        d = _fp16_uniform(rng, 1e-3, 1e-2, (N, nb))
        dmin = _fp16_uniform(rng, 1e-3, 1e-2, (N, nb))
        pairs = rng.integers(0, 256, size=(N, nb, 16), dtype=np.uint8)
        qs = rng.integers(0, 256, size=(N, nb, 64), dtype=np.uint8)
        out[:, :, 0:16] = pairs
        out[:, :, 16:80] = qs
        out[:, :, 80:82] = d.view(np.uint8).reshape(N, nb, 2)
        out[:, :, 82:84] = dmin.view(np.uint8).reshape(N, nb, 2)
    elif wtype == Q3_K:
        d = _fp16_uniform(rng, 1e-3, 1e-2, (N, nb))
        field = rng.integers(0, 256, size=(N, nb, 12), dtype=np.uint8)
        hmask = rng.integers(0, 256, size=(N, nb, 32), dtype=np.uint8)
        qs = rng.integers(0, 256, size=(N, nb, 64), dtype=np.uint8)
        out[:, :, 0:32] = hmask
        out[:, :, 32:96] = qs
        out[:, :, 96:108] = field
        out[:, :, 108:110] = d.view(np.uint8).reshape(N, nb, 2)
    else:
        raise ValueError(f"unknown weight type {wtype}")
    return out.reshape(N, rb)


def make_grad(T: int, N: int, sigma: float, rng: np.random.Generator) -> np.ndarray:
    g = rng.standard_normal((T, N), dtype=np.float32)
    if sigma != 1.0:
        g *= np.float32(sigma)
    return g


def make_input(T: int, K: int, seed: int, sigma: float = 1.0) -> np.ndarray:
    """The input x of the forward mul_mat: T x K float32, N(0, sigma), from
    its own generator (seed) so that it does not disturb a case's draws."""
    return make_grad(T, K, sigma, np.random.default_rng(seed))


def make_case(wtype: int, N: int, K: int, T: int, seed: int, g_sigma: float = 1.0) -> dict:
    """One seeded (W, G) pair in the draw order stated in the module docstring."""
    rng = np.random.Generator(np.random.PCG64(seed))
    W = make_weight(wtype, N, K, rng)
    G = make_grad(T, N, g_sigma, rng)
    return {"type": wtype, "N": N, "K": K, "T": T, "W": W, "G": G, "seed": seed}


# The five named workloads: the up (4096 -> 14336) projection of a 4096-wide
# model with a 14336-wide MLP at T=4096 tokens, its down (14336 -> 4096)
# projection at a LoRA-style T=16, the 5120 x 17408 projection whose F32 copy
# the llama.cpp PR's Memory note sizes, a square 4096 dense projection, and a
# tiny Q8_0 case.
WORKLOADS = {
    "q8_0_n128_k256_t64": dict(type=Q8_0, N=128, K=256, T=64, seed=1001, g_sigma=1.0),
    "dense_n4096_k4096_t512": dict(type=None, N=4096, K=4096, T=512, seed=1002, g_sigma=1.0),
    "q4_0_n17408_k5120_t2048": dict(type=Q4_0, N=17408, K=5120, T=2048, seed=1003, g_sigma=1e-2),
    "q4_k_n14336_k4096_t4096": dict(type=Q4_K, N=14336, K=4096, T=4096, seed=1004, g_sigma=1.0),
    "q4_k_n4096_k14336_t16": dict(type=Q4_K, N=4096, K=14336, T=16, seed=1005, g_sigma=1.0),
    # The same two Q4_K shapes in the other K-quants (a Q4_K_M file puts
    # Q5_K and Q6_K tensors beside the Q4_K ones; Q2_K and Q3_K make the
    # smaller K-quant mixes), with their own seeds.
    "q5_k_n14336_k4096_t4096": dict(type=Q5_K, N=14336, K=4096, T=4096, seed=1006, g_sigma=1.0),
    "q6_k_n14336_k4096_t4096": dict(type=Q6_K, N=14336, K=4096, T=4096, seed=1007, g_sigma=1.0),
    "q5_k_n4096_k14336_t16": dict(type=Q5_K, N=4096, K=14336, T=16, seed=1008, g_sigma=1.0),
    "q6_k_n4096_k14336_t16": dict(type=Q6_K, N=4096, K=14336, T=16, seed=1009, g_sigma=1.0),
    "q2_k_n14336_k4096_t4096": dict(type=Q2_K, N=14336, K=4096, T=4096, seed=1010, g_sigma=1.0),
    "q3_k_n14336_k4096_t4096": dict(type=Q3_K, N=14336, K=4096, T=4096, seed=1011, g_sigma=1.0),
    "q2_k_n4096_k14336_t16": dict(type=Q2_K, N=4096, K=14336, T=16, seed=1012, g_sigma=1.0),
    "q3_k_n4096_k14336_t16": dict(type=Q3_K, N=4096, K=14336, T=16, seed=1013, g_sigma=1.0),
    # The Q4_0 shape in the other 32-element block types, with their own seeds.
    "q4_1_n17408_k5120_t2048": dict(type=Q4_1, N=17408, K=5120, T=2048, seed=1014, g_sigma=1e-2),
    "q5_0_n17408_k5120_t2048": dict(type=Q5_0, N=17408, K=5120, T=2048, seed=1015, g_sigma=1e-2),
    "q5_1_n17408_k5120_t2048": dict(type=Q5_1, N=17408, K=5120, T=2048, seed=1016, g_sigma=1e-2),
    "mxfp4_n17408_k5120_t2048": dict(type=MXFP4, N=17408, K=5120, T=2048, seed=1017, g_sigma=1e-2),
    "nvfp4_n17408_k5120_t2048": dict(type=NVFP4, N=17408, K=5120, T=2048, seed=1018, g_sigma=1e-2),
    "nvfp4_n4096_k14336_t16": dict(type=NVFP4, N=4096, K=14336, T=16, seed=1019, g_sigma=1.0),
    # The small-T backward through the other matrix of the same MLP (W of
    # 14336 rows of 4096): 64 slabs of dst against the 256 CUs.
    "q4_k_n14336_k4096_t16": dict(type=Q4_K, N=14336, K=4096, T=16, seed=1020, g_sigma=1.0),
}


def workload(name: str, wtype: int | None = None) -> dict:
    """Materialise a named workload (the dense one needs wtype F32, F16 or BF16)."""
    spec = dict(WORKLOADS[name])
    t = spec.pop("type")
    if t is None:
        if wtype not in (F32, F16, BF16):
            raise ValueError("the dense workload needs wtype F32, F16 or BF16")
        t = wtype
    elif wtype is not None and wtype != t:
        raise ValueError(f"workload {name} is {TYPE_NAMES[t]}")
    return make_case(t, spec["N"], spec["K"], spec["T"], spec["seed"], spec["g_sigma"])
