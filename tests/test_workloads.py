"""The seeded input generator: deterministic, the stated layouts and
distributions (no GPU)."""

import numpy as np
import pytest
import torch

import workloads as wl


def test_deterministic_and_seed_sensitive():
    a = wl.make_case(wl.Q4_K, 8, 512, 4, seed=3)
    b = wl.make_case(wl.Q4_K, 8, 512, 4, seed=3)
    c = wl.make_case(wl.Q4_K, 8, 512, 4, seed=4)
    assert np.array_equal(a["W"], b["W"]) and np.array_equal(a["G"], b["G"])
    assert not np.array_equal(a["W"], c["W"])


@pytest.mark.parametrize("wtype", [wl.F32, wl.F16, wl.BF16, wl.Q8_0, wl.Q4_0, wl.Q4_1, wl.Q5_0, wl.Q5_1, wl.MXFP4,
                                   wl.NVFP4, wl.Q2_K, wl.Q3_K, wl.Q4_K, wl.Q5_K, wl.Q6_K])
def test_shapes(wtype):
    blk, nbytes = wl.block_geometry(wtype)
    K = 2 * max(blk, 32)
    c = wl.make_case(wtype, 5, K, 3, seed=1)
    assert c["W"].dtype == np.uint8 and c["W"].shape == (5, K // blk * nbytes)
    assert c["G"].dtype == np.float32 and c["G"].shape == (3, 5)


def test_mxfp4_scales_and_codes():
    c = wl.make_case(wl.MXFP4, 64, 1024, 1, seed=2)
    blk = c["W"].reshape(64, 32, 17)
    assert blk[:, :, 0].min() == 117 and blk[:, :, 0].max() == 120
    nib = np.concatenate([blk[:, :, 1:] & 15, blk[:, :, 1:] >> 4])
    assert set(np.unique(nib)) == set(range(16))


def test_nvfp4_scales_and_codes():
    c = wl.make_case(wl.NVFP4, 64, 1024, 1, seed=2)
    blk = c["W"].reshape(64, 16, 36)
    assert blk[:, :, 0:4].min() == 0x08 and blk[:, :, 0:4].max() == 0x37
    nib = np.concatenate([blk[:, :, 4:] & 15, blk[:, :, 4:] >> 4])
    assert set(np.unique(nib)) == set(range(16))


def test_q8_0_codes_and_scales():
    c = wl.make_case(wl.Q8_0, 64, 1024, 1, seed=2)
    blocks = c["W"].reshape(-1, 34)
    d = blocks[:, 0:2].copy().view(np.float16).astype(np.float64).ravel()
    codes = blocks[:, 2:].view(np.int8)
    assert d.min() >= np.float16(1e-3) and d.max() <= np.float16(1e-2)
    assert codes.min() == -127 and codes.max() == 127
    assert abs(codes.mean()) < 1.0


def test_q4_k_fields():
    c = wl.make_case(wl.Q4_K, 64, 1024, 1, seed=2)
    blocks = c["W"].reshape(-1, 144)
    d = blocks[:, 0:2].copy().view(np.float16).astype(np.float64)
    dmin = blocks[:, 2:4].copy().view(np.float16).astype(np.float64)
    for x in (d, dmin):
        assert x.min() >= np.float16(1e-4) and x.max() <= np.float16(1e-3)
    nib = np.concatenate([blocks[:, 16:] & 15, blocks[:, 16:] >> 4]).ravel()
    assert nib.min() == 0 and nib.max() == 15
    counts = np.bincount(nib, minlength=16)
    assert counts.min() > 0.8 * counts.mean()


def test_dense_rounding_is_nearest_even():
    rng = np.random.Generator(np.random.PCG64(9))
    w = rng.standard_normal((3, 100), dtype=np.float32) * np.float32(0.02)
    c16 = wl.make_case(wl.F16, 3, 100, 2, seed=9)
    cbf = wl.make_case(wl.BF16, 3, 100, 2, seed=9)
    c32 = wl.make_case(wl.F32, 3, 100, 2, seed=9)
    assert np.array_equal(c32["W"].view(np.float32), w)
    assert np.array_equal(c16["W"].view(np.float16), w.astype(np.float16))
    ref = torch.from_numpy(w).bfloat16().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(cbf["W"].view(np.uint16), ref)
    # the three dense variants share the gradient
    assert np.array_equal(c16["G"], c32["G"]) and np.array_equal(cbf["G"], c32["G"])


def test_gradient_scale():
    c = wl.make_case(wl.Q4_0, 4096, 32, 8, seed=5, g_sigma=1e-2)
    assert abs(c["G"].std() - 1e-2) < 5e-4


def test_named_workloads_shapes():
    spec = wl.WORKLOADS
    assert spec["q4_k_n14336_k4096_t4096"]["N"] == 14336 and spec["q4_k_n14336_k4096_t4096"]["T"] == 4096
    assert spec["q4_k_n4096_k14336_t16"]["K"] == 14336
    c = wl.workload("q8_0_n128_k256_t64")
    assert c["W"].shape == (128, 272) and c["G"].shape == (64, 128)
    with pytest.raises(ValueError):
        wl.workload("dense_n4096_k4096_t512")
