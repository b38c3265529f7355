"""The C ABI on the host (no GPU): the library loads, exports what the header
declares, and every validation path returns its error before touching a
device."""

import ctypes
import glob
import itertools
import os
import random
import re
import threading

import pytest

import workloads as wl
from conftest import REPO

q = pytest.importorskip("quantized_weight_backward_amd")  # raises if the library is missing

HEADER = os.path.join(REPO, "include", "retro_out_prod.h")
KQUANT_TYPES = (wl.Q2_K, wl.Q3_K, wl.Q4_K, wl.Q5_K, wl.Q6_K)
HEADERS = sorted(glob.glob(os.path.join(REPO, "include", "*.h")))


def declared_functions():
    names = set()
    for path in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names.update(re.findall(r"\b(retro_\w+)\s*\(", text))
    return sorted(names)


def test_library_is_the_in_tree_build():
    assert os.path.dirname(q.LIB_PATH) == os.path.join(REPO, "quantized_weight_backward_amd")
    assert os.path.exists(q.LIB_PATH)


def test_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(q.EXPORTS), names
    for name in names:
        assert hasattr(q.lib, name), name


def test_enum_values_match_header():
    text = open(HEADER).read()
    for name, value in [("RETRO_F32", q.F32), ("RETRO_F16", q.F16), ("RETRO_Q4_0", q.Q4_0), ("RETRO_Q8_0", q.Q8_0),
                        ("RETRO_Q4_K", q.Q4_K), ("RETRO_Q5_K", q.Q5_K), ("RETRO_Q6_K", q.Q6_K),
                        ("RETRO_Q2_K", q.Q2_K), ("RETRO_Q3_K", q.Q3_K), ("RETRO_Q4_1", q.Q4_1),
                        ("RETRO_Q5_0", q.Q5_0), ("RETRO_Q5_1", q.Q5_1), ("RETRO_MXFP4", q.MXFP4),
                        ("RETRO_BF16", q.BF16), ("RETRO_E_TYPE", q.E_TYPE),
                        ("RETRO_E_SHAPE", q.E_SHAPE), ("RETRO_E_NULL", q.E_NULL), ("RETRO_E_ALIGN", q.E_ALIGN),
                        ("RETRO_E_ALIAS", q.E_ALIAS), ("RETRO_E_HIP", q.E_HIP), ("RETRO_E_VARIANT", q.E_VARIANT),
                        ("RETRO_VARIANT_SKINNY", q.VARIANT_SKINNY), ("RETRO_E_WORKSPACE", q.E_WORKSPACE),
                        ("RETRO_VARIANT_SKINNY_SPLIT", q.VARIANT_SKINNY_SPLIT),
                        ("RETRO_VARIANT_TILE_128x256", q.VARIANT_TILE_128x256),
                        ("RETRO_VARIANT_TILE_64x64", q.VARIANT_TILE_64x64)]:
        m = re.search(rf"\b{name}\s*=\s*(-?\d+)", text)
        assert m and int(m.group(1)) == value, name


@pytest.mark.parametrize("wtype", [wl.F32, wl.F16, wl.BF16, wl.Q8_0, wl.Q4_0, wl.Q4_1, wl.Q5_0, wl.Q5_1, wl.MXFP4,
                                   wl.NVFP4, wl.Q2_K, wl.Q3_K, wl.Q4_K, wl.Q5_K, wl.Q6_K])
def test_row_bytes_matches_the_format(wtype):
    blk, nbytes = wl.block_geometry(wtype)
    for nblocks in (0, 1, 3, 16, 56):
        assert q.row_bytes(wtype, nblocks * blk) == nblocks * nbytes
    if blk > 1:
        assert q.row_bytes(wtype, blk + 1) == -1
    assert q.row_bytes(wtype, -blk) == -1


def test_row_bytes_of_the_workloads():
    assert q.row_bytes(q.Q8_0, 256) == 272
    assert q.row_bytes(q.Q4_0, 5120) == 2880
    assert q.row_bytes(q.Q4_K, 4096) == 2304
    assert q.row_bytes(q.Q4_K, 14336) == 8064
    assert q.row_bytes(q.F16, 4096) == 8192
    assert q.row_bytes(q.Q5_K, 4096) == 2816
    assert q.row_bytes(q.Q6_K, 14336) == 11760
    assert q.row_bytes(q.Q2_K, 4096) == 1344
    assert q.row_bytes(q.NVFP4, 5120) == 2880
    assert q.row_bytes(q.Q3_K, 4096) == 1760
    assert q.row_bytes(q.Q4_1, 5120) == 3200
    assert q.row_bytes(q.Q5_0, 5120) == 3520
    assert q.row_bytes(q.Q5_1, 5120) == 3840
    assert q.row_bytes(q.MXFP4, 5120) == 2720
    assert q.row_bytes(99, 256) == -1


def test_supported():
    assert q.supported(q.Q4_K, 4096, 14336, 4096)
    assert q.supported(q.Q4_K, 14336, 4096, 16)
    assert q.supported(q.F16, 7, 3, 1)
    assert q.supported(q.Q8_0, 0, 0, 0)
    assert not q.supported(q.Q4_K, 100, 1, 1)
    assert not q.supported(q.Q4_0, 48, 1, 1)
    assert not q.supported(77, 32, 1, 1)
    assert not q.supported(q.F32, -1, 1, 1)
    assert not q.supported(q.F32, 1, 1 << 31, 1)
    assert not q.supported(q.F32, (1 << 31) - 1, 1, (1 << 31) - 1)  # T*K beyond the byte limit


def test_choice():
    assert q.choice(q.Q4_K, 14336, 4096, 16) == q.VARIANT_SKINNY
    # one round of 256 x 256 tiles (eight MFMA waves per workgroup) ties with
    # two of 128 x 256 by tile area and measures faster; fewer tiles than
    # CUs keep the smaller tiles
    assert q.choice(q.Q4_K, 4096, 14336, 4096) == q.VARIANT_WS_256x256
    assert q.choice(q.Q4_K, 4096, 14336, 8192) == q.VARIANT_WS_256x256
    assert q.choice(q.Q4_K, 4096, 14336, 2048) == q.VARIANT_WS_128x256
    assert q.choice(q.Q4_K, 14336, 4096, 4096) == q.VARIANT_WS_128x256  # 3.5 rounds of 256 x 256
    for wtype in (q.F16, q.BF16, q.Q8_0, q.Q4_0, q.MXFP4):
        assert q.choice(wtype, 4096, 11008, 4096) == q.VARIANT_WS_256x256
    assert q.choice(q.F32, 4096, 11008, 4096) == q.VARIANT_WS_128x256   # F32 rows spill there
    # Q4_0 17408 x 5120 at T = 2048: two launches (test_plan), the first 128 x 256
    assert q.choice(q.Q4_0, 5120, 17408, 2048) == q.VARIANT_WS_128x256
    assert q.choice(q.Q4_0, 5120, 17407, 2048) == q.VARIANT_TILE_64x128  # N % 4 != 0: the fallback family
    for wtype in (q.F32, q.F16, q.BF16, q.Q8_0, q.Q4_0, q.Q4_1, q.Q5_0, q.Q5_1):
        assert q.choice(wtype, 4096, 4096, 512) in q.VARIANT_NAMES
    for wtype in (q.Q4_1, q.Q5_0, q.Q5_1, q.MXFP4):  # the 32-element blocks, as Q4_0
        assert q.choice(wtype, 5120, 17408, 2048) == q.VARIANT_WS_128x256
        assert q.choice(wtype, 5120, 4096, 16) == q.VARIANT_SKINNY
        assert q.choice(wtype, 48, 1, 1) == q.E_SHAPE
    for wtype in (q.F32, q.F16, q.BF16):  # dense rows go to the producer/consumer kernel
        assert q.VARIANT_NAMES[q.choice(wtype, 4096, 4096, 512)].startswith("ws")
    # one 64 x 128 tile per CU (or F32 rows): two pipelines per workgroup
    for wtype in (q.F32, q.F16, q.BF16, q.Q4_0, q.Q8_0):
        assert q.choice(wtype, 4096, 4096, 512) == q.VARIANT_WS2_64x128
    assert q.choice(q.F32, 5120, 64, 2048) == q.VARIANT_WS2_64x128  # short reduction: one launch
    assert q.choice(q.F16, 301, 77, 200) == q.VARIANT_TILE_64x64  # 602-byte rows: no 16-byte units
    assert q.choice(q.Q4_K, 100, 1, 1) == q.E_SHAPE
    for wtype in (q.Q2_K, q.Q3_K, q.Q5_K, q.Q6_K):  # K-quants: 256-column tiles, as Q4_K
        assert q.choice(wtype, 4096, 14336, 4096) == q.VARIANT_WS_256x256
        assert q.choice(wtype, 14336, 4096, 16) == q.VARIANT_SKINNY
        assert not q.variant_applies(q.VARIANT_WS_64x128, wtype, 4096, 14336, 4096)
        assert q.choice(wtype, 128, 1, 1) == q.E_SHAPE
    assert q.choice(5, 32, 1, 1) == q.E_TYPE


def tile_dims(name):
    """(rows of T, columns of K) of a tiled variant's name, e.g. ws_128x256."""
    bt, bk = name.split("_")[-1].split("x")
    return int(bt), int(bk)


def test_plan():
    """Two launches over column ranges of dst where one tile would leave the
    last round over the 256 CUs partly empty and a larger tile fills whole
    rounds (each listed plan measured faster on MI355X than the one launch it
    replaces, e.g. Q4_0 17408 x 5120 at T = 2048: 2.77 against 2.98 ms); one
    launch elsewhere."""
    two = {
        (q.Q4_0, 5120, 17408, 2048): (q.VARIANT_WS_128x256, 4096, q.VARIANT_WS2_64x128),
        (q.Q4_K, 14336, 4096, 4096): (q.VARIANT_WS_128x256, 2048, q.VARIANT_WS_256x256),
        (q.Q4_K, 4352, 4096, 4096): (q.VARIANT_WS_256x256, 4096, q.VARIANT_WS_32x256),
        (q.Q4_K, 11008, 4096, 4096): (q.VARIANT_WS_256x256, 8192, q.VARIANT_WS_64x256),
        # below T = 1024 too: 0.88 against 1.13 ms (Q4_K), 0.91 against 1.15 ms
        # (Q6_K), 1.47 against 2.07 ms (Q2_K at T = 1000), 0.75 against 0.82 ms
        # (Q4_0 4096 x 11008)
        (q.Q4_K, 17408, 5120, 512): (q.VARIANT_WS_128x256, 16384, q.VARIANT_WS_32x256),
        (q.Q6_K, 17408, 5120, 512): (q.VARIANT_WS_128x256, 16384, q.VARIANT_WS_32x256),
        (q.Q2_K, 17408, 5120, 1000): (q.VARIANT_WS_256x256, 16384, q.VARIANT_WS_32x256),
        (q.Q4_0, 11008, 4096, 1000): (q.VARIANT_WS_128x256, 8192, q.VARIANT_WS_32x128),
    }
    for wtype in (q.Q8_0, q.Q4_1, q.Q5_0, q.Q5_1, q.MXFP4, q.NVFP4, q.F16, q.BF16, q.F32):
        two[(wtype, 5120, 17408, 2048)] = (q.VARIANT_WS_128x256, 4096, q.VARIANT_WS2_64x128)
    for (wtype, K, N, T), p in two.items():
        assert q.plan(wtype, K, N, T) == p, (wtype, K, N, T, q.plan_names(wtype, K, N, T))
        assert q.choice(wtype, K, N, T) == p[0]
    one = {
        (q.Q4_K, 4096, 14336, 4096): q.VARIANT_WS_256x256,   # 256 tiles: one whole round
        (q.Q4_K, 14336, 4096, 16): q.VARIANT_SKINNY,
        (q.F32, 4096, 4096, 512): q.VARIANT_WS2_64x128,
        (q.BF16, 4096, 4096, 512): q.VARIANT_WS2_64x128,
        (q.Q8_0, 256, 128, 64): q.VARIANT_WS_32x128,
        (q.Q4_0, 5120, 64, 2048): q.VARIANT_WS_64x128,        # saves less than a launch costs
        (q.Q4_K, 4096, 14336, 2048): q.VARIANT_WS_128x256,
    }
    for (wtype, K, N, T), v in one.items():
        assert q.plan(wtype, K, N, T) == (v, K, 0), (wtype, K, N, T, q.plan_names(wtype, K, N, T))
    assert q.plan_names(q.Q4_0, 5120, 17408, 2048) == "ws_128x256[0:4096]+ws2_64x128[4096:5120]"
    v0, v1, ks = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    assert q.lib.retro_out_prod_plan(q.Q4_0, 5120, 17408, 2048, None, ctypes.byref(ks), ctypes.byref(v1)) == q.E_NULL
    assert q.lib.retro_out_prod_plan(q.Q4_K, 100, 1, 1, ctypes.byref(v0), ctypes.byref(ks),
                                     ctypes.byref(v1)) == q.E_SHAPE


def test_plan_invariants_over_shapes():
    """Every two-launch plan over a grid of shapes splits at a whole block
    whose W bytes and dst column keep 16-byte alignment, runs variants that
    apply to their parts, and gives its first part whole rounds of tiles."""
    Ks = (1024, 2304, 4352, 5120, 11008, 14336)
    Ns = (64, 4096, 17408)
    Ts = (17, 100, 512, 2048, 4096)
    split = 0
    for wtype in q.TYPES.values():
        blk = {q.F32: 1, q.F16: 1, q.BF16: 1, q.NVFP4: 64}.get(wtype, 256 if wtype in KQUANT_TYPES else 32)
        for K, N, T in itertools.product(Ks, Ns, Ts):
            if K % blk or q.row_bytes(wtype, K) < 0:
                continue
            v0, ks, v1 = q.plan(wtype, K, N, T)
            assert q.choice(wtype, K, N, T) == v0
            if ks == K:
                assert v1 == 0
                continue
            split += 1
            assert 0 < ks < K and ks % blk == 0 and ks % 4 == 0, (wtype, K, N, T, ks)
            assert q.row_bytes(wtype, ks) % 16 == 0, (wtype, K, ks)
            assert q.variant_applies(v0, wtype, ks, N, T) and q.variant_applies(v1, wtype, K - ks, N, T)
            bt, bk = tile_dims(q.VARIANT_NAMES[v0])
            assert ks % bk == 0 and (-(-T // bt) * (ks // bk)) % 256 == 0, (wtype, K, N, T, q.VARIANT_NAMES[v0], ks)
    assert split > 20


def test_plan_is_the_same_from_the_cache():
    """Plans are kept per thread for the last few shapes: asking for more
    shapes than it holds, in two orders, gives the same answers."""
    shapes = [(q.Q4_0, 5120, 17408, 2048), (q.Q4_K, 14336, 4096, 4096), (q.Q8_0, 256, 128, 64),
              (q.F32, 4096, 4096, 512), (q.Q4_K, 4352, 4096, 4096), (q.MXFP4, 5120, 17408, 2048),
              (q.Q4_K, 14336, 4096, 16), (q.F16, 11008, 4096, 4096)]
    first = [q.plan(*sh) for sh in shapes]
    for _ in range(3):
        assert [q.plan(*sh) for sh in reversed(shapes)] == first[::-1]
        assert [q.choice(*sh) for sh in shapes] == [p[0] for p in first]


def test_workspace_size():
    """The n-split skinny kernel's workspace: 1 KiB of counters and two 4 KiB
    slots per CU for each block of 16 rows of G (T <= 48), taken
    automatically only with few slabs and enough rows."""
    def full(T=16):
        return 4 * 256 + 2 * 256 * 16 * 64 * 4 * (-(-T // 16))
    split = q.VARIANT_SKINNY_SPLIT
    assert q.workspace_size(q.Q4_K, 4096, 14336, 16) == full()    # 64 slabs
    assert q.workspace_size(q.Q4_0, 5120, 4096, 16) == full()     # 80 slabs
    assert q.workspace_size(q.Q4_K, 11008, 4096, 16) == full()    # 172 slabs
    assert q.workspace_size(q.Q4_K, 14336, 4096, 16) == 0         # 224 slabs: the skinny kernel
    assert q.workspace_size(q.Q8_0, 256, 128, 16) == 0            # too few rows to share
    assert q.workspace_size(q.Q4_K, 4096, 14336, 17) == full(17)  # two blocks of G
    assert q.workspace_size(q.Q4_K, 4096, 14336, 48) == full(48)
    assert q.workspace_size(q.Q4_K, 4096, 14336, 512) == full(48)  # passes of 48 rows of G
    for wtype in q.TYPES.values():
        K = 256 * 8
        assert q.workspace_size(wtype, K, 4096, 16, split) == full()
        assert q.workspace_size(wtype, K, 4096, 40, split) == full(40)
        assert q.workspace_size(wtype, K, 4096, 49, split) == full(48)
        assert q.workspace_size(wtype, K, 4088, 16, split) == q.E_VARIANT   # N % 16 != 0
        assert q.workspace_size(wtype, K, 0, 16, split) == q.E_VARIANT
    assert q.workspace_size(q.F32, 4094, 4096, 16, split) == q.E_VARIANT     # K % 4 != 0
    assert q.variant_applies(q.VARIANT_SKINNY, q.Q4_K, 4096, 4096, 64)          # passes of 64 rows of G
    assert q.variant_applies(q.VARIANT_SKINNY, q.Q4_K, 4096, 4096, 4096)
    assert not q.variant_applies(q.VARIANT_SKINNY_16, q.Q4_K, 4096, 4096, 17)   # sixteen waves: T <= 16
    assert q.workspace_size(q.Q4_K, 4096, 4096, 512, q.VARIANT_WS_128x256) == 0
    assert q.workspace_size(q.Q4_K, 4096, 4096, 512, q.VARIANT_SKINNY) == 0
    assert q.workspace_size(q.Q4_K, 4096, 4096, 512, q.VARIANT_SKINNY_16) == q.E_VARIANT
    assert q.workspace_size(q.Q4_K, 100, 16, 16) == q.E_SHAPE
    assert q.workspace_size(5, 32, 16, 16) == q.E_TYPE
    # the split needs the workspace call: the others refuse it
    assert not q.variant_applies(split, q.Q4_K, 4096, 4096, 16)
    assert q.lib.retro_out_prod_variant(split, q.Q4_K, 0x100000, 0x2000000, 0x3000000, 4096, 4096, 16,
                                        None) == q.E_VARIANT


def test_workspace_call_validation():
    """Errors of retro_out_prod_ws, all returned before any launch."""
    f = q.lib.retro_out_prod_ws
    W, G, D, WS = 0x10000000, 0x20000000, 0x30000000, 0x40000000
    full = q.workspace_size(q.Q4_K, 4096, 4096, 16, q.VARIANT_SKINNY_SPLIT)
    split = q.VARIANT_SKINNY_SPLIT
    args = (q.Q4_K, W, G, D, 4096, 4096, 16)
    assert f(split, q.Q4_K, W, G, D, 4096, 4096, 17, WS, full, None) == q.E_WORKSPACE  # two blocks need more
    assert f(split, *args, None, 0, None) == q.E_WORKSPACE
    assert f(split, *args, WS, full - 1, None) == q.E_WORKSPACE
    assert f(split, *args, WS + 4, full, None) == q.E_WORKSPACE          # not 16-byte aligned
    assert f(split, *args, D - 16, full, None) == q.E_WORKSPACE          # overlaps dst
    assert f(split, *args, W, full, None) == q.E_WORKSPACE               # overlaps W
    assert f(q.VARIANT_AUTO, *args, G + 64, full, None) == q.E_WORKSPACE  # overlaps G
    assert f(split, q.Q4_K, W, G, D, 4096, 4096, 49, WS, full, None) == q.E_WORKSPACE  # three blocks
    assert f(split, q.Q4_K, W, G, W, 4096, 4096, 16, WS, full, None) == q.E_ALIAS
    assert f(split, q.Q4_K, W, None, D, 4096, 4096, 16, WS, full, None) == q.E_NULL
    assert f(split, q.Q4_K, W, G, D, 100, 4096, 16, WS, full, None) == q.E_SHAPE
    assert f(99, *args, WS, full, None) == q.E_VARIANT
    assert f(split, q.Q4_K, W, G, D, 4096, 4096, 0, WS, full, None) == q.OK   # nothing to compute


def test_plans_from_many_threads():
    """The plan cache is per thread: eight threads asking for interleaved
    shapes at once (ctypes releases the GIL around each call) all get the
    plans one thread gets alone."""
    shapes = [(q.Q4_0, 5120, 17408, 2048), (q.Q4_K, 14336, 4096, 4096), (q.Q8_0, 256, 128, 64),
              (q.F32, 4096, 4096, 512), (q.Q4_K, 4352, 4096, 4096), (q.MXFP4, 5120, 17408, 2048),
              (q.Q4_K, 14336, 4096, 16), (q.F16, 11008, 4096, 4096), (q.Q6_K, 11008, 4096, 100)]
    want = [(q.plan(*sh), q.mul_mat_plan(*sh)) for sh in shapes]
    errors = []

    def worker(seed):
        order = list(range(len(shapes)))
        random.Random(seed).shuffle(order)
        for _ in range(200):
            for i in order:
                got = (q.plan(*shapes[i]), q.mul_mat_plan(*shapes[i]))
                if got != want[i]:
                    errors.append((seed, shapes[i], got, want[i]))
                    return

    threads = [threading.Thread(target=worker, args=(s,)) for s in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors[:3]


def test_mul_mat_plan():
    """The forward splits W's rows the same way: 128 x 128 tiles over 16384
    rows (8 whole rounds at T = 2048) and one round of 64 x 128 over the
    rest, where one launch would run 17 rounds of 64 x 128."""
    for wtype in (q.Q4_0, q.MXFP4, q.Q8_0):
        assert q.mul_mat_plan(wtype, 5120, 17408, 2048) == (q.VARIANT_WS_128x128, 16384, q.VARIANT_WS_64x128)
        assert q.mul_mat_choice(wtype, 5120, 17408, 2048) == q.VARIANT_WS_128x128
    for args, v in (((q.Q4_K, 4096, 14336, 4096), q.VARIANT_WS_128x128), ((q.F32, 4096, 4096, 512), q.VARIANT_WS_64x128),
                    ((q.Q4_K, 14336, 4096, 16), q.VARIANT_SKINNY), ((q.F16, 301, 64, 100), q.VARIANT_SIMPLE)):
        assert q.mul_mat_plan(*args) == (v, args[2], 0), args
    v0, v1, ns = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    assert q.lib.retro_mul_mat_plan(q.Q4_0, 5120, 17408, 2048, ctypes.byref(v0), None, ctypes.byref(v1)) == q.E_NULL
    # the two ops' plans are kept apart in the per-thread cache
    for _ in range(2):
        assert q.plan(q.Q4_0, 5120, 17408, 2048) == (q.VARIANT_WS_128x256, 4096, q.VARIANT_WS2_64x128)
        assert q.mul_mat_plan(q.Q4_0, 5120, 17408, 2048) == (q.VARIANT_WS_128x128, 16384, q.VARIANT_WS_64x128)


def test_mul_mat_plan_invariants_over_shapes():
    split = 0
    for wtype in q.TYPES.values():
        blk = {q.F32: 1, q.F16: 1, q.BF16: 1, q.NVFP4: 64}.get(wtype, 256 if wtype in KQUANT_TYPES else 32)
        for K, N, T in itertools.product((1024, 4096, 5120), (4096, 11008, 14336, 17408), (17, 512, 2048, 4096)):
            if K % blk:
                continue
            v0, ns, v1 = q.mul_mat_plan(wtype, K, N, T)
            assert q.mul_mat_choice(wtype, K, N, T) == v0
            if ns == N:
                assert v1 == 0
                continue
            split += 1
            bt, bn = tile_dims(q.VARIANT_NAMES[v0])
            assert 0 < ns < N and ns % bn == 0 and (ns * q.row_bytes(wtype, K)) % 16 == 0
            assert (-(-T // bt) * (ns // bn)) % 256 == 0, (wtype, K, N, T, ns)
            assert q.mul_mat_variant_applies(v0, wtype, K, ns, T) and q.mul_mat_variant_applies(v1, wtype, K, N - ns, T)
    assert split > 10


def test_mul_mat_row_split_validation():
    rs = q.lib.retro_mul_mat_row_split
    W, X, Y = 0x100000, 0x2000000, 0x3000000
    a, b = q.VARIANT_WS_128x128, q.VARIANT_WS_64x128
    assert rs(a, 128, b, q.Q4_0, W, X, None, 512, 256, 40, None) == q.E_NULL
    assert rs(a, 0, b, q.Q4_0, W, X, Y, 512, 256, 40, None) == q.E_SHAPE
    assert rs(a, 256, b, q.Q4_0, W, X, Y, 512, 256, 40, None) == q.E_SHAPE
    assert rs(a, 126, b, q.Q4_0, W, X, Y, 512, 256, 40, None) == q.E_ALIGN    # not a multiple of 4 rows
    assert rs(a, 100, b, q.Q8_0, W, X, Y, 416, 256, 40, None) == q.E_ALIGN    # 100 rows of 442 bytes
    assert rs(q.VARIANT_SKINNY, 128, b, q.F16, W, X, Y, 301, 256, 40, None) == q.E_VARIANT  # x rows of 301
    assert rs(42, 128, b, q.Q4_0, W, X, Y, 512, 256, 40, None) == q.E_VARIANT
    assert rs(a, 128, b, 5, W, X, Y, 512, 256, 40, None) == q.E_TYPE
    assert rs(a, 128, b, q.Q4_0, W, X, Y, 512, 256, 0, None) == q.OK         # nothing to compute


def test_views_plan():
    """Batches count toward the rounds: 16 matrices of Q4_0 200 x 1280 with
    N = 2048 fill whole rounds of 128 x 128 tiles on 1024 columns."""
    rb = q.row_bytes(q.Q4_0, 1280)
    for sgt, sgn in ((2048, 1), (1, 200)):
        assert q.views_plan(q.Q4_0, 1280, 2048, 200, rb, sgt, sgn, 1280, 4, 4) == (
            q.VARIANT_WS_128x128, 1024, q.VARIANT_WS_32x128)
    assert q.views_plan(q.Q4_0, 1280, 2048, 200, rb, 2048, 1, 1280, 1, 1)[1] == 1280
    assert q.views_plan(q.Q4_0, 5120, 17408, 2048, q.row_bytes(q.Q4_0, 5120), 17408, 1, 5120) == \
        q.plan(q.Q4_0, 5120, 17408, 2048)


def test_column_split_validation():
    """Errors of the two-launch entry point, all found before any launch
    (fake addresses, never dereferenced)."""
    cs = q.lib.retro_out_prod_column_split
    W, G, D = 0x100000, 0x200000, 0x300000
    a, b = q.VARIANT_WS_128x256, q.VARIANT_WS_64x128
    assert cs(a, 256, b, q.Q4_0, W, G, None, 512, 4, 40, None) == q.E_NULL
    assert cs(a, 0, b, q.Q4_0, W, G, D, 512, 4, 40, None) == q.E_SHAPE      # empty first part
    assert cs(a, 512, b, q.Q4_0, W, G, D, 512, 4, 40, None) == q.E_SHAPE    # empty second part
    assert cs(a, 48, b, q.Q4_0, W, G, D, 512, 4, 40, None) == q.E_SHAPE     # not a whole block
    assert cs(a, 160, b, q.Q4_0, W, G, D, 512, 4, 40, None) == q.E_ALIGN    # 90 bytes of W before it
    assert cs(a, 128, b, q.Q8_0, W, G, D, 512, 4, 40, None) == q.E_ALIGN    # 136 bytes
    assert cs(a, 256, b, q.Q4_K, W, G, D, 512, 4, 40, None) == q.E_VARIANT  # 128-column tile on Q4_K
    assert cs(q.VARIANT_SKINNY_16, 256, b, q.Q4_0, W, G, D, 512, 4, 17, None) == q.E_VARIANT
    assert cs(42, 256, b, q.Q4_0, W, G, D, 512, 4, 40, None) == q.E_VARIANT
    assert cs(a, 256, b, q.Q4_0, W, G, D, 0, 4, 40, None) == q.E_SHAPE      # K = 0: no split point
    assert cs(a, 256, b, 5, W, G, D, 512, 4, 40, None) == q.E_TYPE
    # nothing to compute: checked, then no launch
    assert cs(a, 256, b, q.Q4_0, W, G, D, 512, 4, 0, None) == q.OK
    assert cs(q.VARIANT_AUTO, 256, q.VARIANT_AUTO, q.Q4_0, W, G, D, 512, 4, 0, None) == q.OK


def test_variant_applies():
    assert q.variant_applies(q.VARIANT_SKINNY, q.Q4_K, 14336, 4096, 16)
    assert not q.variant_applies(q.VARIANT_SKINNY_16, q.Q4_K, 14336, 4096, 17)
    assert q.variant_applies(q.VARIANT_TILE_128x256, q.Q4_K, 4096, 14336, 4096)
    assert not q.variant_applies(q.VARIANT_TILE_128x128, q.Q4_K, 4096, 14336, 4096)
    assert q.variant_applies(q.VARIANT_WS_128x256, q.Q4_K, 4096, 14336, 4096)
    assert q.variant_applies(q.VARIANT_WS_256x256, q.Q4_K, 4096, 14336, 4096)
    assert q.variant_applies(q.VARIANT_WS_256x256, q.F32, 300, 76, 200)
    assert not q.variant_applies(q.VARIANT_WS_256x256, q.F32, 300, 77, 200)  # G rows not 16-byte units
    assert q.variant_applies(q.VARIANT_WS_128x128, q.F32, 300, 76, 200)      # K % 4 == 0
    assert q.variant_applies(q.VARIANT_WS_128x128, q.F16, 300, 76, 200)
    assert not q.variant_applies(q.VARIANT_WS_128x128, q.F16, 301, 76, 200)  # K % 4 != 0
    assert not q.variant_applies(q.VARIANT_WS_128x128, q.F32, 300, 77, 200)  # G rows not 16-byte units
    assert not q.variant_applies(q.VARIANT_WS_128x256, q.Q4_K, 4096, 14335, 4096)
    assert q.variant_applies(q.VARIANT_TILE_128x128, q.F16, 301, 77, 200)
    assert not q.variant_applies(99, q.F32, 32, 32, 32)
    assert not q.variant_applies(q.VARIANT_TILE_64x64, q.Q4_K, 100, 1, 1)   # bad shape
    for v in q.VARIANT_NAMES:
        assert q.variant_applies(v, q.Q8_0, 0, 5, 5)                        # empty output


def test_strided_variant_applies():
    rb = q.row_bytes(q.Q4_0, 512)
    assert q.variant_applies_strided(q.VARIANT_WS_64x128, q.Q4_0, 512, 77, 200, rb, 80, 512)    # G rows 16-byte units
    assert not q.variant_applies_strided(q.VARIANT_WS_64x128, q.Q4_0, 512, 77, 200, rb, 77, 512)
    assert q.variant_applies_strided(q.VARIANT_TILE_64x128, q.Q4_0, 512, 77, 200, rb, 77, 512)
    assert not q.variant_applies_strided(q.VARIANT_TILE_64x128, q.Q4_0, 512, 77, 200, rb, 76, 512)  # ldg < N
    assert not q.variant_applies_strided(q.VARIANT_TILE_64x128, q.Q4_0, 512, 77, 200, rb - 1, 80, 512)
    assert q.variant_applies_strided(q.VARIANT_SKINNY, q.Q4_0, 512, 77, 16, rb + 100, 1000, 600)
    # W rows must keep the alignment of a contiguous row's blocks
    assert not q.variant_applies_strided(q.VARIANT_SKINNY, q.Q4_0, 512, 77, 16, rb + 101, 1000, 600)
    assert not q.variant_applies_strided(q.VARIANT_SKINNY, q.Q4_K, 256, 8, 16, 144 + 8, 8, 256)
    assert q.variant_applies_strided(q.VARIANT_SKINNY, q.Q4_K, 256, 8, 16, 144 + 16, 8, 256)
    assert not q.variant_applies_strided(q.VARIANT_SKINNY, q.F32, 64, 8, 16, 258, 8, 64)
    assert q.variant_applies_strided(q.VARIANT_SKINNY, q.Q5_1, 64, 8, 16, 56, 8, 64)
    assert not q.variant_applies_strided(q.VARIANT_SKINNY, q.Q5_1, 64, 8, 16, 52, 8, 64)
    # contiguous strides: the same answers as the contiguous query
    for v in q.VARIANT_NAMES:
        assert q.variant_applies_strided(v, q.Q4_K, 768, 96, 130, q.row_bytes(q.Q4_K, 768), 96, 768) == \
            q.variant_applies(v, q.Q4_K, 768, 96, 130)


def test_batched_validation():
    b = q.lib.retro_out_prod_batched
    # (type, W, ldw, sw2, sw3, G, ldg, sg2, sg3, dst, ldd, sd2, sd3, K, N, T, ne02, ne03, ne2, ne3, stream)
    W, G, D = 0x100000, 0x200000, 0x300000
    ok = dict(sw=(64, 128), sg=(16, 32), sd=(16, 32), ne=(1, 1, 2, 2))

    def call(sw=ok["sw"], sg=ok["sg"], sd=ok["sd"], ne=ok["ne"], w=W, g=G, d=D):
        return b(q.F32, w, 16, sw[0], sw[1], g, 4, sg[0], sg[1], d, 4, sd[0], sd[1], 4, 4, 4, *ne, None)
    assert call(ne=(2, 1, 3, 2)) == q.E_SHAPE           # ne02 does not divide ne2
    assert call(ne=(0, 1, 2, 2)) == q.E_SHAPE           # no W matrix
    assert call(ne=(1, 1, 300, 300)) == q.E_SHAPE       # beyond 65535 batches
    assert call(sg=(-16, 32)) == q.E_SHAPE              # negative stride
    assert call(sw=(8, 128)) == q.E_ALIGN               # W matrices not 16-byte aligned
    assert call(sd=(18, 36)) == q.E_ALIGN
    assert call(sd=(8, 32)) == q.E_ALIAS                # dst matrices (16 floats) overlap along i2
    assert call(sd=(16, 16)) == q.E_ALIAS               # ... and along i3
    assert call(d=0x100010) == q.E_ALIAS                # dst over W
    assert call(ne=(1, 1, 0, 2), w=None, g=None, d=None) == q.OK   # no batches: a no-op
    assert call(w=None) == q.E_NULL


def test_views_validation_and_choice():
    v = q.lib.retro_out_prod_views
    # (type, W, ldw, sw2, sw3, G, sgt, sgn, sg2, sg3, dst, ldd, sd2, sd3, K, N, T, ne02, ne03, ne2, ne3, stream)
    W, G, D = 0x100000, 0x200000, 0x300000

    def call(sgt, sgn, K=8, N=6, T=5, g=G, d=D):
        return v(q.F32, W, 4 * K, 0, 0, g, sgt, sgn, 0, 0, d, K, 0, 0, K, N, T, 1, 1, 1, 1, None)
    assert call(6, 2) == q.E_SHAPE                       # neither stride is 1
    assert call(5, 1) == q.E_SHAPE                       # rows shorter than N
    assert call(1, 4) == q.E_SHAPE                       # columns shorter than T
    assert call(1, 5, g=0x200004) == q.E_ALIGN
    # G stored t-fastest spans (N - 1) * sgn + T floats: 4 * 30 = 120 bytes
    assert call(1, 5, d=G + 112) == q.E_ALIAS

    assert call(1, 5, d=G + 128, T=0) == q.OK              # no rows: a no-op
    assert call(1, 5, g=None) == q.E_NULL
    # the same contract through the query functions
    assert q.variant_applies_views(q.VARIANT_WS_64x128, q.Q4_0, 512, 64, 100, 288, 1, 100, 512)
    assert not q.variant_applies_views(q.VARIANT_WS_64x128, q.Q4_0, 512, 64, 100, 288, 1, 101, 512)
    assert q.variant_applies_views(q.VARIANT_TILE_64x128, q.Q4_0, 512, 64, 100, 288, 1, 101, 512)
    assert q.variant_applies_views(q.VARIANT_SKINNY, q.Q4_0, 512, 64, 16, 288, 1, 17, 512)
    assert not q.variant_applies_views(q.VARIANT_SKINNY, q.Q4_0, 512, 64, 16, 288, 1, 15, 512)
    # G stored t-fastest takes the same kernels as rows at the benchmarked shapes
    rb = q.row_bytes(q.Q4_K, 4096)
    assert q.choice_views(q.Q4_K, 4096, 14336, 4096, rb, 1, 4096, 4096) == q.choice(q.Q4_K, 4096, 14336, 4096)
    assert q.choice_views(q.Q4_K, 14336, 4096, 16, q.row_bytes(q.Q4_K, 14336), 1, 16, 14336) == q.VARIANT_SKINNY
    # a column stride off the 16-byte grid leaves the single-role tiles
    assert q.choice_views(q.Q4_0, 4096, 4096, 1000, q.row_bytes(q.Q4_0, 4096), 1, 1001, 4096) in (
        q.VARIANT_TILE_128x256, q.VARIANT_TILE_128x128, q.VARIANT_TILE_64x256, q.VARIANT_TILE_64x128,
        q.VARIANT_TILE_64x64)
    # rows: the strided entry point's rule
    assert q.choice_views(q.Q4_0, 4096, 4096, 1000, q.row_bytes(q.Q4_0, 4096), 4096, 1, 4096) == q.choice(
        q.Q4_0, 4096, 4096, 1000)
    assert q.choice_views(q.Q4_0, 4096, 4096, 1000, q.row_bytes(q.Q4_0, 4096), 3, 3, 4096) == q.E_SHAPE


def test_split_variant_applies():
    """The exact-split variant takes the five K-quant types with G by rows in
    16-byte units, and nothing else; it is never the automatic choice."""
    v = q.VARIANT_SPLIT_128x256
    assert q.variant_applies(v, q.Q4_K, 4096, 14336, 4096)
    assert q.variant_applies(v, q.Q4_K, 256, 36, 5)
    assert not q.variant_applies(v, q.Q4_K, 256, 33, 5)           # G rows of 33 floats
    for wtype in (q.Q2_K, q.Q3_K, q.Q5_K, q.Q6_K):
        assert q.variant_applies(v, wtype, 4096, 14336, 4096)
        assert not q.variant_applies(v, wtype, 256, 33, 5)
    for wtype in (q.F32, q.F16, q.BF16, q.Q8_0, q.Q4_0, q.Q4_1, q.Q5_0, q.Q5_1, q.MXFP4):
        assert not q.variant_applies(v, wtype, 4096, 4096, 512)
    rb = q.row_bytes(q.Q4_K, 512)
    assert not q.variant_applies_views(v, q.Q4_K, 512, 64, 100, rb, 1, 100, 512)   # G stored t-fastest
    assert q.variant_applies_views(v, q.Q4_K, 512, 64, 100, rb, 68, 1, 512)
    for T in (1, 16, 17, 4096):
        assert q.choice(q.Q4_K, 4096, 14336, T) != v
    # the 128-column tile: the 32-element block types with an exact decoded
    # value of at most 16 bits, and the 16-bit dense types with 16-byte rows
    v2 = q.VARIANT_SPLIT_128x128
    for wtype in (q.Q4_0, q.Q5_0, q.MXFP4, q.BF16, q.F16):
        assert q.variant_applies(v2, wtype, 5120, 17408, 2048)
        assert q.variant_applies(v2, wtype, 352, 64, 140)            # partial last tile
        assert not q.variant_applies(v2, wtype, 5120, 33, 2048)      # G rows of 33 floats
        assert q.choice(wtype, 5120, 17408, 2048) != v2
    for wtype in (q.F32, q.Q8_0, q.Q4_1, q.Q5_1, q.Q4_K, q.Q6_K):
        assert not q.variant_applies(v2, wtype, 4096, 4096, 512)
    for wtype in (q.Q4_0, q.BF16):
        assert not q.variant_applies(v, wtype, 4096, 4096, 512)
    rb = q.row_bytes(q.BF16, 64)
    assert q.variant_applies_views(v2, q.BF16, 64, 64, 100, rb, 68, 1, 64)
    assert not q.variant_applies_views(v2, q.BF16, 64, 64, 100, rb + 8, 68, 1, 64)  # rows 8-byte aligned


def test_mul_mat_validation_and_choice():
    mm = q.lib.retro_mul_mat
    # (type, W, X, Y, K, N, T, stream)
    assert mm(99, None, None, None, 32, 1, 1, None) == q.E_TYPE
    assert mm(q.Q4_K, None, None, None, 128, 1, 1, None) == q.E_SHAPE
    assert mm(q.F32, None, None, None, 4, 0, 4, None) == q.OK            # no outputs
    assert mm(q.F32, None, None, None, 4, 4, 4, None) == q.E_NULL
    assert mm(q.F32, 0x100004, 0x200000, 0x300000, 4, 4, 4, None) == q.E_ALIGN
    assert mm(q.F32, 0x100000, 0x200000, 0x100020, 4, 4, 4, None) == q.E_ALIAS   # Y over W
    assert q.lib.retro_mul_mat_variant(q.VARIANT_WS_128x256, q.F32, 0x100000, 0x200000, 0x300000, 4, 4, 4,
                                       None) == q.E_VARIANT
    assert q.mul_mat_choice(q.Q4_K, 4096, 14336, 4096) == q.VARIANT_WS_128x128
    assert q.mul_mat_choice(q.Q4_K, 14336, 4096, 16) == q.VARIANT_SKINNY
    assert q.mul_mat_choice(q.Q4_K, 14336, 4096, 17) == q.VARIANT_SKINNY     # passes: 32 tiles of 32 x 128
    assert q.mul_mat_choice(q.Q4_K, 14336, 4096, 128) == q.VARIANT_SKINNY
    assert q.mul_mat_choice(q.Q4_K, 4096, 14336, 64) == q.VARIANT_WS_32x128   # 224 tiles: one round
    assert q.mul_mat_choice(q.F16, 301, 64, 100) == q.VARIANT_SIMPLE      # x rows not in 16-byte units
    assert q.mul_mat_choice(q.F16, 301, 64, 9) == q.VARIANT_SIMPLE
    assert q.mul_mat_choice(q.F16, 300, 64, 9) == q.VARIANT_SKINNY
    assert not q.mul_mat_variant_applies(q.VARIANT_WS_64x128, q.F16, 301, 64, 100)
    assert q.mul_mat_variant_applies(q.VARIANT_SIMPLE, q.F16, 301, 64, 100)
    for wtype in (q.Q8_0, q.Q4_0, q.MXFP4, q.Q2_K, q.Q6_K, q.BF16):
        assert q.mul_mat_choice(wtype, 4096, 4096, 512) in (q.VARIANT_WS_128x128, q.VARIANT_WS_64x128)


def test_strerror_covers_every_code():
    for code in (q.OK, q.E_TYPE, q.E_SHAPE, q.E_NULL, q.E_ALIGN, q.E_ALIAS, q.E_HIP, q.E_VARIANT):
        s = q.strerror(code)
        assert s and s != "unknown error code"
    assert q.strerror(-99) == "unknown error code"


def test_validation_errors_before_any_device_work():
    lib = q.lib
    # bad type / shape
    assert lib.retro_out_prod(99, None, None, None, 32, 1, 1, None) == q.E_TYPE
    assert lib.retro_out_prod(q.Q4_K, None, None, None, 128, 1, 1, None) == q.E_SHAPE
    assert lib.retro_out_prod(q.Q4_0, None, None, None, 40, 1, 1, None) == q.E_SHAPE
    assert lib.retro_out_prod(q.F32, None, None, None, -1, 1, 1, None) == q.E_SHAPE
    assert lib.retro_out_prod(q.F32, None, None, None, 1, -1, 1, None) == q.E_SHAPE
    assert lib.retro_out_prod(q.F32, None, None, None, 1, 1, 1 << 31, None) == q.E_SHAPE
    # empty outputs are no-ops even with NULL buffers
    assert lib.retro_out_prod(q.F32, None, None, None, 0, 5, 5, None) == q.OK
    assert lib.retro_out_prod(q.Q4_K, None, None, None, 256, 5, 0, None) == q.OK
    # NULL buffers
    assert lib.retro_out_prod(q.F32, None, None, None, 4, 4, 4, None) == q.E_NULL
    assert lib.retro_out_prod(q.F32, 0x1000, 0x2000, None, 4, 4, 4, None) == q.E_NULL
    assert lib.retro_out_prod(q.F32, None, 0x2000, 0x3000, 4, 4, 4, None) == q.E_NULL
    # misaligned (fake addresses, never dereferenced)
    assert lib.retro_out_prod(q.F32, 0x100004, 0x200000, 0x300000, 4, 4, 4, None) == q.E_ALIGN
    assert lib.retro_out_prod(q.F32, 0x100000, 0x200008, 0x300000, 4, 4, 4, None) == q.E_ALIGN
    assert lib.retro_out_prod(q.F32, 0x100000, 0x200000, 0x300002, 4, 4, 4, None) == q.E_ALIGN
    # aliasing: dst (4x4 floats = 64 B) overlapping W (4 rows x 16 B) or G
    assert lib.retro_out_prod(q.F32, 0x100000, 0x200000, 0x100030, 4, 4, 4, None) == q.E_ALIAS
    assert lib.retro_out_prod(q.F32, 0x100000, 0x200000, 0x1FFFD0, 4, 4, 4, None) == q.E_ALIAS
    # variants
    assert lib.retro_out_prod_variant(42, q.F32, 0x100000, 0x200000, 0x300000, 4, 4, 4, None) == q.E_VARIANT
    assert lib.retro_out_prod_variant(q.VARIANT_SKINNY_16, q.F32, 0x100000, 0x200000, 0x300000, 4, 4, 17,
                                      None) == q.E_VARIANT
    assert lib.retro_out_prod_variant(q.VARIANT_TILE_128x128, q.Q4_K, 0x100000, 0x200000, 0x300000, 256, 4, 64,
                                      None) == q.E_VARIANT
    # strides: each at least its row, valid strides behave as retro_out_prod
    st = lib.retro_out_prod_strided
    assert st(q.F32, 0x100000, 15, 0x200000, 4, 0x300000, 4, 4, 4, 4, None) == q.E_SHAPE  # ldw < row bytes
    assert st(q.F32, 0x100000, 16, 0x200000, 3, 0x300000, 4, 4, 4, 4, None) == q.E_SHAPE  # ldg < N
    assert st(q.F32, 0x100000, 16, 0x200000, 4, 0x300000, 3, 4, 4, 4, None) == q.E_SHAPE  # ldd < K
    assert st(q.F32, 0x100000, 1 << 60, 0x200000, 4, 0x300000, 4, 4, 4, 4, None) == q.E_SHAPE  # W span too large
    assert st(q.F32, None, 0, None, 5, None, 0, 0, 5, 5, None) == q.OK                  # empty output
    assert st(q.F32, 0x100000, 16, 0x200008, 8, 0x300000, 4, 4, 4, 4, None) == q.E_ALIGN
    assert st(q.F32, 0x100000, 18, 0x200000, 4, 0x300000, 4, 4, 4, 4, None) == q.E_ALIGN  # ldw % 4 != 0
    assert st(q.Q4_0, 0x100000, 19, 0x200000, 4, 0x300000, 32, 32, 4, 4, None) == q.E_ALIGN  # ldw odd
    # dst rows 100 floats apart span (3 * 100 + 4) * 4 bytes from 0x100000: they reach W at 0x100400
    assert st(q.F32, 0x100400, 16, 0x200000, 4, 0x100000, 100, 4, 4, 4, None) == q.E_ALIAS
    assert lib.retro_out_prod_strided_variant(42, q.F32, 0x100000, 16, 0x200000, 4, 0x300000, 4, 4, 4, 4,
                                              None) == q.E_VARIANT
    # dequantize
    assert lib.retro_dequantize(99, None, None, 32, 1, None) == q.E_TYPE
    assert lib.retro_dequantize(q.Q4_K, None, None, 32, 1, None) == q.E_SHAPE
    assert lib.retro_dequantize(q.Q4_K, None, None, 0, 5, None) == q.OK
    assert lib.retro_dequantize(q.Q4_K, None, None, 256, 5, None) == q.E_NULL
    assert lib.retro_dequantize(q.Q4_K, 0x100001, 0x200000, 256, 5, None) == q.E_ALIGN
    assert lib.retro_dequantize(q.Q4_K, 0x100000, 0x100100, 256, 5, None) == q.E_ALIAS


def test_python_binding_rejects_host_tensors():
    import torch

    with pytest.raises(ValueError):
        q.out_prod(q.F32, torch.zeros(16, dtype=torch.uint8), torch.zeros(1, 4), 1)


def test_probe_validation():
    """The measured-ceiling probes refuse bad arguments before any launch."""
    mfma, copy = q.lib.retro_probe_mfma, q.lib.retro_probe_copy
    assert q.lib.retro_probe_sink_floats() == 2048 * 256
    # (kind, sink, iterations, flops, stream)
    assert mfma(2, 0x100000, 10, None, None) == q.E_TYPE
    assert mfma(q.PROBE_MFMA_F32, 0x100000, 0, None, None) == q.E_SHAPE
    assert mfma(q.PROBE_MFMA_BF16, 0x100000, (1 << 20) + 1, None, None) == q.E_SHAPE
    assert mfma(q.PROBE_MFMA_F32, None, 10, None, None) == q.E_NULL
    assert mfma(q.PROBE_MFMA_F32, 0x100002, 10, None, None) == q.E_ALIGN
    mix = q.lib.retro_probe_mfma_valu
    # (mfma_iterations, valu_iterations, sink, flops, valu_instructions, stream)
    assert mix(-1, 0, 0x100000, None, None, None) == q.E_SHAPE
    assert mix(0, (1 << 20) + 1, 0x100000, None, None, None) == q.E_SHAPE
    assert mix(1, 1, None, None, None, None) == q.E_NULL
    assert mix(1, 1, 0x100001, None, None, None) == q.E_ALIGN
    # (src, dst, bytes, stream)
    assert copy(0x100000, 0x200000, -16, None) == q.E_SHAPE
    assert copy(0x100000, 0x200000, 24, None) == q.E_SHAPE
    assert copy(None, None, 0, None) == q.OK
    assert copy(None, 0x200000, 16, None) == q.E_NULL
    assert copy(0x100008, 0x200000, 16, None) == q.E_ALIGN
    assert copy(0x100000, 0x100010, 64, None) == q.E_ALIAS


def test_noalloc_validation():
    """retro_out_prod_noalloc checks its arguments before it looks up its
    static array or touches a device."""
    f = q.lib.retro_out_prod_noalloc
    W, G, D = 0x10000000, 0x20000000, 0x30000000
    split = q.VARIANT_SKINNY_SPLIT
    assert f(split, q.F32, W, G, D, 4094, 4096, 16, None) == q.E_VARIANT  # K % 4 != 0
    assert f(split, q.Q4_K, W, G, D, 4096, 4088, 16, None) == q.E_VARIANT
    assert f(q.VARIANT_AUTO, q.Q4_K, W, None, D, 4096, 4096, 16, None) == q.E_NULL
    assert f(q.VARIANT_AUTO, q.Q4_K, W, G, W, 4096, 4096, 16, None) == q.E_ALIAS
    assert f(q.VARIANT_AUTO, q.Q4_K, W + 4, G, D, 4096, 4096, 16, None) == q.E_ALIGN
    assert f(q.VARIANT_AUTO, 5, W, G, D, 4096, 4096, 16, None) == q.E_TYPE
    assert f(99, q.Q4_K, W, G, D, 4096, 4096, 16, None) == q.E_VARIANT
    assert f(split, q.Q4_K, W, G, D, 4096, 4096, 0, None) == q.OK
