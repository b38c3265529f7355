"""The workspace entry point, retro_out_prod_ws, and its n-split skinny
kernel against the CPU oracle on cuda:0: every weight type, shares shorter
and longer than a slab, idle waves, a partial last slab, determinism, the
counters left at zero, and the choice between the split and the kernels of
retro_out_prod. Bars as in test_gpu_parity.py."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from test_gpu_parity import KQUANTS, ORACLE_THREADS, TYPES, check_close, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import quantized_weight_backward_amd as q

    return q


@pytest.fixture(scope="module")
def ws(q):
    return q.new_workspace()


def counters(q, ws):
    """The workspace's counter words (zero between calls)."""
    torch.cuda.synchronize()
    return ws[: 4 * 256].view(torch.int32).cpu().numpy()


def split(q, ws, c, variant=None):
    W, G = dev(c["W"]), dev(c["G"])
    out = torch.full((c["T"], c["K"]), float("nan"), dtype=torch.float32, device="cuda")
    v = q.VARIANT_SKINNY_SPLIT if variant is None else variant
    q.out_prod_ws(c["type"], W, G, c["K"], ws, out=out, variant=v)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def block_k(wtype, slabs_wanted):
    """A K near slabs_wanted 64-column slabs, in whole blocks, ending in a
    partial slab where the block allows it."""
    blk = 256 if wtype in KQUANTS else (64 if wtype == wl.NVFP4 else 32)
    k = slabs_wanted * 64 - 32
    return max(blk, k // blk * blk)


# (slabs, N, T): shares of a few groups (idle waves, many pieces per slab),
# of about a slab, and longer than a slab (whole slabs inside a share: 260
# slabs); N = 16 puts every slab whole in one share; T from 1 to 48 in one
# pass over W, and T = 100 in three (48, 48 and 4 rows of G).
SHAPES = [(12, 1024, 16), (12, 16, 5), (40, 4096, 1), (100, 2048, 16), (260, 32, 3), (20, 512, 40), (30, 256, 48),
          (12, 1024, 17), (12, 512, 100)]


@pytest.mark.parametrize("wtype", TYPES)
@pytest.mark.parametrize("slabs,N,T", SHAPES)
def test_split_matches_oracle(q, ws, wtype, slabs, N, T):
    K = block_k(wtype, slabs)
    c = wl.make_case(wtype, N, K, T, seed=900 + slabs + N + T)
    assert q.workspace_size(wtype, K, N, T, q.VARIANT_SKINNY_SPLIT) > 0
    _, acc, ab = oracle.out_prod(wtype, c["W"], c["G"], K, nthreads=ORACLE_THREADS)
    y = split(q, ws, c)
    check_close(y, acc, ab, (wtype, K, N, T))
    assert not counters(q, ws).any()
    # the same bits again: slots are added in a fixed order whoever finishes last
    y2 = split(q, ws, c)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("wtype", [t for t in TYPES if t not in (wl.F32, wl.Q2_K, wl.NVFP4)])
@pytest.mark.parametrize("T", [16, 33])
def test_split_f32_twin(q, ws, wtype, T):
    """The split on Qx and on F32 rows holding the decoded values sum the same
    products in the same order (both with eight waves)."""
    K = block_k(wtype, 30)
    c = wl.make_case(wtype, 512, K, T, seed=950)
    w32 = oracle.dequantize(wtype, c["W"], K)
    twin = dict(c, type=wl.F32, W=w32.view(np.uint8))
    a, b = split(q, ws, c), split(q, ws, twin)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_auto_takes_the_split_where_it_pays(q, ws):
    """Q4_K, K = 4096, N = 14336, T = 16 (64 slabs): the automatic choice with
    a workspace runs the split, without one (or with one too small) what
    retro_out_prod runs; the 224-slab shape keeps the skinny kernel."""
    K, N, T = 4096, 14336, 16
    assert q.workspace_size(q.Q4_K, K, N, T) == q.workspace_size(q.Q4_K, K, N, T, q.VARIANT_SKINNY_SPLIT) > 0
    assert q.workspace_size(q.Q4_K, 14336, 4096, 16) == 0
    c = wl.workload("q4_k_n14336_k4096_t16")
    W, G = dev(c["W"]), dev(c["G"])
    forced = q.out_prod_ws(q.Q4_K, W, G, K, ws, variant=q.VARIANT_SKINNY_SPLIT)
    auto = q.out_prod_ws(q.Q4_K, W, G, K, ws)
    plain = q.out_prod(q.Q4_K, W, G, K)
    no_ws = q.out_prod_ws(q.Q4_K, W, G, K, None)
    small = q.out_prod_ws(q.Q4_K, W, G, K, ws[:4096])
    torch.cuda.synchronize()
    assert torch.equal(auto.view(torch.int32), forced.view(torch.int32))
    assert torch.equal(no_ws.view(torch.int32), plain.view(torch.int32))
    assert torch.equal(small.view(torch.int32), plain.view(torch.int32))
    _, acc, ab = oracle.out_prod(q.Q4_K, c["W"], c["G"], K, nthreads=ORACLE_THREADS)
    check_close(auto.cpu().numpy(), acc, ab, "split, whole output")
    check_close(plain.cpu().numpy(), acc, ab, "skinny, whole output")
    assert not counters(q, ws).any()


def test_shapes_in_turn_share_one_workspace(q, ws):
    """Calls of different shapes and types, back to back on one stream, each
    leave the counters at zero for the next."""
    shapes = [(wl.Q4_0, 2048, 4096 - 32, 16), (wl.Q6_K, 256, 2048, 4), (wl.BF16, 4096, 1000, 16)]
    cases = [wl.make_case(wt, n, k, t, seed=970 + i) for i, (wt, n, k, t) in enumerate(shapes)]
    cases.append(cases[0])  # the first call again, after the others
    outs = []
    for c in cases:
        W, G = dev(c["W"]), dev(c["G"])
        outs.append(q.out_prod_ws(c["type"], W, G, c["K"], ws, variant=q.VARIANT_SKINNY_SPLIT))
    torch.cuda.synchronize()
    assert not counters(q, ws).any()
    for c, y in zip(cases, outs):
        _, acc, ab = oracle.out_prod(c["type"], c["W"], c["G"], c["K"], nthreads=ORACLE_THREADS)
        check_close(y.cpu().numpy(), acc, ab, (c["type"], c["K"], c["N"], c["T"]))
    assert torch.equal(outs[0].view(torch.int32), outs[3].view(torch.int32))


def test_two_streams_with_their_own_workspaces(q):
    """Split calls on two streams at once, each stream with its own
    workspace, give the bits of the same calls made one after another."""
    cases = [wl.make_case(wl.Q4_K, 1024, 2048, 16, seed=975), wl.make_case(wl.Q4_0, 2048, 1024 - 32, 9, seed=976)]
    ins = [(dev(c["W"]), dev(c["G"])) for c in cases]
    want = [q.out_prod_ws(c["type"], W, G, c["K"], q.new_workspace(), variant=q.VARIANT_SKINNY_SPLIT)
            for c, (W, G) in zip(cases, ins)]
    spaces = [q.new_workspace(), q.new_workspace()]
    outs = [[torch.empty_like(y) for _ in range(4)] for y in want]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for i in range(4):
        for j, (c, (W, G)) in enumerate(zip(cases, ins)):
            with torch.cuda.stream(streams[j]):
                q.out_prod_ws(c["type"], W, G, c["K"], spaces[j], out=outs[j][i], variant=q.VARIANT_SKINNY_SPLIT,
                              stream=streams[j])
    torch.cuda.synchronize()
    for j in range(2):
        assert not counters(q, spaces[j]).any()
        for y in outs[j]:
            assert torch.equal(y.view(torch.int32), want[j].view(torch.int32)), (j, cases[j]["type"])


def test_other_variants_through_the_workspace_call(q, ws):
    """Variants that need no workspace run as retro_out_prod_variant would."""
    c = wl.make_case(wl.Q8_0, 300, 512, 40, seed=980)
    W, G = dev(c["W"]), dev(c["G"])
    for v in (q.VARIANT_WS_64x128, q.VARIANT_TILE_64x64, q.VARIANT_AUTO):
        assert q.workspace_size(wl.Q8_0, 512, 300, 40, v) == 0
        a = q.out_prod_ws(wl.Q8_0, W, G, 512, ws, variant=v)
        b = q.out_prod(wl.Q8_0, W, G, 512, variant=v)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), v


def test_workspace_errors_on_the_device_path(q, ws):
    """A forced split without a usable workspace is refused before any launch;
    dst is left untouched."""
    c = wl.make_case(wl.Q4_K, 64, 1024, 16, seed=990)
    W, G = dev(c["W"]), dev(c["G"])
    out = torch.full((16, 1024), 7.0, device="cuda")
    f = q.lib.retro_out_prod_ws
    st = torch.cuda.current_stream().cuda_stream
    args = (q.VARIANT_SKINNY_SPLIT, q.Q4_K, W.data_ptr(), G.data_ptr(), out.data_ptr(), 1024, 64, 16)
    assert f(*args, None, 0, st) == q.E_WORKSPACE
    assert f(*args, ws.data_ptr(), 1024, st) == q.E_WORKSPACE
    assert f(*args, ws.data_ptr() + 4, ws.numel() - 4, st) == q.E_WORKSPACE
    assert f(*args, out.data_ptr(), ws.numel(), st) == q.E_WORKSPACE  # overlaps dst
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
