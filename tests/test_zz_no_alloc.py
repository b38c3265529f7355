"""retro_out_prod_noalloc, the entry point for callers that cannot allocate,
through the C ABI on cuda:0: its output equals that of retro_out_prod_ws with
a caller-owned workspace (the same kernels, so bit for bit) and the oracle,
on two calls in a row, the second with a smaller input, and a call that
needs no workspace equals retro_out_prod."""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from test_gpu_parity import ORACLE_THREADS, check_close, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import quantized_weight_backward_amd as q

    return q


def noalloc(q, c, variant):
    W, G = dev(c["W"]), dev(c["G"])
    out = torch.full((c["T"], c["K"]), float("nan"), dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    rc = q.lib.retro_out_prod_noalloc(variant, c["type"], W.data_ptr(), G.data_ptr(), out.data_ptr(), c["K"], c["N"],
                                      c["T"], st)
    assert rc == q.OK, q.strerror(rc)
    return W, G, out


def with_workspace(q, c, W, G, variant):
    ws = q.new_workspace()
    out = torch.full((c["T"], c["K"]), float("nan"), dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    rc = q.lib.retro_out_prod_ws(variant, c["type"], W.data_ptr(), G.data_ptr(), out.data_ptr(), c["K"], c["N"],
                                 c["T"], ws.data_ptr(), ws.numel(), st)
    assert rc == q.OK, q.strerror(rc)
    return out


@pytest.mark.parametrize("variant_name", ["auto", "skinny_split"])
def test_noalloc_matches_the_workspace_call_on_two_calls(q, variant_name):
    variant = q.VARIANT_AUTO if variant_name == "auto" else q.VARIANT_SKINNY_SPLIT
    # a large call (64 slabs, 896 row groups per slab), then a smaller one
    # of another type that leaves part of the array from the first call
    cases = [wl.make_case(wl.Q4_K, 14336, 4096, 16, seed=1001), wl.make_case(wl.Q4_0, 2048, 2048 - 32, 8, seed=1002)]
    for c in cases:
        assert q.workspace_size(c["type"], c["K"], c["N"], c["T"], variant) > 0
        W, G, got = noalloc(q, c, variant)
        want = with_workspace(q, c, W, G, variant)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), want.view(torch.int32)), c["type"]
        _, acc, ab = oracle.out_prod(c["type"], c["W"], c["G"], c["K"], nthreads=ORACLE_THREADS)
        check_close(got.cpu().numpy(), acc, ab, (c["type"], c["K"], c["N"], c["T"]))


def test_noalloc_without_the_split_is_retro_out_prod(q):
    c = wl.make_case(wl.Q8_0, 300, 512, 40, seed=1003)  # T > 16: a tiled kernel, no workspace
    assert q.workspace_size(wl.Q8_0, 512, 300, 40) == 0
    W, G, got = noalloc(q, c, q.VARIANT_AUTO)
    want = q.out_prod(wl.Q8_0, W, G, 512)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), want.view(torch.int32))
