"""The entry points under HIP graph capture: they allocate nothing and clear
nothing with memset nodes (the workspace calls' counters are left at zero by
the kernel itself), so a captured sequence of calls replays on new
inputs and matches eager calls bit for bit (the kernels are deterministic).
Inputs are updated eagerly between replays; only library calls are captured."""

import numpy as np
import pytest
import torch

import workloads as wl

q = pytest.importorskip("quantized_weight_backward_amd")

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_captured_calls_replay_like_eager_calls():
    rng = np.random.default_rng(2024)
    # large-T producer/consumer kernel, skinny kernel, exact split, a strided
    # view of G and dst, the forward, and the n-split skinny kernel through
    # a caller workspace and through the library's static one (its counters
    # are reset by the kernel, never by a memset)
    big = wl.make_case(wl.Q4_K, 96, 512, 160, seed=2101)
    thin = wl.make_case(wl.Q4_0, 80, 352, 9, seed=2102)
    spl = wl.make_case(wl.MXFP4, 64, 384, 130, seed=2103)
    few = wl.make_case(wl.Q4_K, 1024, 1024, 16, seed=2104)
    nof = wl.make_case(wl.Q6_K, 512, 768, 5, seed=2105)
    Wb, Wt, Ws, Wf, Wn = dev(big["W"]), dev(thin["W"]), dev(spl["W"]), dev(few["W"]), dev(nof["W"])
    Gb = dev(big["G"])
    Gt = dev(thin["G"])
    Gs = dev(spl["G"])
    Gf = dev(few["G"])
    Gn = dev(nof["G"])
    work = q.new_workspace()
    gpad = torch.zeros((thin["T"], thin["N"] + 12), device="cuda")
    Gv = gpad[:, 4:4 + thin["N"]]
    X = torch.randn((7, big["K"]), device="cuda")
    outs = {
        "big": torch.empty((big["T"], big["K"]), device="cuda"),
        "thin": torch.empty((thin["T"], thin["K"]), device="cuda"),
        "split": torch.empty((spl["T"], spl["K"]), device="cuda"),
        "view": torch.empty((thin["T"], thin["K"] + 8), device="cuda")[:, 8:],
        "mm": torch.empty((7, big["N"]), device="cuda"),
        "ws": torch.empty((few["T"], few["K"]), device="cuda"),
        "noalloc": torch.empty((nof["T"], nof["K"]), device="cuda"),
    }

    def calls(o):
        q.out_prod(wl.Q4_K, Wb, Gb, big["K"], out=o["big"])
        q.out_prod(wl.Q4_0, Wt, Gt, thin["K"], out=o["thin"])
        q.out_prod(wl.MXFP4, Ws, Gs, spl["K"], out=o["split"], variant=q.VARIANT_SPLIT_128x128)
        q.out_prod(wl.Q4_0, Wt, Gv, thin["K"], out=o["view"])
        q.mul_mat(wl.Q4_K, Wb, X, out=o["mm"])
        q.out_prod_ws(wl.Q4_K, Wf, Gf, few["K"], work, out=o["ws"], variant=q.VARIANT_SKINNY_SPLIT)
        q.out_prod_noalloc(wl.Q6_K, Wn, Gn, nof["K"], out=o["noalloc"], variant=q.VARIANT_SKINNY_SPLIT)

    assert q.choice(wl.Q4_K, big["K"], big["N"], big["T"]) not in (q.VARIANT_SKINNY, q.VARIANT_SIMPLE)
    assert q.choice(wl.Q4_0, thin["K"], thin["N"], thin["T"]) == q.VARIANT_SKINNY

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls(outs)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls(outs)

    ref = {k: torch.empty_like(v) for k, v in outs.items()}
    ref["view"] = torch.empty((thin["T"], thin["K"] + 8), device="cuda")[:, 8:]
    for rep in range(4):
        # new inputs, written eagerly into the captured buffers
        Gb.copy_(dev(rng.standard_normal(Gb.shape).astype(np.float32)))
        Gt.copy_(dev(rng.standard_normal(Gt.shape).astype(np.float32)))
        Gs.copy_(dev(rng.standard_normal(Gs.shape).astype(np.float32)))
        Gv.copy_(dev(rng.standard_normal(Gv.shape).astype(np.float32)))
        X.copy_(dev(rng.standard_normal(X.shape).astype(np.float32)))
        Gf.copy_(dev(rng.standard_normal(Gf.shape).astype(np.float32)))
        Gn.copy_(dev(rng.standard_normal(Gn.shape).astype(np.float32)))
        for v in outs.values():
            v.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        calls(ref)
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(outs[k], ref[k]), (rep, k)
            assert torch.isfinite(outs[k]).all().item(), (rep, k)
