"""Calls from several host threads at once, each on its own stream: the
library keeps no mutable state between calls (its launch status is read per
thread), so every result equals the one a single thread gets. ctypes
releases the interpreter lock during a foreign call, so the calls do overlap
on the host."""

import threading

import numpy as np
import pytest
import torch

import workloads as wl

q = pytest.importorskip("quantized_weight_backward_amd")

pytestmark = pytest.mark.gpu

CASES = [(wl.Q4_K, 96, 512, 160, q.VARIANT_AUTO), (wl.Q4_0, 80, 352, 9, q.VARIANT_AUTO),
         (wl.MXFP4, 64, 384, 130, q.VARIANT_SPLIT_128x128), (wl.Q6_K, 40, 256, 70, q.VARIANT_AUTO),
         (wl.BF16, 72, 264, 33, q.VARIANT_AUTO), (wl.Q2_K, 52, 512, 200, q.VARIANT_SPLIT_128x256)]


def test_concurrent_host_threads_match_one_thread():
    inputs = []
    for i, (wtype, N, K, T, v) in enumerate(CASES):
        c = wl.make_case(wtype, N, K, T, seed=2300 + i)
        inputs.append((wtype, K, v, torch.from_numpy(c["W"]).cuda(), torch.from_numpy(c["G"]).cuda()))
    ref = [q.out_prod(wtype, W, G, K, variant=v) for wtype, K, v, W, G in inputs]
    torch.cuda.synchronize()

    rounds, nthreads = 6, 4
    results = [[None] * len(inputs) for _ in range(nthreads)]
    errors = []
    start = threading.Barrier(nthreads)

    def work(tid):
        try:
            stream = torch.cuda.Stream()
            outs = [torch.empty_like(r) for r in ref]
            start.wait()
            with torch.cuda.stream(stream):
                for r in range(rounds):
                    for j in range(len(inputs)):
                        k = (j + tid + r) % len(inputs)  # threads walk the cases in different orders
                        wtype, K, v, W, G = inputs[k]
                        q.out_prod(wtype, W, G, K, out=outs[k], variant=v)
            stream.synchronize()
            results[tid] = outs
        except Exception as e:  # reported from the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(t,)) for t in range(nthreads)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    for tid in range(nthreads):
        for k, r in enumerate(ref):
            assert torch.equal(results[tid][k], r), (tid, k)
