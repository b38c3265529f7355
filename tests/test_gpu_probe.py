"""The measured-ceiling probes on the GPU: the copy is exact, the matrix-core
loops report the work they perform and leave finite sums. (They compute
nothing of OUT_PROD; bench.py times them.)"""

import numpy as np
import pytest
import torch

q = pytest.importorskip("quantized_weight_backward_amd")

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 16, 3 << 20])
def test_copy_probe_is_exact(nbytes):
    g = torch.Generator(device="cpu").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).cuda()
    dst = torch.zeros_like(src)
    q.probe_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


@pytest.mark.parametrize("kind,per_mfma", [(q.PROBE_MFMA_F32, 4096), (q.PROBE_MFMA_BF16, 32768)])
def test_mfma_probe(kind, per_mfma):
    sink = q.probe_sink()
    sink.fill_(float("nan"))
    flops = q.probe_mfma(kind, sink, 16)
    torch.cuda.synchronize()
    assert flops == 2048 * 4 * 16 * 4 * per_mfma
    s = sink.cpu().numpy()
    assert np.isfinite(s).all() and (s > 0).all()


@pytest.mark.parametrize("mfma_it,valu_it", [(16, 0), (0, 16), (16, 32)])
def test_mfma_valu_probe(mfma_it, valu_it):
    sink = q.probe_sink()
    sink.fill_(float("nan"))
    flops, instrs = q.probe_mfma_valu(sink, mfma_it, valu_it)
    torch.cuda.synchronize()
    assert flops == 512 * 4 * mfma_it * 4 * 2048
    assert instrs == 512 * 4 * valu_it * 16
    s = sink[:512 * 512].cpu().numpy().reshape(512, 8, 64)
    assert np.isfinite(s).all()
    # MFMA waves: 0 with no iterations, positive sums otherwise; FMA waves
    # end near their start values 1 + lane/1024 + chain, summed over 8 chains
    assert (s[:, :4] > 0).all() if mfma_it else (s[:, :4] == 0).all()
    lanes = 8 * (1 + np.arange(64) / 1024) + 28
    assert np.allclose(s[:, 4:], lanes, rtol=1e-4)
