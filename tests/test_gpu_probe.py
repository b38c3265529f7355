"""The measured-ceiling probes on the GPU: the copy is exact, the matrix-core
loop reports the FLOPs it performs and leaves finite sums. (They compute
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
