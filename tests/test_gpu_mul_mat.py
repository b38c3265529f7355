"""mul_mat, the forward y = x W^T through the packed weight, on cuda:0
against the CPU oracle (oracle.mul_mat), with the bars of the OUT_PROD
parity tests: NMSE <= 1e-7, max relative error <= 1e-5 per output (relative
to sum_k |W[n][k] x[t][k]|), and the internal 2e-6 gate.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

NMSE_MAX = 1e-7
REL_MAX = 1e-5
REL_TIGHT = 2e-6
ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))

TYPES = [wl.F32, wl.F16, wl.BF16, wl.Q8_0, wl.Q4_0, wl.Q4_1, wl.Q5_0, wl.Q5_1, wl.MXFP4, wl.NVFP4, wl.Q2_K, wl.Q3_K,
         wl.Q4_K, wl.Q5_K, wl.Q6_K]
VARIANTS = ["auto", "ws_256x128", "ws_128x128", "ws_64x128", "ws_32x128", "skinny", "simple"]
# K per type: several 32-column chunks and, for the K-quants, several
# super-blocks; dense K not a multiple of 32 (a partial last chunk)
K_OF = {wl.F32: 300, wl.F16: 264, wl.BF16: 520, wl.Q8_0: 416, wl.Q4_0: 352, wl.Q4_1: 192, wl.Q5_0: 416,
        wl.Q5_1: 352, wl.MXFP4: 352, wl.NVFP4: 320, wl.Q2_K: 512, wl.Q3_K: 768, wl.Q4_K: 768, wl.Q5_K: 512, wl.Q6_K: 768}
# (T, N): ragged in both, one below the 32-row tile, one spanning several tiles
SHAPES = [(200, 77), (20, 130), (67, 256), (16, 100), (5, 33)]


@pytest.fixture(scope="module")
def q():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import quantized_weight_backward_amd as q
    return q


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def vid(q, name):
    return q.VARIANT_AUTO if name == "auto" else {v: k for k, v in q.VARIANT_NAMES.items()}[name]


def check_close(y, acc, ab, label=""):
    e = oracle.errors(y, acc, ab)
    assert e["nonfinite"] == 0, (label, e)
    assert e["nmse"] <= NMSE_MAX, (label, e)
    assert e["max_rel"] <= REL_MAX, (label, e)
    assert e["max_rel"] <= REL_TIGHT, (label, e)
    return e


def run(q, wtype, W, x, N, variant="auto", prefill=float("nan")):
    out = torch.full((x.shape[0], N), prefill, dtype=torch.float32, device="cuda")
    q.mul_mat(wtype, dev(W), dev(x), N=N, out=out, variant=vid(q, variant))
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("wtype", TYPES)
@pytest.mark.parametrize("shape", SHAPES)
def test_mul_mat_matches_oracle(q, wtype, shape):
    T, N = shape
    K = K_OF[wtype]
    c = wl.make_case(wtype, N, K, 1, seed=700 + T)
    x = wl.make_input(T, K, seed=800 + N)
    _, acc, ab = oracle.mul_mat(wtype, c["W"], x, K, nthreads=ORACLE_THREADS)
    ran = []
    for v in VARIANTS:
        if v != "auto" and not q.mul_mat_variant_applies(vid(q, v), wtype, K, N, T):
            continue
        check_close(run(q, wtype, c["W"], x, N, v), acc, ab, v)
        ran.append(v)
    dense = wtype in (wl.F32, wl.F16, wl.BF16)
    tiled = {"ws_256x128", "ws_128x128", "ws_64x128", "ws_32x128"}
    assert ("simple" in ran) and (tiled <= set(ran)) == (not dense or K % 4 == 0), ran
    assert "skinny" in ran, ran  # any T, one pass per 16 rows of x


@pytest.mark.parametrize("wtype", [wl.Q4_K, wl.Q6_K, wl.MXFP4, wl.NVFP4, wl.Q5_1, wl.BF16])
def test_mul_mat_f32_twin_on_device(q, wtype):
    """The same tile on identical decoded values: bit-identical to the F32
    weight holding them."""
    K = K_OF[wtype]
    c = wl.make_case(wtype, 96, K, 1, seed=41)
    x = wl.make_input(130, K, seed=42)
    w32 = oracle.dequantize(wtype, c["W"], K)
    for v in ["ws_128x128", "ws_32x128"]:
        a = run(q, wtype, c["W"], x, 96, v)
        b = run(q, wl.F32, w32.view(np.uint8), x, 96, v)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), v


def test_mul_mat_decode_through_identity(q):
    """x = I (T = K): y[t][n] = W[n][t], the decoded weight transposed, bit
    for bit, for every type through the automatically chosen kernel."""
    for wtype in TYPES:
        K = 256 if wtype not in (wl.F32, wl.F16, wl.BF16) else 64
        c = wl.make_case(wtype, 40, K, 1, seed=43)
        ref = oracle.dequantize(wtype, c["W"], K)
        y = run(q, wtype, c["W"], np.eye(K, dtype=np.float32), 40)
        assert np.array_equal(y, ref.T), wl.TYPE_NAMES[wtype]


def test_mul_mat_edges(q):
    # K = 0: the empty sum
    out = torch.full((5, 7), 3.0, device="cuda")
    q.mul_mat(wl.F32, torch.zeros(0, dtype=torch.uint8, device="cuda"), torch.zeros((5, 0), device="cuda"), N=7,
              out=out)
    torch.cuda.synchronize()
    assert not out.any()
    # dense K % 4 != 0 takes the simple kernel
    assert q.mul_mat_choice(wl.F16, 301, 64, 100) == q.VARIANT_SIMPLE
    c = wl.make_case(wl.F16, 64, 301, 1, seed=44)
    x = wl.make_input(100, 301, seed=45)
    _, acc, ab = oracle.mul_mat(wl.F16, c["W"], x, 301)
    check_close(run(q, wl.F16, c["W"], x, 64), acc, ab, "simple")
    # every output written, deterministic
    c = wl.make_case(wl.Q4_K, 70, 512, 1, seed=46)
    x = wl.make_input(90, 512, seed=47)
    a = run(q, wl.Q4_K, c["W"], x, 70, prefill=float("nan"))
    b = run(q, wl.Q4_K, c["W"], x, 70, prefill=1e30)
    assert np.isfinite(a).all() and np.array_equal(a.view(np.uint32), b.view(np.uint32))


# (type, K, N, T, n_split, variant0, variant1): ragged parts, every kernel
# family, split points that keep W's and Y's 16-byte alignment
ROW_SPLITS = [
    (wl.Q4_0, 352, 300, 200, 256, "ws_128x128", "ws_64x128"),
    (wl.Q4_K, 768, 260, 67, 128, "ws_32x128", "ws_128x128"),
    (wl.F32, 300, 200, 130, 128, "ws_256x128", "simple"),
    (wl.MXFP4, 352, 260, 16, 128, "skinny", "skinny"),
    (wl.BF16, 520, 136, 90, 4, "simple", "ws_64x128"),
    (wl.Q8_0, 416, 200, 40, 104, "auto", "auto"),
    (wl.NVFP4, 320, 160, 33, 128, "ws_128x128", "ws_32x128"),
]


@pytest.mark.parametrize("wtype,K,N,T,ns,v0,v1", ROW_SPLITS)
def test_mul_mat_row_split_matches_parts_and_oracle(q, wtype, K, N, T, ns, v0, v1):
    """retro_mul_mat_row_split: the whole Y (NaN-prefilled) within the bars of
    the oracle, and each column range of Y bit-identical to its variant run
    alone on those rows of W."""
    c = wl.make_case(wtype, N, K, 1, seed=900 + N)
    x = wl.make_input(T, K, seed=901 + T)
    out = torch.full((T, N), float("nan"), device="cuda")
    q.mul_mat_row_split(wtype, dev(c["W"]), dev(x), N, vid(q, v0), ns, vid(q, v1), out=out)
    torch.cuda.synchronize()
    y = out.cpu().numpy()
    _, acc, ab = oracle.mul_mat(wtype, c["W"], x, K, nthreads=ORACLE_THREADS)
    check_close(y, acc, ab, f"{v0}+{v1}")
    rows = np.asarray(c["W"]).reshape(N, wl.row_bytes(wtype, K))
    for part, v, cols in ((rows[:ns], v0, slice(0, ns)), (rows[ns:], v1, slice(ns, N))):
        n = part.shape[0]
        assert v == "auto" or q.mul_mat_variant_applies(vid(q, v), wtype, K, n, T), v
        alone = run(q, wtype, np.ascontiguousarray(part), x, n, v)
        assert np.array_equal(y[:, cols].view(np.uint32), alone.view(np.uint32)), v


@pytest.mark.parametrize("name", ["q4_k_n14336_k4096_t4096", "q4_0_n17408_k5120_t2048", "mxfp4_n17408_k5120_t2048"])
def test_mul_mat_full_size_sampled_rows(q, name):
    """The forward at the OUT_PROD workloads' weights (y = x W^T with x of
    T x K), checked on sampled t rows the oracle computes one by one; the
    17408-row weights run their two-launch plan."""
    c = wl.workload(name)
    K, N, T = c["K"], c["N"], c["T"]
    print(f"mul_mat {name}: {q.mul_mat_plan_names(c['type'], K, N, T)}", flush=True)
    x = wl.make_input(T, K, seed=1100)
    y = q.mul_mat(c["type"], dev(c["W"]), dev(x), N=N)
    again = q.mul_mat(c["type"], dev(c["W"]), dev(x), N=N)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all().item() and torch.equal(y, again)
    rows = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(6).integers(0, T, size=10)]))
    _, acc, ab = oracle.mul_mat(c["type"], c["W"], x, K, rows=rows, nthreads=ORACLE_THREADS)
    e = check_close(y[torch.from_numpy(rows).cuda()].cpu().numpy(), acc, ab, name)
    print(f"mul_mat {name}: nmse={e['nmse']:.3e} max_rel={e['max_rel']:.3e}")
