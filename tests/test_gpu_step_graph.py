"""A decode step captured as one HIP graph ("Kernel-Level Optimisations for
LLM Inference and Training", section "Fusion, CUDA graphs and
torch.compile": small-batch decode gains most from graphs). A reduced step
runs every GEMM shape of the decode-step mix at M = 8 on tile-layout weights,
in the configurations the library picks (the ones the step-mix bench
captures): square, MLP up, MLP down and vocabulary, some twice, all on one
stream and one shared workspace. Every replay, with eager work and
synchronizations between the replays, must give the eager outputs bit for
bit; the eager outputs must be within tolerance of the oracle (the
vocabulary layer on regenerated sampled block rows)."""
import numpy as np
import pytest

import oracle
from gpu_util import announce, dev_bf16, host_bits, need_gpu, torch
from workloads import WORKLOADS, act_bf16, weight_rows_bf16

pytestmark = pytest.mark.gpu

TOL = dict(rel=2.0 ** -7, abs_rms=1e-3)
M = 8
ORDER = ["square", "mlp_up", "vocab", "mlp_down", "square", "vocab", "mlp_down", "mlp_up"]


@pytest.fixture(scope="module")
def fp8bs():
    need_gpu()
    import fp8_block_scaled_fp8bs_amd as m
    m.load()
    return m


@pytest.fixture(scope="module")
def step(fp8bs):
    """Seeded weights (quantized and rearranged on the GPU) and activations
    of the four shapes, one output buffer per GEMM of the step."""
    st = {}
    for name in ("square", "mlp_up", "mlp_down", "vocab"):
        wl = WORKLOADS[name]
        announce("step weight", name, wl.n, wl.k)
        wq, ws = fp8bs.quantize_weight(dev_bf16(wl.weight()))
        wt = fp8bs.pack_weight(wq)
        x_bits = act_bf16(wl.x_seed, wl.col_seed, 32, wl.k, wl.n_outlier, wl.outlier_factor)[:M]
        st[name] = dict(wq=wq if name != "vocab" else None, wt=wt, ws=ws, x_bits=x_bits,
                        x=dev_bf16(x_bits))
        if name == "vocab":
            del wq
        torch.cuda.synchronize()
    need = max(fp8bs.workspace_bytes(M, WORKLOADS[n].n, WORKLOADS[n].k) for n in st)
    work = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    outs = [torch.empty((M, WORKLOADS[n].n), dtype=torch.bfloat16, device="cuda") for n in ORDER]
    return st, work, outs


def run_step(fp8bs, st, work, outs):
    for name, y in zip(ORDER, outs):
        s = st[name]
        fp8bs.gemm_tiles(s["x"], s["wt"], s["ws"], out=y, workspace=work)


def test_captured_step_matches_eager_and_oracle(fp8bs, step):
    st, work, outs = step
    for name in ("square", "mlp_up", "mlp_down", "vocab"):
        wl = WORKLOADS[name]
        announce("step config", name, fp8bs.tiles_select_config(M, wl.n, wl.k))
    run_step(fp8bs, st, work, outs)
    torch.cuda.synchronize()
    eager = [host_bits(y) for y in outs]
    # the same GEMM twice in the step gives the same bits
    for i, a in enumerate(ORDER):
        for j in range(i + 1, len(ORDER)):
            if ORDER[j] == a:
                assert np.array_equal(eager[i], eager[j]), (a, i, j)
    # eager outputs against the oracle
    for name in ("square", "mlp_up", "mlp_down"):
        wl = WORKLOADS[name]
        s = st[name]
        wq_ref, ws_ref = oracle.quantize_weight_ref(wl.weight())
        assert np.array_equal(s["wq"].cpu().numpy(), wq_ref)
        xq, xs = oracle.quantize_act_ref(s["x_bits"])
        ref = oracle.gemm_ref(xq, xs, wq_ref, ws_ref)
        rep = oracle.tolerance_report(eager[ORDER.index(name)], ref, **TOL)
        assert rep["finite"] and rep["n_bad"] == 0, (name, rep)
    wl = WORKLOADS["vocab"]
    xq, xs = oracle.quantize_act_ref(st["vocab"]["x_bits"])
    yv = eager[ORDER.index("vocab")]
    nbn = wl.n // 128
    refs, gots = [], []
    for c in (0, 7, nbn // 3, nbn - 1):
        qr, sr = oracle.quantize_weight_ref(weight_rows_bf16(wl.w_seed, c, 128, wl.k))
        refs.append(oracle.gemm_ref(xq, xs, qr, sr))
        gots.append(yv[:, c * 128:(c + 1) * 128])
    rep = oracle.tolerance_report(np.concatenate(gots, 1), np.concatenate(refs, 1), **TOL)
    assert rep["finite"] and rep["n_bad"] == 0, ("vocab", rep)

    # the step as one graph, replayed with eager work in between
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run_step(fp8bs, st, work, outs)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_step(fp8bs, st, work, outs)
    sq = st["square"]
    for rep_i in range(3):
        for y in outs:
            y.fill_(0)
        # eager work on the same workspace between replays
        fp8bs.gemm_tiles(sq["x"][:3].contiguous(), sq["wt"], sq["ws"], workspace=work)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, y in enumerate(outs):
            assert np.array_equal(host_bits(y), eager[i]), f"replay {rep_i}, GEMM {i} ({ORDER[i]})"
