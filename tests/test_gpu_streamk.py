"""GPU parity of the stream-K decode GEMM (path MFMA_STREAMK) against the CPU
oracle: every compiled kernel shape, both weight layouts, K cut into one or
several chunks, tiles cut into pieces by uneven stream-K runs (ragged K),
m on both sides of 16; full outputs within 2^-7 |ref| + 1e-3 rms(ref) of the
fp64 reference on the same codes; the pre-quantized route and the tile
layout give the same bits as the fused row-major call; run-to-run bit
identity; workspaces that start as arbitrary bytes and are shared between
calls and graph replays."""
import numpy as np
import pytest

import oracle
from gpu_util import announce, dev_bf16, host_bits, need_gpu, same_bits_f32, torch
from workloads import WORKLOADS, act_bf16, bf16_from_f32

pytestmark = pytest.mark.gpu

TOL = dict(rel=2.0 ** -7, abs_rms=1e-3)

# (streaming waves, tiles in flight per wave, tiles requested before the cast)
SK_SHAPES = [(8, 7, 2), (6, 8, 3)]


@pytest.fixture(scope="module")
def fp8bs():
    need_gpu()
    import fp8_block_scaled_fp8bs_amd as m
    m.load()
    return m


class Problem:
    def __init__(self, fp8bs, w_bits, x_bits):
        self.w_bits, self.x_bits = w_bits, x_bits
        self.x = dev_bf16(x_bits)
        self.wq, self.ws = fp8bs.quantize_weight(dev_bf16(w_bits))
        self.wt = fp8bs.pack_weight(self.wq)
        self.wq_ref, self.ws_ref = oracle.quantize_weight_ref(w_bits)
        assert np.array_equal(self.wq.cpu().numpy(), self.wq_ref)
        assert same_bits_f32(self.ws.cpu().numpy(), self.ws_ref)
        self.xq_ref, self.xs_ref = oracle.quantize_act_ref(x_bits)

    def ref(self, m):
        return oracle.gemm_ref(self.xq_ref[:m], self.xs_ref[:m], self.wq_ref, self.ws_ref)


def _random_problem(fp8bs, m, n, k, seed):
    rng = np.random.default_rng(seed)
    w = bf16_from_f32((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[:, rng.choice(k, max(1, k // 100), replace=False)] *= 10
    return Problem(fp8bs, w, bf16_from_f32(x))


# (n, k, split): K = 13 blocks cut into runs of 3-4 units (tiles in up to 5
# pieces); K = 8 blocks as 4 chunks of whole cells (every tile 4 pieces);
# 8 whole tiles per workgroup plus a stream-K part of 1-unit runs; 2 chunks
PROBLEMS = {"ragged": (5120, 1664, 1), "chunks": (5120, 1024, 4), "wide": (34816, 256, 1),
            "two_chunks": (4096, 1024, 2)}


@pytest.fixture(scope="module")
def problems(fp8bs):
    out = {}
    for i, (name, (n, k, _)) in enumerate(PROBLEMS.items()):
        announce("stream-K problem", name, n, k)
        out[name] = _random_problem(fp8bs, 32, n, k, 4100 + i)
    torch.cuda.synchronize()
    return out


def _run(fp8bs, pr, cfg, m):
    import dataclasses
    x = pr.x[:m].contiguous()
    y = fp8bs.gemm_ex(cfg, pr.wq, pr.ws, x=x)
    xq, xs = fp8bs.quantize_act(x)
    yq = fp8bs.gemm_ex(cfg, pr.wq, pr.ws, x_q=xq, x_s=xs)
    tcfg = dataclasses.replace(cfg, weight_layout=fp8bs.LAYOUT_TILES)
    yt = fp8bs.gemm_ex(tcfg, pr.wt, pr.ws, x=x)
    torch.cuda.synchronize()
    yb = host_bits(y)
    rep = oracle.tolerance_report(yb, pr.ref(m), **TOL)
    assert rep["finite"] and rep["n_bad"] == 0, f"{cfg} m={m}: {rep}"
    assert np.array_equal(yb, host_bits(yq)), f"pre-quantized route differs {cfg} m={m}"
    assert np.array_equal(yb, host_bits(yt)), f"tile layout differs {cfg} m={m}"
    return yb


def _cases():
    out = []
    for shape in SK_SHAPES:
        for m in (1, 5, 8, 16, 17, 32):
            out.append(("ragged", shape, m))
        for name in ("chunks", "wide", "two_chunks"):
            for m in (3, 8, 24):
                out.append((name, shape, m))
    return out


@pytest.mark.parametrize("name,shape,m", _cases())
def test_every_streamk_config(fp8bs, problems, name, shape, m):
    from fp8_block_scaled_fp8bs_amd import GemmConfig
    wk, d, pre = shape
    n, k, split = PROBLEMS[name]
    cfg = GemmConfig(fp8bs.PATH_MFMA_STREAMK, pre, 1, wk, d, split)
    announce("stream-K", name, cfg, "m", m)
    _run(fp8bs, problems[name], cfg, m)


@pytest.mark.parametrize("shape", SK_SHAPES)
@pytest.mark.parametrize("name,m", [("ragged", 8), ("ragged", 1), ("ragged", 20), ("wide", 8),
                                    ("wide", 32)])
def test_whole_tile_partition(fp8bs, problems, name, shape, m):
    """waves_n = 2: whole tiles only, 1 or 2 tiles per workgroup (ragged:
    320 tiles; wide: 2176 tiles, 8 or 9 per workgroup), no workspace."""
    from fp8_block_scaled_fp8bs_amd import GemmConfig
    wk, d, pre = shape
    cfg = GemmConfig(fp8bs.PATH_MFMA_STREAMK, pre, 2, wk, d, 1)
    announce("stream-K whole", name, cfg, "m", m)
    assert fp8bs.config_workspace_bytes(cfg, m, *PROBLEMS[name][:2]) == 0
    _run(fp8bs, problems[name], cfg, m)


@pytest.fixture(scope="module")
def full(fp8bs):
    out = {}
    for name in ("square", "mlp_down"):
        wl = WORKLOADS[name]
        announce("full-size weight", name, wl.n, wl.k)
        x_bits = act_bf16(wl.x_seed, wl.col_seed, 32, wl.k, wl.n_outlier, wl.outlier_factor)
        out[name] = Problem(fp8bs, wl.weight(), x_bits)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name,split,whole", [("square", 1, 0), ("square", 4, 0),
                                              ("mlp_down", 4, 0), ("mlp_down", 8, 0),
                                              ("square", 1, 1)])
@pytest.mark.parametrize("m", [1, 8, 16])
def test_streamk_full_size(fp8bs, full, name, split, whole, m):
    """The square (5120 x 5120) and MLP-down (17408 -> 5120) weights with their
    seeded activations, full output, one and several K chunks, and the
    whole-tile partition."""
    from fp8_block_scaled_fp8bs_amd import GemmConfig
    cfg = GemmConfig(fp8bs.PATH_MFMA_STREAMK, 2, 1 + whole, 8, 7, split)
    announce("stream-K full", name, cfg, "m", m)
    _run(fp8bs, full[name], cfg, m)


def test_streamk_lds_limit_rejected(fp8bs, full):
    """MLP down in one K chunk would stage 136 activation blocks per
    workgroup, more LDS than a compute unit has: a configuration error
    before any launch, not a failed launch."""
    from fp8_block_scaled_fp8bs_amd import Fp8bsError, GemmConfig
    pr = full["mlp_down"]
    with pytest.raises(Fp8bsError) as e:
        fp8bs.gemm_ex(GemmConfig(fp8bs.PATH_MFMA_STREAMK, 2, 1, 8, 7, 1), pr.wq, pr.ws,
                      x=pr.x[:8].contiguous())
    assert e.value.status == 7


def test_streamk_bit_identical_runs_and_reused_workspace(fp8bs, problems):
    """Ten runs give the same bits; so does a workspace that starts as
    arbitrary bytes (stale arrival counters) and is shared by calls of other
    shapes and chunk counts in between."""
    from fp8_block_scaled_fp8bs_amd import GemmConfig
    SKP = fp8bs.PATH_MFMA_STREAMK
    work = torch.empty(1 << 23, dtype=torch.uint8, device="cuda")
    work.fill_(0xA5)
    a, b = problems["ragged"], problems["chunks"]
    ca, cb = GemmConfig(SKP, 2, 1, 8, 7, 1), GemmConfig(SKP, 3, 1, 6, 8, 4)
    xa, xb = a.x[:8].contiguous(), b.x[:16].contiguous()
    ya = fp8bs.gemm_ex(ca, a.wq, a.ws, x=xa)   # fresh workspace
    yb = fp8bs.gemm_ex(cb, b.wq, b.ws, x=xb)
    for rep in range(10):
        y1 = fp8bs.gemm_ex(ca, a.wq, a.ws, x=xa, workspace=work)
        y2 = fp8bs.gemm_ex(cb, b.wq, b.ws, x=xb, workspace=work)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), ya.view(torch.int16)), rep
        assert torch.equal(y2.view(torch.int16), yb.view(torch.int16)), rep


def test_streamk_graph_replays_match_eager(fp8bs, problems):
    """A captured stream-K GEMM, replayed several times with eager calls on
    the same workspace between the replays, gives the eager bits each time."""
    from fp8_block_scaled_fp8bs_amd import GemmConfig
    SKP = fp8bs.PATH_MFMA_STREAMK
    pr, other = problems["ragged"], problems["wide"]
    cfg, cfo = GemmConfig(SKP, 2, 1, 8, 7, 1), GemmConfig(SKP, 2, 1, 8, 7, 1)
    x = pr.x[:8].contiguous()
    work = torch.empty(1 << 23, dtype=torch.uint8, device="cuda")
    y_eager = fp8bs.gemm_ex(cfg, pr.wq, pr.ws, x=x, workspace=work)
    torch.cuda.synchronize()
    out = torch.empty_like(y_eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fp8bs.gemm_ex(cfg, pr.wq, pr.ws, x=x, out=out, workspace=work, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp8bs.gemm_ex(cfg, pr.wq, pr.ws, x=x, out=out, workspace=work)
    for rep in range(4):
        out.fill_(0)
        fp8bs.gemm_ex(cfo, other.wq, other.ws, x=other.x[:3].contiguous(), workspace=work)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), y_eager.view(torch.int16)), f"replay {rep}"
