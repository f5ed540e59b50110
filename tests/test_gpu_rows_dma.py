"""GPU parity of the row-range kernel with the weight stream through LDS
(path MFMA_ROWS_DMA, tile-layout weights, m <= 16) against the CPU oracle:

- full outputs within 2^-7 |ref| + 1e-3 rms(ref) of the fp64 reference on
  the same codes;
- K ranges of one partial step (3 blocks: five compute waves idle), of a
  full and a partial step (13 blocks), of whole steps (40 blocks), and the
  full MLP-up weight (34816 x 5120: 136-row ranges, every one starting or
  ending inside a 16-row tile; the small problems: 8- or 4-row ranges, half
  or a quarter of a tile);
- rings of 3 and 6 stages; m from 1 to 16, where the LDS holds the
  activations beside the ring (others rejected before any launch);
- the same bits as the row-range kernel with 8 waves along K, whose
  products, rescale and summation orders it shares; the pre-quantized route
  equal to the fused cast; run-to-run identity and graph replays."""
import dataclasses

import numpy as np
import pytest

import oracle
from gpu_util import announce, dev_bf16, host_bits, need_gpu, same_bits_f32, torch
from workloads import WORKLOADS, act_bf16, bf16_from_f32

pytestmark = pytest.mark.gpu

TOL = dict(rel=2.0 ** -7, abs_rms=1e-3)
STAGES = [3, 6]


@pytest.fixture(scope="module")
def fp8bs():
    need_gpu()
    import fp8_block_scaled_fp8bs_amd as m
    m.load()
    return m


def dma_cfg(fp8bs, stages):
    from fp8_block_scaled_fp8bs_amd import GemmConfig
    return GemmConfig(fp8bs.PATH_MFMA_ROWS_DMA, 1, 1, 8, stages, 1, weight_layout=fp8bs.LAYOUT_TILES)


def rows_cfg(fp8bs):
    from fp8_block_scaled_fp8bs_amd import GemmConfig
    return GemmConfig(fp8bs.PATH_MFMA_ROWS, 1, 1, 8, 3, 1, weight_layout=fp8bs.LAYOUT_TILES)


def range_rows(n):
    """Rows per workgroup of the row-range kernels on tile-layout weights:
    n over 256 units rounded up to 16 rows, unless that leaves more than 2%
    of the units idle; then to 4 rows."""
    r = -(-n // 256)
    r16 = -(-r // 16) * 16
    return r16 if 50 * -(-n // r16) >= 49 * 256 else -(-r // 4) * 4


def lds_fits(n, k, m, stages):
    """Whether the workgroup's LDS (160 KB) holds the range's weight scales,
    the staged activations (148 bytes per row and block, rounded to 16), two
    partial-exchange areas and the ring of 16 KB stages."""
    rows = range_rows(n)
    nblk = k // 128
    ws = ((rows // 128 + 2) * nblk * 4 + 15) // 16 * 16
    act = (nblk * m * 148 + 15) // 16 * 16
    return ws + act + 2 * 7 * 1024 + stages * 16384 <= 160 * 1024


class Problem:
    def __init__(self, fp8bs, w_bits, x_bits):
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


# (n, k): 3, 13 and 40 K blocks per tile
PROBLEMS = {"k3": (8192, 384), "k13": (1024, 1664), "k40": (2048, 5120)}


@pytest.fixture(scope="module")
def problems(fp8bs):
    out = {}
    for i, (name, (n, k)) in enumerate(PROBLEMS.items()):
        announce("rows-dma problem", name, n, k)
        out[name] = _random_problem(fp8bs, 16, n, k, 5400 + i)
    wl = WORKLOADS["mlp_up"]
    announce("rows-dma problem", "mlp_up", wl.n, wl.k)
    x_bits = act_bf16(wl.x_seed, wl.col_seed, 16, wl.k, wl.n_outlier, wl.outlier_factor)
    out["mlp_up"] = Problem(fp8bs, wl.weight(), x_bits)
    torch.cuda.synchronize()
    return out


def _run(fp8bs, pr, stages, m):
    from fp8_block_scaled_fp8bs_amd import Fp8bsError
    x = pr.x[:m].contiguous()
    n, k = pr.wq.shape[0], x.shape[1]
    cfg = dma_cfg(fp8bs, stages)
    if not lds_fits(n, k, m, stages):
        with pytest.raises(Fp8bsError) as e:
            fp8bs.gemm_ex(cfg, pr.wt, pr.ws, x=x)
        assert e.value.status == 7
        return
    y = fp8bs.gemm_ex(cfg, pr.wt, pr.ws, x=x)
    xq, xs = fp8bs.quantize_act(x)
    yq = fp8bs.gemm_ex(cfg, pr.wt, pr.ws, x_q=xq, x_s=xs)
    yr = fp8bs.gemm_ex(rows_cfg(fp8bs), pr.wt, pr.ws, x=x)
    torch.cuda.synchronize()
    yb = host_bits(y)
    rep = oracle.tolerance_report(yb, pr.ref(m), **TOL)
    assert rep["finite"] and rep["n_bad"] == 0, f"{cfg} m={m}: {rep}"
    assert np.array_equal(yb, host_bits(yq)), f"pre-quantized route differs {cfg} m={m}"
    assert np.array_equal(yb, host_bits(yr)), f"differs from the row-range kernel {cfg} m={m}"


@pytest.mark.parametrize("stages", STAGES)
@pytest.mark.parametrize("name", ["k3", "k13", "k40", "mlp_up"])
@pytest.mark.parametrize("m", [1, 3, 8, 13, 16])
def test_rows_dma_every_config(fp8bs, problems, stages, name, m):
    announce("rows-dma", name, "stages", stages, "m", m)
    _run(fp8bs, problems[name], stages, m)


def test_rows_dma_identity_and_graph_replays(fp8bs, problems):
    """Ten eager runs give the same bits; a captured call replayed with other
    calls in between gives them on every replay."""
    pr, other = problems["mlp_up"], problems["k13"]
    cfg = dma_cfg(fp8bs, 6)
    x = pr.x[:8].contiguous()
    y0 = fp8bs.gemm_ex(cfg, pr.wt, pr.ws, x=x)
    torch.cuda.synchronize()
    for rep in range(10):
        y1 = fp8bs.gemm_ex(cfg, pr.wt, pr.ws, x=x)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y0.view(torch.int16)), rep
    out = torch.empty_like(y0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fp8bs.gemm_ex(cfg, pr.wt, pr.ws, x=x, out=out, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp8bs.gemm_ex(cfg, pr.wt, pr.ws, x=x, out=out)
    for rep in range(4):
        out.fill_(0)
        fp8bs.gemm_ex(cfg, other.wt, other.ws, x=other.x[:5].contiguous())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), y0.view(torch.int16)), f"replay {rep}"


def test_rows_dma_limits_rejected(fp8bs, problems):
    """m > 16, row-major weights, a K split and a tiles_n other than 1 are
    configuration errors before any launch."""
    from fp8_block_scaled_fp8bs_amd import Fp8bsError
    pr = problems["k40"]
    cfg = dma_cfg(fp8bs, 3)
    x = pr.x[:8].contiguous()
    bad = [
        (cfg, pr.wt, torch.zeros((17, 5120), dtype=torch.bfloat16, device="cuda")),
        (dataclasses.replace(cfg, weight_layout=fp8bs.LAYOUT_ROWS), pr.wq, x),
        (dataclasses.replace(cfg, split_k=2), pr.wt, x),
        (dataclasses.replace(cfg, tiles_n=2), pr.wt, x),
    ]
    before = fp8bs.launch_count("gemm_mfma")
    for c, w, xx in bad:
        with pytest.raises(Fp8bsError) as e:
            fp8bs.gemm_ex(c, w, pr.ws, x=xx)
        assert e.value.status == 7, c
    torch.cuda.synchronize()
    assert fp8bs.launch_count("gemm_mfma") == before
