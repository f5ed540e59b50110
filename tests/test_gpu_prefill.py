"""GPU parity of the prefill-size path (m > 32: the tiled matrix-core kernel,
activations cast first) against the CPU oracle: bf16 outputs within
2^-7 |ref| + 1e-3 rms(ref) of the fp64 reference built from the same codes
and scales; fused cast equal bit for bit to quantize-then-multiply; run-to-
run bit identity; ragged m tails, one K block, one 128-row block of n; the
full 8192 x 5120 x 5120 shape on sampled rows."""
import numpy as np
import pytest

import oracle
from gpu_util import announce, dev_bf16, dev_f32, dev_u8, host_bits, need_gpu, same_bits_f32, torch
from workloads import WORKLOADS, act_bf16, bf16_from_f32

pytestmark = pytest.mark.gpu

TOL = dict(rel=2.0 ** -7, abs_rms=1e-3)


@pytest.fixture(scope="module")
def fp8bs():
    need_gpu()
    import fp8_block_scaled_fp8bs_amd as m
    m.load()
    return m


def _problem(fp8bs, m, n, k, seed):
    rng = np.random.default_rng(seed)
    w_bits = bf16_from_f32((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[:, rng.choice(k, max(1, k // 100), replace=False)] *= 10
    x_bits = bf16_from_f32(x)
    wq, ws = fp8bs.quantize_weight(dev_bf16(w_bits))
    wq_ref, ws_ref = oracle.quantize_weight_ref(w_bits)
    assert np.array_equal(wq.cpu().numpy(), wq_ref)
    return x_bits, wq, ws, wq_ref, ws_ref


@pytest.mark.parametrize("m,n,k", [(33, 256, 256), (64, 384, 1024), (127, 128, 128),
                                   (200, 512, 1280), (1000, 1024, 2048), (4096, 256, 640)])
def test_prefill_parity_full_output(fp8bs, m, n, k):
    cfg = fp8bs.select_config(m, n, k)
    announce("prefill parity", m, n, k, cfg)
    assert cfg.path == fp8bs.PATH_PREFILL
    x_bits, wq, ws, wq_ref, ws_ref = _problem(fp8bs, m, n, k, 7000 + m + n + k)
    x = dev_bf16(x_bits)
    y = fp8bs.gemm(x, wq, ws)
    xq, xs = fp8bs.quantize_act(x)
    y_q = fp8bs.gemm_q(xq, xs, wq, ws)
    torch.cuda.synchronize()
    xq_ref, xs_ref = oracle.quantize_act_ref(x_bits)
    assert np.array_equal(xq.cpu().numpy(), xq_ref) and same_bits_f32(xs.cpu().numpy(), xs_ref)
    ref = oracle.gemm_ref(xq_ref, xs_ref, wq_ref, ws_ref)
    rep = oracle.tolerance_report(host_bits(y), ref, **TOL)
    assert rep["finite"] and rep["n_bad"] == 0, rep
    assert np.array_equal(host_bits(y), host_bits(y_q)), "fused cast differs from quantize-then-multiply"


@pytest.mark.parametrize("variant", [(2, 1, 1), (4, 1, 1), (2, 2, 1), (2, 4, 1), (4, 2, 1), (4, 3, 1),
                                     (2, 2, 2), (4, 2, 2), (4, 3, 2)])
@pytest.mark.parametrize("m,n,k,split", [(300, 512, 1280, 1), (129, 768, 2048, 3), (64, 256, 384, 1),
                                         (33, 1024, 128, 1), (520, 256, 2560, 2)])
def test_prefill_every_variant(fp8bs, variant, m, n, k, split):
    """Each compiled prefill kernel (4 or 8 waves; register pipeline, or a
    ring of 2-4 LDS stages filled by direct loads, refilled when the next
    block starts or as soon as a block's operands are in registers), split
    and unsplit, one K block (fewer blocks than stages), ragged m tails: full
    output against the oracle."""
    from fp8_block_scaled_fp8bs_amd import Fp8bsError, GemmConfig
    wn, depth, tn = variant
    cfg = GemmConfig(fp8bs.PATH_PREFILL, tn, wn, 2, depth, split)
    announce("prefill variant", cfg, m, n, k)
    x_bits, wq, ws, wq_ref, ws_ref = _problem(fp8bs, m, n, k, 7400 + m + n + k)
    if n % (64 * wn):
        with pytest.raises(Fp8bsError):
            fp8bs.gemm_ex(cfg, wq, ws, x=dev_bf16(x_bits))
        return
    y = fp8bs.gemm_ex(cfg, wq, ws, x=dev_bf16(x_bits))
    torch.cuda.synchronize()
    xq_ref, xs_ref = oracle.quantize_act_ref(x_bits)
    rep = oracle.tolerance_report(host_bits(y), oracle.gemm_ref(xq_ref, xs_ref, wq_ref, ws_ref), **TOL)
    assert rep["finite"] and rep["n_bad"] == 0, rep
    # run to run: the same bits again
    y2 = fp8bs.gemm_ex(cfg, wq, ws, x=dev_bf16(x_bits))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y), host_bits(y2))


WIDE = [(4, 2), (3, 2)]  # (activation subtiles per wave, LDS stages) of the wide-wave-tile kernels


@pytest.mark.parametrize("layout", ["rows", "tiles"])
@pytest.mark.parametrize("wk,depth", WIDE)
@pytest.mark.parametrize("m,n,k,split", [(300, 512, 1280, 1), (129, 768, 2048, 3), (64, 384, 384, 1),
                                         (33, 1024, 128, 1), (520, 256, 2560, 2),
                                         (1000, 2176, 640, 1), (257, 128, 256, 1),
                                         (130, 256, 12288, 12)])
def test_prefill_wide_wave_tiles(fp8bs, layout, wk, depth, m, n, k, split):
    """The kernels with 64 x 128 or 48 x 128 outputs per wave (256 x 256 or
    192 x 256 output tiles, 8 waves, grid schedule): ragged m tails, an odd
    number of 128-column
    blocks (the last tile one block wide), split and unsplit, one K block
    (fewer blocks than stages), both weight layouts. Full output against the
    oracle, and the same bits as the 128 x 128 direct-load kernel in the same
    split (the same products, rescaled in the same order)."""
    import dataclasses
    from fp8_block_scaled_fp8bs_amd import GemmConfig
    cfg = GemmConfig(fp8bs.PATH_PREFILL, 3, 2, wk, depth, split)
    base = GemmConfig(fp8bs.PATH_PREFILL, 1, 2, 2, 2, split)
    announce("prefill wide wave tiles", cfg, layout, m, n, k)
    x_bits, wq, ws, wq_ref, ws_ref = _problem(fp8bs, m, n, k, 7600 + m + n + k)
    x = dev_bf16(x_bits)
    w = wq
    if layout == "tiles":
        cfg = dataclasses.replace(cfg, weight_layout=fp8bs.LAYOUT_TILES)
        w = fp8bs.pack_weight(wq)
    y = fp8bs.gemm_ex(cfg, w, ws, x=x)
    y_base = fp8bs.gemm_ex(base, wq, ws, x=x)
    xq, xs = fp8bs.quantize_act(x)
    y_q = fp8bs.gemm_ex(cfg, w, ws, x_q=xq, x_s=xs)
    torch.cuda.synchronize()
    xq_ref, xs_ref = oracle.quantize_act_ref(x_bits)
    rep = oracle.tolerance_report(host_bits(y), oracle.gemm_ref(xq_ref, xs_ref, wq_ref, ws_ref), **TOL)
    assert rep["finite"] and rep["n_bad"] == 0, rep
    assert np.array_equal(host_bits(y), host_bits(y_base)), "differs from the 128 x 128 kernel"
    assert np.array_equal(host_bits(y), host_bits(y_q)), "fused cast differs"


@pytest.mark.parametrize("jm", [4, 3])
@pytest.mark.parametrize("layout", ["rows", "tiles"])
@pytest.mark.parametrize("m,n,k", [(2100, 8320, 384), (4096, 4352, 256), (2100, 12800, 256),
                                   (300, 640, 1280), (33, 128, 256)])
def test_prefill_wide_1d_schedule(fp8bs, jm, layout, m, n, k):
    """The 1-D schedule of the wide kernel: whole tiles (256 or 192 rows by
    256 columns) in complete rounds of 256 workgroups, the tiles left over as
    two 128-column halves when those fit in half a round. With 256-row tiles:
    2100 x 8320: 33 x 9 = 297 tiles, 41 left over as 82 halves (the last tile
    column one 128-column block wide, so one half of its tiles is empty; a
    ragged m tail); 4096 x 4352: 272 tiles, 16 left over; 2100 x 12800: 450
    tiles, 194 left over (too many: a last round of whole tiles); 300 x 640:
    6 tiles, all halves; 33 x 128: one half (192-row tiles: 363, 374, 550, 6
    and 1 tiles). Full output against the oracle and the bits of the unsplit
    128 x 128 kernel (every tile, whole or half, runs the whole K range with
    the same products rescaled in the same order); the bits repeat over
    graph replays."""
    import dataclasses
    from fp8_block_scaled_fp8bs_amd import GemmConfig
    cfg = GemmConfig(fp8bs.PATH_PREFILL, 4, 2, jm, 2, 1)
    announce("prefill wide 1-D", cfg, layout, m, n, k)
    x_bits, wq, ws, wq_ref, ws_ref = _problem(fp8bs, m, n, k, 7700 + m + n + k)
    x = dev_bf16(x_bits)
    w = wq
    if layout == "tiles":
        cfg = dataclasses.replace(cfg, weight_layout=fp8bs.LAYOUT_TILES)
        w = fp8bs.pack_weight(wq)
    y = fp8bs.gemm_ex(cfg, w, ws, x=x)
    y1 = fp8bs.gemm_ex(GemmConfig(fp8bs.PATH_PREFILL, 1, 2, 2, 2, 1), wq, ws, x=x)
    xq, xs = fp8bs.quantize_act(x)
    yq = fp8bs.gemm_ex(cfg, w, ws, x_q=xq, x_s=xs)
    torch.cuda.synchronize()
    yb = host_bits(y)
    xq_ref, xs_ref = oracle.quantize_act_ref(x_bits)
    rep = oracle.tolerance_report(yb, oracle.gemm_ref(xq_ref, xs_ref, wq_ref, ws_ref), **TOL)
    assert rep["finite"] and rep["n_bad"] == 0, rep
    assert np.array_equal(yb, host_bits(y1)), "differs from the 128 x 128 kernel"
    assert np.array_equal(yb, host_bits(yq)), "fused cast differs"
    out = torch.empty_like(y)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fp8bs.gemm_ex(cfg, w, ws, x_q=xq, x_s=xs, out=out, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp8bs.gemm_ex(cfg, w, ws, x_q=xq, x_s=xs, out=out)
    for rep_i in range(3):
        out.fill_(0)
        fp8bs.gemm_ex(cfg, w, ws, x_q=xq, x_s=xs)  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(out), yb), f"replay {rep_i}"


@pytest.mark.parametrize("jm", [4, 3])
@pytest.mark.parametrize("layout", ["rows", "tiles"])
@pytest.mark.parametrize("m,n,k", [(300, 640, 1280), (2100, 1280, 384), (33, 640, 256),
                                   (700, 5120, 256), (520, 1920, 640)])
def test_prefill_wide_narrow_tiles(fp8bs, jm, layout, m, n, k):
    """The wide kernel on 160-column tiles (5 weight subtiles per wave; n a
    multiple of 160 and of 128), every tile a unit of the 1-D grid. A wave's
    80 columns start at any multiple of 16 and straddle a 128-column scale
    block in some tiles (columns 80-159, 240-319, ...), so each subtile takes
    its own weight scale. Shapes with 256-row tiles: 8, 72 and 96 tiles (the
    per-XCD order), 4 and 36 tiles (the plain order), ragged m tails. Full
    output against the oracle, the bits of the unsplit 128 x 128 kernel, the
    fused cast against quantize-then-multiply, and graph replays."""
    import dataclasses
    from fp8_block_scaled_fp8bs_amd import GemmConfig
    cfg = GemmConfig(fp8bs.PATH_PREFILL, 5, 2, jm, 2, 1)
    announce("prefill narrow tiles", cfg, layout, m, n, k)
    x_bits, wq, ws, wq_ref, ws_ref = _problem(fp8bs, m, n, k, 7900 + m + n + k)
    x = dev_bf16(x_bits)
    w = wq
    if layout == "tiles":
        cfg = dataclasses.replace(cfg, weight_layout=fp8bs.LAYOUT_TILES)
        w = fp8bs.pack_weight(wq)
    y = fp8bs.gemm_ex(cfg, w, ws, x=x)
    y1 = fp8bs.gemm_ex(GemmConfig(fp8bs.PATH_PREFILL, 1, 2, 2, 2, 1), wq, ws, x=x)
    xq, xs = fp8bs.quantize_act(x)
    yq = fp8bs.gemm_ex(cfg, w, ws, x_q=xq, x_s=xs)
    torch.cuda.synchronize()
    yb = host_bits(y)
    xq_ref, xs_ref = oracle.quantize_act_ref(x_bits)
    rep = oracle.tolerance_report(yb, oracle.gemm_ref(xq_ref, xs_ref, wq_ref, ws_ref), **TOL)
    assert rep["finite"] and rep["n_bad"] == 0, rep
    assert np.array_equal(yb, host_bits(y1)), "differs from the 128 x 128 kernel"
    assert np.array_equal(yb, host_bits(yq)), "fused cast differs"
    out = torch.empty_like(y)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fp8bs.gemm_ex(cfg, w, ws, x_q=xq, x_s=xs, out=out, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp8bs.gemm_ex(cfg, w, ws, x_q=xq, x_s=xs, out=out)
    for rep_i in range(3):
        out.fill_(0)
        fp8bs.gemm_ex(cfg, w, ws, x_q=xq, x_s=xs)  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(out), yb), f"replay {rep_i}"


def test_prefill_narrow_tiles_rejected_off_shape(fp8bs):
    """Narrow tiles need n to be a multiple of 160 and run unsplit: other
    configurations are errors before any launch."""
    from fp8_block_scaled_fp8bs_amd import Fp8bsError, GemmConfig
    before = fp8bs.launch_count("gemm_mfma")
    x_bits, wq, ws, _, _ = _problem(fp8bs, 64, 256, 512, 7801)
    for cfg in (GemmConfig(fp8bs.PATH_PREFILL, 5, 2, 4, 2, 1), GemmConfig(fp8bs.PATH_PREFILL, 5, 2, 3, 2, 2)):
        with pytest.raises(Fp8bsError) as e:
            fp8bs.gemm_ex(cfg, wq, ws, x=dev_bf16(x_bits))
        assert e.value.status == 7
    x_bits, wq, ws, _, _ = _problem(fp8bs, 64, 640, 512, 7802)
    with pytest.raises(Fp8bsError) as e:
        fp8bs.gemm_ex(GemmConfig(fp8bs.PATH_PREFILL, 5, 2, 4, 2, 2), wq, ws, x=dev_bf16(x_bits))
    assert e.value.status == 7
    torch.cuda.synchronize()
    assert fp8bs.launch_count("gemm_mfma") == before


def test_prefill_wide_1d_rejects_split(fp8bs):
    """The 1-D schedule runs every tile over the whole K range: a K split in
    its configuration is a configuration error."""
    from fp8_block_scaled_fp8bs_amd import Fp8bsError, GemmConfig
    x_bits, wq, ws, _, _ = _problem(fp8bs, 64, 256, 512, 7800)
    with pytest.raises(Fp8bsError) as e:
        fp8bs.gemm_ex(GemmConfig(fp8bs.PATH_PREFILL, 4, 2, 4, 2, 2), wq, ws, x=dev_bf16(x_bits))
    assert e.value.status == 7


@pytest.mark.parametrize("m,n,k", [(300, 8192, 256), (1000, 16384, 128), (129, 8320, 256)])
def test_prefill_wide_grid_tile_order(fp8bs, m, n, k):
    """Wide unsplit grids (64 or more 128-column tiles) take the tile order
    remapped per XCD when the tile count is a multiple of 8 (the first two
    shapes) and the plain order otherwise (65 x 2 tiles): full output
    against the oracle, fused cast equal to quantize-then-multiply."""
    cfg = fp8bs.select_config(m, n, k)
    announce("prefill wide grid", m, n, k, cfg)
    assert cfg.path == fp8bs.PATH_PREFILL and cfg.split_k == 1
    x_bits, wq, ws, wq_ref, ws_ref = _problem(fp8bs, m, n, k, 7500 + m + n + k)
    x = dev_bf16(x_bits)
    y = fp8bs.gemm(x, wq, ws)
    xq, xs = fp8bs.quantize_act(x)
    y_q = fp8bs.gemm_q(xq, xs, wq, ws)
    torch.cuda.synchronize()
    xq_ref, xs_ref = oracle.quantize_act_ref(x_bits)
    rep = oracle.tolerance_report(host_bits(y), oracle.gemm_ref(xq_ref, xs_ref, wq_ref, ws_ref), **TOL)
    assert rep["finite"] and rep["n_bad"] == 0, rep
    assert np.array_equal(host_bits(y), host_bits(y_q))


def test_prefill_run_to_run_identity(fp8bs):
    m, n, k = 777, 640, 1152
    x_bits, wq, ws, _, _ = _problem(fp8bs, m, n, k, 7100)
    x = dev_bf16(x_bits)
    first = host_bits(fp8bs.gemm(x, wq, ws))
    for _ in range(5):
        assert np.array_equal(first, host_bits(fp8bs.gemm(x, wq, ws)))


def test_prefill_explicit_config_rules(fp8bs):
    """The prefill kernel takes any m; the decode kernels refuse m > 32."""
    from fp8_block_scaled_fp8bs_amd import Fp8bsError, GemmConfig
    m, n, k = 48, 256, 512
    x_bits, wq, ws, wq_ref, ws_ref = _problem(fp8bs, m, n, k, 7200)
    x = dev_bf16(x_bits)
    with pytest.raises(Fp8bsError):
        fp8bs.gemm_ex(GemmConfig(1, 1, 1, 4, 5), wq, ws, x=x)
    # the prefill kernel at decode sizes too (m = 1, 8, 32)
    xq_ref, xs_ref = oracle.quantize_act_ref(x_bits)
    for mm in (1, 8, 32):
        y = fp8bs.gemm_ex(GemmConfig(5, 1, 2, 2, 1), wq, ws, x=x[:mm].contiguous())
        torch.cuda.synchronize()
        ref = oracle.gemm_ref(xq_ref[:mm], xs_ref[:mm], wq_ref, ws_ref)
        rep = oracle.tolerance_report(host_bits(y), ref, **TOL)
        assert rep["finite"] and rep["n_bad"] == 0, (mm, rep)


def test_prefill_full_size_sampled_rows(fp8bs):
    """8192 activation rows on the 5120 x 5120 square weight (the seeded
    square-workload weight; activations drawn with the square recipe): full
    output rows checked for sampled m, including the first and last."""
    wl = WORKLOADS["square"]
    m = 8192
    announce("prefill full size", m, wl.n, wl.k)
    w_bits = wl.weight()
    x_bits = act_bf16(wl.x_seed, wl.col_seed, m, wl.k, wl.n_outlier, wl.outlier_factor)
    wq, ws = fp8bs.quantize_weight(dev_bf16(w_bits))
    y = fp8bs.gemm(dev_bf16(x_bits), wq, ws)
    torch.cuda.synchronize()
    yb = host_bits(y)
    wq_ref, ws_ref = oracle.quantize_weight_ref(w_bits)
    assert np.array_equal(wq.cpu().numpy(), wq_ref)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, m - 1],
                                     np.random.default_rng(5).choice(m, 27, replace=False)]))
    xq_ref, xs_ref = oracle.quantize_act_ref(x_bits[rows])
    ref = oracle.gemm_ref(xq_ref, xs_ref, wq_ref, ws_ref)
    rep = oracle.tolerance_report(yb[rows], ref, **TOL)
    assert rep["finite"] and rep["n_bad"] == 0, rep


@pytest.mark.parametrize("m", [1024, 128])
def test_prefill_deep_k_split_sampled_rows(fp8bs, m):
    """The MLP-down weight (17408 -> 5120, the seeded workload weight) at
    m = 1024 and 128, where the table splits K of the wide kernel over 3 and
    12 workgroups: sampled full output rows, including the first and last,
    against the oracle; the same bits as the unsplit 1-D schedule would not
    hold (the split partials are summed in split order), so the check is
    the tolerance and run-to-run identity."""
    wl = WORKLOADS["mlp_down"]
    cfg = fp8bs.tiles_select_config(m, wl.n, wl.k)
    announce("prefill deep K", m, wl.n, wl.k, cfg)
    assert (cfg.path, cfg.tiles_n, cfg.split_k) == (fp8bs.PATH_PREFILL, 3, 3 if m == 1024 else 12)
    w_bits = wl.weight()
    x_bits = act_bf16(wl.x_seed, wl.col_seed, m, wl.k, wl.n_outlier, wl.outlier_factor)
    wq, ws = fp8bs.quantize_weight(dev_bf16(w_bits))
    wt = fp8bs.pack_weight(wq)
    x = dev_bf16(x_bits)
    y = fp8bs.gemm_tiles(x, wt, ws)
    y2 = fp8bs.gemm_tiles(x, wt, ws)
    yr = fp8bs.gemm(x, wq, ws)
    torch.cuda.synchronize()
    yb = host_bits(y)
    assert np.array_equal(yb, host_bits(y2)), "run-to-run bits differ"
    assert np.array_equal(yb, host_bits(yr)), "row-major call differs"
    wq_ref, ws_ref = oracle.quantize_weight_ref(w_bits)
    assert np.array_equal(wq.cpu().numpy(), wq_ref)
    rows = np.unique(np.concatenate([[0, 1, min(255, m - 2), min(256, m - 1), m - 1],
                                     np.random.default_rng(6).choice(m, 11, replace=False)]))
    xq_ref, xs_ref = oracle.quantize_act_ref(x_bits[rows])
    rep = oracle.tolerance_report(yb[rows], oracle.gemm_ref(xq_ref, xs_ref, wq_ref, ws_ref), **TOL)
    assert rep["finite"] and rep["n_bad"] == 0, rep


def test_prefill_swiglu(fp8bs):
    """The SwiGLU call at a prefill size: y equals the plain GEMM and h equals
    the standalone epilogue on it, bit for bit."""
    m, n, k = 300, 768, 640
    x_bits, wq, ws, wq_ref, ws_ref = _problem(fp8bs, m, n, k, 7300)
    x = dev_bf16(x_bits)
    y, hq, hs = fp8bs.gemm_swiglu(x, wq, ws)
    y2 = fp8bs.gemm(x, wq, ws)
    hq2, hs2 = fp8bs.swiglu_quant(y)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y), host_bits(y2))
    assert torch.equal(hq, hq2) and torch.equal(hs, hs2)
    xq_ref, xs_ref = oracle.quantize_act_ref(x_bits)
    rep = oracle.tolerance_report(host_bits(y), oracle.gemm_ref(xq_ref, xs_ref, wq_ref, ws_ref), **TOL)
    assert rep["finite"] and rep["n_bad"] == 0, rep
