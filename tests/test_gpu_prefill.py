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
