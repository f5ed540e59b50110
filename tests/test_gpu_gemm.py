"""GPU parity of the GEMM against the CPU oracle: bf16 outputs within
2^-7 |ref| + 1e-3 rms(ref) of the fp64 reference built from the same
(bit-identical) codes and scales; run-to-run bit identity; the fused cast
equal bit for bit to quantize-then-multiply; every compiled kernel
configuration; empty and ragged cases."""
import numpy as np
import pytest

import oracle
from gpu_util import announce, dev_bf16, dev_f32, dev_u8, host_bits, need_gpu, same_bits_f32, torch
from workloads import WORKLOADS, act_bf16, bf16_from_f32, weight_rows_bf16

pytestmark = pytest.mark.gpu

TOL = dict(rel=2.0 ** -7, abs_rms=1e-3)

# (tiles or row groups per wave, waves along N, waves along K, blocks in flight):
# every shape compiled into the library.
MFMA_SHAPES = [(1, 1, 8, 5), (1, 1, 8, 2), (1, 1, 8, 4), (1, 1, 4, 5), (1, 1, 4, 8), (1, 2, 4, 5),
               (1, 2, 4, 2), (2, 1, 8, 2), (2, 1, 4, 4), (4, 1, 8, 1), (4, 1, 4, 2), (2, 1, 8, 4),
               (1, 4, 1, 5), (1, 4, 2, 5), (1, 4, 4, 2), (1, 5, 1, 5), (1, 5, 2, 5), (1, 5, 2, 2),
               (1, 8, 1, 5), (1, 8, 2, 2), (2, 4, 1, 5), (2, 2, 2, 4), (2, 2, 4, 2), (1, 2, 8, 2),
               (1, 5, 1, 10), (2, 5, 1, 5), (1, 4, 1, 10)]
DOT_SHAPES = [(2, 1, 8, 5), (2, 4, 1, 5), (4, 2, 2, 4), (1, 1, 8, 5), (2, 1, 8, 2), (4, 1, 8, 2),
              (2, 2, 4, 4)]
# (waves along K, tiles in flight, tiles issued before the cast) of the
# row-range kernel
ROWS_SHAPES = [(8, 4, 2), (8, 4, 4), (8, 2, 2), (8, 3, 1), (8, 6, 2), (16, 2, 1), (16, 3, 1),
               (4, 8, 2)]
# (waves along K, tiles in flight) of the streaming row-range kernel
STREAM_SHAPES = [(8, 4), (8, 2), (8, 6), (16, 2), (16, 3), (4, 8), (16, 5), (8, 8)]
# (split_k, reduce): no split, second-kernel reduce, last-arriver reduce
SPLITS = [(1, 0), (3, 0), (4, 1), (5, 1)]


@pytest.fixture(scope="module")
def fp8bs():
    need_gpu()
    import fp8_block_scaled_fp8bs_amd as m
    m.load()
    return m


def _assert_close(y_bits, ref, what, rms=None):
    rep = oracle.tolerance_report(y_bits, ref, rms=rms, **TOL)
    assert rep["finite"] and rep["n_bad"] == 0, f"{what}: {rep}"
    return rep


class Problem:
    """Seeded operands on host and device, with the oracle's reference."""

    def __init__(self, fp8bs, w_bits, x_bits):
        self.w_bits, self.x_bits = w_bits, x_bits
        self.w = dev_bf16(w_bits)
        self.x = dev_bf16(x_bits)
        self.wq, self.ws = fp8bs.quantize_weight(self.w)
        self.wq_ref, self.ws_ref = oracle.quantize_weight_ref(w_bits)
        assert np.array_equal(self.wq.cpu().numpy(), self.wq_ref)
        assert same_bits_f32(self.ws.cpu().numpy(), self.ws_ref)
        self.xq_ref, self.xs_ref = oracle.quantize_act_ref(x_bits)
        self._ref = None

    @property
    def ref(self):
        if self._ref is None:
            self._ref = oracle.gemm_ref(self.xq_ref, self.xs_ref, self.wq_ref, self.ws_ref)
        return self._ref


def _random_problem(fp8bs, m, n, k, seed):
    rng = np.random.default_rng(seed)
    w = bf16_from_f32((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[:, rng.choice(k, max(1, k // 100), replace=False)] *= 10
    return Problem(fp8bs, w, bf16_from_f32(x))


def test_tiny_workload_parity_full_output(fp8bs):
    wl = WORKLOADS["tiny"]
    announce("gemm parity tiny m 8 cfg", fp8bs.select_config(8, wl.n, wl.k))
    pr = Problem(fp8bs, wl.weight(), wl.act(8))
    y = fp8bs.gemm(pr.x, pr.wq, pr.ws)
    torch.cuda.synchronize()
    _assert_close(host_bits(y), pr.ref, "tiny m=8")


@pytest.fixture(scope="module")
def full_problems(fp8bs):
    """Seeded full-size weights of the square and MLP shapes (quantized on
    the GPU, bit-checked against the oracle once) and their activations at
    the largest M of the step mix."""
    out = {}
    for name in ("square", "mlp_up", "mlp_down"):
        wl = WORKLOADS[name]
        announce("full-size weight", name, wl.n, wl.k)
        w_bits = wl.weight()
        x_bits = act_bf16(wl.x_seed, wl.col_seed, 32, wl.k, wl.n_outlier, wl.outlier_factor)
        out[name] = Problem(fp8bs, w_bits, x_bits)
        torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", ["square", "mlp_up", "mlp_down"])
@pytest.mark.parametrize("m", [1, 2, 4, 8, 16, 32])
def test_step_mix_shapes_every_m(fp8bs, full_problems, name, m):
    """Every full-size GEMM shape of the decode-step mix (the square, MLP-up
    and MLP-down workloads with their seeded weights and activations) at
    every M it runs at, in the configuration the library picks for it (the
    one the benches time): full output within tolerance of the oracle."""
    pr = full_problems[name]
    cfg = fp8bs.select_config(m, pr.w_bits.shape[0], pr.w_bits.shape[1])
    announce("step-mix shape", name, "m", m, "cfg", cfg)
    x = pr.x[:m].contiguous()
    y = fp8bs.gemm(x, pr.wq, pr.ws)
    torch.cuda.synchronize()
    ref = oracle.gemm_ref(pr.xq_ref[:m], pr.xs_ref[:m], pr.wq_ref, pr.ws_ref)
    _assert_close(host_bits(y), ref, f"{name} m={m} {cfg}")


@pytest.fixture(scope="module")
def vocab_weight(fp8bs):
    wl = WORKLOADS["vocab"]
    announce("vocab weight generation", wl.n, wl.k)
    w = dev_bf16(wl.weight())
    wq, ws = fp8bs.quantize_weight(w)
    del w
    torch.cuda.synchronize()
    return wq, ws


@pytest.mark.parametrize("m", [1, 2, 4, 8, 16, 32])
def test_vocab_parity_sampled_columns(fp8bs, vocab_weight, m):
    """The 248,320-wide output layer at its full size, in the launch
    configuration the library picks; sampled block rows of W are regenerated
    alone and checked (codes bit-exact, outputs within tolerance, with the
    rms over the sampled outputs)."""
    wl = WORKLOADS["vocab"]
    announce("gemm vocab", "m", m, "cfg", fp8bs.select_config(m, wl.n, wl.k))
    wq, ws = vocab_weight
    x_bits = act_bf16(wl.x_seed, wl.col_seed, 32, wl.k, wl.n_outlier, wl.outlier_factor)[:m]
    y = host_bits(fp8bs.gemm(dev_bf16(x_bits), wq, ws))
    xq, xs = oracle.quantize_act_ref(x_bits)
    nbn = wl.n // 128
    cols = (0, 3, 1000, nbn // 2, nbn - 2, nbn - 1)
    refs, gots = [], []
    for c in cols:
        rows = weight_rows_bf16(wl.w_seed, c, 128, wl.k)
        qr, sr = oracle.quantize_weight_ref(rows)
        assert np.array_equal(wq[c * 128:(c + 1) * 128].cpu().numpy(), qr)
        refs.append(oracle.gemm_ref(xq, xs, qr, sr))
        gots.append(y[:, c * 128:(c + 1) * 128])
    _assert_close(np.concatenate(gots, axis=1), np.concatenate(refs, axis=1), f"vocab m={m}")


# One GPU's share of a shape under an 8-way split (the per-GPU kernel of the
# sharded path, run here on one GPU): the vocabulary layer split on 128-row
# block boundaries (ranks 0-3 hold 243 of the 1,940 block rows, ranks 4-7
# hold 242), MLP down split along K (17 of the 136 K blocks per rank).
VOCAB_SHARD_BLOCKS = [243] * 4 + [242] * 4
DOWN_SHARD_KB = 17


@pytest.mark.parametrize("rank", [0, 7])
@pytest.mark.parametrize("m", [1, 8, 16, 24, 32])
def test_vocab_column_shard(fp8bs, vocab_weight, rank, m):
    """A rank's column share of the vocabulary weight is a contiguous slice of
    its block rows with their own scales; the GEMM on it (row-major and tile
    layout, each in the table's configuration for the share's shape) gives
    the columns of the full product: sampled block rows, regenerated alone,
    against the oracle."""
    wl = WORKLOADS["vocab"]
    b0 = sum(VOCAB_SHARD_BLOCKS[:rank])
    b1 = b0 + VOCAB_SHARD_BLOCKS[rank]
    wq, ws = vocab_weight
    wsh, ssh = wq[b0 * 128:b1 * 128], ws[b0:b1]
    n = (b1 - b0) * 128
    announce("vocab shard", rank, "n", n, "m", m, "cfg", fp8bs.select_config(m, n, wl.k))
    x_bits = act_bf16(wl.x_seed, wl.col_seed, 32, wl.k, wl.n_outlier, wl.outlier_factor)[:m]
    x = dev_bf16(x_bits)
    y = host_bits(fp8bs.gemm(x, wsh, ssh))
    yt = host_bits(fp8bs.gemm_tiles(x, fp8bs.pack_weight(wsh), ssh))
    xq, xs = oracle.quantize_act_ref(x_bits)
    refs, gots, gots_t = [], [], []
    for c in (b0, b0 + 1, (b0 + b1) // 2, b1 - 1):
        rows = weight_rows_bf16(wl.w_seed, c, 128, wl.k)
        qr, sr = oracle.quantize_weight_ref(rows)
        refs.append(oracle.gemm_ref(xq, xs, qr, sr))
        gots.append(y[:, (c - b0) * 128:(c - b0 + 1) * 128])
        gots_t.append(yt[:, (c - b0) * 128:(c - b0 + 1) * 128])
    ref = np.concatenate(refs, axis=1)
    _assert_close(np.concatenate(gots, axis=1), ref, f"vocab shard {rank} m={m}")
    _assert_close(np.concatenate(gots_t, axis=1), ref, f"vocab shard {rank} m={m} tiles")


@pytest.mark.parametrize("rank", [0, 7])
@pytest.mark.parametrize("m", [1, 8, 16])
def test_mlp_down_k_shard(fp8bs, full_problems, rank, m):
    """A rank's K share of MLP down: its weight columns hold whole 128x128
    blocks and its activation columns whole 1x128 blocks, so its codes and
    scales are those columns of the full quantization. The GEMM on the share
    (row-major and tile layout, the table's configuration for 5120 x 2176)
    against the oracle on the same slices, full output."""
    pr = full_problems["mlp_down"]
    k0, k1 = 128 * DOWN_SHARD_KB * rank, 128 * DOWN_SHARD_KB * (rank + 1)
    b0, b1 = DOWN_SHARD_KB * rank, DOWN_SHARD_KB * (rank + 1)
    wq = pr.wq[:, k0:k1].contiguous()
    ws = pr.ws[:, b0:b1].contiguous()
    x = pr.x[:m, k0:k1].contiguous()
    announce("mlp_down shard", rank, "k", k1 - k0, "m", m, "cfg", fp8bs.select_config(m, 5120, k1 - k0))
    y = host_bits(fp8bs.gemm(x, wq, ws))
    yt = host_bits(fp8bs.gemm_tiles(x, fp8bs.pack_weight(wq), ws))
    ref = oracle.gemm_ref(pr.xq_ref[:m, k0:k1], pr.xs_ref[:m, b0:b1], pr.wq_ref[:, k0:k1],
                          pr.ws_ref[:, b0:b1])
    _assert_close(y, ref, f"mlp_down shard {rank} m={m}")
    _assert_close(yt, ref, f"mlp_down shard {rank} m={m} tiles")


@pytest.mark.parametrize("name", ["mlp_up", "square"])
@pytest.mark.parametrize("rank", [0, 7])
@pytest.mark.parametrize("m", [1, 8, 16])
def test_column_shard_full_output(fp8bs, full_problems, name, rank, m):
    """A rank's column share of MLP up (34 of 272 block rows) or of the
    square projection (5 of 40) under an 8-way split: a contiguous slice of
    the weight's block rows with their scales, in each layout's table
    configuration for the share's shape; full output against the oracle on
    the same rows."""
    pr = full_problems[name]
    nb = pr.w_bits.shape[0] // 128 // 8
    b0, b1 = nb * rank, nb * (rank + 1)
    wq, ws = pr.wq[b0 * 128:b1 * 128], pr.ws[b0:b1]
    k = pr.w_bits.shape[1]
    announce("column shard", name, rank, "n", (b1 - b0) * 128, "m", m)
    x = pr.x[:m].contiguous()
    y = host_bits(fp8bs.gemm(x, wq, ws))
    yt = host_bits(fp8bs.gemm_tiles(x, fp8bs.pack_weight(wq), ws))
    ref = oracle.gemm_ref(pr.xq_ref[:m], pr.xs_ref[:m], pr.wq_ref[b0 * 128:b1 * 128],
                          pr.ws_ref[b0:b1])
    _assert_close(y, ref, f"{name} shard {rank} m={m} k={k}")
    _assert_close(yt, ref, f"{name} shard {rank} m={m} tiles")


@pytest.mark.parametrize("m", [8, 16])
def test_vocab_run_to_run_bit_identical(fp8bs, vocab_weight, m):
    """The 248,320-wide layer in the configuration each layout's table picks:
    ten runs give the same bits, row-major and tile-layout weights."""
    wl = WORKLOADS["vocab"]
    wq, ws = vocab_weight
    wt = fp8bs.pack_weight(wq)
    x = dev_bf16(act_bf16(wl.x_seed, wl.col_seed, 32, wl.k, wl.n_outlier, wl.outlier_factor)[:m])
    announce("vocab identity", m, fp8bs.select_config(m, wl.n, wl.k), fp8bs.tiles_select_config(m, wl.n, wl.k))
    r0, t0 = fp8bs.gemm(x, wq, ws), fp8bs.gemm_tiles(x, wt, ws)
    for _ in range(10):
        r, t = fp8bs.gemm(x, wq, ws), fp8bs.gemm_tiles(x, wt, ws)
        torch.cuda.synchronize()
        assert torch.equal(r.view(torch.int16), r0.view(torch.int16))
        assert torch.equal(t.view(torch.int16), t0.view(torch.int16))
    del wt


def _configs():
    out = []
    for (tn, wn, wk, d) in MFMA_SHAPES:
        for m in (1, 5, 8, 16, 17, 32):
            for split, red in SPLITS:
                out.append(("mfma", (1, tn, wn, wk, d, split, red), m))
    for (rt, wn, wk, d) in DOT_SHAPES:
        for m in (1, 2, 3, 4):
            for split, red in SPLITS:
                out.append(("dot", (2, rt, wn, wk, d, split, red), m))
    for (wk, d, pre) in ROWS_SHAPES:
        for m in (1, 5, 8, 16, 17, 32):
            out.append(("rows", (3, pre, 1, wk, d, 1, 0), m))
    for (wk, d) in STREAM_SHAPES:
        for m in (1, 5, 8, 9, 16, 17, 32):
            out.append(("stream", (4, 1, 1, wk, d, 1, 0), m))
    return out


@pytest.fixture(scope="module")
def ragged_problem(fp8bs):
    # K = 13 blocks: not a multiple of any waves_k, depth or split count used;
    # N = 1280 is a multiple of every row count (16 .. 128, and 80)
    return _random_problem(fp8bs, 32, 1280, 13 * 128, 77)


@pytest.mark.parametrize("path,cfg,m", _configs())
def test_every_compiled_config(fp8bs, ragged_problem, path, cfg, m):
    from fp8_block_scaled_fp8bs_amd import GemmConfig
    pr = ragged_problem
    c = GemmConfig(*cfg)
    x = pr.x[:m].contiguous()
    ref = oracle.gemm_ref(pr.xq_ref[:m], pr.xs_ref[:m], pr.wq_ref, pr.ws_ref)
    y = fp8bs.gemm_ex(c, pr.wq, pr.ws, x=x)
    torch.cuda.synchronize()
    _assert_close(host_bits(y), ref, f"{path} {cfg} m={m}")
    # the pre-quantized route through the same configuration gives the same bits
    xq, xs = fp8bs.quantize_act(x)
    y2 = fp8bs.gemm_ex(c, pr.wq, pr.ws, x_q=xq, x_s=xs)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_last_arriver_workspace_reuse(fp8bs):
    """Calls with different splits (power of two or not) and shapes share one
    workspace whose counters start as arbitrary bytes, in any order, and
    every result is the one a fresh workspace gives."""
    from fp8_block_scaled_fp8bs_amd import GemmConfig
    pr = _random_problem(fp8bs, 8, 1280, 16 * 128, 91)
    ws = torch.empty(1 << 22, dtype=torch.uint8, device="cuda")
    ws.fill_(0xA5)  # arbitrary initial counter values
    seq = [(2, (1, 1, 1, 8, 5)), (4, (1, 1, 4, 1, 5)), (8, (1, 1, 5, 2, 5)), (16, (1, 1, 1, 4, 5)),
           (3, (1, 1, 4, 1, 5)), (5, (1, 1, 1, 8, 5)), (8, (1, 1, 8, 1, 5)), (7, (1, 2, 2, 2, 4))] * 3
    for split, shape in seq:
        c = GemmConfig(*shape, split_k=split, reduce=1)
        y = fp8bs.gemm_ex(c, pr.wq, pr.ws, x=pr.x, workspace=ws)
        y_fresh = fp8bs.gemm_ex(c, pr.wq, pr.ws, x=pr.x)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_fresh.view(torch.int16)), (split, shape)
        _assert_close(host_bits(y), pr.ref, f"reuse {split} {shape}")


@pytest.mark.parametrize("m,n,k", [(8, 384, 640), (3, 1152, 1920), (16, 2048, 5120), (32, 640, 1024)])
@pytest.mark.parametrize("wk,d,pre", ROWS_SHAPES)
def test_row_range_kernel_uneven_ranges(fp8bs, m, n, k, wk, d, pre):
    """Row ranges that leave the last workgroup short, 4-row ranges and
    partial 16-row tiles; pre-quantized route gives the same bits."""
    from fp8_block_scaled_fp8bs_amd import GemmConfig
    pr = _random_problem(fp8bs, m, n, k, 7 * m + n + k + wk + d)
    c = GemmConfig(3, pre, 1, wk, d)
    y = fp8bs.gemm_ex(c, pr.wq, pr.ws, x=pr.x)
    torch.cuda.synchronize()
    _assert_close(host_bits(y), pr.ref, f"rows {wk},{d} m={m} n={n} k={k}")
    xq, xs = fp8bs.quantize_act(pr.x)
    y2 = fp8bs.gemm_ex(c, pr.wq, pr.ws, x_q=xq, x_s=xs)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


ROWS_REG_SHAPES = [(8, 5, 1), (8, 5, 2), (8, 4, 2)]  # (waves_k, K blocks per wave, pre-cast slots)


@pytest.mark.parametrize("m,n,k", [(1, 384, 640), (8, 4224, 5120), (16, 2048, 4096), (17, 640, 5120),
                                   (20, 1152, 1280), (23, 1536, 3968), (32, 4224, 5120),
                                   (32, 256, 128)])
@pytest.mark.parametrize("wk,nj,pre", ROWS_REG_SHAPES)
def test_rows_reg_kernel(fp8bs, m, n, k, wk, nj, pre):
    """Row-range kernel with register-resident activations: short last
    ranges, partial 16-row tiles, K blocks not a multiple of the waves (waves
    with fewer blocks, one block in all), m on both sides of 16 (per-wave
    cast and, fused above 16 rows, the cast through LDS); the pre-quantized
    route gives the same bits. A K range beyond waves_k * depth blocks is a
    configuration error."""
    from fp8_block_scaled_fp8bs_amd import Fp8bsError, GemmConfig
    c = GemmConfig(fp8bs.PATH_MFMA_ROWS_REG, pre, 1, wk, nj)
    announce("rows reg", c, "m", m, "n", n, "k", k)
    pr = _random_problem(fp8bs, m, n, k, 13 * m + n + k + wk + nj + pre)
    if k // 128 > wk * nj:
        with pytest.raises(Fp8bsError):
            fp8bs.gemm_ex(c, pr.wq, pr.ws, x=pr.x)
        return
    y = fp8bs.gemm_ex(c, pr.wq, pr.ws, x=pr.x)
    torch.cuda.synchronize()
    _assert_close(host_bits(y), pr.ref, f"rows reg {wk},{nj},{pre} m={m} n={n} k={k}")
    xq, xs = fp8bs.quantize_act(pr.x)
    y2 = fp8bs.gemm_ex(c, pr.wq, pr.ws, x_q=xq, x_s=xs)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    with pytest.raises(Fp8bsError):  # no K split on this path
        fp8bs.gemm_ex(GemmConfig(fp8bs.PATH_MFMA_ROWS_REG, pre, 1, wk, nj, 2), pr.wq, pr.ws, x=pr.x)


@pytest.mark.parametrize("m,n,k", [(8, 384, 640), (3, 1152, 1920), (12, 2048, 5120),
                                   (32, 640, 1024), (16, 5120, 2048)])
@pytest.mark.parametrize("wk,d", STREAM_SHAPES)
def test_stream_kernel_uneven_ranges(fp8bs, m, n, k, wk, d):
    """Streaming row-range kernel: short last ranges, partial tiles, K
    blocks not a multiple of the waves, every staging pass count; the
    pre-quantized route gives the same bits."""
    from fp8_block_scaled_fp8bs_amd import GemmConfig
    pr = _random_problem(fp8bs, m, n, k, 11 * m + n + k + wk + d)
    c = GemmConfig(4, 1, 1, wk, d)
    announce("stream", wk, d, "m", m, "n", n, "k", k)
    y = fp8bs.gemm_ex(c, pr.wq, pr.ws, x=pr.x)
    torch.cuda.synchronize()
    _assert_close(host_bits(y), pr.ref, f"stream {wk},{d} m={m} n={n} k={k}")
    xq, xs = fp8bs.quantize_act(pr.x)
    y2 = fp8bs.gemm_ex(c, pr.wq, pr.ws, x_q=xq, x_s=xs)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("name,m", [("square", 8), ("mlp_down", 8), ("tiny", 8)])
def test_run_to_run_bit_identical(fp8bs, name, m):
    wl = WORKLOADS[name]
    pr = Problem(fp8bs, wl.weight(), wl.act(m))
    ys = [fp8bs.gemm(pr.x, pr.wq, pr.ws) for _ in range(10)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(ys[0].view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("name,m", [("square", 1), ("square", 8), ("mlp_down", 8), ("tiny", 8)])
def test_fused_cast_equals_quantize_then_gemm(fp8bs, name, m):
    wl = WORKLOADS[name]
    pr = Problem(fp8bs, wl.weight(), wl.act(m))
    y = fp8bs.gemm(pr.x, pr.wq, pr.ws)
    xq, xs = fp8bs.quantize_act(pr.x)
    assert np.array_equal(xq.cpu().numpy(), pr.xq_ref)
    y2 = fp8bs.gemm_q(xq, xs, pr.wq, pr.ws)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("m,n,k", [(1, 128, 128), (32, 128, 128), (7, 256, 128), (32, 640, 2304),
                                   (3, 1024, 256), (16, 384, 4096)])
def test_small_and_ragged_shapes(fp8bs, m, n, k):
    pr = _random_problem(fp8bs, m, n, k, m * 1000 + n + k)
    y = fp8bs.gemm(pr.x, pr.wq, pr.ws)
    torch.cuda.synchronize()
    _assert_close(host_bits(y), pr.ref, f"auto m={m} n={n} k={k}")


def test_degenerate_inputs(fp8bs):
    """All-zero activation rows (scale 0), an all-zero weight block, and huge
    / tiny magnitudes."""
    rng = np.random.default_rng(5)
    m, n, k = 6, 256, 512
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    w[:128, 128:256] = 0.0
    w[128:, :128] *= 1e30
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[1] = 0.0
    x[2, :128] = -0.0
    x[3] *= 1e-30
    x[4, 300] = 3e5
    pr = Problem(fp8bs, bf16_from_f32(w), bf16_from_f32(x))
    y = fp8bs.gemm(pr.x, pr.wq, pr.ws)
    torch.cuda.synchronize()
    yb = host_bits(y)
    _assert_close(yb, pr.ref, "degenerate")
    assert np.all(oracle.bf16_bits_to_f32(yb[1]) == 0)


def test_empty_extents(fp8bs):
    wq = torch.zeros((256, 256), dtype=torch.uint8, device="cuda")
    ws = torch.ones((2, 2), dtype=torch.float32, device="cuda")
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda")
    y = fp8bs.gemm(x, wq, ws)
    assert y.shape == (0, 256)
    # k == 0: the empty sum
    out = torch.full((4, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    x0 = torch.zeros((4, 0), dtype=torch.bfloat16, device="cuda")
    wq0 = torch.zeros((256, 0), dtype=torch.uint8, device="cuda")
    ws0 = torch.zeros((2, 0), dtype=torch.float32, device="cuda")
    fp8bs.gemm(x0, wq0, ws0, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)


def test_kernels_ran_and_one_runtime(fp8bs):
    before = {k: fp8bs.launch_count(k) for k in ("gemm_mfma", "gemm_dot", "quant_weight")}
    pr = _random_problem(fp8bs, 8, 512, 1024, 3)
    fp8bs.gemm(pr.x, pr.wq, pr.ws)
    fp8bs.gemm(pr.x[:1].contiguous(), pr.wq, pr.ws)
    torch.cuda.synchronize()
    assert fp8bs.launch_count("gemm_mfma") > before["gemm_mfma"]
    assert fp8bs.launch_count("gemm_dot") > before["gemm_dot"]
    assert fp8bs.launch_count("quant_weight") > before["quant_weight"]
    maps = fp8bs.hip_runtime_mappings()
    assert len(maps["libamdhip64"]) == 1 and len(maps["libfp8bs"]) == 1, maps


def test_errors_raise(fp8bs):
    pr = _random_problem(fp8bs, 8, 256, 256, 4)
    with pytest.raises(fp8bs.Fp8bsError):
        bad = torch.zeros((40, 256), dtype=torch.bfloat16, device="cuda")
        fp8bs.gemm_ex(fp8bs.GemmConfig(1, 1, 1, 4, 5), pr.wq, pr.ws, x=bad)  # decode kernel, m > 32


@pytest.mark.parametrize("rows_cfg", [(4, 8, 4), (1, 8, 3), (2, 8, 6), (2, 8, 4)])
@pytest.mark.parametrize("m,n,k,split", [(32, 2048, 2560, 2), (20, 1536, 1664, 3), (9, 1024, 1280, 4)])
def test_rows_split_parity(fp8bs, rows_cfg, m, n, k, split):
    """Row-range kernels with K split over workgroups (fp32 partials summed in
    split order by the reduce kernel): full output within tolerance, fused
    cast equal to quantize-then-multiply, ragged K ranges."""
    from fp8_block_scaled_fp8bs_amd import GemmConfig
    pre, wk, d = rows_cfg
    cfg = GemmConfig(fp8bs.PATH_MFMA_ROWS, pre, 1, wk, d, split)
    announce("rows split", cfg, m, n, k)
    pr = _random_problem(fp8bs, m, n, k, 9000 + m + n + k + split)
    y = fp8bs.gemm_ex(cfg, pr.wq, pr.ws, x=pr.x)
    xq, xs = fp8bs.quantize_act(pr.x)
    yq = fp8bs.gemm_ex(cfg, pr.wq, pr.ws, x_q=xq, x_s=xs)
    torch.cuda.synchronize()
    _assert_close(host_bits(y), pr.ref, f"rows split {cfg}")
    assert np.array_equal(host_bits(y), host_bits(yq))
