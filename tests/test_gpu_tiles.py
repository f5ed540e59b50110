"""GPU tests of the tile layout of the weight codes (fp8bs_pack_weight and
the *_tiles GEMM calls): the rearrangement is the permutation the header
describes, checked against a numpy reshape written from that description;
every tile-layout kernel (decode and prefill sizes) gives the same bits as
the row-major kernel of the same configuration and stays within
2^-7 |ref| + 1e-3 rms(ref) of the CPU oracle; full-size shapes in the
automatic configuration; ragged row ranges (workgroup ranges that do not
start on a 16-row tile); the SwiGLU call; graph replays; determinism."""
import numpy as np
import pytest

import oracle
from gpu_util import announce, dev_bf16, host_bits, need_gpu, same_bits_f32, torch
from workloads import WORKLOADS, act_bf16, bf16_from_f32, weight_rows_bf16

pytestmark = pytest.mark.gpu

TOL = dict(rel=2.0 ** -7, abs_rms=1e-3)

# tile-layout kernels compiled into the library
MFMA_TILES = [(1, 2, 4, 5), (1, 5, 1, 5), (1, 5, 2, 5), (1, 8, 1, 5), (1, 5, 2, 2), (2, 5, 1, 5),
              (1, 1, 4, 5), (1, 1, 8, 5), (4, 1, 4, 2), (1, 2, 4, 2)]
ROWS_TILES = [(8, 4, 4), (8, 3, 1), (8, 6, 2)]   # (waves along K, tiles in flight, pre-cast)
STREAM_TILES = [(8, 6)]                          # (waves along K, tiles in flight)
ROWS_REG_TILES = [(8, 5, 1)]                     # (waves along K, blocks per wave, pre-cast)


@pytest.fixture(scope="module")
def fp8bs():
    need_gpu()
    import fp8_block_scaled_fp8bs_amd as m
    m.load()
    return m


def tiles_reference(codes: np.ndarray) -> np.ndarray:
    """The tile layout from its description: tile (r/16, kb) holds 2 KB;
    KB h holds columns 32g + 16h .. +15 of each quarter g, and inside it the
    16 bytes of (row r%16, quarter g) sit at slot 16g + r%16."""
    n, k = codes.shape
    a = codes.reshape(n // 16, 16, k // 128, 4, 2, 16)      # [tile][row][kb][g][h][byte]
    return np.ascontiguousarray(a.transpose(0, 2, 4, 3, 1, 5)).reshape(n, k)  # [tile][kb][h][g][row][byte]


def _assert_close(y_bits, ref, what, rms=None):
    rep = oracle.tolerance_report(y_bits, ref, rms=rms, **TOL)
    assert rep["finite"] and rep["n_bad"] == 0, f"{what}: {rep}"


def _bits_equal(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("n,k", [(128, 128), (128, 256), (1280, 1664), (5120, 5120)])
def test_pack_is_the_described_permutation(fp8bs, n, k):
    announce("pack", n, k)
    rng = np.random.default_rng(n + k)
    codes = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
    t = fp8bs.pack_weight(torch.from_numpy(codes).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(t.cpu().numpy(), tiles_reference(codes))


def test_pack_single_byte_positions(fp8bs):
    """A lone nonzero byte at W[r][c] lands where the header puts it."""
    n, k = 128, 256
    for (r, c) in [(0, 0), (1, 0), (15, 0), (16, 0), (0, 15), (0, 16), (0, 31), (0, 32),
                   (3, 77), (17, 128 + 100), (31, 255), (127, 255), (100, 130)]:
        codes = np.zeros((n, k), np.uint8)
        codes[r, c] = 7
        t = fp8bs.pack_weight(torch.from_numpy(codes).cuda()).cpu().numpy().reshape(-1)
        kb, g, h, b = c // 128, (c % 128) // 32, (c % 32) // 16, c % 16
        off = ((r // 16) * (k // 128) + kb) * 2048 + h * 1024 + (16 * g + r % 16) * 16 + b
        assert t[off] == 7 and np.count_nonzero(t) == 1, (r, c)


class Problem:
    def __init__(self, fp8bs, w_bits, x_bits):
        self.x = dev_bf16(x_bits)
        self.wq, self.ws = fp8bs.quantize_weight(dev_bf16(w_bits))
        self.wt = fp8bs.pack_weight(self.wq)
        self.wq_ref, self.ws_ref = oracle.quantize_weight_ref(w_bits)
        assert np.array_equal(self.wq.cpu().numpy(), self.wq_ref)
        assert same_bits_f32(self.ws.cpu().numpy(), self.ws_ref)
        self.xq_ref, self.xs_ref = oracle.quantize_act_ref(x_bits)


def _random_problem(fp8bs, m, n, k, seed):
    rng = np.random.default_rng(seed)
    w = bf16_from_f32((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[:, rng.choice(k, max(1, k // 100), replace=False)] *= 10
    return Problem(fp8bs, w, bf16_from_f32(x))


@pytest.fixture(scope="module")
def ragged(fp8bs):
    # K = 13 blocks (not a multiple of any waves_k, depth or split); N = 1280:
    # the row-range kernels give each workgroup 8 rows (16-row ranges would
    # idle most compute units), so ranges start in the middle of 16-row tiles
    return _random_problem(fp8bs, 32, 1280, 13 * 128, 4242)


def _tile_configs():
    out = []
    for (tn, wn, wk, d) in MFMA_TILES:
        for m in (1, 5, 8, 16, 17, 32):
            for split, red in ((1, 0), (3, 0), (4, 1)):
                out.append((1, tn, wn, wk, d, split, red, m))
    for (wk, d, pre) in ROWS_TILES:
        for m in (1, 5, 8, 16, 17, 22):
            out.append((3, pre, 1, wk, d, 1, 0, m))
    for (wk, d) in STREAM_TILES:
        for m in (1, 8, 9, 16, 17, 32):
            out.append((4, 1, 1, wk, d, 1, 0, m))
    for (wk, nj, pre) in ROWS_REG_TILES:
        for m in (1, 8, 16, 17, 24, 32):
            out.append((6, pre, 1, wk, nj, 1, 0, m))
    return out


@pytest.mark.parametrize("cfg", _tile_configs())
def test_every_tile_kernel_matches_row_major_and_oracle(fp8bs, ragged, cfg):
    from fp8_block_scaled_fp8bs_amd import GemmConfig
    *c, m = cfg
    pr = ragged
    rows_cfg = GemmConfig(*c)
    tile_cfg = GemmConfig(*c, weight_layout=fp8bs.LAYOUT_TILES)
    announce("tiles", tile_cfg, m)
    x = pr.x[:m].contiguous()
    y_rows = fp8bs.gemm_ex(rows_cfg, pr.wq, pr.ws, x=x)
    y_tiles = fp8bs.gemm_ex(tile_cfg, pr.wt, pr.ws, x=x)
    xq, xs = fp8bs.quantize_act(x)
    y_tiles_q = fp8bs.gemm_ex(tile_cfg, pr.wt, pr.ws, x_q=xq, x_s=xs)
    torch.cuda.synchronize()
    assert _bits_equal(y_rows, y_tiles), f"{tile_cfg} m={m}: tile layout differs from row-major"
    assert _bits_equal(y_tiles, y_tiles_q)
    ref = oracle.gemm_ref(pr.xq_ref[:m], pr.xs_ref[:m], pr.wq_ref, pr.ws_ref)
    _assert_close(host_bits(y_tiles), ref, f"tiles {tile_cfg} m={m}")


@pytest.fixture(scope="module")
def full(fp8bs):
    out = {}
    for name in ("square", "mlp_up", "mlp_down"):
        wl = WORKLOADS[name]
        announce("full-size tile weight", name, wl.n, wl.k)
        x_bits = act_bf16(wl.x_seed, wl.col_seed, 32, wl.k, wl.n_outlier, wl.outlier_factor)
        out[name] = Problem(fp8bs, wl.weight(), x_bits)
        torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", ["square", "mlp_up", "mlp_down"])
@pytest.mark.parametrize("m", [1, 2, 4, 8, 16, 32])
def test_full_size_auto_config(fp8bs, full, name, m):
    """The automatic tile-layout configuration at every step-mix m: the
    same bits as the row-major kernel of that configuration, within the
    tolerance of the oracle, and the fused call equal to the pre-quantized
    one."""
    from fp8_block_scaled_fp8bs_amd import GemmConfig
    pr = full[name]
    n, k = pr.wq.shape
    cfg = fp8bs.tiles_select_config(m, n, k)
    announce("full tiles", name, m, cfg)
    x = pr.x[:m].contiguous()
    y = fp8bs.gemm_tiles(x, pr.wt, pr.ws)
    xq, xs = fp8bs.quantize_act(x)
    y_q = fp8bs.gemm_q_tiles(xq, xs, pr.wt, pr.ws)
    rows_cfg = GemmConfig(cfg.path, cfg.tiles_n, cfg.waves_n, cfg.waves_k, cfg.depth, cfg.split_k,
                          cfg.reduce, cfg.epilogue)
    y_rows = fp8bs.gemm_ex(rows_cfg, pr.wq, pr.ws, x=x)
    torch.cuda.synchronize()
    assert _bits_equal(y, y_q)
    assert _bits_equal(y, y_rows)
    if m in (1, 8, 32):
        ref = oracle.gemm_ref(pr.xq_ref[:m], pr.xs_ref[:m], pr.wq_ref, pr.ws_ref)
        _assert_close(host_bits(y), ref, f"{name} tiles m={m}")


def test_vocab_sampled_block_rows(fp8bs):
    """The 248,320 x 5,120 output layer in the tile layout at m = 1, 8, 16:
    sampled 128-row block rows of W are regenerated alone and checked (codes
    bit-exact, outputs within tolerance, with the rms over the sampled
    outputs)."""
    wl = WORKLOADS["vocab"]
    w = dev_bf16(wl.weight())
    wq, ws = fp8bs.quantize_weight(w)
    del w
    wt = fp8bs.pack_weight(wq)
    x_bits = act_bf16(wl.x_seed, wl.col_seed, 16, wl.k, wl.n_outlier, wl.outlier_factor)
    nbn = wl.n // 128
    cols = (0, 1, 777, nbn // 2, nbn - 1)
    qrefs = {}
    for c in cols:
        qr, sr = oracle.quantize_weight_ref(weight_rows_bf16(wl.w_seed, c, 128, wl.k))
        assert np.array_equal(wq[c * 128:(c + 1) * 128].cpu().numpy(), qr)
        qrefs[c] = (qr, sr)
    for m in (1, 8, 16):
        announce("vocab tiles", m, fp8bs.tiles_select_config(m, wl.n, wl.k))
        y = host_bits(fp8bs.gemm_tiles(dev_bf16(x_bits[:m]), wt, ws))
        xq, xs = oracle.quantize_act_ref(x_bits[:m])
        refs = [oracle.gemm_ref(xq, xs, *qrefs[c]) for c in cols]
        gots = [y[:, c * 128:(c + 1) * 128] for c in cols]
        _assert_close(np.concatenate(gots, axis=1), np.concatenate(refs, axis=1),
                      f"vocab tiles m={m}")


@pytest.mark.parametrize("name", ["square", "mlp_up", "mlp_down"])
def test_tiles_deterministic(fp8bs, full, name):
    """Ten runs at M = 8 in the configuration each layout's table picks (the
    bench's kernels) give the same bits, on tile-layout and row-major
    weights."""
    pr = full[name]
    x = pr.x[:8].contiguous()
    y0 = fp8bs.gemm_tiles(x, pr.wt, pr.ws)
    r0 = fp8bs.gemm(x, pr.wq, pr.ws)
    for _ in range(10):
        y = fp8bs.gemm_tiles(x, pr.wt, pr.ws)
        r = fp8bs.gemm(x, pr.wq, pr.ws)
        torch.cuda.synchronize()
        assert _bits_equal(y, y0) and _bits_equal(r, r0)


@pytest.mark.parametrize("m,n,k,wn,split", [(300, 512, 1280, 2, 1), (129, 768, 2048, 2, 3),
                                             (64, 256, 384, 2, 1), (1000, 1280, 13 * 128, 2, 1),
                                             (200, 1024, 1024, 4, 1), (33, 512, 128, 2, 1)])
def test_prefill_tiles_matches_row_major_and_oracle(fp8bs, m, n, k, wn, split):
    """The prefill-size kernel (m > 32) on tile-layout weights: the same bits
    as on row-major weights in the same configuration, within the tolerance
    of the oracle; ragged m tails, split K, one K block, both tile widths."""
    from fp8_block_scaled_fp8bs_amd import GemmConfig
    pr = _random_problem(fp8bs, m, n, k, 5000 + m + n + k)
    rows_cfg = GemmConfig(fp8bs.PATH_PREFILL, 1, wn, 2, 2, split)
    tile_cfg = GemmConfig(fp8bs.PATH_PREFILL, 1, wn, 2, 2, split, weight_layout=fp8bs.LAYOUT_TILES)
    announce("prefill tiles", tile_cfg, m, n, k)
    y_rows = fp8bs.gemm_ex(rows_cfg, pr.wq, pr.ws, x=pr.x)
    y_tiles = fp8bs.gemm_ex(tile_cfg, pr.wt, pr.ws, x=pr.x)
    torch.cuda.synchronize()
    assert _bits_equal(y_rows, y_tiles)
    ref = oracle.gemm_ref(pr.xq_ref, pr.xs_ref, pr.wq_ref, pr.ws_ref)
    _assert_close(host_bits(y_tiles), ref, f"prefill tiles {tile_cfg} m={m}")


def test_prefill_tiles_auto(fp8bs, full):
    """gemm_tiles at prefill sizes picks the tile-layout prefill kernel and
    gives the bits of the row-major call (same configuration)."""
    pr = full["square"]
    n, k = pr.wq.shape
    rng = np.random.default_rng(77)
    x = dev_bf16(bf16_from_f32(rng.standard_normal((256, k)).astype(np.float32)))
    cfg = fp8bs.tiles_select_config(256, n, k)
    announce("prefill tiles auto", cfg)
    assert cfg.path == fp8bs.PATH_PREFILL and cfg.weight_layout == fp8bs.LAYOUT_TILES
    y_t = fp8bs.gemm_tiles(x, pr.wt, pr.ws)
    y_r = fp8bs.gemm(x, pr.wq, pr.ws)
    torch.cuda.synchronize()
    assert _bits_equal(y_t, y_r)


def test_tiles_graph_replays_match_eager(fp8bs, full):
    """A tile-layout split configuration (fp32 partials in the workspace and
    the reduce kernel) captured in a HIP graph: every replay, with eager work
    and synchronizations between replays, equals the eager result."""
    pr = full["mlp_down"]
    x = pr.x[:8].contiguous()
    n, k = pr.wq.shape
    cfg = fp8bs.tiles_select_config(8, n, k)
    assert cfg.split_k > 1
    ws = torch.empty(fp8bs.workspace_bytes(8, n, k), dtype=torch.uint8, device="cuda")
    y = torch.empty((8, n), dtype=torch.bfloat16, device="cuda")
    eager = fp8bs.gemm_tiles(x, pr.wt, pr.ws)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        fp8bs.gemm_tiles(x, pr.wt, pr.ws, out=y, workspace=ws)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            fp8bs.gemm_tiles(x, pr.wt, pr.ws, out=y, workspace=ws)
    torch.cuda.synchronize()
    for i in range(4):
        y.zero_()
        ws.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _bits_equal(y, eager), f"replay {i}"
        fp8bs.gemm_tiles(x, pr.wt, pr.ws)  # eager work between replays


@pytest.mark.parametrize("m", [1, 2, 4, 8, 16, 32])
def test_swiglu_tiles(fp8bs, full, m):
    """The up/gate projection with the SwiGLU epilogue on tile-layout
    weights: y equals the plain tile-layout GEMM bit for bit, and h equals
    the standalone epilogue applied to that y (itself checked against the
    oracle in the SwiGLU tests)."""
    pr = full["mlp_up"]
    x = pr.x[:m].contiguous()
    announce("swiglu tiles", m, fp8bs.tiles_select_config(m, *pr.wq.shape))
    y, hq, hs = fp8bs.gemm_swiglu_tiles(x, pr.wt, pr.ws)
    y_plain = fp8bs.gemm_tiles(x, pr.wt, pr.ws)
    hq2, hs2 = fp8bs.swiglu_quant(y)
    torch.cuda.synchronize()
    assert _bits_equal(y, y_plain)
    assert torch.equal(hq, hq2)
    assert same_bits_f32(hs.cpu().numpy(), hs2.cpu().numpy())
