"""GPU parity of the MLP epilogue (SwiGLU on the up/gate projection's output
and the 1 x 128 FP8 cast of its result) against the CPU oracle.

The epilogue turns floating-point values into integer codes, so the checks
are layered:

* standalone epilogue on seeded bf16 inputs: codes and scales bit-exact to
  the oracle, block by block. Kernel and oracle both evaluate h = silu(g) * u
  in fp64 and round it once to bf16; they can differ only through their fp64
  exponential (an ulp or two) and the rounding of one division and one
  product, a relative 2^-50 or so. So where the exact h lies within a
  relative 2^-40 of a bf16 rounding boundary either neighbour is a correct
  bf16 h, and the block passes when the kernel's codes and scale equal the
  oracle's cast of one of those candidate blocks. Everywhere else there is
  exactly one correct answer;
* fused call: y equal bit for bit to the plain GEMM in the same
  configuration and within the GEMM tolerance of the oracle; h equal bit for
  bit to the standalone epilogue applied to that y; and, end to end against
  the oracle's own chain, every dequantized h within a bound derived from the
  GEMM tolerance, with at least 99% of the codes identical.
"""
import dataclasses
import itertools

import numpy as np
import pytest

import oracle
from gpu_util import announce, dev_bf16, host_bits, need_gpu, same_bits_f32, torch
from workloads import WORKLOADS, act_bf16, bf16_from_f32

pytestmark = pytest.mark.gpu

TOL = dict(rel=2.0 ** -7, abs_rms=1e-3)
WINDOW = 2.0 ** -40   # relative distance from a bf16 rounding boundary treated as a tie


@pytest.fixture(scope="module")
def fp8bs():
    need_gpu()
    import fp8_block_scaled_fp8bs_amd as m
    m.load()
    return m


def _host(hq, hs):
    torch.cuda.synchronize()
    return hq.cpu().numpy(), hs.cpu().numpy()


def check_epilogue_exact(y_bits, hq, hs):
    """Block-wise bit-exact comparison of the epilogue with the oracle, with
    the bf16 rounding of h taken as ambiguous within WINDOW of a boundary.
    Returns (blocks, ambiguous blocks)."""
    h = oracle.swiglu_ref(y_bits)
    lo = oracle.bf16_bits_from_f64(h * (1.0 - WINDOW))
    hi = oracle.bf16_bits_from_f64(h * (1.0 + WINDOW))
    rne = oracle.bf16_bits_from_f64(h)
    m, inter = h.shape
    nb = inter // 128
    codes_ref, scales_ref = oracle.quantize_act_ref(rne)
    amb = (lo != hi).reshape(m, nb, 128)
    n_amb = 0
    for r in range(m):
        for b in range(nb):
            sl = slice(128 * b, 128 * b + 128)
            got_c, got_s = hq[r, sl], hs[r, b:b + 1]
            idx = np.flatnonzero(amb[r, b])
            if idx.size == 0:
                assert np.array_equal(got_c, codes_ref[r, sl]), (r, b)
                assert same_bits_f32(got_s, scales_ref[r, b:b + 1]), (r, b, got_s, scales_ref[r, b])
                continue
            n_amb += 1
            assert idx.size <= 8, f"block ({r},{b}) has {idx.size} near-tie elements"
            base = rne[r, sl].copy()
            ok = False
            for choice in itertools.product((0, 1), repeat=idx.size):
                cand = base.copy()
                for j, c in zip(idx, choice):
                    cand[j] = (hi if c else lo)[r, 128 * b + j]
                cc, cs = oracle.quantize_act_ref(cand[None, :])
                if np.array_equal(cc[0], got_c) and same_bits_f32(cs[0], got_s):
                    ok = True
                    break
            assert ok, f"block ({r},{b}): no bf16 rounding of h gives the kernel's codes/scale"
    return m * nb, n_amb


def _y_bits(seed, m, inter, scale=3.0):
    rng = np.random.default_rng(seed)
    y = (rng.standard_normal((m, 2 * inter)) * scale).astype(np.float32)
    return bf16_from_f32(y)


@pytest.mark.parametrize("m,inter,seed", [(1, 128, 1), (3, 384, 2), (8, 1024, 3), (16, 2048, 4),
                                          (32, 640, 5), (8, 17408, 6)])
def test_standalone_epilogue_matches_oracle(fp8bs, m, inter, seed):
    announce("swiglu_quant", "m", m, "inter", inter, "seed", seed)
    y_bits = _y_bits(seed, m, inter)
    hq, hs = _host(*fp8bs.swiglu_quant(dev_bf16(y_bits)))
    blocks, amb = check_epilogue_exact(y_bits, hq, hs)
    assert amb < blocks


def test_standalone_epilogue_special_values(fp8bs):
    """Signed zeros, an all-zero block (scale 0), saturating silu at both
    ends, and one huge outlier per block beside tiny values."""
    m, inter = 4, 512
    g = np.zeros((m, inter), np.float32)
    u = np.zeros((m, inter), np.float32)
    # row 0: gate +0 / -0 against up of both signs: h = +-0 (codes 0x00 / 0x80)
    g[0, :128] = np.where(np.arange(128) % 2, -0.0, 0.0)
    u[0, :128] = np.where(np.arange(128) % 4 < 2, 1.5, -1.5)
    # row 0 block 1: large positive gate (silu(g) = g), large negative gate (silu -> -0)
    g[0, 128:256] = np.where(np.arange(128) % 2, 60.0, -60.0)
    u[0, 128:256] = 2.0
    # row 1: one outlier per block beside tiny values
    rng = np.random.default_rng(11)
    g[1] = rng.standard_normal(inter).astype(np.float32) * 1e-3
    u[1] = rng.standard_normal(inter).astype(np.float32)
    g[1, ::128] = 40.0
    u[1, ::128] = 300.0
    # rows 2, 3: ordinary values of very different magnitudes
    g[2] = rng.standard_normal(inter).astype(np.float32) * 1e-12   # block amax below 2^-60
    u[2] = rng.standard_normal(inter).astype(np.float32) * 1e-10
    g[3] = rng.standard_normal(inter).astype(np.float32) * 8
    u[3] = rng.standard_normal(inter).astype(np.float32) * 1e4
    y_bits = np.concatenate([bf16_from_f32(g), bf16_from_f32(u)], axis=1)
    hq, hs = _host(*fp8bs.swiglu_quant(dev_bf16(y_bits)))
    check_epilogue_exact(y_bits, hq, hs)
    assert hs[0, 0] == 0.0 and hs[0, 2] == 0.0
    assert np.array_equal(hq[0, :128] & 0x80, np.where((np.arange(128) % 2 == 1) ^
                                                        (np.arange(128) % 4 >= 2), 0x80, 0))


def _negative_gate_rows(rng, inter):
    """Gate and up rows whose h needs fp64: gates where e^g is below the
    smallest normal fp32 (g < -87.3) or overflows e^-g in fp32 (g < -88.7),
    with up values from 1 to near the largest bf16 so that h spans normal
    and subnormal bf16 values and zeros."""
    rows_g, rows_u = [], []
    j = np.arange(inter)
    # whole blocks of gates in [-97, -85] with up = 1
    rows_g.append(-85.0 - 12.0 * rng.random(inter))
    rows_u.append(np.ones(inter))
    # mixed blocks: every other gate very negative, the rest ordinary
    g = rng.standard_normal(inter) * 3.0
    g[::2] = -85.0 - 12.0 * rng.random(inter // 2)
    rows_g.append(g)
    rows_u.append(rng.standard_normal(inter) * 4.0)
    # the bf16 neighbours of the fp32 overflow point -88.72 (spacing 0.5 there)
    rows_g.append(np.array([-87.5, -88.0, -88.5, -89.0, -89.5, -90.0, -88.0, -89.0])[j % 8])
    rows_u.append(np.where(j % 3 == 0, 1.0, np.where(j % 3 == 1, -2.5, 1e20)))
    # far below: g in [-180, -87] with up near the top of the bf16 range, so
    # h is normal, subnormal or zero; a block of gates -800 and -1e30 (h = -0)
    g = -87.0 - 93.0 * rng.random(inter)
    g[256:384] = np.where(j[256:384] % 2, -800.0, -1e30)
    rows_g.append(g)
    rows_u.append(np.exp(rng.uniform(0.0, 88.0, inter)) * np.where(j % 5 == 0, -1.0, 1.0))
    return np.array(rows_g, np.float32), np.array(rows_u, np.float32)


def test_standalone_epilogue_very_negative_gates(fp8bs):
    """Gates below -85, where silu(g) = g e^g needs more than fp32 range: the
    kernel's codes and scales equal the oracle's block by block."""
    inter = 512
    g, u = _negative_gate_rows(np.random.default_rng(13), inter)
    y_bits = np.concatenate([bf16_from_f32(g), bf16_from_f32(u)], axis=1)
    hq, hs = _host(*fp8bs.swiglu_quant(dev_bf16(y_bits)))
    blocks, _ = check_epilogue_exact(y_bits, hq, hs)
    assert blocks == 4 * 4
    h = oracle.swiglu_quant_ref(y_bits)[0]
    # the cases reach nonzero h below the fp32 limits, and exact zeros
    hf = oracle.bf16_bits_to_f32(h)
    assert np.any((hf != 0) & (np.abs(hf) < 2.0 ** -126)) and np.any(hf[0] != 0)
    assert np.all(hf[3, 256:384] == 0)


# Every placement of the epilogue on outputs whose gate half is very
# negative: (path, tiles_n, waves_n, waves_k, depth, split_k, reduce, epilogue).
NEG_GATE_CONFIGS = [
    (1, 1, 2, 4, 5, 1, 0, 1),    # inside the MFMA grid kernel
    (3, 4, 1, 8, 4, 1, 0, 1),    # inside the row-range kernel
    (1, 1, 5, 1, 5, 4, 0, 0),    # in the split sum
    (1, 1, 5, 1, 5, 1, 0, 0),    # second kernel
]


@pytest.mark.parametrize("cfg", NEG_GATE_CONFIGS)
def test_fused_very_negative_gates(fp8bs, cfg):
    """A GEMM whose gate outputs fall in [-101, -86] and whose up outputs span
    1e-3 .. 1e30: y equals the plain GEMM and is within tolerance of the
    oracle, h equals the standalone epilogue on that y, and h equals the
    oracle's epilogue applied to the kernel's y, block by block."""
    from fp8_block_scaled_fp8bs_amd import GemmConfig
    c = GemmConfig(*cfg)
    m, inter, k = 8, 640, 512
    rng = np.random.default_rng(21)
    x = (1.0 + 0.01 * rng.standard_normal((m, k))).astype(np.float32)
    n_idx = np.arange(inter)
    w_gate = -(84.0 + 14.0 * (n_idx % 128) / 128.0) / k
    # one magnitude per 128-row block (1e-3 .. 1e29), up to 10x within it, so
    # the block quantization keeps every row's weights
    w_up = 10.0 ** (-3.0 + 8.0 * (n_idx // 128) + (n_idx % 128) / 128.0) / k
    w = np.concatenate([np.repeat(w_gate[:, None], k, 1), np.repeat(w_up[:, None], k, 1)])
    w = w * (1.0 + 0.01 * rng.standard_normal(w.shape))
    pr = Problem(fp8bs, bf16_from_f32(w.astype(np.float32)), bf16_from_f32(x))
    announce("gemm_swiglu very negative gates", c)
    y, hq, hs = fp8bs.gemm_swiglu_ex(c, pr.wq, pr.ws, x=pr.x)
    y_plain = fp8bs.gemm_ex(dataclasses.replace(c, epilogue=0), pr.wq, pr.ws, x=pr.x)
    hq2, hs2 = fp8bs.swiglu_quant(y)
    torch.cuda.synchronize()
    yb = host_bits(y)
    assert np.array_equal(yb, host_bits(y_plain))
    rep = oracle.tolerance_report(yb, pr.ref(m), **TOL)
    assert rep["finite"] and rep["n_bad"] == 0, rep
    gate = oracle.bf16_bits_to_f32(yb[:, :inter])
    assert gate.max() < -80.0 and gate.min() > -105.0
    hq, hs = hq.cpu().numpy(), hs.cpu().numpy()
    assert np.array_equal(hq, hq2.cpu().numpy()) and same_bits_f32(hs, hs2.cpu().numpy())
    check_epilogue_exact(yb, hq, hs)


# --------------------------------------------------------- fused up/gate ---

class Problem:
    def __init__(self, fp8bs, w_bits, x_bits):
        self.w_bits, self.x_bits = w_bits, x_bits
        self.x = dev_bf16(x_bits)
        self.wq, self.ws = fp8bs.quantize_weight(dev_bf16(w_bits))
        self.wq_ref, self.ws_ref = oracle.quantize_weight_ref(w_bits)
        assert np.array_equal(self.wq.cpu().numpy(), self.wq_ref)
        self.xq_ref, self.xs_ref = oracle.quantize_act_ref(x_bits)

    def ref(self, m):
        return oracle.gemm_ref(self.xq_ref[:m], self.xs_ref[:m], self.wq_ref, self.ws_ref)


def _random_problem(fp8bs, m, n, k, seed):
    rng = np.random.default_rng(seed)
    w = bf16_from_f32((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[:, rng.choice(k, max(1, k // 100), replace=False)] *= 10
    return Problem(fp8bs, w, bf16_from_f32(x))


def check_fused(fp8bs, pr, m, cfg, ref):
    """Run the fused call (explicit cfg, or automatic when None) and apply
    the layered checks. Returns the fraction of codes equal to the oracle
    chain's."""
    x = pr.x[:m].contiguous()
    if cfg is None:
        cfg = fp8bs.swiglu_select_config(m, pr.w_bits.shape[0], pr.w_bits.shape[1])
        y, hq, hs = fp8bs.gemm_swiglu(x, pr.wq, pr.ws)
    else:
        y, hq, hs = fp8bs.gemm_swiglu_ex(cfg, pr.wq, pr.ws, x=x)
    y_plain = fp8bs.gemm_ex(dataclasses.replace(cfg, epilogue=0), pr.wq, pr.ws, x=x)
    hq2, hs2 = fp8bs.swiglu_quant(y)
    torch.cuda.synchronize()
    yb = host_bits(y)
    # y: the plain GEMM's bits in the same configuration, within tolerance
    assert np.array_equal(yb, host_bits(y_plain)), f"y differs from the plain GEMM ({cfg})"
    rep = oracle.tolerance_report(yb, ref, **TOL)
    assert rep["finite"] and rep["n_bad"] == 0, f"y vs oracle {cfg}: {rep}"
    # h: the standalone epilogue's bits on that y
    hq, hs = hq.cpu().numpy(), hs.cpu().numpy()
    assert np.array_equal(hq, hq2.cpu().numpy()), f"h codes differ from the standalone epilogue ({cfg})"
    assert same_bits_f32(hs, hs2.cpu().numpy()), f"h scales differ ({cfg})"
    # end to end against the oracle's own chain
    inter = ref.shape[1] // 2
    g, u = ref[:, :inter], ref[:, inter:]
    rms = float(np.sqrt(np.mean(ref * ref)))
    dg = TOL["rel"] * np.abs(g) + TOL["abs_rms"] * rms
    du = TOL["rel"] * np.abs(u) + TOL["abs_rms"] * rms
    h_exact = oracle.silu_ref(g) * u
    # |silu'| <= 1.1 everywhere; bf16 rounding of h; half an E4M3 step of the
    # block's grid (at most 2^-4 |h| for normal codes, s * 2^-10 below them)
    dh = 1.1 * (np.abs(u) + du) * dg + (np.abs(oracle.silu_ref(g)) + 1.1 * dg) * du
    dh = dh + 2.0 ** -8 * (np.abs(h_exact) + dh)
    s = hs.astype(np.float64).repeat(128, axis=1)
    deq = oracle.e4m3_decode(hq) * s
    bound = dh + 2.0 ** -4 * (np.abs(h_exact) + dh) + s * 2.0 ** -10 + 1e-30
    bad = np.abs(deq - h_exact) > bound
    assert not bad.any(), f"{bad.sum()} dequantized h outside the derived bound ({cfg})"
    _, codes_chain, _ = oracle.swiglu_quant_ref(
        np.concatenate([oracle.bf16_bits_from_f64(g), oracle.bf16_bits_from_f64(u)], axis=1))
    same = float(np.mean(codes_chain == hq))
    assert same >= 0.99, f"only {same:.4f} of the codes equal the oracle chain's ({cfg})"
    return same


# Every way of running the epilogue, on shapes that span several 128-column
# blocks, ragged row ranges and split sums: (m, inter, k, config). Configs
# are (path, tiles_n, waves_n, waves_k, depth, split_k, reduce, epilogue);
# epilogue 0 = separate (the split sum, or a second kernel), 1 = in the GEMM.
FUSED_CASES = [
    (1, 640, 256, (1, 1, 1, 4, 5, 1, 0, 1)),
    (3, 640, 1024, (1, 1, 2, 4, 5, 1, 0, 1)),
    (8, 640, 384, (1, 1, 5, 1, 5, 1, 0, 1)),     # 80-column groups straddle the blocks
    (8, 1280, 1024, (1, 2, 4, 1, 5, 1, 0, 1)),
    (16, 384, 2048, (1, 1, 8, 1, 5, 1, 0, 1)),
    (32, 640, 1024, (1, 1, 2, 4, 5, 1, 0, 1)),
    (8, 640, 1024, (3, 4, 1, 8, 4, 1, 0, 1)),    # row-range kernels
    (2, 1280, 512, (3, 1, 1, 8, 3, 1, 0, 1)),
    (16, 640, 1024, (3, 2, 1, 8, 6, 1, 0, 1)),
    (32, 384, 640, (3, 1, 1, 8, 3, 1, 0, 1)),
    (8, 640, 1024, (4, 1, 1, 8, 6, 1, 0, 1)),    # streaming row-range kernel
    (1, 1280, 512, (4, 1, 1, 8, 4, 1, 0, 1)),
    (8, 640, 1024, (6, 1, 1, 8, 5, 1, 0, 1)),    # register-activation row-range kernel
    (24, 1280, 5120, (6, 1, 1, 8, 5, 1, 0, 1)),
    (32, 384, 640, (6, 1, 1, 8, 5, 1, 0, 0)),
    (8, 640, 1024, (1, 1, 5, 1, 5, 4, 0, 0)),    # split sum carrying the epilogue
    (32, 1280, 2048, (1, 1, 8, 1, 5, 4, 0, 0)),
    (4, 640, 1024, (2, 2, 1, 8, 5, 3, 0, 0)),    # DOT with split
    (2, 640, 512, (2, 2, 2, 4, 4, 1, 0, 0)),     # DOT unsplit: second kernel
    (8, 640, 384, (1, 1, 5, 1, 5, 1, 0, 0)),     # MFMA unsplit: second kernel
    (16, 640, 1024, (3, 2, 1, 8, 6, 1, 0, 0)),   # row range unsplit: second kernel
]


@pytest.mark.parametrize("m,inter,k,cfg", FUSED_CASES)
def test_fused_every_configuration_kind(fp8bs, m, inter, k, cfg):
    from fp8_block_scaled_fp8bs_amd import GemmConfig
    c = GemmConfig(*cfg)
    announce("gemm_swiglu", "m", m, "n", 2 * inter, "k", k, "cfg", c)
    pr = _random_problem(fp8bs, m, 2 * inter, k, 1000 + m + inter + k)
    check_fused(fp8bs, pr, m, c, pr.ref(m))


@pytest.fixture(scope="module")
def mlp_up(fp8bs):
    wl = WORKLOADS["mlp_up"]
    announce("full-size up/gate weight", wl.n, wl.k)
    x_bits = act_bf16(wl.x_seed, wl.col_seed, 32, wl.k, wl.n_outlier, wl.outlier_factor)
    pr = Problem(fp8bs, wl.weight(), x_bits)
    torch.cuda.synchronize()
    return pr


@pytest.mark.parametrize("m", [1, 2, 4, 8, 16, 32])
def test_fused_mlp_up_full_size_every_m(fp8bs, mlp_up, m):
    """The 5120 -> 34816 up/gate projection (inter 17408) with its seeded
    weights and activations, in the configuration the library picks (the
    one the bench times)."""
    cfg = fp8bs.swiglu_select_config(m, mlp_up.w_bits.shape[0], mlp_up.w_bits.shape[1])
    announce("gemm_swiglu full mlp_up", "m", m, "cfg", cfg)
    ref = mlp_up.ref(m)
    same = check_fused(fp8bs, mlp_up, m, None, ref)
    announce("codes equal to the oracle chain", round(same, 5))
    if cfg.split_k == 1:
        # the epilogue inside the GEMM, same configuration otherwise
        inside = dataclasses.replace(cfg, epilogue=fp8bs.EPILOGUE_IN_GEMM)
        if cfg.path == fp8bs.PATH_DOT:
            inside = fp8bs.GemmConfig(3, 4, 1, 8, 4, epilogue=fp8bs.EPILOGUE_IN_GEMM)
        announce("gemm_swiglu full mlp_up in-GEMM epilogue", inside)
        check_fused(fp8bs, mlp_up, m, inside, ref)


def test_fused_zero_k_and_empty(fp8bs):
    """k = 0: y = 0 and h = silu(0) * 0 = 0, every scale 0; m = 0 is a no-op."""
    m, n = 4, 512
    x = torch.empty((m, 0), dtype=torch.bfloat16, device="cuda")
    wq = torch.empty((n, 0), dtype=torch.uint8, device="cuda")
    ws = torch.empty((n // 128, 0), dtype=torch.float32, device="cuda")
    y = torch.full((m, n), 7.0, dtype=torch.bfloat16, device="cuda")
    hq = torch.full((m, n // 2), 0x55, dtype=torch.uint8, device="cuda")
    hs = torch.full((m, n // 256), 3.0, dtype=torch.float32, device="cuda")
    fp8bs.gemm_swiglu(x, wq, ws, out=y, h=(hq, hs))
    torch.cuda.synchronize()
    assert not host_bits(y).any() and not hq.cpu().numpy().any() and not hs.cpu().numpy().any()
    x0 = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    pr = _random_problem(fp8bs, 1, 512, 256, 77)
    y0, hq0, hs0 = fp8bs.gemm_swiglu(x0, pr.wq, pr.ws)
    assert y0.shape == (0, 512) and hq0.shape == (0, 256)


def test_fused_workspace_reuse_and_graph_replay(fp8bs):
    """Arrival counters carry a per-launch epoch: one workspace serves
    consecutive calls of different shapes, a last-arriver GEMM in between
    (which leaves its own counters there), and replays of a captured graph,
    each replay interleaved with eager work and checked against the eager
    result."""
    from fp8_block_scaled_fp8bs_amd import GemmConfig
    pa = _random_problem(fp8bs, 8, 1280, 1024, 501)
    pb = _random_problem(fp8bs, 3, 1280, 512, 502)
    work = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    ina = GemmConfig(3, 4, 1, 8, 4, epilogue=1)    # in-GEMM epilogue: arrival counters
    inb = GemmConfig(1, 1, 2, 4, 5, epilogue=1)
    ya, hqa, hsa = fp8bs.gemm_swiglu_ex(ina, pa.wq, pa.ws, x=pa.x, workspace=work)
    yb, hqb, hsb = fp8bs.gemm_swiglu_ex(inb, pb.wq, pb.ws, x=pb.x, workspace=work)
    la = GemmConfig(1, 1, 1, 4, 5, split_k=4, reduce=1)
    fp8bs.gemm_ex(la, pa.wq, pa.ws, x=pa.x, workspace=work)
    ya2, hqa2, hsa2 = fp8bs.gemm_swiglu_ex(ina, pa.wq, pa.ws, x=pa.x, workspace=work)
    torch.cuda.synchronize()
    assert torch.equal(hqa, hqa2) and torch.equal(hsa, hsa2) and torch.equal(ya, ya2)
    blocks, _ = check_epilogue_exact(host_bits(yb), *_host(hqb, hsb))
    assert blocks == 3 * 5
    # graph capture of the fused call (its counters are never cleared by a fill)
    out_y = torch.empty_like(ya)
    out_h = (torch.empty_like(hqa), torch.empty_like(hsa))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fp8bs.gemm_swiglu_ex(ina, pa.wq, pa.ws, x=pa.x, out=out_y, h=out_h, workspace=work,
                             stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp8bs.gemm_swiglu_ex(ina, pa.wq, pa.ws, x=pa.x, out=out_y, h=out_h, workspace=work)
    for rep in range(4):
        out_h[0].fill_(0)
        out_h[1].fill_(-1.0)
        fp8bs.gemm_swiglu_ex(inb, pb.wq, pb.ws, x=pb.x, workspace=work)   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_h[0], hqa) and torch.equal(out_h[1], hsa), f"replay {rep}"
        assert torch.equal(out_y, ya), f"replay {rep}"


def test_fused_run_to_run_identity(fp8bs, mlp_up):
    x = mlp_up.x[:8].contiguous()
    first = fp8bs.gemm_swiglu(x, mlp_up.wq, mlp_up.ws)
    for _ in range(5):
        again = fp8bs.gemm_swiglu(x, mlp_up.wq, mlp_up.ws)
        torch.cuda.synchronize()
        for a, b in zip(first, again):
            assert torch.equal(a, b)
