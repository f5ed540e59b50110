"""GPU parity of the quantizers and the E4M3 encoder against the CPU oracle:
bit-exact codes and scales."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
from gpu_util import announce, dev_bf16, dev_f32, host_bits, need_gpu, same_bits_f32, torch
from workloads import WORKLOADS, bf16_from_f32, f32_from_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8bs():
    need_gpu()
    import fp8_block_scaled_fp8bs_amd as m
    m.load()
    return m


def _encode_gpu(fp8bs, bits_lo, bits_hi, mode):
    b = torch.arange(bits_lo, bits_hi, dtype=torch.int64, device="cuda").to(torch.int32)
    return fp8bs.encode_e4m3(b.view(torch.float32), mode=mode).cpu().numpy()


@pytest.mark.parametrize("mode", [1, 2])
def test_encoder_exhaustive_positive_patterns(fp8bs, mode):
    """Every fp32 bit pattern in [+0, 464): the hardware conversion (mode 1)
    and the software encoder (mode 2) against the oracle's encoder."""
    top = 0x43E80000  # 464.0, the midpoint above 448
    chunk = 1 << 24
    ranges = [(lo, min(lo + chunk, top)) for lo in range(0, top, chunk)]
    announce("encoder exhaustive", "mode", mode, "chunks", len(ranges))
    from oracle_pool import encode_range
    with ThreadPoolExecutor(max_workers=12) as pool:
        for (lo, hi), want in zip(ranges, pool.map(encode_range, ranges)):
            got = _encode_gpu(fp8bs, lo, hi, mode)
            if not np.array_equal(got, want):
                bad = np.nonzero(got != want)[0][:8]
                pats = [hex(lo + int(i)) for i in bad]
                raise AssertionError(f"mode {mode}: mismatch at patterns {pats}: "
                                     f"got {[hex(got[i]) for i in bad]} want {[hex(want[i]) for i in bad]}")


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_encoder_negative_and_special_values(fp8bs, mode):
    rng = np.random.default_rng(21)
    bits = rng.integers(0x80000000, 0xC3E80000, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    specials = np.array([0x80000000, 0x00000000, 0x80000001, 0x00000001, 0x3A800000, 0xBA800000,
                         0x43E00000, 0xC3E00000, 0x43E7FFFF, 0xC3E7FFFF], dtype=np.uint32)
    v = np.concatenate([bits, specials]).view(np.float32)
    got = fp8bs.encode_e4m3(dev_f32(v), mode=mode).cpu().numpy()
    assert np.array_equal(got, oracle.e4m3_encode(v))


def test_software_encoder_saturates(fp8bs):
    v = np.array([464.0, 500.0, 1e30, 3.4e38, -464.0, -1e30], dtype=np.float32)
    got = fp8bs.encode_e4m3(dev_f32(v), mode=2).cpu().numpy()
    assert np.array_equal(got, oracle.e4m3_encode(v))


def _check_weight(fp8bs, w_bits):
    w = dev_bf16(w_bits)
    q, s = fp8bs.quantize_weight(w)
    qr, sr = oracle.quantize_weight_ref(w_bits)
    assert np.array_equal(q.cpu().numpy(), qr)
    assert same_bits_f32(s.cpu().numpy(), sr)


@pytest.mark.parametrize("name", ["tiny", "square", "mlp_up", "mlp_down"])
def test_quantize_weight_bit_exact(fp8bs, name):
    wl = WORKLOADS[name]
    announce("quantize_weight", name, wl.n, wl.k)
    _check_weight(fp8bs, wl.weight())


@pytest.mark.parametrize("name", ["tiny", "square", "mlp_up", "mlp_down", "vocab"])
def test_quantize_act_bit_exact(fp8bs, name):
    wl = WORKLOADS[name]
    x_bits = wl.act()
    announce("quantize_act", name, x_bits.shape)
    q, s = fp8bs.quantize_act(dev_bf16(x_bits))
    qr, sr = oracle.quantize_act_ref(x_bits)
    assert np.array_equal(q.cpu().numpy(), qr)
    assert same_bits_f32(s.cpu().numpy(), sr)


def _crafted_blocks():
    """1x128 blocks covering every (amax mantissa, x mantissa, exponent gap)
    combination at several binades, the slow-quotient range (tiny amax),
    bf16 subnormals, huge amax, signed zeros and all-zero blocks."""
    rows = []
    mant = np.arange(128, 256, dtype=np.float64) / 128.0  # 1.0 .. 1.9921875 (8 bits)
    for e_amax in (-100, -60, -59, -20, 0, 15, 60, 120, 127):
        for ma in mant:
            amax = ma * 2.0 ** e_amax
            xs = []
            for d in range(0, 25):
                for mx in mant:
                    x = mx * 2.0 ** (e_amax - d)
                    if x <= amax:
                        xs.append(x)
            xs = np.array(xs)
            xs[1::2] *= -1
            for i in range(0, len(xs), 127):
                blk = np.zeros(128)
                part = xs[i:i + 127]
                blk[0] = amax if i % 2 == 0 else -amax
                blk[1:1 + len(part)] = part
                rows.append(blk)
    # tiny amax: bf16 subnormals and just above
    for b in list(range(1, 128)) + [0x0080, 0x0100, 0x01FF]:
        blk = np.zeros(128)
        amax = float(f32_from_bf16(np.array([b], np.uint16))[0])
        blk[0] = amax
        blk[1:] = amax * np.linspace(-1, 1, 127)
        rows.append(blk)
    z = np.zeros(128)
    rows.append(z.copy())
    nz = np.zeros(128)
    nz[::3] = -0.0
    rows.append(nz)
    mixed = np.zeros(128)
    mixed[5] = 3.0
    mixed[7] = -0.0
    rows.append(mixed)
    x = np.array(rows, dtype=np.float32)
    return bf16_from_f32(x)


def test_quantize_act_crafted_blocks_bit_exact(fp8bs):
    x_bits = _crafted_blocks()
    # every value must be exactly representable in bf16 (the generator built them so)
    announce("quantize_act crafted", x_bits.shape)
    q, s = fp8bs.quantize_act(dev_bf16(x_bits))
    qr, sr = oracle.quantize_act_ref(x_bits)
    got = q.cpu().numpy()
    if not np.array_equal(got, qr):
        r, c = np.nonzero(got != qr)
        raise AssertionError(f"{len(r)} codes differ; first rows {r[:5]} cols {c[:5]} "
                             f"got {got[r[:5], c[:5]]} want {qr[r[:5], c[:5]]}")
    assert same_bits_f32(s.cpu().numpy(), sr)


def test_quantize_weight_crafted_blocks_bit_exact(fp8bs):
    """The same crafted rows, stacked into 128x128 weight blocks."""
    x = _crafted_blocks()
    r = (x.shape[0] // 128) * 128
    w = np.ascontiguousarray(x[:r].reshape(-1, 128, 128).transpose(1, 0, 2).reshape(128, -1))
    announce("quantize_weight crafted", w.shape)
    _check_weight(fp8bs, w)


@pytest.mark.parametrize("m,k", [(1, 128), (3, 384), (37, 1280), (4096, 256)])
def test_quantize_act_ragged_row_counts(fp8bs, m, k):
    rng = np.random.default_rng(m + k)
    x_bits = bf16_from_f32((rng.standard_normal((m, k)) * 3).astype(np.float32))
    q, s = fp8bs.quantize_act(dev_bf16(x_bits))
    qr, sr = oracle.quantize_act_ref(x_bits)
    assert np.array_equal(q.cpu().numpy(), qr) and same_bits_f32(s.cpu().numpy(), sr)


def test_quantize_weight_vocab_sampled_block_rows(fp8bs):
    """The 248,320 x 5,120 output-layer weight: quantize all of it on the GPU,
    check sampled 128-row block rows bit-exact (each regenerated alone)."""
    from workloads import weight_rows_bf16
    wl = WORKLOADS["vocab"]
    announce("quantize_weight vocab full", wl.n, wl.k)
    w = dev_bf16(wl.weight())
    q, s = fp8bs.quantize_weight(w)
    del w
    nbn = wl.n // 128
    for c in (0, 1, 777, nbn // 2, nbn - 1):
        rows = weight_rows_bf16(wl.w_seed, c, 128, wl.k)
        qr, sr = oracle.quantize_weight_ref(rows)
        assert np.array_equal(q[c * 128:(c + 1) * 128].cpu().numpy(), qr), c
        assert same_bits_f32(s[c].cpu().numpy(), sr[0]), c
