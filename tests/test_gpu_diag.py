"""GPU checks of the measurement kernels the benchmark relies on: the
streaming-read ceiling in every mode runs over ranges that end inside a
1 KB piece and a 16-byte load, one launch per call; the copy kernel copies
exactly the bytes given; the wall-clock timestamps advance; invalid modes are
rejected before any launch."""
import numpy as np
import pytest

from gpu_util import announce, need_gpu, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8bs():
    need_gpu()
    import fp8_block_scaled_fp8bs_amd as m
    m.load()
    return m


@pytest.mark.parametrize("depth", [0, 4, 8, 16])
@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (1040, 3), (26214400 + 48, 256),
                                           (5 * 1024 * 1024 + 16 * 7, 160)])
def test_stream_ceiling_modes_run(fp8bs, depth, nbytes, blocks):
    announce("diag stream", depth, nbytes, blocks)
    buf = torch.zeros(nbytes + 4096, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    before = fp8bs.launch_count("diag")
    fp8bs.diag_stream(buf, sink, blocks=blocks, depth=depth, nbytes=nbytes)
    torch.cuda.synchronize()
    assert fp8bs.launch_count("diag") == before + 1
    assert int(sink.abs().sum()) == 0


def test_stream_ceiling_rejects_bad_mode(fp8bs):
    from fp8_block_scaled_fp8bs_amd import Fp8bsError
    buf = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    before = fp8bs.launch_count("diag")
    for depth, nbytes, blocks in ((3, 4096, 4), (0, 4008, 4), (0, 4096, 0)):
        with pytest.raises(Fp8bsError):
            fp8bs.diag_stream(buf, sink, blocks=blocks, depth=depth, nbytes=nbytes)
    assert fp8bs.launch_count("diag") == before


def test_copy_and_timestamps(fp8bs):
    rng = np.random.default_rng(91)
    src_h = rng.integers(0, 256, size=3 * 1024 * 1024 + 48, dtype=np.uint8)
    src = torch.from_numpy(src_h).cuda()
    dst = torch.zeros_like(src)
    ts = torch.zeros(2, dtype=torch.int64, device="cuda")
    fp8bs.diag_timestamp(ts[0:1])
    fp8bs.diag_copy(src, dst)
    fp8bs.diag_timestamp(ts[1:2])
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy(), src_h)
    t0, t1 = (int(v) for v in ts.cpu())
    assert t1 > t0 > 0
