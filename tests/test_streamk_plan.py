"""Host-side checks of the stream-K work partition, through the C ABI
(fp8bs_streamk_plan_check runs the partition code the kernel runs, on the
CPU): every (16-row tile, K block) unit is computed by exactly one
workgroup, each workgroup stays inside one K chunk, and the pieces of every
tile that is cut between workgroups are listed in K order in distinct
workspace slots, which is the order the last arriving workgroup adds them
in. Also the configuration rules of the path."""
import ctypes

import pytest

OK, UNSUPPORTED = 0, 1


@pytest.fixture(scope="module")
def fp8bs():
    import os
    import fp8_block_scaled_fp8bs_amd as m
    if not os.path.exists(m.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    m.load()
    return m


# (n, k, split): the decode shapes of the workloads, ragged K, uneven
# stream-K runs, whole-cell plans with several K chunks
VALID = [(5120, 5120, 1), (5120, 5120, 4), (5120, 5120, 8), (5120, 17408, 1), (5120, 17408, 4),
         (5120, 17408, 8), (34816, 5120, 1), (34816, 5120, 2), (34816, 5120, 4),
         (248320, 5120, 1), (248320, 5120, 8), (5120, 1024, 1), (5120, 1024, 4),
         (5120, 1664, 1), (4096, 1024, 2), (34816, 256, 1), (16384, 640, 1),
         (6144, 2944, 1), (4096, 128, 1)]


@pytest.mark.parametrize("n,k,split", VALID)
def test_plan_covers_every_unit_once(fp8bs, n, k, split):
    assert fp8bs.streamk_plan_check(n, k, split, 256) == OK


@pytest.mark.parametrize("n,k", [(5120, 5120), (34816, 5120), (248320, 5120), (5120, 17408),
                                 (4096, 1024), (6144, 2944), (4224, 256)])
def test_whole_tile_plan(fp8bs, n, k):
    """Whole-tile partition: every unit once, no tile cut (one piece each),
    tile counts per workgroup differing by at most one; only one K chunk."""
    assert fp8bs.streamk_plan_check(n, k, 1, 256, whole=True) == OK
    assert fp8bs.streamk_plan_check(n, k, 2, 256, whole=True) == UNSUPPORTED
    assert fp8bs.streamk_plan_check(n, k, 1, n // 16 + 1, whole=True) == UNSUPPORTED


@pytest.mark.parametrize("workgroups", [1, 7, 64, 255, 300])
def test_plan_other_workgroup_counts(fp8bs, workgroups):
    """The partition arithmetic does not assume 256 workgroups."""
    for n, k in ((5120, 5120), (5120, 1664), (34816, 1024)):
        r = fp8bs.streamk_plan_check(n, k, 1, workgroups)
        assert r in (OK, UNSUPPORTED), (n, k, workgroups, r)
    assert fp8bs.streamk_plan_check(5120, 5120, 1, 64) == OK


@pytest.mark.parametrize("n,k,split", [
    (512, 1024, 1),      # fewer units than workgroups in the stream-K part
    (5120, 5120, 2),     # a stream-K part with split > 1
    (5120, 5120, 3),     # split does not divide the K blocks
    (5120, 5120, 0),
    (4608, 3200, 1),     # a cell cut into more pieces than the kernel adds
    (5120, 2048, 16),    # more chunks than pieces the kernel adds
    (248320, 5120, 4),   # a stream-K part with split > 1
])
def test_plan_rejected(fp8bs, n, k, split):
    assert fp8bs.streamk_plan_check(n, k, split, 256) == UNSUPPORTED


def test_streamk_config_rules(fp8bs):
    """Explicit stream-K configurations: the shape must have a supported
    plan, waves_n must be 1, m at most 32; the workspace holds the pieces and
    one counter per tile."""
    from fp8_block_scaled_fp8bs_amd import GemmConfig
    lib = fp8bs.load()
    P = 0x100000
    E_CFG, E_WS = 7, 4

    def ex(cfg, m=8, n=5120, k=5120, wbytes=1 << 24):
        c = cfg._c()
        return lib.fp8bs_gemm_ex(P, None, None, m, P, P, n, k, P, P, wbytes, ctypes.byref(c), None)
    SKP = fp8bs.PATH_MFMA_STREAMK
    assert ex(GemmConfig(SKP, 2, 1, 8, 7, split_k=3)) == E_CFG            # 3 does not divide 40
    assert ex(GemmConfig(SKP, 2, 3, 8, 7)) == E_CFG                       # waves_n: 1 or 2
    assert ex(GemmConfig(SKP, 2, 2, 8, 7, split_k=4)) == E_CFG            # whole tiles: one chunk
    assert fp8bs.config_workspace_bytes(GemmConfig(SKP, 2, 2, 8, 7), 8, 5120, 5120) == 0
    assert ex(GemmConfig(SKP, 2, 1, 8, 7), n=512, k=1024) == E_CFG        # too few units
    assert ex(GemmConfig(SKP, 2, 1, 8, 7, reduce=1)) == E_CFG
    assert ex(GemmConfig(SKP, 2, 1, 8, 5)) == E_CFG                       # not compiled
    assert ex(GemmConfig(SKP, 2, 1, 8, 7), wbytes=0) == E_WS
    need = fp8bs.config_workspace_bytes(GemmConfig(SKP, 2, 1, 8, 7), 8, 5120, 5120)
    assert need >= 256 * 4 * 1024 + 320 * 8
    assert ex(GemmConfig(SKP, 2, 1, 8, 7), wbytes=need - 16) == E_WS
    need32 = fp8bs.config_workspace_bytes(GemmConfig(SKP, 2, 1, 8, 7, split_k=4), 32, 5120, 5120)
    assert need32 >= (5 * 256 + 256 * 4) * 2048
    import torch
    if not torch.cuda.is_available():
        assert ex(GemmConfig(SKP, 2, 1, 8, 7), wbytes=need) == 5              # reaches the device check
