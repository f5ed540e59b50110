"""The entry point that allocates nothing (fp8bs_gemm_noalloc), called through
the C ABI: on two calls in a row (the second with a smaller input) its
output equals fp8bs_gemm's with a caller workspace bit for bit (the same
configuration), on shapes whose kernels use the scratch (split-K partials
summed by a second kernel, the prefill path's cast activations) and on one
that needs none; and one result within tolerance of the oracle. A shape
whose configuration needs more scratch than the fixed maximum is rejected
before any launch."""
import ctypes

import numpy as np
import pytest

import oracle
from gpu_util import announce, dev_bf16, host_bits, need_gpu, torch
from workloads import WORKLOADS, act_bf16, bf16_from_f32

pytestmark = pytest.mark.gpu

TOL = dict(rel=2.0 ** -7, abs_rms=1e-3)


@pytest.fixture(scope="module")
def fp8bs():
    need_gpu()
    import fp8_block_scaled_fp8bs_amd as m
    m.load()
    return m


def _abi_noalloc(lib, x, wq, ws, y):
    m, k = x.shape
    n = wq.shape[0]
    stream = torch.cuda.current_stream().cuda_stream
    return lib.fp8bs_gemm_noalloc(ctypes.c_void_p(x.data_ptr()), m, ctypes.c_void_p(wq.data_ptr()),
                                  ctypes.c_void_p(ws.data_ptr()), n, k,
                                  ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(stream))


def _abi_gemm(lib, x, wq, ws, y, work):
    m, k = x.shape
    n = wq.shape[0]
    stream = torch.cuda.current_stream().cuda_stream
    return lib.fp8bs_gemm(ctypes.c_void_p(x.data_ptr()), m, ctypes.c_void_p(wq.data_ptr()),
                          ctypes.c_void_p(ws.data_ptr()), n, k, ctypes.c_void_p(y.data_ptr()),
                          ctypes.c_void_p(work.data_ptr()), work.numel(), ctypes.c_void_p(stream))


@pytest.mark.parametrize("name,m1,m2", [("mlp_down", 8, 3), ("square", 32, 16), ("square", 8, 1),
                                        ("tiny", 96, 40)])
def test_noalloc_matches_gemm_two_calls(fp8bs, name, m1, m2):
    lib = fp8bs.load()
    wl = WORKLOADS[name]
    announce("noalloc", name, m1, m2, fp8bs.select_config(m1, wl.n, wl.k),
             fp8bs.select_config(m2, wl.n, wl.k))
    w = dev_bf16(wl.weight())
    wq, ws = fp8bs.quantize_weight(w)
    x_bits = act_bf16(wl.x_seed, wl.col_seed, max(m1, m2), wl.k, wl.n_outlier, wl.outlier_factor)
    x = dev_bf16(x_bits)
    work = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    outs = []
    for m in (m1, m2):     # two calls in a row, the second smaller
        xm = x[:m].contiguous()
        y_na = torch.full((m, wl.n), 3.0, dtype=torch.bfloat16, device="cuda")
        y_ref = torch.empty((m, wl.n), dtype=torch.bfloat16, device="cuda")
        assert _abi_noalloc(lib, xm, wq, ws, y_na) == 0
        assert _abi_gemm(lib, xm, wq, ws, y_ref, work) == 0
        outs.append((m, y_na, y_ref))
    torch.cuda.synchronize()
    for m, y_na, y_ref in outs:
        assert np.array_equal(host_bits(y_na), host_bits(y_ref)), (name, m)
    # the smaller call against the oracle
    m, y_na, _ = outs[1]
    xq, xs = oracle.quantize_act_ref(x_bits[:m])
    wq_ref, ws_ref = oracle.quantize_weight_ref(wl.weight())
    rep = oracle.tolerance_report(host_bits(y_na), oracle.gemm_ref(xq, xs, wq_ref, ws_ref), **TOL)
    assert rep["finite"] and rep["n_bad"] == 0, rep


def test_noalloc_rejects_beyond_scratch(fp8bs):
    """A prefill call whose cast activations and split partials exceed the
    fixed scratch: FP8BS_ERR_WORKSPACE, and the output is untouched."""
    lib = fp8bs.load()
    assert lib.fp8bs_gemm_noalloc_max_scratch() == 8 << 20
    m, n, k = 2048, 5120, 5120
    need = fp8bs.workspace_bytes(m, n, k)
    assert need > 8 << 20
    x = torch.zeros((m, k), dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros((n, k), dtype=torch.uint8, device="cuda")
    ws = torch.ones((n // 128, k // 128), dtype=torch.float32, device="cuda")
    y = torch.full((m, n), 5.0, dtype=torch.bfloat16, device="cuda")
    assert _abi_noalloc(lib, x, wq, ws, y) == 4
    torch.cuda.synchronize()
    assert torch.all(y == 5.0)
