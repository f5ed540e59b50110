"""C-ABI checks that need no GPU: the library loads, exports every function
include/fp8bs.h declares, binds to the HIP runtime torch loaded, and rejects
bad arguments before any HIP call (argument checks precede the device
check, so on a machine without a GPU a valid call reports ERR_DEVICE)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8bs.h")

OK, E_NULL, E_SHAPE, E_ALIGN, E_WS, E_DEV, E_LAUNCH, E_CFG = range(8)


@pytest.fixture(scope="module")
def lib():
    import fp8_block_scaled_fp8bs_amd as fp8bs
    if not os.path.exists(fp8bs.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    return fp8bs.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8bs_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("fp8bs_quantize_weight", "fp8bs_quantize_act", "fp8bs_gemm"):
        assert required in names


def test_library_exports_every_declared_function(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", lib._name], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing


def test_hip_imports_exist_in_torch_runtime(lib):
    """Every HIP runtime symbol the library imports is exported by the
    runtime copy that torch ships (the one it binds to at load time)."""
    import torch
    torch_hip = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
    if not os.path.exists(torch_hip):
        pytest.skip("torch does not bundle its own HIP runtime")
    need = subprocess.run(["nm", "-D", "--undefined-only", lib._name], capture_output=True,
                          text=True, check=True).stdout
    have = subprocess.run(["nm", "-D", "--defined-only", torch_hip], capture_output=True,
                          text=True, check=True).stdout
    have_names = {l.split()[-1].split("@")[0] for l in have.splitlines() if l.strip()}
    need_names = [l.split()[-1].split("@")[0] for l in need.splitlines()
                  if "hip" in l.lower() and l.strip()]
    assert need_names and all(n in have_names for n in need_names), need_names


def test_single_hip_runtime_mapped(lib):
    import fp8_block_scaled_fp8bs_amd as fp8bs
    maps = fp8bs.hip_runtime_mappings()
    assert len(maps["libfp8bs"]) == 1
    assert len(maps["libamdhip64"]) == 1, maps


def test_status_strings(lib):
    for s in range(8):
        assert lib.fp8bs_status_string(s).decode().startswith("FP8BS_")
    assert b"gfx950" in lib.fp8bs_build_info()


P = 0x100000  # a fake, 256-byte aligned "device" pointer: never dereferenced


def gemm(lib, x=P, m=8, w=P, ws=P, n=512, k=1024, y=P, work=None, wbytes=0):
    return lib.fp8bs_gemm(x, m, w, ws, n, k, y, work, wbytes, None)


def test_gemm_argument_errors_before_any_launch(lib):
    assert gemm(lib, n=500) == E_SHAPE
    assert gemm(lib, k=1000) == E_SHAPE
    assert gemm(lib, m=(1 << 20) + 1) == E_SHAPE
    assert gemm(lib, m=33) == E_WS       # prefill sizes cast X into the workspace first
    assert gemm(lib, m=-1) == E_SHAPE
    assert gemm(lib, x=None) == E_NULL
    assert gemm(lib, w=None) == E_NULL
    assert gemm(lib, ws=None) == E_NULL
    assert gemm(lib, y=None) == E_NULL
    assert gemm(lib, x=P + 2) == E_ALIGN
    assert gemm(lib, w=P + 8) == E_ALIGN
    assert gemm(lib, ws=P + 2) == E_ALIGN
    assert gemm(lib, y=P + 4) == E_ALIGN
    # empty extents are no-ops and touch nothing
    assert gemm(lib, m=0, x=None, y=None) == OK
    assert gemm(lib, n=0, w=None, ws=None) == OK
    # a valid call gets as far as the device check (no GPU here)
    import torch
    if not torch.cuda.is_available():
        assert gemm(lib, work=P, wbytes=1 << 24) == E_DEV


def test_gemm_check_order(lib):
    """Every GEMM entry point checks shape, then NULL pointers, then
    alignment, then the configuration, then the workspace, then the device:
    with several faults in one call the earliest check decides."""
    big_n = 1 << 31                       # n / 128 = 2^24: column indices overflow 32 bits
    # a bad shape wins over NULL and misaligned pointers
    assert gemm(lib, x=None, n=500) == E_SHAPE
    assert gemm(lib, x=None, y=None, w=None, k=1000) == E_SHAPE
    assert gemm(lib, x=P + 2, m=-1) == E_SHAPE
    assert gemm(lib, n=big_n) == E_SHAPE
    assert gemm(lib, x=None, n=big_n) == E_SHAPE
    assert gemm(lib, m=33, k=1 << 24) == E_SHAPE          # prefill offsets need k < 2^24
    assert lib.fp8bs_gemm_q(None, None, 8, P, P, 500, 1024, P, None, 0, None) == E_SHAPE
    assert lib.fp8bs_gemm_tiles(None, 8, P, P, big_n, 1024, P, None, 0, None) == E_SHAPE
    assert lib.fp8bs_gemm_q_tiles(None, None, 8, P, P, 512, 1000, P, None, 0, None) == E_SHAPE
    assert lib.fp8bs_gemm_ex(None, None, None, 8, P, P, 500, 1024, P, None, 0, None, None) == E_SHAPE
    assert lib.fp8bs_gemm_swiglu(None, 8, P, P, 640, 1024, P, P, P, None, 0, None) == E_SHAPE
    assert lib.fp8bs_gemm_swiglu_ex(None, None, None, 8, P, P, 640, 1024, P, P, P, None, 0,
                                    None, None) == E_SHAPE
    assert lib.fp8bs_pack_weight(None, big_n, 128, None, None) == E_SHAPE
    # the largest n the kernels index passes the shape check
    assert gemm(lib, x=None, n=big_n - 128) == E_NULL
    # NULL wins over misalignment and a missing workspace
    assert gemm(lib, x=None, w=P + 8, n=5120, k=17408) == E_NULL
    assert lib.fp8bs_gemm_q(P, None, 8, P + 8, P, 512, 1024, P, None, 0, None) == E_NULL
    # misalignment wins over a missing workspace
    assert gemm(lib, y=P + 4, n=5120, k=17408) == E_ALIGN
    # the configuration is checked before the workspace
    import fp8_block_scaled_fp8bs_amd as fp8bs
    c = fp8bs._Config(1, 3, 1, 1, 4, 2, 0, 0)   # 3 tiles per wave is not compiled
    assert lib.fp8bs_gemm_ex(P, None, None, 8, P, P, 512, 1024, P, None, 0, ctypes.byref(c),
                             None) == E_CFG


def test_gemm_workspace_checked(lib):
    import fp8_block_scaled_fp8bs_amd as fp8bs
    cfg = fp8bs.select_config(8, 5120, 17408)
    need = fp8bs.workspace_bytes(8, 5120, 17408)
    assert cfg.split_k > 1 and need >= cfg.split_k * 8 * 5120 * 4
    assert gemm(lib, n=5120, k=17408) == E_WS
    assert gemm(lib, n=5120, k=17408, work=P, wbytes=need - 16) == E_WS
    assert gemm(lib, n=5120, k=17408, work=P + 4, wbytes=need) == E_ALIGN


def test_quantizer_argument_errors(lib):
    assert lib.fp8bs_quantize_weight(P, 100, 128, P, P, None) == E_SHAPE
    assert lib.fp8bs_quantize_weight(P, 128, 130, P, P, None) == E_SHAPE
    assert lib.fp8bs_quantize_weight(None, 128, 128, P, P, None) == E_NULL
    assert lib.fp8bs_quantize_weight(P + 1, 128, 128, P, P, None) == E_ALIGN
    assert lib.fp8bs_quantize_weight(None, 0, 128, None, None, None) == OK
    assert lib.fp8bs_quantize_act(P, 3, 100, P, P, None) == E_SHAPE
    assert lib.fp8bs_quantize_act(P, 3, 128, None, P, None) == E_NULL
    assert lib.fp8bs_quantize_act(P, 3, 128, P, P + 1, None) == E_ALIGN
    assert lib.fp8bs_quantize_act(None, 0, 128, None, None, None) == OK
    assert lib.fp8bs_encode_e4m3(P, 4, P, 3, None) == E_SHAPE
    assert lib.fp8bs_encode_e4m3(P, 0, P, 0, None) == OK


def test_explicit_config_validation(lib):
    import fp8_block_scaled_fp8bs_amd as fp8bs
    from fp8_block_scaled_fp8bs_amd import GemmConfig
    c = fp8bs._Config(1, 3, 1, 1, 4, 1, 0, 0)  # 3 tiles per wave is not compiled
    r = lib.fp8bs_gemm_ex(P, None, None, 8, P, P, 512, 1024, P, None, 0, ctypes.byref(c), None)
    assert r == E_CFG
    c = GemmConfig(1, 1, 1, 4, 5, split_k=3, reduce=7)._c()  # unknown reduce mode
    r = lib.fp8bs_gemm_ex(P, None, None, 8, P, P, 512, 1024, P, P, 1 << 20, ctypes.byref(c), None)
    assert r == E_CFG
    c = GemmConfig(1, 1, 4, 1, 4, split_k=9)._c()  # more splits than K blocks (8)
    r = lib.fp8bs_gemm_ex(P, None, None, 8, P, P, 512, 1024, P, P, 1 << 20, ctypes.byref(c), None)
    assert r == E_CFG
    c = GemmConfig(2, 2, 1, 8, 5)._c()  # DOT path takes at most 4 rows
    r = lib.fp8bs_gemm_ex(P, None, None, 8, P, P, 512, 1024, P, None, 0, ctypes.byref(c), None)
    assert r == E_CFG
    assert lib.fp8bs_gemm_ex(P, None, None, 8, P, P, 512, 1024, P, None, 0, None, None) == E_NULL


def test_config_table_is_a_pure_function_of_shape(lib):
    import fp8_block_scaled_fp8bs_amd as fp8bs
    shapes = [(m, n, k) for m in (1, 2, 3, 8, 16, 17, 32)
              for (n, k) in ((512, 1024), (5120, 5120), (34816, 5120), (5120, 17408),
                             (248320, 5120), (31104, 5120), (128, 128))]
    for s in shapes:
        a, b = fp8bs.select_config(*s), fp8bs.select_config(*s)
        assert a == b
        assert 1 <= a.split_k <= s[2] // 128
        if a.path not in (3, 4):  # the row-range paths split n over the compute units
            rows = (8 if a.path == fp8bs.PATH_DOT else 16) * a.tiles_n * a.waves_n
            assert s[1] % rows == 0
        if a.path == fp8bs.PATH_DOT:
            assert s[0] <= 4
    with pytest.raises(fp8bs.Fp8bsError):
        fp8bs.select_config(8, 100, 128)


def swiglu(lib, x=P, m=8, w=P, ws=P, n=1024, k=1024, y=P, hq=P, hs=P, work=P, wbytes=1 << 20):
    return lib.fp8bs_gemm_swiglu(x, m, w, ws, n, k, y, hq, hs, work, wbytes, None)


def test_swiglu_argument_errors_before_any_launch(lib):
    """The fused up/gate + SwiGLU call and the standalone epilogue check
    their arguments in the documented order before touching the device."""
    assert swiglu(lib, n=640) == E_SHAPE        # n/2 not a multiple of 128
    assert swiglu(lib, m=(1 << 20) + 1) == E_SHAPE
    assert swiglu(lib, k=1000) == E_SHAPE
    assert swiglu(lib, x=None) == E_NULL
    assert swiglu(lib, hq=None) == E_NULL
    assert swiglu(lib, hs=None) == E_NULL
    assert swiglu(lib, y=None) == E_NULL
    assert swiglu(lib, hq=P + 8) == E_ALIGN
    assert swiglu(lib, hs=P + 2) == E_ALIGN
    assert swiglu(lib, k=17408, work=None, wbytes=0) == E_WS   # split-K partials
    assert swiglu(lib, m=0, x=None, y=None, hq=None, hs=None) == OK
    assert lib.fp8bs_swiglu_quant(P, 8, 100, P, P, None) == E_SHAPE
    assert lib.fp8bs_swiglu_quant(None, 8, 128, P, P, None) == E_NULL
    assert lib.fp8bs_swiglu_quant(P, 8, 128, P + 4, P, None) == E_ALIGN
    assert lib.fp8bs_swiglu_quant(None, 0, 128, None, None, None) == OK
    import torch
    if not torch.cuda.is_available():
        assert swiglu(lib) == E_DEV
        assert lib.fp8bs_swiglu_quant(P, 8, 128, P, P, None) == E_DEV


def test_swiglu_config_rules(lib):
    """Configurations that cannot carry the epilogue are refused; the
    automatic choice is the plain GEMM's, with the separate epilogue."""
    import fp8_block_scaled_fp8bs_amd as fp8bs
    from fp8_block_scaled_fp8bs_amd import GemmConfig

    def ex(cfg, n=1024, k=1024, m=8):
        c = cfg._c()
        return lib.fp8bs_gemm_swiglu_ex(P, None, None, m, P, P, n, k, P, P, P, P, 1 << 24,
                                        ctypes.byref(c), None)
    IN = fp8bs.EPILOGUE_IN_GEMM
    assert ex(GemmConfig(2, 2, 1, 8, 5, epilogue=IN), m=2) == E_CFG          # DOT in the GEMM
    assert ex(GemmConfig(1, 1, 1, 4, 5, split_k=4, epilogue=IN)) == E_CFG    # split in the GEMM
    assert ex(GemmConfig(1, 1, 1, 4, 5, split_k=4, reduce=1)) == E_CFG       # last-arriver
    assert ex(GemmConfig(3, 2, 1, 8, 2, epilogue=IN)) == E_CFG               # rows shape not compiled
    assert ex(GemmConfig(1, 1, 1, 4, 5, epilogue=2)) == E_CFG                # unknown placement
    for m in (1, 2, 3, 8, 16, 32):
        for n, k in ((34816, 5120), (5120, 5120), (1024, 17408), (256, 128)):
            c = fp8bs.swiglu_select_config(m, n, k)
            assert c == fp8bs.select_config(m, n, k) and c.epilogue == fp8bs.EPILOGUE_SEPARATE
            need = fp8bs.swiglu_workspace_bytes(m, n, k)
            assert need == (c.split_k * m * n * 4 if c.split_k > 1 else 0)
            cin = GemmConfig(1, 1, 1, 4, 5, epilogue=IN)
            assert fp8bs.swiglu_workspace_bytes(m, n, k, cin) >= (n // 256) * 8
    with pytest.raises(fp8bs.Fp8bsError):
        fp8bs.swiglu_select_config(8, 384, 128)


def test_tile_layout_argument_errors(lib):
    """Weight rearrangement and the tile-layout GEMM calls check their
    arguments before any launch."""
    assert lib.fp8bs_pack_weight(P, 100, 128, P, None) == E_SHAPE
    assert lib.fp8bs_pack_weight(P, 128, 130, P, None) == E_SHAPE
    assert lib.fp8bs_pack_weight(None, 128, 128, P, None) == E_NULL
    assert lib.fp8bs_pack_weight(P, 128, 128, None, None) == E_NULL
    assert lib.fp8bs_pack_weight(P + 8, 128, 128, P, None) == E_ALIGN
    assert lib.fp8bs_pack_weight(P, 128, 128, P + 4, None) == E_ALIGN
    assert lib.fp8bs_pack_weight(None, 0, 128, None, None) == OK
    assert lib.fp8bs_pack_weight(P, 1 << 22, 1 << 21, P, None) == E_SHAPE  # grid past 2^31 - 1
    g = lib.fp8bs_gemm_tiles
    assert g(P, (1 << 20) + 1, P, P, 512, 1024, P, P, 1 << 20, None) == E_SHAPE
    assert g(P, 33, P, P, 512, 1024, P, None, 0, None) == E_WS  # prefill casts X into it
    assert g(P, 8, P, P, 500, 1024, P, P, 1 << 20, None) == E_SHAPE
    assert g(None, 8, P, P, 512, 1024, P, P, 1 << 20, None) == E_NULL
    assert g(P, 8, P + 8, P, 512, 1024, P, P, 1 << 20, None) == E_ALIGN
    assert lib.fp8bs_gemm_q_tiles(P, P, -1, P, P, 512, 1024, P, P, 1 << 20, None) == E_SHAPE
    assert lib.fp8bs_gemm_q_tiles(P, None, 8, P, P, 512, 1024, P, P, 1 << 20, None) == E_NULL
    import torch
    if not torch.cuda.is_available():
        assert lib.fp8bs_pack_weight(P, 128, 128, P, None) == E_DEV
        assert g(P, 8, P, P, 512, 1024, P, P, 1 << 20, None) == E_DEV


def test_tile_layout_config_rules(lib):
    """The tile-layout table picks a kernel with a tile-layout build for
    every decode m, as a pure function of the shape; the in-GEMM SwiGLU
    epilogue and prefill configurations reject the tile layout; the
    workspace query covers both layouts."""
    import fp8_block_scaled_fp8bs_amd as fp8bs
    from fp8_block_scaled_fp8bs_amd import GemmConfig
    for (n, k) in ((512, 1024), (5120, 5120), (34816, 5120), (5120, 17408), (248320, 5120),
                   (31104, 5120)):
        for m in range(1, 33):
            t = fp8bs.tiles_select_config(m, n, k)
            r = fp8bs.select_config(m, n, k)
            assert t.weight_layout == fp8bs.LAYOUT_TILES and r.weight_layout == fp8bs.LAYOUT_ROWS
            assert t.path in (fp8bs.PATH_MFMA, 3, 4, 6, fp8bs.PATH_MFMA_ROWS_DMA)
            assert t == fp8bs.tiles_select_config(m, n, k)
            assert 1 <= t.split_k <= k // 128
            if t.path == fp8bs.PATH_MFMA:
                assert n % (16 * t.tiles_n * t.waves_n) == 0
            assert fp8bs.workspace_bytes(m, n, k) >= fp8bs.config_workspace_bytes(t, m, n, k)
    t = fp8bs.tiles_select_config(64, 5120, 5120)
    assert t.path == fp8bs.PATH_PREFILL and t.weight_layout == fp8bs.LAYOUT_TILES
    assert t == fp8bs.tiles_select_config(64, 5120, 5120)
    c = GemmConfig(1, 1, 1, 4, 5, epilogue=1, weight_layout=fp8bs.LAYOUT_TILES)._c()
    r = lib.fp8bs_gemm_swiglu_ex(P, None, None, 8, P, P, 1024, 1024, P, P, P, P, 1 << 20,
                                 ctypes.byref(c), None)
    assert r == E_CFG  # the epilogue inside the GEMM has no tile-layout build
    assert lib.fp8bs_gemm_swiglu_tiles(P, 65536, P, P, 1024, 1024, P, P, P, P, 1 << 20, None) == E_SHAPE
    assert lib.fp8bs_gemm_swiglu_tiles(P, 8, P, P, 1152, 1024, P, P, P, P, 1 << 20, None) == E_SHAPE
    assert lib.fp8bs_gemm_swiglu_tiles(None, 8, P, P, 1024, 1024, P, P, P, P, 1 << 20, None) == E_NULL
    import torch
    if not torch.cuda.is_available():
        c = GemmConfig(1, 1, 1, 4, 5, weight_layout=fp8bs.LAYOUT_TILES)._c()
        r = lib.fp8bs_gemm_swiglu_ex(P, None, None, 8, P, P, 1024, 1024, P, P, P, P, 1 << 20,
                                     ctypes.byref(c), None)
        assert r == E_DEV
        assert lib.fp8bs_gemm_swiglu_tiles(P, 8, P, P, 1024, 1024, P, P, P, P, 1 << 20, None) == E_DEV
    c = GemmConfig(5, 2, 2, 2, 2, weight_layout=fp8bs.LAYOUT_TILES)._c()  # no early-refill tile build
    r = lib.fp8bs_gemm_ex(P, None, None, 64, P, P, 512, 1024, P, P, 1 << 24, ctypes.byref(c), None)
    assert r == E_CFG
    # the prefill kernel's 32-bit offsets: k >= 2^24 is a shape error, in either layout
    for layout in (fp8bs.LAYOUT_ROWS, fp8bs.LAYOUT_TILES):
        c = GemmConfig(5, 1, 2, 2, 2, weight_layout=layout)._c()
        r = lib.fp8bs_gemm_ex(P, None, None, 64, P, P, 512, 1 << 24, P, P, 1 << 40,
                              ctypes.byref(c), None)
        assert r == E_SHAPE
    c = GemmConfig(1, 1, 1, 4, 5, weight_layout=2)._c()
    r = lib.fp8bs_gemm_ex(P, None, None, 8, P, P, 512, 1024, P, None, 0, ctypes.byref(c), None)
    assert r == E_CFG
    c = GemmConfig(2, 2, 2, 4, 4, weight_layout=fp8bs.LAYOUT_TILES)._c()  # no DOT tile build
    r = lib.fp8bs_gemm_ex(P, None, None, 1, P, P, 512, 1024, P, None, 0, ctypes.byref(c), None)
    assert r == E_CFG


def test_prefill_wide_configs_checked_before_any_launch(lib):
    """The wide prefill kernel's 1-D schedule (tiles_n 4) takes no K split,
    and it launches one workgroup per whole or half 256 x 256 tile on a
    one-dimensional grid, so a shape with more than 2^31 - 1 such
    workgroups is a configuration error for it; the table picks the grid
    schedule (tiles_n 3) there instead. All of this is decided before any
    device call."""
    import fp8_block_scaled_fp8bs_amd as fp8bs
    c = fp8bs._Config(5, 4, 2, 4, 2, 2, 0, 0, 0)             # 1-D schedule with a K split
    assert lib.fp8bs_gemm_ex(None, P, P, 4096, P, P, 5120, 5120, P, None, 0, ctypes.byref(c),
                             None) == E_CFG
    m, n = 1 << 20, (1 << 31) - 128                           # 4096 x 8,388,608 whole tiles
    c = fp8bs._Config(5, 4, 2, 4, 2, 1, 0, 0, 0)
    assert lib.fp8bs_gemm_ex(None, P, P, m, P, P, n, 128, P, None, 0, ctypes.byref(c),
                             None) == E_CFG
    cfg = fp8bs.select_config(m, n, 128)
    assert (cfg.path, cfg.tiles_n, cfg.split_k) == (fp8bs.PATH_PREFILL, 3, 1)
    cfg = fp8bs.select_config(8192, 5120, 5120)
    assert (cfg.path, cfg.tiles_n, cfg.waves_n, cfg.waves_k, cfg.split_k) == (fp8bs.PATH_PREFILL, 4, 2, 4, 1)
    cfg = fp8bs.select_config(1024, 4096, 4096)               # 64 tiles: the 128 x 128 kernel
    assert (cfg.path, cfg.tiles_n) == (fp8bs.PATH_PREFILL, 1)


def test_vocab_rows_dma_table(lib):
    """The vocabulary layer at m = 9-16 on tile-layout weights takes the
    row-range kernel with the weight stream through LDS (3 stages); at
    m = 1-8, on row-major weights and where the LDS cannot hold the
    activations beside the ring, it does not."""
    import fp8_block_scaled_fp8bs_amd as fp8bs
    for m in (9, 12, 16):
        c = fp8bs.tiles_select_config(m, 248320, 5120)
        assert (c.path, c.waves_k, c.depth, c.split_k) == (fp8bs.PATH_MFMA_ROWS_DMA, 8, 3, 1), (m, c)
        assert fp8bs.select_config(m, 248320, 5120).path != fp8bs.PATH_MFMA_ROWS_DMA
    for m in (1, 4, 8, 17, 32):
        assert fp8bs.tiles_select_config(m, 248320, 5120).path != fp8bs.PATH_MFMA_ROWS_DMA
    # 16 rows of a K = 8192 range: 118 KB of staged activations leave no room for the ring
    assert fp8bs.tiles_select_config(16, 131072, 8192).path != fp8bs.PATH_MFMA_ROWS_DMA


def test_prefill_narrow_tiles_table_and_limits(lib):
    """Narrow (64 JM) x 160 tiles: the table takes them where n is a multiple
    of 640 and they make one round of 192 to 256 workgroups (256-row tiles
    first); elsewhere it keeps the wide or the 128 x 128 kernel. A narrow
    configuration on n not a multiple of 160, or with a K split, is a
    configuration error before any device call."""
    import fp8_block_scaled_fp8bs_amd as fp8bs
    want = {(2048, 5120, 5120): (5, 4), (2048, 5120, 17408): (5, 4), (1024, 5120, 5120): (5, 3),
            (1536, 5120, 5120): (5, 4), (4096, 5120, 5120): (4, 4), (8192, 5120, 17408): (4, 4),
            (2048, 34816, 5120): (4, 4), (512, 5120, 5120): (1, 2),
            (256, 34816, 5120): (4, 4), (128, 34816, 5120): (1, 2)}
    for (m, n, k), (tn, wk) in want.items():
        for sel in (fp8bs.select_config, fp8bs.tiles_select_config):
            cfg = sel(m, n, k)
            assert cfg.path == fp8bs.PATH_PREFILL and cfg.split_k == 1 or tn == 1, (m, n, k, cfg)
            assert (cfg.tiles_n, cfg.waves_k) == (tn, wk), (m, n, k, cfg)
    # deep K (k >= 12288, m > 64): the wide kernel's grid schedule with K
    # split so that tiles x split fill one round of 256 workgroups
    deep = {(1024, 5120, 17408): (3, 4, 3), (512, 5120, 17408): (3, 4, 6),
            (128, 5120, 17408): (3, 4, 12), (64, 5120, 17408): (1, 2, 7)}
    for (m, n, k), want_cfg in deep.items():
        for sel in (fp8bs.select_config, fp8bs.tiles_select_config):
            cfg = sel(m, n, k)
            assert (cfg.tiles_n, cfg.waves_k, cfg.split_k) == want_cfg, (m, n, k, cfg)
    for n, split in ((5248, 1), (5120, 2)):
        c = fp8bs._Config(5, 5, 2, 4, 2, split, 0, 0, 0)
        assert lib.fp8bs_gemm_ex(None, P, P, 2048, P, P, n, 5120, P, None, 0, ctypes.byref(c),
                                 None) == E_CFG


def test_one_round_wide_n_class(lib):
    """Shapes whose 128-row weight blocks number 200 to 256 (one GPU's 8-way
    column share of the vocabulary layer, 31104 x 5120) take the grid kernel
    with 8 waves along N, one workgroup per block row, where it fits (K split
    in two at m = 32 on tile-layout weights); wider shapes (MLP up, 272 block
    rows) keep the wide-N choices."""
    import fp8_block_scaled_fp8bs_amd as fp8bs
    for m in (5, 8, 16, 24):
        for t in (fp8bs.tiles_select_config(m, 31104, 5120), fp8bs.select_config(m, 31104, 5120)):
            assert (t.path, t.tiles_n, t.waves_n, t.waves_k, t.depth, t.split_k) == \
                (fp8bs.PATH_MFMA, 1, 8, 1, 5, 1), (m, t)
    t = fp8bs.tiles_select_config(32, 31104, 5120)
    assert (t.path, t.waves_n, t.waves_k, t.split_k) == (fp8bs.PATH_MFMA, 8, 1, 2), t
    t = fp8bs.tiles_select_config(4, 31104, 5120)
    assert (t.path, t.waves_n, t.waves_k, t.split_k) == (fp8bs.PATH_MFMA, 2, 4, 1), t
    assert fp8bs.select_config(32, 31104, 5120).path != fp8bs.PATH_MFMA
    for m in (8, 16):
        assert fp8bs.tiles_select_config(m, 34816, 5120).path == 3
        assert fp8bs.tiles_select_config(m, 32896, 5120).path == 3  # 257 block rows


def test_deep_k_small_m_tiles_unsplit(lib):
    """On tile-layout weights the MLP-down shape (17408 -> 5120) at m = 1-2
    takes the grid kernel without a K split (no reduce kernel); from m = 3 K
    stays split."""
    import fp8_block_scaled_fp8bs_amd as fp8bs
    for m in (1, 2):
        t = fp8bs.tiles_select_config(m, 5120, 17408)
        assert (t.path, t.waves_n, t.waves_k, t.split_k) == (fp8bs.PATH_MFMA, 2, 4, 1), (m, t)
    assert fp8bs.tiles_select_config(3, 5120, 17408).split_k > 1
