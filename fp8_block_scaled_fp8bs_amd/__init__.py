"""Python binding of libfp8bs: the FP8 (E4M3) 128x128 block-scaled decode GEMM
for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libfp8bs.so, reached through its C ABI (include/fp8bs.h) with
ctypes. PyTorch provides device memory and the stream. If the library is not
built, or a call returns a non-OK status, a Python exception is raised;
there is no other implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch  # loaded first so that libfp8bs binds to the HIP runtime torch uses

__all__ = [
    "Fp8bsError", "GemmConfig", "load", "library_path",
    "quantize_weight", "quantize_act", "gemm", "gemm_q", "gemm_ex", "gemm_noalloc",
    "pack_weight", "gemm_tiles", "gemm_q_tiles", "tiles_select_config", "gemm_swiglu_tiles",
    "workspace_bytes", "config_workspace_bytes", "select_config",
    "swiglu_quant", "gemm_swiglu", "gemm_swiglu_ex", "swiglu_select_config",
    "swiglu_workspace_bytes",
    "encode_e4m3", "launch_count", "build_info", "diag_read", "diag_copy", "diag_stream",
    "streamk_plan_check", "PATH_MFMA_STREAMK", "PATH_MFMA_ROWS_DMA", "diag_timestamp", "diag_timestamp_hz",
    "hip_runtime_mappings", "PATH_MFMA", "PATH_DOT", "REDUCE_KERNEL",
    "REDUCE_LAST_ARRIVER", "EPILOGUE_SEPARATE", "EPILOGUE_IN_GEMM", "LAYOUT_ROWS",
    "LAYOUT_TILES", "COUNTER",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libfp8bs.so")
_LIB = None

PATH_AUTO, PATH_MFMA, PATH_DOT, PATH_MFMA_ROWS, PATH_MFMA_STREAM, PATH_PREFILL = 0, 1, 2, 3, 4, 5
PATH_MFMA_ROWS_REG = 6
PATH_MFMA_STREAMK = 7
PATH_MFMA_ROWS_DMA = 8
REDUCE_KERNEL, REDUCE_LAST_ARRIVER = 0, 1
EPILOGUE_SEPARATE, EPILOGUE_IN_GEMM = 0, 1
LAYOUT_ROWS, LAYOUT_TILES = 0, 1
COUNTER = {"quant_weight": 0, "quant_act": 1, "gemm_mfma": 2, "gemm_dot": 3,
           "split_reduce": 4, "encode": 5, "diag": 6, "swiglu": 7, "pack": 8}


class Fp8bsError(RuntimeError):
    """A libfp8bs call returned a non-OK status."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class _Config(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in
                ("path", "tiles_n", "waves_n", "waves_k", "depth", "split_k", "reduce",
                 "epilogue", "weight_layout")]


@dataclass(frozen=True)
class GemmConfig:
    """Mirror of fp8bs_gemm_config (see include/fp8bs.h)."""
    path: int
    tiles_n: int
    waves_n: int
    waves_k: int
    depth: int
    split_k: int = 1
    reduce: int = REDUCE_KERNEL
    epilogue: int = EPILOGUE_SEPARATE
    weight_layout: int = LAYOUT_ROWS

    def _c(self) -> _Config:
        return _Config(self.path, self.tiles_n, self.waves_n, self.waves_k, self.depth,
                       self.split_k, self.reduce, self.epilogue, self.weight_layout)

    @staticmethod
    def _from_c(c: _Config) -> "GemmConfig":
        return GemmConfig(c.path, c.tiles_n, c.waves_n, c.waves_k, c.depth, c.split_k, c.reduce,
                          c.epilogue, c.weight_layout)


def library_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libfp8bs.so (built in-tree); raises if it is missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                           "(hipcc for gfx950) first")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "fp8bs_quantize_weight": (i32, [vp, i64, i64, vp, vp, vp]),
        "fp8bs_quantize_act": (i32, [vp, i64, i64, vp, vp, vp]),
        "fp8bs_gemm": (i32, [vp, i64, vp, vp, i64, i64, vp, vp, sz, vp]),
        "fp8bs_gemm_q": (i32, [vp, vp, i64, vp, vp, i64, i64, vp, vp, sz, vp]),
        "fp8bs_gemm_noalloc": (i32, [vp, i64, vp, vp, i64, i64, vp, vp]),
        "fp8bs_gemm_noalloc_max_scratch": (sz, []),
        "fp8bs_gemm_workspace_bytes": (sz, [i64, i64, i64]),
        "fp8bs_gemm_select_config": (i32, [i64, i64, i64, ctypes.POINTER(_Config)]),
        "fp8bs_gemm_config_workspace_bytes": (sz, [ctypes.POINTER(_Config), i64, i64, i64]),
        "fp8bs_gemm_ex": (i32, [vp, vp, vp, i64, vp, vp, i64, i64, vp, vp, sz,
                                ctypes.POINTER(_Config), vp]),
        "fp8bs_pack_weight": (i32, [vp, i64, i64, vp, vp]),
        "fp8bs_gemm_tiles": (i32, [vp, i64, vp, vp, i64, i64, vp, vp, sz, vp]),
        "fp8bs_gemm_q_tiles": (i32, [vp, vp, i64, vp, vp, i64, i64, vp, vp, sz, vp]),
        "fp8bs_gemm_tiles_select_config": (i32, [i64, i64, i64, ctypes.POINTER(_Config)]),
        "fp8bs_gemm_swiglu_tiles": (i32, [vp, i64, vp, vp, i64, i64, vp, vp, vp, vp, sz, vp]),
        "fp8bs_swiglu_quant": (i32, [vp, i64, i64, vp, vp, vp]),
        "fp8bs_gemm_swiglu": (i32, [vp, i64, vp, vp, i64, i64, vp, vp, vp, vp, sz, vp]),
        "fp8bs_gemm_swiglu_ex": (i32, [vp, vp, vp, i64, vp, vp, i64, i64, vp, vp, vp, vp, sz,
                                       ctypes.POINTER(_Config), vp]),
        "fp8bs_gemm_swiglu_select_config": (i32, [i64, i64, i64, ctypes.POINTER(_Config)]),
        "fp8bs_gemm_swiglu_workspace_bytes": (sz, [ctypes.POINTER(_Config), i64, i64, i64]),
        "fp8bs_encode_e4m3": (i32, [vp, i64, vp, i32, vp]),
        "fp8bs_status_string": (ctypes.c_char_p, [i32]),
        "fp8bs_launch_count": (ctypes.c_uint64, [i32]),
        "fp8bs_build_info": (ctypes.c_char_p, []),
        "fp8bs_diag_read": (i32, [vp, sz, vp, i32, vp]),
        "fp8bs_diag_copy": (i32, [vp, vp, sz, vp]),
        "fp8bs_diag_stream": (i32, [vp, sz, vp, i32, i32, vp]),
        "fp8bs_diag_timestamp": (i32, [vp, vp]),
        "fp8bs_diag_timestamp_hz": (ctypes.c_uint64, []),
        "fp8bs_streamk_plan_check": (i32, [i64, i64, i32, i32, i32]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _LIB = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        msg = load().fp8bs_status_string(status).decode()
        raise Fp8bsError(status, msg)


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str, ndim: int) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor")
    return t.data_ptr()


def quantize_weight(w: torch.Tensor, out=None, stream=None):
    """bf16 W[n][k] -> (E4M3 codes uint8 [n][k], fp32 scales [n/128][k/128])."""
    n, k = w.shape
    q, s = out if out is not None else (
        torch.empty((n, k), dtype=torch.uint8, device=w.device),
        torch.empty((n // 128, k // 128), dtype=torch.float32, device=w.device))
    _check(load().fp8bs_quantize_weight(_dev(w, torch.bfloat16, "w", 2), n, k,
                                        _dev(q, torch.uint8, "w_fp8", 2),
                                        _dev(s, torch.float32, "w_scale", 2), _stream(stream)))
    return q, s


def quantize_act(x: torch.Tensor, out=None, stream=None):
    """bf16 X[m][k] -> (E4M3 codes uint8 [m][k], fp32 scales [m][k/128])."""
    m, k = x.shape
    q, s = out if out is not None else (
        torch.empty((m, k), dtype=torch.uint8, device=x.device),
        torch.empty((m, k // 128), dtype=torch.float32, device=x.device))
    _check(load().fp8bs_quantize_act(_dev(x, torch.bfloat16, "x", 2), m, k,
                                     _dev(q, torch.uint8, "x_fp8", 2),
                                     _dev(s, torch.float32, "x_scale", 2), _stream(stream)))
    return q, s


def workspace_bytes(m: int, n: int, k: int) -> int:
    return int(load().fp8bs_gemm_workspace_bytes(m, n, k))


def config_workspace_bytes(cfg: GemmConfig, m: int, n: int, k: int) -> int:
    c = cfg._c()
    return int(load().fp8bs_gemm_config_workspace_bytes(ctypes.byref(c), m, n, k))


def select_config(m: int, n: int, k: int) -> GemmConfig:
    c = _Config()
    _check(load().fp8bs_gemm_select_config(m, n, k, ctypes.byref(c)))
    return GemmConfig._from_c(c)


def _out_ws(m, n, device, out, workspace, need):
    """Output tensor and workspace of one call. Returns (y, workspace tensor,
    pointer, bytes): the caller keeps the workspace tensor referenced until the
    launch is queued (a workspace freed earlier could be handed to another
    tensor of the same call) and then passes it to _done."""
    y = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=device)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return y, workspace, ws_ptr, ws_len


def _done(workspace, stream) -> None:
    """After the launch: a workspace used on a stream other than the current
    one is recorded on that stream, so the caching allocator does not reuse it
    before the kernels that read it have run."""
    if workspace is not None and stream is not None:
        workspace.record_stream(stream)


def gemm(x: torch.Tensor, w_q: torch.Tensor, w_s: torch.Tensor, out=None, workspace=None,
         stream=None) -> torch.Tensor:
    """Y[m][n] (bf16) = X[m][k] . W^T with the per-row 1x128 FP8 cast fused in."""
    m, k = x.shape
    n = w_q.shape[0]
    y, wst, ws, wl = _out_ws(m, n, x.device, out, workspace, workspace_bytes(m, n, k))
    _check(load().fp8bs_gemm(_dev(x, torch.bfloat16, "x", 2), m,
                             _dev(w_q, torch.uint8, "w_fp8", 2), _dev(w_s, torch.float32, "w_scale", 2),
                             n, k, _dev(y, torch.bfloat16, "y", 2), ws, wl, _stream(stream)))
    _done(wst, stream)
    return y


def gemm_noalloc(x: torch.Tensor, w_q: torch.Tensor, w_s: torch.Tensor, out: torch.Tensor,
                 stream=None) -> torch.Tensor:
    """gemm() through the entry point that allocates nothing: the library's
    fixed per-GPU scratch replaces the workspace (out must be given)."""
    m, k = x.shape
    n = w_q.shape[0]
    _check(load().fp8bs_gemm_noalloc(_dev(x, torch.bfloat16, "x", 2), m,
                                     _dev(w_q, torch.uint8, "w_fp8", 2),
                                     _dev(w_s, torch.float32, "w_scale", 2), n, k,
                                     _dev(out, torch.bfloat16, "y", 2), _stream(stream)))
    return out


def gemm_q(x_q: torch.Tensor, x_s: torch.Tensor, w_q: torch.Tensor, w_s: torch.Tensor,
           out=None, workspace=None, stream=None) -> torch.Tensor:
    """Same product from pre-quantized activations (codes and scales)."""
    m, k = x_q.shape
    n = w_q.shape[0]
    y, wst, ws, wl = _out_ws(m, n, x_q.device, out, workspace, workspace_bytes(m, n, k))
    _check(load().fp8bs_gemm_q(_dev(x_q, torch.uint8, "x_fp8", 2), _dev(x_s, torch.float32, "x_scale", 2),
                               m, _dev(w_q, torch.uint8, "w_fp8", 2),
                               _dev(w_s, torch.float32, "w_scale", 2), n, k,
                               _dev(y, torch.bfloat16, "y", 2), ws, wl, _stream(stream)))
    _done(wst, stream)
    return y


def pack_weight(w_q: torch.Tensor, out=None, stream=None) -> torch.Tensor:
    """Weight codes [n][k] (row-major) rearranged into the tile layout the
    *_tiles GEMM calls read (include/fp8bs.h); returned as a uint8 [n][k]
    tensor whose bytes are in that layout."""
    n, k = w_q.shape
    t = out if out is not None else torch.empty((n, k), dtype=torch.uint8, device=w_q.device)
    _check(load().fp8bs_pack_weight(_dev(w_q, torch.uint8, "w_fp8", 2), n, k,
                                    _dev(t, torch.uint8, "w_tiles", 2), _stream(stream)))
    return t


def tiles_select_config(m: int, n: int, k: int) -> GemmConfig:
    c = _Config()
    _check(load().fp8bs_gemm_tiles_select_config(m, n, k, ctypes.byref(c)))
    return GemmConfig._from_c(c)


def gemm_tiles(x: torch.Tensor, w_t: torch.Tensor, w_s: torch.Tensor, out=None, workspace=None,
               stream=None) -> torch.Tensor:
    """gemm() on weights in the tile layout (pack_weight)."""
    m, k = x.shape
    n = w_t.shape[0]
    y, wst, ws, wl = _out_ws(m, n, x.device, out, workspace, workspace_bytes(m, n, k))
    _check(load().fp8bs_gemm_tiles(_dev(x, torch.bfloat16, "x", 2), m,
                                   _dev(w_t, torch.uint8, "w_tiles", 2),
                                   _dev(w_s, torch.float32, "w_scale", 2), n, k,
                                   _dev(y, torch.bfloat16, "y", 2), ws, wl, _stream(stream)))
    _done(wst, stream)
    return y


def gemm_q_tiles(x_q: torch.Tensor, x_s: torch.Tensor, w_t: torch.Tensor, w_s: torch.Tensor,
                 out=None, workspace=None, stream=None) -> torch.Tensor:
    """gemm_q() on weights in the tile layout."""
    m, k = x_q.shape
    n = w_t.shape[0]
    y, wst, ws, wl = _out_ws(m, n, x_q.device, out, workspace, workspace_bytes(m, n, k))
    _check(load().fp8bs_gemm_q_tiles(_dev(x_q, torch.uint8, "x_fp8", 2),
                                     _dev(x_s, torch.float32, "x_scale", 2), m,
                                     _dev(w_t, torch.uint8, "w_tiles", 2),
                                     _dev(w_s, torch.float32, "w_scale", 2), n, k,
                                     _dev(y, torch.bfloat16, "y", 2), ws, wl, _stream(stream)))
    _done(wst, stream)
    return y


def gemm_ex(cfg: GemmConfig, w_q: torch.Tensor, w_s: torch.Tensor, x: torch.Tensor | None = None,
            x_q: torch.Tensor | None = None, x_s: torch.Tensor | None = None, out=None,
            workspace=None, stream=None) -> torch.Tensor:
    """GEMM with an explicit kernel configuration; x (bf16, fused cast) or
    x_q/x_s (pre-quantized)."""
    if x is not None:
        m, k = x.shape
        xp, xqp, xsp = _dev(x, torch.bfloat16, "x", 2), None, None
        device = x.device
    else:
        m, k = x_q.shape
        xp = None
        xqp, xsp = _dev(x_q, torch.uint8, "x_fp8", 2), _dev(x_s, torch.float32, "x_scale", 2)
        device = x_q.device
    n = w_q.shape[0]
    y, wst, ws, wl = _out_ws(m, n, device, out, workspace, config_workspace_bytes(cfg, m, n, k))
    c = cfg._c()
    _check(load().fp8bs_gemm_ex(xp, xqp, xsp, m, _dev(w_q, torch.uint8, "w_fp8", 2),
                                _dev(w_s, torch.float32, "w_scale", 2), n, k,
                                _dev(y, torch.bfloat16, "y", 2), ws, wl, ctypes.byref(c),
                                _stream(stream)))
    _done(wst, stream)
    return y


def _h_out(m, inter, device, h):
    if h is not None:
        return h
    return (torch.empty((m, inter), dtype=torch.uint8, device=device),
            torch.empty((m, inter // 128), dtype=torch.float32, device=device))


def swiglu_quant(y: torch.Tensor, h=None, stream=None):
    """MLP epilogue alone: y[m][2I] bf16 (gate | up) -> (codes uint8 [m][I],
    fp32 scales [m][I/128]) of h = silu(gate) * up."""
    m, n2 = y.shape
    inter = n2 // 2
    hq, hs = _h_out(m, inter, y.device, h)
    _check(load().fp8bs_swiglu_quant(_dev(y, torch.bfloat16, "y", 2), m, inter,
                                     _dev(hq, torch.uint8, "h_fp8", 2),
                                     _dev(hs, torch.float32, "h_scale", 2), _stream(stream)))
    return hq, hs


def swiglu_select_config(m: int, n: int, k: int) -> GemmConfig:
    c = _Config()
    _check(load().fp8bs_gemm_swiglu_select_config(m, n, k, ctypes.byref(c)))
    return GemmConfig._from_c(c)


def swiglu_workspace_bytes(m: int, n: int, k: int, cfg: GemmConfig | None = None) -> int:
    c = cfg._c() if cfg is not None else None
    return int(load().fp8bs_gemm_swiglu_workspace_bytes(
        ctypes.byref(c) if c is not None else None, m, n, k))


def gemm_swiglu(x: torch.Tensor, w_q: torch.Tensor, w_s: torch.Tensor, out=None, h=None,
                workspace=None, stream=None):
    """Up/gate projection with the SwiGLU epilogue fused in: returns
    (y [m][n] bf16, h codes [m][n/2], h scales [m][n/256])."""
    m, k = x.shape
    n = w_q.shape[0]
    y, wst, ws, wl = _out_ws(m, n, x.device, out, workspace, swiglu_workspace_bytes(m, n, k))
    hq, hs = _h_out(m, n // 2, x.device, h)
    _check(load().fp8bs_gemm_swiglu(_dev(x, torch.bfloat16, "x", 2), m,
                                    _dev(w_q, torch.uint8, "w_fp8", 2),
                                    _dev(w_s, torch.float32, "w_scale", 2), n, k,
                                    _dev(y, torch.bfloat16, "y", 2),
                                    _dev(hq, torch.uint8, "h_fp8", 2),
                                    _dev(hs, torch.float32, "h_scale", 2), ws, wl,
                                    _stream(stream)))
    _done(wst, stream)
    return y, hq, hs


def gemm_swiglu_tiles(x: torch.Tensor, w_t: torch.Tensor, w_s: torch.Tensor, out=None, h=None,
                      workspace=None, stream=None):
    """gemm_swiglu() on weights in the tile layout (pack_weight): y as
    gemm_tiles() gives it, h as swiglu_quant(y)."""
    m, k = x.shape
    n = w_t.shape[0]
    y, wst, ws, wl = _out_ws(m, n, x.device, out, workspace, workspace_bytes(m, n, k))
    hq, hs = _h_out(m, n // 2, x.device, h)
    _check(load().fp8bs_gemm_swiglu_tiles(_dev(x, torch.bfloat16, "x", 2), m,
                                          _dev(w_t, torch.uint8, "w_tiles", 2),
                                          _dev(w_s, torch.float32, "w_scale", 2), n, k,
                                          _dev(y, torch.bfloat16, "y", 2),
                                          _dev(hq, torch.uint8, "h_fp8", 2),
                                          _dev(hs, torch.float32, "h_scale", 2), ws, wl,
                                          _stream(stream)))
    _done(wst, stream)
    return y, hq, hs


def gemm_swiglu_ex(cfg: GemmConfig, w_q: torch.Tensor, w_s: torch.Tensor,
                   x: torch.Tensor | None = None, x_q: torch.Tensor | None = None,
                   x_s: torch.Tensor | None = None, out=None, h=None, workspace=None,
                   stream=None):
    """gemm_swiglu with an explicit kernel configuration."""
    if x is not None:
        m, k = x.shape
        xp, xqp, xsp = _dev(x, torch.bfloat16, "x", 2), None, None
        device = x.device
    else:
        m, k = x_q.shape
        xp = None
        xqp, xsp = _dev(x_q, torch.uint8, "x_fp8", 2), _dev(x_s, torch.float32, "x_scale", 2)
        device = x_q.device
    n = w_q.shape[0]
    y, wst, ws, wl = _out_ws(m, n, device, out, workspace, swiglu_workspace_bytes(m, n, k, cfg))
    hq, hs = _h_out(m, n // 2, device, h)
    c = cfg._c()
    _check(load().fp8bs_gemm_swiglu_ex(xp, xqp, xsp, m, _dev(w_q, torch.uint8, "w_fp8", 2),
                                       _dev(w_s, torch.float32, "w_scale", 2), n, k,
                                       _dev(y, torch.bfloat16, "y", 2),
                                       _dev(hq, torch.uint8, "h_fp8", 2),
                                       _dev(hs, torch.float32, "h_scale", 2), ws, wl,
                                       ctypes.byref(c), _stream(stream)))
    _done(wst, stream)
    return y, hq, hs


def encode_e4m3(v: torch.Tensor, mode: int = 0, out=None, stream=None) -> torch.Tensor:
    """fp32 values -> E4M3 codes (mode 0: quantizers' encoder, 1: hardware, 2: software)."""
    v = v.reshape(-1)
    o = out if out is not None else torch.empty(v.numel(), dtype=torch.uint8, device=v.device)
    _check(load().fp8bs_encode_e4m3(_dev(v, torch.float32, "in", 1), v.numel(),
                                    _dev(o, torch.uint8, "out", 1), mode, _stream(stream)))
    return o


def launch_count(which: str | int) -> int:
    idx = COUNTER[which] if isinstance(which, str) else int(which)
    return int(load().fp8bs_launch_count(idx))


def build_info() -> str:
    return load().fp8bs_build_info().decode()


def diag_read(t: torch.Tensor, sink: torch.Tensor, blocks: int = 0, stream=None) -> None:
    nbytes = t.numel() * t.element_size()
    _check(load().fp8bs_diag_read(t.data_ptr(), nbytes, sink.data_ptr(), blocks, _stream(stream)))


def diag_stream(t: torch.Tensor, sink: torch.Tensor, blocks: int = 256, depth: int = 8,
                stream=None, nbytes: int | None = None) -> None:
    """Streaming-read ceiling kernel over the first nbytes (default: all) of t
    (depth 0: direct-to-LDS loads by 4 waves per workgroup)."""
    nb = t.numel() * t.element_size() if nbytes is None else int(nbytes)
    _check(load().fp8bs_diag_stream(t.data_ptr(), nb, sink.data_ptr(), blocks, depth,
                                    _stream(stream)))


def diag_timestamp(out: torch.Tensor, stream=None) -> None:
    """Write the GPU wall clock into out (an int64 tensor of at least one
    element) when the launch runs."""
    _check(load().fp8bs_diag_timestamp(out.data_ptr(), _stream(stream)))


def diag_timestamp_hz() -> int:
    return int(load().fp8bs_diag_timestamp_hz())


def streamk_plan_check(n: int, k: int, split: int, workgroups: int = 256,
                       whole: bool = False) -> int:
    """Host-side self-check of the stream-K work partition (0 = consistent,
    1 = not a supported partition, other values: the first inconsistency)."""
    return int(load().fp8bs_streamk_plan_check(n, k, split, workgroups, int(whole)))


def diag_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst too small")
    _check(load().fp8bs_diag_copy(src.data_ptr(), dst.data_ptr(), nbytes, _stream(stream)))


def hip_runtime_mappings() -> dict:
    """Which HIP runtime files and which libfp8bs are mapped into this process
    (read from /proc/self/maps): a check that exactly one runtime is in use."""
    hip, ours = set(), set()
    with open("/proc/self/maps") as f:
        for line in f:
            parts = line.split()
            if len(parts) >= 6:
                path = parts[5]
                base = os.path.basename(path)
                if base.startswith("libamdhip64"):
                    hip.add(os.path.realpath(path))
                elif base == "libfp8bs.so":
                    ours.add(os.path.realpath(path))
    return {"libamdhip64": sorted(hip), "libfp8bs": sorted(ours)}
