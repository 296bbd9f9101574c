"""Python binding of libuocr.so (ctypes).

Argument marshalling only: each function checks the tensors it is given
(device, dtype, shape, contiguity), turns them into raw device pointers and
calls the C entry point of the same name on the current HIP stream.  Every
step of the computation runs in the gfx950 kernels of libuocr.so; there is no
fallback.  If the library is not built, loading fails with an error.

Names, argument order and semantics follow include/uocr.h.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libuocr.so")
# the same sources with the fused SR-SWA step's phase stamps compiled in
STAMPS_LIB_PATH = os.path.join(_HERE, "libuocr_stamps.so")

UOCR_F32, UOCR_BF16 = 0, 1
_TORCH_DTYPE = {UOCR_F32: torch.float32, UOCR_BF16: torch.bfloat16}
_DTYPE_CODE = {"f32": UOCR_F32, "bf16": UOCR_BF16}

STATUS = {0: "UOCR_OK", -1: "UOCR_ERR_NULL", -2: "UOCR_ERR_SHAPE", -3: "UOCR_ERR_DTYPE",
          -4: "UOCR_ERR_WORKSPACE", -5: "UOCR_ERR_ALIGN", -6: "UOCR_ERR_UNSUPPORTED",
          -7: "UOCR_ERR_HIP"}


class UocrError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} -> {STATUS.get(status, status)}: {detail}")
        self.status = status


class _Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("prefix_cap", ctypes.c_int32), ("window", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class _Route(ctypes.Structure):
    _fields_ = [("block_size", ctypes.c_int32), ("idx_dim", ctypes.c_int32), ("topk", ctypes.c_int32)]


class _Rope(ctypes.Structure):
    _fields_ = [("page", ctypes.c_void_p), ("offset", ctypes.c_void_p), ("page_mod", ctypes.c_int32),
                ("base", ctypes.c_float)]


@dataclasses.dataclass(frozen=True)
class Shape:
    batch: int
    heads: int
    head_dim: int
    prefix_cap: int
    window: int = 128
    dtype: int = UOCR_BF16
    scale: Optional[float] = None

    def c(self) -> _Shape:
        s = 1.0 / math.sqrt(self.head_dim) if self.scale is None else self.scale
        return _Shape(self.batch, self.heads, self.head_dim, self.prefix_cap, self.window, self.dtype, s)

    @property
    def units(self) -> int:
        return self.batch * self.heads

    @property
    def nb_cap(self) -> int:
        return -(-self.prefix_cap // 32)

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TORCH_DTYPE[self.dtype]

    @staticmethod
    def of(workload, prefix_cap: Optional[int] = None) -> "Shape":
        """Shape of a synth.Workload."""
        return Shape(workload.batch, workload.heads, workload.head_dim,
                     workload.prefix_len if prefix_cap is None else prefix_cap, workload.window,
                     _DTYPE_CODE[workload.dtype], workload.scale)


@dataclasses.dataclass(frozen=True)
class Route:
    block_size: int = 32
    idx_dim: int = 32
    topk: int = 16

    def c(self) -> _Route:
        return _Route(self.block_size, self.idx_dim, self.topk)


_lib = None
_lib_path = LIB_PATH
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t


def use_phase_stamps() -> None:
    """Make this process load libuocr_stamps.so instead of libuocr.so: the
    same entry points, with the fused SR-SWA step recording its phase stamps
    (read with uocr_phase_stamps).  Must come before the first call."""
    global _lib_path
    if _lib is not None and _lib_path != STAMPS_LIB_PATH:
        raise RuntimeError("libuocr.so is already loaded in this process")
    _lib_path = STAMPS_LIB_PATH


def load_library():
    """Load libuocr.so (once; libuocr_stamps.so after use_phase_stamps()).
    torch is imported first so that the process has a single HIP runtime.
    Raises if the library has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_lib_path):
        raise RuntimeError(f"{_lib_path} is missing: build it with "
                           "`python -m long_context_decode_attn_amd.build` (needs hipcc)")
    lib = ctypes.CDLL(_lib_path)
    SP, RP = ctypes.POINTER(_Shape), ctypes.POINTER(_Route)
    sig = {
        "uocr_ring_append": (ctypes.c_int, [SP, _P, _P, _P, _P, _P, _P]),
        "uocr_rswa_splits": (_I32, [SP, _I32]),
        "uocr_rswa_workspace_bytes": (_SZ, [SP, _I32]),
        "uocr_rswa_decode": (ctypes.c_int, [SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _I32, _P]),
        "uocr_rswa_decode_static": (ctypes.c_int, [SP, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P]),
        "uocr_block_index_build": (ctypes.c_int, [SP, RP, _P, _P, _P, _P, _P]),
        "uocr_block_index_range": (ctypes.c_int, [SP, RP, _P, _P, _P, _P, _I32, _I32, _P]),
        "uocr_block_score": (ctypes.c_int, [SP, RP, _P, _P, _P, _P, _P, _P]),
        "uocr_entmax15_topk": (ctypes.c_int, [SP, RP, _P, _P, _P, _P, _P, _P]),
        "uocr_prefill_route": (ctypes.c_int, [SP, RP, _P, _I32, _P, _P, _P, _P, _P, _P, _P, _P]),
        "uocr_ngram_ban": (ctypes.c_int, [_I32, _P, _I32, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _I32, _I32,
                                          _P]),
        "uocr_rope_page2d": (ctypes.c_int, [SP, _P, _P, _I32, _P, _P, _I32, ctypes.c_float, _P]),
        "uocr_srswa_splits": (_I32, [SP, RP, _I32]),
        "uocr_srswa_workspace_bytes": (_SZ, [SP, RP, _I32]),
        "uocr_srswa_decode": (ctypes.c_int, [SP, RP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _I32, _P]),
        "uocr_rswa_step": (ctypes.c_int, [SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _I32, _P, _P]),
        "uocr_srswa_step": (ctypes.c_int, [SP, RP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                           _P, _I32, _P, _P]),
        "uocr_calib_read": (ctypes.c_int, [_P, _SZ, _I32, _P, _P]),
        "uocr_calib_empty": (ctypes.c_int, [_I32, _I32, _P]),
        "uocr_calib_pull": (ctypes.c_int, [_P, _SZ, _I32, _I32, _I32, _P, _P]),
        "uocr_calib_start": (ctypes.c_int, [_I32, _I32, _P, _P]),
        "uocr_calib_exchange": (ctypes.c_int, [_I32, _I32, _I32, _P, _P, _P, _P]),
        "uocr_phase_stamps": (ctypes.c_int, [_P, _I32, _P]),
        "uocr_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "uocr_last_error": (ctypes.c_char_p, []),
        "uocr_version": (ctypes.c_int, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


EXPORTED = ("uocr_ring_append", "uocr_rswa_splits", "uocr_rswa_workspace_bytes",
            "uocr_rswa_decode", "uocr_rswa_decode_static", "uocr_block_index_build", "uocr_block_index_range", "uocr_block_score", "uocr_entmax15_topk",
            "uocr_prefill_route", "uocr_ngram_ban", "uocr_rope_page2d",
            "uocr_srswa_splits", "uocr_srswa_workspace_bytes", "uocr_srswa_decode", "uocr_rswa_step", "uocr_srswa_step",
            "uocr_status_string", "uocr_last_error", "uocr_version",
            "uocr_calib_read", "uocr_calib_empty", "uocr_calib_pull", "uocr_calib_start", "uocr_calib_exchange",
            "uocr_phase_stamps")


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------
def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(t: Optional[torch.Tensor], name: str, dtype: torch.dtype, shape, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _call(fn: str, *args) -> None:
    lib = load_library()
    rc = getattr(lib, fn)(*args)
    if rc != 0:
        raise UocrError(fn, rc, lib.uocr_last_error().decode())


# ----------------------------------------------------------------------------
# entry points
# ----------------------------------------------------------------------------
def uocr_ring_append(shape: Shape, k_ring, v_ring, k_new, v_new, t_gen, stream=None) -> None:
    B, H, D, n, dt = shape.batch, shape.heads, shape.head_dim, shape.window, shape.torch_dtype
    _check(k_ring, "k_ring", dt, (B, H, n, D))
    _check(v_ring, "v_ring", dt, (B, H, n, D))
    _check(k_new, "k_new", dt, (B, H, D))
    _check(v_new, "v_new", dt, (B, H, D))
    _check(t_gen, "t_gen", torch.int32, (B,))
    _call("uocr_ring_append", ctypes.byref(shape.c()), _ptr(k_ring), _ptr(v_ring), _ptr(k_new),
          _ptr(v_new), _ptr(t_gen), _stream(stream))


def uocr_rswa_splits(shape: Shape, num_splits: int = 0) -> int:
    return int(load_library().uocr_rswa_splits(ctypes.byref(shape.c()), num_splits))


def uocr_rswa_workspace_bytes(shape: Shape, num_splits: int = 0) -> int:
    return int(load_library().uocr_rswa_workspace_bytes(ctypes.byref(shape.c()), num_splits))


def uocr_srswa_splits(shape: Shape, route: Route, num_splits: int = 0) -> int:
    return int(load_library().uocr_srswa_splits(ctypes.byref(shape.c()), ctypes.byref(route.c()), num_splits))


def alloc_workspace(nbytes: int, device="cuda") -> Optional[torch.Tensor]:
    """A dense-decode workspace of at least `nbytes` bytes (None if 0)."""
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _ws(workspace):
    if workspace is None:
        return None, 0
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def uocr_rswa_decode(shape: Shape, q, k_prefix, v_prefix, prefix_len, k_ring, v_ring, t_gen, out,
                     workspace=None, num_splits: int = 0, stream=None) -> None:
    B, H, D, n, m, dt = shape.batch, shape.heads, shape.head_dim, shape.window, shape.prefix_cap, shape.torch_dtype
    _check(q, "q", dt, (B, H, D))
    _check(k_prefix, "k_prefix", dt, (B, H, m, D))
    _check(v_prefix, "v_prefix", dt, (B, H, m, D))
    _check(prefix_len, "prefix_len", torch.int32, (B,))
    _check(k_ring, "k_ring", dt, (B, H, n, D))
    _check(v_ring, "v_ring", dt, (B, H, n, D))
    _check(t_gen, "t_gen", torch.int32, (B,))
    _check(out, "out", dt, (B, H, D))
    wp, wb = _ws(workspace)
    _call("uocr_rswa_decode", ctypes.byref(shape.c()), _ptr(q), _ptr(k_prefix), _ptr(v_prefix), _ptr(prefix_len),
          _ptr(k_ring), _ptr(v_ring), _ptr(t_gen), _ptr(out), wp, wb, num_splits, _stream(stream))


def uocr_rswa_decode_static(shape: Shape, q, k_prefix, v_prefix, prefix_len, k_ring, v_ring, t_gen, out,
                            num_splits: int = 0, stream=None) -> None:
    """uocr_rswa_decode with the library's static workspace (no workspace argument)."""
    B, H, D, n, m, dt = shape.batch, shape.heads, shape.head_dim, shape.window, shape.prefix_cap, shape.torch_dtype
    _check(q, "q", dt, (B, H, D))
    _check(k_prefix, "k_prefix", dt, (B, H, m, D))
    _check(v_prefix, "v_prefix", dt, (B, H, m, D))
    _check(prefix_len, "prefix_len", torch.int32, (B,))
    _check(k_ring, "k_ring", dt, (B, H, n, D))
    _check(v_ring, "v_ring", dt, (B, H, n, D))
    _check(t_gen, "t_gen", torch.int32, (B,))
    _check(out, "out", dt, (B, H, D))
    _call("uocr_rswa_decode_static", ctypes.byref(shape.c()), _ptr(q), _ptr(k_prefix), _ptr(v_prefix),
          _ptr(prefix_len), _ptr(k_ring), _ptr(v_ring), _ptr(t_gen), _ptr(out), num_splits, _stream(stream))


def uocr_block_index_build(shape: Shape, route: Route, k_prefix, prefix_len, proj, kbar_idx, stream=None) -> None:
    B, H, D, m, dt = shape.batch, shape.heads, shape.head_dim, shape.prefix_cap, shape.torch_dtype
    _check(k_prefix, "k_prefix", dt, (B, H, m, D))
    _check(prefix_len, "prefix_len", torch.int32, (B,))
    _check(proj, "proj", torch.float32, (D, route.idx_dim))
    _check(kbar_idx, "kbar_idx", torch.float32, (B, H, shape.nb_cap, route.idx_dim))
    _call("uocr_block_index_build", ctypes.byref(shape.c()), ctypes.byref(route.c()), _ptr(k_prefix),
          _ptr(prefix_len), _ptr(proj), _ptr(kbar_idx), _stream(stream))


def uocr_block_index_range(shape: Shape, route: Route, k_prefix, prefix_len, proj, kbar_idx, first_block: int,
                           last_block: int, stream=None) -> None:
    B, H, D, m, dt = shape.batch, shape.heads, shape.head_dim, shape.prefix_cap, shape.torch_dtype
    _check(k_prefix, "k_prefix", dt, (B, H, m, D))
    _check(prefix_len, "prefix_len", torch.int32, (B,))
    _check(proj, "proj", torch.float32, (D, route.idx_dim))
    _check(kbar_idx, "kbar_idx", torch.float32, (B, H, shape.nb_cap, route.idx_dim))
    _call("uocr_block_index_range", ctypes.byref(shape.c()), ctypes.byref(route.c()), _ptr(k_prefix),
          _ptr(prefix_len), _ptr(proj), _ptr(kbar_idx), first_block, last_block, _stream(stream))


def uocr_block_score(shape: Shape, route: Route, q, proj, kbar_idx, prefix_len, scores, stream=None) -> None:
    B, H, D, dt = shape.batch, shape.heads, shape.head_dim, shape.torch_dtype
    _check(q, "q", dt, (B, H, D))
    _check(proj, "proj", torch.float32, (D, route.idx_dim))
    _check(kbar_idx, "kbar_idx", torch.float32, (B, H, shape.nb_cap, route.idx_dim))
    _check(prefix_len, "prefix_len", torch.int32, (B,))
    _check(scores, "scores", torch.float32, (B, H, shape.nb_cap))
    _call("uocr_block_score", ctypes.byref(shape.c()), ctypes.byref(route.c()), _ptr(q), _ptr(proj),
          _ptr(kbar_idx), _ptr(prefix_len), _ptr(scores), _stream(stream))


def uocr_entmax15_topk(shape: Shape, route: Route, scores, prefix_len, sel_idx, sel_prob, sel_bias,
                       stream=None) -> None:
    B, H, k = shape.batch, shape.heads, route.topk
    _check(scores, "scores", torch.float32, (B, H, shape.nb_cap))
    _check(prefix_len, "prefix_len", torch.int32, (B,))
    _check(sel_idx, "sel_idx", torch.int32, (B, H, k))
    _check(sel_prob, "sel_prob", torch.float32, (B, H, k), optional=True)
    _check(sel_bias, "sel_bias", torch.float32, (B, H, k))
    _call("uocr_entmax15_topk", ctypes.byref(shape.c()), ctypes.byref(route.c()), _ptr(scores), _ptr(prefix_len),
          _ptr(sel_idx), _ptr(sel_prob), _ptr(sel_bias), _stream(stream))


def uocr_prefill_route(shape: Shape, route: Route, q, q_pos, proj, kbar, prefix_len, sel_idx, sel_prob, sel_bias,
                       stream=None) -> None:
    """q [B][H][tq][D]; q_pos [B] int32; outputs [B][H][tq][topk]."""
    B, H, D, k = shape.batch, shape.heads, shape.head_dim, route.topk
    tq = int(q.shape[2]) if q.dim() == 4 else -1
    _check(q, "q", shape.torch_dtype, (B, H, tq, D))
    _check(q_pos, "q_pos", torch.int32, (B,))
    _check(proj, "proj", torch.float32, (D, 32))
    _check(kbar, "kbar", torch.float32, (B, H, shape.nb_cap, 32), optional=shape.nb_cap == 0)
    _check(prefix_len, "prefix_len", torch.int32, (B,))
    _check(sel_idx, "sel_idx", torch.int32, (B, H, tq, k))
    _check(sel_prob, "sel_prob", torch.float32, (B, H, tq, k), optional=True)
    _check(sel_bias, "sel_bias", torch.float32, (B, H, tq, k))
    _call("uocr_prefill_route", ctypes.byref(shape.c()), ctypes.byref(route.c()), _ptr(q), tq, _ptr(q_pos),
          _ptr(proj), _ptr(kbar), _ptr(prefix_len), _ptr(sel_idx), _ptr(sel_prob), _ptr(sel_bias),
          _stream(stream))


def uocr_ngram_ban(tokens, n_gen, page_tokens, logits, ngram: int, window: int, page_token: int = 0,
                   eos_token: int = 0, max_page_tokens: int = 0, stream=None) -> None:
    """tokens [B][ring_cap] int32 (position pos at pos % ring_cap); n_gen,
    page_tokens [B] int32; logits [B][vocab] float32 or bfloat16, in place."""
    B, V = int(logits.shape[0]), int(logits.shape[1]) if logits.dim() == 2 else -1
    if logits.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("logits must be float32 or bfloat16")
    _check(logits, "logits", logits.dtype, (B, V))
    _check(tokens, "tokens", torch.int32, (B, int(tokens.shape[1]) if tokens.dim() == 2 else -1))
    _check(n_gen, "n_gen", torch.int32, (B,))
    _check(page_tokens, "page_tokens", torch.int32, (B,), optional=max_page_tokens <= 0)
    dt = 0 if logits.dtype == torch.float32 else 1
    _call("uocr_ngram_ban", B, _ptr(tokens), int(tokens.shape[1]), _ptr(n_gen), _ptr(page_tokens), ngram, window,
          page_token, eos_token, max_page_tokens, _ptr(logits), V, dt, _stream(stream))


def uocr_rope_page2d(shape: Shape, x, page, offset, page_mod: int = 2, base: float = 10000.0, y=None,
                     stream=None) -> None:
    """x (and y, if given) [B][H][T][D] in shape's dtype, rotated in place;
    page, offset [B][T] int32: the position of each token, shared by its heads."""
    B, H, D, dt = shape.batch, shape.heads, shape.head_dim, shape.torch_dtype
    T = int(x.shape[2]) if x.dim() == 4 else -1
    _check(x, "x", dt, (B, H, T, D))
    _check(y, "y", dt, (B, H, T, D), optional=True)
    _check(page, "page", torch.int32, (B, T))
    _check(offset, "offset", torch.int32, (B, T))
    _call("uocr_rope_page2d", ctypes.byref(shape.c()), _ptr(x), _ptr(y), T, _ptr(page), _ptr(offset), page_mod,
          base, _stream(stream))


def uocr_srswa_workspace_bytes(shape: Shape, route: Route, num_splits: int = 0) -> int:
    return int(load_library().uocr_srswa_workspace_bytes(ctypes.byref(shape.c()), ctypes.byref(route.c()),
                                                         num_splits))


def uocr_srswa_decode(shape: Shape, route: Route, q, k_prefix, v_prefix, prefix_len, sel_idx, sel_bias,
                      k_ring, v_ring, t_gen, out, workspace=None, num_splits: int = 0, stream=None) -> None:
    B, H, D, n, m, dt = shape.batch, shape.heads, shape.head_dim, shape.window, shape.prefix_cap, shape.torch_dtype
    _check(q, "q", dt, (B, H, D))
    _check(k_prefix, "k_prefix", dt, (B, H, m, D))
    _check(v_prefix, "v_prefix", dt, (B, H, m, D))
    _check(prefix_len, "prefix_len", torch.int32, (B,))
    _check(sel_idx, "sel_idx", torch.int32, (B, H, route.topk))
    _check(sel_bias, "sel_bias", torch.float32, (B, H, route.topk), optional=True)
    _check(k_ring, "k_ring", dt, (B, H, n, D))
    _check(v_ring, "v_ring", dt, (B, H, n, D))
    _check(t_gen, "t_gen", torch.int32, (B,))
    _check(out, "out", dt, (B, H, D))
    _call("uocr_srswa_decode", ctypes.byref(shape.c()), ctypes.byref(route.c()), _ptr(q), _ptr(k_prefix),
          _ptr(v_prefix), _ptr(prefix_len), _ptr(sel_idx), _ptr(sel_bias), _ptr(k_ring), _ptr(v_ring),
          _ptr(t_gen), _ptr(out), *_ws(workspace), num_splits, _stream(stream))


def _rope(rope, batch: int):
    """rope = None or (page, offset, page_mod, base) with page, offset [B] int32
    device tensors: the position of each sequence's new token."""
    if rope is None:
        return None
    page, offset, page_mod, base = rope
    _check(page, "rope page", torch.int32, (batch,))
    _check(offset, "rope offset", torch.int32, (batch,))
    return ctypes.byref(_Rope(page.data_ptr(), offset.data_ptr(), page_mod, base))


def uocr_rswa_step(shape: Shape, q, k_new, v_new, k_prefix, v_prefix, prefix_len, k_ring, v_ring, t_gen_in,
                   t_gen_out, out, workspace=None, num_splits: int = 0, rope=None, stream=None) -> None:
    B, H, D, n, m, dt = shape.batch, shape.heads, shape.head_dim, shape.window, shape.prefix_cap, shape.torch_dtype
    for t, name, shp in [(q, "q", (B, H, D)), (k_new, "k_new", (B, H, D)), (v_new, "v_new", (B, H, D)),
                         (k_prefix, "k_prefix", (B, H, m, D)), (v_prefix, "v_prefix", (B, H, m, D)),
                         (k_ring, "k_ring", (B, H, n, D)), (v_ring, "v_ring", (B, H, n, D)), (out, "out", (B, H, D))]:
        _check(t, name, dt, shp)
    _check(prefix_len, "prefix_len", torch.int32, (B,))
    _check(t_gen_in, "t_gen_in", torch.int32, (B,))
    _check(t_gen_out, "t_gen_out", torch.int32, (B,))
    wp, wb = _ws(workspace)
    _call("uocr_rswa_step", ctypes.byref(shape.c()), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_prefix),
          _ptr(v_prefix), _ptr(prefix_len), _ptr(k_ring), _ptr(v_ring), _ptr(t_gen_in), _ptr(t_gen_out), _ptr(out),
          wp, wb, num_splits, _rope(rope, B), _stream(stream))


def uocr_srswa_step(shape: Shape, route: Route, q, k_new, v_new, k_prefix, v_prefix, prefix_len, proj, kbar_idx,
                    k_ring, v_ring, t_gen_in, t_gen_out, sel_idx, sel_prob, sel_bias, out, num_splits: int = 0,
                    rope=None, stream=None) -> None:
    B, H, D, n, m, dt, k = (shape.batch, shape.heads, shape.head_dim, shape.window, shape.prefix_cap,
                            shape.torch_dtype, route.topk)
    for t, name, shp in [(q, "q", (B, H, D)), (k_new, "k_new", (B, H, D)), (v_new, "v_new", (B, H, D)),
                         (k_prefix, "k_prefix", (B, H, m, D)), (v_prefix, "v_prefix", (B, H, m, D)),
                         (k_ring, "k_ring", (B, H, n, D)), (v_ring, "v_ring", (B, H, n, D)), (out, "out", (B, H, D))]:
        _check(t, name, dt, shp)
    _check(prefix_len, "prefix_len", torch.int32, (B,))
    _check(proj, "proj", torch.float32, (D, route.idx_dim))
    _check(kbar_idx, "kbar_idx", torch.float32, (B, H, shape.nb_cap, route.idx_dim))
    _check(t_gen_in, "t_gen_in", torch.int32, (B,))
    _check(t_gen_out, "t_gen_out", torch.int32, (B,))
    _check(sel_idx, "sel_idx", torch.int32, (B, H, k))
    _check(sel_prob, "sel_prob", torch.float32, (B, H, k), optional=True)
    _check(sel_bias, "sel_bias", torch.float32, (B, H, k))
    _call("uocr_srswa_step", ctypes.byref(shape.c()), ctypes.byref(route.c()), _ptr(q), _ptr(k_new), _ptr(v_new),
          _ptr(k_prefix), _ptr(v_prefix), _ptr(prefix_len), _ptr(proj), _ptr(kbar_idx), _ptr(k_ring), _ptr(v_ring),
          _ptr(t_gen_in), _ptr(t_gen_out), _ptr(sel_idx), _ptr(sel_prob), _ptr(sel_bias), _ptr(out), num_splits,
          _rope(rope, B), _stream(stream))


# ----------------------------------------------------------------------------
# measurement kernels (include/uocr_calib.h)
# ----------------------------------------------------------------------------
def _calib_call(fn: str, *args) -> None:
    rc = getattr(load_library(), fn)(*args)
    if rc != 0:
        raise UocrError(fn, rc, STATUS.get(rc, str(rc)))


def uocr_calib_read(src: torch.Tensor, nontemporal: bool, sink: torch.Tensor, stream=None) -> None:
    """Stream the whole of src (a device tensor, size a multiple of 16 bytes)."""
    _check(sink, "sink", torch.int32, (4096,))
    _calib_call("uocr_calib_read", _ptr(src), src.numel() * src.element_size(), int(nontemporal), _ptr(sink),
                _stream(stream))


def uocr_calib_empty(groups: int, threads: int, stream=None) -> None:
    _calib_call("uocr_calib_empty", groups, threads, _stream(stream))


def uocr_calib_pull(src: torch.Tensor, bytes_per_group: int, groups: int, threads: int, nontemporal: bool,
                    sink: torch.Tensor, stream=None) -> None:
    if src.numel() * src.element_size() < bytes_per_group * groups:
        raise ValueError("src is smaller than groups x bytes_per_group")
    _check(sink, "sink", torch.int32, (groups,))
    _calib_call("uocr_calib_pull", _ptr(src), bytes_per_group, groups, threads, int(nontemporal), _ptr(sink),
                _stream(stream))


def uocr_calib_start(groups: int, threads: int, stamps: torch.Tensor, stream=None) -> None:
    _check(stamps, "stamps", torch.int64, (groups,))
    _calib_call("uocr_calib_start", groups, threads, _ptr(stamps), _stream(stream))


def uocr_calib_exchange(mode: int, units: int, split: int, part: torch.Tensor, count: torch.Tensor,
                        out: torch.Tensor, stream=None) -> None:
    _check(part, "part", torch.float32, (units * split * 130,))
    _check(count, "count", torch.int32, (units,))
    _check(out, "out", torch.float32, (units * 130,))
    _calib_call("uocr_calib_exchange", mode, units, split, _ptr(part), _ptr(count), _ptr(out), _stream(stream))


def uocr_phase_stamps(units: int, stream=None) -> np.ndarray:
    """The phase stamps of units [0, units) of the latest fused SR-SWA steps,
    [units][64] uint64 (slots as in include/uocr_calib.h); raises UocrError
    (UOCR_ERR_UNSUPPORTED) unless use_phase_stamps() came first."""
    out = np.zeros((units, 64), dtype=np.uint64)
    rc = load_library().uocr_phase_stamps(ctypes.c_void_p(out.ctypes.data), int(units), _stream(stream))
    if rc != 0:
        raise UocrError("uocr_phase_stamps", rc, uocr_last_error())
    return out


def uocr_version() -> int:
    return int(load_library().uocr_version())


def uocr_status_string(status: int) -> str:
    return load_library().uocr_status_string(status).decode()


def uocr_last_error() -> str:
    return load_library().uocr_last_error().decode()
