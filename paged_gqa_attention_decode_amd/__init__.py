"""MI355X (gfx950) paged grouped-query attention: Python binding of ``libpaged_attn.so``.

The functions below carry the names of the C ABI in ``include/paged_attn.h`` and do only
argument marshalling: they read shapes off torch tensors, check dtype/device/contiguity,
pass raw device pointers and the current HIP stream, and raise ``PagedAttnError`` on a
non-zero status.  Every step of the computation runs in the HIP kernels; there is no CPU
or eager-torch fallback.  If the library has not been built, the first call raises.

Build:  ``python -m paged_gqa_attention_decode_amd.build``
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpaged_attn.so")
# The checked build: the same entry points, which also report out-of-range device metadata
# (PA_EDATA) after synchronising.  Selected with use_checked_library() or, at import,
# PAGED_ATTN_CHECKED=1 in the environment.
CHECKED_LIB_PATH = os.path.join(_HERE, "libpaged_attn_checked.so")

PA_OK, PA_EINVAL, PA_EUNSUPPORTED, PA_ELAUNCH, PA_EDATA, PA_ESCRATCH = 0, -1, -2, -3, -4, -5
PA_F32, PA_F16, PA_BF16 = 0, 1, 2
PA_ROPE_ADJACENT, PA_ROPE_HALVES = 0, 1

C_FUNCTIONS = ("paged_attn_status_string", "paged_attn_decode_workspace_bytes",
               "paged_attn_decode", "paged_attn_decode_fused",
               "paged_attn_decode_fused_counters", "paged_attn_decode_fused_noalloc",
               "paged_attn_noalloc_scratch_bytes", "paged_attn_combine", "paged_attn_prefill",
               "kv_page_write", "kv_page_write_rope")


class PagedAttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({paged_attn_status_string(status)})")


_libs = {}
_checked = os.environ.get("PAGED_ATTN_CHECKED", "") == "1"


def use_checked_library(flag: bool = True) -> None:
    """Route the functions of this module to the checked build (flag=True) or back."""
    global _checked
    _checked = bool(flag)


def raw_library(checked: bool | None = None):
    """The loaded ``ctypes.CDLL`` with argument types set (pointers as ``c_void_p``): the
    product library, or the checked build when selected."""
    path = CHECKED_LIB_PATH if (_checked if checked is None else checked) else LIB_PATH
    if path not in _libs:
        if not os.path.exists(path):
            raise ImportError(
                f"{path} is missing: build it with "
                "`python -m paged_gqa_attention_decode_amd.build` (there is no fallback)")
        lib = ctypes.CDLL(path)
        p, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        lib.paged_attn_status_string.argtypes = [i]
        lib.paged_attn_status_string.restype = ctypes.c_char_p
        lib.paged_attn_decode_workspace_bytes.argtypes = [i, i, i, i]
        lib.paged_attn_decode_workspace_bytes.restype = ctypes.c_size_t
        lib.paged_attn_decode.argtypes = [p, p, p, i, p, p, i, i, i, i, i, i, i, f, i, i, p, p,
                                          p]
        lib.paged_attn_decode_fused.argtypes = [p, p, p, p, p, i, p, p, i, i, i, i, i, i, i, f,
                                                i, i, p, p, p, p, p]
        lib.paged_attn_decode_fused_noalloc.argtypes = [p, p, p, p, p, i, p, p, i, i, i, i, i,
                                                        i, i, f, i, i, p, p]
        lib.paged_attn_noalloc_scratch_bytes.argtypes = []
        lib.paged_attn_noalloc_scratch_bytes.restype = ctypes.c_size_t
        lib.paged_attn_decode_fused_counters.argtypes = [i, i, i]
        lib.paged_attn_decode_fused_counters.restype = ctypes.c_size_t
        lib.paged_attn_combine.argtypes = [p, p, i, i, i, i, p, p]
        lib.paged_attn_prefill.argtypes = [p, p, p, i, p, p, i, i, i, i, i, i, i, i, i, i, f,
                                           p, p]
        lib.kv_page_write.argtypes = [p, p, p, p, i, p, p, p, i, i, i, i, i, i, i, p]
        lib.kv_page_write_rope.argtypes = [p, p, p, p, i, p, p, p, p, i, p, i, i, i, i, i, i,
                                           i, i, p]
        for name in ("paged_attn_decode", "paged_attn_decode_fused",
                     "paged_attn_decode_fused_noalloc", "paged_attn_combine",
                     "paged_attn_prefill", "kv_page_write", "kv_page_write_rope"):
            getattr(lib, name).restype = ctypes.c_int
        _libs[path] = lib
    return _libs[path]


def paged_attn_status_string(status: int) -> str:
    return raw_library().paged_attn_status_string(int(status)).decode()


def paged_attn_decode_workspace_bytes(num_seqs: int, num_q_heads: int, head_dim: int,
                                      num_splits: int) -> int:
    return int(raw_library().paged_attn_decode_workspace_bytes(num_seqs, num_q_heads,
                                                                head_dim, num_splits))


# ----------------------------------------------------------------------------- marshalling

def _torch():
    import torch
    return torch


def _kv_dtype(t) -> int:
    torch = _torch()
    codes = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}
    if t.dtype not in codes:
        raise TypeError(f"K/V cache dtype must be float32, float16 or bfloat16, got {t.dtype}")
    return codes[t.dtype]


def _dev(t, name, dtype=None, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if t.device.index != torch.cuda.current_device():
        # The library launches on the current device (its stream, its CU count).
        raise ValueError(f"{name} is on {t.device}, but the current device is "
                         f"cuda:{torch.cuda.current_device()}; call under "
                         f"torch.cuda.device({t.device.index})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream):
    torch = _torch()
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _ok(fn, status):
    if status != PA_OK:
        raise PagedAttnError(fn, status)


# ----------------------------------------------------------------------------- entry points

def paged_attn_decode(q, k_pages, v_pages, page_table, context_lens, scale: float,
                      partial_o, partial_ml, stream=None, window: int = 0) -> None:
    """Split-KV decode partials.  q [B,Hq,D] f32; pages [P,ps,Hkv,D]; page_table [B,maxp]
    int32; context_lens [B] int32; partial_o [B,Hq,S,D] f32; partial_ml [B,Hq,S,2] f32.
    window > 0 attends only the last `window` positions of each context."""
    torch = _torch()
    B, Hq, D = q.shape
    P, ps, Hkv, Dk = k_pages.shape
    S = partial_o.shape[2] if partial_o.dim() == 4 else -1
    if Dk != D or tuple(v_pages.shape) != tuple(k_pages.shape) or v_pages.dtype != k_pages.dtype:
        raise ValueError("k_pages / v_pages shapes or dtypes disagree with q")
    if tuple(partial_o.shape) != (B, Hq, S, D) or tuple(partial_ml.shape) != (B, Hq, S, 2):
        raise ValueError("partial_o must be [B,Hq,S,D] and partial_ml [B,Hq,S,2]")
    if page_table.shape[0] != B or tuple(context_lens.shape) != (B,):
        raise ValueError("page_table must be [B, max_pages] and context_lens [B]")
    rc = raw_library().paged_attn_decode(
        _dev(q, "q", torch.float32, 3), _dev(k_pages, "k_pages", ndim=4),
        _dev(v_pages, "v_pages", ndim=4), _kv_dtype(k_pages),
        _dev(page_table, "page_table", torch.int32, 2),
        _dev(context_lens, "context_lens", torch.int32, 1), B, Hq, Hkv, D, ps, P,
        page_table.shape[1], float(scale), int(window), S,
        _dev(partial_o, "partial_o", torch.float32),
        _dev(partial_ml, "partial_ml", torch.float32), _stream_handle(stream))
    _ok("paged_attn_decode", rc)


def paged_attn_decode_fused_counters(num_seqs: int, num_q_heads: int,
                                     num_kv_heads: int) -> int:
    return int(raw_library().paged_attn_decode_fused_counters(num_seqs, num_q_heads,
                                                               num_kv_heads))


def paged_attn_decode_fused(q, k_new, v_new, k_pages, v_pages, page_table, context_lens,
                            scale: float, partial_o, partial_ml, counters, out,
                            stream=None, window: int = 0) -> None:
    """One-launch decode step: writes the current token (k_new/v_new [B,Hkv,D]) into its
    page, computes the split partials and merges them into out [B,Hq,D] f32.  counters is a
    uint32 buffer (int32 tensor) of paged_attn_decode_fused_counters(...) entries, zero
    before the first call; each call leaves it zero.  window > 0 attends only the last
    `window` positions of each context."""
    torch = _torch()
    B, Hq, D = q.shape
    P, ps, Hkv, Dk = k_pages.shape
    S = partial_o.shape[2] if partial_o.dim() == 4 else -1
    if Dk != D or tuple(v_pages.shape) != tuple(k_pages.shape) or v_pages.dtype != k_pages.dtype:
        raise ValueError("k_pages / v_pages shapes or dtypes disagree with q")
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != (B, Hkv, D) or t.dtype != k_pages.dtype:
            raise ValueError(f"{name} must be [B, Hkv, D] in the cache dtype")
    if tuple(partial_o.shape) != (B, Hq, S, D) or tuple(partial_ml.shape) != (B, Hq, S, 2):
        raise ValueError("partial_o must be [B,Hq,S,D] and partial_ml [B,Hq,S,2]")
    if tuple(out.shape) != (B, Hq, D):
        raise ValueError("out must be [B,Hq,D]")
    need = paged_attn_decode_fused_counters(B, Hq, Hkv)
    if counters.dtype != torch.int32 or counters.numel() < need:
        raise ValueError(f"counters must be an int32 tensor of at least {need} entries")
    rc = raw_library().paged_attn_decode_fused(
        _dev(q, "q", torch.float32, 3), _dev(k_new, "k_new", ndim=3),
        _dev(v_new, "v_new", ndim=3), _dev(k_pages, "k_pages", ndim=4),
        _dev(v_pages, "v_pages", ndim=4), _kv_dtype(k_pages),
        _dev(page_table, "page_table", torch.int32, 2),
        _dev(context_lens, "context_lens", torch.int32, 1), B, Hq, Hkv, D, ps, P,
        page_table.shape[1], float(scale), int(window), S,
        _dev(partial_o, "partial_o", torch.float32),
        _dev(partial_ml, "partial_ml", torch.float32), _dev(counters, "counters"),
        _dev(out, "out", torch.float32, 3), _stream_handle(stream))
    _ok("paged_attn_decode_fused", rc)


def paged_attn_noalloc_scratch_bytes() -> int:
    return int(raw_library().paged_attn_noalloc_scratch_bytes())


def paged_attn_decode_fused_noalloc(q, k_new, v_new, k_pages, v_pages, page_table,
                                    context_lens, scale: float, num_splits: int, out,
                                    stream=None, window: int = 0) -> None:
    """paged_attn_decode_fused with the split partials and counters in the library's fixed
    per-GPU workspace instead of caller buffers (for callers that cannot allocate, e.g.
    under graph capture).  Raises PagedAttnError with PA_ESCRATCH when the call's split
    workspace does not fit; calls on one GPU must not overlap in time."""
    torch = _torch()
    B, Hq, D = q.shape
    P, ps, Hkv, Dk = k_pages.shape
    if Dk != D or tuple(v_pages.shape) != tuple(k_pages.shape) or v_pages.dtype != k_pages.dtype:
        raise ValueError("k_pages / v_pages shapes or dtypes disagree with q")
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != (B, Hkv, D) or t.dtype != k_pages.dtype:
            raise ValueError(f"{name} must be [B, Hkv, D] in the cache dtype")
    if tuple(out.shape) != (B, Hq, D):
        raise ValueError("out must be [B,Hq,D]")
    rc = raw_library().paged_attn_decode_fused_noalloc(
        _dev(q, "q", torch.float32, 3), _dev(k_new, "k_new", ndim=3),
        _dev(v_new, "v_new", ndim=3), _dev(k_pages, "k_pages", ndim=4),
        _dev(v_pages, "v_pages", ndim=4), _kv_dtype(k_pages),
        _dev(page_table, "page_table", torch.int32, 2),
        _dev(context_lens, "context_lens", torch.int32, 1), B, Hq, Hkv, D, ps, P,
        page_table.shape[1], float(scale), int(window), int(num_splits),
        _dev(out, "out", torch.float32, 3), _stream_handle(stream))
    _ok("paged_attn_decode_fused_noalloc", rc)


def paged_attn_combine(partial_o, partial_ml, out, stream=None) -> None:
    """Merge split partials into out [B,Hq,D] f32."""
    torch = _torch()
    B, Hq, S, D = partial_o.shape
    if tuple(partial_ml.shape) != (B, Hq, S, 2) or tuple(out.shape) != (B, Hq, D):
        raise ValueError("partial_ml must be [B,Hq,S,2] and out [B,Hq,D]")
    rc = raw_library().paged_attn_combine(
        _dev(partial_o, "partial_o", torch.float32, 4),
        _dev(partial_ml, "partial_ml", torch.float32, 4), B, Hq, D, S,
        _dev(out, "out", torch.float32, 3), _stream_handle(stream))
    _ok("paged_attn_combine", rc)


def paged_attn_prefill(q, k_pages, v_pages, page_table, seg_desc, max_chunk_len: int,
                       scale: float, out, stream=None) -> None:
    """Causal packed prefill.  q/out [T,Hq,D] f32; seg_desc [nseg,4] int32 on the device;
    max_chunk_len is the host copy of the longest chunk (sizes the grid)."""
    torch = _torch()
    T, Hq, D = q.shape
    P, ps, Hkv, Dk = k_pages.shape
    if Dk != D or tuple(v_pages.shape) != tuple(k_pages.shape) or v_pages.dtype != k_pages.dtype:
        raise ValueError("k_pages / v_pages shapes or dtypes disagree with q")
    if tuple(out.shape) != (T, Hq, D):
        raise ValueError("out must have q's shape")
    if seg_desc.dim() != 2 or seg_desc.shape[1] != 4:
        raise ValueError("seg_desc must be [num_segs, 4]")
    rc = raw_library().paged_attn_prefill(
        _dev(q, "q", torch.float32, 3), _dev(k_pages, "k_pages", ndim=4),
        _dev(v_pages, "v_pages", ndim=4), _kv_dtype(k_pages),
        _dev(page_table, "page_table", torch.int32, 2),
        _dev(seg_desc, "seg_desc", torch.int32, 2), seg_desc.shape[0], page_table.shape[0],
        T, int(max_chunk_len), Hq, Hkv, D, ps, P, page_table.shape[1], float(scale),
        _dev(out, "out", torch.float32, 3), _stream_handle(stream))
    _ok("paged_attn_prefill", rc)


def kv_page_write(k_new, v_new, k_pages, v_pages, page_table, token_table_index,
                  token_position, stream=None) -> None:
    """Copy k_new/v_new [T,Hkv,D] into their (page, slot), bit-exact."""
    torch = _torch()
    P, ps, Hkv, D = k_pages.shape
    T = k_new.shape[0]
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != (T, Hkv, D) or t.dtype != k_pages.dtype:
            raise ValueError(f"{name} must be [T, Hkv, D] in the cache dtype")
    if tuple(v_pages.shape) != tuple(k_pages.shape) or v_pages.dtype != k_pages.dtype:
        raise ValueError("k_pages / v_pages disagree")
    if tuple(token_table_index.shape) != (T,) or tuple(token_position.shape) != (T,):
        raise ValueError("token_table_index and token_position must be [T]")
    rc = raw_library().kv_page_write(
        _dev(k_new, "k_new", ndim=3), _dev(v_new, "v_new", ndim=3),
        _dev(k_pages, "k_pages", ndim=4), _dev(v_pages, "v_pages", ndim=4),
        _kv_dtype(k_pages), _dev(page_table, "page_table", torch.int32, 2),
        _dev(token_table_index, "token_table_index", torch.int32, 1),
        _dev(token_position, "token_position", torch.int32, 1), T, page_table.shape[0], Hkv,
        D, ps, P, page_table.shape[1], _stream_handle(stream))
    _ok("kv_page_write", rc)


def kv_page_write_rope(k_new, v_new, k_pages, v_pages, page_table, token_table_index,
                       token_position, inv_freq, style=PA_ROPE_HALVES, q=None,
                       stream=None) -> None:
    """Rotate k_new [T,Hkv,D] f32 by RoPE at token_position, round K and V to the pool dtype
    and write them into their (page, slot); rotate q [T,Hq,D] f32 in place if given.
    inv_freq is [D/2] f32; style PA_ROPE_ADJACENT pairs dims (2i, 2i+1), PA_ROPE_HALVES
    pairs (i, i + D/2)."""
    torch = _torch()
    P, ps, Hkv, D = k_pages.shape
    T = k_new.shape[0]
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != (T, Hkv, D) or t.dtype != torch.float32:
            raise ValueError(f"{name} must be [T, Hkv, D] float32")
    if tuple(v_pages.shape) != tuple(k_pages.shape) or v_pages.dtype != k_pages.dtype:
        raise ValueError("k_pages / v_pages disagree")
    if tuple(token_table_index.shape) != (T,) or tuple(token_position.shape) != (T,):
        raise ValueError("token_table_index and token_position must be [T]")
    if tuple(inv_freq.shape) != (D // 2,):
        raise ValueError("inv_freq must be [D/2]")
    hq = 0
    if q is not None:
        if q.dim() != 3 or q.shape[0] != T or q.shape[2] != D:
            raise ValueError("q must be [T, Hq, D] float32")
        hq = q.shape[1]
    rc = raw_library().kv_page_write_rope(
        _dev(k_new, "k_new", torch.float32, 3), _dev(v_new, "v_new", torch.float32, 3),
        _dev(k_pages, "k_pages", ndim=4), _dev(v_pages, "v_pages", ndim=4),
        _kv_dtype(k_pages), _dev(page_table, "page_table", torch.int32, 2),
        _dev(token_table_index, "token_table_index", torch.int32, 1),
        _dev(token_position, "token_position", torch.int32, 1),
        _dev(inv_freq, "inv_freq", torch.float32, 1), int(style),
        None if q is None else _dev(q, "q", torch.float32, 3), hq, T, page_table.shape[0], Hkv,
        D, ps, P, page_table.shape[1], _stream_handle(stream))
    _ok("kv_page_write_rope", rc)
