"""f64 CPU oracle for paged grouped-query attention — TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  It wraps ``oracle.c`` (plain C, IEEE double, single-threaded) through
ctypes and shares nothing with the HIP library: its own header, its own build, no common
helpers.  Arrays go in and out as numpy arrays:

* K/V pools are ``float32`` arrays for f32 and ``uint16`` bit patterns for f16 and bf16,
  shaped ``[num_pages, page_size, Hkv, D]``;
* ``q`` is ``float32`` ``[tokens, Hq, D]``; page tables, lengths, descriptors are ``int32``;
* results are ``float64``.

What each function computes, and the passages it follows, is documented in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}


def _compile(out_path: str, defines=()) -> str:
    tmp = out_path + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fPIC", "-fno-fast-math",
           "-ffp-contract=off", "-shared"] + ["-D%s" % d for d in defines] + \
          ["-o", tmp, _SRC, "-lm"]
    subprocess.check_call(cmd, cwd=_HERE)
    os.replace(tmp, out_path)
    return out_path


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc -O2 (no fast-math, no FMA contraction) into liboracle.so."""
    newest = max(os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "oracle.h")))
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < newest:
        _compile(_LIB_PATH)
    return _LIB_PATH


def _bind(path: str):
    lib = ctypes.CDLL(path)
    p = ctypes.c_void_p
    i = ctypes.c_int
    f = ctypes.c_float
    lib.oracle_decode.argtypes = [p, p, p, i, p, p, i, i, i, i, i, i, f, i, p]
    lib.oracle_decode_partials.argtypes = [p, p, p, i, p, p, i, i, i, i, i, i, f, i, i, p, p, p]
    lib.oracle_combine.argtypes = [p, p, p, i, i, i, i, p]
    lib.oracle_prefill.argtypes = [p, p, p, i, p, p, i, i, i, i, i, i, i, i, f, p, p]
    lib.oracle_kv_write.argtypes = [p, p, p, p, i, p, p, p, i, i, i, i, i, i, i]
    lib.oracle_widen.argtypes = [i, p, ctypes.c_int64, p]
    lib.oracle_widen.restype = None
    lib.oracle_split_range.argtypes = [i, i, i, ctypes.POINTER(i), ctypes.POINTER(i)]
    lib.oracle_kv_write_rope.argtypes = [p, p, p, p, i, p, p, p, p, i, p, i, i, i, i, i, i, i, i]
    lib.oracle_round_to.argtypes = [i, p, ctypes.c_int64, p]
    lib.oracle_round_to.restype = None
    for name in ("oracle_decode", "oracle_decode_partials", "oracle_combine",
                 "oracle_prefill", "oracle_kv_write", "oracle_split_range",
                 "oracle_kv_write_rope"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


_default = None


def _load():
    global _default
    if _default is None:
        _default = Oracle(build())
    return _default


def mutant(k: int) -> "Oracle":
    """An oracle built with planted mistake k (CPU mutation test only)."""
    path = os.path.join(_HERE, "_mutants", "liboracle_mut%d.so" % k)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
        _compile(path, defines=["ORACLE_MUTANT=%d" % k])
    return Oracle(path)


MUTANTS = {
    1: "f16 subnormals decoded with exponent -14 instead of -24",
    2: "slot = (t + 1) % page_size in the gather",
    3: "scale dropped from the score",
    4: "V accumulation reads K",
    5: "GQA map h -> h % Hkv instead of h / (Hq/Hkv)",
    6: "split chunk = floor(n / S) instead of ceil",
    7: "combine weights every split by 1 instead of exp(m_s - M)",
    8: "causal bound exclusive (row at P sees 0..P-1)",
    9: "prefill ignores absolute_start",
    10: "page write slot off by one",
    11: "prefill reads page-table row 0 for every segment",
    12: "RoPE turns pairs the wrong way (sin negated)",
    13: "RoPE rotates K at position + 1",
    14: "sliding window starts one position late",
}


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _pool(a, dtype: str):
    want = np.float32 if dtype == "f32" else np.uint16
    if a.dtype != want:
        raise TypeError(f"pool for {dtype} must be {np.dtype(want).name}, got {a.dtype}")
    return np.ascontiguousarray(a)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"{what}: oracle rejected the arguments (code {rc})")


class Oracle:
    """Bound instance of one oracle build (the normal one, or a planted-mistake mutant)."""

    def __init__(self, path: str):
        self.path = path
        self._lib = _bind(path)

    def widen(self, bits_or_values: np.ndarray, dtype: str) -> np.ndarray:
        """Exact f64 value of every element (f32 values, or f16/bf16 bit patterns)."""
        src = _pool(bits_or_values, dtype)
        out = np.empty(src.size, dtype=np.float64)
        self._lib.oracle_widen(DTYPE_CODES[dtype], _ptr(src), src.size, _ptr(out))
        return out.reshape(src.shape)

    def split_range(self, n: int, num_splits: int, split: int) -> tuple:
        lo, hi = ctypes.c_int(), ctypes.c_int()
        _check(self._lib.oracle_split_range(n, num_splits, split, ctypes.byref(lo), ctypes.byref(hi)),
               "split_range")
        return lo.value, hi.value

    def decode(self, q, k_pages, v_pages, dtype, page_table, context_lens, scale,
               window=0) -> np.ndarray:
        """Attention of each sequence's single query row over its whole context (over its
        last `window` positions when window > 0), f64."""
        q = _c(q, np.float32)
        kp, vp = _pool(k_pages, dtype), _pool(v_pages, dtype)
        table = _c(page_table, np.int32)
        ctx = _c(context_lens, np.int32)
        B, Hq, D = q.shape
        _, ps, Hkv, _ = kp.shape
        out = np.empty((B, Hq, D), dtype=np.float64)
        _check(self._lib.oracle_decode(_ptr(q), _ptr(kp), _ptr(vp), DTYPE_CODES[dtype], _ptr(table),
                                     _ptr(ctx), B, Hq, Hkv, D, ps, table.shape[1],
                                     float(scale), int(window), _ptr(out)), "decode")
        return out

    def decode_partials(self, q, k_pages, v_pages, dtype, page_table, context_lens, scale, num_splits,
                        window=0):
        """Per-split (O [B,Hq,S,D], m [B,Hq,S], l [B,Hq,S]) in natural-log units, f64."""
        q = _c(q, np.float32)
        kp, vp = _pool(k_pages, dtype), _pool(v_pages, dtype)
        table = _c(page_table, np.int32)
        ctx = _c(context_lens, np.int32)
        B, Hq, D = q.shape
        _, ps, Hkv, _ = kp.shape
        S = int(num_splits)
        po = np.empty((B, Hq, S, D), dtype=np.float64)
        pm = np.empty((B, Hq, S), dtype=np.float64)
        pl = np.empty((B, Hq, S), dtype=np.float64)
        _check(self._lib.oracle_decode_partials(_ptr(q), _ptr(kp), _ptr(vp), DTYPE_CODES[dtype],
                                              _ptr(table), _ptr(ctx), B, Hq, Hkv, D, ps,
                                              table.shape[1], float(scale), int(window), S, _ptr(po),
                                              _ptr(pm), _ptr(pl)), "decode_partials")
        return po, pm, pl

    def combine(self, partial_o, partial_m, partial_l) -> np.ndarray:
        """Log-sum-exp merge of split partials (inputs widened to f64), out [B,Hq,D]."""
        po = _c(partial_o, np.float64)
        pm = _c(partial_m, np.float64)
        pl = _c(partial_l, np.float64)
        B, Hq, S, D = po.shape
        out = np.empty((B, Hq, D), dtype=np.float64)
        _check(self._lib.oracle_combine(_ptr(po), _ptr(pm), _ptr(pl), B, Hq, D, S, _ptr(out)),
               "combine")
        return out

    def prefill(self, q, k_pages, v_pages, dtype, page_table, seg_desc, scale, out_init=None):
        """Causal packed prefill.  Returns (out [T,Hq,D] f64, causal positions per head).

        Rows covered by no segment keep ``out_init`` (NaN if not given)."""
        q = _c(q, np.float32)
        kp, vp = _pool(k_pages, dtype), _pool(v_pages, dtype)
        table = _c(page_table, np.int32)
        desc = _c(seg_desc, np.int32).reshape(-1, 4)
        T, Hq, D = q.shape
        _, ps, Hkv, _ = kp.shape
        out = (np.full((T, Hq, D), np.nan) if out_init is None
               else np.array(out_init, dtype=np.float64, copy=True))
        count = ctypes.c_int64(0)
        _check(self._lib.oracle_prefill(_ptr(q), _ptr(kp), _ptr(vp), DTYPE_CODES[dtype], _ptr(table),
                                      _ptr(desc), desc.shape[0], table.shape[0], T, Hq, Hkv, D, ps,
                                      table.shape[1], float(scale), _ptr(out),
                                      ctypes.cast(ctypes.byref(count), ctypes.c_void_p)), "prefill")
        return out, int(count.value)

    def kv_write(self, k_new, v_new, k_pages, v_pages, dtype, page_table, token_table_index,
                 token_position):
        """Return copies of the pools after the page write (inputs are not modified)."""
        kp = _pool(k_pages, dtype).copy()
        vp = _pool(v_pages, dtype).copy()
        kn, vn = _pool(k_new, dtype), _pool(v_new, dtype)
        table = _c(page_table, np.int32)
        owner = _c(token_table_index, np.int32)
        pos = _c(token_position, np.int32)
        P, ps, Hkv, D = kp.shape
        _check(self._lib.oracle_kv_write(_ptr(kn), _ptr(vn), _ptr(kp), _ptr(vp), DTYPE_CODES[dtype],
                                       _ptr(table), _ptr(owner), _ptr(pos), owner.shape[0],
                                       table.shape[0], Hkv, D, ps, P, table.shape[1]), "kv_write")
        return kp, vp


    def kv_write_rope(self, k_new, v_new, k_pages, v_pages, dtype, page_table,
                      token_table_index, token_position, inv_freq, style, q=None):
        """Return (K pool, V pool, q) after the page write with rotary position embedding.

        k_new, v_new are f32 [T, Hkv, D]; the pools are copied, not modified; q (f32
        [T, Hq, D], optional) is returned rotated (a copy), or None."""
        kp = _pool(k_pages, dtype).copy()
        vp = _pool(v_pages, dtype).copy()
        kn, vn = _c(k_new, np.float32), _c(v_new, np.float32)
        table = _c(page_table, np.int32)
        owner = _c(token_table_index, np.int32)
        pos = _c(token_position, np.int32)
        freq = _c(inv_freq, np.float32)
        P, ps, Hkv, D = kp.shape
        qq = None if q is None else np.array(q, dtype=np.float32, order="C", copy=True)
        hq = 0 if qq is None else qq.shape[1]
        _check(self._lib.oracle_kv_write_rope(
            _ptr(kn), _ptr(vn), _ptr(kp), _ptr(vp), DTYPE_CODES[dtype], _ptr(table), _ptr(owner),
            _ptr(pos), _ptr(freq), int(style), None if qq is None else _ptr(qq), hq,
            owner.shape[0], table.shape[0], Hkv, D, ps, P, table.shape[1]), "kv_write_rope")
        return kp, vp, qq

    def round_to(self, values, dtype: str) -> np.ndarray:
        """f64 values rounded to a pool dtype (through f32, ties to even): float32 values, or
        uint16 bit patterns for f16 / bf16."""
        src = _c(values, np.float64)
        out = np.empty(src.shape, dtype=np.float32 if dtype == "f32" else np.uint16)
        self._lib.oracle_round_to(DTYPE_CODES[dtype], _ptr(src), src.size, _ptr(out))
        return out


def widen(*a, **k):
    return _load().widen(*a, **k)


def split_range(*a, **k):
    return _load().split_range(*a, **k)


def decode(*a, **k):
    return _load().decode(*a, **k)


def decode_partials(*a, **k):
    return _load().decode_partials(*a, **k)


def combine(*a, **k):
    return _load().combine(*a, **k)


def prefill(*a, **k):
    return _load().prefill(*a, **k)


def kv_write(*a, **k):
    return _load().kv_write(*a, **k)


def kv_write_rope(*a, **k):
    return _load().kv_write_rope(*a, **k)


def round_to(*a, **k):
    return _load().round_to(*a, **k)
