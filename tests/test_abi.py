"""CPU: the C-ABI library loads, exports every function include/paged_attn.h declares, and
its host-side validation rejects malformed calls before anything reaches the device.

Every call here either carries an invalid argument or is an empty call; none can launch."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import paged_gqa_attention_decode_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_attn.h")
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: each call fails validation first
NULL = ctypes.c_void_p(0)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


def test_header_lists_the_four_entry_points():
    names = header_functions()
    for n in ("paged_attn_decode", "paged_attn_combine", "paged_attn_prefill",
              "kv_page_write", "paged_attn_decode_workspace_bytes",
              "paged_attn_status_string", "paged_attn_decode_fused",
              "paged_attn_decode_fused_counters", "kv_page_write_rope"):
        assert n in names
    assert set(names) == set(pa.C_FUNCTIONS)


@pytest.mark.parametrize("checked", [False, True], ids=["product", "checked"])
def test_library_exports_every_declared_symbol(checked):
    path = pa.CHECKED_LIB_PATH if checked else pa.LIB_PATH
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [n for n in header_functions() if n not in exported]
    assert not missing, missing
    lib = pa.raw_library(checked=checked)
    for n in header_functions():
        assert hasattr(lib, n)


def test_status_strings():
    assert pa.paged_attn_status_string(0) == "ok"
    assert pa.paged_attn_status_string(-1) == "invalid argument"
    assert pa.paged_attn_status_string(-2) == "unsupported configuration"
    assert pa.paged_attn_status_string(-3) == "kernel launch failed"
    assert pa.paged_attn_status_string(-4) == "device metadata out of range (checked build)"
    assert pa.paged_attn_status_string(-5) == "larger than the fixed no-allocation workspace"
    assert pa.paged_attn_status_string(42) == "unknown status"


def test_workspace_bytes():
    assert pa.paged_attn_decode_workspace_bytes(1, 40, 128, 32) == 40 * 32 * 130 * 4
    assert pa.paged_attn_decode_workspace_bytes(16, 64, 128, 16) == 16 * 64 * 16 * 130 * 4
    assert pa.paged_attn_decode_workspace_bytes(0, 40, 128, 32) == 0
    assert pa.paged_attn_decode_workspace_bytes(1, 40, 128, 0) == 0


# decode(q, k, v, dtype, table, ctx, B, Hq, Hkv, D, ps, P, maxp, scale, window, S, po, pml,
#        stream)
GOOD_DECODE = dict(q=FAKE, k=FAKE, v=FAKE, dtype=1, table=FAKE, ctx=FAKE, B=1, Hq=40, Hkv=8,
                   D=128, ps=16, P=204, maxp=204, scale=0.0884, window=0, S=32, po=FAKE,
                   pml=FAKE)


def decode(**kw):
    a = dict(GOOD_DECODE, **kw)
    return pa.raw_library().paged_attn_decode(
        a["q"], a["k"], a["v"], a["dtype"], a["table"], a["ctx"], a["B"], a["Hq"], a["Hkv"],
        a["D"], a["ps"], a["P"], a["maxp"], a["scale"], a["window"], a["S"], a["po"], a["pml"],
        NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0, q=NULL), pa.PA_OK),                  # empty batch: valid, nothing enqueued
    (dict(B=-1), pa.PA_EINVAL),
    (dict(q=NULL), pa.PA_EINVAL),
    (dict(k=NULL), pa.PA_EINVAL),
    (dict(po=NULL), pa.PA_EINVAL),
    (dict(pml=NULL), pa.PA_EINVAL),
    (dict(table=NULL), pa.PA_EINVAL),
    (dict(ctx=NULL), pa.PA_EINVAL),
    (dict(Hq=41, q=NULL), pa.PA_EINVAL),            # Hq not a multiple of Hkv
    (dict(Hq=41), pa.PA_EINVAL),
    (dict(Hkv=0), pa.PA_EINVAL),
    (dict(D=96), pa.PA_EUNSUPPORTED),
    (dict(D=256, dtype=0), pa.PA_EUNSUPPORTED),     # head_dim 256 is built for 16-bit K/V
    (dict(D=512), pa.PA_EUNSUPPORTED),
    (dict(D=256, q=NULL), pa.PA_EINVAL),
    (dict(D=0), pa.PA_EINVAL),
    (dict(ps=12), pa.PA_EUNSUPPORTED),
    (dict(ps=0), pa.PA_EINVAL),
    (dict(ps=8192), pa.PA_EUNSUPPORTED),
    (dict(S=0), pa.PA_EINVAL),
    (dict(S=5000), pa.PA_EUNSUPPORTED),
    (dict(dtype=7), pa.PA_EINVAL),
    (dict(Hq=65 * 8), pa.PA_EUNSUPPORTED),          # group of 65 query heads
    (dict(scale=math.nan), pa.PA_EINVAL),
    (dict(scale=math.inf), pa.PA_EINVAL),
    (dict(maxp=2 ** 28, ps=16), pa.PA_EINVAL),      # capacity overflows int32
    (dict(P=0), pa.PA_EINVAL),
    (dict(B=70000), pa.PA_EUNSUPPORTED),
])
def test_decode_validation(kw, status):
    assert decode(**kw) == status


def test_fused_counters_and_validation():
    lib = pa.raw_library()
    # one per (sequence, KV head, group of 8 query heads), doubled to cover head_dim 256
    # (groups of 4 there), each in a 128-byte line of its own (32 uint32 words)
    assert pa.paged_attn_decode_fused_counters(1, 40, 8) == 8 * 2 * 32
    assert pa.paged_attn_decode_fused_counters(16, 64, 8) == 128 * 2 * 32
    assert pa.paged_attn_decode_fused_counters(2, 12 * 16, 12) == 2 * 12 * 2 * 2 * 32   # G=16
    assert pa.paged_attn_decode_fused_counters(1, 41, 8) == 0
    f = lib.paged_attn_decode_fused
    # (q, k_new, v_new, kp, vp, dtype, table, ctx, B, Hq, Hkv, D, ps, P, maxp, scale, window,
    #  S, po, pml, counters, out, stream)
    good = [FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, 1, 40, 8, 128, 16, 204, 204, 0.0884,
            0, 32, FAKE, FAKE, FAKE, FAKE, NULL]

    def call(over):
        args = list(good)
        for k, v in over.items():
            args[k] = v
        return f(*args)

    assert call({8: 0, 0: NULL}) == pa.PA_OK
    for i in (0, 1, 2, 3, 4, 6, 7, 18, 19, 20, 21):
        assert call({i: NULL}) == pa.PA_EINVAL, i
    assert call({11: 96}) == pa.PA_EUNSUPPORTED
    assert call({11: 256, 5: 0}) == pa.PA_EUNSUPPORTED
    assert call({17: 0}) == pa.PA_EINVAL
    assert call({9: 41}) == pa.PA_EINVAL


def test_combine_validation():
    c = pa.raw_library().paged_attn_combine
    assert c(FAKE, FAKE, 0, 40, 128, 32, FAKE, NULL) == pa.PA_OK
    assert c(NULL, FAKE, 1, 40, 128, 32, FAKE, NULL) == pa.PA_EINVAL
    assert c(FAKE, FAKE, 1, 40, 128, 32, NULL, NULL) == pa.PA_EINVAL
    assert c(FAKE, FAKE, 1, 40, 96, 32, FAKE, NULL) == pa.PA_EUNSUPPORTED
    assert c(FAKE, FAKE, 1, 40, 128, 0, FAKE, NULL) == pa.PA_EINVAL
    assert c(FAKE, FAKE, 1, 0, 128, 32, FAKE, NULL) == pa.PA_EINVAL
    assert c(FAKE, FAKE, -1, 40, 128, 32, FAKE, NULL) == pa.PA_EINVAL


def test_prefill_validation():
    p = pa.raw_library().paged_attn_prefill
    # (q, k, v, dtype, table, desc, nseg, ntab, T, maxchunk, Hq, Hkv, D, ps, P, maxp, scale,
    #  out, stream)
    good = [FAKE, FAKE, FAKE, 0, FAKE, FAKE, 1, 1, 512, 512, 12, 12, 64, 16, 32, 32, 0.125,
            FAKE, NULL]

    def call(over):
        args = list(good)
        for k, v in over.items():
            args[k] = v
        return p(*args)

    assert call({6: 0}) == pa.PA_OK                     # no segments
    assert call({9: 0, 0: NULL}) == pa.PA_OK            # max_chunk_len 0
    assert call({0: NULL}) == pa.PA_EINVAL
    assert call({5: NULL}) == pa.PA_EINVAL
    assert call({17: NULL}) == pa.PA_EINVAL
    assert call({7: 0}) == pa.PA_EINVAL                 # no page tables
    assert call({6: -1}) == pa.PA_EINVAL
    assert call({10: 13}) == pa.PA_EINVAL               # 13 % 12
    assert call({12: 80}) == pa.PA_EUNSUPPORTED
    assert call({12: 256}) == pa.PA_EUNSUPPORTED        # head_dim 256: decode only
    assert call({13: 24}) == pa.PA_EUNSUPPORTED
    assert call({3: 3}) == pa.PA_EINVAL
    assert call({16: math.nan}) == pa.PA_EINVAL
    assert call({6: 70000}) == pa.PA_EUNSUPPORTED


def test_kv_write_validation():
    w = pa.raw_library().kv_page_write
    # (k_new, v_new, k_pages, v_pages, dtype, table, owner, pos, T, ntab, Hkv, D, ps, P,
    #  maxp, stream)
    good = [FAKE, FAKE, FAKE, FAKE, 2, FAKE, FAKE, FAKE, 16, 16, 8, 128, 32, 8192, 128, NULL]

    def call(over):
        args = list(good)
        for k, v in over.items():
            args[k] = v
        return w(*args)

    assert call({8: 0, 0: NULL}) == pa.PA_OK            # no tokens
    assert call({8: -1}) == pa.PA_EINVAL
    for i in (0, 1, 2, 3, 5, 6, 7):
        assert call({i: NULL}) == pa.PA_EINVAL, i
    assert call({9: 0}) == pa.PA_EINVAL
    assert call({11: 512}) == pa.PA_EUNSUPPORTED
    assert call({11: 96}) == pa.PA_EUNSUPPORTED
    assert call({12: 48}) == pa.PA_EUNSUPPORTED
    assert call({4: -1}) == pa.PA_EINVAL
    assert call({10: 0}) == pa.PA_EINVAL


def test_kv_write_rope_validation():
    w = pa.raw_library().kv_page_write_rope
    # (k_new, v_new, k_pages, v_pages, dtype, table, owner, pos, inv_freq, style, q, Hq, T,
    #  ntab, Hkv, D, ps, P, maxp, stream)
    good = [FAKE, FAKE, FAKE, FAKE, 2, FAKE, FAKE, FAKE, FAKE, 1, FAKE, 64, 16, 16, 8, 128, 32,
            8192, 128, NULL]

    def call(over):
        args = list(good)
        for k, v in over.items():
            args[k] = v
        return w(*args)

    assert call({12: 0, 0: NULL}) == pa.PA_OK           # no tokens
    assert call({12: -1}) == pa.PA_EINVAL
    for i in (0, 1, 2, 3, 5, 6, 7, 8):
        assert call({i: NULL}) == pa.PA_EINVAL, i
    assert call({9: 2}) == pa.PA_EINVAL                  # unknown pairing style
    assert call({9: -1}) == pa.PA_EINVAL
    assert call({11: 0}) == pa.PA_EINVAL                 # q given without query heads
    assert call({13: 0}) == pa.PA_EINVAL
    assert call({15: 96}) == pa.PA_EUNSUPPORTED
    assert call({16: 48}) == pa.PA_EUNSUPPORTED
    assert call({4: 7}) == pa.PA_EINVAL
    assert call({14: 0}) == pa.PA_EINVAL


def test_python_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 8, 64)
    k = torch.zeros(16, 16, 2, 64)
    with pytest.raises(ValueError, match="device"):
        pa.paged_attn_decode(q, k, k, torch.zeros(1, 16, dtype=torch.int32),
                             torch.ones(1, dtype=torch.int32), 0.125,
                             torch.zeros(1, 8, 4, 64), torch.zeros(1, 8, 4, 2))


# decode_fused_noalloc(q, k_new, v_new, k, v, dtype, table, ctx, B, Hq, Hkv, D, ps, P, maxp,
#                      scale, window, S, out, stream)
def noalloc(**kw):
    a = dict(GOOD_DECODE, **kw)
    return pa.raw_library().paged_attn_decode_fused_noalloc(
        a["q"], FAKE, FAKE, a["k"], a["v"], a["dtype"], a["table"], a["ctx"], a["B"], a["Hq"],
        a["Hkv"], a["D"], a["ps"], a["P"], a["maxp"], a["scale"], a["window"], a["S"], FAKE, NULL)


def test_noalloc_workspace_limits_are_checked_before_the_device():
    """The no-allocation step rejects a call whose partials or counters do not fit its fixed
    array with PA_ESCRATCH, and malformed arguments with PA_EINVAL, before any device call."""
    assert pa.paged_attn_noalloc_scratch_bytes() == 16 << 20
    assert noalloc(S=0) == pa.PA_EINVAL
    assert noalloc(Hq=41) == pa.PA_EINVAL
    assert noalloc(B=-1) == pa.PA_EINVAL
    # 64 sequences x 64 heads x 512 splits x 130 floats = 1.09 GB of partials
    assert noalloc(B=64, Hq=64, Hkv=8, S=512) == pa.PA_ESCRATCH
    # 1000 sequences x 8 KV heads x 2 counters = 16,000 counters > 8,192 (1 MiB of 128-byte
    # counter lines); the partials (1000 x 8 x 130 floats) would fit
    assert noalloc(B=1000, Hq=8, Hkv=8, S=1, D=128) == pa.PA_ESCRATCH
    assert noalloc(B=0) == pa.PA_OK


def test_probe_library_is_separate_and_rejects_bad_shapes():
    """The measurement kernels live in their own library: it exports the three probes, the
    attention library exports none of them, and a shape the walk does not cover is refused
    on the host (return value hipErrorInvalidValue, nothing launched)."""
    from paged_gqa_attention_decode_amd import build as hip_build
    out = subprocess.run(["nm", "-D", "--defined-only", hip_build.LIB_PROBES],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    probes = {"pa_probe_read_walk", "pa_probe_read_plain", "pa_probe_empty"}
    assert probes <= exported
    main = subprocess.run(["nm", "-D", "--defined-only", pa.LIB_PATH], capture_output=True,
                          text=True, check=True).stdout
    assert not any(p in main for p in probes)
    lib = ctypes.CDLL(hip_build.LIB_PROBES)
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.pa_probe_read_walk.argtypes = [vp, vp, i, vp, vp, i, i, i, i, i, i, i, i, i, vp, vp]
    lib.pa_probe_read_plain.argtypes = [vp, vp, ctypes.c_size_t, i, vp, vp]
    lib.pa_probe_empty.argtypes = [i, vp]
    invalid = 1  # hipErrorInvalidValue
    # rows of 24 bytes (head_dim 12 x 2 bytes) are not a whole number of 16-byte pieces
    assert lib.pa_probe_read_walk(FAKE, FAKE, 2, FAKE, FAKE, 1, 1, 12, 16, 4, 4, 1, 0, 0,
                                  FAKE, NULL) == invalid
    # a page size that is not a power of two; a table wider than the staged 4096 entries
    assert lib.pa_probe_read_walk(FAKE, FAKE, 2, FAKE, FAKE, 1, 1, 128, 24, 4, 4, 1, 0, 0,
                                  FAKE, NULL) == invalid
    assert lib.pa_probe_read_walk(FAKE, FAKE, 2, FAKE, FAKE, 1, 1, 128, 16, 4, 4097, 1, 0, 0,
                                  FAKE, NULL) == invalid
    # ranking a batch of more than 64 sequences
    assert lib.pa_probe_read_walk(FAKE, FAKE, 2, FAKE, FAKE, 65, 1, 128, 16, 4, 4, 1, 0, 4,
                                  FAKE, NULL) == invalid
    assert lib.pa_probe_read_plain(FAKE, FAKE, 24, 4, FAKE, NULL) == invalid
    assert lib.pa_probe_empty(0, NULL) == invalid
