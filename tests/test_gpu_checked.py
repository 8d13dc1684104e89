"""GPU: the checked build (libpaged_attn_checked.so, -DPAGED_ATTN_CHECKED).

Valid calls return OK with the same bits as the product library.  Device metadata out of its
documented range -- which every build clamps or skips, so no access leaves its buffer --
makes the checked call return PA_EDATA (after synchronising), while the product library
returns OK; the next valid checked call is OK again (the flags are cleared when read)."""
import numpy as np
import pytest
import torch

import paged_gqa_attention_decode_amd as pa
from compare import assert_bitwise
from gpu_helpers import DEV, DecodeRun, announce, dev, host
from paged_gqa_attention_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


@pytest.fixture
def checked():
    pa.use_checked_library(True)
    yield
    pa.use_checked_library(False)


def _decode_case(ctx=(100, 1000, 37), dtype="f16"):
    rng = wl.rng_for([800, len(ctx)])
    return wl.make_decode_case(rng, batch=len(ctx), hq=8, hkv=2, head_dim=128, page_size=16,
                               dtype=dtype, ctx=list(ctx), num_splits=8)


# f16 runs the matrix-core decode body, f32 the vector-unit body: both mark the same flags.
DECODE_DTYPES = pytest.mark.parametrize("dtype", ["f16", "f32"])


def _prefill_case():
    rng = wl.rng_for(801)
    return wl.make_prefill_case(rng, hq=12, hkv=3, head_dim=64, page_size=16, dtype="bf16",
                                lens=[37, 20], starts=[0, 40])


def _expect_edata(fn, what):
    with pytest.raises(pa.PagedAttnError) as e:
        fn()
    assert e.value.status == pa.PA_EDATA, f"{what}: {e.value}"


def _prefill(c, table=None, desc=None):
    kp, vp = dev(c.k_pages, c.dtype), dev(c.v_pages, c.dtype)
    t = dev(c.page_table if table is None else table)
    pa.kv_page_write(dev(c.k_new, c.dtype), dev(c.v_new, c.dtype), kp, vp, dev(c.page_table),
                     dev(c.token_table_index), dev(c.token_position))
    out = torch.zeros(c.q.shape, device=DEV)
    pa.paged_attn_prefill(dev(c.q), kp, vp, t, dev(c.seg_desc if desc is None else desc),
                          c.max_chunk_len, c.scale, out)
    torch.cuda.synchronize()
    return host(out)


@DECODE_DTYPES
def test_valid_calls_match_the_product_library(checked, dtype):
    announce(f"checked build: valid calls ({dtype} decode)")
    case = _decode_case(dtype=dtype)
    a, f = DecodeRun(case).step(), DecodeRun(case).fused_step()
    p = _prefill(_prefill_case())
    pa.use_checked_library(False)
    b, g = DecodeRun(case).step(), DecodeRun(case).fused_step()
    q = _prefill(_prefill_case())
    pa.use_checked_library(True)
    assert_bitwise(a, b, "decode: checked vs product")
    assert_bitwise(f, g, "single-launch step: checked vs product")
    assert_bitwise(p, q, "prefill: checked vs product")


@DECODE_DTYPES
def test_decode_page_id_out_of_range(checked, dtype):
    announce(f"checked build: decode with a page id past the pool ({dtype})")
    case = _decode_case(dtype=dtype)
    case.page_table = case.page_table.copy()
    case.page_table[1, 3] = case.k_pages.shape[0]      # inside sequence 1's 1000 positions
    run = DecodeRun(case)
    run.write()                                        # the current token's page is valid
    _expect_edata(lambda: pa.paged_attn_decode(run.q, run.kp, run.vp, run.table, run.ctx,
                                               case.scale, run.po, run.pml), "decode")
    _expect_edata(lambda: DecodeRun(case).fused_step(), "single-launch step")
    DecodeRun(_decode_case(dtype=dtype)).step()        # clean again
    pa.use_checked_library(False)
    DecodeRun(case).step()                             # the product library clamps: OK


@DECODE_DTYPES
def test_decode_length_past_capacity(checked, dtype):
    announce(f"checked build: decode length past the table's capacity ({dtype})")
    case = _decode_case(dtype=dtype)
    run = DecodeRun(case)
    run.write()
    cap = case.page_table.shape[1] * case.k_pages.shape[1]
    run.ctx = dev(np.array([100, cap + 5, 37], np.int32))
    _expect_edata(lambda: pa.paged_attn_decode(run.q, run.kp, run.vp, run.table, run.ctx,
                                               case.scale, run.po, run.pml), "length")
    run.ctx = dev(np.array([100, 0, 37], np.int32))    # an empty sequence is valid
    pa.paged_attn_decode(run.q, run.kp, run.vp, run.table, run.ctx, case.scale, run.po,
                         run.pml)
    torch.cuda.synchronize()


def test_page_writes(checked):
    announce("checked build: page writes")
    case = _decode_case()
    run = DecodeRun(case)
    run.write()                                        # valid
    run.owner = dev(np.array([0, -1, 2], np.int32))    # -1: an explicit skip, not an error
    run.write()
    run.owner = dev(np.array([0, 3, 2], np.int32))     # no table row 3
    _expect_edata(run.write, "owner past the table rows")
    run.owner = dev(case.token_table_index)
    table = case.page_table.copy()
    table[0, (int(case.token_position[0])) // 16] = -1  # the current token's page is missing
    run.table = dev(table)
    _expect_edata(run.write, "missing page")
    run.table = dev(case.page_table)
    k = torch.randn(3, 2, 128, device=DEV)
    v = torch.randn(3, 2, 128, device=DEV)
    freq = torch.ones(64, device=DEV)
    pa.kv_page_write_rope(k, v, run.kp, run.vp, run.table, run.owner, run.pos, freq,
                          pa.PA_ROPE_HALVES)
    _expect_edata(lambda: pa.kv_page_write_rope(k, v, run.kp, run.vp, run.table,
                                                dev(np.array([0, 5, 2], np.int32)), run.pos,
                                                freq, pa.PA_ROPE_HALVES), "rope write owner")


def test_prefill_metadata(checked):
    announce("checked build: prefill descriptors and page ids")
    c = _prefill_case()
    desc = c.seg_desc.copy()
    desc[1, 0] = c.q.shape[0]                          # starts past the packed rows
    _expect_edata(lambda: _prefill(c, desc=desc), "descriptor start")
    desc = c.seg_desc.copy()
    desc[1, 1] = 0                                     # an empty segment is valid
    _prefill(c, desc=desc)
    table = c.page_table.copy()
    table[1, 0] = c.k_pages.shape[0] + 7               # a history page of segment 1
    _expect_edata(lambda: _prefill(c, table=table), "page id")
    pa.use_checked_library(False)
    _prefill(c, table=table)                           # the product library clamps: OK


DECODE_NAMES = [n for n, w in wl.WORKLOADS.items() if w.kind == "decode"]
PREFILL_NAMES = [n for n, w in wl.WORKLOADS.items() if w.kind == "prefill"]


@pytest.mark.parametrize("name", DECODE_NAMES + PREFILL_NAMES)
def test_named_workloads_raise_nothing(checked, name):
    """Valid metadata never trips a check: every named workload at full size runs through the
    checked build (write, split partials, merge, and the single-launch step; or the prefill)
    and gives the product library's bits."""
    announce(f"checked build: named workload {name}")
    w = wl.WORKLOADS[name]
    if w.kind == "decode":
        case = wl.workload_decode_case(w)
        got = (DecodeRun(case).step(), DecodeRun(case).fused_step())
        pa.use_checked_library(False)
        ref = (DecodeRun(case).step(), DecodeRun(case).fused_step())
    else:
        c = wl.workload_prefill_case(w)
        got = (_prefill(c),)
        pa.use_checked_library(False)
        ref = (_prefill(c),)
    pa.use_checked_library(True)
    for g, r in zip(got, ref):
        assert_bitwise(g, r, f"{name}: checked vs product")
