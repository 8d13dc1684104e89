"""GPU: seeded random configurations over the supported space, each against the oracle.

Decode draws the pool dtype, head_dim (256 with 16-bit pools only), the group size, the page
size, the split count, a sliding window or none, and a batch of mixed context lengths
(empty sequences included); the single-launch step must also give the three-launch step's
bits.  Prefill draws packs of segments with histories, GQA, dtypes and page sizes.  Every
configuration is valid input; the draws are fixed by the case index, so a failure names a
reproducible case."""
import numpy as np
import pytest
import torch

import oracle
import paged_gqa_attention_decode_amd as pa
from compare import assert_bitwise, assert_within, second_bar, tolerance
from gpu_helpers import DEV, DecodeRun, announce, dev, host
from paged_gqa_attention_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _decode_config(i):
    r = np.random.default_rng([20260908, 900, i])
    dtype = ["f32", "f16", "bf16"][r.integers(3)]
    d = [64, 128, 256, 256][r.integers(4)] if dtype != "f32" else [64, 128][r.integers(2)]
    hkv = int(r.choice([1, 2, 4, 8]))
    g = int(r.choice([1, 2, 3, 4, 5, 7, 8, 12, 16]))
    ps = int(r.choice([1, 4, 16, 32, 128]))
    S = int(r.choice([1, 3, 8, 16, 32, 100]))
    batch = int(r.integers(1, 5))
    ctx = [int(c) for c in r.integers(1, 700, size=batch)]
    ctx = [ctx[0]] + [0 if r.random() < 0.2 else n for n in ctx[1:]]   # some free slots
    window = int(r.choice([0, 0, 0, 1, 37, 100, 256, 1000]))
    return dict(dtype=dtype, d=d, hkv=hkv, hq=hkv * g, ps=ps, S=S, ctx=ctx, window=window)


def _prefill_config(i):
    r = np.random.default_rng([20260908, 901, i])
    dtype = ["f32", "f16", "bf16"][r.integers(3)]
    d = [64, 128][r.integers(2)]
    hkv = int(r.choice([1, 2, 3, 4]))
    g = int(r.choice([1, 2, 3, 4, 8]))
    ps = int(r.choice([1, 8, 16, 64]))
    nseg = int(r.integers(1, 4))
    lens = [int(x) for x in r.integers(1, 160, size=nseg)]
    starts = [int(x) for x in r.integers(0, 300, size=nseg)]
    gap = int(r.integers(0, 3))
    return dict(dtype=dtype, d=d, hkv=hkv, hq=hkv * g, ps=ps, lens=lens, starts=starts,
                gap=gap)


@pytest.mark.parametrize("i", range(48))
def test_random_decode(i):
    c = _decode_config(i)
    announce(f"random decode {i}: {c}")
    rng = wl.rng_for([902, i])
    case = wl.make_decode_case(rng, batch=len(c["ctx"]), hq=c["hq"], hkv=c["hkv"],
                               head_dim=c["d"], page_size=c["ps"], dtype=c["dtype"],
                               ctx=c["ctx"], num_splits=c["S"], window=c["window"])
    run = DecodeRun(case)
    out = run.step()
    kp, vp = oracle.kv_write(case.k_new, case.v_new, case.k_pages, case.v_pages, case.dtype,
                             case.page_table, case.token_table_index, case.token_position)
    live = [b for b, n in enumerate(c["ctx"]) if n > 0]
    ref = oracle.decode(case.q[live], kp, vp, case.dtype, case.page_table[live],
                        case.context_lens[live], case.scale, window=c["window"])
    assert_within(out[live], ref, *tolerance(case.dtype), f"random decode {i}")
    assert_within(out[live], ref, *second_bar(case.dtype), f"random decode {i}, second bar")
    empty = [b for b, n in enumerate(c["ctx"]) if n == 0]
    assert np.all(out[empty] == 0.0), "empty sequences give zero rows"
    fused = DecodeRun(case).fused_step()
    assert_bitwise(fused, out, f"random decode {i}: single launch vs three launches")


@pytest.mark.parametrize("i", range(32))
def test_random_prefill(i):
    c = _prefill_config(i)
    announce(f"random prefill {i}: {c}")
    rng = wl.rng_for([903, i])
    case = wl.make_prefill_case(rng, hq=c["hq"], hkv=c["hkv"], head_dim=c["d"],
                                page_size=c["ps"], dtype=c["dtype"], lens=c["lens"],
                                starts=c["starts"], gap_rows=c["gap"])
    kp, vp = dev(case.k_pages, case.dtype), dev(case.v_pages, case.dtype)
    table = dev(case.page_table)
    pa.kv_page_write(dev(case.k_new, case.dtype), dev(case.v_new, case.dtype), kp, vp, table,
                     dev(case.token_table_index), dev(case.token_position))
    out = torch.full(case.q.shape, 7.0, device=DEV)
    pa.paged_attn_prefill(dev(case.q), kp, vp, table, dev(case.seg_desc), case.max_chunk_len,
                          case.scale, out)
    torch.cuda.synchronize()
    got = host(out)
    rk, rv = oracle.kv_write(case.k_new, case.v_new, case.k_pages, case.v_pages, case.dtype,
                             case.page_table, case.token_table_index, case.token_position)
    ref, _ = oracle.prefill(case.q, rk, rv, case.dtype, case.page_table, case.seg_desc,
                            case.scale)
    covered = case.token_table_index >= 0
    assert np.all(got[~covered] == 7.0), "rows outside every segment stay untouched"
    assert_within(got[covered], ref[covered], *tolerance(case.dtype), f"random prefill {i}")


@pytest.mark.parametrize("g,hkv,d", [(9, 1, 128), (25, 1, 128), (19, 2, 64), (33, 1, 128),
                                     (60, 1, 64), (9, 1, 256)])
def test_decode_group_sizes_split_over_head_groups(g, hkv, d):
    """Group sizes whose query heads the host spreads over several workgroups when the grid
    would leave compute units idle (batch 1, few splits): every head is computed once and
    matches the oracle, and the single-launch step gives the same bits."""
    announce(f"decode group size {g} hkv={hkv} d={d}")
    rng = wl.rng_for([904, g, hkv, d])
    case = wl.make_decode_case(rng, batch=1, hq=g * hkv, hkv=hkv, head_dim=d, page_size=16,
                               dtype="bf16", ctx=[421], num_splits=3)
    out = DecodeRun(case).step()
    kp, vp = oracle.kv_write(case.k_new, case.v_new, case.k_pages, case.v_pages, case.dtype,
                             case.page_table, case.token_table_index, case.token_position)
    ref = oracle.decode(case.q, kp, vp, case.dtype, case.page_table, case.context_lens,
                        case.scale)
    assert_within(out, ref, *tolerance(case.dtype), f"group {g}")
    assert_bitwise(DecodeRun(case).fused_step(), out, f"group {g}: single launch vs three")
