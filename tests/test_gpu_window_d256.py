"""GPU: sliding-window decode and head_dim 256 (vllm.cpp PR #383: the decode kernel's windowed
arm and its head_dim-256 instantiation) against the f64 oracle, through the C ABI.

Bars as for every decode: |gpu - ref| <= 1e-5 for f32 K/V, <= 2e-3 + 1e-2 |ref| for f16/bf16;
the current token's page write bit-exact; split partials compared as (m, l, O/l) under the
same partition rule (the splits partition the attended positions); the single-launch step
bit-identical to write -> split decode -> merge, and its counters left at zero."""
import numpy as np
import pytest
import torch

import oracle
import paged_gqa_attention_decode_amd as pa
from compare import assert_bitwise, assert_within, tolerance
from gpu_helpers import DEV, DecodeRun, announce, dev, host
from paged_gqa_attention_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

BOUNDARY_CTX = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 255, 256, 257,
                511, 512, 685, 941, 1000, 1023, 1024, 1919, 1920, 1921, 2807, 2808, 3254,
                4095, 4096]


def oracle_step(case, window):
    kp, vp = oracle.kv_write(case.k_new, case.v_new, case.k_pages, case.v_pages, case.dtype,
                             case.page_table, case.token_table_index, case.token_position)
    out = oracle.decode(case.q, kp, vp, case.dtype, case.page_table, case.context_lens,
                        case.scale, window=window)
    return kp, vp, out


def check(case, S, window, what, fused=True):
    run = DecodeRun(case, num_splits=S, window=window)
    out = run.step()
    kp, vp, ref = oracle_step(case, window)
    assert_bitwise(host(run.kp), kp, f"{what}: K pool after the write")
    atol, rtol = tolerance(case.dtype)
    assert_within(out, ref, atol, rtol, f"{what}: output")
    # partials under the windowed partition
    po = host(run.po).astype(np.float64)
    pml = host(run.pml).astype(np.float64)
    ro, rm, rl = oracle.decode_partials(case.q, kp, vp, case.dtype, case.page_table,
                                        case.context_lens, case.scale, S, window=window)
    m, l = pml[..., 0], pml[..., 1]
    idle = rl == 0
    assert np.array_equal(l == 0, idle), f"{what}: idle-split pattern differs"
    live = ~idle
    assert_within(m[live], rm[live], 1e-4, 1e-6, f"{what}: split max m")
    assert_within(l[live], rl[live], 0.0, 2e-4, f"{what}: split sum l")
    assert_within(po[live] / l[live][:, None], ro[live] / rl[live][:, None], atol, rtol,
                  f"{what}: split O/l")
    if fused:
        f = DecodeRun(case, num_splits=S, window=window)
        fo = f.fused_step()
        assert_bitwise(fo, out, f"{what}: single-launch step vs three launches")
        assert_bitwise(host(f.kp), kp, f"{what}: K pool after the fused write")
        assert int(f.counters.abs().sum().item()) == 0, f"{what}: counters left at zero"


@pytest.mark.parametrize("geom", [
    # hq, hkv, d, ps, dtype, S, window
    (40, 8, 128, 16, "f16", 32, 1),
    (40, 8, 128, 16, "f16", 32, 100),
    (40, 8, 128, 16, "f16", 32, 1000),
    (28, 4, 128, 16, "f16", 8, 4096),
    (64, 8, 128, 32, "bf16", 8, 512),
    (8, 2, 64, 16, "f32", 16, 33),
    (12, 12, 64, 1, "f32", 4, 257),
], ids=lambda g: "hq{}_hkv{}_d{}_ps{}_{}_S{}_w{}".format(*g))
def test_window_boundary_lengths(geom):
    hq, hkv, d, ps, dtype, S, w = geom
    announce(f"window decode {geom}")
    rng = wl.rng_for([500, hq, hkv, d, ps, w])
    ctx = BOUNDARY_CTX if ps > 1 else [c for c in BOUNDARY_CTX if c <= 1100]
    case = wl.make_decode_case(rng, batch=len(ctx), hq=hq, hkv=hkv, head_dim=d, page_size=ps,
                               dtype=dtype, ctx=ctx, num_splits=S)
    check(case, S, w, f"window {geom}")


@pytest.mark.parametrize("geom", [
    # hq, hkv, ps, dtype, S, window
    (16, 8, 16, "bf16", 16, 0),        # GQA group 2
    (32, 4, 16, "f16", 8, 0),          # group 8: two head groups of 4 per KV head
    (20, 4, 32, "bf16", 4, 0),         # group 5: head groups of 3 and 2
    (4, 4, 16, "bf16", 32, 0),         # MHA
    (16, 8, 16, "bf16", 16, 700),      # windowed
], ids=lambda g: "d256_hq{}_hkv{}_ps{}_{}_S{}_w{}".format(*g))
def test_head_dim_256(geom):
    hq, hkv, ps, dtype, S, w = geom
    announce(f"head_dim 256 decode {geom}")
    rng = wl.rng_for([510, hq, hkv, ps, w])
    ctx = [c for c in BOUNDARY_CTX if c <= 2808]
    case = wl.make_decode_case(rng, batch=len(ctx), hq=hq, hkv=hkv, head_dim=256, page_size=ps,
                               dtype=dtype, ctx=ctx, num_splits=S)
    check(case, S, w, f"d256 {geom}")


def test_head_dim_256_gqa_equals_mha_bitwise():
    """A query head's result is bit-identical whether its KV head serves 8 query heads or,
    with K/V repeated per group, just one (head_dim 256)."""
    rng = wl.rng_for(520)
    hq, hkv, d, ps = 16, 2, 256, 16
    case = wl.make_decode_case(rng, batch=3, hq=hq, hkv=hkv, head_dim=d, page_size=ps,
                               dtype="bf16", ctx=[1, 700, 2049], num_splits=8)
    announce("head_dim 256 GQA == MHA")
    gqa = DecodeRun(case).step()
    g = hq // hkv
    mha = wl.make_decode_case(rng, batch=3, hq=hq, hkv=hq, head_dim=d, page_size=ps,
                              dtype="bf16", ctx=[1, 700, 2049], num_splits=8)
    mha.q[:] = case.q
    mha.k_pages = np.repeat(case.k_pages, g, axis=2)
    mha.v_pages = np.repeat(case.v_pages, g, axis=2)
    mha.k_new = np.repeat(case.k_new, g, axis=1)
    mha.v_new = np.repeat(case.v_new, g, axis=1)
    mha.page_table = case.page_table.copy()
    mha.context_lens = case.context_lens.copy()
    mha.token_table_index = case.token_table_index.copy()
    mha.token_position = case.token_position.copy()
    out = DecodeRun(mha).step()
    assert_bitwise(out, gqa, "head_dim 256: GQA == MHA with K/V repeated")


@pytest.mark.parametrize("S", [1, 16, 33])
def test_combine_head_dim_256(S):
    announce(f"combine d=256 S={S}")
    rng = wl.rng_for([530, S])
    o, ml = wl.make_partials(rng, batch=3, hq=16, head_dim=256, num_splits=S, all_empty_rows=2)
    ref = oracle.combine(o, ml[..., 0], ml[..., 1])
    out = torch.full((3, 16, 256), float("nan"), device=DEV)
    pa.paged_attn_combine(dev(o), dev(ml), out)
    torch.cuda.synchronize()
    assert_within(host(out), ref, 1e-5, 0.0, f"combine d=256 S={S}")
