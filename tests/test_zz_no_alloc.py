"""GPU: paged_attn_decode_fused_noalloc, the single-launch decode step whose split workspace is
the library's fixed per-GPU array, against paged_attn_decode_fused with caller buffers.

Calls in a row on one GPU, each with a smaller problem than the one before (so the array
holds the previous call's partials and a different counter layout when the next one runs),
over both decode bodies and a batch the matrix-core body ranks:
each must give paged_attn_decode_fused's output and pools bit for bit, and the smaller ones
also match the oracle within their tolerance.  A call whose workspace exceeds the
array is rejected with PA_ESCRATCH before anything is enqueued."""
import numpy as np
import pytest
import torch

import oracle
import paged_gqa_attention_decode_amd as pa
from compare import assert_bitwise, assert_within, tolerance
from gpu_helpers import DEV, DecodeRun, announce, host
from paged_gqa_attention_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _noalloc_step(case):
    run = DecodeRun(case)
    B, Hq, D = case.q.shape
    out = torch.full((B, Hq, D), float("nan"), device=DEV)
    pa.paged_attn_decode_fused_noalloc(run.q, run.k_new, run.v_new, run.kp, run.vp, run.table,
                                       run.ctx, case.scale, run.S, out, window=run.window)
    torch.cuda.synchronize()
    return host(out), host(run.kp), host(run.vp)


def _fused_step(case):
    run = DecodeRun(case)
    out = run.fused_step()
    return out, host(run.kp), host(run.vp)


def test_noalloc_step_equals_fused_step_on_calls_in_a_row():
    first = wl.make_decode_case(wl.rng_for(950), batch=16, hq=64, hkv=8, head_dim=128,
                                page_size=32, dtype="bf16", ctx_range=(64, 4096),
                                num_pages=2048, num_splits=16)
    second = wl.make_decode_case(wl.rng_for(951), batch=3, hq=40, hkv=8, head_dim=128,
                                 page_size=16, dtype="f16", ctx=[3254, 17, 900], num_splits=32)
    # a third, smaller still, on an f32 pool (the vector-unit decode body)
    third = wl.make_decode_case(wl.rng_for(955), batch=2, hq=8, hkv=2, head_dim=64,
                                page_size=16, dtype="f32", ctx=[256, 31], num_splits=4)
    # a fourth, the smallest: a bf16 batch whose grid is resident at once, so the matrix-core
    # body ranks it (longest first)
    fourth = wl.make_decode_case(wl.rng_for(956), batch=2, hq=8, hkv=2, head_dim=64,
                                 page_size=16, dtype="bf16", ctx=[45, 300], num_splits=2)
    cases = (first, second, third, fourth)
    sizes = [pa.paged_attn_decode_workspace_bytes(c.q.shape[0], c.q.shape[1], c.q.shape[2],
                                                  c.num_splits) for c in cases]
    assert sizes[3] < sizes[2] < sizes[1] < sizes[0] <= pa.paged_attn_noalloc_scratch_bytes()
    for name, case in (("first (batch 16, 16 splits)", first), ("second (batch 3)", second),
                       ("third (f32, batch 2)", third), ("fourth (ranked bf16, batch 2)", fourth)):
        announce(f"no-alloc decode step, {name}")
        got, gk, gv = _noalloc_step(case)
        ref, rk, rv = _fused_step(case)
        assert_bitwise(got, ref, f"{name}: output")
        assert_bitwise(gk, rk, f"{name}: K pool")
        assert_bitwise(gv, rv, f"{name}: V pool")
        if case is not first:
            kp, vp = oracle.kv_write(case.k_new, case.v_new, case.k_pages, case.v_pages,
                                     case.dtype, case.page_table, case.token_table_index,
                                     case.token_position)
            want = oracle.decode(case.q, kp, vp, case.dtype, case.page_table,
                                 case.context_lens, case.scale)
            assert_within(got, want, *tolerance(case.dtype), f"{name} vs the oracle")


def test_noalloc_step_rejects_a_workspace_larger_than_the_array():
    announce("no-alloc decode step: oversize rejection")
    case = wl.make_decode_case(wl.rng_for(952), batch=2, hq=8, hkv=2, head_dim=64,
                               page_size=16, dtype="f32", ctx=[40, 7], num_splits=2)
    run = DecodeRun(case)
    out = torch.zeros(2, 8, 64, device=DEV)
    # 4096 splits x 2 sequences x 8 heads x 66 floats = 17.3 MB > 16 MiB.
    with pytest.raises(pa.PagedAttnError) as err:
        pa.paged_attn_decode_fused_noalloc(run.q, run.k_new, run.v_new, run.kp, run.vp,
                                           run.table, run.ctx, case.scale, 4096, out)
    assert err.value.status == pa.PA_ESCRATCH
    torch.cuda.synchronize()
    assert np.all(host(out) == 0.0), "a rejected call writes nothing"


def test_noalloc_step_in_a_graph():
    """The use the entry is for: captured once into a HIP graph (no allocation in the call)
    and replayed three times, with eager work between the replays (another no-allocation
    call on a different problem, which overwrites the array's partials); every replay equals
    the eager single-launch step bit for bit."""
    announce("no-alloc decode step captured in a graph")
    case = wl.make_decode_case(wl.rng_for(953), batch=4, hq=40, hkv=8, head_dim=128,
                               page_size=16, dtype="f16", ctx=[3254, 1, 640, 2049],
                               num_splits=32)
    other = wl.make_decode_case(wl.rng_for(954), batch=2, hq=64, hkv=8, head_dim=128,
                                page_size=32, dtype="bf16", ctx=[4000, 77], num_splits=8)
    eager, _, _ = _fused_step(case)
    _noalloc_step(other)  # the array's address is looked up here, outside the capture

    run = DecodeRun(case)
    B, Hq, D = case.q.shape
    out = torch.full((B, Hq, D), float("nan"), device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            pa.paged_attn_decode_fused_noalloc(run.q, run.k_new, run.v_new, run.kp, run.vp,
                                               run.table, run.ctx, case.scale, run.S, out)
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_bitwise(host(out), eager, f"replay {i}")
        _noalloc_step(other)
