"""GPU: the entry points captured in HIP graphs on a side stream.

A serving loop captures a decode step (or a prefill) once and replays it.  Each graph here is
replayed three times with the program's own eager work and synchronisations between the
replays, and every replay must equal the eager result bit for bit.  The single-launch decode
step keeps its only state in the caller's counters, which every call leaves at zero, so it
needs no clearing node in the graph."""
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


def _eager_noise(run):
    """Unrelated eager work between replays: the three-launch step on the same case (it
    writes the same current token, so the pool it leaves is the one the graph expects)."""
    run.step()
    x = torch.randn(1 << 20, device=DEV)
    (x * 2.0).sum().item()


@pytest.mark.parametrize("dtype,hq,hkv,d,S", [("f16", 40, 8, 128, 32), ("bf16", 64, 8, 128, 8),
                                               ("f32", 8, 2, 64, 16), ("f16", 40, 8, 128, 1)])
def test_decode_fused_step_in_a_graph(dtype, hq, hkv, d, S):
    announce(f"graph: single-launch decode {dtype} {hq}/{hkv} d={d} S={S}")
    rng = wl.rng_for([700, hq, d])
    case = wl.make_decode_case(rng, batch=3, hq=hq, hkv=hkv, head_dim=d, page_size=16,
                               dtype=dtype, ctx=[100, 1000, 37], num_splits=S)
    eager = DecodeRun(case).fused_step()

    run = DecodeRun(case)
    noise = DecodeRun(case)
    B, Hq, D = case.q.shape
    run.counters = torch.zeros(pa.paged_attn_decode_fused_counters(B, Hq, hkv),
                               dtype=torch.int32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            pa.paged_attn_decode_fused(run.q, run.k_new, run.v_new, run.kp, run.vp, run.table,
                                       run.ctx, case.scale, run.po, run.pml, run.counters,
                                       run.out)
    torch.cuda.synchronize()
    for i in range(3):
        run.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_bitwise(host(run.out), eager, f"replay {i}")
        assert int(run.counters.abs().sum().item()) == 0, "counters must be left at zero"
        _eager_noise(noise)
    assert_bitwise(host(noise.out), eager, "three-launch step between replays")


def test_write_and_prefill_in_a_graph():
    announce("graph: kv_page_write + prefill")
    rng = wl.rng_for(701)
    c = wl.make_prefill_case(rng, hq=12, hkv=3, head_dim=64, page_size=16, dtype="bf16",
                             lens=[17, 64, 129], starts=[0, 63, 255])

    def buffers():
        return dict(kp=dev(c.k_pages, c.dtype), vp=dev(c.v_pages, c.dtype),
                    table=dev(c.page_table), kn=dev(c.k_new, c.dtype), vn=dev(c.v_new, c.dtype),
                    owner=dev(c.token_table_index), pos=dev(c.token_position), q=dev(c.q),
                    desc=dev(c.seg_desc), out=torch.full(c.q.shape, 7.0, device=DEV))

    def launch(b):
        pa.kv_page_write(b["kn"], b["vn"], b["kp"], b["vp"], b["table"], b["owner"], b["pos"])
        pa.paged_attn_prefill(b["q"], b["kp"], b["vp"], b["table"], b["desc"], c.max_chunk_len,
                              c.scale, b["out"])

    ref = buffers()
    launch(ref)
    torch.cuda.synchronize()
    eager_out, eager_k = host(ref["out"]), host(ref["kp"])

    b = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            launch(b)
    torch.cuda.synchronize()
    for i in range(3):
        b["out"].fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_bitwise(host(b["out"]), eager_out, f"prefill replay {i}")
        assert_bitwise(host(b["kp"]), eager_k, f"pool after replay {i}")
        launch(buffers())               # eager work between replays
        torch.cuda.synchronize()
