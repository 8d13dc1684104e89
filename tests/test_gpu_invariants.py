"""GPU: bit-exact invariants of the HIP path itself.

* context length 1 returns V[0] exactly (exp(0) = 1, sum 1);
* relabelling physical pages changes no bit (paging moves storage, not arithmetic —
  crucible README, "Paged KV cache and continuous batching", Correctness);
* a sequence's output does not depend on its batch companions or their order
  (crucible README, gpu-batch check);
* GQA equals MHA with K/V repeated per group (crucible README, "Tests");
* repeated runs are bit-identical; poisoned never-read bytes never reach an output;
* a prefill segment's rows do not depend on the other segments packed with it;
* sequences of context 0 in a batch give zero rows and leave the other rows unchanged."""
import numpy as np
import pytest
import torch

import paged_gqa_attention_decode_amd as pa
import oracle
from compare import assert_bitwise, assert_within, tolerance
from gpu_helpers import DEV, DecodeRun, announce, dev, host
from paged_gqa_attention_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def f32_values(bits, dtype):
    """Stored cache values as float32 (library conversions; exact for f16 and bf16)."""
    if dtype == "f32":
        return np.asarray(bits, np.float32)
    if dtype == "f16":
        return np.asarray(bits, np.uint16).view(np.float16).astype(np.float32)
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("dtype,hq,hkv,d,S", [("f32", 8, 2, 64, 16), ("f16", 40, 8, 128, 32),
                                               ("bf16", 64, 8, 128, 1), ("bf16", 12, 1, 64, 3)])
def test_ctx1_returns_v0_exactly(dtype, hq, hkv, d, S):
    announce(f"ctx=1 exact {dtype} {hq}/{hkv} d={d} S={S}")
    rng = wl.rng_for([600, hq, d])
    case = wl.make_decode_case(rng, batch=3, hq=hq, hkv=hkv, head_dim=d, page_size=16,
                               dtype=dtype, ctx=[1, 1, 1], num_splits=S)
    out = DecodeRun(case).step()
    expect = np.repeat(f32_values(case.v_new, dtype), hq // hkv, axis=1)
    assert_bitwise(out, expect, "ctx=1")


def _decode(case, S=None, table=None, kp=None, vp=None):
    run = DecodeRun(case, num_splits=S)
    if table is not None:
        run.table = dev(table)
        run.kp = dev(kp, case.dtype)
        run.vp = dev(vp, case.dtype)
    out = run.step()
    return out, host(run.po), host(run.pml)


def test_page_permutation_bitwise():
    announce("page permutation bitwise")
    rng = wl.rng_for(601)
    case = wl.make_decode_case(rng, batch=4, hq=40, hkv=8, head_dim=128, page_size=16,
                               dtype="f16", ctx=[3254, 17, 1000, 129], num_splits=32)
    base = _decode(case)
    pi = rng.permutation(case.k_pages.shape[0])
    kp2 = np.empty_like(case.k_pages)
    vp2 = np.empty_like(case.v_pages)
    kp2[pi] = case.k_pages
    vp2[pi] = case.v_pages
    table2 = np.where(case.page_table >= 0, pi[np.maximum(case.page_table, 0)], -1)
    other = _decode(case, table=table2.astype(np.int32), kp=kp2, vp=vp2)
    for a, b, name in zip(base, other, ("out", "partial_o", "partial_ml")):
        assert_bitwise(a, b, f"page permutation {name}")


@pytest.mark.parametrize("S", [16, 4])
def test_batch_composition_bitwise(S):
    """A sequence's bits do not depend on its batch: alone, batched and in reversed order.
    At 4 splits the batch's 160 workgroups are resident at once, so the 16-bit decode takes it
    longest first (ranked in the kernel); at 16 it runs in grid order."""
    announce(f"batch composition bitwise, {S} splits")
    rng = wl.rng_for(602)
    case = wl.make_decode_case(rng, batch=5, hq=64, hkv=8, head_dim=128, page_size=32,
                               dtype="bf16", ctx=[4096, 64, 1, 2000, 333], num_splits=S)
    full = _decode(case)[0]
    for b in range(5):
        sub = wl.DecodeCase(
            q=case.q[b:b + 1], k_pages=case.k_pages, v_pages=case.v_pages,
            page_table=case.page_table[b:b + 1], context_lens=case.context_lens[b:b + 1],
            k_new=case.k_new[b:b + 1], v_new=case.v_new[b:b + 1],
            token_table_index=np.zeros(1, np.int32), token_position=case.token_position[b:b + 1],
            dtype=case.dtype, scale=case.scale, num_splits=case.num_splits)
        assert_bitwise(_decode(sub)[0][0], full[b], f"sequence {b} alone vs batched")
    order = np.arange(5)[::-1].copy()
    rev = wl.DecodeCase(
        q=case.q[order], k_pages=case.k_pages, v_pages=case.v_pages,
        page_table=case.page_table[order], context_lens=case.context_lens[order],
        k_new=case.k_new[order], v_new=case.v_new[order],
        token_table_index=np.arange(5, dtype=np.int32), token_position=case.token_position[order],
        dtype=case.dtype, scale=case.scale, num_splits=case.num_splits)
    assert_bitwise(_decode(rev)[0][order], full, "reversed batch order")


@pytest.mark.parametrize("g", [4, 5, 7, 8, 12, 33, 64])
def test_gqa_equals_repeated_kv_mha_bitwise(g):
    announce(f"GQA g={g} vs MHA bitwise")
    rng = wl.rng_for([603, g])
    hkv = 2
    case = wl.make_decode_case(rng, batch=2, hq=hkv * g, hkv=hkv, head_dim=128, page_size=16,
                               dtype="f16", ctx=[700, 1641], num_splits=16)
    gqa = _decode(case)[0]
    mha = wl.DecodeCase(
        q=case.q, k_pages=np.repeat(case.k_pages, g, axis=2),
        v_pages=np.repeat(case.v_pages, g, axis=2), page_table=case.page_table,
        context_lens=case.context_lens, k_new=np.repeat(case.k_new, g, axis=1),
        v_new=np.repeat(case.v_new, g, axis=1), token_table_index=case.token_table_index,
        token_position=case.token_position, dtype=case.dtype, scale=case.scale,
        num_splits=case.num_splits)
    assert_bitwise(_decode(mha)[0], gqa, f"GQA g={g} vs MHA")


def test_repeat_runs_bitwise_and_poison_stays_out():
    announce("determinism + poison")
    w = wl.WORKLOADS["decode_hq28_hkv4_d128_ctx1641_f16"]
    case = wl.workload_decode_case(w)
    a = _decode(case)
    b = _decode(case)
    for x, y, name in zip(a, b, ("out", "partial_o", "partial_ml")):
        assert_bitwise(x, y, f"repeat {name}")
    assert np.isfinite(a[0]).all() and np.isfinite(a[1]).all()


@pytest.mark.parametrize("seed,lens,starts", [(604, [17, 64, 129, 257], [0, 63, 255, 512]),
                                              (605, [256, 256, 256, 256], [0, 0, 300, 0])],
                         ids=["histories", "four_256"])
def test_prefill_segment_isolation_bitwise(seed, lens, starts):
    """A segment's rows are identical whether it is prefilled alone or packed with others,
    and whatever its physical pages are.  The four 256-token prompts fill more workgroups
    than two per CU hold at once, so the packed call runs the f32 build budgeted for three
    workgroups per CU and each prompt alone the two-per-CU build: the two must agree."""
    announce(f"prefill segment isolation {lens} {starts}")
    rng = wl.rng_for(seed)
    case = wl.make_prefill_case(rng, hq=12, hkv=3, head_dim=64, page_size=16, dtype="f32",
                                lens=lens, starts=starts)

    def run(c):
        kp, vp = dev(c.k_pages, c.dtype), dev(c.v_pages, c.dtype)
        table = dev(c.page_table)
        pa.kv_page_write(dev(c.k_new, c.dtype), dev(c.v_new, c.dtype), kp, vp, table,
                         dev(c.token_table_index), dev(c.token_position))
        out = torch.zeros(c.q.shape, device=DEV)
        pa.paged_attn_prefill(dev(c.q), kp, vp, table, dev(c.seg_desc), c.max_chunk_len,
                              c.scale, out)
        torch.cuda.synchronize()
        return host(out)

    full = run(case)
    assert np.isfinite(full).all()
    for i in range(len(lens)):
        start, n = int(case.seg_desc[i, 0]), int(case.seg_desc[i, 1])
        rows = slice(start, start + n)
        desc = case.seg_desc[i:i + 1].copy()
        desc[0, 0] = 0
        alone = wl.PrefillCase(
            q=case.q[rows], k_pages=case.k_pages, v_pages=case.v_pages,
            page_table=case.page_table, seg_desc=desc, k_new=case.k_new[rows],
            v_new=case.v_new[rows], token_table_index=case.token_table_index[rows],
            token_position=case.token_position[rows], dtype=case.dtype, scale=case.scale)
        assert_bitwise(run(alone), full[rows], f"segment {i} alone vs packed")


def test_fused_counters_at_any_word_alignment():
    """Each ticket counter has a 128-byte line of its own when the counter buffer starts on
    one; a buffer that starts at any 4-byte offset gives the same bits (only the spacing
    changes), and is left at zero."""
    announce("fused step with an offset counter buffer")
    rng = wl.rng_for(611)
    case = wl.make_decode_case(rng, batch=3, hq=40, hkv=8, head_dim=128, page_size=16,
                               dtype="f16", ctx=[3254, 17, 900], num_splits=32)
    ref = DecodeRun(case, num_splits=32).fused_step()
    run = DecodeRun(case, num_splits=32)
    B, Hq, _ = case.q.shape
    n = pa.paged_attn_decode_fused_counters(B, Hq, case.k_pages.shape[2])
    backing = torch.zeros(n + 7, dtype=torch.int32, device=DEV)
    run.counters = backing[5:5 + n]
    assert run.counters.data_ptr() % 128 != 0
    assert_bitwise(run.fused_step(), ref, "offset counters vs aligned")
    assert_bitwise(run.fused_step(), ref, "offset counters, second call")
    assert int(backing.abs().sum().item()) == 0, "counters must be left at zero"


def test_prefill_segment_order_bitwise():
    """A call with 2..16 segments takes them heaviest first (by last position, ties by
    index).  Any order of the descriptors, with tied segments and an empty descriptor among
    them, gives the same bits, and packed rows that no valid segment covers (gaps, and the
    rows of a descriptor naming a missing table) stay untouched."""
    announce("prefill segment order")
    rng = wl.rng_for(606)
    case = wl.make_prefill_case(rng, hq=12, hkv=3, head_dim=64, page_size=16, dtype="f32",
                                lens=[17, 64, 129, 257, 64], starts=[0, 63, 255, 512, 63],
                                gap_rows=3)
    kp, vp = dev(case.k_pages, case.dtype), dev(case.v_pages, case.dtype)
    table = dev(case.page_table)
    pa.kv_page_write(dev(case.k_new, case.dtype), dev(case.v_new, case.dtype), kp, vp, table,
                     dev(case.token_table_index), dev(case.token_position))
    empty = np.array([[0, 0, 0, 0]], dtype=np.int32)
    # A descriptor naming a table that does not exist, over the gap rows after segment 0: it
    # is skipped, so those rows stay untouched.
    st0, ln0 = int(case.seg_desc[0, 0]), int(case.seg_desc[0, 1])
    bad = np.array([[st0 + ln0, 2, 0, 99]], dtype=np.int32)
    base = np.concatenate([case.seg_desc, empty, bad])

    def run(desc):
        out = torch.full(case.q.shape, float("nan"), device=DEV)
        pa.paged_attn_prefill(dev(case.q), kp, vp, table, dev(np.ascontiguousarray(desc)),
                              case.max_chunk_len, case.scale, out)
        torch.cuda.synchronize()
        return host(out)

    ref = run(base)
    covered = np.zeros(case.q.shape[0], dtype=bool)
    for st, ln, _, _ in case.seg_desc.tolist():
        covered[st:st + ln] = True
    assert np.isfinite(ref[covered]).all() and np.isnan(ref[~covered]).all()
    for perm in ([6, 5, 4, 3, 2, 1, 0], [3, 5, 1, 6, 0, 4, 2], [4, 1, 0, 5, 2, 3, 6]):
        assert_bitwise(run(base[perm]), ref, f"descriptor order {perm}")


@pytest.mark.parametrize("dtype,hq,hkv,d,S", [("f16", 40, 8, 128, 32), ("f32", 12, 3, 64, 7),
                                              ("bf16", 64, 8, 128, 1)])
def test_empty_sequences_in_a_batch(dtype, hq, hkv, d, S):
    """Sequences of context 0 (free slots of a continuous batch) give zero rows and idle
    partials; the other rows are those of the same batch without them, bit for bit; the
    single-launch step agrees with the three-launch step and leaves its counters at zero."""
    announce(f"empty sequences in a batch {dtype} {hq}/{hkv} d={d} S={S}")
    rng = wl.rng_for([606, hq, d])
    ctx = [0, 300, 0, 5]
    case = wl.make_decode_case(rng, batch=4, hq=hq, hkv=hkv, head_dim=d, page_size=16,
                               dtype=dtype, ctx=ctx, num_splits=S)
    run = DecodeRun(case)
    out = run.step()
    po, pml = host(run.po), host(run.pml)
    empty = [0, 2]
    assert np.all(out[empty] == 0.0), "an empty sequence's output must be zero"
    assert np.all(pml[empty][..., 0] == -np.inf) and np.all(pml[empty][..., 1] == 0.0)
    assert np.all(po[empty] == 0.0)
    live = [1, 3]
    sub = wl.DecodeCase(
        q=case.q[live], k_pages=case.k_pages, v_pages=case.v_pages,
        page_table=case.page_table[live], context_lens=case.context_lens[live],
        k_new=case.k_new[live], v_new=case.v_new[live],
        token_table_index=np.arange(2, dtype=np.int32), token_position=case.token_position[live],
        dtype=case.dtype, scale=case.scale, num_splits=case.num_splits)
    assert_bitwise(out[live], DecodeRun(sub).step(), "live rows vs the batch without empties")
    fused = DecodeRun(case)
    got = fused.fused_step()
    assert_bitwise(got, out, "single-launch step vs three launches")
    assert int(fused.counters.abs().sum().item()) == 0, "counters must be left at zero"
    assert_bitwise(host(fused.kp), host(run.kp), "pool after the single-launch write")


def test_fused_step_skips_an_invalid_current_token():
    """The single-launch step stores the current token, and reads it from k_new / v_new, only
    where kv_page_write would store it: a current token whose page id is out of range (batch
    row 0) or whose length is past the table's capacity (row 1) is neither stored nor read
    from k_new / v_new.  Outputs and both pools then equal those of the three-launch step
    bit for bit, and the invalid rows' pool bytes are left as they were."""
    announce("single-launch step with an invalid current-token page id and length")
    rng = wl.rng_for(611)
    ctx = [100, 64, 37]
    case = wl.make_decode_case(rng, batch=3, hq=16, hkv=2, head_dim=128, page_size=16,
                               dtype="bf16", ctx=ctx, num_splits=4, poison=False)
    P = case.k_pages.shape[0]
    cap = case.page_table.shape[1] * 16
    case.page_table[0, (ctx[0] - 1) // 16] = P               # out-of-range page id
    case.context_lens[1] = cap + 5                            # past the table's capacity
    case.token_position[:] = case.context_lens - 1
    three = DecodeRun(case)
    out3 = three.step()
    one = DecodeRun(case)
    out1 = one.fused_step()
    assert_bitwise(out1, out3, "single launch vs three launches")
    assert_bitwise(host(one.kp), host(three.kp), "K pool: single launch vs three launches")
    assert_bitwise(host(one.vp), host(three.vp), "V pool: single launch vs three launches")
    # Only row 2's current slot changed.
    p2 = case.page_table[2, (ctx[2] - 1) // 16]
    for name, pool, before, new in (("K", one.kp, case.k_pages, case.k_new),
                                    ("V", one.vp, case.v_pages, case.v_new)):
        after = host(pool)
        expect = before.copy()
        expect[p2, (ctx[2] - 1) % 16] = new[2]
        assert_bitwise(after, expect, f"{name} pool: only the valid row's slot is written")
    assert int(one.counters.abs().sum().item()) == 0, "counters must be left at zero"


def test_ranked_batch_with_ties_and_free_slots():
    """A batch the 16-bit decode ranks by length (here 12 sequences at 4 splits, resident at
    once): equal lengths, free slots (length 0) and the longest possible length in one batch.
    Every sequence equals its own single-sequence call bit for bit, the single-launch step
    equals the three launches, and the results match the oracle."""
    announce("ranked batch: ties, free slots")
    rng = wl.rng_for(607)
    ctx = [300, 0, 300, 1024, 1, 300, 0, 777, 1024, 2, 300, 64]
    case = wl.make_decode_case(rng, batch=12, hq=16, hkv=4, head_dim=128, page_size=16,
                               dtype="f16", ctx=ctx, max_pages_per_seq=64, num_splits=4)
    run = DecodeRun(case)
    out = run.step()
    assert_bitwise(DecodeRun(case).fused_step(), out, "single launch vs three")
    live = case.context_lens > 0
    assert np.all(out[~live] == 0.0), "free slots give zero rows"
    kp, vp = oracle.kv_write(case.k_new, case.v_new, case.k_pages, case.v_pages, case.dtype,
                             case.page_table, case.token_table_index, case.token_position)
    ref = oracle.decode(case.q[live], kp, vp, case.dtype, case.page_table[live],
                        case.context_lens[live], case.scale)
    assert_within(out[live], ref, *tolerance(case.dtype), "ranked batch vs the oracle")
    for b in np.flatnonzero(live):
        sub = wl.DecodeCase(
            q=case.q[b:b + 1], k_pages=case.k_pages, v_pages=case.v_pages,
            page_table=case.page_table[b:b + 1], context_lens=case.context_lens[b:b + 1],
            k_new=case.k_new[b:b + 1], v_new=case.v_new[b:b + 1],
            token_table_index=np.zeros(1, np.int32), token_position=case.token_position[b:b + 1],
            dtype=case.dtype, scale=case.scale, num_splits=case.num_splits)
        assert_bitwise(DecodeRun(sub).step()[0], out[b], f"sequence {b} alone vs ranked batch")
