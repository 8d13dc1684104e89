"""CPU: the seeded input generator is deterministic and poisons exactly the bytes no call
may read."""
import numpy as np

from paged_gqa_attention_decode_amd import workloads as wl


def test_named_workloads_shapes():
    w = wl.WORKLOADS
    assert w["decode_hq8_hkv2_d64_ctx256_f32"].group == 4
    assert w["decode_hq40_hkv8_d128_ctx3254_f16"].group == 5
    assert w["decode_hq28_hkv4_d128_ctx1641_f16"].group == 7
    assert w["decode_b16_hq64_hkv8_d128_ctx64to4096_bf16"].group == 8
    assert w["prefill_hq12_hkv12_d64_t512_f32"].attn_scale == 0.125
    assert w["decode_hq40_hkv8_d128_ctx3254_f16"].attn_scale == np.float32(1 / np.sqrt(128))


def test_deterministic():
    w = wl.WORKLOADS["decode_hq8_hkv2_d64_ctx256_f32"]
    a = wl.workload_decode_case(w)
    b = wl.workload_decode_case(w)
    for name in ("q", "k_pages", "v_pages", "page_table", "context_lens", "k_new"):
        assert np.array_equal(getattr(a, name).view(np.uint8), getattr(b, name).view(np.uint8))


def test_decode_poison_exact():
    w = wl.WORKLOADS["decode_hq8_hkv2_d64_ctx256_f32"]
    c = wl.workload_decode_case(w)
    # 16 pages x 16 slots; positions 0..254 live, 255 (the current token) poisoned
    live = ~np.isnan(c.k_pages[:, :, 0, 0])
    assert live.sum() == 255
    assert sorted(c.page_table[0].tolist()) == list(range(16))
    last = c.page_table[0, 255 // 16]
    assert np.isnan(c.k_pages[last, 15]).all() and np.isnan(c.v_pages[last, 15]).all()


def test_batch16_contexts_and_rotations():
    w = wl.WORKLOADS["decode_b16_hq64_hkv8_d128_ctx64to4096_bf16"]
    rng = wl.named_rng(w.index)
    c = wl.make_decode_case(rng, batch=2, hq=16, hkv=2, head_dim=128, page_size=32,
                            dtype="bf16", ctx_range=(64, 4096), num_pages=1024, rotations=3,
                            poison=False)
    assert c.page_table.shape == (2, 128)
    assert all(64 <= x <= 4096 for x in c.context_lens)
    used = [set(t[t >= 0].tolist()) for t in [c.page_table] + c.extra_tables]
    assert not (used[0] & used[1]) and not (used[1] & used[2]), "rotations must be disjoint"


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-3], np.float32)
    bits = wl.f32_to_bf16_bits(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: rounds to the even mantissa (1.0)
    assert bits[1] == 0x3F80
    # 1 + 3*2^-8 is a tie between 1+2^-7 and 1+2^-6: rounds to the even one (1 + 2^-6)
    assert bits[2] == 0x3F82
    assert bits[0] == 0x3F80 and bits[3] == 0xC020


def test_prefill_case_layout():
    rng = wl.rng_for(7)
    c = wl.make_prefill_case(rng, hq=4, hkv=2, head_dim=64, page_size=16, dtype="f16",
                             lens=[17, 5], starts=[0, 30], gap_rows=3)
    assert c.seg_desc.tolist() == [[0, 17, 0, 0], [20, 5, 30, 1]]
    assert (c.token_table_index[17:20] == -1).all()
    assert c.token_position[20:25].tolist() == [30, 31, 32, 33, 34]
    # history of segment 1 (positions 0..29) is live; its chunk slots are poisoned
    t1 = c.page_table[1]
    live = ~np.isnan(c.k_pages.view(np.float16)[:, :, 0, 0])
    assert live.sum() == 30
    assert live[t1[0]].all() and live[t1[1], :14].all() and not live[t1[1], 14:].any()


def test_prefill_benchmark_packs_match_the_printed_extents():
    """The three prefill measurement packs are the pages' shapes: their sums of causal
    positions equal the values the crucible results page prints (tests/golden)."""
    printed = {}
    with open(__file__.replace("test_workloads.py", "golden/causal_positions.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, _, _, total = [x.strip() for x in line.split("|")]
            printed[name] = int(total)
    for wname, shape in (("prefill_hq12_hkv3_d64_t512_f32", "single-512"),
                         ("prefill_hq12_hkv3_d64_4x256_f32", "4x256"),
                         ("prefill_hq12_hkv3_d64_hetero_f32", "heterogeneous")):
        c = wl.workload_prefill_case(wl.WORKLOADS[wname], poison=False)
        total = sum(int(a0) * int(n) + int(n) * (int(n) + 1) // 2
                    for _, n, a0, _ in c.seg_desc.tolist())
        assert total == printed[shape], (wname, total, printed[shape])
        assert c.q.shape[0] == c.seg_desc[:, 1].sum()


def test_c4_rotations_exceed_the_last_level_cache():
    w = wl.WORKLOADS["decode_hq28_hkv4_d128_ctx1641_f16"]
    c = wl.workload_decode_case(w, poison=False)
    assert len(c.extra_tables) + 1 == 4
    used = [set(t[t >= 0].tolist()) for t in [c.page_table] + c.extra_tables]
    assert all(not (used[i] & used[j]) for i in range(4) for j in range(i + 1, 4))
    per_layer = 4 * 103 * 16 * 4 * 128 * 2 * 2       # 4 page sets, K and V, f16
    assert w.layers * per_layer > 256 * 2**20
