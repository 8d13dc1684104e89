"""Seeded synthetic inputs for paged GQA attention.

This module only draws and lays out inputs; it computes nothing of the attention method.
Both the HIP path and the f64 oracle receive the arrays it returns, so neither side's
arithmetic can leak into the other's inputs.

Recipe (every case):
  * ``numpy.random.Generator(PCG64)`` from a ``SeedSequence``: the five named workloads use
    ``SeedSequence(20260908).spawn(5)`` (20260908 is the master tensor seed of the crucible
    paged-attention results page), other cases ``SeedSequence([20260908, case_id])``.
  * Draw order: q, K pool, V pool, page permutation, context lengths, new K rows, new V rows.
  * Values ~ N(0, 1) drawn in float32, then rounded to nearest-even into the cache dtype
    (f16 through numpy, bf16 by the usual carry-and-truncate on the f32 bit pattern).
    Normal data is mantissa-dense: it avoids the false pass that small integers give
    (crucible README, "Validation": two ways the test passed for the wrong reason).
  * Physical pages are a random permutation of the pool, so logically adjacent pages are
    never physically adjacent (crucible results: independently shuffled physical maps).
  * ``poison=True`` fills every byte no call may read with NaN: pages owned by nobody,
    slots past each sequence's last position, the current token's slot (its K/V arrives
    through ``kv_page_write``), and page-table entries past the last used page get -1.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

MASTER_SEED = 20260908

NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0}


# --------------------------------------------------------------------------- storage dtypes

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to nearest-even bfloat16; return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values -> the pool's storage array (float32, or uint16 bit patterns)."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return f32_to_f16_bits(x)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def nan_value(dtype: str):
    return np.float32(np.nan) if dtype == "f32" else np.uint16(NAN_BITS[dtype])


def storage_dtype(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


def _normal_pool(rng, shape, dtype, chunk_pages=256):
    """N(0,1) pool drawn page-chunk by page-chunk (same stream as one draw, less memory)."""
    out = np.empty(shape, dtype=storage_dtype(dtype))
    for p0 in range(0, shape[0], chunk_pages):
        p1 = min(shape[0], p0 + chunk_pages)
        out[p0:p1] = to_storage(rng.standard_normal((p1 - p0,) + tuple(shape[1:]),
                                                    dtype=np.float32), dtype)
    return out


def rng_for(case_id) -> np.random.Generator:
    ss = np.random.SeedSequence([MASTER_SEED] + list(np.atleast_1d(case_id).astype(np.int64)))
    return np.random.Generator(np.random.PCG64(ss))


def named_rng(index: int) -> np.random.Generator:
    ss = np.random.SeedSequence(MASTER_SEED).spawn(16)[index]  # child i does not depend on n
    return np.random.Generator(np.random.PCG64(ss))


# --------------------------------------------------------------------------- named workloads

@dataclass(frozen=True)
class Workload:
    """One of the five seeded workloads of this method."""
    name: str
    kind: str                  # "decode" or "prefill"
    index: int                 # SeedSequence child index
    hq: int
    hkv: int
    head_dim: int
    page_size: int
    dtype: str                 # cache dtype; q and outputs are always f32
    batch: int = 1
    ctx: tuple = ()            # fixed decode contexts (empty: drawn from ctx_range)
    ctx_range: tuple = ()      # inclusive [lo, hi] for drawn contexts
    num_pages: int = 0         # pool size (0: exactly the pages the sequences need)
    num_splits: int = 1
    tokens: int = 0            # prefill: packed query rows
    layers: int = 1            # layers per model step (decode step = all layers)
    scale: float = 0.0         # 0: 1/sqrt(head_dim) rounded to f32
    rotations: int = 1         # disjoint page sets the bench cycles through
    window: int = 0            # decode: sliding window in positions (0: whole context)
    seg_lens: tuple = ()       # prefill: chunk lengths of a multi-segment pack (else `tokens`)
    seg_starts: tuple = ()     # prefill: absolute start of each segment
    description: str = ""

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def attn_scale(self) -> float:
        return float(np.float32(self.scale if self.scale else 1.0 / math.sqrt(self.head_dim)))


WORKLOADS = {
    "decode_hq8_hkv2_d64_ctx256_f32": Workload(
        name="decode_hq8_hkv2_d64_ctx256_f32", kind="decode", index=0, hq=8, hkv=2,
        head_dim=64, page_size=16, dtype="f32", ctx=(256,), num_pages=16, num_splits=1,
        scale=0.125,
        description="single-layer paged decode, batch 1, 16 permuted physical pages"),
    "prefill_hq12_hkv12_d64_t512_f32": Workload(
        name="prefill_hq12_hkv12_d64_t512_f32", kind="prefill", index=1, hq=12, hkv=12,
        head_dim=64, page_size=16, dtype="f32", tokens=512, num_pages=32, scale=0.125,
        description="causal packed prefill of one 512-token sequence, 120M-model shape"),
    "decode_hq40_hkv8_d128_ctx3254_f16": Workload(
        name="decode_hq40_hkv8_d128_ctx3254_f16", kind="decode", index=2, hq=40, hkv=8,
        head_dim=128, page_size=16, dtype="f16", ctx=(3254,), num_pages=204, num_splits=32,
        layers=48, description="14B-shape decode, batch 1, 48 layers per step"),
    # Four disjoint page sets per layer pool (4 x 28 x 3.36 MB = 376 MB of K/V, more than the
    # 256 MB last-level cache), cycled step by step, so the step's K/V comes from HBM.
    "decode_hq28_hkv4_d128_ctx1641_f16": Workload(
        name="decode_hq28_hkv4_d128_ctx1641_f16", kind="decode", index=3, hq=28, hkv=4,
        head_dim=128, page_size=16, dtype="f16", ctx=(1641,), num_splits=32, layers=28,
        rotations=4, description="7B-shape decode, batch 1, 28 layers per step"),
    "decode_b16_hq64_hkv8_d128_ctx64to4096_bf16": Workload(
        name="decode_b16_hq64_hkv8_d128_ctx64to4096_bf16", kind="decode", index=4, hq=64,
        hkv=8, head_dim=128, page_size=32, dtype="bf16", batch=16, ctx_range=(64, 4096),
        num_pages=8192, num_splits=4, rotations=6,
        description="continuous-batching decode, 16 sequences in a shared 8192-page pool"),
    # Measurement shapes for the windowed and head_dim-256 decode arms (vllm.cpp PR #383
    # names the arms; it fixes no model shape for them): synthetic, same recipe.
    "decode_b16_hq64_hkv8_d128_ctx64to4096_w1024_bf16": Workload(
        name="decode_b16_hq64_hkv8_d128_ctx64to4096_w1024_bf16", kind="decode", index=5,
        hq=64, hkv=8, head_dim=128, page_size=32, dtype="bf16", batch=16, ctx_range=(64, 4096),
        num_pages=8192, num_splits=2, rotations=6, window=1024,
        description="the continuous-batching decode with a 1024-position sliding window"),
    "decode_hq16_hkv8_d256_ctx4096_bf16": Workload(
        name="decode_hq16_hkv8_d256_ctx4096_bf16", kind="decode", index=6, hq=16, hkv=8,
        head_dim=256, page_size=16, dtype="bf16", ctx=(4096,), num_pages=256, num_splits=32,
        layers=16, description="head_dim-256 decode, batch 1, 16 layers per step"),
    # The 512-token prefill in crucible's production GQA geometry (12 query heads over 3 kv
    # heads) with a bf16 pool: the measurement shape of the 16-bit MFMA prefill.
    "prefill_hq12_hkv3_d64_t512_bf16": Workload(
        name="prefill_hq12_hkv3_d64_t512_bf16", kind="prefill", index=7, hq=12, hkv=3,
        head_dim=64, page_size=16, dtype="bf16", tokens=512, num_pages=32, scale=0.125,
        description="causal packed prefill of one 512-token sequence, GQA 12/3, bf16 pool"),
    # The prefill microbenchmark shapes of crucible's results page, in its production GQA
    # geometry (12 query heads over 3 KV heads, head_dim 64, 16-token pages, f32 pool): one
    # 512-token request, four 256-token requests, and the heterogeneous pack (starts 0, 63,
    # 255, 512; lengths 17, 64, 129, 257), each request with its own page table.
    "prefill_hq12_hkv3_d64_t512_f32": Workload(
        name="prefill_hq12_hkv3_d64_t512_f32", kind="prefill", index=9, hq=12, hkv=3,
        head_dim=64, page_size=16, dtype="f32", tokens=512, scale=0.125,
        description="causal prefill of one 512-token request, GQA 12/3, f32 pool"),
    "prefill_hq12_hkv3_d64_4x256_f32": Workload(
        name="prefill_hq12_hkv3_d64_4x256_f32", kind="prefill", index=10, hq=12, hkv=3,
        head_dim=64, page_size=16, dtype="f32", tokens=1024, seg_lens=(256, 256, 256, 256),
        seg_starts=(0, 0, 0, 0), scale=0.125,
        description="causal packed prefill of four 256-token requests, GQA 12/3, f32 pool"),
    "prefill_hq12_hkv3_d64_hetero_f32": Workload(
        name="prefill_hq12_hkv3_d64_hetero_f32", kind="prefill", index=11, hq=12, hkv=3,
        head_dim=64, page_size=16, dtype="f32", tokens=467, seg_lens=(17, 64, 129, 257),
        seg_starts=(0, 63, 255, 512), scale=0.125,
        description="causal packed prefill of four requests with histories, GQA 12/3, f32"),
    # The 14B decode shape at a serving batch of 128: 1.7 GB of K/V per layer, several times
    # the last-level cache, so the step streams from HBM.  A throughput shape beside the
    # batch-1 one (same recipe; one split per sequence fills the device).
    "decode_b128_hq40_hkv8_d128_ctx3254_f16": Workload(
        name="decode_b128_hq40_hkv8_d128_ctx3254_f16", kind="decode", index=8, hq=40, hkv=8,
        head_dim=128, page_size=16, dtype="f16", batch=128, ctx=(3254,) * 128,
        num_splits=1, description="14B-shape decode, batch 128 sequences of 3254 positions"),
}


# --------------------------------------------------------------------------- decode cases

@dataclass
class DecodeCase:
    q: np.ndarray              # [B, Hq, D] f32
    k_pages: np.ndarray        # [P, ps, Hkv, D] storage dtype
    v_pages: np.ndarray
    page_table: np.ndarray     # [B, max_pages] int32
    context_lens: np.ndarray   # [B] int32, counts the current token
    k_new: np.ndarray          # [B, Hkv, D] storage dtype: K of the current token
    v_new: np.ndarray
    token_table_index: np.ndarray  # [B] int32 (= arange(B))
    token_position: np.ndarray     # [B] int32 (= ctx - 1)
    dtype: str
    scale: float
    num_splits: int
    extra_tables: list = field(default_factory=list)  # other rotations' tables
    window: int = 0            # sliding window in positions (0: whole context)

    @property
    def shape(self):
        B, Hq, D = self.q.shape
        P, ps, Hkv, _ = self.k_pages.shape
        return dict(num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=ps,
                    num_pages=P, max_pages_per_seq=self.page_table.shape[1])


def make_decode_case(rng: np.random.Generator, *, batch, hq, hkv, head_dim, page_size, dtype,
                     ctx=None, ctx_range=None, num_pages=0, max_pages_per_seq=0,
                     num_splits=1, scale=None, poison=True, rotations=1,
                     new_token_in_pool=False, window=0) -> DecodeCase:
    """Draw one decode case.  The current token (position ctx-1) of every sequence arrives
    in k_new/v_new; its pool slot is poisoned unless ``new_token_in_pool``.  With a sliding
    window, the positions before it are poisoned too (no decode may read them)."""
    q = rng.standard_normal((batch, hq, head_dim), dtype=np.float32)
    if ctx is not None:
        ctx_arr = np.broadcast_to(np.asarray(ctx, dtype=np.int64), (batch,)).copy()
        drawn_ctx = False
    else:
        ctx_arr = None
        drawn_ctx = True
    # Pool size: enough pages for every rotation of the longest possible contexts.
    max_ctx = int(ctx_range[1]) if drawn_ctx else int(ctx_arr.max())
    if max_pages_per_seq == 0:
        max_pages_per_seq = max(1, -(-max_ctx // page_size))
    if num_pages == 0:
        if drawn_ctx:
            num_pages = rotations * batch * max_pages_per_seq
        else:   # exactly the pages the sequences need, plus two spare (poisoned) pages
            num_pages = rotations * sum(-(-int(c) // page_size) for c in ctx_arr) + 2
    shape = (num_pages, page_size, hkv, head_dim)
    k_pages = _normal_pool(rng, shape, dtype)
    v_pages = _normal_pool(rng, shape, dtype)
    perm = rng.permutation(num_pages).astype(np.int32)
    if drawn_ctx:
        ctx_arr = rng.integers(int(ctx_range[0]), int(ctx_range[1]) + 1, size=batch)
    k_new = to_storage(rng.standard_normal((batch, hkv, head_dim), dtype=np.float32), dtype)
    v_new = to_storage(rng.standard_normal((batch, hkv, head_dim), dtype=np.float32), dtype)

    need = [-(-int(c) // page_size) for c in ctx_arr]
    if rotations * sum(need) > num_pages:
        raise ValueError("pool too small for the drawn contexts")
    tables = []
    cursor = 0
    for _ in range(rotations):
        table = np.full((batch, max_pages_per_seq), -1, dtype=np.int32)
        for b in range(batch):
            table[b, :need[b]] = perm[cursor:cursor + need[b]]
            cursor += need[b]
        tables.append(table)
    table = tables[0]
    ctx32 = ctx_arr.astype(np.int32)
    pos = (ctx32 - 1).astype(np.int32)
    if new_token_in_pool:
        for b in range(batch):
            p = table[b, pos[b] // page_size]
            k_pages[p, pos[b] % page_size] = k_new[b]
            v_pages[p, pos[b] % page_size] = v_new[b]
    if poison:
        _poison_decode(k_pages, v_pages, table, ctx32, dtype,
                       keep_current=new_token_in_pool, window=window)
    return DecodeCase(q=q, k_pages=k_pages, v_pages=v_pages, page_table=table,
                      context_lens=ctx32, k_new=k_new, v_new=v_new,
                      token_table_index=np.arange(batch, dtype=np.int32), token_position=pos,
                      dtype=dtype,
                      scale=float(np.float32(scale if scale else 1.0 / math.sqrt(head_dim))),
                      num_splits=num_splits, extra_tables=tables[1:], window=int(window))


def _poison_decode(k_pages, v_pages, table, ctx, dtype, keep_current, window=0):
    """NaN into every pool byte no decode of these sequences may read: unowned pages, slots
    past the last position, the current token's slot unless it is kept, and positions
    before a sliding window."""
    num_pages, ps = k_pages.shape[:2]
    live = np.zeros((num_pages, ps), dtype=bool)
    for b in range(table.shape[0]):
        n = int(ctx[b]) if keep_current else int(ctx[b]) - 1
        t0 = max(0, int(ctx[b]) - window) if window > 0 else 0
        for t in range(t0, n):
            live[table[b, t // ps], t % ps] = True
    nan = nan_value(dtype)
    k_pages[~live] = nan
    v_pages[~live] = nan


def workload_decode_case(w: Workload, poison=True, new_token_in_pool=False) -> DecodeCase:
    """The seeded case of a named decode workload (one layer, first rotation)."""
    assert w.kind == "decode"
    rng = named_rng(w.index)
    return make_decode_case(
        rng, batch=w.batch, hq=w.hq, hkv=w.hkv, head_dim=w.head_dim, page_size=w.page_size,
        dtype=w.dtype, ctx=w.ctx if w.ctx else None, ctx_range=w.ctx_range or None,
        num_pages=w.num_pages, num_splits=w.num_splits, scale=w.attn_scale, poison=poison,
        rotations=w.rotations, new_token_in_pool=new_token_in_pool, window=w.window)


# --------------------------------------------------------------------------- prefill cases

@dataclass
class PrefillCase:
    q: np.ndarray              # [T, Hq, D] f32, packed rows of every segment
    k_pages: np.ndarray        # history of every segment present; chunk slots poisoned
    v_pages: np.ndarray
    page_table: np.ndarray     # [num_tables, max_pages] int32
    seg_desc: np.ndarray       # [num_segs, 4] int32 {packed_start, len, abs_start, table}
    k_new: np.ndarray          # [T, Hkv, D]: K of every packed row (written before attention)
    v_new: np.ndarray
    token_table_index: np.ndarray  # [T] owner table row of each packed row
    token_position: np.ndarray     # [T] absolute position of each packed row
    dtype: str
    scale: float

    @property
    def max_chunk_len(self) -> int:
        return int(self.seg_desc[:, 1].max()) if len(self.seg_desc) else 0


def make_prefill_case(rng: np.random.Generator, *, hq, hkv, head_dim, page_size, dtype,
                      lens, starts=None, num_pages=0, scale=None, poison=True,
                      gap_rows=0) -> PrefillCase:
    """Segments with chunk lengths ``lens`` at absolute offsets ``starts`` (default 0), one
    page table per segment, packed back to back (``gap_rows`` uncovered rows between)."""
    lens = [int(x) for x in lens]
    starts = [0] * len(lens) if starts is None else [int(x) for x in starts]
    nseg = len(lens)
    packed = []
    cursor = 0
    for ln in lens:
        packed.append(cursor)
        cursor += ln + gap_rows
    total = max(cursor - gap_rows, 0) if nseg else 0
    hist = [s + ln for s, ln in zip(starts, lens)]
    max_pages = max(1, max(-(-h // page_size) for h in hist)) if nseg else 1
    need = [-(-h // page_size) for h in hist]
    if num_pages == 0:
        num_pages = max(1, sum(need))
    q = rng.standard_normal((max(total, 0), hq, head_dim), dtype=np.float32)
    shape = (num_pages, page_size, hkv, head_dim)
    k_pages = _normal_pool(rng, shape, dtype)
    v_pages = _normal_pool(rng, shape, dtype)
    perm = rng.permutation(num_pages).astype(np.int32)
    k_new = to_storage(rng.standard_normal((max(total, 0), hkv, head_dim), dtype=np.float32),
                       dtype)
    v_new = to_storage(rng.standard_normal((max(total, 0), hkv, head_dim), dtype=np.float32),
                       dtype)
    if sum(need) > num_pages:
        raise ValueError("pool too small")
    table = np.full((max(nseg, 1), max_pages), -1, dtype=np.int32)
    c = 0
    for i in range(nseg):
        table[i, :need[i]] = perm[c:c + need[i]]
        c += need[i]
    desc = np.array([[packed[i], lens[i], starts[i], i] for i in range(nseg)],
                    dtype=np.int32).reshape(nseg, 4)
    owner = np.zeros(max(total, 0), dtype=np.int32)
    pos = np.zeros(max(total, 0), dtype=np.int32)
    covered = np.zeros(max(total, 0), dtype=bool)
    for i in range(nseg):
        owner[packed[i]:packed[i] + lens[i]] = i
        pos[packed[i]:packed[i] + lens[i]] = starts[i] + np.arange(lens[i])
        covered[packed[i]:packed[i] + lens[i]] = True
    if poison:
        live = np.zeros((num_pages, page_size), dtype=bool)
        for i in range(nseg):
            for t in range(starts[i]):                 # history only; chunk arrives by write
                live[table[i, t // page_size], t % page_size] = True
        nan = nan_value(dtype)
        k_pages[~live] = nan
        v_pages[~live] = nan
    # Rows in gaps between segments are not attention rows: mark them with an invalid owner
    # so that a page write of all packed rows skips them.
    owner[~covered] = -1
    return PrefillCase(q=q, k_pages=k_pages, v_pages=v_pages, page_table=table, seg_desc=desc,
                       k_new=k_new, v_new=v_new, token_table_index=owner, token_position=pos,
                       dtype=dtype,
                       scale=float(np.float32(scale if scale else 1.0 / math.sqrt(head_dim))))


def workload_prefill_case(w: Workload, poison=True) -> PrefillCase:
    assert w.kind == "prefill"
    rng = named_rng(w.index)
    lens = list(w.seg_lens) if w.seg_lens else [w.tokens]
    starts = list(w.seg_starts) if w.seg_starts else None
    return make_prefill_case(rng, hq=w.hq, hkv=w.hkv, head_dim=w.head_dim,
                             page_size=w.page_size, dtype=w.dtype, lens=lens, starts=starts,
                             num_pages=w.num_pages, scale=w.attn_scale, poison=poison)


# --------------------------------------------------------------------------- split partials

def make_partials(rng: np.random.Generator, *, batch, hq, head_dim, num_splits,
                  empty_fraction=0.25, all_empty_rows=0):
    """Synthetic split partials for testing the merge on its own: m ~ 4 N(0,1),
    l ~ U(0.5, 64), O ~ N(0,1) * l, a fraction of splits idle (m=-inf, l=0, O=0), and the
    first ``all_empty_rows`` (b, h) rows with every split idle."""
    shape = (batch, hq, num_splits)
    m = (4.0 * rng.standard_normal(shape)).astype(np.float32)
    l = rng.uniform(0.5, 64.0, size=shape).astype(np.float32)
    o = (rng.standard_normal(shape + (head_dim,)).astype(np.float32) * l[..., None])
    empty = rng.random(shape) < empty_fraction
    flat = empty.reshape(-1, num_splits)
    flat[:all_empty_rows] = True
    m[empty] = -np.inf
    l[empty] = 0.0
    o[empty] = 0.0
    ml = np.stack([m, l], axis=-1).astype(np.float32)
    return np.ascontiguousarray(o, dtype=np.float32), np.ascontiguousarray(ml)
