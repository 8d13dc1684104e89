"""GPU: the HIP path against the f64 oracle, element by element, on seeded inputs.

Bars: page writes bit-exact; decode and prefill outputs within max-abs 1e-5 for f32 K/V and
|gpu - ref| <= 2e-3 + 1e-2 |ref| for f16/bf16 K/V.  Split partials are compared as
(m, l, O/l) against the oracle's partials under the same partition rule."""
import math
import os
from concurrent.futures import ThreadPoolExecutor

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


def _rows_in_parallel(fn, rows):
    """fn(chunk of rows) over the rows, chunks run in threads on the host's cores (the oracle
    is a C library whose calls release the interpreter lock), results in row order."""
    workers = max(1, min(16, len(os.sched_getaffinity(0)), len(rows)))
    chunks = [c for c in np.array_split(np.asarray(rows), workers) if len(c)]
    with ThreadPoolExecutor(len(chunks)) as ex:
        parts = list(ex.map(fn, chunks))
    return parts


def oracle_step(case, rows=None):
    """Oracle: page write of the current token, then attention over the whole context (of
    the sequences `rows`, default all; large batches run on all host cores)."""
    rows = np.arange(case.q.shape[0]) if rows is None else rows
    kp, vp = oracle.kv_write(case.k_new, case.v_new, case.k_pages, case.v_pages, case.dtype,
                             case.page_table, case.token_table_index, case.token_position)
    parts = _rows_in_parallel(
        lambda r: oracle.decode(case.q[r], kp, vp, case.dtype, case.page_table[r],
                                case.context_lens[r], case.scale, window=case.window), rows)
    return kp, vp, np.concatenate(parts, axis=0)


def check_partials(run, case, kp, vp, rows=None):
    rows = np.arange(case.q.shape[0]) if rows is None else rows
    po = host(run.po).astype(np.float64)[rows]
    pml = host(run.pml).astype(np.float64)[rows]
    parts = _rows_in_parallel(
        lambda r: oracle.decode_partials(case.q[r], kp, vp, case.dtype, case.page_table[r],
                                         case.context_lens[r], case.scale, run.S,
                                         window=run.window), rows)
    ro, rm, rl = (np.concatenate([p[i] for p in parts], axis=0) for i in range(3))
    m, l = pml[..., 0], pml[..., 1]
    idle = rl == 0
    assert np.array_equal(l == 0, idle), "idle-split pattern differs"
    assert np.all(m[idle] == -np.inf) and np.all(po[idle] == 0.0)
    live = ~idle
    assert_within(m[live], rm[live], 1e-4, 1e-6, "split max m")
    assert_within(l[live], rl[live], 0.0, 2e-4, "split sum l")
    atol, rtol = tolerance(case.dtype)
    assert_within(po[live] / l[live][:, None], ro[live] / rl[live][:, None], atol, rtol,
                  "split O/l")


# ----------------------------------------------------------------------------- page write

@pytest.mark.parametrize("dtype,ps,hkv,d", [("f32", 16, 12, 64), ("f16", 16, 8, 128),
                                             ("bf16", 32, 8, 128), ("f32", 1, 2, 128),
                                             ("bf16", 4096, 1, 64), ("f16", 16, 8, 256),
                                             ("f32", 8, 4, 256)])
def test_kv_page_write_bit_exact(dtype, ps, hkv, d):
    announce(f"kv_page_write {dtype} ps={ps} hkv={hkv} d={d}")
    rng = wl.rng_for([200, ps, hkv, d])
    num_pages, max_pages, ntab = 14, 4, 3
    kp = np.full((num_pages, ps, hkv, d), wl.nan_value(dtype), wl.storage_dtype(dtype))
    vp = kp.copy()
    table = rng.permutation(num_pages)[: ntab * max_pages].reshape(ntab, max_pages)
    table = table.astype(np.int32)
    table[2, 3] = 99                                          # out-of-range page id
    T = 40
    owner = rng.integers(-1, ntab + 1, size=T).astype(np.int32)  # includes -1 and ntab
    cap = max_pages * ps
    pos = rng.integers(0, cap + 2, size=T).astype(np.int32)       # includes cap, cap+1
    # unique (owner, pos) pairs so no two tokens race for one slot
    _, first = np.unique(owner.astype(np.int64) * (cap + 8) + pos, return_index=True)
    keep = np.sort(first)
    owner, pos = owner[keep], pos[keep]
    k_new = wl.to_storage(rng.standard_normal((owner.size, hkv, d)).astype(np.float32), dtype)
    v_new = wl.to_storage(rng.standard_normal((owner.size, hkv, d)).astype(np.float32), dtype)
    rk, rv = oracle.kv_write(k_new, v_new, kp, vp, dtype, table, owner, pos)
    gk, gv = dev(kp, dtype), dev(vp, dtype)
    pa.kv_page_write(dev(k_new, dtype), dev(v_new, dtype), gk, gv, dev(table), dev(owner),
                     dev(pos))
    torch.cuda.synchronize()
    assert_bitwise(host(gk), rk, "K pool")
    assert_bitwise(host(gv), rv, "V pool")


# ----------------------------------------------------------------------------- named decode

DECODE_WORKLOADS = [n for n, w in wl.WORKLOADS.items() if w.kind == "decode"]


@pytest.mark.parametrize("name", DECODE_WORKLOADS)
def test_decode_workload(name):
    """Full-size parity of every named decode workload, in the bench's launch configuration
    (write of the current token -> split decode with the workload's split count -> combine)."""
    w = wl.WORKLOADS[name]
    case = wl.workload_decode_case(w)
    announce(f"decode workload {name} S={case.num_splits} batch {case.q.shape[0]}")
    run = DecodeRun(case)
    out = run.step()
    kp, vp, ref = oracle_step(case)
    assert_bitwise(host(run.kp), kp, "K pool after write")
    atol, rtol = tolerance(case.dtype)
    assert_within(out, ref, atol, rtol, f"decode {name}")
    assert_within(out, ref, *second_bar(case.dtype), f"decode {name}, second bar")
    check_partials(run, case, kp, vp)


@pytest.mark.parametrize("splits", [1, 2, 7, 16, 64, 4096])
def test_decode_split_counts(splits):
    w = wl.WORKLOADS["decode_hq40_hkv8_d128_ctx3254_f16"]
    case = wl.workload_decode_case(w)
    announce(f"decode 14B shape S={splits}")
    run = DecodeRun(case, num_splits=splits)
    out = run.step()
    kp, vp, ref = oracle_step(case)
    assert_within(out, ref, *tolerance("f16"), f"decode S={splits}")
    check_partials(run, case, kp, vp)


BOUNDARY_CTX = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 255, 256, 257,
                511, 512, 685, 941, 1000, 1023, 1024, 1919, 1920, 1921, 2807, 2808, 3254,
                4095, 4096]


@pytest.mark.parametrize("geom", [(40, 8, 128, 16, "f16", 32), (28, 4, 128, 16, "f16", 32),
                                  (64, 8, 128, 32, "bf16", 16), (8, 2, 64, 16, "f32", 16),
                                  (12, 3, 64, 16, "f32", 8), (16, 16, 128, 32, "bf16", 4),
                                  (32, 2, 64, 16, "bf16", 8), (12, 1, 128, 16, "f16", 16),
                                  # the largest group (8 head groups of 8) and a ragged one
                                  # (groups of 7, the last with 5 heads)
                                  (64, 1, 128, 16, "bf16", 8), (33, 1, 64, 16, "f16", 16)],
                         ids=lambda g: "hq{}_hkv{}_d{}_ps{}_{}_S{}".format(*g))
def test_decode_boundary_lengths(geom):
    """Every boundary length of the pages' fixture lists in one batch."""
    hq, hkv, d, ps, dtype, S = geom
    announce(f"decode boundary lengths {geom}")
    rng = wl.rng_for([300, hq, hkv, d, ps])
    case = wl.make_decode_case(rng, batch=len(BOUNDARY_CTX), hq=hq, hkv=hkv, head_dim=d,
                               page_size=ps, dtype=dtype, ctx=BOUNDARY_CTX, num_splits=S)
    run = DecodeRun(case)
    out = run.step()
    kp, vp, ref = oracle_step(case)
    assert_within(out, ref, *tolerance(dtype), f"decode boundary {geom}")
    assert_within(out, ref, *second_bar(dtype), f"decode boundary {geom}, second bar")
    check_partials(run, case, kp, vp)


def test_decode_table_longer_than_lds_stage():
    """Page size 1 with 3000 tokens: the table row exceeds one LDS stage (1024 entries)."""
    announce("decode ps=1 ctx=3000 (segmented table staging)")
    rng = wl.rng_for(301)
    case = wl.make_decode_case(rng, batch=2, hq=8, hkv=2, head_dim=64, page_size=1,
                               dtype="bf16", ctx=[3000, 1500], num_splits=2)
    run = DecodeRun(case)
    out = run.step()
    _, _, ref = oracle_step(case)
    assert_within(out, ref, *tolerance("bf16"), "decode ps=1")


def test_decode_outlier_data():
    """The minfer D3-6 outlier generators (|q| ~ 57, |v| ~ 144) on the 14B geometry."""
    announce("decode outlier data")
    hq, hkv, d, n = 40, 8, 128, 1921
    rng = wl.rng_for(302)
    case = wl.make_decode_case(rng, batch=1, hq=hq, hkv=hkv, head_dim=d, page_size=16,
                               dtype="f16", ctx=[n], num_splits=32, new_token_in_pool=True)
    case.q[:] = np.array([(((i * 37) % 19) / 5.0 - 1.9) * 30.0 for i in range(hq * d)],
                         np.float32).reshape(1, hq, d)
    vals = np.array([(((i * 57) % 11) / 3.0 - 1.8) * 80.0 for i in range(n * hkv * d)],
                    np.float32).reshape(n, hkv, d)
    for t in range(n):
        p = case.page_table[0, t // 16]
        case.v_pages[p, t % 16] = wl.to_storage(vals[t], "f16")
    case.v_new[0] = case.v_pages[case.page_table[0, (n - 1) // 16], (n - 1) % 16]
    run = DecodeRun(case)
    out = run.step()
    _, _, ref = oracle_step(case)
    assert_within(out, ref, *tolerance("f16"), "decode outliers")


# ----------------------------------------------------------------------------- fused step

def _fused_checks(case, S=None, what=""):
    """One-launch step vs the oracle, vs the three-kernel path (bit-identical), counters
    left at zero, and a second call (reusing the counters) bit-identical to the first."""
    fused = DecodeRun(case, num_splits=S)
    out = fused.fused_step()
    kp, vp, ref = oracle_step(case)
    assert_bitwise(host(fused.kp), kp, f"{what} K pool after the fused write")
    assert_bitwise(host(fused.vp), vp, f"{what} V pool after the fused write")
    assert_within(out, ref, *tolerance(case.dtype), f"fused {what}")
    assert_within(out, ref, *second_bar(case.dtype), f"fused {what}, second bar")
    assert int(fused.counters.abs().sum().item()) == 0, "counters must be left at zero"
    again = fused.fused_step()
    assert_bitwise(again, out, f"{what} second fused call")
    three = DecodeRun(case, num_splits=S).step()
    assert_bitwise(out, three, f"{what} fused vs write+decode+combine")
    check_partials(fused, case, kp, vp)


@pytest.mark.parametrize("name", DECODE_WORKLOADS)
def test_decode_fused_workload(name):
    w = wl.WORKLOADS[name]
    case = wl.workload_decode_case(w)
    announce(f"fused decode workload {name}")
    _fused_checks(case, what=name)


@pytest.mark.parametrize("geom", [(40, 8, 128, 16, "f16", 0, [3254, 1, 700]),
                                  (64, 8, 128, 32, "bf16", 0, [2000, 33, 4096]),
                                  (8, 2, 64, 16, "f32", 0, [256, 17]),
                                  (16, 8, 256, 16, "bf16", 0, [1500, 64]),
                                  (28, 4, 128, 16, "f16", 100, [1641, 99, 101])])
def test_decode_fused_one_split(geom):
    """One split per sequence: each workgroup of the single-launch step writes the output
    from its own partial, with no ticket.  Same bars as every single-launch check (oracle,
    three-launch bits, pool bits, counters at zero, repeat call, partials)."""
    hq, hkv, d, ps, dtype, window, ctx = geom
    announce(f"fused decode S=1 {geom}")
    rng = wl.rng_for([330, hq, d, window])
    case = wl.make_decode_case(rng, batch=len(ctx), hq=hq, hkv=hkv, head_dim=d, page_size=ps,
                               dtype=dtype, ctx=ctx, num_splits=1, window=window)
    _fused_checks(case, S=1, what=f"S=1 {geom}")


@pytest.mark.parametrize("splits", [1, 3, 64, 4096])
def test_decode_fused_split_counts(splits):
    case = wl.workload_decode_case(wl.WORKLOADS["decode_hq28_hkv4_d128_ctx1641_f16"])
    announce(f"fused decode 7B shape S={splits}")
    _fused_checks(case, S=splits, what=f"S={splits}")


@pytest.mark.parametrize("geom", [(40, 8, 128, 16, "f16", 32), (8, 2, 64, 16, "f32", 16),
                                  (24, 2, 128, 32, "bf16", 8), (4, 4, 64, 1, "bf16", 5),
                                  (64, 1, 128, 16, "bf16", 8), (33, 3, 128, 16, "f16", 8)],
                         ids=lambda g: "hq{}_hkv{}_d{}_ps{}_{}_S{}".format(*g))
def test_decode_fused_boundary_lengths(geom):
    hq, hkv, d, ps, dtype, S = geom
    announce(f"fused decode boundary lengths {geom}")
    rng = wl.rng_for([310, hq, hkv, d, ps])
    ctx = BOUNDARY_CTX if ps > 1 else [c for c in BOUNDARY_CTX if c <= 1100]
    case = wl.make_decode_case(rng, batch=len(ctx), hq=hq, hkv=hkv, head_dim=d,
                               page_size=ps, dtype=dtype, ctx=ctx, num_splits=S)
    _fused_checks(case, what=f"boundary {geom}")


# ----------------------------------------------------------------------------- combine alone

@pytest.mark.parametrize("d,S", [(64, 1), (64, 16), (128, 32), (128, 33), (128, 4096)])
def test_combine_synthetic_partials(d, S):
    announce(f"combine d={d} S={S}")
    rng = wl.rng_for([400, d, S])
    B = 1 if S > 1024 else 3
    o, ml = wl.make_partials(rng, batch=B, hq=40, head_dim=d, num_splits=S, all_empty_rows=2)
    ref = oracle.combine(o, ml[..., 0], ml[..., 1])
    got = run_combine(o, ml)
    assert np.all(got.reshape(-1, d)[:2] == 0.0), "all-idle rows must be zero"
    err = np.abs(got - ref)
    tol = combine_tolerance(o, ml)
    assert np.all(err <= tol), f"combine d={d} S={S}: max err/tol {np.max(err / tol):.3f}"


def run_combine(o, ml):
    B, H, S, d = o.shape
    out = torch.full((B, H, d), float("nan"), device=DEV)
    pa.paged_attn_combine(dev(o), dev(ml), out)
    torch.cuda.synchronize()
    return host(out)


def combine_tolerance(o, ml):
    """f32 sums over S splits: besides the 1e-5 floor, the summation bound
    2 * S * 2^-24 * (sum_s w_s |O_s|) / (sum_s w_s l_s), w_s = exp(m_s - M), in f64."""
    S = o.shape[-2]
    m64, l64 = ml[..., 0].astype(np.float64), ml[..., 1].astype(np.float64)
    live = l64 > 0
    M = np.max(np.where(live, m64, -np.inf), axis=-1, keepdims=True)
    with np.errstate(invalid="ignore", over="ignore"):
        w = np.where(live, np.exp(m64 - M), 0.0)
        ao = np.where(live[..., None], np.abs(o.astype(np.float64)), 0.0)
        bound = (w[..., None] * ao).sum(-2) / np.maximum((w * l64).sum(-1), 1e-30)[..., None]
    return 1e-5 + 2.0 * S * 2.0 ** -24 * np.nan_to_num(bound)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_combine_idle_contents_and_chunk_order(d):
    """Splits are merged 32 at a time with a running maximum.  Rows whose splits 32..63 are
    all idle (a chunk with nothing live between live ones), whose largest maximum first
    appears in the last chunk, or in the first: within the oracle's bar.  An idle split's m
    and O are never used: NaN in O and a huge m in every idle split give the same bits."""
    S = 96
    announce(f"combine idle contents and chunk order d={d}")
    rng = wl.rng_for([410, d])
    o, ml = wl.make_partials(rng, batch=2, hq=8, head_dim=d, num_splits=S, all_empty_rows=1)
    ml[:, :4, 32:64, 0] = -np.inf
    ml[:, :4, 32:64, 1] = 0.0
    o[:, :4, 32:64, :] = 0.0
    ml[:, 2:4, 90, :] = (40.0, 3.0)   # the row maximum appears in the last chunk
    ml[:, 4:6, 5, :] = (40.0, 3.0)    # ... or in the first, far above the rest
    ref = oracle.combine(o, ml[..., 0], ml[..., 1])
    clean = run_combine(o, ml)
    err = np.abs(clean - ref)
    tol = combine_tolerance(o, ml)
    assert np.all(err <= tol), f"combine d={d}: max err/tol {np.max(err / tol):.3f}"
    assert np.all(clean[0, 0] == 0.0), "an all-idle row must be zero"
    idle = ml[..., 1] == 0.0
    o2, ml2 = o.copy(), ml.copy()
    o2[idle] = np.nan
    ml2[..., 0][idle] = 1e30
    assert_bitwise(run_combine(o2, ml2), clean, f"combine d={d} with garbage in idle splits")


# ----------------------------------------------------------------------------- prefill

def run_prefill(case, out_fill=np.nan):
    dt = case.dtype
    kp, vp = dev(case.k_pages, dt), dev(case.v_pages, dt)
    table = dev(case.page_table)
    pa.kv_page_write(dev(case.k_new, dt), dev(case.v_new, dt), kp, vp, table,
                     dev(case.token_table_index), dev(case.token_position))
    out = torch.full(case.q.shape, float(out_fill), device=DEV)
    pa.paged_attn_prefill(dev(case.q), kp, vp, table, dev(case.seg_desc), case.max_chunk_len,
                          case.scale, out)
    torch.cuda.synchronize()
    return host(out), host(kp), host(vp)


def oracle_prefill(case):
    kp, vp = oracle.kv_write(case.k_new, case.v_new, case.k_pages, case.v_pages, case.dtype,
                             case.page_table, case.token_table_index, case.token_position)
    out, count = oracle.prefill(case.q, kp, vp, case.dtype, case.page_table, case.seg_desc,
                                case.scale)
    return out, kp, vp, count


def test_prefill_workload():
    w = wl.WORKLOADS["prefill_hq12_hkv12_d64_t512_f32"]
    case = wl.workload_prefill_case(w)
    announce("prefill workload 512 tokens 12/12 d64 f32")
    got, gk, gv = run_prefill(case)
    ref, kp, vp, count = oracle_prefill(case)
    assert count == 131328
    assert_bitwise(gk, kp, "K pool after write")
    assert_within(got, ref, 1e-5, 0.0, "prefill 512")


def test_prefill_workload_bf16():
    """The 16-bit MFMA prefill at its measurement shape.  Besides the bf16 bar, the error
    stays near f32 rounding (2^-16 |x| split residual of Q and P): a kernel that rounded Q or
    P to bf16 once would err by ~1e-3 here."""
    w = wl.WORKLOADS["prefill_hq12_hkv3_d64_t512_bf16"]
    case = wl.workload_prefill_case(w)
    announce("prefill workload 512 tokens 12/3 d64 bf16")
    got, gk, gv = run_prefill(case)
    ref, kp, vp, count = oracle_prefill(case)
    assert count == 131328
    assert_bitwise(gk, kp, "K pool after write")
    assert_within(got, ref, *tolerance("bf16"), "prefill 512 bf16")
    err = float(np.max(np.abs(got.astype(np.float64) - ref)))
    print(f"prefill 512 bf16: max abs error {err:.3e}")
    assert err < 1e-4, err


@pytest.mark.parametrize("name,extent", [("prefill_hq12_hkv3_d64_t512_f32", 131328),
                                         ("prefill_hq12_hkv3_d64_4x256_f32", 131584),
                                         ("prefill_hq12_hkv3_d64_hetero_f32", 212282)])
def test_prefill_benchmark_packs(name, extent):
    """The pages' prefill microbenchmark shapes (crucible results page: single-512, 4x256
    and the heterogeneous pack, GQA 12/3, f32 pool), in the launch configuration the bench
    times, element by element against the oracle."""
    w = wl.WORKLOADS[name]
    case = wl.workload_prefill_case(w)
    announce(f"prefill workload {name}")
    got, gk, gv = run_prefill(case)
    ref, kp, vp, count = oracle_prefill(case)
    assert count == extent
    assert_bitwise(gk, kp, "K pool after write")
    assert_within(got, ref, 1e-5, 0.0, name)


PREFILL_CASES = [
    # hq, hkv, d, ps, dtype, starts, lens, gap
    (12, 3, 64, 16, "f32", [0, 63, 255, 512], [17, 64, 129, 257], 0),   # heterogeneous
    (12, 3, 64, 16, "f32", [64] * 4, [64] * 4, 0),                      # history-64-at-64
    (12, 12, 64, 16, "f32", [0] * 16, [16] * 16, 0),                    # 16x16
    (8, 2, 128, 32, "bf16", [0, 33, 100], [1, 47, 300], 5),
    (40, 8, 128, 16, "f16", [3000], [70], 0),
    (4, 4, 64, 1, "f32", [5, 0], [20, 33], 2),
    (16, 1, 128, 16, "bf16", [0], [129], 0),
    (12, 3, 64, 16, "bf16", [0, 63, 255, 512], [17, 64, 129, 257], 0),  # heterogeneous
    (12, 3, 64, 16, "f16", [64] * 4, [64] * 4, 0),                      # history-64-at-64
    (8, 8, 64, 1, "f16", [5, 0], [20, 33], 2),
    (12, 4, 128, 32, "f16", [0, 2000], [200, 40], 3),
    (8, 2, 128, 16, "bf16", [16400, 0], [64, 31], 0),   # key range past one page-id slice
    (12, 3, 64, 256, "f32", [300, 0], [100, 257], 0),   # large pages
    (8, 4, 128, 4096, "bf16", [5000, 0], [40, 70], 1),  # the largest page size
]


@pytest.mark.parametrize("c", PREFILL_CASES,
                         ids=lambda c: "hq{}_hkv{}_d{}_ps{}_{}_{}segs".format(*c[:5], len(c[5])))
def test_prefill_cases(c):
    hq, hkv, d, ps, dtype, starts, lens, gap = c
    announce(f"prefill {c}")
    rng = wl.rng_for([500, hq, hkv, d, ps, len(starts)])
    case = wl.make_prefill_case(rng, hq=hq, hkv=hkv, head_dim=d, page_size=ps, dtype=dtype,
                                lens=lens, starts=starts, gap_rows=gap)
    got, _, _ = run_prefill(case, out_fill=7.0)
    ref, _, _, _ = oracle_prefill(case)
    covered = case.token_table_index >= 0
    assert np.all(got[~covered] == 7.0), "rows outside every segment must stay untouched"
    assert_within(got[covered], ref[covered], *tolerance(dtype), f"prefill {c}")


# ----------------------------------------------------------------------------- largest grids

MAX_GRID_Z = 65535   # sequences per decode call, segments per prefill call


def test_decode_largest_batch():
    """The largest batch a decode call takes (65,535 sequences, one per grid row), with
    short contexts: every row against the oracle, the page write bit-exact, and the
    single-launch step (131,070 counters) bit-identical to the three launches."""
    announce("decode, 65535 sequences")
    rng = wl.rng_for(340)
    ctx = [int(x) for x in rng.integers(1, 9, size=MAX_GRID_Z)]
    case = wl.make_decode_case(rng, batch=MAX_GRID_Z, hq=2, hkv=1, head_dim=64, page_size=4,
                               dtype="f16", ctx=ctx, num_splits=2)
    run = DecodeRun(case)
    out = run.step()
    kp, vp, ref = oracle_step(case)
    assert_bitwise(host(run.kp), kp, "K pool after write")
    assert_within(out, ref, *tolerance("f16"), "decode, 65535 sequences")
    fused = DecodeRun(case)
    assert_bitwise(fused.fused_step(), out, "single launch vs three launches")
    assert int(fused.counters.abs().sum().item()) == 0, "counters must be left at zero"


def test_prefill_most_segments():
    """The most segments a prefill call takes (65,535, one per grid row), one packed row
    each over a history of 0-7 positions, against the oracle."""
    announce("prefill, 65535 segments")
    rng = wl.rng_for(341)
    starts = [int(x) for x in rng.integers(0, 8, size=MAX_GRID_Z)]
    case = wl.make_prefill_case(rng, hq=2, hkv=1, head_dim=64, page_size=4, dtype="bf16",
                                lens=[1] * MAX_GRID_Z, starts=starts)
    got, gk, _ = run_prefill(case)
    ref, rk, _, _ = oracle_prefill(case)
    assert_bitwise(gk, rk, "K pool after write")
    assert_within(got, ref, *tolerance("bf16"), "prefill, 65535 segments")


def test_decode_million_positions():
    """One sequence of 2^20 positions (65,536 pages of 16, the table staged in many LDS
    slices, 64 splits of 16,384 rows): output and partials against the oracle, and the
    single-launch step bit-identical to the three launches."""
    announce("decode, 2^20 positions")
    rng = wl.rng_for(342)
    case = wl.make_decode_case(rng, batch=1, hq=4, hkv=1, head_dim=128, page_size=16,
                               dtype="bf16", ctx=[1 << 20], num_splits=64)
    run = DecodeRun(case)
    out = run.step()
    kp, vp, ref = oracle_step(case)
    assert_within(out, ref, *tolerance("bf16"), "decode, 2^20 positions")
    check_partials(run, case, kp, vp)
    fused = DecodeRun(case)
    assert_bitwise(fused.fused_step(), out, "single launch vs three launches")


def test_prefill_million_history():
    """Four packed rows at absolute positions 2^20 - 4 ... 2^20 - 1: every row sees a
    history of about a million keys over 65,536 pages (64 slices of staged page ids)."""
    announce("prefill, 2^20-position history")
    rng = wl.rng_for(343)
    case = wl.make_prefill_case(rng, hq=2, hkv=1, head_dim=64, page_size=16, dtype="f16",
                                lens=[4], starts=[(1 << 20) - 4])
    got, gk, _ = run_prefill(case)
    ref, rk, _, _ = oracle_prefill(case)
    assert_bitwise(gk, rk, "K pool after write")
    assert_within(got, ref, *tolerance("f16"), "prefill, 2^20-position history")
