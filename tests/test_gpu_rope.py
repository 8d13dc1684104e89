"""GPU: the page write with rotary position embedding (kv_page_write_rope) against the f64
oracle, element by element, on seeded inputs.

Bars (the pages fix no precision for the rotation; the reading taken here): V is a pure
conversion and must be bit-exact.  K and q are rotated in f32 on the device, with the same f32
angle as the oracle, which rotates in f64 and rounds through f32 to the pool dtype.
- A 16-bit K element may differ from the oracle's by one unit in the last place: the f32
  value can sit on the other side of a rounding boundary.
- An f32 K or q element must lie within 2^-20 (|a| + |b|) of the oracle's, for (a, b) the
  input pair.  That is a few f32 roundings of the two products and of cos and sin.
Untouched bytes keep their NaN poison."""
import numpy as np
import pytest
import torch

import oracle
import paged_gqa_attention_decode_amd as pa
from compare import assert_bitwise
from gpu_helpers import announce, dev, host
from paged_gqa_attention_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

NP_POOL = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16}


def inv_freq(d, base=10000.0):
    return (base ** (-np.arange(d // 2, dtype=np.float64) * 2.0 / d)).astype(np.float32)


def ordered(bits: np.ndarray) -> np.ndarray:
    """16-bit float patterns as integers that increase with the value (sign-magnitude)."""
    b = bits.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def pair_scale(x: np.ndarray, style: int) -> np.ndarray:
    """|a| + |b| of the input pair each element belongs to (same shape as x)."""
    d = x.shape[-1]
    a = np.abs(x.astype(np.float64))
    if style == pa.PA_ROPE_ADJACENT:
        p = a.reshape(*a.shape[:-1], d // 2, 2).sum(-1)
        return np.repeat(p, 2, axis=-1)
    p = a[..., : d // 2] + a[..., d // 2:]
    return np.concatenate([p, p], axis=-1)


def make_case(rng, *, T, hq, hkv, d, ps, dtype, a0, n_tables=1, bad=False):
    """T tokens of one sequence at absolute positions a0 .. a0+T-1 (its table maps exactly
    those pages; every other page id is -1).  With bad=True a few tokens carry an invalid
    owner, a negative position or a missing page."""
    cap_pages = (a0 + T + ps - 1) // ps + 2
    first, last = a0 // ps, (a0 + T - 1) // ps
    n_used = last - first + 1
    P = n_used + 3
    table = np.full((n_tables, cap_pages), -1, np.int32)
    table[0, first:last + 1] = rng.permutation(P)[:n_used]
    owner = np.zeros(T, np.int32)
    pos = (a0 + np.arange(T)).astype(np.int32)
    if bad:
        owner[1] = n_tables          # no such table row
        pos[2] = -5                  # skipped altogether
        owner[3] = -1
        pos[4] = (cap_pages - 1) * ps  # a logical page with id -1
    k_new = rng.standard_normal((T, hkv, d)).astype(np.float32)
    v_new = rng.standard_normal((T, hkv, d)).astype(np.float32)
    q = rng.standard_normal((T, hq, d)).astype(np.float32) if hq else None
    pool = np.full((P, ps, hkv, d), wl.nan_value(dtype), NP_POOL[dtype])
    return dict(k_new=k_new, v_new=v_new, pool=pool, table=table, owner=owner, pos=pos, q=q)


CASES = [
    # (name, T, hq, hkv, d, ps, dtype, a0)
    ("prefill512_12x12_d64_f32", 512, 12, 12, 64, 16, "f32", 0),
    ("decode_40x8_d128_f16", 1, 40, 8, 128, 16, "f16", 3253),
    ("batch16_64x8_d128_bf16", 16, 64, 8, 128, 32, "bf16", 4080),
    ("chunk_at_70000_28x4_d128_bf16", 96, 28, 4, 128, 16, "bf16", 70001),
    ("no_query_8x2_d64_f16", 40, 0, 2, 64, 1, "f16", 12345),
    ("d256_16x8_bf16", 24, 16, 8, 256, 16, "bf16", 4000),
]


@pytest.mark.parametrize("style", [pa.PA_ROPE_ADJACENT, pa.PA_ROPE_HALVES],
                         ids=["adjacent", "halves"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_rope_write_vs_oracle(case, style):
    name, T, hq, hkv, d, ps, dtype, a0 = case
    rng = wl.rng_for(30_000 + 7 * T + d + a0 + style)
    c = make_case(rng, T=T, hq=hq, hkv=hkv, d=d, ps=ps, dtype=dtype, a0=a0, bad=T >= 8)
    freq = inv_freq(d)
    rk, rv, rq = oracle.kv_write_rope(c["k_new"], c["v_new"], c["pool"], c["pool"], dtype,
                                      c["table"], c["owner"], c["pos"], freq, style, q=c["q"])
    announce(f"kv_page_write_rope {name} style={style}")
    kp, vp = dev(c["pool"], dtype), dev(c["pool"], dtype)
    qd = None if c["q"] is None else dev(c["q"])
    pa.kv_page_write_rope(dev(c["k_new"]), dev(c["v_new"]), kp, vp, dev(c["table"]),
                          dev(c["owner"]), dev(c["pos"]), dev(freq), style, q=qd)
    torch.cuda.synchronize()
    gk, gv = host(kp), host(vp)
    assert_bitwise(gv, rv, f"{name}: V (conversion only)")
    # Rows never written keep their poison on both sides, bit for bit.
    poison = np.isnan(oracle.widen(rk, dtype))
    assert np.array_equal(poison, np.isnan(oracle.widen(gk, dtype))), "written slots differ"
    if dtype == "f32":
        # Each written K element against its own input pair.
        ref = rk[~poison].astype(np.float64)
        got = gk[~poison].astype(np.float64)
        assert np.all(np.isfinite(got))
        scale = np.zeros_like(rk, dtype=np.float64)
        _fill_written_scale(scale, c, style, ps)
        bound = 2.0 ** -20 * scale[~poison]
        assert np.all(np.abs(got - ref) <= bound), \
            f"{name}: K max excess {np.max(np.abs(got - ref) - bound):.3e}"
    else:
        diff = np.abs(ordered(gk[~poison]) - ordered(rk[~poison]))
        assert diff.max() <= 1, f"{name}: K differs by {diff.max()} ulp"
        print(f"{name}: K bit-identical {100.0 * np.mean(diff == 0):.3f}%")
    if c["q"] is not None:
        gq = host(qd).astype(np.float64)
        bound = 2.0 ** -20 * pair_scale(c["q"], style)
        assert np.all(np.abs(gq - rq.astype(np.float64)) <= bound), f"{name}: q outside bound"
        skipped = c["pos"] < 0
        assert_bitwise(host(qd)[skipped], c["q"][skipped], "negative position leaves q alone")


def _fill_written_scale(scale, c, style, ps):
    """scale[page, slot, h, :] = |a| + |b| of each element's input pair, for written slots."""
    s = pair_scale(c["k_new"], style)
    tbl = c["table"]
    for i in range(c["k_new"].shape[0]):
        o, p = int(c["owner"][i]), int(c["pos"][i])
        if o < 0 or o >= tbl.shape[0] or p < 0 or p >= tbl.shape[1] * ps:
            continue
        page = int(tbl[o, p // ps])
        if page < 0 or page >= scale.shape[0]:
            continue
        scale[page, p % ps] = s[i]


def test_rope_angle_zero_is_the_plain_write():
    """All frequencies 0: the rotated write equals kv_page_write of the converted rows, bit
    for bit (both on the device), and q is unchanged."""
    rng = wl.rng_for(30_101)
    for dtype in ("f16", "bf16", "f32"):
        c = make_case(rng, T=33, hq=4, hkv=4, d=128, ps=16, dtype=dtype, a0=500, bad=True)
        announce(f"kv_page_write_rope angle 0 {dtype}")
        kp, vp = dev(c["pool"], dtype), dev(c["pool"], dtype)
        qd = dev(c["q"])
        pa.kv_page_write_rope(dev(c["k_new"]), dev(c["v_new"]), kp, vp, dev(c["table"]),
                              dev(c["owner"]), dev(c["pos"]),
                              torch.zeros(64, device="cuda"), pa.PA_ROPE_HALVES, q=qd)
        k2, v2 = dev(c["pool"], dtype), dev(c["pool"], dtype)
        tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
        pa.kv_page_write(dev(c["k_new"]).to(tdt), dev(c["v_new"]).to(tdt), k2, v2,
                         dev(c["table"]), dev(c["owner"]), dev(c["pos"]))
        torch.cuda.synchronize()
        assert_bitwise(host(kp), host(k2), f"angle 0 K {dtype}")
        assert_bitwise(host(vp), host(v2), f"angle 0 V {dtype}")
        assert_bitwise(host(qd), c["q"], "angle 0 leaves q")
