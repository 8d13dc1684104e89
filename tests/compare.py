"""Element-wise comparison gates used by every parity test.

Two gates, both reporting max_abs, max_rel (denominator floored at 1e-6, as on the crucible
paged-attention results page) and the bitwise-equal percentage (the vllm.cpp PR #383
"Evidence" table reports the same three columns):

* ``assert_bitwise`` — identical bits (page writes, invariants of one implementation);
* ``assert_within``  — |got - ref| <= atol + rtol * |ref| for every element, the gate form
  of the crucible results page.

A failure names the worst element and the first few failing indices, so an injected error
is localised (the comparator self-test of the vllm.cpp PR #383 "Evidence" section).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# Tolerances for GPU results against the f64 oracle.
F32_ATOL = 1e-5          # f32 K/V: max-abs 1e-5
F32_RTOL = 0.0
HALF_ATOL = 2e-3         # f16/bf16 K/V: 2e-3 absolute plus 1e-2 relative
HALF_RTOL = 1e-2


def tolerance(dtype: str):
    return (F32_ATOL, F32_RTOL) if dtype == "f32" else (HALF_ATOL, HALF_RTOL)


# A second, tighter bar beside the gate above for f16/bf16 K/V on standard-normal data.  The
# path computes in f32 over exactly widened K/V (the query and the softmax weights carried as
# two 16-bit terms, residual below 2^-16 of the value), so its error stays near f32 rounding,
# ~1e-5 here; one dropped position of a 3254-position context moves an output by ~3e-4, and
# one 16-bit rounding of the query or the weights by ~1e-3, both caught by 1e-4.
HALF_SECOND_ATOL = 1e-4


def second_bar(dtype: str):
    return (F32_ATOL, 0.0) if dtype == "f32" else (HALF_SECOND_ATOL, 0.0)


@dataclass
class Report:
    n: int
    max_abs: float
    max_rel: float
    bitwise_pct: float
    worst: tuple
    failing: list

    def __str__(self):
        return (f"n={self.n} max_abs={self.max_abs:.3e} max_rel={self.max_rel:.3e} "
                f"bitwise={self.bitwise_pct:.4f}% worst={self.worst} "
                f"failing(first)={self.failing[:8]}")


def report(got, ref, atol=0.0, rtol=0.0) -> Report:
    got = np.asarray(got)
    ref = np.asarray(ref)
    if got.shape != ref.shape:
        raise AssertionError(f"shape mismatch {got.shape} vs {ref.shape}")
    g = got.astype(np.float64)
    r = ref.astype(np.float64)
    n = g.size
    both_nan = np.isnan(g) & np.isnan(r)
    diff = np.where(both_nan, 0.0, np.abs(g - r))
    diff = np.where(np.isnan(diff), np.inf, diff)
    rel = diff / np.maximum(np.abs(r), 1e-6)
    bad = diff > atol + rtol * np.abs(np.where(np.isnan(r), 0.0, r))
    if got.dtype == ref.dtype:
        same = got.view(np.uint8).reshape(n, -1) if n else np.zeros((0, 1), np.uint8)
        other = ref.view(np.uint8).reshape(n, -1) if n else np.zeros((0, 1), np.uint8)
        bitwise = float(np.all(same == other, axis=1).mean() * 100) if n else 100.0
    else:
        bitwise = float(np.mean(g == r) * 100) if n else 100.0
    worst = np.unravel_index(int(np.argmax(diff)), diff.shape) if n else ()
    failing = [tuple(int(i) for i in idx) for idx in np.argwhere(bad)[:16]]
    return Report(n, float(diff.max()) if n else 0.0, float(rel.max()) if n else 0.0, bitwise,
                  tuple(int(i) for i in worst), failing)


def assert_within(got, ref, atol, rtol=0.0, what=""):
    rep = report(got, ref, atol, rtol)
    if rep.failing:
        raise AssertionError(f"{what}: tolerance gate atol={atol} rtol={rtol} failed: {rep}")
    return rep


def assert_bitwise(got, ref, what=""):
    got = np.ascontiguousarray(got)
    ref = np.ascontiguousarray(ref)
    if got.shape != ref.shape or got.dtype != ref.dtype:
        raise AssertionError(f"{what}: {got.shape}/{got.dtype} vs {ref.shape}/{ref.dtype}")
    a = got.view(np.uint8).reshape(got.size, -1) if got.size else got
    b = ref.view(np.uint8).reshape(ref.size, -1) if ref.size else ref
    if got.size and not np.array_equal(a, b):
        diff_rows = np.flatnonzero(np.any(a != b, axis=1))
        idx = [tuple(int(i) for i in np.unravel_index(int(k), got.shape)) for k in diff_rows[:8]]
        rep = report(got, ref)
        raise AssertionError(f"{what}: {diff_rows.size} of {got.size} elements differ in bits; "
                             f"first {idx}; {rep}")
