"""Pins of the CPU oracle's building blocks against closed forms, hand-derived
examples, brute force and exhaustive scans (no GPU).

Each test fixes one part of the oracle with something other than the oracle's
own formula, so that a dropped term, a wrong sign or index, or a transposed
operand fails here.
"""

import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

from oracle import hardkv_oracle as orc

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _vec(spec, n=128):
    v = np.full(n, spec["fill"], np.float32)
    for k, x in spec.get("set", {}).items():
        v[int(k)] = x
    return v


def _nearest_f32(x: Fraction) -> np.float32:
    """Correctly rounded (ties to even) float32 of an exact rational."""
    f = np.float32(float(x))
    best = None
    for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        err = abs(Fraction(float(cand)) - x)
        key = (err, int(np.array(cand).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return np.float32(best[1])


# ---- score: pairwise tree and max-pooling -------------------------------------------------
def test_pairwise_tree_golden():
    g = _gold("score_tree.json")
    for case in g["cases"]:
        q, k = _vec(case["q"]), _vec(case["k"])
        got = orc.dot_pairwise(q, k)
        assert got == np.float32(case["pairwise"]), case["name"]
        if "left_to_right" in case:
            acc = np.float32(0)
            for x in (q * k):
                acc = np.float32(acc + x)
            assert acc == np.float32(case["left_to_right"]) and acc != got
        if "exact_rounded" in case:
            exact = _nearest_f32(sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(q, k)))
            assert exact == np.float32(case["exact_rounded"]) and exact != got
        if "strided" in case:
            # the other tree shape: level l+1 element i = level l element i + element i + n/2
            lvl = (q * k).astype(np.float32)
            while lvl.size > 1:
                h = lvl.size // 2
                lvl = (lvl[:h] + lvl[h:]).astype(np.float32)
            assert lvl[0] == np.float32(case["strided"]) and lvl[0] != got


def test_signed_zero_score_is_plus_zero():
    g = _gold("score_tree.json")["signed_zero"]
    q = np.full((g["group"], 128), g["q_fill"], np.float32)
    k = np.full(128, g["k_fill"], np.float32)
    s = orc.score_row(q, k)
    assert int(np.array(s).view(np.uint32)) == g["score_bits"]


def test_score_error_bound_against_exact_sum():
    """|d - exact| <= gamma_7 * sum |products| (pairwise depth 7), exact via fsum (I10)."""
    rng = np.random.default_rng(5)
    u = 2.0 ** -24
    gamma7 = 7 * u / (1 - 7 * u)
    for trial in range(300):
        scale = 10.0 ** rng.uniform(-3, 3)
        q = (rng.standard_normal(128) * scale).astype(np.float32)
        k = rng.standard_normal(128).astype(np.float32)
        if trial % 3 == 0:  # bf16-valued operands
            q = (q.view(np.uint32) & 0xFFFF0000).view(np.float32)
            k = (k.view(np.uint32) & 0xFFFF0000).view(np.float32)
        prods = [float(a) * float(b) for a, b in zip(q, k)]  # exact in binary64
        exact = math.fsum(prods)
        bound = gamma7 * math.fsum(abs(p) for p in prods) + 128 * 2.0 ** -149
        d = float(orc.dot_pairwise(q, k))
        assert abs(d - exact) <= bound


def test_score_group_max_g1_and_permutation():
    """G = 1 gives the plain dot; permuting the group's queries leaves the score bit-identical (I9)."""
    rng = np.random.default_rng(6)
    for _ in range(100):
        q = rng.standard_normal((4, 128)).astype(np.float32)
        k = rng.standard_normal(128).astype(np.float32)
        s1 = orc.score_row(q[:1], k)
        assert s1 == orc.dot_pairwise(q[0], k)
        s = orc.score_row(q, k)
        assert s == max(orc.dot_pairwise(q[g], k) for g in range(4))
        for perm in ([3, 2, 1, 0], [1, 3, 0, 2]):
            assert orc.score_row(q[perm], k) == s


# ---- calibration constants -----------------------------------------------------------------
def test_poly_coeffs_correctly_rounded():
    getcontext().prec = 60
    ln2 = Decimal(2).ln()
    got = orc.poly_coeffs()
    assert got.size == 10
    for i in range(10):
        exact = Fraction(ln2 ** i / math.factorial(i))
        assert got[i] == _nearest_f32(exact), i
    assert got[0] == np.float32(1.0)


def test_kappa_and_pq_closed_forms():
    g = _gold("calibration.json")
    getcontext().prec = 60
    exact = Decimal(1) / Decimal(2).ln() / Decimal(128).sqrt()
    assert abs(Decimal(g["kappa_D128_tau1"]["decimal"]) - exact) < Decimal("1e-16")
    assert orc.kappa(128, 1.0) == _nearest_f32(Fraction(exact))
    for D, tau in ((64, 1.0), (128, 0.5), (128, 3.0), (256, 1.7)):
        ex = Fraction(Decimal(1) / Decimal(2).ln() / Decimal(D).sqrt() / Decimal(float(np.float32(tau))))
        k = orc.kappa(D, tau)
        assert abs(Fraction(float(k)) - ex) <= Fraction(float(np.spacing(k))) / 2 * Fraction(1001, 1000)
    assert orc.kappa(128, float("inf")) == 0.0
    for p, v in g["pq"].items():
        if p == "derivation":
            continue
        assert orc.pq(float(p)) == v


def test_weight_at_integer_exponents():
    g = _gold("calibration.json")["weight_at_integer_t"]
    for t, w in g["cases"]:
        assert orc.weight(float(t), 0.0, 1.0) == w, t
        assert orc.weight_of_t(np.array([t], np.float32))[0] == w


def test_exp2_polynomial_exhaustive_monotone_and_accurate():
    """Every fp32 f in [2^-25, 1): 2^f by the polynomial is non-decreasing, within
    2 ulp of binary64 exp2 and at most 2; below 2^-25 it is exactly 1 (I8)."""
    lo = int(np.array(2.0 ** -25, np.float32).view(np.uint32))
    hi = int(np.array(1.0, np.float32).view(np.uint32))
    step = 1 << 23
    prev_last = np.float32(1.0)
    max_ulp = 0.0
    for start in range(lo, hi, step):
        f = np.arange(start, min(start + step, hi), dtype=np.uint32).view(np.float32)
        y = orc.exp2_poly(f)
        ref = np.exp2(f.astype(np.float64))
        ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
        max_ulp = max(max_ulp, float((np.abs(y.astype(np.float64) - ref) / ulp).max()))
        assert np.all(np.diff(y) >= 0)
        assert y[0] >= prev_last
        prev_last = y[-1]
    assert max_ulp <= 2.0, max_ulp
    assert prev_last <= np.float32(2.0)  # joins 2^(n+1) * 1 at the next integer
    rng = np.random.default_rng(1)
    tiny = (rng.uniform(0, 1, 200000) * 2.0 ** rng.uniform(-150, -25, 200000)).astype(np.float32)
    tiny = np.concatenate([tiny, np.array([0.0, np.nextafter(np.float32(2 ** -25), np.float32(0))], np.float32)])
    assert np.all(orc.exp2_poly(tiny) == np.float32(1.0))


def test_weight_monotone_across_reduction_boundaries():
    """w(t) is non-decreasing where floor(t) changes (at integers) and elsewhere, and is
    2^(24+t) within one part in 10^6 (plus the floor)."""
    ts = []
    for k in range(0, 61):
        for c in (np.float32(-k), np.float32(-k - 0.5)):
            for d in range(-8, 9):
                x = c
                step = np.float32(np.inf) if d > 0 else np.float32(-np.inf)
                for _ in range(abs(d)):
                    x = np.nextafter(x, step)
                ts.append(x)
    ts = np.unique(np.array(ts + [np.float32(-60.0), np.float32(0.0)], np.float32))
    ts = ts[(ts >= -60.0) & (ts <= 0)]
    w = orc.weight_of_t(ts)
    assert np.all(np.diff(w.astype(np.int64)) >= 0)
    rng = np.random.default_rng(2)
    t = np.sort(np.concatenate([rng.uniform(-60, 0, 100000), -(2.0 ** rng.uniform(-140, 0, 20000))]).astype(np.float32))
    w = orc.weight_of_t(t).astype(np.float64)
    assert np.all(np.diff(w) >= 0)
    ref = np.exp2(t.astype(np.float64) + 24)
    assert np.all(np.abs(w - np.maximum(1.0, np.floor(ref))) <= ref * 1e-6 + 1)
    assert orc.weight_of_t(np.array([-60.5, -1e30, -np.inf, -0.0], np.float32)).tolist() == [1, 1, 1, 1 << 24]


# ---- top-p -------------------------------------------------------------------------------
def test_topp_golden_examples():
    for ex in _gold("calibration.json")["topp_examples"]:
        k, sel, _ = orc.topp(np.array(ex["w"]), np.array(ex["pos"]), ex["p"])
        assert k == ex["kstar"]
        assert sorted(np.array(ex["pos"])[sel].tolist()) == ex["selected"]


def _pq_py(p):
    return int(round(p * 65536.0))  # Python rounds half to even on the exact binary value


def _brute_force(w, pos, p):
    """Minimal |S| with mass >= T, then maximal mass, then lexicographically smallest
    ascending position tuple, over all 2^n subsets."""
    n = len(w)
    WU = int(np.sum(w, dtype=np.uint64))
    T = -(-_pq_py(p) * WU // 65536)
    masks = np.arange(1 << n, dtype=np.int64)
    bits = ((masks[:, None] >> np.arange(n)) & 1).astype(bool)
    mass = bits.astype(np.int64) @ w.astype(np.int64)
    size = bits.sum(1)
    ok = mass >= T
    kmin = size[ok].min()
    cand = ok & (size == kmin)
    best_mass = mass[cand].max()
    cand &= mass == best_mass
    tuples = [tuple(sorted(pos[bits[i]].tolist())) for i in np.nonzero(cand)[0]]
    return int(kmin), min(tuples)


@pytest.mark.parametrize("seed", range(40))
def test_topp_brute_force(seed):
    """The sorted-prefix selection equals the brute-force definition over all subsets (I2)."""
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 15))
    hi = int(rng.choice([3, 8, 50, 1 << 24]))
    w = rng.integers(1, hi + 1, n).astype(np.uint32)
    pos = rng.permutation(1000)[:n].astype(np.int64)
    p = float(rng.choice([0.01, 0.3, 0.5, 0.8, 0.9, 0.95, 0.99, 1.0, rng.uniform(0.01, 1)]))
    k, sel, T = orc.topp(w, pos, p)
    kb, tup = _brute_force(w, pos, p)
    assert k == kb
    assert tuple(sorted(pos[sel].tolist())) == tup
    # minimal prefix: mass(S) >= T and dropping the lightest selected token falls below (I1)
    ms = int(w[sel].astype(np.int64).sum())
    assert ms >= T and ms - int(w[sel].min()) < T


def test_topp_p1_selects_all_and_monotone_in_p():
    rng = np.random.default_rng(9)
    for _ in range(50):
        n = int(rng.integers(1, 400))
        w = rng.integers(1, 1 << 24, n).astype(np.uint32)
        w[rng.integers(0, n, n // 3)] = w[0]  # ties
        pos = np.arange(n, dtype=np.int64) * 3 + 7
        k, sel, _ = orc.topp(w, pos, 1.0)
        assert k == n and sel.all()  # I3
        order = np.lexsort((pos, -w.astype(np.int64)))  # (w desc, pos asc)
        prev = 0
        for p in (0.1, 0.5, 0.8, 0.9, 0.99, 1.0):  # I5: nested prefixes of one order; top-k equal
            k, sel, _ = orc.topp(w, pos, p)
            assert k >= prev
            prev = k
            assert set(np.nonzero(sel)[0]) == set(order[:k].tolist())


def test_topp_empty():
    k, sel, T = orc.topp(np.zeros(0, np.uint32), np.zeros(0, np.int64), 0.9)
    assert k == 0 and T == 0
