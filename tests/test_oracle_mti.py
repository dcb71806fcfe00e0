"""Pins of the oracle's memory-time controller (the Rewrite Cache / Sparse Loading switch of
the HARD-KV technical summary 2.C, read as a memory-time integral over the selection step and
the H steps that reuse it): hand-derived decisions, thresholds and reselection periods, and
the step under the controller (no GPU)."""

import numpy as np
import pytest

from oracle import hardkv_oracle as orc
from synth import make_inputs, tiny_workload
from synth.configs import COND_MERGE


def costs(**kw):
    base = dict(mti_horizon=0, mti_c_view=0, mti_c_write=0, mti_c_scan=0, mti_c_hold=0, mti_c_score=0,
                mti_c_gather=[0] * 9, mti_fixed=0)
    base.update(kw)
    return base


def test_no_reuse_never_rewrites():
    """H = 0 (a selection every step): the view would never be read, so no budget is
    rewritten, whatever the costs."""
    rng = np.random.default_rng(3)
    for _ in range(200):
        m = costs(mti_horizon=0, mti_c_view=int(rng.integers(0, 1 << 20)),
                  mti_c_write=int(rng.integers(0, 1 << 20)), mti_c_scan=int(rng.integers(0, 1 << 20)),
                  mti_c_gather=[int(x) for x in rng.integers(0, 1 << 20, 9)],
                  mti_fixed=int(rng.integers(0, 1 << 30)))
        n = int(rng.integers(1, 5000))
        k = int(rng.integers(0, n + 1))
        assert not orc.mti_rewrite(m, k, n)
    assert orc.mti_thresholds(costs(mti_c_gather=[5] * 9), 100) == (0, -1)


def test_dense_mask_upper_threshold():
    """c_view 100, c_write 250, gathers 400 fs per row below a fully kept pool and 100 at it,
    H = 1: a rewrite costs 250 + 100 = 350 per row against 400 gathered, so every budget
    below the survivor count is rewritten; at k* = n the mask covers the whole pool (400 ->
    100) and it is not.  (L_lower, L_upper) = (1, n - 1)."""
    m = costs(mti_horizon=1, mti_c_view=100, mti_c_write=250, mti_c_gather=[400] * 8 + [100])
    assert orc.mti_thresholds(m, 64) == (1, 63)
    assert orc.mti_rewrite(m, 63, 64) and not orc.mti_rewrite(m, 64, 64)
    assert not orc.mti_rewrite(m, 0, 64)


def test_fixed_cost_lower_threshold():
    """The same costs with a fixed 10000 fs per rewritten head: a rewrite wins when
    350 k + 10000 < 400 k, i.e. k > 200; with n = 1000 survivors, k = 1000 falls in the
    dense eighth.  (L_lower, L_upper) = (201, 999); 200 is a tie (80000 = 80000), which
    stays with Sparse Loading."""
    m = costs(mti_horizon=1, mti_c_view=100, mti_c_write=250, mti_c_gather=[400] * 8 + [100], mti_fixed=10000)
    assert orc.mti_thresholds(m, 1000) == (201, 999)
    assert not orc.mti_rewrite(m, 200, 1000) and orc.mti_rewrite(m, 201, 1000)


def test_density_buckets():
    """The gather cost is taken from the kept eighth floor(8 k* / n): with n = 800, k* = 99
    is bucket 0 and k* = 100 bucket 1; only bucket 0 makes gathers dear enough."""
    m = costs(mti_horizon=2, mti_c_view=10, mti_c_write=100, mti_c_gather=[100, 40] + [40] * 7)
    # bucket 0: 100 + 2*10 = 120 < 2*100 = 200 -> rewrite; bucket 1: 120 < 80 -> no
    assert orc.mti_rewrite(m, 99, 800) and not orc.mti_rewrite(m, 100, 800)
    assert orc.mti_thresholds(m, 800) == (1, 99)


def test_scan_and_hold_terms():
    """Walking the mask over n survivors costs the sparse side n c_scan per reused step;
    holding a view row costs the rewrite side c_hold per row and step.  c_view 10,
    c_write 30, gathers 20, H = 2: per row 30 + 20 = 50 against 40, so no rewrite; with
    c_scan 1 and n = 1000 the sparse side gains 2000 and a head of k* = 100 (5000 against
    4000 + 2000) is rewritten, one of k* = 300 (15000 against 12000 + 2000) is not; a
    c_hold of 10 adds 2000 to the rewrite of k* = 100 (7000 against 6000): not rewritten."""
    base = dict(mti_horizon=2, mti_c_view=10, mti_c_write=30, mti_c_gather=[20] * 9)
    assert not orc.mti_rewrite(costs(**base), 100, 1000)
    assert orc.mti_rewrite(costs(**base, mti_c_scan=1), 100, 1000)
    assert not orc.mti_rewrite(costs(**base, mti_c_scan=1), 300, 1000)
    assert not orc.mti_rewrite(costs(**base, mti_c_scan=1, mti_c_hold=10), 100, 1000)


def test_horizon_break_even():
    """With a view read 97000 fs, a write 68000 fs and a gather 124000 fs per row, a rewrite
    pays once H (124000 - 97000) > 68000, i.e. from H = 3 reused steps on."""
    for H, want in ((1, False), (2, False), (3, True), (10, True)):
        m = costs(mti_horizon=H, mti_c_view=97000, mti_c_write=68000, mti_c_gather=[124000] * 9)
        assert orc.mti_rewrite(m, 5000, 15000) == want, H


def test_period_closed_form():
    """With the gathers as cheap as the view (so Sparse Loading, k* g per step, whatever R)
    and a score of n_pool c_score = 50 c_view per selection, the memory time per step is
    k* g + c_view (50 / R + (R - 1) / 2): 9.556, 9.5, 9.545 for R = 9, 10, 11 -> R = 10; a
    cap of 6 gives 6; the score for free gives R = 1."""
    m = costs(mti_c_view=100, mti_c_write=10 ** 6, mti_c_gather=[100] * 9, mti_c_score=50)
    assert orc.mti_period(m, 100, 80, 40, 100) == 10
    assert orc.mti_period(m, 100, 80, 40, 6) == 6
    assert orc.mti_period(costs(mti_c_view=100, mti_c_gather=[100] * 9), 100, 80, 40, 100) == 1


def test_period_switches_policy_with_the_horizon():
    """When a longer period also makes the rewrite pay (H >= 3 with the break-even costs
    above), the period's cost uses the cheaper policy at its own H: a brute-force sum over
    the period confirms the chosen R is the minimum per step."""
    m = costs(mti_c_view=97000, mti_c_write=68000, mti_c_gather=[124000] * 9, mti_c_score=44000)
    n_pool, n, k = 15873, 15809, 11000

    def per_step(R):
        H = R - 1
        sparse = (H + 1) * k * 124000
        rewrite = k * 124000 + k * 68000 + H * k * 97000
        pol = rewrite if rewrite < sparse else sparse
        return (n_pool * 44000 + pol + 97000 * H * (H + 1) // 2) / R

    R = orc.mti_period(m, n_pool, n, k, 400)
    assert R == min(range(1, 401), key=lambda r: (per_step(r), r))
    assert R > 4


def test_step_under_the_controller():
    """The step with the controller rewrites exactly the heads the decision picks from
    their own k* and survivor count, leaves the others' views untouched, and attends the
    same output as rewriting every head."""
    wl = tiny_workload(batch=3, num_kv_heads=2, num_q_heads=8, cond_mode=COND_MERGE, ctx_len=700,
                       ctx_min=300, sparse_cap=256, steps=1, top_p=0.9, heavy=(0, 40))
    inp = make_inputs(wl)
    # costs under which some heads are rewritten and some not: 250 k + 300 k + 250 < 600 k,
    # a lower threshold at k* = 6 (the budgets here are 2 to 9)
    m = costs(mti_horizon=3, mti_c_view=100, mti_c_write=250, mti_c_gather=[200] * 9, mti_fixed=250)
    ref = orc.Oracle(wl)
    mo = orc.Oracle(wl, regularize=3, mti=m)
    for o in (ref, mo):
        assert o.prefill(inp.k_ctx, inp.v_ctx, inp.ctx_len) == 0
    out_ref = ref.step(inp.q[0], inp.k_new[0], inp.v_new[0])
    out_m = mo.step(inp.q[0], inp.k_new[0], inp.v_new[0])
    np.testing.assert_array_equal(out_ref, out_m)
    np.testing.assert_array_equal(ref.budget, mo.budget)
    picked = set()
    for b in range(wl.batch):
        t = int(mo.seq_len[b])
        for h in range(wl.num_kv_heads):
            n = max(0, t - wl.dense_window) - int(mo.pool_head[b, h])
            want = orc.mti_rewrite(m, int(mo.budget[b, h]), n)
            assert bool(mo.regularized[b, h]) == want
            picked.add(want)
            k = int(mo.budget[b, h])
            if want:
                np.testing.assert_array_equal(mo.view_k[b, h, :k], ref.view_k[b, h, :k])
                np.testing.assert_array_equal(mo.view_pos[b, h, :k], ref.view_pos[b, h, :k])
            else:
                assert np.all(mo.view_pos[b, h] == -1)
    assert picked == {True, False}  # the case exercises both sides
