"""Pins of the oracle's destructive selection (HARD-KV technical summary 2.A: the sparse tier
retains only the tokens top-p selects; read as a mode in which a selection drops for good the
survivors it does not keep, with selections on the caller's schedule): with p = 1 it is the
per-step view; with every weight equal (tau -> inf) the budgets, kept positions and merged
slots follow closed forms; on random heads a selection only ever keeps rows the last one kept
or rows that arrived since (no GPU)."""

import numpy as np
import pytest

from oracle import hardkv_oracle as orc
from synth import make_inputs, tiny_workload
from synth.configs import COND_EVICT, COND_MERGE

BK = 64


def _kept_positions(o, b, h):
    P = o.wl.P_blk
    c = int(o.pool_head[b, h])
    t = int(o.seq_len[b])
    pend = max(int(getattr(o.wl, "sink", 0)), t - o.wl.dense_window)
    out = []
    for p in range(c, pend):
        if (int(o.mask[b, h, (p // BK) % P]) >> (p % BK)) & 1:
            out.append(p)
    return out


@pytest.mark.parametrize("cond", [COND_MERGE, COND_EVICT])
def test_p1_is_the_view(cond):
    """p = 1 keeps every survivor, so nothing is ever dropped: destructive and per-step view
    selection leave the same state and outputs bit for bit, over selections, steps that reuse
    them and condensations."""
    wl = tiny_workload(cond_mode=cond, top_p=1.0, ctx_len=500, ctx_min=300, sparse_cap=256,
                       condensed_slots=3, steps=6)
    inp = make_inputs(wl)
    a = orc.Oracle(wl)
    d = orc.Oracle(wl, selection=orc.SEL_DESTRUCTIVE)
    for o in (a, d):
        assert o.prefill(inp.k_ctx, inp.v_ctx, inp.ctx_len) == 0
    for s, kind in enumerate("srsrrs"):
        if kind == "s":
            oa = a.step(inp.q[s], inp.k_new[s], inp.v_new[s])
            od = d.step(inp.q[s], inp.k_new[s], inp.v_new[s])
        else:
            oa = a.step_reuse(inp.q[s], inp.k_new[s], inp.v_new[s])
            od = d.step_reuse(inp.q[s], inp.k_new[s], inp.v_new[s])
        np.testing.assert_array_equal(oa, od)
        for n in ("mask", "budget", "weights", "w_all", "w_u", "thresh", "pool_head", "cond_kn", "cond_vn",
                  "cond_omega", "cond_n", "cond_cursor"):
            np.testing.assert_array_equal(getattr(a, n), getattr(d, n), err_msg=f"step {s} {n}")


def test_equal_weights_closed_form():
    """tau -> inf: every row in play weighs 2^24, so a selection keeps the k = ceil(p_q n / 65536)
    lowest positions of the n rows in play.  After a first selection over the N survivors and a
    arrivals, the destructive second selection chooses among k1 + a rows (the per-step view
    among N + a): k2 = ceil(p_q (k1 + a) / 65536), the k2 lowest of the kept rows and arrivals;
    the dropped rows weigh 0."""
    W, a_steps = 32, 20
    wl = tiny_workload(batch=2, num_kv_heads=2, num_q_heads=8, dense_window=W, sparse_cap=4096, ctx_len=900,
                       ctx_min=600, cond_mode=COND_MERGE, top_p=0.8, steps=2 + a_steps, heavy=(0, 0))
    inp = make_inputs(wl)
    tau = np.full(2, np.inf, np.float32)
    d = orc.Oracle(wl, tau=tau, selection=orc.SEL_DESTRUCTIVE)
    v = orc.Oracle(wl, tau=tau)
    for o in (d, v):
        assert o.prefill(inp.k_ctx, inp.v_ctx, inp.ctx_len) == 0
        o.step(inp.q[0], inp.k_new[0], inp.v_new[0])
    pq = orc.pq(0.8)
    first = {}
    for b in range(wl.batch):
        t = int(d.seq_len[b])
        n = t - W  # every survivor (no sinks, nothing condensed)
        k1 = -(-pq * n // 65536)
        for h in range(wl.num_kv_heads):
            assert int(d.budget[b, h]) == k1
            first[b, h] = _kept_positions(d, b, h)
            assert first[b, h] == list(range(k1))
    for s in range(1, 1 + a_steps):
        for o in (d, v):
            o.step_reuse(inp.q[s], inp.k_new[s], inp.v_new[s])
    s = 1 + a_steps
    for o in (d, v):
        o.step(inp.q[s], inp.k_new[s], inp.v_new[s])
    P = wl.P_blk
    for b in range(wl.batch):
        t = int(d.seq_len[b])
        pend = t - W
        t1 = t - (a_steps + 1)
        arrivals = list(range(t1 - W, pend))  # the pool end at the first selection, to now
        for h in range(wl.num_kv_heads):
            live = first[b, h] + arrivals
            k2 = -(-pq * len(live) // 65536)
            assert int(d.budget[b, h]) == k2
            assert _kept_positions(d, b, h) == sorted(live)[:k2]
            assert int(v.budget[b, h]) == -(-pq * pend // 65536)
            for p in range(pend):
                w = int(d.weights[b, h, (p // BK) % P * BK + p % BK])
                assert w == (1 << 24 if p in set(live) else 0), p


def test_merge_of_a_block_with_dropped_rows():
    """tau -> inf with a condensation at the second selection: each merged block adds to its
    slot only its rows in play, Omega = (rows in play of the block) / (rows in play of the
    pool), n = rows in play of the block, and the key numerator their plain sum over the rows
    in play of the pool."""
    W = 32
    L0 = W + 256 + 30
    wl = tiny_workload(batch=2, num_kv_heads=2, num_q_heads=8, dense_window=W, sparse_cap=256, ctx_len=L0,
                       ctx_min=None, cond_mode=COND_MERGE, condensed_slots=8, top_p=0.2, steps=70, heavy=(0, 0),
                       dtype="f32")
    inp = make_inputs(wl)
    d = orc.Oracle(wl, tau=np.full(2, np.inf, np.float32), selection=orc.SEL_DESTRUCTIVE)
    assert d.prefill(inp.k_ctx, inp.v_ctx, inp.ctx_len) == 0
    # the pool holds 287 rows: one block condenses and the first selection keeps the 45
    # lowest of the 223 survivors (positions 64 .. 108), so the next oldest block is part
    # dropped
    d.step(inp.q[0], inp.k_new[0], inp.v_new[0])
    assert np.all(d.n_condense == 1)
    kept1 = {(b, h): _kept_positions(d, b, h) for b in range(2) for h in range(2)}
    c1 = d.pool_head.copy()
    n0 = d.cond_n.copy()
    om0 = d.cond_omega.copy()
    kn0 = d.cond_kn.copy()
    for s in range(1, 69):
        d.step_reuse(inp.q[s], inp.k_new[s], inp.v_new[s])
    d.step(inp.q[69], inp.k_new[69], inp.v_new[69])
    for b in range(2):
        t = int(d.seq_len[b])
        pend = t - W
        arr_lo = (t - 69) - W  # the pool end at the first selection
        for h in range(2):
            live = sorted(set(kept1[b, h]) | set(range(arr_lo, pend)))
            E = int(d.n_condense[b, h])
            assert E >= 1
            c = int(c1[b, h])
            cur = (int(d.cond_cursor[b, h]) - E) % 8
            keys = np.concatenate([inp.k_ctx[b, h, :L0].float().numpy(),
                                   inp.k_new[:70, b, h].float().numpy()]).astype(np.float64)
            assert 0 < len([p for p in live if c <= p < c + BK]) < BK  # the first merged block is part dropped
            for e in range(E):
                blk = [p for p in live if c + BK * e <= p < c + BK * (e + 1)]
                sl = (cur + e) % 8
                assert int(d.cond_n[b, h, sl]) - int(n0[b, h, sl]) == len(blk)
                np.testing.assert_allclose(d.cond_omega[b, h, sl] - om0[b, h, sl], len(blk) / len(live),
                                           rtol=1e-13, atol=1e-15)
                want = keys[blk].sum(0) / len(live) if blk else np.zeros(wl.head_dim)
                np.testing.assert_allclose(d.cond_kn[b, h, sl] - kn0[b, h, sl], want, rtol=1e-11, atol=1e-13)


def test_selection_keeps_only_rows_in_play():
    """Random heads, selections every 3 steps: every kept position was kept by the previous
    selection or arrived after it, every dropped survivor weighs 0, a row once dropped is
    never kept again, and the rows in play are calibrated against their own maximum (each
    weight equals the pinned weight function of its score and that maximum)."""
    wl = tiny_workload(batch=3, num_kv_heads=2, num_q_heads=8, cond_mode=COND_MERGE, ctx_len=700, ctx_min=400,
                       sparse_cap=512, condensed_slots=4, top_p=0.9, steps=13)
    inp = make_inputs(wl)
    d = orc.Oracle(wl, selection=orc.SEL_DESTRUCTIVE)
    assert d.prefill(inp.k_ctx, inp.v_ctx, inp.ctx_len) == 0
    prev = None
    dropped = {(b, h): set() for b in range(3) for h in range(2)}
    P = wl.P_blk
    for s in range(13):
        if s % 3:
            d.step_reuse(inp.q[s], inp.k_new[s], inp.v_new[s])
            continue
        pend_prev = d.pend_sel.copy()
        d.step(inp.q[s], inp.k_new[s], inp.v_new[s])
        cur = {}
        for b in range(3):
            t = int(d.seq_len[b])
            pend = t - wl.dense_window
            for h in range(2):
                kept = set(_kept_positions(d, b, h))
                cur[b, h] = kept
                if prev is not None:
                    ok = prev[b, h] | set(range(int(pend_prev[b, h]), pend))
                    assert kept <= ok
                    assert not (kept & dropped[b, h])
                    for p in range(int(d.pool_head[b, h]), pend):
                        if p not in ok:
                            assert int(d.weights[b, h, (p // BK) % P * BK + p % BK]) == 0
                    dropped[b, h] |= set(range(int(d.pool_head[b, h]), pend)) - kept
                    # the calibration maximum over the rows in play, this selection's pool
                    c0 = int(d.pool_head[b, h]) - BK * int(d.n_condense[b, h])
                    live = [p for p in range(c0, pend) if p in ok]
                    rows = [(p // BK) % P * BK + p % BK for p in live]
                    m = max(float(d.scores[b, h, r]) for r in rows)
                    kap = orc.kappa(wl.head_dim, wl.tau)
                    for r in rows[:: max(1, len(rows) // 50)]:
                        assert int(d.weights[b, h, r]) == orc.weight(float(d.scores[b, h, r]), m, kap)
                else:
                    dropped[b, h] |= set(range(int(d.pool_head[b, h]), pend)) - kept
        prev = cur


def test_destructive_needs_a_fixed_temperature_and_no_pipeline():
    wl = tiny_workload()
    with pytest.raises(ValueError):
        orc.Oracle(wl, selection=orc.SEL_DESTRUCTIVE, calibration=1)
    inp = make_inputs(wl)
    d = orc.Oracle(wl, selection=orc.SEL_DESTRUCTIVE)
    assert d.prefill(inp.k_ctx, inp.v_ctx, inp.ctx_len) == 0
    d.step_reuse(inp.q[0], inp.k_new[0], inp.v_new[0])
    with pytest.raises(RuntimeError):
        d.twin().select_ahead(inp.q[0], d.seq_len)
