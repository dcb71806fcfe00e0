"""Pins of the oracle's whole step (no GPU): closed forms and identities that the
tiered step must reduce to, and the ring bookkeeping against logical positions."""

import numpy as np
import pytest
import torch

from oracle import hardkv_oracle as orc
from synth import make_inputs, tiny_workload
from synth.configs import COND_EVICT, COND_MERGE, COND_OFF


def _f32(x: torch.Tensor) -> np.ndarray:
    return x.float().cpu().numpy()


def _run(wl, inp, steps=1, **kw):
    o = orc.Oracle(wl, **kw)
    assert o.prefill(inp.k_ctx, inp.v_ctx, inp.ctx_len) == 0
    outs = [o.step(inp.q[s], inp.k_new[s], inp.v_new[s]) for s in range(steps)]
    return o, outs


def _positions_kv(inp, b, h, steps):
    """Keys and values of positions [0, t) of unit (b, h) after `steps` appends."""
    L = int(inp.ctx_len[b])
    k = np.concatenate([_f32(inp.k_ctx[b, h, :L]), _f32(inp.k_new[:steps, b, h])], 0)
    v = np.concatenate([_f32(inp.v_ctx[b, h, :L]), _f32(inp.v_new[:steps, b, h])], 0)
    return k, v


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_p1_off_equals_full_attention(dtype):
    """p = 1 with condensation off: the tiers hold every position once, in order, so the
    tiered attention equals full attention over [0, t) bit for bit, and a library
    softmax attention in binary64 to 1e-12 (I4)."""
    steps = 3
    wl = tiny_workload(dtype=dtype, cond_mode=COND_OFF, top_p=1.0, steps=steps)
    inp = make_inputs(wl)
    o, outs = _run(wl, inp, steps)
    G, D = wl.group, wl.head_dim
    for b in range(wl.batch):
        for h in range(wl.num_kv_heads):
            k, v = _positions_kv(inp, b, h, steps)
            assert o.budget[b, h] == int(inp.ctx_len[b]) + steps - wl.dense_window
            for g in range(G):
                qh = h * G + g
                q = _f32(inp.q[steps - 1, b, qh])
                full = orc.full_attention(q, k, v)
                assert np.array_equal(outs[-1][b, qh], full)
                ref = torch.nn.functional.scaled_dot_product_attention(
                    torch.from_numpy(q.astype(np.float64))[None, None, None],
                    torch.from_numpy(k.astype(np.float64))[None, None],
                    torch.from_numpy(v.astype(np.float64))[None, None])[0, 0, 0].numpy()
                np.testing.assert_allclose(full, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sink_p1_off_equals_full_attention(dtype):
    """A sink prefix of S = 64 with p = 1 and condensation off: sink rows, view rows and
    the dense window hold every position once, in order, so the output equals full
    attention over [0, t) bit for bit; the budget counts the pool alone, [S, t - W)."""
    steps = 3
    wl = tiny_workload(dtype=dtype, cond_mode=COND_OFF, top_p=1.0, steps=steps, sink=64)
    inp = make_inputs(wl)
    o, outs = _run(wl, inp, steps)
    G = wl.group
    for b in range(wl.batch):
        for h in range(wl.num_kv_heads):
            k, v = _positions_kv(inp, b, h, steps)
            assert o.budget[b, h] == int(inp.ctx_len[b]) + steps - wl.dense_window - wl.sink
            for g in range(G):
                qh = h * G + g
                full = orc.full_attention(_f32(inp.q[steps - 1, b, qh]), k, v)
                assert np.array_equal(outs[-1][b, qh], full)


def test_sink_tier_placement():
    """Positions below S sit in the sink rows, from the context and from appends, and in
    no other tier: the pool starts at S and the dense ring holds [max(S, t - W), t).
    Contexts shorter than S grow across it."""
    S, W, steps = 128, 32, 80
    wl = tiny_workload(sink=S, dense_window=W, ctx_len=100, ctx_min=40, steps=steps, cond_mode=COND_MERGE,
                       sparse_cap=128, condensed_slots=2)
    inp = make_inputs(wl)
    o = orc.Oracle(wl)
    assert o.prefill(inp.k_ctx, inp.v_ctx, inp.ctx_len) == 0
    for s in range(steps + 1):
        for b in range(wl.batch):
            t = int(o.seq_len[b])
            L = int(inp.ctx_len[b])
            for h in range(wl.num_kv_heads):
                # keys of positions [0, t) in storage form
                k = np.concatenate([orc._store_np(inp.k_ctx[b, h, :L]), orc._store_np(inp.k_new[:s, b, h])], 0)
                n = min(S, t)
                assert np.array_equal(o.sink_k[b, h, :n], k[:n])
                assert int(o.pool_head[b, h]) >= S
                lo = min(t, max(S, t - W))
                for p in range(lo, t):
                    assert np.array_equal(o.dense_k[b, h, p % W], k[p])
        if s < steps:
            o.step(inp.q[s], inp.k_new[s], inp.v_new[s])


def test_sink_keeps_a_dominant_first_token():
    """Position 0 carries a key that dominates every query and a distinct value.  Under
    eviction with a small sparse cap it leaves the cache without a sink, and the output
    moves away from its value; with S = 64 it stays, and the output is its value."""
    wl = tiny_workload(cond_mode=COND_EVICT, sparse_cap=64, ctx_len=400, ctx_min=400, steps=2)
    inp = make_inputs(wl)
    q = inp.q.float()
    q[..., 0] = 8.0
    inp.q = q.to(inp.q.dtype)
    k = inp.k_ctx.float()
    k[:, :, 0] = 0.0
    k[:, :, 0, 0] = 64.0
    inp.k_ctx = k.to(inp.k_ctx.dtype)
    v = inp.v_ctx.float()
    v[:, :, 0] = 3.0
    inp.v_ctx = v.to(inp.v_ctx.dtype)
    res = {}
    for S in (0, 64):
        o, outs = _run(wl.with_(sink=S), inp, wl.steps)
        res[S] = outs[-1]
    assert np.abs(res[64] - 3.0).max() < 1e-3
    assert np.abs(res[0] - 3.0).max() > 0.5


def test_kappa_zero_closed_form():
    """tau -> inf makes every weight 2^24, so k* = ceil(p_q |U| / 65536) and the
    selection is the lowest positions of U (I6)."""
    wl = tiny_workload(top_p=0.9, cond_mode=COND_EVICT)
    inp = make_inputs(wl)
    o, _ = _run(wl, inp, tau=np.full(wl.num_kv_heads, np.inf, np.float32))
    for b in range(wl.batch):
        for h in range(wl.num_kv_heads):
            c, E = int(o.pool_head[b, h]), int(o.n_condense[b, h])
            pend = int(o.seq_len[b]) - wl.dense_window
            nU = pend - c
            k = -(-58982 * nU // 65536)
            assert o.budget[b, h] == k
            np.testing.assert_array_equal(o.selected_positions(b, h), np.arange(c, c + k))
            idx = o.pool_row_index(np.arange(c - 64 * E, pend))
            assert np.all(o.weights[b, h, idx] == 1 << 24)


@pytest.mark.parametrize("p", [0.5, 0.9, 0.99])
def test_step_selection_matches_logical_restatement(p):
    """Scores, weights, E, U, mask and view of the step equal the pinned building
    blocks applied to the logical positions (ring indexing, plan, survivors) (I7)."""
    wl = tiny_workload(top_p=p, cond_mode=COND_MERGE, heavy=(0, 5))
    inp = make_inputs(wl)
    o, _ = _run(wl, inp)
    G, W = wl.group, wl.dense_window
    for b in range(wl.batch):
        t = int(inp.ctx_len[b]) + 1
        pend = t - W
        N = pend
        E = max(0, -(-(N - wl.sparse_cap) // 64))
        assert np.all(o.n_condense[b] == E) and np.all(o.pool_head[b] == 64 * E)
        for h in range(wl.num_kv_heads):
            k, v = _positions_kv(inp, b, h, 1)
            q = _f32(inp.q[0, b, h * G:(h + 1) * G])
            s = np.array([orc.score_row(q, k[j]) for j in range(pend)], np.float32)
            rows = o.pool_row_index(np.arange(pend))
            assert np.array_equal(o.scores[b, h, rows].view(np.uint32), s.view(np.uint32))
            m = s.max()
            kap = orc.kappa(wl.head_dim, 1.0)
            w = np.array([orc.weight(x, m, kap) for x in s], np.uint32)
            assert np.array_equal(o.weights[b, h, rows], w)
            assert int(o.w_all[b, h]) == int(w.sum(dtype=np.uint64))
            u0 = 64 * E
            kstar, sel, T = orc.topp(w[u0:], np.arange(u0, pend), p)
            assert o.budget[b, h] == kstar and int(o.thresh[b, h]) == T
            chosen = np.arange(u0, pend)[sel]
            np.testing.assert_array_equal(o.selected_positions(b, h), chosen)
            # mask: one bit per selected position, nothing else
            mask = np.zeros(wl.P_blk, np.uint64)
            for j in chosen:
                mask[(j // 64) % wl.P_blk] |= np.uint64(1) << np.uint64(j % 64)
            np.testing.assert_array_equal(o.mask[b, h], mask)
            assert sum(bin(int(x)).count("1") for x in o.mask[b, h]) == kstar
            # view rows are bit copies of the selected positions, in ascending order
            vk = o.view_k[b, h, :kstar]
            src = inp.k_ctx[b, h].contiguous().view(torch.int16).numpy().view(np.uint16)
            np.testing.assert_array_equal(vk, src[chosen])
            assert np.all(np.diff(chosen) > 0)


def test_merge_identical_block_is_lossless():
    """A block of 64 identical tokens merged into an empty slot attends exactly like
    the 64 tokens (ln n bias), with p = 1 so nothing else is dropped (I11)."""
    W, S = 32, 256
    wl = tiny_workload(batch=1, num_kv_heads=2, num_q_heads=8, dense_window=W, sparse_cap=S,
                       ctx_len=S + W, ctx_min=None, cond_mode=COND_MERGE, top_p=1.0, heavy=(0, 0))
    inp = make_inputs(wl)
    inp.k_ctx[:, :, :64] = inp.k_ctx[:, :, :1]
    inp.v_ctx[:, :, :64] = inp.v_ctx[:, :, :1]
    o, outs = _run(wl, inp)
    assert np.all(o.n_condense == 1) and np.all(o.pool_head == 64)
    assert np.all(o.cond_n.sum(-1) == 64) and np.all(o.cond_cursor == 1)
    for h in range(wl.num_kv_heads):
        k, v = _positions_kv(inp, 0, h, 1)
        np.testing.assert_allclose(o.cond_kn[0, h, 0] / o.cond_omega[0, h, 0], k[0], rtol=1e-12)
        for g in range(wl.group):
            qh = h * wl.group + g
            full = orc.full_attention(_f32(inp.q[0, 0, qh]), k, v)
            np.testing.assert_allclose(outs[0][0, qh], full, rtol=1e-12, atol=1e-14)


def test_merge_weights_tau_inf_closed_form():
    """tau -> inf makes every calibrated probability equal: each pool token's weight is
    the maximum 2^24, so the merge weight of a token is 1/N over the N pool tokens of the
    step (including the condensing blocks), a merged block's Omega is 64/N and its Kn, Vn
    the plain sums of its keys and values over N (I6 with I11's numerators).  A weight
    normalised per block (Omega = 1) or over the survivors only (64/(N - 64E)) fails."""
    W, S, E = 32, 128, 2
    L0 = W + S + 64 * E - 1  # the first step's pool holds S + 64E tokens: E blocks condense
    wl = tiny_workload(batch=2, num_kv_heads=2, num_q_heads=8, dense_window=W, sparse_cap=S,
                       ctx_len=L0, ctx_min=None, cond_mode=COND_MERGE, condensed_slots=4,
                       top_p=0.9, heavy=(0, 0), dtype="f32")
    inp = make_inputs(wl)
    o, _ = _run(wl, inp, tau=np.full(wl.num_kv_heads, np.inf, np.float32))
    N = L0 + 1 - W
    assert np.all(o.n_condense == E)
    assert np.all(o.w_all == np.uint64(N) << np.uint64(24))
    for b in range(wl.batch):
        for h in range(wl.num_kv_heads):
            k, v = _positions_kv(inp, b, h, 1)
            for e in range(E):
                blk = slice(64 * e, 64 * (e + 1))
                np.testing.assert_allclose(o.cond_omega[b, h, e], 64.0 / N, rtol=1e-13)
                np.testing.assert_allclose(o.cond_kn[b, h, e], k[blk].astype(np.float64).sum(0) / N,
                                           rtol=1e-11, atol=1e-14)
                np.testing.assert_allclose(o.cond_vn[b, h, e], v[blk].astype(np.float64).sum(0) / N,
                                           rtol=1e-11, atol=1e-14)
            assert np.all(o.cond_omega[b, h, E:] == 0) and np.all(o.cond_n[b, h, E:] == 0)


def test_merge_weights_two_token_classes():
    """Merge weights fixed by construction, across two condensations with different pool
    masses into one slot.  Each query is the unit vector e_0, so a token's score is exactly
    its key's first element, chosen 0 (class A) or -3 (class B); with tau such that
    kappa = fp32(log2(e) / (sqrt(128) tau)) is exactly 1, t = s - max s is 0 or -3 and the
    weights are exactly 2^24 and 2^21 (the integer-exponent weights of the calibration
    golden file).  With C = 1 both condensed blocks land in slot 0, so
    Omega = sum over block 0 of w / W_1 + sum over block 1 of w / W_2, with W_1, W_2 the
    pool masses of the two steps summed here by hand; Kn and Vn are the same weighted sums
    of the raw keys and values (the weighted merging of tier 3, technical summary 2.A)."""
    W, S = 32, 128
    L0 = W + S + 63  # step 1 condenses block [0, 64), step 2 block [64, 128)
    wl = tiny_workload(batch=1, num_kv_heads=1, num_q_heads=4, dense_window=W, sparse_cap=S,
                       ctx_len=L0, ctx_min=None, cond_mode=COND_MERGE, condensed_slots=1,
                       top_p=0.9, heavy=(0, 0), dtype="f32", steps=2)
    inp = make_inputs(wl)
    rng = np.random.default_rng(11)
    cls_a = rng.random(L0 + 2) < 0.3  # class of every position [0, L0 + 2)
    cls_a[[5, 100, 150]] = True       # a class-A token in each step's pool: max s = 0
    first = np.where(cls_a, 0.0, -3.0).astype(np.float32)
    inp.k_ctx[0, 0, :L0, 0] = torch.from_numpy(first[:L0])
    inp.k_new[:, 0, 0, 0] = torch.from_numpy(first[L0:L0 + 2])
    inp.q.zero_()
    inp.q[..., 0] = 1.0
    tau = np.float32(1.4426950408889634 / np.sqrt(128.0))
    assert np.float32(1.4426950408889634 / (np.sqrt(128.0) * np.float64(tau))) == np.float32(1.0)
    assert orc.kappa(128, float(tau)) == np.float32(1.0)
    o, _ = _run(wl, inp, steps=2, tau=np.array([tau], np.float32))
    w = np.where(cls_a, 1 << 24, 1 << 21).astype(np.int64)
    W1 = int(w[0:L0 + 1 - W].sum())        # pool of step 1: [0, 192)
    W2 = int(w[64:L0 + 2 - W].sum())       # pool of step 2: [64, 193)
    assert W1 != W2
    assert int(o.w_all[0, 0]) == W2 and int(o.pool_head[0, 0]) == 128
    k, v = _positions_kv(inp, 0, 0, 2)
    om = np.concatenate([w[0:64] / W1, w[64:128] / W2])
    assert o.cond_n[0, 0, 0] == 128 and o.cond_cursor[0, 0] == 0
    np.testing.assert_allclose(o.cond_omega[0, 0, 0], om.sum(), rtol=1e-13)
    kv = k[:128].astype(np.float64)
    vv = v[:128].astype(np.float64)
    np.testing.assert_allclose(o.cond_kn[0, 0, 0], (om[:, None] * kv).sum(0), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(o.cond_vn[0, 0, 0], (om[:, None] * vv).sum(0), rtol=1e-11, atol=1e-14)


def test_condense_bookkeeping_modes():
    """Merged slots count 64 tokens per condensed block; evict leaves the slots
    untouched; off never condenses (I11)."""
    base = dict(ctx_len=700, ctx_min=400, sparse_cap=128, dense_window=32, condensed_slots=3)
    for mode in (COND_MERGE, COND_EVICT, COND_OFF):
        wl = tiny_workload(cond_mode=mode, **base)
        inp = make_inputs(wl)
        o, _ = _run(wl, inp, steps=1)
        for b in range(wl.batch):
            N = int(inp.ctx_len[b]) + 1 - wl.dense_window
            E = max(0, -(-(N - 128) // 64)) if mode != COND_OFF else 0
            assert np.all(o.n_condense[b] == E)
            assert np.all(o.pool_head[b] == 64 * E)
            if mode == COND_MERGE:
                assert np.all(o.cond_n[b].sum(-1) == 64 * E)
                assert np.all(o.cond_cursor[b] == E % 3)
                # ring wrap: slot s received ceil((E - s) / 3) blocks
                for s in range(3):
                    assert np.all(o.cond_n[b, :, s] == 64 * len(range(s, E, 3)))
            else:
                assert np.all(o.cond_n[b] == 0) and np.all(o.cond_omega[b] == 0)
            if mode == COND_OFF:
                assert np.all(o.budget[b] > 0)
    assert o.error_word == 0


def test_one_token_and_equal_keys():
    """One token: the output is its value.  Equal keys: the mean of the values (I12)."""
    wl = tiny_workload(batch=1, ctx_len=0, ctx_min=None, heavy=(0, 0))
    inp = make_inputs(wl)
    o, outs = _run(wl, inp)
    for qh in range(wl.num_q_heads):
        np.testing.assert_array_equal(outs[0][0, qh], _f32(inp.v_new[0, 0, qh // wl.group]).astype(np.float64))
    wl = tiny_workload(batch=1, ctx_len=20, ctx_min=None, heavy=(0, 0))
    inp = make_inputs(wl)
    inp.k_ctx[:] = inp.k_ctx[:, :, :1]
    inp.k_new[:] = inp.k_ctx[:, :, 0]
    o, outs = _run(wl, inp)
    for qh in range(wl.num_q_heads):
        h = qh // wl.group
        mean = np.concatenate([_f32(inp.v_ctx[0, h, :20]), _f32(inp.v_new[0, 0, h])[None]]).astype(np.float64).mean(0)
        np.testing.assert_allclose(outs[0][0, qh], mean, rtol=1e-12, atol=1e-14)


def test_error_bits():
    # pool overflow in mode off
    wl = tiny_workload(cond_mode=COND_OFF, ctx_len=400, ctx_min=None, pool_blocks=5, view_cap=320)
    inp = make_inputs(wl)
    o = orc.Oracle(wl)
    assert o.prefill(inp.k_ctx, inp.v_ctx, inp.ctx_len) == -3  # does not fit
    wl = tiny_workload(cond_mode=COND_OFF, ctx_len=320 + 32 - 1, ctx_min=None, pool_blocks=5, view_cap=320, steps=2)
    inp = make_inputs(wl)
    o = orc.Oracle(wl)
    assert o.prefill(inp.k_ctx, inp.v_ctx, inp.ctx_len) == 0
    o.step(inp.q[0], inp.k_new[0], inp.v_new[0])
    assert o.error_word == 0
    o.step(inp.q[1], inp.k_new[1], inp.v_new[1])
    assert o.error_word & 1
    # non-finite score
    wl = tiny_workload()
    inp = make_inputs(wl)
    inp.k_ctx[0, 0, 5, 0] = float("inf")
    o, _ = _run(wl, inp)
    assert o.error_word & 4


def test_streaming_invariants():
    """Over many steps the pool head stays block aligned, the pool stays within S_cap
    after condensation, and t advances by one per step."""
    wl = tiny_workload(steps=70, ctx_len=330, ctx_min=300, cond_mode=COND_MERGE, condensed_slots=2)
    inp = make_inputs(wl)
    o = orc.Oracle(wl)
    o.prefill(inp.k_ctx, inp.v_ctx, inp.ctx_len)
    total_E = np.zeros((wl.batch, wl.num_kv_heads), np.int64)
    for s in range(wl.steps):
        o.step(inp.q[s], inp.k_new[s], inp.v_new[s], attend=(s % 10 == 0))
        total_E += o.n_condense
        assert np.all(o.seq_len == inp.ctx_len.numpy() + s + 1)
        assert np.all(o.pool_head % 64 == 0)
        N = o.seq_len[:, None] - wl.dense_window - o.pool_head
        assert np.all(N <= wl.sparse_cap) and np.all(N >= 0)
        assert np.all(o.budget >= 1)
    assert np.all(o.cond_n.sum(-1) == 64 * total_E)
    assert o.error_word == 0


# ---- regularize policy: Rewrite Cache vs Sparse Loading ------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sparse_loading_attends_the_same_rows(dtype):
    """Sparse Loading reads the kept rows from the pool instead of the view; the view rows
    are bit copies of those pool rows in the same order, so the attention output is the
    same bit for bit over several steps, masks and budgets agree, and no view row or
    view position is written."""
    wl = tiny_workload(dtype=dtype, cond_mode=COND_MERGE, steps=3, ctx_len=500, ctx_min=100)
    inp = make_inputs(wl)
    o_rw, outs_rw = _run(wl, inp, 3)
    o_sp, outs_sp = _run(wl, inp, 3, regularize=1)
    for a, b in zip(outs_rw, outs_sp):
        assert np.array_equal(a, b)
    for n in ("mask", "budget", "weights", "cond_kn", "cond_n", "pool_head"):
        assert np.array_equal(getattr(o_rw, n), getattr(o_sp, n)), n
    assert not o_sp.regularized.any() and o_rw.regularized.all()
    assert (o_sp.view_pos == -1).all() and not o_sp.view_k.any()
    for b in range(wl.batch):
        for h in range(wl.num_kv_heads):
            np.testing.assert_array_equal(o_sp.selected_positions(b, h), o_rw.selected_positions(b, h))


def test_mti_thresholds_pick_heads_by_budget():
    """MTI policy: a head is rewritten iff L_lower <= k* <= L_upper; rewritten heads hold
    the same view as under Rewrite Cache, the others keep whatever the view held before;
    the attention output does not depend on the choice."""
    wl = tiny_workload(cond_mode=COND_EVICT, steps=2, heavy=(0, 6), batch=4)
    inp = make_inputs(wl)
    o_rw, outs_rw = _run(wl, inp, 1)
    vals = np.unique(o_rw.budget)
    assert len(vals) >= 3, vals
    lo, hi = int(vals[1]), int(vals[-2])
    o_m, outs_m = _run(wl, inp, 1, regularize=2, mti_lower=lo, mti_upper=hi)
    assert np.array_equal(outs_rw[0], outs_m[0])
    rw = (o_m.budget >= lo) & (o_m.budget <= hi)
    assert rw.any() and (~rw).any()
    np.testing.assert_array_equal(o_m.regularized.astype(bool), rw)
    for b in range(wl.batch):
        for h in range(wl.num_kv_heads):
            k = int(o_m.budget[b, h])
            if rw[b, h]:
                np.testing.assert_array_equal(o_m.view_k[b, h, :k], o_rw.view_k[b, h, :k])
                np.testing.assert_array_equal(o_m.view_pos[b, h, :k], o_rw.view_pos[b, h, :k])
            else:
                assert (o_m.view_pos[b, h] == -1).all()


# ---- Flatten Index to the sum (packed, CSR views) --------------------------------------
@pytest.mark.parametrize("policy", [0, 2])
def test_packed_views_are_the_concatenation(policy):
    """The sum layout packs each rewritten head's view rows (the same rows as the
    maximum-length layout) in unit order: view_off is the exclusive prefix sum of the
    rewritten budgets, the packed rows and positions are the per-head ones concatenated,
    and attention is unchanged."""
    wl = tiny_workload(cond_mode=COND_MERGE, steps=2, heavy=(0, 6), batch=4, ctx_len=500, ctx_min=100)
    inp = make_inputs(wl)
    pol = dict(regularize=policy)
    if policy == 2:
        o0, _ = _run(wl, inp, 1)
        vals = np.unique(o0.budget)
        pol.update(mti_lower=int(vals[1]), mti_upper=int(vals[-2]))
    total = wl.batch * wl.num_kv_heads * wl.V_cap
    o_max, outs_max = _run(wl, inp, 2, **pol)
    o_sum, outs_sum = _run(wl, inp, 2, view_layout=1, view_total=total, **pol)
    for a, b in zip(outs_max, outs_sum):
        assert np.array_equal(a, b)
    n = (o_sum.budget * o_sum.regularized).ravel().astype(np.int64)
    np.testing.assert_array_equal(o_sum.view_off, np.concatenate([[0], np.cumsum(n)]))
    for u in range(wl.batch * wl.num_kv_heads):
        b, h = divmod(u, wl.num_kv_heads)
        k, off = int(n[u]), int(o_sum.view_off[u])
        np.testing.assert_array_equal(o_sum.view_k[off:off + k], o_max.view_k[b, h, :k])
        np.testing.assert_array_equal(o_sum.view_v[off:off + k], o_max.view_v[b, h, :k])
        np.testing.assert_array_equal(o_sum.view_pos[off:off + k], o_max.view_pos[b, h, :k])
    assert o_sum.error_word == 0


def test_packed_views_overflow():
    """Fewer packed rows than the budgets need: the overflow bit, and rows past the end are
    not written (the ones before are the concatenation's prefix)."""
    wl = tiny_workload(cond_mode=COND_EVICT, steps=1)
    inp = make_inputs(wl)
    o_max, _ = _run(wl, inp, 1)
    need = int(o_max.budget.sum())
    o, _ = _run(wl, inp, 1, view_layout=1, view_total=need - 5)
    assert o.error_word & 2
    flat = np.concatenate([o_max.view_pos[b, h, :o_max.budget[b, h]]
                           for b in range(wl.batch) for h in range(wl.num_kv_heads)])
    np.testing.assert_array_equal(o.view_pos, flat[:need - 5])


# ---- calibration temperature fitted by entropy ------------------------------------------
_GRID_LOG2 = 24.0 / 16 ** 5   # width of the last bracket of the search, in log2 tau


def _dots(q, k):
    """Pairwise-tree dots of every query with every key, as the score computes them."""
    return np.array([[orc.dot_pairwise(qg, kr) for kr in k] for qg in q], np.float32)


@pytest.mark.parametrize("G", [1, 4])
def test_fit_tau_identical_queries_gives_one(G):
    """With every query of the group equal (G = 1 is the plain case), the max-pooled score
    is the raw dot, so the calibrated softmax at tau = 1 is the raw attention and has its
    entropy: the fitted tau is 1 to within the last bracket of the search."""
    rng = np.random.default_rng(11)
    q1 = rng.standard_normal(128).astype(np.float32)
    k = rng.standard_normal((300, 128)).astype(np.float32)
    d = _dots(np.repeat(q1[None], G, 0), k)
    s = d.max(0)
    tau, h = orc.fit_tau(d, s)
    assert abs(np.log2(tau)) <= _GRID_LOG2 + 1e-12, tau
    assert abs(orc.calibrated_entropy(s, 1.0) - h) < 1e-12


def test_fit_tau_matches_target_entropy():
    """For a real group (different queries) the fitted tau reproduces the target entropy up
    to the slope of the entropy over the last bracket, and sharper calibrated softmaxes
    (smaller tau) have lower entropy."""
    rng = np.random.default_rng(12)
    q = rng.standard_normal((4, 128)).astype(np.float32) * np.array([[0.5], [1.0], [2.0], [3.0]], np.float32)
    k = rng.standard_normal((500, 128)).astype(np.float32)
    d = _dots(q, k)
    s = d.max(0)
    tau, h = orc.fit_tau(d, s)
    lo, hi = tau * 2 ** -_GRID_LOG2, tau * 2 ** _GRID_LOG2
    e_lo, e_hi = orc.calibrated_entropy(s, lo), orc.calibrated_entropy(s, hi)
    assert e_lo - 1e-9 <= h <= e_hi + 1e-9, (e_lo, h, e_hi)
    ts = [0.1, 0.3, 1.0, 3.0]
    es = [orc.calibrated_entropy(s, t) for t in ts]
    assert all(a < b for a, b in zip(es, es[1:])), es


def test_entropy_calibration_step_uses_the_fitted_tau():
    """The step with the fitted temperature equals the step with that temperature given per
    unit (the override the GPU parity uses), and reports the temperature it used."""
    wl = tiny_workload(cond_mode=COND_MERGE, steps=1, ctx_len=500, ctx_min=100)
    inp = make_inputs(wl)
    o_fit, outs_fit = _run(wl, inp, 1, calibration=1)
    taus = o_fit.tau_fit.copy()
    assert np.all(taus > 0) and np.all(np.isfinite(taus))
    o_ovr, outs_ovr = _run(wl, inp, 1, calibration=1, tau_unit=taus)
    for n in ("weights", "mask", "budget", "thresh"):
        assert np.array_equal(getattr(o_fit, n), getattr(o_ovr, n)), n
    assert np.array_equal(outs_fit[0], outs_ovr[0])
    np.testing.assert_array_equal(o_ovr.tau_fit, taus)


# ---- steps that reuse the last selection ---------------------------------------------------
def _reuse_run(wl, inp, pattern, **kw):
    """pattern: a string of 's' (a step with selection) and 'r' (a step reusing it)."""
    o = orc.Oracle(wl, **kw)
    assert o.prefill(inp.k_ctx, inp.v_ctx, inp.ctx_len) == 0
    outs = []
    for s, ch in enumerate(pattern):
        if ch == "s":
            outs.append(o.step(inp.q[s], inp.k_new[s], inp.v_new[s]))
        else:
            outs.append(o.step_reuse(inp.q[s], inp.k_new[s], inp.v_new[s]))
    return o, outs


@pytest.mark.parametrize("pattern", ["srrr", "rrsr", "r"])
def test_reuse_p1_off_equals_full_attention(pattern):
    """p = 1 without condensation: the last selection kept its whole pool and every later
    pool position is attended in full, so each step, with or without selection (before
    the first selection too), is full attention over [0, t) bit for bit."""
    steps = len(pattern)
    wl = tiny_workload(cond_mode=COND_OFF, top_p=1.0, steps=steps)
    inp = make_inputs(wl)
    o, outs = _reuse_run(wl, inp, pattern)
    G = wl.group
    for s in range(steps):
        for b in range(wl.batch):
            for h in range(wl.num_kv_heads):
                k, v = _positions_kv(inp, b, h, s + 1)
                for g in range(G):
                    qh = h * G + g
                    full = orc.full_attention(_f32(inp.q[s, b, qh]), k, v)
                    assert np.array_equal(outs[s][b, qh], full), (s, b, h, g)


@pytest.mark.parametrize("policy", [0, 1])
def test_reuse_attends_the_selection_and_what_came_after(policy):
    """Eviction at p = 0.9, one selection and then three steps without one: the attended
    set is the selection's kept positions, every pool position that arrived after it and
    the dense window, so the output is full attention over exactly those positions, in
    order (Rewrite Cache: from the view; Sparse Loading: from the pool through the mask)."""
    pattern = "srrr"
    wl = tiny_workload(steps=len(pattern), dense_window=16)
    inp = make_inputs(wl)
    o = orc.Oracle(wl, regularize=policy)
    assert o.prefill(inp.k_ctx, inp.v_ctx, inp.ctx_len) == 0
    outs = [o.step(inp.q[0], inp.k_new[0], inp.v_new[0])]
    kept = {(b, h): o.selected_positions(b, h) for b in range(wl.batch) for h in range(wl.num_kv_heads)}
    t_sel = o.seq_len.copy()
    assert all(len(kept[u]) == o.budget[u] for u in kept) and o.budget.min() > 0
    for s in range(1, len(pattern)):
        outs.append(o.step_reuse(inp.q[s], inp.k_new[s], inp.v_new[s]))
        assert np.array_equal(o.seq_len, t_sel + s)
    G, W = wl.group, wl.dense_window
    s = len(pattern) - 1
    for b in range(wl.batch):
        t = int(o.seq_len[b])
        for h in range(wl.num_kv_heads):
            k, v = _positions_kv(inp, b, h, s + 1)
            pos = np.concatenate([kept[b, h], np.arange(int(t_sel[b]) - W, t - W), np.arange(t - W, t)])
            assert np.all(np.diff(pos) > 0)
            for g in range(G):
                qh = h * G + g
                ref = orc.full_attention(_f32(inp.q[s, b, qh]), k[pos], v[pos])
                assert np.array_equal(outs[s][b, qh], ref), (b, h, g)


def test_reuse_then_select_condenses_the_grown_pool():
    """Steps without selection condense nothing, so the pool grows past S_cap; the next
    selection condenses it back (its E counts the blocks the reuse steps added), and the
    pool head and cursor advance as in a run of selections that kept up."""
    pattern = "s" + "r" * 70 + "s"
    wl = tiny_workload(steps=len(pattern), ctx_len=330, ctx_min=300, cond_mode=COND_MERGE, condensed_slots=3,
                       dense_window=16)
    inp = make_inputs(wl)
    o, _ = _reuse_run(wl, inp, pattern)
    N = o.seq_len[:, None] - wl.dense_window - o.pool_head
    assert np.all(N <= wl.sparse_cap) and np.all(o.pool_head % 64 == 0)
    assert np.all(o.n_condense >= 1) and o.error_word == 0
    assert np.all(o.cond_n.sum(-1) == 64 * (o.pool_head // 64))


def test_reuse_with_sinks_p1_off_equals_full_attention():
    """A sink prefix of S = 64 under steps that reuse a selection: at p = 1 without
    condensation every step is still full attention over [0, t) bit for bit."""
    pattern = "srrsr"
    wl = tiny_workload(cond_mode=COND_OFF, top_p=1.0, steps=len(pattern), sink=64)
    inp = make_inputs(wl)
    o, outs = _reuse_run(wl, inp, pattern)
    G = wl.group
    for s in range(len(pattern)):
        for b in range(wl.batch):
            for h in range(wl.num_kv_heads):
                k, v = _positions_kv(inp, b, h, s + 1)
                for g in range(G):
                    full = orc.full_attention(_f32(inp.q[s, b, h * G + g]), k, v)
                    assert np.array_equal(outs[s][b, h * G + g], full), (s, b, h, g)


def test_reuse_with_merged_slots_matches_a_flat_softmax():
    """With merged slots, a step that reuses the selection attends: each occupied slot as
    one entry with key Kn/Omega, value Vn/Omega and logit bias ln n, then the kept rows,
    the positions since the selection and the dense window.  A plain binary64 softmax
    over exactly those entries, built here from the state and the inputs, agrees to
    1e-12."""
    pattern = "srrr"
    wl = tiny_workload(steps=len(pattern), cond_mode=COND_MERGE, ctx_len=500, ctx_min=400, condensed_slots=3,
                       dense_window=16)
    inp = make_inputs(wl)
    o = orc.Oracle(wl)
    assert o.prefill(inp.k_ctx, inp.v_ctx, inp.ctx_len) == 0
    o.step(inp.q[0], inp.k_new[0], inp.v_new[0])
    assert o.cond_n.sum() > 0
    kept = {(b, h): o.selected_positions(b, h) for b in range(wl.batch) for h in range(wl.num_kv_heads)}
    t_sel = o.seq_len.copy()
    outs = None
    for s in range(1, len(pattern)):
        outs = o.step_reuse(inp.q[s], inp.k_new[s], inp.v_new[s])
    s = len(pattern) - 1
    G, W, D = wl.group, wl.dense_window, wl.head_dim
    for b in range(wl.batch):
        t = int(o.seq_len[b])
        for h in range(wl.num_kv_heads):
            k, v = _positions_kv(inp, b, h, s + 1)
            pos = np.concatenate([kept[b, h], np.arange(int(t_sel[b]) - W, t - W), np.arange(t - W, t)])
            occ = np.nonzero(o.cond_n[b, h] > 0)[0]
            om = o.cond_omega[b, h][occ][:, None]
            keys = np.concatenate([o.cond_kn[b, h][occ] / om, k[pos].astype(np.float64)])
            vals = np.concatenate([o.cond_vn[b, h][occ] / om, v[pos].astype(np.float64)])
            bias = np.concatenate([np.log(o.cond_n[b, h][occ].astype(np.float64)), np.zeros(len(pos))])
            for g in range(G):
                q = _f32(inp.q[s, b, h * G + g]).astype(np.float64)
                lg = keys @ q / np.sqrt(D) + bias
                e = np.exp(lg - lg.max())
                ref = (e[:, None] * vals).sum(0) / e.sum()
                np.testing.assert_allclose(outs[b, h * G + g], ref, rtol=1e-12, atol=1e-14)
