"""Pins of the oracle's asynchronous pipeline (technical summary 2.A: the four stages run as
an asynchronous pipeline; reading: the next selection is made on the side for the step it is
launched at, while steps continue on the current selection, and switched in later): a
selection switched in at once is the step's own selection; with p = 1 and no condensation
every step of a pipelined schedule is full attention; a lagged switch merges exactly the
blocks planned at the snapshot, with the snapshot's weights (no GPU)."""

import numpy as np
import pytest
import torch

from oracle import hardkv_oracle as orc
from synth import make_inputs, tiny_workload
from synth.configs import COND_MERGE, COND_OFF


def _f32(x):
    return x.float().cpu().numpy()


def test_switch_at_once_is_the_steps_own_selection():
    """Ahead at step 1 (after its append) and switched in at once leaves the selection state
    bit-identical to a step with selection at 1; the next steps that reuse it then give the
    same outputs bit for bit."""
    wl = tiny_workload(cond_mode=COND_MERGE, ctx_len=500, ctx_min=300, sparse_cap=192, condensed_slots=3,
                       steps=4)
    inp = make_inputs(wl)
    ref, a = orc.Oracle(wl), orc.Oracle(wl)
    for o in (ref, a):
        assert o.prefill(inp.k_ctx, inp.v_ctx, inp.ctx_len) == 0
        o.step(inp.q[0], inp.k_new[0], inp.v_new[0])
    ref.step(inp.q[1], inp.k_new[1], inp.v_new[1])
    a.step_reuse(inp.q[1], inp.k_new[1], inp.v_new[1])  # the append of step 1 (and a's own attention)
    b = a.twin()
    b.select_ahead(inp.q[1], a.seq_len)
    b.condense_plan()
    for n in ("mask", "budget", "n_condense", "w_all", "w_u", "thresh", "regularized", "pool_head", "cond_n",
              "cond_cursor", "pend_sel", "weights", "scores", "seq_len"):
        assert np.array_equal(getattr(ref, n), getattr(b, n)), n
    for n in ("cond_kn", "cond_vn", "cond_omega"):
        assert np.array_equal(getattr(ref, n), getattr(b, n)), n
    for bb in range(wl.batch):
        for h in range(wl.num_kv_heads):
            k = int(ref.budget[bb, h])
            assert np.array_equal(ref.view_k[bb, h, :k], b.view_k[bb, h, :k])
            assert np.array_equal(ref.view_pos[bb, h, :k], b.view_pos[bb, h, :k])
    for s in (2, 3):
        o1 = ref.step_reuse(inp.q[s], inp.k_new[s], inp.v_new[s])
        o2 = b.step_reuse(inp.q[s], inp.k_new[s], inp.v_new[s])
        assert np.array_equal(o1, o2), s


@pytest.mark.parametrize("lag", [1, 3])
def test_pipeline_p1_off_is_full_attention(lag):
    """p = 1 with condensation off: whichever selection a step attends (the current one, or
    one made ahead and switched in `lag` steps later), its kept rows, the positions since it
    and the dense window hold every position once, so every step is full attention (1e-12)."""
    steps = 8
    wl = tiny_workload(cond_mode=COND_OFF, top_p=1.0, steps=steps, ctx_len=200, ctx_min=150)
    inp = make_inputs(wl)
    cur = orc.Oracle(wl)
    assert cur.prefill(inp.k_ctx, inp.v_ctx, inp.ctx_len) == 0
    ahead, switch_at = None, None
    G = wl.group
    for s in range(steps):
        if s == 0:
            out = cur.step(inp.q[s], inp.k_new[s], inp.v_new[s])
        else:
            if s == switch_at:
                ahead.condense_plan()
                ahead.seq_len[:] = cur.seq_len
                cur, ahead, switch_at = ahead, None, None
            out = cur.step_reuse(inp.q[s], inp.k_new[s], inp.v_new[s])
            if s == 2:  # a selection made ahead for step 2, switched in `lag` steps later
                ahead = cur.twin()
                ahead.select_ahead(inp.q[s], cur.seq_len)
                switch_at = s + lag
        for b in range(wl.batch):
            L = int(inp.ctx_len[b])
            k = np.concatenate([_f32(inp.k_ctx[b, :, :L]), _f32(inp.k_new[:s + 1, b]).transpose(1, 0, 2)], 1)
            v = np.concatenate([_f32(inp.v_ctx[b, :, :L]), _f32(inp.v_new[:s + 1, b]).transpose(1, 0, 2)], 1)
            for qh in range(wl.num_q_heads):
                full = orc.full_attention(_f32(inp.q[s, b, qh]), k[qh // G], v[qh // G])
                np.testing.assert_allclose(out[b, qh], full, rtol=1e-12, atol=1e-13)


def test_lagged_switch_merges_the_snapshot_blocks():
    """tau -> inf (every weight 2^24): the selection made ahead at a pool of N_snap tokens plans
    E blocks and merge weights 1/N_snap; switched in 3 steps later (the pool has grown by 3),
    each merged slot holds Omega = 64 / N_snap and the plain key sum over N_snap, and the pool
    head moves by 64 E."""
    W, S = 32, 128
    L0 = W + S + 64 + 10  # one block to condense at the first selection
    wl = tiny_workload(batch=2, num_kv_heads=2, num_q_heads=8, dense_window=W, sparse_cap=S, ctx_len=L0,
                       ctx_min=None, cond_mode=COND_MERGE, condensed_slots=4, steps=6, heavy=(0, 0), dtype="f32")
    inp = make_inputs(wl)
    cur = orc.Oracle(wl, tau=np.full(2, np.inf, np.float32))
    assert cur.prefill(inp.k_ctx, inp.v_ctx, inp.ctx_len) == 0
    cur.step_reuse(inp.q[0], inp.k_new[0], inp.v_new[0])  # no selection yet: append only
    ahead = cur.twin()
    ahead.select_ahead(inp.q[0], cur.seq_len)
    N_snap = L0 + 1 - W
    E = -(-(N_snap - S) // 64)
    assert np.all(ahead.n_condense == E) and np.all(cur.pool_head == 0)
    for s in (1, 2, 3):
        cur.step_reuse(inp.q[s], inp.k_new[s], inp.v_new[s])
    ahead.condense_plan()
    assert np.all(cur.pool_head == 64 * E)  # shared with the state made ahead
    for b in range(wl.batch):
        for h in range(wl.num_kv_heads):
            L = int(inp.ctx_len[b])
            keys = _f32(inp.k_ctx[b, h, :L]).astype(np.float64)
            for e in range(E):
                np.testing.assert_allclose(cur.cond_omega[b, h, e], 64.0 / N_snap, rtol=1e-13)
                np.testing.assert_allclose(cur.cond_kn[b, h, e], keys[64 * e:64 * (e + 1)].sum(0) / N_snap,
                                           rtol=1e-11, atol=1e-14)
    assert np.all(cur.cond_cursor == E % 4)
