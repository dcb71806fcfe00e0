"""The asynchronous pipeline on the GPU against the oracle: a selection made ahead on a second
stream (hardkv_select_fork on the main stream right after the append of the step it is made
for, hardkv_select_ahead on the side stream) while the main stream keeps taking steps that
reuse the current selection, then switched in (hardkv_condense on the state made ahead).
Selection state bit for bit, attention within 2e-3 at every step."""

import numpy as np
import pytest
import torch

from synth import tiny_workload
from synth.configs import COND_EVICT, COND_MERGE

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    from decode_kv_cache_02_amd import hardkv as hk
    hk.require_gpu()


def _check_selection(g, o, wl, tag):
    """The selection buffers of a GPU state against an oracle state, bit for bit."""
    from parity import raw
    for n in ("budget", "n_condense", "regularized"):
        assert np.array_equal(getattr(g, n).cpu().numpy(), getattr(o, n)), f"{tag} {n}"
    for n in ("w_all", "w_u", "thresh"):
        assert np.array_equal(getattr(g, n).cpu().numpy().view(np.uint64), getattr(o, n)), f"{tag} {n}"
    assert np.array_equal(g.mask.cpu().numpy().view(np.uint64), o.mask), f"{tag} mask"
    budget = o.budget
    vp, vk, vv = g.view_pos.cpu().numpy(), raw(g.view_k), raw(g.view_v)
    for b in range(wl.batch):
        for h in range(wl.num_kv_heads):
            if not o.regularized[b, h]:
                continue
            k = min(int(budget[b, h]), wl.V_cap)
            assert np.array_equal(vp[b, h, :k], o.view_pos[b, h, :k]), f"{tag} view_pos {b} {h}"
            assert np.array_equal(vk[b, h, :k], o.view_k[b, h, :k]), f"{tag} view_k {b} {h}"
            assert np.array_equal(vv[b, h, :k], o.view_v[b, h, :k]), f"{tag} view_v {b} {h}"


def _part(p):
    return p[0], p[1] - p[0]


def _check_cache(g, o, tag):
    from parity import COND_TOL, row_rel_err
    for n in ("pool_head", "cond_cursor", "cond_n", "seq_len"):
        assert np.array_equal(getattr(g, n).cpu().numpy(), getattr(o, n)), f"{tag} {n}"
    on = o.cond_n > 0
    if on.any():
        for n in ("cond_kn", "cond_vn"):
            e = row_rel_err(getattr(g, n).cpu().numpy()[on], getattr(o, n)[on])
            assert e <= COND_TOL, f"{tag} {n} {e}"
        om_g, om_o = g.cond_omega.cpu().numpy()[on], o.cond_omega[on]
        assert np.max(np.abs(om_g - om_o) / np.abs(om_o)) <= COND_TOL, f"{tag} cond_omega"


PIPE_CASES = {
    # fork at step 2, switch `lag` steps later; a second round forks again from the switched state
    "merge_lag1": (dict(cond_mode=COND_MERGE, ctx_len=500, ctx_min=300, sparse_cap=192, condensed_slots=3), 1),
    "merge_lag3": (dict(cond_mode=COND_MERGE, ctx_len=500, ctx_min=300, sparse_cap=192, condensed_slots=3), 3),
    "evict_f32_lag2": (dict(dtype="f32", cond_mode=COND_EVICT), 2),
    "g8_lag2": (dict(num_q_heads=16, num_kv_heads=2, cond_mode=COND_MERGE), 2),
    "sparse_policy_lag2": (dict(cond_mode=COND_MERGE, ctx_len=500, ctx_min=300, regularize=1), 2),
    "batch16_lag1": (dict(batch=16, cond_mode=COND_MERGE, ctx_len=600, ctx_min=100), 1),
    # the selection made ahead in parts, one after each step before the switch, on the main stream
    "batch16_spread3": (dict(batch=16, cond_mode=COND_MERGE, ctx_len=600, ctx_min=100), -3),
    "mixed_spread2": (dict(batch=5, num_q_heads=12, num_kv_heads=3, cond_mode=COND_EVICT), -2),
}


@pytest.mark.parametrize("name", list(PIPE_CASES))
def test_pipeline_parity(name):
    from decode_kv_cache_02_amd import hardkv as hk
    from parity import Pair
    kw, lag = PIPE_CASES[name]
    spread = lag < 0  # the selection in parts on the main stream, one after each step before the switch
    lag = abs(lag)
    kw = dict(kw)
    reg = kw.pop("regularize", 0)
    steps = 2 + 2 * (lag + 2)
    wl = tiny_workload(steps=steps, **kw)
    print(f"case {name}: lag {lag} {wl}", flush=True)
    pr = Pair(wl, regularize=reg)
    o_cur, cpu = pr.orcs[None]
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    pr.step()  # step 0: a selection as usual
    s = 1
    for rnd in range(2):
        # the fork step: a step that reuses the current selection, then the fork behind its append
        st_next = pr.st.twin()
        pr.step_reuse()
        hk.hardkv_select_fork(pr.cfg, st_next, pr.st, main)
        q_fork = pr.inp.q[s]
        units = wl.batch * wl.num_kv_heads
        parts = [(i * units // lag, (i + 1) * units // lag) for i in range(lag)]
        if spread:
            done = None
            hk.hardkv_select_ahead(pr.cfg, st_next, q_fork, main, *_part(parts[0]))
        else:
            forked = torch.cuda.Event()
            forked.record(main)
            with torch.cuda.stream(side):
                side.wait_event(forked)
                hk.hardkv_select_ahead(pr.cfg, st_next, q_fork, side)
                done = torch.cuda.Event()
                done.record(side)
        o_next = o_cur.twin()
        o_next.select_ahead(cpu.q[s], o_cur.seq_len)
        s += 1
        for i in range(lag - 1):  # steps on the current selection while the selection is made
            pr.step_reuse()
            if spread:
                hk.hardkv_select_ahead(pr.cfg, st_next, q_fork, main, *_part(parts[i + 1]))
            s += 1
        # the switch
        if done is not None:
            main.wait_event(done)
        torch.cuda.synchronize()
        _check_selection(st_next, o_next, wl, f"{name} round {rnd} ahead")
        hk.hardkv_condense(pr.cfg, st_next, main)
        o_next.condense_plan()
        o_next.seq_len[:] = o_cur.seq_len
        torch.cuda.synchronize()
        _check_cache(st_next, o_next, f"{name} round {rnd} switch")
        pr.st, o_cur = st_next, o_next
        pr.orcs[None] = (o_cur, cpu)
        pr.step_reuse()  # the first step on the switched selection
        s += 1
    assert int(pr.st.error_word[0].item()) == 0


def test_switch_at_once_equals_the_step():
    """Fork, ahead and switch with nothing in between give hardkv_step's selection state and
    condensed tier bit for bit, and the same outputs on the steps that reuse it."""
    from decode_kv_cache_02_amd import hardkv as hk
    from synth import make_inputs
    wl = tiny_workload(cond_mode=COND_MERGE, ctx_len=500, ctx_min=300, sparse_cap=192, condensed_slots=3, steps=4)
    inp = make_inputs(wl, device="cuda")
    cfg = hk.Config.from_workload(wl)
    ref, cur = hk.State(cfg), hk.State(cfg)
    out_r = torch.zeros((wl.batch, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
    out_c = torch.zeros_like(out_r)
    for st in (ref, cur):
        hk.hardkv_prefill(cfg, st, inp.k_ctx, inp.v_ctx, inp.ctx_len)
    hk.hardkv_step(cfg, ref, inp.q[0], inp.k_new[0], inp.v_new[0], out_r)
    hk.hardkv_step(cfg, cur, inp.q[0], inp.k_new[0], inp.v_new[0], out_c)
    hk.hardkv_step(cfg, ref, inp.q[1], inp.k_new[1], inp.v_new[1], out_r)
    nxt = cur.twin()
    hk.hardkv_append(cfg, cur, inp.k_new[1], inp.v_new[1])
    hk.hardkv_select_fork(cfg, nxt, cur)
    hk.hardkv_select_ahead(cfg, nxt, inp.q[1])
    hk.hardkv_condense(cfg, nxt)
    torch.cuda.synchronize()
    # (the weights and scores by ring row are compared where both states scored: the pool of
    # the step; rows outside it keep whatever each state held)
    for n in ("mask", "budget", "n_condense", "w_all", "w_u", "thresh", "regularized", "cond_n",
              "cond_kn", "cond_vn", "cond_omega", "cond_cursor", "pool_head", "seq_len"):
        assert torch.equal(getattr(ref, n), getattr(nxt, n)), n
    P = wl.P_blk
    t = ref.seq_len.cpu().numpy()
    c0 = (ref.pool_head - 64 * ref.n_condense).cpu().numpy()
    for b in range(wl.batch):
        for h in range(wl.num_kv_heads):
            pos = np.arange(c0[b, h], max(0, t[b] - wl.dense_window))
            rows = torch.from_numpy((pos // 64) % P * 64 + pos % 64).cuda()
            for n in ("weights", "scores"):
                assert torch.equal(getattr(ref, n)[b, h][rows], getattr(nxt, n)[b, h][rows]), (n, b, h)
    k = ref.budget.cpu().numpy()
    for b in range(wl.batch):
        for h in range(wl.num_kv_heads):
            kk = int(k[b, h])
            assert torch.equal(ref.view_k[b, h, :kk], nxt.view_k[b, h, :kk])
            assert torch.equal(ref.view_pos[b, h, :kk], nxt.view_pos[b, h, :kk])
    for s in (2, 3):
        hk.hardkv_step_reuse(cfg, ref, inp.q[s], inp.k_new[s], inp.v_new[s], out_r)
        hk.hardkv_step_reuse(cfg, nxt, inp.q[s], inp.k_new[s], inp.v_new[s], out_c)
        torch.cuda.synchronize()
        assert torch.equal(out_r, out_c), s


def _two_periods(hk, cfg, cur, nxt, inp, steps, outs, main, side, R, lag):
    """Two periods of R steps that reuse the current selection; at the first step of each the
    next selection is forked and made ahead on the side stream, switched in `lag` steps
    later (the states swap roles at each switch)."""
    done = None
    for i, s in enumerate(steps):
        k = i % R
        if k == lag and done is not None:
            main.wait_event(done)
            hk.hardkv_condense(cfg, nxt, main)
            cur, nxt = nxt, cur
            done = None
        hk.hardkv_step_reuse(cfg, cur, inp.q[s], inp.k_new[s], inp.v_new[s], outs[i], main)
        if k == 0:
            hk.hardkv_select_fork(cfg, nxt, cur, main)
            ev = torch.cuda.Event()
            ev.record(main)
            side.wait_event(ev)
            hk.hardkv_select_ahead(cfg, nxt, inp.q[s], side)
            done = torch.cuda.Event()
            done.record(side)
    if done is not None:
        main.wait_event(done)
    return cur, nxt


@pytest.mark.parametrize("layout", ["ring", "shared"])
def test_pipeline_captured_in_a_graph(layout):
    """Two pipelined periods (fork, selection ahead on a second stream, switch) captured in
    one HIP graph with the cross-stream waits and replayed give the eager run's outputs at
    every step and its state bit for bit."""
    from decode_kv_cache_02_amd import hardkv as hk
    from synth import make_inputs
    R, lag = 3, 2
    wl = tiny_workload(batch=4, cond_mode=COND_MERGE, ctx_len=600, ctx_min=100, steps=1 + 2 * R)
    inp = make_inputs(wl, device="cuda")
    cfg = hk.Config.from_workload(wl)
    if layout == "shared":
        nb = hk.hardkv_shared_pool_blocks(cfg, inp.ctx_len.cpu(), wl.steps)
        cfg = hk.Config.from_workload(wl, pool_layout=hk.HARDKV_POOL_SHARED, pool_total_blocks=nb)
    physical = ("pool_k", "pool_v", "block_table", "free_list") if layout == "shared" else ()
    shape = (wl.batch, wl.num_q_heads, wl.head_dim)
    runs = []
    for _ in range(2):
        st = hk.State(cfg)
        hk.hardkv_prefill(cfg, st, inp.k_ctx, inp.v_ctx, inp.ctx_len)
        first = torch.zeros(shape, dtype=torch.float32, device="cuda")
        hk.hardkv_step(cfg, st, inp.q[0], inp.k_new[0], inp.v_new[0], first)  # the selection to start from
        runs.append((st, st.twin(), [torch.zeros(shape, dtype=torch.float32, device="cuda") for _ in range(2 * R)]))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    steps = list(range(1, 1 + 2 * R))
    (ea, eb, eouts), (ga, gb, gouts) = runs
    _two_periods(hk, cfg, ea, eb, inp, steps, eouts, torch.cuda.current_stream(), side, R, lag)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _two_periods(hk, cfg, ga, gb, inp, steps, gouts, torch.cuda.current_stream(), side, R, lag)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    for i in range(2 * R):
        assert torch.equal(eouts[i], gouts[i]), f"step {i}"
    for e, gg in ((ea, ga), (eb, gb)):
        for n, t in e.tensors().items():
            if n == "workspace" or n in physical:
                continue
            assert torch.equal(t, getattr(gg, n)), n
    assert int(ea.error_word[0].item()) == 0
