"""Checkpoint and resume: the state is plain caller-owned device memory (the cache, the
selection arrays, the counters and the workspace, which keeps each head's last plan for
the steps that reuse it), so a snapshot is a copy of every state buffer.  Run k steps,
snapshot, run on; then restore the snapshot into the same state, into a freshly allocated
one, and from a copy written and read back through torch.save / torch.load(weights_only),
and run the same steps again: every output and every result array is bit-identical."""

import io

import pytest
import torch

from decode_kv_cache_02_amd import hardkv as hk
from synth import make_inputs, tiny_workload
from synth.configs import COND_EVICT, COND_MERGE

pytestmark = pytest.mark.gpu

# result arrays that every kernel writes deterministically (the shared pool's block table
# and free list hold blocks in an order that atomics decide, and the workspace holds
# scratch of the same kind, so those are compared through the results they produce)
RESULTS = ("dense_k", "dense_v", "view_k", "view_v", "view_pos", "cond_kn", "cond_vn", "cond_omega", "cond_n",
           "cond_cursor", "seq_len", "pool_head", "scores", "weights", "mask", "budget", "n_condense", "w_all",
           "w_u", "thresh", "regularized", "error_word")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    hk.require_gpu()


CASES = {
    # (workload, config extras, steps before the snapshot, steps after it; s: a step with
    # selection, r: a step that reuses the last one)
    "merge": (dict(cond_mode=COND_MERGE, ctx_len=600, ctx_min=300, sparse_cap=256, condensed_slots=3), {}, "ssr",
              "srrs"),
    "evict_f32_sink": (dict(dtype="f32", cond_mode=COND_EVICT, sink=64, ctx_len=500, ctx_min=100), {}, "sr", "rss"),
    "shared_pool": (dict(batch=4, cond_mode=COND_MERGE, ctx_len=600, ctx_min=100), dict(pool_layout=1), "ss",
                    "srsr"),
    "destructive": (dict(cond_mode=COND_MERGE, ctx_len=600, ctx_min=300, sparse_cap=256, condensed_slots=3),
                    dict(selection=1), "srs", "rsrs"),
}


def _buffers(st):
    return {n: getattr(st, n) for n in hk._STATE_PTRS if getattr(st, n, None) is not None}


def _run(cfg, st, inp, pattern, s0, out):
    outs = []
    for i, ch in enumerate(pattern):
        s = s0 + i
        if ch == "s":
            hk.hardkv_step(cfg, st, inp.q[s], inp.k_new[s], inp.v_new[s], out)
        else:
            hk.hardkv_step_reuse(cfg, st, inp.q[s], inp.k_new[s], inp.v_new[s], out)
        outs.append(out.clone())
    torch.cuda.synchronize()
    return outs


def _results(st):
    return {n: getattr(st, n).clone() for n in RESULTS if getattr(st, n, None) is not None}


def _same(a, b, tag):
    for n in a:
        x, y = a[n], b[n]
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.uint8) if y.dtype == torch.bfloat16 else y), f"{tag}: {n} differs"


@pytest.mark.parametrize("name", list(CASES))
def test_snapshot_restore_resume(name):
    kw, extra, before, after = CASES[name]
    wl = tiny_workload(steps=len(before) + len(after), **kw)
    print(f"case {name}: {before}|{after} {extra}", flush=True)
    inp = make_inputs(wl, device="cuda")
    if extra.get("pool_layout") == 1:
        ring = hk.Config.from_workload(wl)
        extra = dict(extra, pool_total_blocks=hk.hardkv_shared_pool_blocks(ring, inp.ctx_len.cpu(), wl.steps))
    cfg = hk.Config.from_workload(wl, **extra)
    st = hk.State(cfg)
    out = torch.zeros((wl.batch, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
    hk.hardkv_prefill(cfg, st, inp.k_ctx, inp.v_ctx, inp.ctx_len)
    _run(cfg, st, inp, before, 0, out)
    snap = {n: t.clone() for n, t in _buffers(st).items()}
    outs_a = _run(cfg, st, inp, after, len(before), out)
    res_a = _results(st)

    # restored in place (the same buffers, so a captured graph of the step stays valid)
    for n, t in _buffers(st).items():
        t.copy_(snap[n])
    outs_b = _run(cfg, st, inp, after, len(before), out)
    for i, (x, y) in enumerate(zip(outs_a, outs_b)):
        assert torch.equal(x, y), f"in place: output of step {i} after the snapshot differs"
    _same(res_a, _results(st), "in place")

    # restored into a freshly allocated state, from a copy that went through host memory
    # and a serialized file
    buf = io.BytesIO()
    torch.save({n: t.cpu() for n, t in snap.items()}, buf)
    buf.seek(0)
    host = torch.load(buf, weights_only=True)
    fresh = hk.State(cfg)
    for n, t in _buffers(fresh).items():
        t.copy_(host[n])
    out2 = torch.zeros_like(out)
    outs_c = _run(cfg, fresh, inp, after, len(before), out2)
    for i, (x, y) in enumerate(zip(outs_a, outs_c)):
        assert torch.equal(x, y), f"fresh state: output of step {i} after the snapshot differs"
    _same(res_a, _results(fresh), "fresh state")
    assert int(fresh.error_word[0].item()) == 0
