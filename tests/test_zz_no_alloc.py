"""hardkv_step_noalloc (the step with the library's static scratch in place of the state's
workspace) gives exactly what hardkv_step gives, through the C ABI, on two calls in a row
whose second layer is smaller than the first: every output and every state buffer, bit
for bit, over several steps."""

import numpy as np
import pytest
import torch

from synth import get_workload, make_inputs, tiny_workload
from synth.configs import COND_MERGE

pytestmark = pytest.mark.gpu

# the first layer larger than the second; the scratch keeps the first one's contents
LAYERS = [
    ("merge_bf16_b6", tiny_workload(batch=6, num_q_heads=16, num_kv_heads=4, cond_mode=COND_MERGE,
                                    ctx_len=900, ctx_min=500, sparse_cap=256, condensed_slots=3, steps=3)),
    ("evict_f32_b2", tiny_workload(batch=2, dtype="f32", ctx_len=300, ctx_min=100, steps=2)),
]

STATE = ("dense_k", "dense_v", "pool_k", "pool_v", "view_k", "view_v", "view_pos", "cond_kn", "cond_vn",
         "cond_omega", "cond_n", "cond_cursor", "seq_len", "pool_head", "scores", "weights", "mask",
         "budget", "n_condense", "w_all", "w_u", "thresh", "regularized", "error_word")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    from decode_kv_cache_02_amd import hardkv as hk
    hk.require_gpu()


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                       b.view(torch.uint8) if b.dtype != torch.uint8 else b)


def _run_pair(wl):
    from decode_kv_cache_02_amd import hardkv as hk
    dev = "cuda:0"
    inp = make_inputs(wl, device=dev)
    cfg = hk.Config.from_workload(wl)
    assert hk.hardkv_workspace_size(cfg) <= hk.HARDKV_STATIC_SCRATCH_BYTES
    ref, na = hk.State(cfg, device=dev), hk.State(cfg, device=dev)
    for st in (ref, na):
        hk.hardkv_prefill(cfg, st, inp.k_ctx, inp.v_ctx, inp.ctx_len)
    o_ref = torch.zeros((wl.batch, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device=dev)
    o_na = torch.full_like(o_ref, float("nan"))
    for s in range(wl.steps):
        hk.hardkv_step(cfg, ref, inp.q[s], inp.k_new[s], inp.v_new[s], o_ref)
        hk.hardkv_step_noalloc(cfg, na, inp.q[s], inp.k_new[s], inp.v_new[s], o_na)
        torch.cuda.synchronize()
        assert torch.isfinite(o_ref).all()
        assert _same(o_ref, o_na), f"output differs at step {s}"
        for n in STATE:
            assert _same(getattr(ref, n), getattr(na, n)), f"{n} differs at step {s}"
    assert int(ref.error_word[0].item()) == 0


def test_noalloc_matches_step_on_two_layers_in_a_row():
    for name, wl in LAYERS:
        print(f"layer {name}: {wl}", flush=True)
        _run_pair(wl)


def test_noalloc_16k_layer_then_a_tiny_one():
    """A 16k-context batch of 4 (fused products in hardkv_step, plain ones in the no-alloc
    step: the same bits) and then a tiny layer."""
    wl = get_workload("c2").with_(batch=4, steps=2)
    print(f"layer c2 batch 4: {wl}", flush=True)
    _run_pair(wl)
    _run_pair(LAYERS[1][1])


def test_noalloc_over_a_shared_pool():
    """The no-alloc step over the shared block pool: the same outputs and selection state as
    hardkv_step (the pools' physical blocks may be taken in another order, so the pool
    arrays are compared through the outputs)."""
    from decode_kv_cache_02_amd import hardkv as hk
    wl = tiny_workload(batch=6, num_q_heads=16, num_kv_heads=4, cond_mode=COND_MERGE, ctx_len=900, ctx_min=300,
                       sparse_cap=256, condensed_slots=3, steps=3)
    print(f"shared pool: {wl}", flush=True)
    dev = "cuda:0"
    inp = make_inputs(wl, device=dev)
    nb = hk.hardkv_shared_pool_blocks(hk.Config.from_workload(wl), inp.ctx_len.cpu(), wl.steps)
    cfg = hk.Config.from_workload(wl, pool_layout=hk.HARDKV_POOL_SHARED, pool_total_blocks=nb)
    ref, na = hk.State(cfg, device=dev), hk.State(cfg, device=dev)
    for st in (ref, na):
        hk.hardkv_prefill(cfg, st, inp.k_ctx, inp.v_ctx, inp.ctx_len)
    o_ref = torch.zeros((wl.batch, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device=dev)
    o_na = torch.full_like(o_ref, float("nan"))
    for s in range(wl.steps):
        hk.hardkv_step(cfg, ref, inp.q[s], inp.k_new[s], inp.v_new[s], o_ref)
        hk.hardkv_step_noalloc(cfg, na, inp.q[s], inp.k_new[s], inp.v_new[s], o_na)
        torch.cuda.synchronize()
        assert _same(o_ref, o_na), f"output differs at step {s}"
        for n in STATE:
            if n in ("pool_k", "pool_v"):
                continue
            assert _same(getattr(ref, n), getattr(na, n)), f"{n} differs at step {s}"
        assert int(ref.free_top[0].item()) == int(na.free_top[0].item())
    assert int(ref.error_word[0].item()) == 0


def test_noalloc_rejects_a_step_beyond_its_scratch():
    from decode_kv_cache_02_amd import hardkv as hk
    import ctypes as C
    wl = get_workload("c3").with_(batch=128)
    cfg = hk.Config.from_workload(wl)
    assert hk.hardkv_workspace_size(cfg) > hk.HARDKV_STATIC_SCRATCH_BYTES
    st = hk.hardkv_state()
    assert hk.lib().hardkv_step_noalloc(C.byref(cfg.c), C.byref(st), None, None, None, None, None) \
        == hk.HARDKV_ESCRATCH
