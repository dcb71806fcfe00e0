"""Parity on the five benchmark workloads at their full sizes, with the kernels and
launch geometry bench.py times.  Small layers are compared with the oracle on every
(sequence, KV head) unit; large ones on a sample of units run by the oracle one by one,
and on every unit through properties that hold at any size."""

import numpy as np
import pytest
import torch

from synth import get_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    from decode_kv_cache_02_amd import hardkv as hk
    hk.require_gpu()
    yield
    torch.cuda.empty_cache()


def _sample_units(wl, n, seed, lens=None):
    rng = np.random.default_rng(seed)
    units = {(0, 0), (wl.batch - 1, wl.num_kv_heads - 1)}
    if lens is not None:  # the shortest and the longest sequences
        units |= {(int(np.argmin(lens)), 1 % wl.num_kv_heads), (int(np.argmax(lens)), 2 % wl.num_kv_heads)}
    while len(units) < min(n, wl.batch * wl.num_kv_heads):
        units.add((int(rng.integers(wl.batch)), int(rng.integers(wl.num_kv_heads))))
    return sorted(units)


def test_c1_full_layer():
    """Batch 1, fp32, 4096-token context with 16 planted heavy keys per head."""
    from parity import Pair, check_layer_properties
    wl = get_workload("c1").with_(steps=3)
    print("workload", wl.name, flush=True)
    pr = Pair(wl)
    for _ in range(wl.steps):
        pr.step()
        check_layer_properties(pr)


def test_c2_full_layer():
    """Batch 16, 16k context, per-head query temperature in [0.3, 3], p = 0.95."""
    from parity import Pair, check_layer_properties
    wl = get_workload("c2").with_(steps=2)
    print("workload", wl.name, flush=True)
    pr = Pair(wl)
    for _ in range(wl.steps):
        pr.step()
        check_layer_properties(pr)


def test_c2_sink_prefix():
    """The same layer with the first 1024 positions kept as a sink tier: every unit."""
    from parity import Pair, check_layer_properties
    wl = get_workload("c2").with_(steps=2, sink=1024)
    print("workload", wl.name, "sink", wl.sink, flush=True)
    pr = Pair(wl)
    for _ in range(wl.steps):
        pr.step()
        check_layer_properties(pr)


def test_c2_memory_time_controller():
    """The same layer under the memory-time controller: the default per-row costs, a horizon
    of 7 reused steps (a rewrite saves 7 (124000 - 97000) - 68000 = 121000 fs per kept row)
    and a fixed cost per head of 121000 fs times 10000, so heads keeping more than 10000
    rows are rewritten and the others gathered; every unit's rewrite flag, mask, budget and
    views against the oracle, then two steps that reuse the selection."""
    from parity import Pair, check_layer_properties
    wl = get_workload("c2").with_(steps=3)
    print("workload", wl.name, "memory-time controller", flush=True)
    pr = Pair(wl, regularize=3, mti=dict(mti_horizon=7, mti_fixed=121000 * 10000))
    pr.step()
    check_layer_properties(pr)
    rw = pr.st.regularized.cpu().numpy()
    assert rw.any() and not rw.all(), rw
    pr.step_reuse()
    pr.step_reuse()


@pytest.mark.parametrize("p", [0.8, 0.9, 0.99])
def test_c3_mixed_lengths(p):
    """Batch 64, lengths 8k..32k, 0..64 heavy keys per head, the first step condenses up
    to 377 blocks per head into 256 slots (ring wrap)."""
    from parity import Pair, check_layer_properties
    wl = get_workload("c3")
    print("workload", wl.name, "p", p, flush=True)
    from synth import make_inputs
    inp = make_inputs(wl, device="cuda")
    lens = inp.ctx_len.cpu().numpy()
    pr = Pair(wl, inputs=inp, top_p=p, oracle_units=_sample_units(wl, 24, 3, lens))
    pr.drop_context()
    pr.step()
    check_layer_properties(pr)
    assert int(pr.st.n_condense.max()) > 256  # the condensed ring wrapped


def test_c3_shared_pool():
    """c3 in the shared block pool sized by the prefilled lengths: about 60% of the rings'
    blocks; the same outputs and selection bits as the ring layout, sampled units against
    the oracle, the layer's properties (views read through the block table) and the
    conservation of blocks after the step."""
    from decode_kv_cache_02_amd import hardkv as hk
    from parity import Pair, check_layer_properties
    from synth import make_inputs
    wl = get_workload("c3")
    print("workload", wl.name, "shared pool", flush=True)
    inp = make_inputs(wl, device="cuda")
    lens = inp.ctx_len.cpu().numpy()
    ring_cfg = hk.Config.from_workload(wl)
    ring = hk.State(ring_cfg)
    hk.hardkv_prefill(ring_cfg, ring, inp.k_ctx, inp.v_ctx, inp.ctx_len)
    out_ring = torch.zeros((wl.batch, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
    hk.hardkv_step(ring_cfg, ring, inp.q[0], inp.k_new[0], inp.v_new[0], out_ring)
    torch.cuda.synchronize()
    keep = {n: getattr(ring, n).clone() for n in ("mask", "budget", "n_condense", "cond_kn", "cond_omega")}
    del ring
    torch.cuda.empty_cache()
    pr = Pair(wl, inputs=inp, oracle_units=_sample_units(wl, 16, 7, lens), pool_layout=hk.HARDKV_POOL_SHARED)
    nb = int(pr.cfg.c.pool_total_blocks)
    ratio = nb / (wl.batch * wl.num_kv_heads * wl.P_blk)
    print(f"shared pool {nb} blocks, {ratio:.3f} of the rings", flush=True)
    assert ratio < 0.7
    pr.drop_context()
    pr.step()
    check_layer_properties(pr)
    assert torch.equal(pr.out, out_ring)
    for n, t in keep.items():
        assert torch.equal(getattr(pr.st, n), t), n


def test_c4_streaming_256_steps():
    """Batch 4, 128k context, 256 decode steps; blocks condense at steps 1, 65, 129, 193."""
    from parity import Pair, check_layer_properties
    wl = get_workload("c4")
    print("workload", wl.name, flush=True)
    pr = Pair(wl, oracle_units=[(0, 0), (1, 3), (2, 5), (3, 7)])
    pr.drop_context()
    sampled = {0, 1, 63, 64, 65, 128, 200, 255}
    for s in range(wl.steps):
        full = s in sampled
        pr.step(attend=full, check_attend=full, check_views=full)
        if full:
            check_layer_properties(pr)
            print("step", s, "ok", flush=True)
    assert int(pr.st.seq_len[0]) == 131072 + 256


def test_c4_streaming_destructive():
    """The streaming workload under destructive selection: every selection chooses among
    the last one's kept rows and the arrivals since, so the kept set shrinks to a few rows
    per head; selection state on the sampled units at every step, attention and views at
    the sampled steps, the layer's properties on every unit."""
    from decode_kv_cache_02_amd import hardkv as hk
    from parity import Pair, check_layer_properties
    wl = get_workload("c4")
    print("workload", wl.name, "destructive", flush=True)
    pr = Pair(wl, oracle_units=[(0, 1), (1, 6), (2, 2), (3, 4)], selection=hk.HARDKV_SEL_DESTRUCTIVE)
    pr.drop_context()
    sampled = {0, 1, 2, 64, 65, 130, 255}
    for s in range(wl.steps):
        full = s in sampled
        pr.step(attend=full, check_attend=full, check_views=full)
        if full:
            check_layer_properties(pr)
            print("step", s, "ok, budgets", pr.st.budget.flatten()[:8].tolist(), flush=True)
    assert int(pr.st.seq_len[0]) == 131072 + 256
    assert int(pr.st.error_word[0].item()) == 0


@pytest.mark.parametrize("layer", [0, 17, 31])
def test_c5_layers(layer):
    """Layers of the 32-layer batch-32, 16k-context step (each layer is independent)."""
    from parity import Pair, check_layer_properties
    wl = get_workload("c5")
    print("workload", wl.name, "layer", layer, flush=True)
    pr = Pair(wl, layer=layer, oracle_units=_sample_units(wl, 12, 50 + layer))
    pr.drop_context()
    pr.step()
    check_layer_properties(pr)
