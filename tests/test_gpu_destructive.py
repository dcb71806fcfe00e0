"""Destructive selection on the GPU against the oracle (a selection drops for good the
survivors it does not keep; the next one chooses among its kept rows and the positions that
arrived since): every selection state array bit for bit, the condensed tier within 1e-4 and
the attention within 2e-3 at every step, over fused, composed and reusing steps."""

import pytest

from synth import tiny_workload
from synth.configs import COND_EVICT, COND_MERGE

pytestmark = pytest.mark.gpu

DESTRUCTIVE = 1


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    from decode_kv_cache_02_amd import hardkv as hk
    hk.require_gpu()
    assert hk.HARDKV_SEL_DESTRUCTIVE == DESTRUCTIVE


CASES = {
    # (workload, extra Pair arguments, pattern: s fused step, c composed calls, r reuse)
    # a selection every step: the tier shrinks to what top-p keeps of the arrivals
    "merge_every_step": (dict(cond_mode=COND_MERGE, ctx_len=500, ctx_min=300, sparse_cap=256, condensed_slots=3),
                         {}, "ssssss"),
    "evict_f32": (dict(dtype="f32", cond_mode=COND_EVICT, ctx_len=500, ctx_min=200), {}, "srrscs"),
    # blocks with dropped rows condense (every selection after the first condenses)
    "merge_condensing": (dict(cond_mode=COND_MERGE, ctx_len=700, ctx_min=500, sparse_cap=192, condensed_slots=4,
                              top_p=0.5), {}, "s" + "r" * 70 + "sr"),
    "g8": (dict(num_q_heads=16, num_kv_heads=2, cond_mode=COND_MERGE, ctx_len=600, ctx_min=300), {}, "srrrsrs"),
    "batch16": (dict(batch=16, cond_mode=COND_MERGE, ctx_len=600, ctx_min=100), {}, "srrsrrs"),
    "sink": (dict(sink=64, cond_mode=COND_MERGE, ctx_len=500, ctx_min=100), {}, "srrsrs"),
    "sparse_policy": (dict(cond_mode=COND_MERGE, ctx_len=500, ctx_min=100), dict(regularize=1), "srrsrs"),
    "packed": (dict(cond_mode=COND_MERGE, ctx_len=500, ctx_min=100), "packed", "srrss"),
    "shared_pool": (dict(batch=4, cond_mode=COND_MERGE, ctx_len=600, ctx_min=100), dict(pool_layout=1), "srrsrs"),
    # the split select (five slices of the ring)
    "split": (dict(pool_blocks=1100, sparse_cap=4096, ctx_len=3000, ctx_min=2000, cond_mode=COND_MERGE),
              {}, "srrs"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_destructive_parity(name):
    from parity import Pair, check_layer_properties
    kw, extra, pattern = CASES[name]
    wl = tiny_workload(steps=len(pattern), **kw)
    if extra == "packed":
        extra = dict(view_layout=1, view_total=wl.batch * wl.num_kv_heads * wl.V_cap)
    print(f"case {name}: {pattern} {extra} {wl}", flush=True)
    pr = Pair(wl, selection=DESTRUCTIVE, **extra)
    for ch in pattern:
        if ch == "r":
            pr.step_reuse()
        else:
            pr.step(fused=(ch == "s"))
            if not pr.packed:
                check_layer_properties(pr)
    assert int(pr.st.error_word[0].item()) == 0
