"""No kernel writes outside the buffers it is given: every state buffer (and the
workspace) sits between guard zones filled with a byte pattern, and after prefills, steps
with and without selection and the separate calls, the guards are unchanged, for layouts
that fill each capacity (pool ring wrap, condensed ring wrap, packed views that overflow
their rows, sinks, split select, split entropy fit, the shared pool, destructive selection)."""

import pytest
import torch

from decode_kv_cache_02_amd import hardkv as hk
from synth import make_inputs, tiny_workload
from synth.configs import COND_EVICT, COND_MERGE

pytestmark = pytest.mark.gpu

GUARD = 4096  # bytes on each side (keeps every buffer 16-byte aligned)
PATTERN = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    hk.require_gpu()


class GuardedState(hk.State):
    """hk.State whose buffers are views into larger allocations with guard zones."""

    def __init__(self, cfg, device="cuda"):
        super().__init__(cfg, device=device)
        self.guarded = {}
        for n in hk._STATE_PTRS:
            t = getattr(self, n)
            if t is None:
                continue
            nb = t.numel() * t.element_size()
            big = torch.full((GUARD + nb + GUARD,), PATTERN, dtype=torch.uint8, device=t.device)
            big[GUARD:GUARD + nb].copy_(t.contiguous().view(-1).view(torch.uint8))
            setattr(self, n, big[GUARD:GUARD + nb].view(t.dtype).view(t.shape))
            self.guarded[n] = (big, nb)
        self._bind()

    def check(self, tag):
        torch.cuda.synchronize()
        for n, (big, nb) in self.guarded.items():
            for part, zone in (("before", big[:GUARD]), ("after", big[GUARD + nb:])):
                bad = (zone != PATTERN).nonzero()
                assert bad.numel() == 0, f"{tag}: {n} written {part} its buffer at byte {int(bad[0])}"


CASES = {
    "merge_wrap_g8": dict(num_q_heads=16, num_kv_heads=2, cond_mode=COND_MERGE, sparse_cap=128, condensed_slots=3,
                          ctx_len=700, ctx_min=500, steps=4),
    "evict_f32_batch3": dict(dtype="f32", batch=3, steps=4),
    "sink": dict(sink=128, cond_mode=COND_MERGE, ctx_len=500, ctx_min=60, steps=4),
    "split_select": dict(pool_blocks=1100, sparse_cap=4096, ctx_len=3000, ctx_min=2000, cond_mode=COND_MERGE, steps=3),
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("layout", ["maxlen", "packed_short", "shared", "shared_short", "destructive"])
def test_guards_untouched(name, layout):
    kw = dict(CASES[name])
    steps = kw.pop("steps")
    wl = tiny_workload(steps=steps + 2, **kw)
    inp = make_inputs(wl, device="cuda")
    extra = {}
    if layout == "packed_short":  # fewer packed rows than the budgets need: overflow bit, no write past
        extra = dict(view_layout=hk.HARDKV_VIEW_SUM, view_total=wl.batch * wl.num_kv_heads * 40)
    elif layout.startswith("shared"):  # the shared block pool, sized for the steps or a block short of the prefill
        ring = hk.Config.from_workload(wl)
        need = (hk.hardkv_shared_pool_blocks(ring, inp.ctx_len.cpu(), steps + 2) if layout == "shared"
                else hk.hardkv_shared_pool_blocks(ring, inp.ctx_len.cpu(), 0) - 1)
        extra = dict(pool_layout=hk.HARDKV_POOL_SHARED, pool_total_blocks=need)
    elif layout == "destructive":  # (with the fixed temperature only)
        extra = dict(selection=hk.HARDKV_SEL_DESTRUCTIVE)
    cals = (hk.HARDKV_CAL_FIXED,) if layout == "destructive" else (hk.HARDKV_CAL_FIXED, hk.HARDKV_CAL_ENTROPY)
    for cal in cals:
        cfg = hk.Config.from_workload(wl, calibration=cal, **extra)
        st = GuardedState(cfg)
        out = torch.zeros((wl.batch, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
        hk.hardkv_prefill(cfg, st, inp.k_ctx, inp.v_ctx, inp.ctx_len)
        st.check(f"{name} {layout} cal {cal} prefill")
        for s in range(steps):
            hk.hardkv_step(cfg, st, inp.q[s], inp.k_new[s], inp.v_new[s], out)
        hk.hardkv_step_reuse(cfg, st, inp.q[steps], inp.k_new[steps], inp.v_new[steps], out)
        s = steps + 1
        hk.hardkv_append(cfg, st, inp.k_new[s], inp.v_new[s])
        hk.hardkv_select(cfg, st, inp.q[s])
        hk.hardkv_regularize(cfg, st)
        hk.hardkv_condense(cfg, st)
        hk.hardkv_attend(cfg, st, inp.q[s], out)
        hk.hardkv_attend_sparse(cfg, st, inp.q[s], out)
        for k in range(hk.hardkv_step_num_stages()):
            if k not in (0, 3):  # the repeatable stages once more
                hk.hardkv_step_stage(cfg, st, inp.q[s], inp.k_new[s], inp.v_new[s], out, k)
        st.check(f"{name} {layout} cal {cal} steps")
        if layout == "packed_short":
            assert int(st.error_word[0].item()) & hk.HARDKV_ERR_VIEW_OVERFLOW
        if layout == "shared_short":
            assert int(st.error_word[0].item()) & hk.HARDKV_ERR_POOL_OVERFLOW
