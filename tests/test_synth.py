"""The seeded input generator: draws reproduce, shapes and storage types follow the
workload, lengths and heavy positions stay in range, heavy keys point along their group's
mean query, and bf16 storage is round-to-nearest-even of the float32 draw."""

import numpy as np
import torch

from synth import WORKLOADS, make_inputs, tiny_workload
from synth.generate import storage_dtype


def test_draws_reproduce_and_layers_differ():
    wl = tiny_workload(steps=2, heavy=(2, 5))
    a, b = make_inputs(wl), make_inputs(wl)
    for n in ("k_ctx", "v_ctx", "q", "k_new", "v_new", "ctx_len"):
        assert torch.equal(getattr(a, n), getattr(b, n)), n
    assert all(np.array_equal(x, y) for x, y in zip(a.heavy, b.heavy))
    c = make_inputs(wl, layer=1)
    assert not torch.equal(a.k_ctx, c.k_ctx) and not torch.equal(a.q, c.q)
    d = make_inputs(wl.with_(seed=wl.seed + 1))
    assert not torch.equal(a.k_new, d.k_new)


def test_shapes_types_and_ranges():
    for kw in (dict(), dict(dtype="f32", batch=3, num_q_heads=16, num_kv_heads=4, ctx_len=300, ctx_min=100)):
        wl = tiny_workload(steps=3, **kw)
        inp = make_inputs(wl)
        B, Hq, H, D = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
        L = inp.ctx_len.numpy()
        assert inp.ctx_len.dtype == torch.int64 and L.shape == (B,)
        assert L.min() >= (wl.ctx_min if wl.ctx_min is not None else wl.ctx_len) and L.max() <= wl.ctx_len
        dt = storage_dtype(wl)
        assert inp.k_ctx.shape == (B, H, int(L.max()), D) and inp.k_ctx.dtype == dt
        assert inp.q.shape == (3, B, Hq, D) and inp.q.dtype == dt
        assert inp.k_new.shape == (3, B, H, D) and inp.v_new.dtype == dt
        for b in range(B):  # rows past a sequence's length are zero
            assert not inp.k_ctx[b, :, int(L[b]):].any()
        for b in range(B):
            for h in range(H):
                pos = inp.heavy[b * H + h]
                lo, hi = wl.heavy
                assert len(pos) <= hi and np.all(np.diff(pos) > 0)
                assert pos.size == 0 or (pos.min() >= 0 and pos.max() < int(L[b]) - wl.dense_window)


def test_heavy_keys_point_along_the_group_query():
    """A planted key's component along the unit mean query of its group is scale * |qbar|
    (up to the bf16 rounding of the key), far above an ordinary key's."""
    wl = tiny_workload(steps=1, heavy=(3, 3), dtype="f32")
    inp = make_inputs(wl)
    G = wl.group
    for b in range(wl.batch):
        for h in range(wl.num_kv_heads):
            qbar = inp.q[0, b, h * G:(h + 1) * G].double().mean(0)
            u = qbar / qbar.norm()
            pos = inp.heavy[b * wl.num_kv_heads + h]
            assert len(pos) == 3
            along = inp.k_ctx[b, h, torch.from_numpy(pos)].double() @ u
            assert torch.allclose(along, torch.full_like(along, wl.heavy_scale * float(qbar.norm())), rtol=1e-5)
            others = np.setdiff1d(np.arange(int(inp.ctx_len[b]) - wl.dense_window), pos)
            assert float((inp.k_ctx[b, h, torch.from_numpy(others)].double() @ u).abs().max()) < along.min()


def test_bf16_storage_rounds_to_nearest_even():
    """The draws are rounded from float32 to bf16 to nearest, ties to even: checked
    against an integer implementation of that rounding on the bit patterns."""
    wl = tiny_workload(steps=2)
    a = make_inputs(wl)
    f = make_inputs(wl.with_(dtype="f32"))
    x = f.k_new.contiguous().view(torch.int32).numpy().astype(np.int64) & 0xFFFFFFFF
    lsb = (x >> 16) & 1
    expect = ((x + 0x7FFF + lsb) >> 16) & 0xFFFF
    got = a.k_new.contiguous().view(torch.int16).numpy().astype(np.int64) & 0xFFFF
    assert np.array_equal(got, expect)


def test_workload_shapes_follow_the_configurations():
    """The five workloads: head geometry as configured, and every pool ring big enough for
    the first append after its longest context and for S_cap plus the block that tips it
    into condensation (condensation keeps it there over the streaming steps)."""
    for name, wl in WORKLOADS.items():
        assert wl.head_dim == 128 and wl.num_q_heads % wl.num_kv_heads == 0
        assert wl.P_blk * 64 >= wl.ctx_len - wl.dense_window + 1 - wl.sink, name
        assert wl.sparse_cap % 64 == 0 and wl.P_blk * 64 >= wl.sparse_cap + 64, name
