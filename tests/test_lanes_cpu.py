"""Host logic of the lane helpers (CPU): a micro-batch shares its lane's inputs and cache
copies and owns every buffer a step writes, so several micro-batches' steps can run at once."""
import torch

import synth
from synth import workloads as W


def _ptrs(t):
    return t.data_ptr() if t is not None else None


def test_micro_batch_shares_inputs_and_owns_step_buffers():
    from compressed_sparse_long_amd import lanes
    csa = W.Lane("csa", (9000, 4001, 0), (9000, 4001, 0), T=1, H=16, m=4, k=64, HI=4)
    hca = W.Lane("hca", (5000, 300), (5000, 300), T=1, H=16, m=128)
    inp = synth.generate(W.Workload("mb_cpu", 3, (csa, hca)))
    for ln in lanes.build_lanes(inp, device="cpu"):
        ln.rotate(3)
        mb = ln.micro_batch()
        # inputs, caches and offsets: the very same tensors
        for name in ("kv", "z", "q", "kv_off", "ent_off", "q_pos", "first_new", "qI", "w", "kI"):
            if getattr(ln, name, None) is not None:
                assert getattr(mb, name) is getattr(ln, name), name
        assert [_ptrs(c) for c in mb.ckv_copies] == [_ptrs(c) for c in ln.ckv_copies]
        # every buffer a step writes (other than the cache's newest entries): new memory, same shape
        owned = [n for n in ("scores", "idx", "out", "lse", "topk_ws", "attn_ws") if getattr(ln, n, None) is not None]
        assert {"out", "lse", "attn_ws"} <= set(owned)
        if ln.lane.kind == "csa":
            assert {"scores", "idx", "topk_ws"} <= set(owned)
        for n in owned:
            a, b = getattr(ln, n), getattr(mb, n)
            assert a.shape == b.shape and a.dtype == b.dtype, n
            assert _ptrs(a) != _ptrs(b), f"{n} is shared"
        # a second micro-batch owns its buffers too
        mb2 = ln.micro_batch()
        for n in owned:
            assert _ptrs(getattr(mb2, n)) not in (_ptrs(getattr(ln, n)), _ptrs(getattr(mb, n))), n
