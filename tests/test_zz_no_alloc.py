"""csl_csa_decode_step_static (GPU): the decode step with its workspaces in the library's own
scratch array equals csl_csa_decode_step with caller workspaces, bit for bit, on two calls in
a row, the second with a smaller input (the array keeps the first call's contents)."""
import math

import pytest
import torch

import synth
from synth import workloads as W

pytestmark = pytest.mark.gpu


def _one(lane, seed):
    from compressed_sparse_long_amd import csa_decode_step_static, lanes
    print(f"static-scratch step: lengths={lane.lengths} k={lane.k} H={lane.H}", flush=True)
    inp = synth.generate(W.Workload("static_scratch", seed, (lane,)))
    (cl,) = lanes.build_lanes(inp)
    cl.compress_all()
    ckv0 = cl.ckv.clone()
    cl.step()                                    # caller workspaces (csl_csa_decode_step)
    torch.cuda.synchronize()
    ref = {"ckv": cl.ckv, "scores": cl.scores, "idx": cl.idx, "out": cl.out, "lse": cl.lse}
    got = {"ckv": ckv0, "scores": torch.full_like(cl.scores, math.nan), "idx": torch.full_like(cl.idx, -7),
           "out": torch.full_like(cl.out, math.nan), "lse": torch.full_like(cl.lse, math.nan)}
    csa_decode_step_static(cl.kv, cl.z, cl.kv_off, cl.ent_off, cl.first_new, cl.n_new, got["ckv"], cl.qI, cl.w,
                           cl.kI, got["scores"], cl.k, got["idx"], cl.q, cl.W, got["out"], cl.q_pos, cl.m,
                           lse=got["lse"], scale=cl.scale, max_entries=cl.max_entries)
    torch.cuda.synchronize()
    for name in ref:
        if name == "scores":
            for b in range(lane.B):
                n = lane.entries[b]
                assert torch.equal(got[name][b, :, :n], ref[name][b, :, :n]), f"scores of row {b} differ"
        else:
            assert torch.equal(got[name], ref[name]), f"{name} differs"
    print(f"  equal: ckv, scores, idx, out, lse", flush=True)


def test_static_scratch_step_equals_step_twice():
    # first call: long rows (candidate lists in the scratch, 9 attention splits per row)
    _one(W.Lane("csa", (300000, 70000, 1001), (300000, 70000, 1001), T=1, H=64, m=4, k=1024, HI=8), 61)
    # second call, smaller: shorter rows, fewer heads, other top-k and split layout
    _one(W.Lane("csa", (150000, 4099, 9), (150000, 4099, 9), T=1, H=16, m=4, k=128, HI=8), 62)
