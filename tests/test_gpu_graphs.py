"""The decode steps captured in a HIP graph and replayed (GPU), as the benchmark times them.

Each replay must give the eager step's outputs bit for bit. Between replays the outputs are
overwritten by eager work and the device is synchronised, so a replay that skipped a write,
or a captured clear that only took effect once, would show."""
import pytest
import torch

import synth
from synth import workloads as W

pytestmark = pytest.mark.gpu


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


@pytest.mark.parametrize("kind", ["csa", "hca"])
def test_step_graph_replays_equal_eager(kind):
    from compressed_sparse_long_amd import lanes
    if kind == "csa":
        lane = W.Lane("csa", (300000, 70000, 5), (300000, 70000, 5), T=1, H=64, m=4, k=1024, HI=8)
    else:
        lane = W.Lane("hca", (131072, 9000, 100), (131072, 9000, 100), T=1, H=64, m=128)
    print(f"graph replays: {kind}", flush=True)
    inp = synth.generate(W.Workload("graph", 17, (lane,)), parts=("kv", "z", "q", "qI", "kI", "w"))
    (cl,) = lanes.build_lanes(inp)
    cl.rotate(2)
    cl.compress_all()
    outs = ["out", "lse"] + (["idx", "scores"] if kind == "csa" else [])

    def snapshot():
        return [getattr(cl, n).clone() for n in outs] + [c.clone() for c in cl.ckv_copies]

    def poison():  # a sentinel that compares equal where a step writes nothing (scores past n_vis)
        for n in outs:
            t = getattr(cl, n)
            t.fill_(-7 if t.dtype == torch.int32 else -123.0)

    refs = []
    poison()
    for r in range(2):  # eager steps on both rotated copies
        cl.step(r)
        torch.cuda.synchronize()
        refs.append(snapshot())
    g = _capture(lambda: [cl.step(r) for r in range(2)])
    for rep in range(3):
        poison()  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for a, b, name in zip(got, refs[1], outs + [f"ckv{i}" for i in range(len(cl.ckv_copies))]):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager step"
