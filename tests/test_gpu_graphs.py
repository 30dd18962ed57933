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


@pytest.mark.parametrize("kind", ["csa", "hca", "mixed"])
def test_micro_batches_in_flight_equal_serial_steps(kind):
    """Several micro-batches in flight (one graph, a chain of steps per micro-batch and lane
    on parallel branches, as the benchmark times them): every micro-batch's outputs equal the
    eager step's bit for bit, on every replay."""
    from compressed_sparse_long_amd import lanes
    csa = W.Lane("csa", (300000, 70000, 5), (300000, 70000, 5), T=1, H=64, m=4, k=1024, HI=8)
    hca = W.Lane("hca", (131072, 9000, 100), (131072, 9000, 100), T=1, H=64, m=128)
    chosen = {"csa": (csa,), "hca": (hca,), "mixed": (csa, hca)}[kind]
    print(f"micro-batches in flight: {kind}", flush=True)
    inp = synth.generate(W.Workload("inflight", 19, chosen), parts=("kv", "z", "q", "qI", "kI", "w"))
    ls = lanes.build_lanes(inp)
    M = 3
    for cl in ls:
        cl.rotate(2 * M)
        cl.compress_all()
    names = [["out", "lse"] + (["idx", "scores"] if cl.lane.kind == "csa" else []) for cl in ls]
    for cl in ls:
        cl.step(0)
    torch.cuda.synchronize()
    refs = [[getattr(cl, n).clone() for n in nn] for cl, nn in zip(ls, names)]
    ref_cache = [cl.ckv_copies[0].clone() for cl in ls]
    mbs = [[cl] + [cl.micro_batch() for _ in range(M - 1)] for cl in ls]
    own = [[c for c in range(2 * M) if c % M == i] for i in range(M)]
    g = lanes.in_flight_graph([[lambda mb=mbs[j][i], r=r: mb.step(r) for r in own[i]]
                               for j in range(len(ls)) for i in range(M)])
    for rep in range(3):
        for row in mbs:
            for mb in row:  # eager work between the replays
                for n in ("out", "lse", "idx", "scores"):
                    t = getattr(mb, n, None)
                    if t is not None:
                        t.fill_(-7 if t.dtype == torch.int32 else -123.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j, row in enumerate(mbs):
            for i, mb in enumerate(row):
                for n, ref in zip(names[j], refs[j]):
                    t = getattr(mb, n)
                    if n == "scores":  # only the visible entries are written
                        for b, e in enumerate(mb.lane.entries):
                            assert torch.equal(t[b, 0, :e], ref[b, 0, :e]), f"replay {rep}: {n} of micro-batch {i}"
                    else:
                        assert torch.equal(t, ref), f"replay {rep}: {n} of micro-batch {i}, lane {j}"
            for c in ls[j].ckv_copies:
                assert torch.equal(c, ref_cache[j]), f"replay {rep}: a cache copy of lane {j} differs"
