"""The fused decode step (csl_csa_decode_step) against the four entry points called one after
the other (GPU). Same inputs, same starting cache; the newest compressed rows are set to a
sentinel first, so both paths must write them. The indexer scores and the selected ids come
from the same kernels and must match exactly; the newest compressed rows and the attention
output may differ only by the accumulation order of the two compression layouts.
"""
import pytest
import torch

import synth
from synth import workloads as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("lengths,m,has_z,k,HI,fp8,H,overlap", [
    ((600000, 300000, 4000), 4, True, 1024, 8, False, 64, False),  # long rows: candidate lists, compression in the indexer launch
    ((4096,), 4, False, 64, 4, False, 16, False),                  # short row: one-workgroup selection, uniform weights
    ((200000, 70000, 0), 8, True, 512, 8, True, 32, False),        # m = 8, fp8 keys, an empty sequence
    ((100000, 50001), 2, True, 256, 16, False, 64, False),         # m = 2, 16 indexer heads
    ((65536,), 16, True, 128, 8, False, 16, False),                # m = 16: compression in its own launch
    # overlapped compression (series a and b)
    ((600000, 300000, 4000), 4, True, 1024, 8, False, 64, True),   # carried by the indexer launch
    ((4, 9000, 7), 4, True, 64, 8, False, 16, True),               # a one-entry sequence: series a only
    ((4096,), 8, False, 64, 4, False, 16, True),                   # uniform weights over 2m = 16 rows
    ((65536,), 16, True, 128, 8, False, 16, True),                 # m = 16: its own launch
])
def test_csa_decode_step_matches_separate_calls(lengths, m, has_z, k, HI, fp8, H, overlap):
    _step_vs_calls(lengths, m, has_z, k, HI, fp8, H, overlap, extras=False)


@pytest.mark.parametrize("lengths,m,k,H,overlap", [
    ((600000, 300000, 4000), 4, 1024, 64, False),
    ((600000, 4), 4, 1024, 64, True),
    ((4096,), 4, 64, 16, False),
])
def test_csa_decode_step_with_sink_and_rope_matches_separate_calls(lengths, m, k, H, overlap):
    """The step forwards the attention extras (per-head sink, partial RoPE) unchanged."""
    _step_vs_calls(lengths, m, True, k, 8, False, H, overlap, extras=True)


def _step_vs_calls(lengths, m, has_z, k, HI, fp8, H, overlap, extras):
    from compressed_sparse_long_amd import lanes
    print(f"step lengths={lengths} m={m} z={has_z} k={k} HI={HI} fp8={fp8} H={H} overlap={overlap} "
          f"extras={extras}", flush=True)
    lane = W.Lane("csa", tuple(lengths), tuple(lengths), T=1, H=H, m=m, k=k, HI=HI, kI_fp8=fp8)
    parts = ("kv", "z", "q", "qI", "kI", "w") + (("kv_b", "z_b") if overlap else ())
    inp = synth.generate(W.Workload("step", 11 + m, (lane,), z_present=has_z), parts=parts)
    (cl,) = lanes.build_lanes(inp)
    if extras:
        cl.sink = W.normal_f32(11 + m, W.S_EXTRA + 7, (H,), std=2.0).cuda()
        cl.rope_dims, cl.rope_base = 64, 10000.0
    cl.compress_all()
    E = lane.entries
    newest = [(int(cl.ent_off[b]) + int(cl.first_new[b]), int(cl.ent_off[b]) + E[b]) for b in range(lane.B)]
    for lo, hi in newest:
        cl.ckv[lo:hi] = 7.0
    start = cl.ckv.clone()

    def run(fused):
        cl.ckv.copy_(start)
        cl.scores.fill_(float("nan"))
        cl.idx.fill_(-7)
        cl.out.fill_(float("nan"))
        cl.step(0, fused=fused)
        torch.cuda.synchronize()
        return cl.ckv.clone(), cl.scores.clone(), cl.idx.clone(), cl.out.clone(), cl.lse.clone()

    ref = run(False)
    got = run(True)
    for lo, hi in newest:
        if hi > lo:
            assert not torch.any(got[0][lo:hi] == 7.0), "the step left newest entries uncompressed"
    torch.testing.assert_close(got[0].float(), ref[0].float(), rtol=8e-3, atol=1e-3)
    for b in range(lane.B):
        n = E[b]
        assert torch.equal(got[1][b, 0, :n], ref[1][b, 0, :n]), f"scores differ, b={b}"
    assert torch.equal(got[2], ref[2]), "selected ids differ"
    torch.testing.assert_close(got[3], ref[3], rtol=0, atol=2e-3)
    torch.testing.assert_close(got[4], ref[4], rtol=0, atol=2e-3)


def test_csa_decode_step_repeats_identically():
    """Two calls in a row on the same inputs give bit-identical results."""
    from compressed_sparse_long_amd import lanes
    lane = W.Lane("csa", (300000, 120000), (300000, 120000), T=1, H=64, m=4, k=1024, HI=8)
    inp = synth.generate(W.Workload("step2", 5, (lane,)))
    (cl,) = lanes.build_lanes(inp)
    cl.compress_all()
    outs = []
    for _ in range(2):
        cl.step(0)
        torch.cuda.synchronize()
        outs.append((cl.idx.clone(), cl.out.clone(), cl.ckv.clone()))
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(outs[0][2], outs[1][2])


@pytest.mark.parametrize("lengths,q_pos,T,k,HI,overlap,fmt", [
    ((40000, 9000, 3001), (39000, 8000, 2001), 24, 512, 8, False, None),  # prefill rows: equal bit for bit
    ((20000, 7000), (19500, 6900), 40, 256, 16, True, None),
    ((30000, 5000, 800), (29000, 4000, 700), 24, 300, 8, False, "mxfp4"),
])
def test_csa_step_without_scores_matches_step_with_scores(lengths, q_pos, T, k, HI, overlap, fmt):
    """With no score buffer the step selects with the indexer fused with top-k: for query
    batches where indexer_scores takes its prefill tiling (B*T >= 64, T >= 16) the compressed
    rows, the ids and the attention equal the scored step's exactly."""
    from compressed_sparse_long_amd import lanes
    print(f"scoreless step lengths={lengths} T={T} k={k} HI={HI} overlap={overlap} fmt={fmt}", flush=True)
    lane = W.Lane("csa", tuple(lengths), tuple(q_pos), T=T, H=16, m=4, k=k, HI=HI, kI_fp4=fmt == "mxfp4")
    parts = ("kv", "z", "q", "qI", "kI", "w") + (("kv_b", "z_b") if overlap else ())
    inp = synth.generate(W.Workload("step_nos", 17 + T, (lane,)), parts=parts)
    res = []
    for scoreless in (False, True):
        (cl,) = lanes.build_lanes(inp, scoreless=scoreless)
        cl.compress_all()
        assert (cl.scores is None) == scoreless
        cl.idx.fill_(-7)
        cl.step(0)
        torch.cuda.synchronize()
        res.append((cl.ckv.clone(), cl.idx.clone(), cl.out.clone(), cl.lse.clone()))
    for a, b, what in zip(res[0], res[1], ("ckv", "idx", "out", "lse")):
        assert torch.equal(a, b), f"{what} differs without scores"
