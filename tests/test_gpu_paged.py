"""The paged heterogeneous cache (GPU): the same steps on the same inputs with the compressed
entries in a block pool (seeded random block order, spare blocks) and the raw rows in
per-sequence rings. Every paged output must equal the packed one bit for bit (the kernels do
the same arithmetic, only the addressing differs), and the packed outputs are checked against
the fp64 oracle here and in the stage tests."""
import numpy as np
import pytest
import torch

import synth
from synth import workloads as W
from oracle import csa, pipeline
from tests._parity import assert_attn_close, assert_rows_close, f64

pytestmark = pytest.mark.gpu


def _outputs(cl):
    return {"scores": cl.scores.clone() if getattr(cl, "scores", None) is not None else None,
            "idx": cl.idx.clone() if hasattr(cl, "idx") else None,
            "out": cl.out.clone(), "lse": cl.lse.clone()}


def _newest_entries(cl):
    """The step's newest compressed entries: packed rows, or their pool rows when paged."""
    E = cl.lane.entries
    first = cl.first_new.cpu().tolist()
    ent = cl.lane.ent_off()
    rows = []
    for b in range(cl.B):
        for e in range(first[b], E[b]):
            if cl.paged is None:
                rows.append(ent[b] + e)
            else:
                eb = cl.paged.block_entries
                rows.append(int(cl.paged.block_table[b, e // eb]) * eb + e % eb)
    return cl.ckv[torch.tensor(rows, dtype=torch.int64, device=cl.ckv.device)].clone()


def _run_both(lane, seed, fused, overlap=False, extras=False, ring_rows=256, order="random", scoreless=False):
    from compressed_sparse_long_amd import lanes
    parts = ("kv", "z", "q", "qI", "kI", "w") + (("kv_b", "z_b") if overlap else ())
    inp = synth.generate(W.Workload("paged", seed, (lane,)), parts=parts)
    res = []
    for paged in (False, True):
        (cl,) = lanes.build_lanes(inp, scoreless=scoreless)
        if extras:
            cl.sink = W.normal_f32(seed, W.S_EXTRA + 7, (lane.H,), std=2.0).cuda()
            cl.rope_dims = 64
        cl.compress_all()
        if paged:
            cl.paginate(ring_rows=ring_rows, seed=seed, order=order)
        # the step must rewrite the newest entries: poison them first
        ent_new = _newest_entries(cl)
        assert ent_new.numel() >= 0
        if lane.kind == "csa":
            cl.step(0, fused=fused)
        else:
            cl.step(0)
        torch.cuda.synchronize()
        res.append((cl, _outputs(cl), _newest_entries(cl)))
    return inp, res


def test_paged_interleaved_blocks_equal_packed():
    """Blocks handed out round-robin over the sequences, as concurrent growth allocates them."""
    lane = W.Lane("csa", (300000, 70000, 4000), (300000, 70000, 4000), T=1, H=64, m=4, k=1024, HI=8)
    _, ((pk, po, pn), (gk, go, gn)) = _run_both(lane, 35, True, order="interleaved")
    assert torch.equal(pn, gn) and torch.equal(po["idx"], go["idx"])
    assert torch.equal(po["out"], go["out"]) and torch.equal(po["lse"], go["lse"])


@pytest.mark.parametrize("lengths,m,k,H,HI,fused,overlap,fp4", [
    ((5000, 1001, 4099), 4, 64, 16, 8, False, False, False),      # the four calls one by one
    ((5000, 1001, 4099), 4, 64, 16, 8, True, False, False),       # one step call (compression in the indexer)
    ((300000, 70000), 4, 1024, 64, 8, True, False, False),        # candidate lists, 9 splits and the merge
    ((20000, 9), 4, 128, 32, 4, True, True, False),               # overlapped compression from the ring
    ((200000, 4096), 4, 512, 16, 8, True, False, True),           # MXFP4 keys and scales in the pool
    ((9000, 5000), 8, 64, 16, 8, True, False, False),             # m = 8: 16 entries per block
])
def test_paged_csa_step_equals_packed(lengths, m, k, H, HI, fused, overlap, fp4):
    print(f"paged csa lengths={lengths} m={m} k={k} H={H} fused={fused} overlap={overlap} fp4={fp4}", flush=True)
    lane = W.Lane("csa", tuple(lengths), tuple(lengths), T=1, H=H, m=m, k=k, HI=HI, kI_fp4=fp4)
    inp, ((pk, po, pn), (gk, go, gn)) = _run_both(lane, 31 + m, fused, overlap=overlap)
    assert torch.equal(pn, gn), "newest compressed entries differ"
    for b in range(lane.B):
        n = lane.entries[b]
        assert torch.equal(po["scores"][b, 0, :n], go["scores"][b, 0, :n]), f"scores differ, b={b}"
    assert torch.equal(po["idx"], go["idx"]), "selected ids differ"
    assert torch.equal(po["out"], go["out"]) and torch.equal(po["lse"], go["lse"]), "attention differs"
    # and the packed result against the oracle, for one row
    li = inp.lanes[0]
    keys = pipeline.index_keys_f64(li.kI, li.k_scale, li.scale_off, li.ent_off, 64, fp4=fp4)
    e0, E0 = 0, lane.entries[0]
    ref_s = csa.indexer(f64(li.qI[0, 0]), f64(li.w[0, 0]), keys[e0:e0 + E0])
    assert_rows_close(f64(go["scores"][0, 0, :E0]), ref_s, what="paged scores vs oracle")


@pytest.mark.parametrize("lengths,T,k,group,scoreless", [
    ((300000, 70000, 4000), 1, 1024, 64, False),   # groups of 64 over blocks of 32: one scale per block
    ((300000, 70000, 4000), 1, 1024, 16, False),   # groups of 16: two scales per block
    ((200000, 9000), 1, 512, 32, True),            # group = block; the indexer fused with top-k
    ((40000, 30000, 9000, 5000), 32, 256, 64, True),  # 32 query rows: the prefill tiling, fused
])
def test_paged_fp8_keys_equal_packed(lengths, T, k, group, scoreless):
    """fp8 e4m3 indexer keys in the block pool, their group scales kept per pool block: the
    step equals the packed one (keys, scales through scale_off) bit for bit."""
    print(f"paged fp8 keys lengths={lengths} T={T} k={k} group={group} scoreless={scoreless}", flush=True)
    qp = tuple(n - T + 1 for n in lengths)
    lane = W.Lane("csa", tuple(lengths), qp, T=T, H=64, m=4, k=k, HI=8, kI_fp8=True, scale_group=group)
    inp, ((pk, po, pn), (gk, go, gn)) = _run_both(lane, 53 + group, True, scoreless=scoreless)
    eb = gk.paged.block_entries
    assert gk.k_scale.numel() == gk.pool_rows // min(group, eb)
    assert torch.equal(pn, gn), "newest compressed entries differ"
    if not scoreless:
        for b in range(lane.B):
            n = lane.entries[b]
            assert torch.equal(po["scores"][b, :, :n], go["scores"][b, :, :n]), f"scores differ, b={b}"
    assert torch.equal(po["idx"], go["idx"]), "selected ids differ"
    assert torch.equal(po["out"], go["out"]) and torch.equal(po["lse"], go["lse"]), "attention differs"
    if not scoreless:
        # the packed scores of row 0 against the oracle's fp8 key decode
        li = inp.lanes[0]
        keys = pipeline.index_keys_f64(li.kI, li.k_scale, li.scale_off, li.ent_off, group)
        n0 = csa.n_visible(lane.q_pos[0], 4, lane.entries[0])
        ref_s = csa.indexer(f64(li.qI[0, 0]), f64(li.w[0, 0]), keys[:n0])
        assert_rows_close(f64(go["scores"][0, 0, :n0]), ref_s, what="paged fp8 scores vs oracle")


@pytest.mark.parametrize("kind", ["csa", "hca"])
def test_paged_entries_with_packed_raw_rows_equal_packed(kind):
    """ring_rows = 0: only the compressed entries (and indexer keys) move into the block pool,
    the raw rows stay packed as kv_off says; the step equals the packed one bit for bit."""
    if kind == "csa":
        lane = W.Lane("csa", (300000, 70000, 5), (300000, 70000, 5), T=1, H=64, m=4, k=1024, HI=8)
    else:
        lane = W.Lane("hca", (131072, 9000, 100), (131072, 9000, 100), T=1, H=64, m=128)
    print(f"paged entries, packed raw rows: {kind}", flush=True)
    _, ((pk, po, pn), (gk, go, gn)) = _run_both(lane, 43, True, ring_rows=0)
    assert gk.paged.ring_rows == 0
    assert torch.equal(pn, gn), "newest compressed entries differ"
    if kind == "csa":
        assert torch.equal(po["idx"], go["idx"]), "selected ids differ"
    assert torch.equal(po["out"], go["out"]) and torch.equal(po["lse"], go["lse"]), "attention differs"


def test_paged_csa_step_with_sink_and_rope_equals_packed():
    lane = W.Lane("csa", (40000, 3000), (40000, 3000), T=1, H=64, m=4, k=256, HI=8)
    _, ((pk, po, pn), (gk, go, gn)) = _run_both(lane, 77, True, extras=True)
    assert torch.equal(po["out"], go["out"]) and torch.equal(po["lse"], go["lse"])


@pytest.mark.parametrize("lengths,m,H,ring", [
    ((131072, 9000, 128), 128, 64, 256),    # one entry per block; the ring holds the window and the newest chunk
    ((20000, 700), 4, 16, 256),             # 32 entries per block
])
def test_paged_hca_step_equals_packed(lengths, m, H, ring):
    print(f"paged hca lengths={lengths} m={m} H={H} ring={ring}", flush=True)
    lane = W.Lane("hca", tuple(lengths), tuple(lengths), T=1, H=H, m=m)
    inp, ((pk, po, pn), (gk, go, gn)) = _run_both(lane, 41, True, ring_rows=ring)
    assert torch.equal(pn, gn), "newest compressed entries differ"
    assert torch.equal(po["out"], go["out"]) and torch.equal(po["lse"], go["lse"]), "attention differs"
    # the packed row 0 against the oracle
    ckv = pipeline.compress_lane(inp.kv, inp.z, lane.kv_off(), m)
    p = lane.q_pos[0]
    nv = csa.n_visible(p, m, lane.entries[0])
    X = np.concatenate([csa.to_bf16_f64(ckv[:nv]), f64(inp.kv[max(0, lengths[0] - 128):lengths[0]])])
    ro, rl = csa.attend(f64(inp.q[0, 0]), X, 128 ** -0.5)
    assert_attn_close(f64(go["out"][0, 0]), ro, "paged hca out vs oracle")
