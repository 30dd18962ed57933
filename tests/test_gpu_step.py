"""The fused decode step (csl_csa_decode_step) against the four entry points called one after
the other (GPU). Same inputs, same starting cache; the newest compressed rows are set to a
sentinel first, so both paths must write them. The indexer scores and the selected ids come
from the same kernels and must match exactly; the newest compressed rows and the attention
output may differ only by the accumulation order of the two compression layouts.
"""
import numpy as np
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
    # rows of 2^18 entries beside a row too dense for candidate lists, a row with fewer entries
    # than k and an empty row; fp8 keys; overlapped compression
    ((1 << 20, 40000, 4000, 3), 4, True, 1024, 8, False, 64, False),
    ((1 << 20, 600001), 4, True, 1024, 8, True, 64, False),
    ((1 << 20, 5), 4, True, 1024, 8, False, 64, True),
    # short rows, one attention workgroup each, which then selects the row's top-k itself: rows
    # with fewer entries than k, an empty row; 64 and 32 heads; fp8 keys
    ((16000, 3000, 100, 0, 8192), 4, True, 128, 8, False, 64, False),
    ((6000, 300, 8), 4, True, 100, 4, True, 32, False),
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


def test_csa_decode_step_finishes_crowded_rows_exactly():
    """The best keys of one row crowd into four 512-entry slices: their candidate lists cannot
    prove the selection, and the finishing step must search the whole row. The step then equals
    the separate calls and is a valid top-k of the oracle's scores."""
    from compressed_sparse_long_amd import lanes
    from oracle import csa, pipeline
    from tests._parity import f64, topk_band_check
    lane = W.Lane("csa", (1 << 20, 300000), (1 << 20, 300000), T=1, H=64, m=4, k=1024, HI=8)
    inp = synth.generate(W.Workload("crowd", 23, (lane,)))
    li = inp.lanes[0]
    lead = li.qI[0, 0].float().sum(0)
    li.kI[1000:3048] = (lead * 4 + 0.05 * li.kI[1000:3048].float()).to(torch.bfloat16)
    (cl,) = lanes.build_lanes(inp)
    cl.compress_all()
    res = []
    for fused in (False, True):
        cl.idx.fill_(-7)
        cl.step(0, fused=fused)
        torch.cuda.synchronize()
        res.append((cl.idx.clone(), cl.out.clone()))
    assert torch.equal(res[0][0], res[1][0]), "selected ids differ"
    torch.testing.assert_close(res[1][1], res[0][1], rtol=0, atol=2e-3)
    got = res[1][0].cpu().numpy()
    assert np.sum((got[0, 0] >= 1000) & (got[0, 0] < 3048)) > 512, "the crowded slices hold most winners"
    keys = pipeline.index_keys_f64(li.kI)
    for b in range(lane.B):
        e0, e1 = lane.ent_off()[b], lane.ent_off()[b + 1]
        ref_s = csa.indexer(f64(li.qI[b, 0]), f64(li.w[b, 0]), keys[e0:e1])
        topk_band_check(got[b, 0], ref_s, lane.k, what=f"b={b}")


@pytest.mark.parametrize("lengths,H,win", [
    ((4096, 2000, 300), 16, 128),   # 4 waves, 3 tiles (one wave group per tile)
    ((12000, 4000, 100), 128, 64),  # 16 waves in two groups of 8, 2 tiles, 3,000 entries
])
def test_csa_decode_step_selects_ties_by_lowest_id(lengths, H, win):
    """Short rows (one attention workgroup each, which makes the row's selection) whose indexer
    keys take three values, so their scores tie in large blocks: the step's ids equal
    topk_select's and a brute-force order of the step's own scores (score descending, lower id
    first)."""
    from compressed_sparse_long_amd import lanes
    print(f"ties lengths={lengths} H={H} W={win}", flush=True)
    lane = W.Lane("csa", lengths, lengths, T=1, H=H, m=4, W=win, k=64, HI=4)
    inp = synth.generate(W.Workload("ties", 31, (lane,)))
    li = inp.lanes[0]
    base = li.kI[:3].clone()
    li.kI[:] = base[torch.arange(li.kI.shape[0]) % 3]
    (cl,) = lanes.build_lanes(inp)
    cl.compress_all()
    res = []
    for fused in (False, True):
        cl.idx.fill_(-7)
        cl.step(0, fused=fused)
        torch.cuda.synchronize()
        res.append((cl.idx.clone(), cl.scores.clone(), cl.out.clone()))
    assert torch.equal(res[0][0], res[1][0]), "selected ids differ"
    torch.testing.assert_close(res[1][2], res[0][2], rtol=0, atol=2e-3)
    for b in range(lane.B):
        n = lane.entries[b]
        s = res[1][1][b, 0, :n].cpu().numpy()
        best = sorted(range(n), key=lambda i: (-float(s[i]), i))[:min(n, lane.k)]
        want = sorted(best) + [-1] * (lane.k - len(best))
        assert res[1][0][b, 0].tolist() == want, f"b={b}: not the k best with lower ids first"
        assert len(set(s.tolist())) <= 4, "the keys were meant to tie"


def test_csa_decode_step_repeats_on_1m_rows():
    """Calls in a row on 2^18-entry rows (the headline shape): every call selects the same
    entries as the separate calls."""
    from compressed_sparse_long_amd import lanes
    lane = W.Lane("csa", (1 << 20, 1 << 20, 70000), (1 << 20, 1 << 20, 70000), T=1, H=64, m=4, k=1024, HI=8)
    inp = synth.generate(W.Workload("fin_reset", 29, (lane,)))
    (cl,) = lanes.build_lanes(inp)
    cl.compress_all()
    cl.step(0, fused=False)
    torch.cuda.synchronize()
    ref = cl.idx.clone()
    for rep in range(4):
        cl.idx.fill_(-7)
        cl.step(0)
        torch.cuda.synchronize()
        assert torch.equal(cl.idx, ref), f"call {rep}: selected ids differ"


def test_single_split_attention_writes_no_workspace():
    """A step whose attention runs in one split per row needs no workspace: with RoPE and a
    sink it must leave the bytes around the (16-byte) buffer it was given untouched (the RoPE
    table for the merge was once written there regardless)."""
    from compressed_sparse_long_amd import attn_workspace_bytes, lanes
    inp = synth.generate("csa_decode_4k")
    (cl,) = lanes.build_lanes(inp)
    assert attn_workspace_bytes(cl.B, cl.T, cl.H, 128, cl.k + cl.W) == 0
    cl.rope_dims = 64
    cl.sink = W.normal_f32(3, W.S_EXTRA + 7, (cl.H,), std=2.0).cuda()
    guard = torch.full((1 << 16,), 0x5A, dtype=torch.uint8, device="cuda")
    cl.attn_ws = guard[4096:4096 + 16]
    cl.compress_all()
    cl.step()
    torch.cuda.synchronize()
    assert torch.all(guard == 0x5A), "bytes around the workspace were written"
    assert bool(torch.isfinite(cl.out).all())


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


# ------------------------------------------------------------------ the HCA step

def _hca_step_vs_calls(lengths, q_pos, m, H, T, first, max_new, has_z=True, extras=False):
    """csl_hca_decode_step against compress_kv then hca_attn_decode on the same inputs and the
    same starting cache, whose entries [first_b, first_b + max_new) are set to a sentinel first:
    both paths must write them, and no attention may read the sentinel (an attention workgroup
    whose keys include an entry being rewritten pools it itself)."""
    import compressed_sparse_long_amd as csl
    from oracle import csa, pipeline
    from tests._parity import assert_attn_close, assert_rows_close, f64
    print(f"hca step lengths={lengths} q_pos={q_pos} m={m} H={H} T={T} first={first} max_new={max_new} "
          f"z={has_z} extras={extras}", flush=True)
    seed = 91 + m + H + T
    B = len(lengths)
    kv_off = torch.tensor([0] + list(np.cumsum(lengths)), dtype=torch.int64)
    E = [n // m for n in lengths]
    ent_off = torch.tensor([0] + list(np.cumsum(E)), dtype=torch.int64)
    kv = W.normal_bf16(seed, W.S_EXTRA + 1, (max(int(kv_off[-1]), 1), 128))
    z = W.normal_bf16(seed, W.S_EXTRA + 2, (max(int(kv_off[-1]), 1), 128)) if has_z else None
    q = W.normal_bf16(seed, W.S_EXTRA + 3, (B, T, H, 128))
    sink = W.normal_f32(seed, W.S_EXTRA + 4, (H,), std=2.0).cuda() if extras else None
    rope = 64 if extras else 0
    d_kv, d_z, d_q = kv.cuda(), (z.cuda() if has_z else None), q.cuda()
    d_kvo, d_eo = kv_off.cuda(), ent_off.cuda()
    qp = torch.tensor(q_pos, dtype=torch.int64).cuda()
    fe = torch.tensor(first, dtype=torch.int64).cuda()
    max_e = max(E + [1])
    ckv0 = torch.empty((max(int(ent_off[-1]), 1), 128), dtype=torch.bfloat16, device="cuda")
    csl.compress_kv(d_kv, d_z, d_kvo, d_eo, m, ckv0, max_new_entries=max_e)
    newest = [(int(ent_off[b]) + first[b], int(ent_off[b]) + min(E[b], first[b] + max_new)) for b in range(B)]
    for lo, hi in newest:
        ckv0[lo:hi] = 7.0
    res = []
    for fused in (False, True):
        ckv = ckv0.clone()
        out = torch.full((B, T, H, 128), float("nan"), device="cuda")
        lse = torch.full((B, T, H), float("nan"), device="cuda")
        if fused:
            csl.hca_decode_step(d_kv, d_z, d_kvo, d_eo, fe, max_new, ckv, d_q, 128, out, qp, m, max_e, lse=lse,
                                sink=sink, rope_dims=rope)
        else:
            csl.compress_kv(d_kv, d_z, d_kvo, d_eo, m, ckv, first_entry=fe, max_new_entries=max_new)
            csl.hca_attn_decode(d_q, ckv, d_kv, d_kvo, d_eo, qp, m, 128, out, lse=lse, max_entries=max_e, sink=sink,
                                rope_dims=rope)
        torch.cuda.synchronize()
        res.append((ckv, out, lse))
    (rc, ro, rl), (gc, go, gl) = res
    for lo, hi in newest:
        assert not torch.any(gc[lo:hi] == 7.0), "the step left new entries uncompressed"
    # the two compression layouts may round the pooled sums in another order: one bf16 unit
    torch.testing.assert_close(gc.float(), rc.float(), rtol=8e-3, atol=1e-3)
    torch.testing.assert_close(go, ro, rtol=0, atol=2e-3)
    torch.testing.assert_close(gl, rl, rtol=0, atol=2e-3)
    # and the fused step against the oracle: its entries against the oracle's pooling, its
    # attention against the oracle's over those entries
    ref_c = pipeline.compress_lane(kv, z, kv_off, m)
    for b in range(B):
        lo, hi = int(ent_off[b]), int(ent_off[b + 1])
        if hi > lo:
            assert_rows_close(f64(gc[lo:hi]), ref_c[lo:hi], bf16=True, what=f"entries of seq {b}")
    oo, ol = pipeline.hca_attn_lane(q, gc.cpu(), kv, kv_off, ent_off, torch.tensor(q_pos), m, 128, 128 ** -0.5,
                                    sink=None if sink is None else sink.cpu().numpy(), rope_dims=rope)
    assert_attn_close(f64(go), oo, "out")
    assert_attn_close(f64(gl), ol, "lse")


@pytest.mark.parametrize("lengths,q_pos,m,H,T,first,max_new,has_z,extras", [
    # decode: each sequence's newest complete entry, which its query sees only where the length
    # is not a multiple of m (the 200-row and 70000-row sequences)
    ((131072, 131072, 9000, 200), (131071, 131071, 8999, 199), 128, 64, 1, (1023, 1023, 69, 0), 1, True, False),
    ((131072, 70000), (131071, 69999), 128, 16, 1, (1023, 545), 1, False, True),
    ((40000, 9000), (39999, 8999), 4, 32, 1, (9999, 2249), 1, True, False),
    # entries the queries do see: the attention workgroups pool them themselves
    ((131072, 9000), (131072, 9000), 128, 64, 1, (1021, 67), 3, True, True),
    ((20000, 3000), (20000, 3000), 4, 128, 1, (4900, 700), 60, True, False),
    ((20000,), (19000,), 4, 16, 40, (4700,), 70, True, False),      # 40 positions, the prefetching tile loop
    # splits of 3 tiles walked by the prefetching loop, the compression in the same launch, the
    # two rewritten entries seen by every row: pooled into the side rows, copied in the last round
    ((600007,), (599992,), 128, 16, 16, (4685,), 2, True, False),
    ((600007,), (599992,), 128, 64, 16, (4685,), 2, True, True),
])
def test_hca_decode_step_matches_separate_calls(lengths, q_pos, m, H, T, first, max_new, has_z, extras):
    _hca_step_vs_calls(lengths, q_pos, m, H, T, first, max_new, has_z, extras)


@pytest.mark.parametrize("fp8", [False, True])
def test_ragged_batch_indexer_matches_each_sequence_alone(fp8):
    """A ragged batch with a 2^18-entry row beside short and empty rows (one workgroup per
    sequence and slice of the longest row, most of them past their sequence's end): every
    sequence's scores equal, bit for bit, those of a call on that sequence alone, its selected
    ids equal, and the step equals the separate calls."""
    from compressed_sparse_long_amd import indexer_scores, lanes, topk_select, topk_workspace_bytes
    lengths = (1 << 20, 3001, 0, 70000, 9, 400000)
    lane = W.Lane("csa", lengths, lengths, T=1, H=64, m=4, k=1024, HI=8, kI_fp8=fp8)
    print(f"ragged batch indexer, fp8={fp8}", flush=True)
    inp = synth.generate(W.Workload("compact", 31, (lane,)))
    (cl,) = lanes.build_lanes(inp)
    cl.compress_all()
    cl.scores.fill_(-5.0)
    cl.step(0, fused=False)
    torch.cuda.synchronize()
    ref_idx, ref_out, scores = cl.idx.clone(), cl.out.clone(), cl.scores.clone()
    cl.idx.fill_(-7)
    cl.step(0)
    torch.cuda.synchronize()
    assert torch.equal(cl.idx, ref_idx), "the step's ids differ from the separate calls"
    torch.testing.assert_close(cl.out, ref_out, rtol=0, atol=2e-3)
    E = lane.entries
    for b in range(lane.B):
        eo = cl.ent_off[b:b + 2]
        s1 = torch.full((1, 1, max(E[b], 1)), -5.0, dtype=torch.float32, device="cuda")
        ws = torch.zeros(max(topk_workspace_bytes(1, 1, max(E[b], 1), lane.k), 16), dtype=torch.uint8, device="cuda")
        indexer_scores(cl.qI[b:b + 1], cl.w[b:b + 1], cl.kI, eo, cl.q_pos[b:b + 1], lane.m, s1,
                       max_entries=max(E[b], 1), k_scale=cl.k_scale, scale_off=None if cl.scale_off is None
                       else cl.scale_off[b:b + 2], scale_group=cl.scale_group, topk_ws=ws, topk_k=lane.k)
        i1 = torch.full((1, 1, lane.k), -7, dtype=torch.int32, device="cuda")
        topk_select(s1, eo, cl.q_pos[b:b + 1], lane.m, lane.k, i1, ws=ws, max_entries=max(E[b], 1), prepared=True)
        torch.cuda.synchronize()
        assert torch.equal(scores[b, 0, :E[b]], s1[0, 0, :E[b]]), f"scores of sequence {b} differ"
        assert torch.equal(ref_idx[b], i1[0]), f"ids of sequence {b} differ"


@pytest.mark.parametrize("lengths,k,HI,fp8,H,crowd", [
    ((1 << 20, 40000, 4000, 3), 1024, 8, False, 64, False),  # list rows, a row too dense for lists, short rows
    ((1 << 20, 300001), 1024, 8, True, 64, False),           # fp8 keys
    ((600000, 300000), 512, 16, False, 32, False),           # 16 indexer heads
    ((400000, 200000), 256, 4, False, 16, False),            # 4 indexer heads
    ((1 << 20, 300000), 1024, 8, False, 64, True),           # row 0's winners crowd into 4 slices
    ((1 << 20, 300000), 1024, 8, True, 64, True),            # the same with fp8 keys
])
def test_scores_on_demand_matches_step_with_scores(lengths, k, HI, fp8, H, crowd):
    """Scores on demand: the step keeps no scores for rows selected from candidate lists, and
    selects the same ids with the same outputs, bit for bit. Rows too dense for lists keep
    their scores; a row whose winners crowd into a few slices (its lists cannot prove the
    selection) has its crowded slices' scores recomputed, equal bit for bit to the indexer's."""
    from compressed_sparse_long_amd import lanes
    lane = W.Lane("csa", lengths, lengths, T=1, H=H, m=4, k=k, HI=HI, kI_fp8=fp8)
    print(f"scores on demand: {lengths} k={k} HI={HI} fp8={fp8} crowd={crowd}", flush=True)
    inp = synth.generate(W.Workload("on_demand", 37, (lane,)))
    li = inp.lanes[0]
    if crowd:  # the best keys of row 0 in entries 1024 .. 3071 (four slices)
        if fp8:
            li.k_scale[16:48] *= 100.0
        else:
            lead = li.qI[0, 0].float().sum(0)
            li.kI[1024:3072] = (lead * 4 + 0.05 * li.kI[1024:3072].float()).to(torch.bfloat16)
    (cl,) = lanes.build_lanes(inp)
    cl.compress_all()
    cl.step(0)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (cl.idx, cl.out, cl.lse, cl.scores, cl.ckv)]
    if crowd:
        got0 = ref[0][0, 0].cpu().numpy()
        assert np.sum((got0 >= 1024) & (got0 < 3072)) > k // 2, "the crowded slices hold most winners"
    cl.scores_on_demand = True
    cl.scores.fill_(-5.0)
    cl.idx.fill_(-7)
    cl.step(0)
    torch.cuda.synchronize()
    assert torch.equal(cl.idx, ref[0]), "selected ids differ"
    assert torch.equal(cl.out, ref[1]), "out differs"
    assert torch.equal(cl.lse, ref[2]), "lse differs"
    assert torch.equal(cl.ckv, ref[4]), "compressed cache differs"
    E = lane.entries
    for b in range(lane.B):
        n = min(E[b], lane.q_pos[b] // lane.m)
        row = cl.scores[b, 0, :n]
        dense = 64 * k > 5 * n
        if dense:
            assert torch.equal(row, ref[3][b, 0, :n]), f"scores of row {b} differ"
        elif crowd and b == 0:
            # rebuilt for the exact pass: the indexer's scores wherever a winner could be (the
            # crowded slices recomputed whole, the listed entries of the others), elsewhere a NaN
            # with every bit set, which the pass skips
            have = ~torch.isnan(row)
            assert bool((row[~have].view(torch.int32) == -1).all()), "placeholders are not the all-ones NaN"
            assert torch.equal(row[have], ref[3][b, 0, :n][have]), "recomputed scores differ"
            assert bool(have[1024:3072].all()), "the crowded slices were not recomputed"
        else:
            assert bool((row == -5.0).all()), f"row {b} selected from lists kept scores"


def test_scores_on_demand_is_ignored_for_a_paged_cache():
    """With the cache paged the step writes every score whatever scores_on_demand says (the
    finishing step recomputes rows from the packed layout only): the same ids, outputs and
    scores as the paged step with scores."""
    from compressed_sparse_long_amd import lanes
    lane = W.Lane("csa", (1 << 20, 300001), (1 << 20, 300001), T=1, H=64, m=4, k=1024, HI=8)
    print("scores on demand, paged", flush=True)
    inp = synth.generate(W.Workload("on_demand_paged", 43, (lane,)))
    (cl,) = lanes.build_lanes(inp)
    cl.compress_all()
    cl.paginate(ring_rows=256)
    cl.step(0)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (cl.idx, cl.out, cl.lse, cl.scores)]
    cl.scores_on_demand = True
    cl.scores.fill_(-5.0)
    cl.idx.fill_(-7)
    cl.step(0)
    torch.cuda.synchronize()
    assert torch.equal(cl.idx, ref[0]) and torch.equal(cl.out, ref[1]) and torch.equal(cl.lse, ref[2])
    for b, e in enumerate(lane.entries):
        assert torch.equal(cl.scores[b, 0, :e], ref[3][b, 0, :e]), f"scores of row {b} not written"
