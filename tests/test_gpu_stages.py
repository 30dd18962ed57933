"""Stage-isolated parity of every HIP entry point against the fp64 oracle (GPU).

Inputs come from the seeded generators in ``synth``; both sides consume the same values.
Shapes span several kernel tiles plus ragged tails, empty sequences and the degenerate
cases of each stage. Tolerances are the ones written in tests/_parity.py.
"""
import math

import numpy as np
import pytest
import torch

import synth
from synth import workloads as W
from oracle import csa, pipeline
from tests._parity import (assert_attn_close, assert_rows_close, dev, f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csl():
    import compressed_sparse_long_amd as lib
    return lib


def _offsets(lengths, m):
    kv_off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    ent_off = np.concatenate([[0], np.cumsum([n // m for n in lengths])]).astype(np.int64)
    return torch.from_numpy(kv_off), torch.from_numpy(ent_off)


# ------------------------------------------------------------------------------- compress

@pytest.mark.parametrize("m,D,lengths,has_z", [
    (4, 128, [4096, 0, 3, 37, 1001], True),
    (128, 128, [131072 // 8, 127, 300], True),
    (1, 64, [77, 5], True),
    (3, 64, [1000, 2], True),
    (16, 256, [999], True),
    (4, 128, [513, 64], False),
    (128, 512, [1024], True),
    (128, 64, [20000, 300], True),    # D = 64, m = 128: rows split over 2 waves (few entries)
    (256, 128, [10000], True),        # m = 256: rows split over 4 waves, two loads rounds
])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_compress_matches_oracle(csl, m, D, lengths, has_z, out_dtype):
    print(f"compress m={m} D={D} lengths={lengths} z={has_z} out={out_dtype}", flush=True)
    rows = sum(lengths)
    kv = W.normal_bf16(11, W.S_EXTRA + 2, (rows, D))
    z = W.normal_bf16(11, W.S_EXTRA + 3, (rows, D), std=2.0) if has_z else None
    kv_off, ent_off = _offsets(lengths, m)
    E = int(ent_off[-1])
    out = torch.full((E + 1, D), float("nan"), dtype=out_dtype, device="cuda")
    csl.compress_kv(dev(kv), dev(z), dev(kv_off), dev(ent_off), m, out, max_new_entries=max(1, E))
    torch.cuda.synchronize()
    ref = pipeline.compress_lane(kv, z, kv_off.tolist(), m)
    got = f64(out)
    if E:
        assert_rows_close(got[:E], ref, bf16=(out_dtype == torch.bfloat16), what="compress")
    assert np.isnan(got[E]).all(), "wrote past the last entry"


def test_compress_newest_chunk_only(csl):
    """first_entry = E_b - 1 recompresses just the last complete chunk of each sequence."""
    m, D = 4, 128
    lengths = [4096, 1023, 8]
    kv = W.normal_bf16(12, W.S_EXTRA + 2, (sum(lengths), D))
    z = W.normal_bf16(12, W.S_EXTRA + 3, (sum(lengths), D))
    kv_off, ent_off = _offsets(lengths, m)
    E = [n // m for n in lengths]
    first = torch.tensor([e - 1 for e in E], dtype=torch.int64)
    out = torch.full((int(ent_off[-1]), D), float("nan"), dtype=torch.float32, device="cuda")
    csl.compress_kv(dev(kv), dev(z), dev(kv_off), dev(ent_off), m, out, first_entry=dev(first), max_new_entries=1)
    torch.cuda.synchronize()
    got = f64(out)
    ref = pipeline.compress_lane(kv, z, kv_off.tolist(), m)
    for b in range(3):
        last = int(ent_off[b + 1]) - 1
        assert_rows_close(got[last], ref[last], what=f"newest entry of seq {b}")
        assert np.isnan(got[int(ent_off[b]):last]).all()


# ------------------------------------------------------------------ overlapped compression

def _two_series(seed, rows, D, has_z):
    kv_a = W.normal_bf16(seed, W.S_EXTRA + 2, (rows, D))
    kv_b = W.normal_bf16(seed, W.S_EXTRA + 4, (rows, D))
    if not has_z:
        return kv_a, None, kv_b, None
    z_a = W.normal_bf16(seed, W.S_EXTRA + 3, (rows, D), std=2.0)
    z_b = W.normal_bf16(seed, W.S_EXTRA + 5, (rows, D), std=2.0)
    return kv_a, z_a, kv_b, z_b


@pytest.mark.parametrize("m,D,lengths,has_z", [
    (4, 128, [4096, 0, 3, 4, 7, 37, 1001], True),   # N < m, N = m (entry 0 only), ragged tails
    (4, 128, [513, 64], False),
    (1, 64, [77, 5], True),
    (3, 64, [1000, 2], True),
    (16, 256, [999], True),
    (64, 512, [4096, 100], True),
    (128, 128, [16384, 127, 300], True),            # few entries: 256 rows over 4 waves
    (128, 64, [20000, 300], True),
    (4, 128, [50000, 4099], True),                  # many entries: one wave walks each entry
])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_compress_overlap_matches_oracle(csl, m, D, lengths, has_z, out_dtype):
    print(f"compress_overlap m={m} D={D} lengths={lengths} z={has_z} out={out_dtype}", flush=True)
    kv_a, z_a, kv_b, z_b = _two_series(14, sum(lengths), D, has_z)
    kv_off, ent_off = _offsets(lengths, m)
    E = int(ent_off[-1])
    out = torch.full((E + 1, D), float("nan"), dtype=out_dtype, device="cuda")
    csl.compress_kv_overlap(dev(kv_a), dev(z_a), dev(kv_b), dev(z_b), dev(kv_off), dev(ent_off), m, out,
                            max_new_entries=max(1, E))
    torch.cuda.synchronize()
    ref = pipeline.compress_overlap_lane(kv_a, z_a, kv_b, z_b, kv_off.tolist(), m)
    got = f64(out)
    if E:
        assert_rows_close(got[:E], ref, bf16=(out_dtype == torch.bfloat16), what="compress_overlap")
    assert np.isnan(got[E]).all(), "wrote past the last entry"


def test_compress_overlap_newest_chunk_only(csl):
    """first_entry = E_b - 1 recompresses the newest entry of each sequence, pooling its own
    series-a block with the series-b block before it (a one-entry sequence: series a only)."""
    m, D = 4, 128
    lengths = [4096, 1023, 8, 5]
    kv_a, z_a, kv_b, z_b = _two_series(15, sum(lengths), D, True)
    kv_off, ent_off = _offsets(lengths, m)
    E = [n // m for n in lengths]
    first = torch.tensor([e - 1 for e in E], dtype=torch.int64)
    out = torch.full((int(ent_off[-1]), D), float("nan"), dtype=torch.bfloat16, device="cuda")
    csl.compress_kv_overlap(dev(kv_a), dev(z_a), dev(kv_b), dev(z_b), dev(kv_off), dev(ent_off), m, out,
                            first_entry=dev(first), max_new_entries=1)
    torch.cuda.synchronize()
    got = f64(out)
    ref = pipeline.compress_overlap_lane(kv_a, z_a, kv_b, z_b, kv_off.tolist(), m)
    for b in range(len(lengths)):
        last = int(ent_off[b + 1]) - 1
        assert_rows_close(got[last], ref[last], bf16=True, what=f"newest overlapped entry of seq {b}")
        assert np.isnan(got[int(ent_off[b]):last]).all(), "wrote an older entry"


def test_compress_overlap_argument_errors(csl):
    """z_a and z_b must come together; kv_b is required; a bad call enqueues nothing."""
    kv_off, ent_off = _offsets([16], 4)
    kv = torch.zeros(16, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.full((4, 128), float("nan"), dtype=torch.float32, device="cuda")
    with pytest.raises(csl.CslError) as e:
        csl.compress_kv_overlap(kv, kv, kv, None, dev(kv_off), dev(ent_off), 4, out)
    assert e.value.status == 1
    torch.cuda.synchronize()
    assert torch.isnan(out).all()


# ------------------------------------------------------------------------------- indexer

def _index_lane(HI, T, lengths, q_pos, fp8=False, seed=21, fp4=False):
    lane = W.Lane("csa", tuple(lengths), tuple(q_pos), T=T, H=16, m=4, k=8, HI=HI, kI_fp8=fp8, kI_fp4=fp4)
    return synth.generate(W.Workload("idx", seed, (lane,)), parts=("qI", "kI", "w")).lanes[0]


@pytest.mark.parametrize("HI", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("T,lengths,q_pos", [
    (1, [4096, 0, 50, 9000], [4096, 0, 50, 9000]),
    (3, [2000, 333], [1500, 100]),
    (24, [4000, 1200, 64, 3000], [3900, 1000, 0, 2000]),
])
def test_indexer_matches_oracle(csl, HI, T, lengths, q_pos):
    _run_indexer(csl, HI, T, lengths, q_pos, fp8=False)


@pytest.mark.parametrize("HI,T", [(8, 1), (4, 20)])
def test_indexer_fp8_keys_match_oracle(csl, HI, T):
    _run_indexer(csl, HI, T, [70000, 1000, 130], [70000, 900, 130], fp8=True)


@pytest.mark.parametrize("HI,T,lengths,q_pos", [
    (8, 1, [300000, 1000, 130, 0], [300000, 900, 130, 0]),      # decode tiling with top-k candidate lists
    (4, 20, [70000, 1000, 130], [69000, 900, 60]),              # prefill tiling
    (16, 3, [2000, 333], [1500, 100]),
    (1, 1, [4096], [4096]),
])
def test_indexer_mxfp4_keys_match_oracle(csl, HI, T, lengths, q_pos):
    _run_indexer(csl, HI, T, lengths, q_pos, fp8=False, fp4=True)


def _run_indexer(csl, HI, T, lengths, q_pos, fp8, fp4=False):
    print(f"indexer HI={HI} T={T} lengths={lengths} fp8={fp8} fp4={fp4}", flush=True)
    li = _index_lane(HI, T, lengths, q_pos, fp8, fp4=fp4)
    B = len(lengths)
    E = li.lane.entries
    ld = max(max(E), 1) + 5
    scores = torch.full((B, T, ld), float("nan"), dtype=torch.float32, device="cuda")
    topk = {}
    if fp4 and T == 1 and max(E) > 34816:  # the candidate-list path of the decode kernel too
        topk = dict(topk_ws=torch.zeros(csl.topk_workspace_bytes(B, T, max(E), 64), dtype=torch.uint8,
                                        device="cuda"), topk_k=64)
    csl.indexer_scores(dev(li.qI), dev(li.w), dev(li.kI), dev(li.ent_off), dev(li.q_pos), 4, scores,
                       max_entries=max(E), k_scale=dev(li.k_scale), scale_off=dev(li.scale_off), scale_group=64,
                       k_format="mxfp4" if fp4 else None, **topk)
    torch.cuda.synchronize()
    keys = pipeline.index_keys_f64(li.kI, li.k_scale, li.scale_off, li.ent_off, 64, fp4=fp4)
    ref = pipeline.indexer_lane(li.qI, li.w, keys, li.ent_off, li.q_pos, 4)
    got = f64(scores)
    for b in range(B):
        for t in range(T):
            n = len(ref[b][t])
            assert_rows_close(got[b, t, :n], ref[b][t], what=f"scores b={b} t={t}")
            assert np.isnan(got[b, t, n:]).all(), f"wrote beyond n_visible at b={b} t={t}"
            assert np.all(got[b, t, :n] >= 0)


# ------------------------------------------------------------------------------- top-k

@pytest.mark.parametrize("case", [
    dict(E=[1000, 70, 5, 0], q_pos=[4000, 280, 20, 0], T=2, k=64, levels=0),
    dict(E=[1024], q_pos=[4096], T=1, k=64, levels=7),
    dict(E=[5000, 3000], q_pos=[20000, 12000], T=1, k=512, levels=0, neg=True),
    dict(E=[34816], q_pos=[131072], T=6, k=512, levels=0),
    dict(E=[34816], q_pos=[131072], T=3, k=512, levels=3),
    dict(E=[262144, 100000], q_pos=[1 << 20, 400000], T=1, k=1024, levels=0),
    dict(E=[262144], q_pos=[1 << 20], T=2, k=1024, levels=200),
    dict(E=[60000, 50000], q_pos=[240000, 200000], T=1, k=1000, levels=1),
    dict(E=[70000, 500], q_pos=[280000, 2000], T=1, k=4096, levels=0, neg=True),
    # rows up to 2^20 (four 8-slot chunks per finishing thread)
    dict(E=[1 << 20, 300000], q_pos=[1 << 22, 1200000], T=1, k=1024, levels=0),
    # ties at the k-th key that the candidate lists still prove: the lower ids must win
    dict(E=[262144], q_pos=[1 << 20], T=1, k=1024, levels=100000),
    dict(E=[262144, 90000], q_pos=[1 << 20, 360000], T=1, k=2048, levels=20000, neg=True),
])
def test_topk_bit_exact(csl, case):
    print(f"topk {case}", flush=True)
    E, T, k = case["E"], case["T"], case["k"]
    B = len(E)
    ld = max(E) + 3
    s = synth.random_scores(31 + len(E) + k, B * T, ld, levels=case["levels"], neg=case.get("neg", False))
    scores = s.view(B, T, ld)
    ent_off = torch.tensor(np.concatenate([[0], np.cumsum(E)]), dtype=torch.int64)
    q_pos = torch.tensor(case["q_pos"], dtype=torch.int64)
    idx = torch.full((B, T, k), -7, dtype=torch.int32, device="cuda")
    need = csl.topk_workspace_bytes(B, T, max(E), k)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda")
    for rep in range(3):  # each call must leave the workspace ready for the next one
        idx.fill_(-7)
        csl.topk_select(dev(scores), dev(ent_off), dev(q_pos), 4, k, idx, ws=ws, max_entries=max(E))
        torch.cuda.synchronize()
        got = idx.cpu().numpy()
        for b in range(B):
            for t in range(T):
                n = csa.n_visible(int(q_pos[b]) + t, 4, E[b])
                ref = csa.topk(scores[b, t, :n].numpy(), k)
                assert np.array_equal(got[b, t], ref), f"rep={rep} b={b} t={t}"


@pytest.mark.parametrize("skew", [False, True])
def test_indexer_prepared_topk_matches_oracle(csl, skew):
    """Long rows: the indexer leaves slice candidates and the selection finishes from them.
    With skew the best keys crowd into two slices, the lists cannot prove the k-th exact,
    and the selection must fall back to a pass over the whole row."""
    from tests._parity import topk_band_check
    print(f"prepared top-k skew={skew}", flush=True)
    lane = W.Lane("csa", (1 << 20, 300000, 4000), (1 << 20, 300000, 4000), T=1, H=64, m=4, k=1024, HI=8)
    li = synth.generate(W.Workload("prep", 7, (lane,)), parts=("qI", "kI", "w")).lanes[0]
    kI = li.kI.clone()
    if skew:
        lead = li.qI[0, 0].float().sum(0)
        kI[1000:3048] = (lead * 4 + 0.05 * kI[1000:3048].float()).to(torch.bfloat16)
    E = lane.entries
    B = len(E)
    scores = torch.empty((B, 1, max(E)), device="cuda")
    ws = torch.zeros(csl.topk_workspace_bytes(B, 1, max(E), 1024), dtype=torch.uint8, device="cuda")
    idx = torch.empty((B, 1, 1024), dtype=torch.int32, device="cuda")
    idx2 = torch.empty_like(idx)
    d = dict(ent_off=dev(li.ent_off), q_pos=dev(li.q_pos))
    for rep in range(2):
        csl.indexer_scores(dev(li.qI), dev(li.w), dev(kI), d["ent_off"], d["q_pos"], 4, scores, topk_ws=ws,
                           topk_k=1024)
        csl.topk_select(scores, d["ent_off"], d["q_pos"], 4, 1024, idx, ws=ws, prepared=True)
        csl.topk_select(scores, d["ent_off"], d["q_pos"], 4, 1024, idx2, ws=ws, prepared=False)
        torch.cuda.synchronize()
        assert torch.equal(idx, idx2), "selection from candidate lists differs from the full path"
    keys = pipeline.index_keys_f64(kI)
    got = idx.cpu().numpy()
    for b in range(B):
        ref_s = csa.indexer(f64(li.qI[b, 0]), f64(li.w[b, 0]), keys[int(li.ent_off[b]):int(li.ent_off[b + 1])])
        topk_band_check(got[b, 0], ref_s, 1024, what=f"b={b}")


# ------------------------------------------------------------------------------- attention

def _attn_inputs(lengths, m, H, T, q_pos, seed):
    D = 128
    kv_off, ent_off = _offsets(lengths, m)
    kv = W.normal_bf16(seed, W.S_EXTRA + 4, (sum(lengths), D))
    ckv = W.normal_bf16(seed, W.S_EXTRA + 5, (max(int(ent_off[-1]), 1), D), std=0.5)
    q = W.normal_bf16(seed, W.S_EXTRA + 6, (len(lengths), T, H, D))
    return kv, ckv, q, kv_off, ent_off, torch.tensor(q_pos, dtype=torch.int64)


@pytest.mark.parametrize("H,T,lengths,q_pos,k,n_win,fill", [
    (16, 1, [4096], [4096], 64, 128, 1.0),
    (64, 1, [1 << 16, 4000, 300], [1 << 16, 4000, 300], 1024, 128, 1.0),
    (64, 2, [20000, 90], [19000, 60], 512, 128, 0.6),
    (32, 3, [5000], [100], 100, 128, 1.0),
    (64, 1, [4096, 4096], [4096, 4096], 0, 128, 1.0),
    (16, 1, [800, 800], [800, 800], 256, 0, 0.3),
    (128, 1, [9000], [9000], 200, 50, 1.0),
    (64, 40, [3000], [2500], 96, 128, 0.9),
    (16, 1, [4096], [4096], 32, 16, 1.0),         # one tile per row: the single-tile kernel
    (48, 2, [300, 50], [300, 50], 40, 24, 0.8),   # 3 head groups, at most one tile
    (80, 300, [5000], [4000], 64, 64, 1.0),       # 300 rows: one split per row, no merge
    (32, 300, [6000], [5000], 256, 128, 0.9),     # 2 splits of 3 tiles: the prefetching tile loop + merge
])
def test_sparse_attention_matches_oracle(csl, H, T, lengths, q_pos, k, n_win, fill):
    print(f"sparse attn H={H} T={T} lengths={lengths} k={k} n_win={n_win} fill={fill}", flush=True)
    m = 4
    kv, ckv, q, kv_off, ent_off, qp = _attn_inputs(lengths, m, H, T, q_pos, 41 + H + T)
    B = len(lengths)
    nvis = [[csa.n_visible(q_pos[b] + t, m, lengths[b] // m) for t in range(T)] for b in range(B)]
    idx = torch.full((B, T, k), -1, dtype=torch.int32)
    for b in range(B):
        sel = synth.random_selection(500 + b, T, nvis[b], k, fill=fill) if k else None
        if k:
            idx[b] = sel
    sc = 1 / math.sqrt(128)
    out = torch.full((B, T, H, 128), float("nan"), device="cuda")
    lse = torch.full((B, T, H), float("nan"), device="cuda")
    csl.sparse_attn_decode(dev(q), dev(ckv), dev(idx), dev(kv), dev(kv_off), dev(ent_off), dev(qp), n_win, out,
                           lse=lse, scale=sc)
    torch.cuda.synchronize()
    ro, rl = pipeline.sparse_attn_lane(q, ckv, idx.numpy(), kv, kv_off, ent_off, qp, n_win, sc)
    assert_attn_close(f64(out), ro, "out")
    assert_attn_close(f64(lse), rl, "lse")


def test_sparse_attention_ignores_out_of_range_ids_and_empty_sets(csl):
    m, H, k = 4, 64, 128
    lengths = [1000, 1000]
    kv, ckv, q, kv_off, ent_off, qp = _attn_inputs(lengths, m, H, 1, [1000, 1000], 77)
    idx = synth.random_selection(9, 2, [250, 250], k).view(2, 1, k)
    bad = idx.clone()
    bad[0, 0, 5] = 250 + 17          # beyond E_b: treated as padding
    bad[1, 0, :] = -1                # nothing selected
    out = torch.empty((2, 1, H, 128), device="cuda")
    lse = torch.empty((2, 1, H), device="cuda")
    csl.sparse_attn_decode(dev(q), dev(ckv), dev(bad), dev(kv), dev(kv_off), dev(ent_off), dev(qp), 0, out, lse=lse)
    torch.cuda.synchronize()
    ref_idx = bad.clone()
    ref_idx[0, 0, 5] = -1
    ro, rl = pipeline.sparse_attn_lane(q, ckv, ref_idx.numpy(), kv, kv_off, ent_off, qp, 0, 128 ** -0.5)
    assert_attn_close(f64(out), ro, "out")
    assert np.all(f64(out)[1] == 0) and np.all(np.isneginf(f64(lse)[1]))


@pytest.mark.parametrize("H,T,lengths,q_pos,m,n_win", [
    (64, 1, [131072, 131072], [131072, 131072], 128, 128),
    (64, 1, [1 << 20, 70000, 100], [1 << 20, 70000, 100], 128, 128),
    (16, 4, [9000], [7000], 4, 128),
    (64, 1, [127, 128, 129], [127, 128, 129], 128, 128),
    (32, 2, [5000], [5000], 4, 0),
    (96, 1, [2000, 700], [2000, 700], 128, 32),   # at most 47 keys: the single-tile kernel, 6 head groups
    (16, 300, [40000], [39000], 128, 128),        # 2 splits of 4 tiles: the prefetching tile loop, dense
])
def test_hca_attention_matches_oracle(csl, H, T, lengths, q_pos, m, n_win):
    print(f"hca attn H={H} T={T} lengths={lengths} m={m} n_win={n_win}", flush=True)
    kv, ckv, q, kv_off, ent_off, qp = _attn_inputs(lengths, m, H, T, q_pos, 61 + H)
    B = len(lengths)
    max_e = max(n // m for n in lengths)
    out = torch.full((B, T, H, 128), float("nan"), device="cuda")
    lse = torch.full((B, T, H), float("nan"), device="cuda")
    csl.hca_attn_decode(dev(q), dev(ckv), dev(kv), dev(kv_off), dev(ent_off), dev(qp), m, n_win, out, lse=lse,
                        max_entries=max_e)
    torch.cuda.synchronize()
    ro, rl = pipeline.hca_attn_lane(q, ckv, kv, kv_off, ent_off, qp, m, n_win, 128 ** -0.5)
    assert_attn_close(f64(out), ro, "out")
    assert_attn_close(f64(lse), rl, "lse")


# ------------------------------------------------- attention extras: sink and partial RoPE

@pytest.mark.parametrize("kind,H,T,lengths,q_pos,k,m,n_win,rope,base,with_sink", [
    ("csa", 64, 1, [(1 << 20) + 3, 4000], [(1 << 20) + 3, 4000], 1024, 4, 128, 64, 10000.0, True),  # 9 splits + merge
    ("csa", 16, 1, [4096], [4096], 32, 4, 16, 64, 10000.0, True),          # one split: the kernel's own epilogue
    ("csa", 64, 300, [5000], [4000], 64, 4, 64, 64, 10000.0, True),        # 300 positions, one split per row
    ("csa", 32, 300, [6000], [5000], 256, 4, 128, 64, 160000.0, True),     # prefetching loop + merge, base 160000
    ("csa", 48, 2, [300, 50], [300, 50], 40, 4, 24, 64, 10000.0, False),   # 3 head groups, no sink
    ("csa", 64, 1, [9000], [9000], 200, 4, 50, 0, 10000.0, True),          # sink alone
    ("hca", 64, 1, [131072, 9000], [131072, 9000], 0, 128, 128, 64, 10000.0, True),
    ("hca", 16, 4, [9000], [7000], 0, 4, 128, 64, 500000.0, False),
    ("hca", 16, 300, [40000], [39000], 0, 128, 128, 64, 10000.0, True),   # 2 splits of 4 tiles + merge
])
def test_attention_extras_match_oracle(csl, kind, H, T, lengths, q_pos, k, m, n_win, rope, base, with_sink):
    print(f"attn extras {kind} H={H} T={T} lengths={lengths} k={k} m={m} n_win={n_win} rope={rope} "
          f"base={base} sink={with_sink}", flush=True)
    kv, ckv, q, kv_off, ent_off, qp = _attn_inputs(lengths, m, H, T, q_pos, 71 + H + T)
    B = len(lengths)
    sink = None
    if with_sink:
        sink = W.normal_f32(71 + H, W.S_EXTRA + 7, (H,), std=2.0)
        sink[0] = float("-inf")          # a head without a sink
        sink[1] = 9.0                    # a head whose sink outweighs every key
    out = torch.full((B, T, H, 128), float("nan"), device="cuda")
    lse = torch.full((B, T, H), float("nan"), device="cuda")
    sc = 128 ** -0.5
    if kind == "csa":
        nvis = [[csa.n_visible(q_pos[b] + t, m, lengths[b] // m) for t in range(T)] for b in range(B)]
        idx = torch.stack([synth.random_selection(600 + b, T, nvis[b], k, fill=0.9) for b in range(B)])
        csl.sparse_attn_decode(dev(q), dev(ckv), dev(idx), dev(kv), dev(kv_off), dev(ent_off), dev(qp), n_win, out,
                               lse=lse, scale=sc, sink=dev(sink), rope_dims=rope, rope_base=base)
        torch.cuda.synchronize()
        ro, rl = pipeline.sparse_attn_lane(q, ckv, idx.numpy(), kv, kv_off, ent_off, qp, n_win, sc,
                                           sink=None if sink is None else sink.numpy(), rope_dims=rope,
                                           rope_base=base)
    else:
        max_e = max(n // m for n in lengths)
        csl.hca_attn_decode(dev(q), dev(ckv), dev(kv), dev(kv_off), dev(ent_off), dev(qp), m, n_win, out, lse=lse,
                            scale=sc, max_entries=max_e, sink=dev(sink), rope_dims=rope, rope_base=base)
        torch.cuda.synchronize()
        ro, rl = pipeline.hca_attn_lane(q, ckv, kv, kv_off, ent_off, qp, m, n_win, sc,
                                        sink=None if sink is None else sink.numpy(), rope_dims=rope, rope_base=base)
    assert_attn_close(f64(out), ro, "out")
    assert_attn_close(f64(lse), rl, "lse")


def test_attention_extras_on_empty_sets(csl):
    """A row that sees nothing: output 0 and lse equal to each head's sink logit."""
    H, k = 16, 64
    lengths = [1000, 1000]
    kv, ckv, q, kv_off, ent_off, qp = _attn_inputs(lengths, 4, H, 1, [1000, 1000], 78)
    idx = torch.full((2, 1, k), -1, dtype=torch.int32)
    sink = W.normal_f32(78, W.S_EXTRA + 7, (H,), std=2.0)
    out = torch.full((2, 1, H, 128), float("nan"), device="cuda")
    lse = torch.full((2, 1, H), float("nan"), device="cuda")
    csl.sparse_attn_decode(dev(q), dev(ckv), dev(idx), dev(kv), dev(kv_off), dev(ent_off), dev(qp), 0, out, lse=lse,
                           sink=dev(sink), rope_dims=64)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    # the kernel keeps logits in base 2 (a log2(e) prescale, then ln 2 back): a few ulps
    torch.testing.assert_close(lse.cpu(), sink.view(1, 1, H).expand(2, 1, H), rtol=1e-6, atol=1e-6)


def test_attention_extras_argument_errors(csl):
    lengths = [256]
    kv, ckv, q, kv_off, ent_off, qp = _attn_inputs(lengths, 4, 16, 1, [256], 79)
    idx = torch.zeros((1, 1, 8), dtype=torch.int32, device="cuda")
    out = torch.full((1, 1, 16, 128), float("nan"), device="cuda")
    for kw, status in (({"rope_dims": 48}, 2), ({"rope_dims": 32}, 2), ({"rope_dims": 64, "rope_base": 1.0}, 1),
                       ({"rope_dims": -32}, 1), ({"rope_dims": 64, "rope_base": float("inf")}, 1)):
        with pytest.raises(csl.CslError) as e:
            csl.sparse_attn_decode(dev(q), dev(ckv), idx, dev(kv), dev(kv_off), dev(ent_off), dev(qp), 0, out, **kw)
        assert e.value.status == status, kw
    torch.cuda.synchronize()
    assert torch.isnan(out).all()


def test_calls_are_deterministic(csl):
    lane = W.Lane("csa", (200000,), (200000,), T=1, H=64, m=4, k=1024, HI=8)
    li = synth.generate(W.Workload("det", 5, (lane,)), parts=("qI", "kI", "w")).lanes[0]
    E = lane.entries[0]
    outs = []
    for _ in range(2):
        s = torch.empty((1, 1, E), device="cuda")
        csl.indexer_scores(dev(li.qI), dev(li.w), dev(li.kI), dev(li.ent_off), dev(li.q_pos), 4, s)
        idx = torch.empty((1, 1, 1024), dtype=torch.int32, device="cuda")
        csl.topk_select(s, dev(li.ent_off), dev(li.q_pos), 4, 1024, idx)
        outs.append((s.cpu(), idx.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
