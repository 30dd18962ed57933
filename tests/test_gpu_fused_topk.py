"""The indexer fused with top-k (csl_indexer_topk), which never writes the score matrix (GPU).

Where indexer_scores takes its prefill tiling (B*T >= 64, T >= 16) the fused call must
return exactly what indexer_scores followed by topk_select returns: the same scores and the
same choice. Every case is also checked against the fp64 oracle's top-k within the boundary
band. Cases cover every indexer head count, the three key formats, ragged lengths and
query tiles, rows shorter than k, k at its limit, heavy exact ties (duplicated keys) and a
paged cache.
"""
import numpy as np
import pytest
import torch

import synth
from synth import workloads as W
from oracle import csa, pipeline
from tests._parity import dev, f64, topk_band_check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csl():
    import compressed_sparse_long_amd as lib
    return lib


def _lane(HI, T, lengths, q_pos, seed, fmt=None):
    lane = W.Lane("csa", tuple(lengths), tuple(q_pos), T=T, H=16, m=4, k=8, HI=HI, kI_fp8=fmt == "fp8",
                  kI_fp4=fmt == "mxfp4")
    return synth.generate(W.Workload("fused", seed, (lane,)), parts=("qI", "kI", "w")).lanes[0]


def _args(li, fmt):
    return dict(k_scale=dev(li.k_scale), scale_off=dev(li.scale_off), scale_group=64,
                k_format="mxfp4" if fmt == "mxfp4" else None)


def _fused(csl, li, kI, k, fmt, paged=None):
    B, T = li.qI.shape[:2]
    E = li.lane.entries
    idx = torch.full((B, T, k), -7, dtype=torch.int32, device="cuda")
    csl.indexer_topk(dev(li.qI), dev(li.w), kI, dev(li.ent_off), dev(li.q_pos), 4, k, idx,
                     max_entries=max(max(E), 1), paged=paged, **_args(li, fmt))
    return idx


def _unfused(csl, li, kI, k, fmt):
    B, T = li.qI.shape[:2]
    E = li.lane.entries
    me = max(max(E), 1)
    scores = torch.empty((B, T, me), dtype=torch.float32, device="cuda")
    csl.indexer_scores(dev(li.qI), dev(li.w), kI, dev(li.ent_off), dev(li.q_pos), 4, scores, max_entries=me,
                       **_args(li, fmt))
    idx = torch.full((B, T, k), -7, dtype=torch.int32, device="cuda")
    csl.topk_select(scores, dev(li.ent_off), dev(li.q_pos), 4, k, idx, max_entries=me)
    return idx


def _oracle_check(li, kI_cpu, got, k, fmt, rows=None):
    keys = pipeline.index_keys_f64(kI_cpu, li.k_scale, li.scale_off, li.ent_off, 64, fp4=fmt == "mxfp4")
    B, T = li.qI.shape[:2]
    ent = [int(x) for x in li.ent_off]
    for b in range(B):
        for t in (range(T) if rows is None else rows):
            if t >= T:
                continue
            nv = csa.n_visible(int(li.q_pos[b]) + t, 4, ent[b + 1] - ent[b])
            ref = csa.indexer(f64(li.qI[b, t]), f64(li.w[b, t]), keys[ent[b]:ent[b] + nv])
            topk_band_check(got[b, t], ref, k, what=f"b={b} t={t}")


@pytest.mark.parametrize("HI,T,lengths,q_pos,k,fmt", [
    (8, 40, [9000, 4100, 60, 2049], [8900, 4000, 0, 2000], 64, None),     # ragged rows, one short of k
    (8, 16, [20000, 3333, 7001, 500], [19000, 3300, 7001, 400], 512, None),
    (8, 33, [12000, 10000], [11900, 9900], None, None),                   # k at its limit (one workgroup per CU)
    (8, 16, [40000, 9000, 600, 5000], [39000, 8900, 500, 4900], 1024, None),  # the Pro top-k: past two workgroups' buffers
    (8, 16, [20000, 7000], [19000, 6900], 673, None),                     # the first k of the wide shape
    (8, 16, [20000, 7000], [19000, 6900], 672, None),                     # the last k of the narrow one
    (4, 20, [30000, 5000], [29000, 4900], 1500, "fp8"),
    (16, 24, [16000, 2500, 900], [15990, 2400, 800], None, None),         # HI = 16; k at its limit
    (4, 20, [5000, 1300, 2222, 17], [4900, 1250, 2100, 0], 100, None),
    (2, 17, [3000, 2000, 1000, 4000], [2999, 1999, 999, 3999], 37, None),
    (1, 64, [2500], [2400], 8, None),
    (1, 64, [9000], [8800], None, None),                                  # HI = 1; k at its limit
    (8, 18, [8000, 3000, 600, 5000], [7900, 2900, 500, 4900], 256, "fp8"),
    (8, 16, [10000, 2000, 700, 3000], [9900, 1900, 600, 2900], 512, "mxfp4"),
])
def test_fused_equals_scores_then_select(csl, HI, T, lengths, q_pos, k, fmt):
    k = k or csl.indexer_topk_max_k(HI)
    print(f"fused top-k HI={HI} T={T} lengths={lengths} k={k} fmt={fmt}", flush=True)
    li = _lane(HI, T, lengths, q_pos, 41 + HI + T, fmt)
    kI = dev(li.kI)
    got = _fused(csl, li, kI, k, fmt)
    ref = _unfused(csl, li, kI, k, fmt)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), "fused selection differs from indexer_scores + topk_select"
    _oracle_check(li, li.kI, got.cpu().numpy(), k, fmt, rows=[0, 1, T // 2, T - 1])


@pytest.mark.parametrize("distinct", [1, 7, 300])
def test_fused_ties_to_lower_ids(csl, distinct):
    """Keys repeated from a few distinct rows: equal keys give bit-equal scores, so the
    selection rests on the lower-id rule, across the candidate buffer's cuts."""
    print(f"fused top-k ties distinct={distinct}", flush=True)
    li = _lane(8, 16, [12000, 5000, 4000, 1000], [12000, 4990, 3000, 900], 77)
    E = int(li.ent_off[-1])
    src = torch.arange(E) % distinct
    kI_cpu = li.kI[src].contiguous()
    kI = dev(kI_cpu)
    for k in (1, 300, csl.indexer_topk_max_k(8)):
        got = _fused(csl, li, kI, k, None)
        ref = _unfused(csl, li, kI, k, None)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"k={k}"
    _oracle_check(li, kI_cpu, got.cpu().numpy(), csl.indexer_topk_max_k(8), None, rows=[0, 15])


def test_fused_paged_equals_packed(csl):
    from compressed_sparse_long_amd import PagedCache
    print("fused top-k paged", flush=True)
    li = _lane(8, 20, [16000, 6000, 300], [15900, 5900, 200], 91)
    E = li.lane.entries
    eb = 32
    nblk = [(e + eb - 1) // eb for e in E]
    total = sum(nblk) + 3
    perm = torch.randperm(total, generator=torch.Generator().manual_seed(5)).to(torch.int32)
    table = torch.zeros((len(E), max(nblk)), dtype=torch.int32)
    used = 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[used:used + n]
        used += n
    rows = torch.cat([table[b].long()[torch.arange(e) // eb] * eb + torch.arange(e) % eb for b, e in enumerate(E)])
    pool = torch.zeros((total * eb, 64), dtype=li.kI.dtype)
    pool[rows] = li.kI
    paged = PagedCache(dev(table), eb, total * eb, 0)
    got = _fused(csl, li, dev(pool), 512, None, paged=paged)
    ref = _fused(csl, li, dev(li.kI), 512, None)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


def test_fused_short_decode_rows_match_oracle(csl):
    """T = 1 rows (indexer_scores would take its decode tiling, whose head sum runs in
    another order): the selection still matches the oracle within the boundary band."""
    print("fused top-k decode rows", flush=True)
    li = _lane(8, 1, [40000, 3000, 10], [40000, 3000, 10], 13)
    got = _fused(csl, li, dev(li.kI), 512, None)
    torch.cuda.synchronize()
    _oracle_check(li, li.kI, got.cpu().numpy(), 512, None)


@pytest.mark.parametrize("k", [None, 1024])
def test_fused_prefill_workload_equals_scores_then_select(csl, k):
    """The 8K-query prefill on a 128K context at full size (8,192 rows x ~34K entries), at its
    k = 512 and at the Pro top-k of 1024."""
    print(f"fused top-k prefill 8k on 128k k={k}", flush=True)
    inp = synth.generate("csa_prefill_8k_on_128k", parts=("qI", "kI", "w"))
    li = inp.lanes[0]
    k = k or li.lane.k
    kI = dev(li.kI)
    got = _fused(csl, li, kI, k, None)
    ref = _unfused(csl, li, kI, k, None)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    _oracle_check(li, li.kI, got.cpu().numpy(), k, None, rows=[0, 4097, li.qI.shape[1] - 1])


def test_fused_argument_errors(csl):
    li = _lane(8, 16, [1000], [1000], 3)
    idx = torch.empty((1, 16, 8), dtype=torch.int32, device="cuda")
    base = (dev(li.qI), dev(li.w), dev(li.kI), dev(li.ent_off), dev(li.q_pos), 4)
    kmax = csl.indexer_topk_max_k(8)
    assert kmax == 1952 and csl.indexer_topk_max_k(16) == 1952 and csl.indexer_topk_max_k(1) == 672
    assert csl.indexer_topk_max_k(4) == 1952 and csl.indexer_topk_max_k(2) == 1952
    assert csl.indexer_topk_max_k(3) == 0
    with pytest.raises(csl.CslError, match="k must be in"):
        csl.indexer_topk(*base, kmax + 1, torch.empty((1, 16, kmax + 1), dtype=torch.int32, device="cuda"),
                         max_entries=250)
    with pytest.raises(csl.CslError, match="k must be in"):
        csl.indexer_topk(*base, 0, idx, max_entries=250)
    csl.indexer_topk(*base, 8, idx, max_entries=0)  # nothing visible: all padding
    torch.cuda.synchronize()
    assert bool((idx == -1).all())
