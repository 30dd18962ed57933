"""End-to-end parity of the five workloads at their full sizes (GPU).

Each test runs the whole lane on the GPU (bulk compression of the context, then one step:
newest-chunk compression, indexer, top-k and sparse attention for CSA; dense attention
for HCA) with exactly the launch configuration the benchmark times, and checks it against
the fp64 oracle run on the same seeded inputs. Where a full oracle pass would take too
long, sampled outputs are computed one by one (compressed entries, query rows) and every
output is checked for properties that hold at any size.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import csa, pipeline
from tests._parity import (assert_attn_close, assert_rows_close, f64, topk_band_check)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lanes_mod():
    from compressed_sparse_long_amd import lanes
    return lanes


def _oracle_entries(kv, z, row0, m, ids):
    """Oracle compressed rows of entries ``ids`` of the sequence whose raw rows start at row0."""
    ids = np.asarray(ids, dtype=np.int64)
    if ids.size == 0:
        return np.zeros((0, kv.shape[1]))
    rows = (row0 + ids[:, None] * m + np.arange(m)[None, :]).reshape(-1)
    rt = torch.from_numpy(rows)
    kvs = f64(kv.index_select(0, rt))
    zs = None if z is None else f64(z.index_select(0, rt))
    return csa.compress(kvs, zs, m)


def _oracle_overlap_entries(kv_a, z_a, kv_b, z_b, row0, m, ids):
    """Oracle overlapped entries ``ids`` of the sequence whose raw rows start at row0: entry i
    is entry 1 of the two-block sequence made of blocks i-1 and i of both series (entry 0:
    entry 0 of block 0 alone)."""
    out = np.zeros((len(ids), kv_a.shape[1]))
    for j, i in enumerate(np.asarray(ids, dtype=np.int64).tolist()):
        lo = row0 + m * max(i - 1, 0)
        hi = row0 + m * (i + 1)
        loc = [None if t is None else f64(t[lo:hi]) for t in (kv_a, z_a, kv_b, z_b)]
        out[j] = csa.compress_overlap(*loc, m)[min(i, 1)]
    return out


def _oracle_attention(q_bt, kv, z, lane, b, p, sel, scale, entries_fn=None, extras=None):
    """Oracle attention of one query row: its selected entries (oracle-compressed, in the bf16
    cache format) followed by the raw window rows. ``entries_fn(row0, m, ids)`` gives the
    compressed entries (default: single-series compression of kv, z); ``extras`` is
    (sink, rope_dims, rope_base) or None."""
    row0 = lane.kv_off()[b]
    n_b = lane.lengths[b]
    if entries_fn is None:
        entries_fn = lambda r0, m, ids: _oracle_entries(kv, z, r0, m, ids)
    comp = csa.to_bf16_f64(entries_fn(row0, lane.m, sel))
    win = list(csa.window_rows(p, n_b, lane.W))
    wrows = f64(kv[row0 + win[0]: row0 + win[-1] + 1]) if win else np.zeros((0, kv.shape[1]))
    X = np.concatenate([comp, wrows], axis=0)
    if extras is None:
        return csa.attend(f64(q_bt), X, scale)
    sink, rope_dims, rope_base = extras
    return csa.attend_at(f64(q_bt), X, scale, p, sink, rope_dims, rope_base)


def _entry_rows(cl, lane, b, ids):
    """Cache rows of entries ``ids`` of sequence b: packed, or their pool rows when paged."""
    ids = torch.from_numpy(np.asarray(ids, dtype=np.int64))
    if cl.paged is None:
        return lane.ent_off()[b] + ids
    eb = cl.paged.block_entries
    return cl.paged.block_table[b].cpu().to(torch.int64)[ids // eb] * eb + ids % eb


def _check_compressed_sample(cl, kv, z, lane, nsample, seed, entries_fn=None):
    g = np.random.default_rng(seed)
    ckv = cl.ckv
    if entries_fn is None:
        entries_fn = lambda r0, m, ids: _oracle_entries(kv, z, r0, m, ids)
    for b in range(lane.B):
        E = lane.entries[b]
        if E == 0:
            continue
        ids = np.unique(np.concatenate([[0, 1, E - 1], g.integers(0, E, size=min(nsample, E))]))
        ids = ids[ids < E]
        ref = entries_fn(lane.kv_off()[b], lane.m, ids)
        got = f64(ckv[_entry_rows(cl, lane, b, ids).to(ckv.device)])
        assert_rows_close(got, ref, bf16=True, what=f"compressed entries of seq {b}")


def _check_csa_row(cl, inp, li, b, t, keys_f64, entries_fn=None, extras=None):
    lane = li.lane
    p = lane.q_pos[b] + t
    E = lane.entries[b]
    n = csa.n_visible(p, lane.m, E)
    e0 = lane.ent_off()[b]
    ref_s = csa.indexer(f64(li.qI[b, t]), f64(li.w[b, t]), keys_f64[e0:e0 + n])
    got_s = f64(cl.scores[b, t, :n])
    assert_rows_close(got_s, ref_s, what=f"scores b={b} t={t}")
    got_idx = cl.idx[b, t].cpu().numpy()
    same = topk_band_check(got_idx, ref_s, lane.k, what=f"top-k b={b} t={t}")
    # the band check has shown the GPU's selection to be a valid top-k of the oracle's
    # scores; the attention is then held to the oracle's attention over that same selection
    sel = got_idx[got_idx >= 0]
    ro, rl = _oracle_attention(inp.q[li.q_slice][b, t], inp.kv, inp.z, lane, b, p, sel, cl.scale, entries_fn,
                               extras)
    tag = "" if same else " (band swap: oracle over the GPU's selection)"
    go, gl = f64(cl.out[b, t]), f64(cl.lse[b, t])
    assert_attn_close(go, ro, f"out b={b} t={t}{tag}")
    assert_attn_close(gl, rl, f"lse b={b} t={t}{tag}")


def _csa_keys(li):
    return pipeline.index_keys_f64(li.kI, li.k_scale, li.scale_off, li.ent_off, li.lane.scale_group,
                                   fp4=getattr(li.lane, "kI_fp4", False))


def _run(lanes_mod, name, overlap=False, extras=None, fp4=False, paged=None):
    print(f"workload {name}{' (overlapped compression)' if overlap else ''}"
          f"{' (sink, rope)' if extras else ''}{' (MXFP4 keys)' if fp4 else ''}"
          f"{f' (paged, {paged} blocks)' if paged else ''}: generating inputs", flush=True)
    parts = ("kv", "z", "q", "qI", "kI", "w") + (("kv_b", "z_b") if overlap else ())
    wl = synth.WORKLOADS[name]
    if fp4:
        from synth import workloads as W
        wl = W.with_lanes(wl, kI_fp4=True)
    inp = synth.generate(wl, parts=parts)
    print(f"workload {name}: running on the GPU", flush=True)
    cls = lanes_mod.build_lanes(inp)
    for cl in cls:
        if extras is not None:
            cl.sink = extras[0].to(cl.q.device)
            cl.rope_dims, cl.rope_base = extras[1], extras[2]
        cl.compress_all()
        if paged:
            # entries, indexer keys (and fp8 scales) into the block pool, raw rows into rings
            cl.paginate(ring_rows=256, seed=5, order=paged)
        cl.step()
    torch.cuda.synchronize()
    print(f"workload {name}: checking against the oracle", flush=True)
    return inp, cls


def test_csa_decode_4k(lanes_mod):
    inp, (cl,) = _run(lanes_mod, "csa_decode_4k")
    li = inp.lanes[0]
    # the cache holds one bf16 rounding of each fp32 entry: compare with the unrounded oracle
    ref_ckv = pipeline.compress_lane(inp.kv, inp.z, li.kv_off, 4)
    assert_rows_close(f64(cl.ckv), ref_ckv, bf16=True, what="ckv")
    _check_csa_row(cl, inp, li, 0, 0, _csa_keys(li))


def test_hca_decode_128k(lanes_mod):
    inp, (cl,) = _run(lanes_mod, "hca_decode_128k")
    li = inp.lanes[0]
    lane = li.lane
    for b in range(lane.B):
        E = lane.entries[b]
        ref = _oracle_entries(inp.kv, inp.z, lane.kv_off()[b], lane.m, np.arange(E))
        e0 = lane.ent_off()[b]
        assert_rows_close(f64(cl.ckv[e0:e0 + E]), ref, bf16=True, what=f"ckv seq {b}")
        p = lane.q_pos[b]
        nv = csa.n_visible(p, lane.m, E)
        ro, rl = _oracle_attention(inp.q[b, 0], inp.kv, inp.z, lane, b, p, np.arange(nv), cl.scale)
        assert_attn_close(f64(cl.out[b, 0]), ro, f"out b={b}")
        assert_attn_close(f64(cl.lse[b, 0]), rl, f"lse b={b}")


def test_csa_decode_1m(lanes_mod):
    inp, (cl,) = _run(lanes_mod, "csa_decode_1m")
    li = inp.lanes[0]
    _check_compressed_sample(cl, inp.kv, inp.z, li.lane, 2048, 1)
    keys = _csa_keys(li)
    for b in range(li.lane.B):
        _check_csa_row(cl, inp, li, b, 0, keys)


def _overlap_fn(inp):
    return lambda r0, m, ids: _oracle_overlap_entries(inp.kv, inp.z, inp.kv_b, inp.z_b, r0, m, ids)


def _sink(H, seed):
    import synth.workloads as W
    return W.normal_f32(seed, W.S_EXTRA + 7, (H,), std=2.0)


def test_csa_decode_4k_overlapped(lanes_mod):
    """The small CSA workload with overlapped (dual-series) compression: every compressed
    entry, then the step's scores, selection and attention over those entries."""
    inp, (cl,) = _run(lanes_mod, "csa_decode_4k", overlap=True)
    li = inp.lanes[0]
    ref_ckv = pipeline.compress_overlap_lane(inp.kv, inp.z, inp.kv_b, inp.z_b, li.kv_off, 4)
    assert_rows_close(f64(cl.ckv), ref_ckv, bf16=True, what="ckv (overlapped)")
    _check_csa_row(cl, inp, li, 0, 0, _csa_keys(li), _overlap_fn(inp))


def test_csa_decode_1m_overlapped_with_sink_and_rope(lanes_mod):
    """4 x 1M-token CSA decode with every option of the method: overlapped compression, a
    per-head attention sink and partial RoPE on the last 64 dims (query at p, output at -p).
    Sampled entries of the bulk pass, then every query row."""
    inp, (cl,) = _run(lanes_mod, "csa_decode_1m", overlap=True,
                      extras=(_sink(64, 8), 64, 10000.0))
    li = inp.lanes[0]
    _check_compressed_sample(cl, inp.kv, inp.z, li.lane, 1024, 5, _overlap_fn(inp))
    keys = _csa_keys(li)
    ex = (_sink(64, 8).numpy(), 64, 10000.0)
    for b in range(li.lane.B):
        _check_csa_row(cl, inp, li, b, 0, keys, _overlap_fn(inp), ex)


def test_hca_decode_128k_with_sink_and_rope(lanes_mod):
    """The HCA workload with a per-head sink and partial RoPE."""
    inp, (cl,) = _run(lanes_mod, "hca_decode_128k", extras=(_sink(64, 9), 64, 10000.0))
    li = inp.lanes[0]
    lane = li.lane
    ex = (_sink(64, 9).numpy(), 64, 10000.0)
    for b in range(lane.B):
        p = lane.q_pos[b]
        nv = csa.n_visible(p, lane.m, lane.entries[b])
        ro, rl = _oracle_attention(inp.q[b, 0], inp.kv, inp.z, lane, b, p, np.arange(nv), cl.scale, None, ex)
        assert_attn_close(f64(cl.out[b, 0]), ro, f"out b={b}")
        assert_attn_close(f64(cl.lse[b, 0]), rl, f"lse b={b}")


def test_csa_decode_1m_mxfp4_keys(lanes_mod):
    """4 x 1M-token CSA decode with MXFP4 indexer keys: every row's scores against the
    oracle on the decoded keys, the selection (boundary band) and the attention."""
    inp, (cl,) = _run(lanes_mod, "csa_decode_1m", fp4=True)
    li = inp.lanes[0]
    keys = _csa_keys(li)
    for b in range(li.lane.B):
        _check_csa_row(cl, inp, li, b, 0, keys)


def test_csa_decode_1m_paged(lanes_mod):
    """4 x 1M-token CSA decode with the cache paged: compressed entries and indexer keys in a
    pool of 32-entry blocks (seeded random block order) and raw rows in 256-row rings; every
    query row against the oracle."""
    print("workload csa_decode_1m (paged): generating inputs", flush=True)
    inp = synth.generate("csa_decode_1m")
    (cl,) = lanes_mod.build_lanes(inp)
    cl.compress_all()
    cl.paginate(ring_rows=256, seed=3)
    cl.step()
    torch.cuda.synchronize()
    print("workload csa_decode_1m (paged): checking against the oracle", flush=True)
    li = inp.lanes[0]
    keys = _csa_keys(li)
    for b in range(li.lane.B):
        _check_csa_row(cl, inp, li, b, 0, keys)


def test_csa_prefill_8k_on_128k(lanes_mod):
    inp, (cl,) = _run(lanes_mod, "csa_prefill_8k_on_128k")
    li = inp.lanes[0]
    lane = li.lane
    _check_compressed_sample(cl, inp.kv, inp.z, lane, 2048, 2)
    # every row: a valid ascending selection of exactly k visible entries
    idx = cl.idx[0].cpu().numpy()
    nv = np.array([csa.n_visible(lane.q_pos[0] + t, lane.m, lane.entries[0]) for t in range(lane.T)])
    assert np.all(idx >= 0) and np.all(idx < nv[:, None])
    assert np.all(np.diff(idx, axis=1) > 0)
    # every row: finite, non-negative visible scores (w >= 0) and finite outputs
    sc = cl.scores[0]
    col = torch.arange(sc.shape[1], device=sc.device)[None, :]
    vis = col < torch.from_numpy(nv).to(sc.device)[:, None]
    assert bool(torch.isfinite(sc[vis]).all()) and bool((sc[vis] >= 0).all())
    assert bool(torch.isfinite(cl.out).all()) and bool(torch.isfinite(cl.lse).all())
    keys = _csa_keys(li)
    # 512 rows spread evenly over the chunk (first and last included) plus the rows around
    # the 4-row compression blocks at the start, against the oracle one by one
    even = np.linspace(0, lane.T - 1, 512).round().astype(int).tolist()
    rows = sorted(set(even + [0, 1, 2, 3, 4, 5, lane.T - 2, lane.T - 1]))
    assert len(rows) >= 512 and rows[0] == 0 and rows[-1] == lane.T - 1
    for t in rows:
        _check_csa_row(cl, inp, li, 0, t, keys)


def test_csa_prefill_8k_on_128k_without_scores(lanes_mod):
    """The same prefill step with the indexer fused with top-k (no 1.14 GB score matrix):
    the ids and the attention equal the scored step's bit for bit."""
    print("workload csa_prefill_8k_on_128k without scores: generating inputs", flush=True)
    inp = synth.generate("csa_prefill_8k_on_128k")
    res = []
    for scoreless in (False, True):
        (cl,) = lanes_mod.build_lanes(inp, scoreless=scoreless)
        cl.compress_all()
        cl.step()
        torch.cuda.synchronize()
        res.append((cl.idx.clone(), cl.out.clone(), cl.lse.clone()))
        del cl
        torch.cuda.empty_cache()
    for a, b, what in zip(res[0], res[1], ("idx", "out", "lse")):
        assert torch.equal(a, b), f"{what} differs without scores"


@pytest.mark.parametrize("paged", [None, "random"])
def test_mixed_decode_b32(lanes_mod, paged):
    """Config 5; paged: the same step with both lanes' caches in block pools (the CSA lane's
    fp8 indexer keys with their group scales kept per pool block) and raw rows in rings."""
    inp, (csa_l, hca_l) = _run(lanes_mod, "mixed_decode_b32", paged=paged)
    if paged:
        assert csa_l.paged is not None and hca_l.paged is not None
        assert csa_l.k_scale.numel() == csa_l.pool_rows >> 5  # groups of 64 over blocks of 32: one per block
    li_c, li_h = inp.lanes
    keys = _csa_keys(li_c)
    for b in range(li_c.lane.B):
        _check_csa_row(csa_l, inp, li_c, b, 0, keys)
    _check_compressed_sample(csa_l, inp.kv, inp.z, li_c.lane, 256, 4)
    lane = li_h.lane
    for b in range(lane.B):
        E = lane.entries[b]
        p = lane.q_pos[b]
        nv = csa.n_visible(p, lane.m, E)
        ro, rl = _oracle_attention(inp.q[li_h.q_slice][b, 0], inp.kv, inp.z, lane, b, p, np.arange(nv), hca_l.scale)
        assert_attn_close(f64(hca_l.out[b, 0]), ro, f"hca out b={b}")
        assert_attn_close(f64(hca_l.lse[b, 0]), rl, f"hca lse b={b}")
