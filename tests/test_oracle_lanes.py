"""Pins of the oracle's batch drivers (oracle/pipeline.py) on ragged, multi-row inputs (CPU).

The per-row functions of oracle/csa.py are pinned in test_oracle.py. Here the drivers that
loop over packed sequences and query rows are checked on B = 3 sequences of unequal length
with T = 2 query rows each, against values computed a different way:
  * the fp8 key decode with per-sequence group scales ([P1] section 4.2, low-precision
    indexer keys) against the fp32 values the keys were encoded from, with group
    magnitudes chosen so that a scale taken from the wrong group or sequence is off by a
    factor of two or more;
  * the indexer, sparse and HCA attention drivers against per-row calls with the row's own
    slice of the packed arrays and its own position, and against torch's
    scaled_dot_product_attention at m = 1 without a window, where CSA with every visible
    entry selected and HCA are both plain causal attention over the raw rows
    ([P5] the attention formula; [P2] "Heavily Compressed Attention").
"""
import math

import numpy as np
import torch

import synth
from oracle import csa, pipeline
from synth import workloads as W


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------- fp8 keys, group scales

def test_index_keys_fp8_synth_lane_reproduces_the_draws():
    """A ragged fp8 lane of three sequences whose entry counts are not multiples of the
    64-entry group: every decoded key equals its fp32 draw to e4m3 precision (3 mantissa
    bits, subnormal quantum 2^-9 of the scale)."""
    lane = W.Lane("csa", (1000, 333, 523), (1000, 333, 523), T=1, H=16, m=4, k=8, HI=4, kI_fp8=True)
    wl = W.Workload("fp8_ragged", 11, (lane,))
    li = synth.generate(wl, parts=("kI",)).lanes[0]
    E = sum(lane.entries)
    assert lane.entries == [250, 83, 130]
    x = W.normal_f32(11, W.S_KI, (E * 64,), std=0.125).view(E, 64).double().numpy()
    got = pipeline.index_keys_f64(li.kI, li.k_scale, li.scale_off, li.ent_off, lane.scale_group)
    sc = li.k_scale.double().numpy()
    # the scale of entry e: by hand, group by group of each sequence
    grp = np.concatenate([np.arange(250) // 64, 4 + np.arange(83) // 64, 6 + np.arange(130) // 64])
    tol = np.abs(x) * 2.0 ** -4 + sc[grp][:, None] * 2.0 ** -9
    assert np.all(np.abs(got - x) <= tol)


def test_index_keys_fp8_scale_is_per_sequence_group():
    """Keys whose groups differ in magnitude by powers of two (sequence b, group j scaled by
    2^(3b + j)); sequence lengths 70, 129 and 5 entries put group borders at different
    global offsets, so a scale looked up by global entry index, by the wrong sequence, or
    per entry instead of per group misses by at least a factor of two."""
    r = _rng(3)
    ents = [70, 129, 5]
    blocks = []
    for b, e in enumerate(ents):
        x = r.standard_normal((e, 64)) * 0.125
        mag = np.exp2(3.0 * b + np.arange(e) // 64)
        blocks.append(x * mag[:, None])
    x = np.concatenate(blocks).astype(np.float32)
    codes, scales = W._encode_e4m3(torch.from_numpy(x), ents, 64)
    ent_off = np.concatenate([[0], np.cumsum(ents)])
    scale_off = [0, 2, 5, 6]                       # ceil(70/64), ceil(129/64), ceil(5/64)
    assert scales.shape == (6,)
    got = pipeline.index_keys_f64(codes, scales, scale_off, ent_off, 64)
    xd = x.astype(np.float64)
    assert np.all(np.abs(got - xd) <= np.abs(xd) * 2.0 ** -4 + np.abs(xd).max(axis=1, keepdims=True) * 2.0 ** -8)
    # every group's largest key is encoded at the top of the e4m3 range
    for b, e in enumerate(ents):
        for j in range(0, e, 64):
            tile = got[ent_off[b] + j: ent_off[b] + min(e, j + 64)]
            ref = xd[ent_off[b] + j: ent_off[b] + min(e, j + 64)]
            np.testing.assert_allclose(np.abs(tile).max(), np.abs(ref).max(), rtol=2.0 ** -4)


def test_index_keys_bf16_and_group_of_one():
    r = _rng(4)
    kb = torch.from_numpy(r.standard_normal((9, 64))).to(torch.bfloat16)
    np.testing.assert_array_equal(pipeline.index_keys_f64(kb), kb.double().numpy())
    # scale_group = 1: one scale per entry (the per-row reading of the group scale)
    x = (r.standard_normal((7, 64)) * np.exp2(np.arange(7))[:, None]).astype(np.float32)
    codes, scales = W._encode_e4m3(torch.from_numpy(x), [7], 1)
    got = pipeline.index_keys_f64(codes, scales, [0, 7], [0, 7], 1)
    assert np.all(np.abs(got - x) <= np.abs(x) * 2.0 ** -4 + np.abs(x).max(axis=1, keepdims=True) * 2.0 ** -8)


# ------------------------------------------------------------- multi-row drivers, B=3, T=2

def _ragged(seed, lengths, q_pos, m, D=32, H=4, HI=2, CI=16, T=2):
    r = _rng(seed)
    N = sum(lengths)
    kv = torch.from_numpy(r.standard_normal((N, D))).to(torch.bfloat16)
    z = torch.from_numpy(r.standard_normal((N, D))).to(torch.bfloat16)
    q = torch.from_numpy(r.standard_normal((len(lengths), T, H, D))).to(torch.bfloat16)
    qI = torch.from_numpy(r.standard_normal((len(lengths), T, HI, CI)))
    w = torch.from_numpy(r.random((len(lengths), T, HI)))
    kv_off = np.concatenate([[0], np.cumsum(lengths)]).tolist()
    ents = [n // m for n in lengths]
    ent_off = np.concatenate([[0], np.cumsum(ents)]).tolist()
    keys = r.standard_normal((sum(ents), CI))
    return kv, z, q, qI, w, keys, kv_off, ent_off


def test_indexer_lane_rows_see_their_own_position():
    """Rows (b, t) at p = q_pos[b] + t: the score row has floor(p/m) entries (capped by the
    sequence's entries), counted here by hand, with each score the weighted ReLU sum."""
    m = 4
    lengths = [61, 40, 23]           # 15, 10 and 5 entries
    q_pos = [51, 39, 30]             # rows see 12/13, 9/10 and 5/5 entries
    kv, z, q, qI, w, keys, kv_off, ent_off = _ragged(5, lengths, q_pos, m)
    sc = pipeline.indexer_lane(qI, w, keys, ent_off, q_pos, m)
    expect_n = [[12, 13], [9, 10], [5, 5]]
    qd, wd = qI.double().numpy(), w.double().numpy()
    for b in range(3):
        kb = keys[ent_off[b]:ent_off[b + 1]]
        for t in range(2):
            n = expect_n[b][t]
            assert sc[b][t].shape == (n,)
            ref = np.maximum(kb[:n] @ qd[b, t].T, 0.0) @ wd[b, t]          # [n, HI] @ [HI]
            np.testing.assert_allclose(sc[b][t], ref, rtol=1e-13, atol=1e-15)
    # the lane equals per-row calls of the per-row function
    for b in range(3):
        for t in range(2):
            n = csa.n_visible(q_pos[b] + t, m, ent_off[b + 1] - ent_off[b])
            np.testing.assert_array_equal(sc[b][t], csa.indexer(qd[b, t], wd[b, t],
                                                                 keys[ent_off[b]:ent_off[b] + n]))


def test_sparse_and_hca_lanes_equal_per_row_calls():
    m, W_ = 4, 8
    lengths = [61, 40, 23]
    q_pos = [51, 39, 21]
    kv, z, q, qI, w, keys, kv_off, ent_off = _ragged(6, lengths, q_pos, m)
    ckv = csa.to_bf16_f64(pipeline.compress_lane(kv, z, kv_off, m))
    k = 6
    r = _rng(7)
    idx = np.full((3, 2, k), -1, dtype=np.int64)
    for b in range(3):
        for t in range(2):
            nv = csa.n_visible(q_pos[b] + t, m, ent_off[b + 1] - ent_off[b])
            sel = np.sort(r.choice(nv, size=min(k - 1, nv), replace=False))
            idx[b, t, :len(sel)] = sel
    sc = 1 / math.sqrt(32)
    o, lse = pipeline.sparse_attn_lane(q, ckv, idx, kv, kv_off, ent_off, q_pos, W_, sc)
    oh, lh = pipeline.hca_attn_lane(q, ckv, kv, kv_off, ent_off, q_pos, m, W_, sc)
    qd, kvd = q.double().numpy(), kv.double().numpy()
    for b in range(3):
        ckv_b = ckv[ent_off[b]:ent_off[b + 1]]
        kv_b = kvd[kv_off[b]:kv_off[b + 1]]
        for t in range(2):
            p = q_pos[b] + t
            ro, rl = csa.sparse_attn(qd[b, t], ckv_b, kv_b, idx[b, t], p, W_, sc)
            np.testing.assert_array_equal(o[b, t], ro)
            np.testing.assert_array_equal(lse[b, t], rl)
            ro, rl = csa.hca_attn(qd[b, t], ckv_b, kv_b, p, m, W_, sc)
            np.testing.assert_array_equal(oh[b, t], ro)
            np.testing.assert_array_equal(lh[b, t], rl)
            # the attended set by hand: the selected entries, then raw rows max(0, p-7)..p
            sel = idx[b, t][idx[b, t] >= 0]
            hi = min(p, lengths[b] - 1)
            X = np.concatenate([ckv_b[sel], kv_b[max(0, hi - W_ + 1):hi + 1]])
            eo, el = csa.attend(qd[b, t], X, sc)
            np.testing.assert_allclose(o[b, t], eo, rtol=1e-13, atol=1e-14)


def _sdpa_causal_rows(q_bt, rows, sc):
    qt = torch.from_numpy(q_bt)[None, :, None, :]
    kt = torch.from_numpy(rows)[None, None].expand(1, q_bt.shape[0], -1, -1)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=sc)[0, :, 0, :].numpy()


def test_lanes_at_m1_without_window_are_causal_sdpa():
    """m = 1, no window: entry s is raw row s, a row at p sees rows s < p; CSA with every
    visible id selected and HCA both equal SDPA over those rows, row by row (B = 3, T = 2)."""
    lengths = [37, 20, 9]
    q_pos = [30, 18, 7]
    kv, z, q, qI, w, keys, kv_off, ent_off = _ragged(8, lengths, q_pos, 1)
    ckv = pipeline.compress_lane(kv, z, kv_off, 1)          # m = 1: the rows themselves
    np.testing.assert_array_equal(ckv, kv.double().numpy())
    k = 40
    idx = np.full((3, 2, k), -1, dtype=np.int64)
    for b in range(3):
        for t in range(2):
            nv = min(q_pos[b] + t, lengths[b])
            idx[b, t, :nv] = np.arange(nv)
    sc = 1 / math.sqrt(32)
    o, _ = pipeline.sparse_attn_lane(q, ckv, idx, kv, kv_off, ent_off, q_pos, 0, sc)
    oh, _ = pipeline.hca_attn_lane(q, ckv, kv, kv_off, ent_off, q_pos, 1, 0, sc)
    qd, kvd = q.double().numpy(), kv.double().numpy()
    for b in range(3):
        for t in range(2):
            nv = min(q_pos[b] + t, lengths[b])
            ref = _sdpa_causal_rows(qd[b, t], kvd[kv_off[b]:kv_off[b] + nv], sc)
            np.testing.assert_allclose(o[b, t], ref, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(oh[b, t], ref, rtol=1e-12, atol=1e-13)


def test_csa_step_chains_the_lane_drivers():
    """pipeline.csa_step on B = 3, T = 2 equals compress -> bf16 -> indexer -> top-k ->
    attention composed here from per-row calls."""
    m, k, W_ = 4, 3, 5
    lengths = [61, 40, 23]
    q_pos = [51, 39, 21]
    kv, z, q, qI, w, keys, kv_off, ent_off = _ragged(9, lengths, q_pos, m)
    sc = 0.2
    ckv, scores, idx, o, lse = pipeline.csa_step(kv, z, q, qI, w, keys, kv_off, q_pos, m, k, W_, sc)
    kvd, zd, qd = kv.double().numpy(), z.double().numpy(), q.double().numpy()
    for b in range(3):
        kv_b, z_b = kvd[kv_off[b]:kv_off[b + 1]], zd[kv_off[b]:kv_off[b + 1]]
        ckv_b = csa.to_bf16_f64(csa.compress(kv_b, z_b, m))
        np.testing.assert_array_equal(ckv[ent_off[b]:ent_off[b + 1]], ckv_b)
        for t in range(2):
            p = q_pos[b] + t
            nv = csa.n_visible(p, m, len(ckv_b))
            s = csa.indexer(qI.double().numpy()[b, t], w.double().numpy()[b, t], keys[ent_off[b]:ent_off[b] + nv])
            sel = csa.topk(s, k)
            np.testing.assert_array_equal(idx[b, t], sel)
            ro, rl = csa.sparse_attn(qd[b, t], ckv_b, kv_b, sel, p, W_, sc)
            np.testing.assert_array_equal(o[b, t], ro)
            np.testing.assert_array_equal(lse[b, t], rl)
