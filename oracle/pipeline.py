"""Batched drivers of the fp64 oracle over packed, ragged sequences -- TEST INFRASTRUCTURE.

Packed layout (the same as the inputs in ``synth``): sequence b owns raw rows
[kv_off[b], kv_off[b+1]) of ``kv``/``z``, compressed entries [ent_off[b], ent_off[b+1]),
and its query row t sits at absolute position q_pos[b] + t.
Each driver loops explicitly over sequence, query row and head, calling ``oracle.csa``.
"""
from __future__ import annotations

import numpy as np

from . import csa


def f64(t) -> np.ndarray:
    """fp64 numpy copy of a CPU tensor or array (bf16 values are exact in fp64)."""
    if hasattr(t, "detach"):
        import torch
        return t.detach().to(torch.float64).cpu().numpy()
    return np.asarray(t, dtype=np.float64)


def compress_lane(kv, z, kv_off, m: int) -> np.ndarray:
    """All compressed entries of every sequence, packed: [sum_b floor(N_b/m), D]."""
    kv_off = [int(x) for x in kv_off]
    out = []
    for b in range(len(kv_off) - 1):
        lo, hi = kv_off[b], kv_off[b + 1]
        kvb = f64(kv[lo:hi])
        zb = None if z is None else f64(z[lo:hi])
        out.append(csa.compress(kvb, zb, m))
    return np.concatenate(out, axis=0) if out else np.zeros((0, 0))


def compress_overlap_lane(kv_a, z_a, kv_b, z_b, kv_off, m: int) -> np.ndarray:
    """All dual-series (overlapped) compressed entries of every sequence, packed."""
    kv_off = [int(x) for x in kv_off]
    out = []
    for b in range(len(kv_off) - 1):
        lo, hi = kv_off[b], kv_off[b + 1]
        za = None if z_a is None else f64(z_a[lo:hi])
        zb = None if z_b is None else f64(z_b[lo:hi])
        out.append(csa.compress_overlap(f64(kv_a[lo:hi]), za, f64(kv_b[lo:hi]), zb, m))
    return np.concatenate(out, axis=0) if out else np.zeros((0, 0))


def index_keys_f64(kI, k_scale=None, scale_off=None, ent_off=None, group: int = 64, fp4: bool = False) -> np.ndarray:
    """Indexer keys as fp64; fp8 codes are decoded and multiplied by their group's scale;
    MXFP4 keys (``fp4``: packed codes [E, 32] and E8M0 scales [E, 2]) are decoded per block."""
    if fp4:
        pk = kI.numpy() if hasattr(kI, "numpy") else kI
        sc = k_scale.numpy() if hasattr(k_scale, "numpy") else k_scale
        return csa.decode_mxfp4_rows(pk, sc)
    if k_scale is None:
        return f64(kI)
    codes = np.asarray(kI.numpy() if hasattr(kI, "numpy") else kI, dtype=np.uint8)
    vals = csa.decode_e4m3(codes)
    sc = f64(k_scale)
    out = np.empty_like(vals)
    ent_off = [int(x) for x in ent_off]
    scale_off = [int(x) for x in scale_off]
    for b in range(len(ent_off) - 1):
        e0, e1 = ent_off[b], ent_off[b + 1]
        grp = scale_off[b] + np.arange(e1 - e0) // group     # key s of sequence b uses scale s // group
        out[e0:e1] = vals[e0:e1] * sc[grp][:, None]
    return out


def indexer_lane(qI, w, keys_f64, ent_off, q_pos, m: int) -> list:
    """Scores per (b, t): list over b of lists over t of fp64 arrays of length n_visible."""
    qI = f64(qI)
    w = f64(w)
    ent_off = [int(x) for x in ent_off]
    out = []
    for b in range(qI.shape[0]):
        E = ent_off[b + 1] - ent_off[b]
        kb = keys_f64[ent_off[b]:ent_off[b + 1]]
        rows = []
        for t in range(qI.shape[1]):
            p = int(q_pos[b]) + t
            nv = csa.n_visible(p, m, E)
            rows.append(csa.indexer(qI[b, t], w[b, t], kb[:nv]))
        out.append(rows)
    return out


def topk_lane(scores, k: int) -> np.ndarray:
    """Top-k ids per (b, t) from nested per-row score arrays: int64 [B, T, k]."""
    B = len(scores)
    T = len(scores[0])
    out = np.full((B, T, k), -1, dtype=np.int64)
    for b in range(B):
        for t in range(T):
            out[b, t] = csa.topk(scores[b][t], k)
    return out


def sparse_attn_lane(q, ckv, idx, kv, kv_off, ent_off, q_pos, W: int, scale: float, sink=None, rope_dims: int = 0,
                     rope_base: float = 10000.0):
    """CSA attention for every (b, t): o [B, T, H, D], lse [B, T, H]."""
    q = f64(q)
    B, T, H, D = q.shape
    o = np.zeros((B, T, H, D))
    lse = np.zeros((B, T, H))
    kv_off = [int(x) for x in kv_off]
    ent_off = [int(x) for x in ent_off]
    idx = np.asarray(idx)
    for b in range(B):
        ckv_b = f64(ckv[ent_off[b]:ent_off[b + 1]])
        kv_b = f64(kv[kv_off[b]:kv_off[b + 1]])
        for t in range(T):
            o[b, t], lse[b, t] = csa.sparse_attn(q[b, t], ckv_b, kv_b, idx[b, t],
                                                 int(q_pos[b]) + t, W, scale, sink, rope_dims, rope_base)
    return o, lse


def hca_attn_lane(q, ckv, kv, kv_off, ent_off, q_pos, m: int, W: int, scale: float, sink=None, rope_dims: int = 0,
                  rope_base: float = 10000.0):
    """HCA attention for every (b, t): o [B, T, H, D], lse [B, T, H]."""
    q = f64(q)
    B, T, H, D = q.shape
    o = np.zeros((B, T, H, D))
    lse = np.zeros((B, T, H))
    kv_off = [int(x) for x in kv_off]
    ent_off = [int(x) for x in ent_off]
    for b in range(B):
        ckv_b = f64(ckv[ent_off[b]:ent_off[b + 1]])
        kv_b = f64(kv[kv_off[b]:kv_off[b + 1]])
        for t in range(T):
            o[b, t], lse[b, t] = csa.hca_attn(q[b, t], ckv_b, kv_b, int(q_pos[b]) + t, m, W, scale, sink, rope_dims,
                                              rope_base)
    return o, lse


def csa_step(kv, z, q, qI, w, keys_f64, kv_off, q_pos, m: int, k: int, W: int, scale: float):
    """Whole CSA lane for every (b, t): compress (rounded to the bf16 cache format), index,
    select, attend. Returns (ckv_bf16_f64, scores, idx, o, lse)."""
    ckv = csa.to_bf16_f64(compress_lane(kv, z, kv_off, m))
    ent = [0]
    kv_off_l = [int(x) for x in kv_off]
    for b in range(len(kv_off_l) - 1):
        ent.append(ent[-1] + (kv_off_l[b + 1] - kv_off_l[b]) // m)
    scores = indexer_lane(qI, w, keys_f64, ent, q_pos, m)
    idx = topk_lane(scores, k)
    o, lse = sparse_attn_lane(q, ckv, idx, kv, kv_off, ent, q_pos, W, scale)
    return ckv, scores, idx, o, lse
