"""Per-step fp64 oracle of hybrid compressed attention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may
import this module. Nothing here is shared with, or imported by, the HIP library.

Pages cited (titles as published):
  [P1] "1M Context != Lossless Long Memory: What DeepSeek-V4 Reveals About the
       Engineering Tradeoffs" (wiki.gxlh.xyz/doc/1210)
  [P2] "DeepSeek-V4: Million-Token Context via Hybrid Compressed Attention"
       (zhongzhoutan-coder.github.io, DeepSeek-V4 training notes)
  [P3] "DeepSeek-V4 的暗线之一：分层记忆比输入框更关键" (blog.xieydd.top/deepseek-v4-memory-part1)
  [P5] "DeepSeek-V4 technical report" breakdown (deconstructedpapers.com)

Readings where the pages leave a step open (each is listed in the design notes):
  * compression weights: an explicit per-token, per-dimension logit array Z; the softmax
    runs over the m rows of one chunk, separately for every dimension ([P3] section 3,
    whose toy weights sum to one down each dimension). Z absent means uniform weights.
  * the hot path uses single-series compression for both CSA and HCA; CSA's overlapped
    dual series is the alternative compress_overlap, whose entry 0 pools series a alone.
  * one softmax covers the selected compressed entries and the raw window rows together,
    with no de-duplication between the two lanes; the attention sink, when given, is a
    per-head logit exp(z'_h) added to that softmax's denominator, carrying no value.
  * partial RoPE, when asked for, rotates the query's and the output's last dims (pairs of
    adjacent dims, angle pos * base^(-2j/R)); key rows are taken as stored.
  * a query at absolute position p sees compressed entries s < floor(p/m) (never its own
    block, [P1] section 6.1) and the window of the W newest raw rows j <= p that exist.
  * top-k keeps the k largest scores, lower entry id first on ties, and returns the ids
    in ascending order padded with -1.
  * an empty attention set yields a zero output and lse = -inf (the sink logit, if given).
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------- numbers

def decode_e4m3(codes) -> np.ndarray:
    """Value of OCP fp8 E4M3FN codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
    no infinities, S.1111.111 is NaN, exponent 0 is subnormal: f * 2^-9).

    The pages use low-precision (FP8 / FP4) indexer keys ([P1] section 2, footnote 3;
    section 4.2); the format itself is the published OCP 8-bit floating point definition.
    """
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 0xF
    f = b & 0x7
    normal = s * (1.0 + f / 8.0) * np.exp2(e - 7.0)
    sub = s * f * 2.0 ** -9
    out = np.where(e == 0, sub, normal)
    return np.where((e == 15) & (f == 7), np.nan, out)


def decode_e2m1(codes) -> np.ndarray:
    """Value of 4-bit E2M1 codes (1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit;
    exponent 0 is subnormal: m * 0.5; no infinities or NaN), the element format of OCP MXFP4.

    The pages run the indexer in FP4 ([P1] section 2, footnote 3; section 4.2: FP4 dot
    products; [P2] 'Where It Breaks': the FP4 QK indexer); the format is the published
    OCP microscaling definition.
    """
    c = np.asarray(codes, dtype=np.int64) & 0xF
    sgn = np.where(c >> 3, -1.0, 1.0)
    e = (c >> 1) & 0x3
    mbit = c & 0x1
    val = np.where(e == 0, mbit * 0.5, (1.0 + mbit / 2.0) * np.exp2(e - 1.0))
    return sgn * val


def decode_e8m0(codes) -> np.ndarray:
    """Value of 8-bit E8M0 scale codes: 2^(e - 127); e = 255 is NaN (OCP microscaling
    shared-scale format)."""
    e = np.asarray(codes, dtype=np.int64)
    return np.where(e == 255, np.nan, np.exp2(e - 127.0))


def decode_mxfp4_rows(packed, scales) -> np.ndarray:
    """MXFP4 rows to fp64: ``packed`` uint8 [E, C/2] holds element 2j in the low nibble and
    element 2j+1 in the high nibble of byte j; ``scales`` uint8 [E, C/32] holds one E8M0 scale
    per block of 32 consecutive elements. value = e2m1(code) * 2^(e - 127)."""
    pk = np.asarray(packed, dtype=np.uint8)
    E, half = pk.shape
    codes = np.empty((E, 2 * half), dtype=np.uint8)
    codes[:, 0::2] = pk & 0xF
    codes[:, 1::2] = pk >> 4
    sc = decode_e8m0(np.asarray(scales, dtype=np.uint8))          # [E, C/32]
    return decode_e2m1(codes) * np.repeat(sc, 32, axis=1)


def to_bf16_f64(x) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 (8 significant bits, ties to even), as fp64.

    Used only to model the bf16 cache format of compressed entries when the oracle's own
    compressed rows feed its attention step.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    fin = np.isfinite(x)
    xf = x[fin]
    mant, ex = np.frexp(xf)              # xf = mant * 2^ex, 0.5 <= |mant| < 1
    # normal bf16 numbers carry 8 significant bits; below 2^-126 the quantum is 2^-133
    q_ex = np.maximum(ex - 8, -133)
    r = np.rint(np.ldexp(xf, -q_ex))    # rint rounds half to even
    y = np.ldexp(r, q_ex)
    y[np.abs(y) > 3.3895313892515355e38] = np.inf * np.sign(y[np.abs(y) > 3.3895313892515355e38])
    out[fin] = y
    out[~fin] = x[~fin]
    return out


# ----------------------------------------------------------------------------- geometry

def n_visible(p: int, m: int, n_entries: int) -> int:
    """Compressed entries a query at absolute position p may see: s < floor(p/m), capped by
    the entries that exist. A query never sees the block it falls in ([P1] section 6.1)."""
    return max(0, min(p // m, n_entries))


def window_rows(p: int, n_rows: int, W: int) -> range:
    """The W newest raw rows j with j <= p and j < n_rows ([P1] section 6; [P2] 'KV Cache
    Management': the window lives uncompressed in the state cache)."""
    if W <= 0 or n_rows <= 0:
        return range(0, 0)
    hi = min(p, n_rows - 1)
    lo = max(0, hi - W + 1)
    return range(lo, hi + 1)


# ----------------------------------------------------------------------------- a1 compress

def compress_entry(kv_rows, z_rows=None) -> np.ndarray:
    """One compressed entry from the m raw rows of its chunk.

    C[d] = sum_r w_r[d] * kv[r, d] with w[:, d] = softmax over the chunk rows of z[:, d].
    [P3] section 3 (compressed KV entry: per-dimension weights S_r from a softmax of Z,
    applied elementwise to the content rows and summed); [P2] 'Deep Dive', CSA step 2 and
    HCA 'How it works' (every m tokens become one entry by a softmax-weighted sum).
    """
    kv = np.asarray(kv_rows, dtype=np.float64)
    m = kv.shape[0]
    if z_rows is None:
        w = np.full(kv.shape, 1.0 / m)
    else:
        z = np.asarray(z_rows, dtype=np.float64)
        mu = z.max(axis=0, keepdims=True)
        e = np.exp(z - mu)
        w = e / e.sum(axis=0, keepdims=True)
    return (w * kv).sum(axis=0)


def compress(kv, z, m: int, entries=None) -> np.ndarray:
    """Compressed entries of one sequence: entry i pools raw rows [m*i, m*i + m).

    Trailing rows (N mod m) stay uncompressed ([P2] 'KV Cache Management': the tail lives
    in the state cache). ``entries`` restricts the output to the listed entry ids.
    """
    kv = np.asarray(kv, dtype=np.float64)
    n_ent = kv.shape[0] // m
    ids = np.arange(n_ent) if entries is None else np.asarray(entries, dtype=np.int64)
    D = kv.shape[1]
    rows = (ids[:, None] * m + np.arange(m)[None, :])          # [E, m] raw row ids
    kc = kv[rows]                                              # [E, m, D]
    if z is None:
        w = np.full(kc.shape, 1.0 / m)
    else:
        zc = np.asarray(z, dtype=np.float64)[rows]
        mu = zc.max(axis=1, keepdims=True)                     # softmax over the m rows
        e = np.exp(zc - mu)
        w = e / e.sum(axis=1, keepdims=True)
    out = (w * kc).sum(axis=1)
    return out.reshape(len(ids), D)


def compress_overlap(kv_a, z_a, kv_b, z_b, m: int, entries=None) -> np.ndarray:
    """Compressed entries of one CSA sequence from two overlapping series a and b.

    Entry i pools 2m rows under one softmax per dimension: rows [m*i, m*i + m) of series a
    and rows [m*(i-1), m*i) of series b, the block before it ([P2] 'Deep Dive', CSA
    dual-series KV compression; [P1] section 4.3, overlap compression: the b block is
    shared with the neighbouring entry). Entry 0 has no preceding block; its softmax runs
    over its m series-a rows alone (reading: the b range is empty there). With z_a and
    z_b both None the weights are uniform over the rows pooled. Both series have the same
    row count N; entries i < floor(N/m) exist, so the last b block is never pooled.
    """
    kv_a = np.asarray(kv_a, dtype=np.float64)
    kv_b = np.asarray(kv_b, dtype=np.float64)
    assert kv_a.shape == kv_b.shape
    assert (z_a is None) == (z_b is None)
    n_ent = kv_a.shape[0] // m
    ids = np.arange(n_ent) if entries is None else np.asarray(entries, dtype=np.int64)
    has_b = ids > 0                                            # [E]
    rows_a = ids[:, None] * m + np.arange(m)[None, :]          # [E, m]
    rows_b = np.where(has_b[:, None], rows_a - m, 0)           # [E, m]; a dummy row when absent
    x = np.concatenate([kv_a[rows_a], kv_b[rows_b]], axis=1)   # [E, 2m, D]
    if z_a is None:
        logits = np.zeros(x.shape)
    else:
        logits = np.concatenate([np.asarray(z_a, dtype=np.float64)[rows_a],
                                 np.asarray(z_b, dtype=np.float64)[rows_b]], axis=1)
    # an absent b block takes no weight
    logits[:, m:, :] = np.where(has_b[:, None, None], logits[:, m:, :], -np.inf)
    mu = logits.max(axis=1, keepdims=True)                     # one softmax over all 2m rows
    e = np.exp(logits - mu)
    w = e / e.sum(axis=1, keepdims=True)
    return (w * x).sum(axis=1).reshape(len(ids), kv_a.shape[1])


# ----------------------------------------------------------------------------- a2 indexer

def indexer(q_idx, w, keys) -> np.ndarray:
    """Lightning-indexer scores I(t, s) = sum_j w_j * ReLU(q_j . k_s) for every key row s.

    [P5] (Lightning Indexer score: per-head dot product, ReLU, learned head weights summed);
    [P2] 'Deep Dive', CSA: the indexer scores compressed indexer keys K^IComp with
    per-head queries q^I and head weights. No 1/sqrt(d) scale appears in the score.
    """
    q = np.asarray(q_idx, dtype=np.float64)     # [HI, CI]
    wt = np.asarray(w, dtype=np.float64)        # [HI]
    k = np.asarray(keys, dtype=np.float64)      # [n, CI]
    acc = np.zeros(k.shape[0])
    for j in range(q.shape[0]):
        acc += wt[j] * np.maximum(k @ q[j], 0.0)
    return acc


# ----------------------------------------------------------------------------- a3 top-k

def topk(scores, k: int) -> np.ndarray:
    """Ids of the k highest scores, ties to the lower id, returned ascending, -1 padded.

    [P2] 'Deep Dive', CSA: only the top-k scoring compressed blocks reach core attention.
    Comparisons use the scores as given (-0.0 equals +0.0); NaN is not allowed.
    """
    s = np.asarray(scores)
    assert not np.isnan(s).any(), "NaN scores are outside the contract"
    n = s.shape[0]
    keep = min(k, n)
    order = np.lexsort((np.arange(n), -s))     # primary: score descending, then id ascending
    out = np.full(k, -1, dtype=np.int64)
    out[:keep] = np.sort(order[:keep])
    return out


# ----------------------------------------------------------------------------- a4/a5 attention

def attend(q, X, scale: float, sink=None):
    """Shared-KV multi-query attention of H query heads over key=value rows X.

    o_h = sum_x softmax_x(scale * q_h . x) * x and lse_h = log sum_x exp(scale * q_h . x).
    [P5] (Attention(Q,K,V) = softmax(Q K^T / sqrt(d_k)) V); [P2] 'Deep Dive', CSA core
    attention: every head reads the same entries, which act as both keys and values.

    ``sink`` (per-head logits z'_h, [H]) adds exp(z'_h) to head h's softmax denominator
    ([P1] section 7, the attention sink: the weights may then sum to less than one). The
    sink carries no value, and lse_h = log(exp(z'_h) + sum_x exp(scale * q_h . x)).
    """
    q = np.asarray(q, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64).reshape(-1, q.shape[1])
    H, D = q.shape
    zs = np.full(H, -np.inf) if sink is None else np.asarray(sink, dtype=np.float64).reshape(H)
    o = np.zeros((H, D))
    lse = zs.copy()                       # no key: the denominator is the sink alone
    if X.shape[0] == 0:
        return o, lse
    for h in range(H):
        logit = (X @ q[h]) * scale
        mu = max(logit.max(), zs[h])
        e = np.exp(logit - mu)
        den = e.sum() + np.exp(zs[h] - mu)
        o[h] = (e @ X) / den
        lse[h] = mu + np.log(den)
    return o, lse


def rope(x, pos: float, R: int, base: float) -> np.ndarray:
    """Rotary position encoding of the last R dimensions of x (any leading shape) at
    position ``pos``; the other dimensions pass through.

    [P1] section 8 (partial RoPE: only the last 64 dimensions of queries and KV vectors are
    rotated; the attention output is rotated at the negated query position). The rotation
    itself is the original RoPE: inside the last R dims, pair j = (x[2j], x[2j+1]) turns by
    the angle pos * base^(-2j/R), counter-clockwise.
    """
    x = np.array(x, dtype=np.float64)
    if R == 0:
        return x
    D = x.shape[-1]
    j = np.arange(R // 2)
    ang = float(pos) * np.power(float(base), -2.0 * j / R)
    c, s_ = np.cos(ang), np.sin(ang)
    a = x[..., D - R::2].copy()
    b = x[..., D - R + 1::2].copy()
    x[..., D - R::2] = a * c - b * s_
    x[..., D - R + 1::2] = a * s_ + b * c
    return x


def attend_at(q, X, scale: float, p: int, sink=None, rope_dims: int = 0, rope_base: float = 10000.0):
    """attend() for a query at absolute position p with the per-query extras of the core
    attention: the query's last rope_dims dims rotated at p before the scores, the output's
    rotated back at -p ([P1] section 8, inverse RoPE on the output), and the sink. Key rows
    enter as given (their own rotation, if any, is applied where they are written)."""
    qr = rope(q, p, rope_dims, rope_base)
    o, lse = attend(qr, X, scale, sink)
    return rope(o, -p, rope_dims, rope_base), lse


def sparse_attn(q, ckv_b, kv_b, idx, p: int, W: int, scale: float, sink=None, rope_dims: int = 0,
                rope_base: float = 10000.0):
    """CSA core attention for one query row: the selected compressed entries (ids >= 0)
    plus the raw window rows, under one softmax ([P2] 'Putting It Together': MQA over the
    top-k entries plus 128 sliding-window entries)."""
    ckv_b = np.asarray(ckv_b, dtype=np.float64)
    kv_b = np.asarray(kv_b, dtype=np.float64)
    sel = [int(i) for i in np.asarray(idx).ravel() if i >= 0]
    assert all(i < ckv_b.shape[0] for i in sel), "selected id beyond the sequence's entries"
    rows = [ckv_b[i] for i in sel] + [kv_b[j] for j in window_rows(p, kv_b.shape[0], W)]
    X = np.array(rows).reshape(len(rows), np.asarray(q).shape[1])
    return attend_at(q, X, scale, p, sink, rope_dims, rope_base)


def hca_attn(q, ckv_b, kv_b, p: int, m: int, W: int, scale: float, sink=None, rope_dims: int = 0,
             rope_base: float = 10000.0):
    """HCA attention for one query row: every visible compressed entry plus the raw window
    rows, under one softmax ([P1] section 5.1; [P2] 'Heavily Compressed Attention')."""
    ckv_b = np.asarray(ckv_b, dtype=np.float64)
    kv_b = np.asarray(kv_b, dtype=np.float64)
    nv = n_visible(p, m, ckv_b.shape[0])
    rows = [ckv_b[s] for s in range(nv)] + [kv_b[j] for j in window_rows(p, kv_b.shape[0], W)]
    X = np.array(rows).reshape(len(rows), np.asarray(q).shape[1])
    return attend_at(q, X, scale, p, sink, rope_dims, rope_base)
