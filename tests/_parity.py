"""Comparison rules shared by the GPU parity tests (not a test module).

Tolerances (written out here and used by every GPU test):
  * compressed entries and indexer scores: per element |g - r| <= 1e-3 * max(|r|, rms(row)),
    where the row is one compressed entry's D values or one query row's visible scores;
    bf16 outputs additionally get the bf16 rounding step, 2^-8 * |r|.
  * top-k ids: bit-exact when both sides see the same fp32 scores; against fp64 oracle
    scores, ids may differ only among entries whose score lies within 1e-3 * tau of the
    oracle's k-th score tau.
  * attention outputs and lse: max |g - r| <= 2e-3.
"""
import numpy as np
import torch

REL = 1e-3
ATTN_ABS = 2e-3


def f64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def assert_rows_close(g, r, rel=REL, bf16=False, what=""):
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    if r.size == 0:
        return
    r2 = r.reshape(-1, r.shape[-1]) if r.ndim > 1 else r.reshape(1, -1)
    g2 = g.reshape(r2.shape)
    rms = np.sqrt(np.mean(r2 ** 2, axis=1, keepdims=True))
    tol = rel * np.maximum(np.abs(r2), rms)
    if bf16:
        tol = tol + 2.0 ** -8 * np.abs(r2)
    bad = np.abs(g2 - r2) > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} elements off, first at {tuple(i)}: gpu={g2[tuple(i)]!r} "
                             f"oracle={r2[tuple(i)]!r} tol={tol[tuple(i)]!r}")


def assert_attn_close(g, r, what="", atol=ATTN_ABS):
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    both_inf = np.isneginf(g) & np.isneginf(r)
    diff = np.where(both_inf, 0.0, np.abs(g - r))
    assert not np.isnan(diff).any(), f"{what}: NaN in comparison"
    m = diff.max() if diff.size else 0.0
    print(f"  {what}: max abs err {m:.3e} (bound {atol})", flush=True)
    assert m <= atol, f"{what}: max abs err {m:.3e} > {atol}"


def topk_band_check(gpu_ids, oracle_scores, k, rel=REL, what=""):
    """Top-k set from fp32 GPU scores against fp64 oracle scores (ties to lower id).

    Returns True when the two sets are identical, False when they differ only inside the
    boundary band; raises otherwise."""
    s = np.asarray(oracle_scores, dtype=np.float64)
    n = s.shape[0]
    ids = np.asarray(gpu_ids)
    keep = min(k, n)
    got = ids[ids >= 0]
    assert len(got) == keep and np.all(ids[keep:] == -1), f"{what}: wrong count/padding"
    assert np.all(np.diff(got) > 0), f"{what}: ids not strictly ascending"
    if keep == n:
        assert np.array_equal(got, np.arange(n)), what
        return True
    order = np.lexsort((np.arange(n), -s))
    ref = set(order[:keep].tolist())
    gs = set(got.tolist())
    if gs == ref:
        return True
    tau = s[order[keep - 1]]
    band = set(np.nonzero(np.abs(s - tau) <= rel * abs(tau))[0].tolist())
    assert gs - band == ref - band, f"{what}: sets differ outside the 1e-3 band"
    assert not any(s[i] < tau * (1 - rel) for i in gs), f"{what}: selected a score below the band"
    return False


def dev(t, device="cuda"):
    return None if t is None else t.to(device, non_blocking=False).contiguous()
