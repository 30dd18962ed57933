"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics (CPU only).

Each test names what pins it: the worked example printed on a page, a closed form, an
invariant, a special case that reduces to a library routine, or brute force on tiny inputs.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

from oracle import csa, pipeline

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(s):
    return np.random.default_rng(1000 + s)


# ------------------------------------------------------------------------------ compress

def _load_p3():
    rows = {}
    with open(os.path.join(GOLDEN, "p3_compress_example.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, *v = line.split()
            rows[k] = [float(x) for x in v]
    C = np.array([rows[f"C{i}"] for i in range(4)])
    S = np.array([rows[f"S{i}"] for i in range(4)])
    return C, S, np.array(rows["expected"])


def test_compress_p3_worked_example():
    """[P3] section 3 toy chunk: weights S (columns sum to 1) pool C0..C3 into [0.7, 0.6, 0.6]."""
    C, S, expected = _load_p3()
    np.testing.assert_allclose(S.sum(axis=0), 1.0, rtol=0, atol=1e-15)
    got = csa.compress(C, np.log(S), 4)
    np.testing.assert_allclose(got[0], expected, rtol=0, atol=1e-14)
    np.testing.assert_allclose(csa.compress_entry(C, np.log(S)), expected, rtol=0, atol=1e-14)


def test_compress_softmax_axis_is_chunk_rows():
    """The same page's rows S_r do not sum to 1 across dimensions (S0 sums to 0.9): a softmax
    over the dimension axis would not reproduce S, so the example fixes the axis."""
    C, S, expected = _load_p3()
    assert abs(S[0].sum() - 0.9) < 1e-12
    wrong = (np.exp(np.log(S)) / np.exp(np.log(S)).sum(axis=1, keepdims=True) * C).sum(axis=0)
    assert np.abs(wrong - expected).max() > 0.05


def test_compress_m1_is_identity():
    r = _rng(1)
    kv, z = r.standard_normal((37, 8)), r.standard_normal((37, 8))
    np.testing.assert_array_equal(csa.compress(kv, z, 1), kv)


def test_compress_uniform_weights_give_mean():
    r = _rng(2)
    kv = r.standard_normal((4 * 9 + 3, 5))
    ref = kv[:36].reshape(9, 4, 5).mean(axis=1)
    np.testing.assert_allclose(csa.compress(kv, None, 4), ref, rtol=1e-15, atol=1e-15)
    const = np.tile(r.standard_normal((9, 1, 5)), (1, 4, 1)).reshape(36, 5)
    const = np.concatenate([const, np.zeros((3, 5))])
    np.testing.assert_allclose(csa.compress(kv, const, 4), ref, rtol=1e-13, atol=1e-14)


def test_compress_dominant_row_selects_it():
    r = _rng(3)
    m, E, D = 8, 5, 6
    kv = r.standard_normal((m * E, D))
    z = np.zeros((m * E, D))
    pick = r.integers(0, m, size=(E, D))
    for i in range(E):
        for d in range(D):
            z[i * m + pick[i, d], d] = 800.0   # would overflow exp() without the max shift
    got = csa.compress(kv, z, m)
    for i in range(E):
        for d in range(D):
            assert got[i, d] == kv[i * m + pick[i, d], d]


def test_compress_brute_force_tiny():
    """Pure-Python evaluation of sum_r exp(z_r)/sum exp(z) * kv_r on small chunks."""
    r = _rng(4)
    for m in (1, 2, 3, 4, 7):
        N, D = m * 5 + (m - 1), 3
        kv, z = r.standard_normal((N, D)), r.standard_normal((N, D)) * 3
        got = csa.compress(kv, z, m)
        assert got.shape == (N // m, D)
        for i in range(N // m):
            for d in range(D):
                zs = [z[i * m + j, d] for j in range(m)]
                den = sum(math.exp(v) for v in zs)
                ref = sum(math.exp(zs[j]) / den * kv[i * m + j, d] for j in range(m))
                assert abs(got[i, d] - ref) < 1e-12


def test_compress_within_chunk_permutation_and_bounds():
    r = _rng(5)
    m, E, D = 4, 30, 16
    kv, z = r.standard_normal((m * E, D)), r.standard_normal((m * E, D))
    base = csa.compress(kv, z, m)
    perm = np.concatenate([i * m + r.permutation(m) for i in range(E)])
    np.testing.assert_allclose(csa.compress(kv[perm], z[perm], m), base, rtol=1e-13, atol=1e-14)
    lo = kv.reshape(E, m, D).min(axis=1)
    hi = kv.reshape(E, m, D).max(axis=1)
    assert np.all(base >= lo - 1e-12) and np.all(base <= hi + 1e-12)
    sub = csa.compress(kv, z, m, entries=[3, 17, 0])
    np.testing.assert_array_equal(sub, base[[3, 17, 0]])


# ------------------------------------------------------------------- overlapped compression

def _two_series(seed, m, E, D, tail=0, zscale=1.0):
    r = _rng(seed)
    N = m * E + tail
    return (r.standard_normal((N, D)), r.standard_normal((N, D)) * zscale,
            r.standard_normal((N, D)), r.standard_normal((N, D)) * zscale)


def test_overlap_p3_chunk_beside_a_constant_block():
    """[P3] section 3 toy chunk as the series-a block of entry 1, beside a series-b block of
    four equal rows V. With z_a = ln(S/2) and z_b = ln(1/8) every column of the joint
    weights sums to one, so the joint softmax reproduces S/2 and 1/8 exactly and the entry
    is the midpoint of the page's result and V. Dropping either series, or normalising
    the two blocks separately, misses it."""
    C, S, expected = _load_p3()
    V = np.array([2.0, 4.0, 6.0])
    kv_a = np.concatenate([np.zeros((4, 3)), C])
    z_a = np.concatenate([np.zeros((4, 3)), np.log(S / 2)])
    kv_b = np.concatenate([np.tile(V, (4, 1)), np.zeros((4, 3))])
    z_b = np.concatenate([np.full((4, 3), np.log(1 / 8)), np.zeros((4, 3))])
    got = csa.compress_overlap(kv_a, z_a, kv_b, z_b, 4)
    np.testing.assert_allclose(got[1], (expected + V) / 2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(got[1], [1.35, 2.3, 3.3], rtol=0, atol=1e-14)


def test_overlap_entry0_pools_series_a_only():
    """Entry 0 has no earlier block: it equals single-series compression of its a rows,
    whatever series b holds."""
    kv_a, z_a, kv_b, z_b = _two_series(10, 4, 6, 8)
    got = csa.compress_overlap(kv_a, z_a, kv_b, z_b, 4)
    np.testing.assert_allclose(got[0], csa.compress(kv_a, z_a, 4)[0], rtol=1e-14, atol=1e-14)
    got2 = csa.compress_overlap(kv_a, z_a, kv_b * 5 + 1, z_b - 3, 4)
    np.testing.assert_array_equal(got2[0], got[0])


def test_overlap_series_b_absent_reduces_to_single_series():
    """Logits of -inf on series b remove it: every entry is single-series compression of a."""
    kv_a, z_a, kv_b, _ = _two_series(11, 4, 9, 5, tail=3)
    got = csa.compress_overlap(kv_a, z_a, kv_b, np.full(kv_b.shape, -np.inf), 4)
    np.testing.assert_allclose(got, csa.compress(kv_a, z_a, 4), rtol=1e-14, atol=1e-14)


def test_overlap_block_reach():
    """Series-a block j feeds entry j only; series-b block j feeds entry j+1 only, and the
    last b block feeds nothing ([P2] 'Deep Dive': C^b covers [m(i-1), mi-1] for entry i)."""
    m, E, D = 4, 7, 3
    kv_a, z_a, kv_b, z_b = _two_series(12, m, E, D)
    base = csa.compress_overlap(kv_a, z_a, kv_b, z_b, m)
    for j in range(E):
        for which in ("a", "b"):
            ka, kb = kv_a.copy(), kv_b.copy()
            (ka if which == "a" else kb)[j * m:(j + 1) * m] += 10.0
            got = csa.compress_overlap(ka, z_a, kb, z_b, m)
            changed = set(np.nonzero(np.abs(got - base).max(axis=1) > 1e-9)[0].tolist())
            want = {j} if which == "a" else ({j + 1} if j + 1 < E else set())
            assert changed == want, (which, j, changed)


def test_overlap_uniform_weights_give_mean():
    """No logits (or equal logits): entry i > 0 is the mean of its 2m rows, entry 0 the
    mean of its m series-a rows."""
    m, E, D = 4, 6, 5
    kv_a, _, kv_b, _ = _two_series(13, m, E, D, tail=2)
    ref = np.empty((E, D))
    ref[0] = kv_a[:m].mean(axis=0)
    for i in range(1, E):
        ref[i] = np.concatenate([kv_a[i * m:(i + 1) * m], kv_b[(i - 1) * m:i * m]]).mean(axis=0)
    np.testing.assert_allclose(csa.compress_overlap(kv_a, None, kv_b, None, m), ref, rtol=1e-14, atol=1e-14)
    zc = np.full(kv_a.shape, 0.37)
    np.testing.assert_allclose(csa.compress_overlap(kv_a, zc, kv_b, zc, m), ref, rtol=1e-13, atol=1e-14)


def test_overlap_brute_force_tiny():
    """Pure-Python joint softmax over the 2m (or m) rows of each entry."""
    for m in (1, 2, 3, 4, 5):
        E, D = 5, 3
        kv_a, z_a, kv_b, z_b = _two_series(14 + m, m, E, D, tail=m - 1, zscale=3.0)
        got = csa.compress_overlap(kv_a, z_a, kv_b, z_b, m)
        assert got.shape == (E, D)
        for i in range(E):
            for d in range(D):
                pool = [(z_a[i * m + j, d], kv_a[i * m + j, d]) for j in range(m)]
                if i > 0:
                    pool += [(z_b[(i - 1) * m + j, d], kv_b[(i - 1) * m + j, d]) for j in range(m)]
                den = sum(math.exp(zz) for zz, _ in pool)
                ref = sum(math.exp(zz) / den * v for zz, v in pool)
                assert abs(got[i, d] - ref) < 1e-12


def test_overlap_is_single_series_over_spliced_chunks():
    """Splicing each entry's b block and a block into one 2m-row chunk of a new sequence
    turns the dual series into single-series compression with ratio 2m; the bounds of a
    convex combination hold too."""
    m, E, D = 4, 8, 6
    kv_a, z_a, kv_b, z_b = _two_series(20, m, E, D)
    got = csa.compress_overlap(kv_a, z_a, kv_b, z_b, m)
    kv_s = np.concatenate([np.concatenate([kv_b[(i - 1) * m:i * m], kv_a[i * m:(i + 1) * m]]) for i in range(1, E)])
    z_s = np.concatenate([np.concatenate([z_b[(i - 1) * m:i * m], z_a[i * m:(i + 1) * m]]) for i in range(1, E)])
    np.testing.assert_allclose(got[1:], csa.compress(kv_s, z_s, 2 * m), rtol=1e-13, atol=1e-14)
    lo = kv_s.reshape(E - 1, 2 * m, D).min(axis=1)
    hi = kv_s.reshape(E - 1, 2 * m, D).max(axis=1)
    assert np.all(got[1:] >= lo - 1e-12) and np.all(got[1:] <= hi + 1e-12)
    sub = csa.compress_overlap(kv_a, z_a, kv_b, z_b, m, entries=[5, 0, 2])
    np.testing.assert_array_equal(sub, got[[5, 0, 2]])


def test_overlap_lane_is_per_sequence():
    """The packed driver restarts the block count at every sequence: each sequence's entry 0
    sees no b rows of the sequence before it."""
    r = _rng(21)
    lens = [9, 3, 17, 8]
    off = np.concatenate([[0], np.cumsum(lens)])
    N = off[-1]
    kv_a, z_a, kv_b, z_b = (r.standard_normal((N, 4)) for _ in range(4))
    got = pipeline.compress_overlap_lane(kv_a, z_a, kv_b, z_b, off, 4)
    ref = np.concatenate([csa.compress_overlap(kv_a[lo:hi], z_a[lo:hi], kv_b[lo:hi], z_b[lo:hi], 4)
                          for lo, hi in zip(off[:-1], off[1:])])
    assert got.shape == (sum(n // 4 for n in lens), 4)
    np.testing.assert_array_equal(got, ref)


# ------------------------------------------------------------------------------ fp8 / bf16

def test_e4m3_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = csa.decode_e4m3(codes)
    np.testing.assert_array_equal(got, ref)
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x38] == 1.0
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and got[0x80] == 0.0


def test_e2m1_decode_table_and_e4m3_reencoding():
    """The 16 E2M1 codes give +-{0, 0.5, 1, 1.5, 2, 3, 4, 6} (OCP MXFP4 element table), and
    each equals the E4M3 value of the same sign, exponent (rebiased 1 -> 7) and mantissa
    bit, decoded by the torch-pinned E4M3 path."""
    got = csa.decode_e2m1(np.arange(16))
    np.testing.assert_array_equal(got[:8], [0, 0.5, 1, 1.5, 2, 3, 4, 6])
    np.testing.assert_array_equal(got[8:], -got[:8])
    for c in range(16):
        sgn, e, mb = c >> 3, (c >> 1) & 3, c & 1
        if e == 0:
            ref = (-1) ** sgn * mb * 0.5
        else:
            e4 = (sgn << 7) | ((e - 1 + 7) << 3) | (mb << 2)
            ref = csa.decode_e4m3(np.array([e4], dtype=np.uint8))[0]
        assert got[c] == ref, c


def test_e8m0_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = csa.decode_e8m0(codes)
    np.testing.assert_array_equal(got[:255], ref[:255])
    assert np.isnan(got[255]) and np.isnan(ref[255]) and got[127] == 1.0


def test_mxfp4_rows_elementwise():
    """Packed rows decode element by element: element i comes from nibble i % 2 of byte
    i // 2 and is scaled by block i // 32's E8M0 scale."""
    r = _rng(40)
    pk = r.integers(0, 256, size=(5, 32)).astype(np.uint8)
    sc = r.integers(100, 150, size=(5, 2)).astype(np.uint8)
    got = csa.decode_mxfp4_rows(pk, sc)
    table = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    for e in range(5):
        for i in range(64):
            code = (int(pk[e, i // 2]) >> (4 * (i % 2))) & 0xF
            v = (-1 if code & 8 else 1) * table[code & 7] * 2.0 ** (int(sc[e, i // 32]) - 127)
            assert got[e, i] == v


def test_bf16_rounding_matches_torch_on_fp32_values():
    r = _rng(6)
    x = (r.standard_normal(20000) * np.exp2(r.integers(-30, 30, 20000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(csa.to_bf16_f64(x.astype(np.float64)), ref)
    # ties go to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    assert csa.to_bf16_f64(np.array([1 + 2 ** -8]))[0] == 1.0
    assert csa.to_bf16_f64(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6
    # an fp64 value just above a tie must round up (fp32 double rounding would not)
    assert csa.to_bf16_f64(np.array([1 + 2 ** -8 + 2 ** -40]))[0] == 1 + 2 ** -7


# ------------------------------------------------------------------------------ indexer

def test_indexer_hand_example():
    """I = sum_j w_j ReLU(q_j . k): q0=[1,0], q1=[0,1], w=[1,3]."""
    q = np.array([[1.0, 0.0], [0.0, 1.0]])
    w = np.array([1.0, 3.0])
    keys = np.array([[2.0, -1.0], [-1.0, 2.0], [-1.0, -1.0], [0.5, 0.5]])
    np.testing.assert_array_equal(csa.indexer(q, w, keys), [2.0, 6.0, 0.0, 2.0])


def test_indexer_single_head_is_relu_of_matmul():
    r = _rng(7)
    q, keys = r.standard_normal((1, 64)), r.standard_normal((500, 64))
    np.testing.assert_allclose(csa.indexer(q, [1.0], keys), np.maximum(np.matmul(keys, q[0]), 0),
                               rtol=1e-14, atol=1e-14)


def test_indexer_nonnegative_linear_and_homogeneous():
    r = _rng(8)
    q, keys = r.standard_normal((8, 64)) / 8, r.standard_normal((300, 64)) / 8
    w1, w2 = r.random(8), r.random(8)
    s1, s2 = csa.indexer(q, w1, keys), csa.indexer(q, w2, keys)
    assert np.all(s1 >= 0) and np.all(s2 >= 0)
    np.testing.assert_allclose(csa.indexer(q, w1 + 2 * w2, keys), s1 + 2 * s2, rtol=1e-12, atol=1e-15)
    # ReLU(c x) = c ReLU(x) for c > 0: a per-key scale factors out of the score
    np.testing.assert_allclose(csa.indexer(q, w1, keys * 0.37), 0.37 * s1, rtol=1e-12, atol=1e-15)
    # flipping every query flips which side of zero each dot falls on
    s_neg = csa.indexer(-q, w1, keys)
    both = csa.indexer(q, w1, keys) + s_neg
    dots = np.abs(keys @ q.T) @ w1
    np.testing.assert_allclose(both, dots, rtol=1e-12, atol=1e-15)


def test_indexer_brute_force_tiny():
    r = _rng(9)
    q, w, keys = r.standard_normal((3, 5)), r.random(3), r.standard_normal((7, 5))
    got = csa.indexer(q, w, keys)
    for s in range(7):
        ref = 0.0
        for j in range(3):
            dot = sum(q[j, d] * keys[s, d] for d in range(5))
            ref += w[j] * (dot if dot > 0 else 0.0)
        assert abs(got[s] - ref) < 1e-13


# ------------------------------------------------------------------------------ top-k

def _brute_topk(s, k):
    order = sorted(range(len(s)), key=lambda i: (-float(s[i]), i))
    sel = sorted(order[:min(k, len(s))])
    return sel + [-1] * (k - len(sel))


@pytest.mark.parametrize("levels", [0, 3, 20])
def test_topk_brute_force(levels):
    r = _rng(10 + levels)
    for n in (1, 5, 33, 200):
        for k in (1, 4, 32, 250):
            s = r.standard_normal(n).astype(np.float32) if levels == 0 else \
                r.integers(0, levels, n).astype(np.float32)
            assert list(csa.topk(s, k)) == _brute_topk(s, k)


def test_topk_ties_padding_and_signed_zero():
    assert list(csa.topk(np.ones(10, np.float32), 4)) == [0, 1, 2, 3]
    assert list(csa.topk(np.array([5.0, 1.0, 7.0]), 5)) == [0, 1, 2, -1, -1]
    assert list(csa.topk(np.array([-0.0, 0.0, -0.0, 0.0]), 2)) == [0, 1]
    assert list(csa.topk(np.zeros(0), 3)) == [-1, -1, -1]


def test_topk_permutation_moves_only_ids():
    r = _rng(11)
    s = r.standard_normal(1000)
    perm = r.permutation(1000)
    a = set(csa.topk(s, 50).tolist())
    b = set(perm[csa.topk(s[perm], 50)].tolist())
    assert a == b


# ------------------------------------------------------------------------------ attention

def _sdpa(q, X, scale):
    qt = torch.from_numpy(q)[None, :, None, :]             # [1, H, 1, D]
    kt = torch.from_numpy(X)[None, None].expand(1, q.shape[0], -1, -1)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=scale)
    return out[0, :, 0, :].numpy()


def test_attend_matches_sdpa_and_logsumexp():
    from scipy.special import logsumexp
    r = _rng(12)
    q, X = r.standard_normal((16, 32)), r.standard_normal((50, 32))
    sc = 1 / math.sqrt(32)
    o, lse = csa.attend(q, X, sc)
    np.testing.assert_allclose(o, _sdpa(q, X, sc), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, logsumexp((q @ X.T) * sc, axis=1), rtol=1e-13)


def test_attend_single_key_and_empty_set():
    r = _rng(13)
    q, x = r.standard_normal((4, 8)), r.standard_normal((1, 8))
    o, lse = csa.attend(q, x, 0.5)
    np.testing.assert_allclose(o, np.repeat(x, 4, axis=0), rtol=1e-15)
    np.testing.assert_allclose(lse, 0.5 * (q @ x[0]), rtol=1e-14)
    o, lse = csa.attend(q, np.zeros((0, 8)), 0.5)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_attend_split_merge_invariant():
    """Attention over a union equals the LSE-weighted merge of attention over its parts."""
    r = _rng(14)
    q, X = r.standard_normal((8, 16)), r.standard_normal((90, 16))
    o, lse = csa.attend(q, X, 0.25)
    parts = [csa.attend(q, X[a:b], 0.25) for a, b in ((0, 13), (13, 60), (60, 90))]
    L = np.logaddexp.reduce(np.stack([p[1] for p in parts]), axis=0)
    merged = sum(np.exp(p[1] - L)[:, None] * p[0] for p in parts)
    np.testing.assert_allclose(merged, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(L, lse, rtol=1e-13)


def test_sparse_attn_window_only_and_hca_equals_full_selection():
    r = _rng(15)
    N, D, H, m, W = 300, 16, 4, 4, 32
    kv, z, q = r.standard_normal((N, D)), r.standard_normal((N, D)), r.standard_normal((H, D))
    ckv = csa.compress(kv, z, m)
    p = N
    o0, l0 = csa.sparse_attn(q, ckv, kv, np.full(8, -1), p, W, 0.25)
    ow, lw = csa.attend(q, kv[N - W:N], 0.25)
    np.testing.assert_allclose(o0, ow, rtol=1e-14)
    nv = csa.n_visible(p, m, ckv.shape[0])
    oh, lh = csa.hca_attn(q, ckv, kv, p, m, W, 0.25)
    os_, ls = csa.sparse_attn(q, ckv, kv, np.arange(nv), p, W, 0.25)
    np.testing.assert_allclose(oh, os_, rtol=1e-14)
    np.testing.assert_allclose(lh, ls, rtol=1e-14)


# ----------------------------------------------------------------- attention sink and RoPE

def test_sink_is_a_zero_value_key_in_sdpa():
    """[P1] section 7: the sink adds exp(z'_h) to head h's denominator and carries nothing.
    Per head, that is a library attention with separate keys and values over X plus one
    extra key whose logit is z'_h and whose value row is zero."""
    r = _rng(30)
    H, D, n = 6, 16, 40
    q, X = r.standard_normal((H, D)), r.standard_normal((n, D))
    z = np.array([-3.0, 0.0, 1.5, 4.0, 9.0, -np.inf])
    sc = 0.3
    o, lse = csa.attend(q, X, sc, sink=z)
    for h in range(H):
        if np.isfinite(z[h]):
            ks = q[h] * (z[h] / (sc * q[h] @ q[h]))          # sc * q_h . ks = z_h
            K = np.vstack([X, ks])
            V = np.vstack([X, np.zeros(D)])
        else:
            K, V = X, X
        qt = torch.from_numpy(q[h])[None, None, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, torch.from_numpy(K)[None, None], torch.from_numpy(V)[None, None], scale=sc)[0, 0, 0].numpy()
        np.testing.assert_allclose(o[h], ref, rtol=1e-12, atol=1e-13)


def test_sink_closed_form_and_limits():
    """out_sink = out * sigmoid(lse - z), lse_sink = logaddexp(lse, z); the weights then sum
    to 1 - exp(z - lse_sink) (read off with identity keys); no keys: out 0, lse z."""
    r = _rng(31)
    H, D = 5, 12
    q, X = r.standard_normal((H, D)), r.standard_normal((30, D))
    z = r.standard_normal(H) * 3
    o, lse = csa.attend(q, X, 0.4)
    os_, ls = csa.attend(q, X, 0.4, sink=z)
    np.testing.assert_allclose(os_, o / (1 + np.exp(z - lse))[:, None], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(ls, np.logaddexp(lse, z), rtol=1e-14)
    oi, li = csa.attend(q, np.eye(D), 0.4, sink=z)
    np.testing.assert_allclose(oi.sum(axis=1), 1 - np.exp(z - li), rtol=1e-13)
    oe, le = csa.attend(q, np.zeros((0, D)), 0.4, sink=z)
    assert np.all(oe == 0) and np.array_equal(le, z)
    on, ln = csa.attend(q, X, 0.4, sink=np.full(H, -np.inf))
    np.testing.assert_array_equal(on, o)
    np.testing.assert_array_equal(ln, lse)


def test_rope_textbook_values():
    """The first rotated pair turns by pos radians; pair j by pos * base^(-2j/R), so at
    pos = base^(2j/R) it turns by one radian; the dimensions before the last R pass."""
    D, R = 16, 8
    e = np.zeros(D)
    e[D - R] = 1.0                                   # pair 0, first component
    y = csa.rope(e, 0.7, R, 10000.0)
    np.testing.assert_allclose(y[D - R:D - R + 2], [math.cos(0.7), math.sin(0.7)], rtol=1e-15, atol=1e-16)
    e2 = np.zeros(D)
    e2[D - R + 5] = 1.0                              # pair 2, second component
    y2 = csa.rope(e2, 100.0, R, 10000.0)             # 10000^(-4/8) = 1/100: one radian
    np.testing.assert_allclose(y2[D - R + 4:D - R + 6], [-math.sin(1.0), math.cos(1.0)], rtol=1e-14, atol=1e-15)
    x = _rng(32).standard_normal((3, D))
    np.testing.assert_array_equal(csa.rope(x, 123.0, R, 10000.0)[:, :D - R], x[:, :D - R])
    np.testing.assert_array_equal(csa.rope(x, 123.0, 0, 10000.0), x)


def test_rope_is_complex_rotation_and_a_group():
    """Pairs as complex numbers are multiplied by exp(i * angle); rotations compose, p then
    -p is the identity, norms of pairs are kept, and q.k after rotating q at p and k at j
    depends on j - p only (the relative-position property)."""
    r = _rng(33)
    D, R, base = 128, 64, 10000.0
    x = r.standard_normal((4, D))
    y = csa.rope(x, 1048577.0, R, base)
    zc = x[:, D - R::2] + 1j * x[:, D - R + 1::2]
    ang = 1048577.0 * base ** (-np.arange(0, R, 2) / R)
    w = zc * np.exp(1j * ang)
    np.testing.assert_allclose(y[:, D - R::2], w.real, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y[:, D - R + 1::2], w.imag, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(csa.rope(csa.rope(x, 700.0, R, base), 300.0, R, base), csa.rope(x, 1000.0, R, base),
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(csa.rope(y, -1048577.0, R, base), x, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(np.hypot(y[:, D - R::2], y[:, D - R + 1::2]), np.abs(zc), rtol=1e-13)
    qv, kv = r.standard_normal(D), r.standard_normal(D)
    s1 = csa.rope(qv, 5000.0, R, base) @ csa.rope(kv, 4000.0, R, base)
    s2 = csa.rope(qv, 905000.0, R, base) @ csa.rope(kv, 904000.0, R, base)
    assert abs(s1 - s2) < 1e-9


def test_attend_at_inverse_rope_makes_positions_relative():
    """[P1] section 8: a value row stored rotated at its own position j, read by a query at p
    whose output is rotated at -p, comes out rotated at j - p. With one key the output is
    that key, so attend_at returns rope(v, j - p); with no rope and no sink it is attend."""
    r = _rng(34)
    H, D, R = 4, 32, 16
    q, v = r.standard_normal((H, D)), r.standard_normal(D)
    j, p = 777, 1000
    o, _ = csa.attend_at(q, csa.rope(v, j, R, 500.0)[None], 0.2, p, rope_dims=R, rope_base=500.0)
    np.testing.assert_allclose(o, np.tile(csa.rope(v, j - p, R, 500.0), (H, 1)), rtol=1e-11, atol=1e-12)
    X = r.standard_normal((20, D))
    a = csa.attend_at(q, X, 0.2, p)
    b = csa.attend(q, X, 0.2)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_m1_full_topk_no_window_reduces_to_dense_attention():
    """With m=1, k = every entry and no window, the whole CSA lane is dense
    softmax(Q K^T / sqrt(d)) V over the context (K = V)."""
    r = _rng(16)
    N, D, H, HI, CI = 96, 32, 8, 4, 16
    kv = torch.from_numpy(r.standard_normal((N, D))).to(torch.bfloat16)
    z = torch.from_numpy(r.standard_normal((N, D))).to(torch.bfloat16)
    q = torch.from_numpy(r.standard_normal((1, 1, H, D))).to(torch.bfloat16)
    qI = torch.from_numpy(r.standard_normal((1, 1, HI, CI)))
    w = torch.from_numpy(r.random((1, 1, HI)))
    keys = r.standard_normal((N, CI))
    sc = 1 / math.sqrt(D)
    ckv, scores, idx, o, lse = pipeline.csa_step(kv, z, q, qI, w, keys, [0, N], [N], 1, N, 0, sc)
    assert sorted(idx[0, 0].tolist()) == list(range(N))
    qf, kf = pipeline.f64(q)[0, 0], pipeline.f64(kv)
    np.testing.assert_allclose(o[0, 0], _sdpa(qf, kf, sc), rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------------------ geometry

def test_entry_counts_and_attended_set_size():
    assert [n // m for n, m in ((4096, 4), (131072, 128), (1 << 20, 4), (139264, 4))] == \
        [1024, 1024, 262144, 34816]
    N = 1 << 20
    win = csa.window_rows(N, N, 128)
    assert (win.start, win.stop) == (N - 128, N)
    assert 1024 + len(win) == 1152          # [P2] 'Putting It Together': ~1152 entries
    assert csa.n_visible(N, 4, N // 4) == 262144


def test_hca_plus_window_covers_every_prior_token():
    """[P1] section 6.2: with n_win = m', the window covers exactly the block HCA cannot see."""
    mp = 128
    for N in (mp * 3, mp * 3 + 1, mp * 7 + 77, 5000):
        for p in list(range(N - 300, N)) + [N]:
            if p < 0:
                continue
            nv = csa.n_visible(p, mp, N // mp)
            seen = set(range(nv * mp)) | set(csa.window_rows(p, N, mp))
            prior = set(range(min(p, N)))
            assert prior <= seen


def test_own_block_never_visible():
    for m in (4, 128):
        for p in range(0, 4 * m + 3):
            nv = csa.n_visible(p, m, 10 ** 6)
            assert nv * m <= p                # visible entries cover only rows < p
            assert p // m >= nv               # the block holding p is not visible


def test_window_clamps_at_context_start():
    assert list(csa.window_rows(5, 100, 128)) == list(range(0, 6))
    assert list(csa.window_rows(3, 3, 128)) == [0, 1, 2]
    assert list(csa.window_rows(0, 0, 128)) == []
    assert list(csa.window_rows(10, 20, 0)) == []


def test_topk_selection_size_is_k():
    r = _rng(17)
    for n in (10, 1000):
        for k in (5, 64, 2000):
            sel = csa.topk(r.random(n), k)
            assert (sel >= 0).sum() == min(k, n)
            good = sel[sel >= 0]
            assert np.all(np.diff(good) > 0)
