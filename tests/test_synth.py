"""The seeded input generators: determinism, chunk regeneration and workload shapes (CPU)."""
import numpy as np
import torch

import synth
from synth import workloads as W
from oracle import csa


def test_draws_are_deterministic_and_chunk_addressable():
    a = W.normal_bf16(7, W.S_KV, (3 * W.CHUNK // 128 + 50, 128))
    b = W.normal_bf16(7, W.S_KV, (3 * W.CHUNK // 128 + 50, 128))
    assert torch.equal(a, b)
    lo, hi = W.CHUNK // 128 - 5, 2 * W.CHUNK // 128 + 9   # straddles two chunk borders
    assert torch.equal(W.kv_rows_bf16(7, W.S_KV, lo, hi, 128), a[lo:hi])
    assert not torch.equal(a, W.normal_bf16(8, W.S_KV, a.shape))


def test_workload_geometry():
    wl = synth.WORKLOADS
    assert wl["csa_decode_4k"].lanes[0].entries == [1024]
    assert wl["hca_decode_128k"].lanes[0].entries == [1024] * 8
    assert wl["csa_decode_1m"].lanes[0].entries == [262144] * 4
    assert wl["csa_prefill_8k_on_128k"].lanes[0].entries == [34816]
    mixed = wl["mixed_decode_b32"]
    L = list(mixed.lanes[0].lengths) + list(mixed.lanes[1].lengths)
    assert len(L) == 32 and all((1 << 16) <= x < (1 << 20) for x in L)
    assert mixed.lanes[1].row_base == sum(mixed.lanes[0].lengths)
    assert L == synth.draw_lengths(4, 32)


def test_small_workload_generation_and_fp8_encoding():
    lane = W.Lane("csa", (1000, 333), (1000, 333), T=2, H=16, m=4, k=8, HI=4, kI_fp8=True)
    wl = W.Workload("t", 3, (lane,))
    inp = synth.generate(wl)
    li = inp.lanes[0]
    assert inp.kv.shape == (1333, 128) and inp.kv.dtype == torch.bfloat16
    assert inp.q.shape == (2, 2, 16, 128)
    assert li.qI.shape == (2, 2, 4, 64) and li.w.shape == (2, 2, 4)
    assert li.kI.dtype == torch.uint8 and li.kI.shape == (250 + 83, 64)
    assert li.k_scale.shape == (4 + 2,)
    assert li.scale_off.tolist() == [0, 4, 6]
    # decode * scale reproduces the fp32 draw to e4m3 precision (3 mantissa bits)
    x = W.normal_f32(3, W.S_KI, (333 * 64,), std=0.125).view(333, 64).double().numpy()
    dec = csa.decode_e4m3(li.kI.numpy())
    sc = li.k_scale.double().numpy()
    grp = np.concatenate([np.arange(250) // 64, 4 + np.arange(83) // 64])
    y = dec * sc[grp][:, None]
    assert np.all(np.abs(y - x) <= np.abs(x) * 2 ** -4 + sc[grp][:, None] * 2 ** -9 + 1e-12)
    assert np.all(np.abs(dec) <= 448)


def test_random_stage_inputs():
    s = synth.random_scores(1, 3, 100, levels=4)
    assert s.shape == (3, 100) and len(torch.unique(s)) <= 4
    z = synth.random_scores(2, 2, 50, neg=True)
    assert (z == 0).any()
    sel = synth.random_selection(3, 4, [10, 3, 0, 100], 8, fill=0.75)
    assert sel.shape == (4, 8)
    for r, n in enumerate([10, 3, 0, 100]):
        good = sel[r][sel[r] >= 0]
        assert len(good) == min(8, n, round(0.75 * min(8, n)))
        assert torch.all(good < n) and torch.all(good[1:] > good[:-1])


def test_mxfp4_encoding_rounds_to_the_grid():
    """Every decoded key lies on the E2M1 grid of its block's scale, within half a grid step
    of the fp32 value (or saturated at 6 * scale), with the block maximum at 4..8 scales;
    an all-zero block encodes as zero codes with the smallest scale."""
    r = np.random.default_rng(5)
    x = (r.standard_normal((300, 64)) * 0.125).astype(np.float32)
    x[7, :32] = 0.0
    pk, sc = W._encode_mxfp4(torch.from_numpy(x))
    assert pk.shape == (300, 32) and sc.shape == (300, 2)
    d = csa.decode_mxfp4_rows(pk.numpy(), sc.numpy())
    scale = np.repeat(csa.decode_e8m0(sc.numpy()), 32, axis=1)
    y = np.abs(x) / scale
    step = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
    sat = y >= 6
    err = np.abs(d - x) / scale
    assert np.all(err[~sat] <= step[~sat] / 2 + 1e-12)
    assert np.all(np.abs(d[sat]) == 6 * scale[sat])
    amax = np.abs(x.reshape(300, 2, 32)).max(axis=2)
    s_blk = csa.decode_e8m0(sc.numpy())
    nz = amax > 0
    assert np.all(amax[nz] / s_blk[nz] >= 4) and np.all(amax[nz] / s_blk[nz] < 8)
    assert np.all(pk.numpy()[7, :16] == 0) and sc.numpy()[7, 0] == 0


def test_fp4_lane_generation():
    lane = W.Lane("csa", (1000, 333), (1000, 333), T=1, H=16, m=4, k=8, HI=4, kI_fp4=True)
    li = synth.generate(W.Workload("t4", 3, (lane,))).lanes[0]
    assert li.kI.dtype == torch.uint8 and li.kI.shape == (250 + 83, 32)
    assert li.k_scale.dtype == torch.uint8 and li.k_scale.shape == (250 + 83, 2)
