"""Workload descriptions and seeded input generation.

Every array is drawn from its own counter-addressed stream: chunk ``c`` of stream
``s`` under seed ``seed`` comes from ``numpy.random.PCG64(SeedSequence([seed, s, c]))``.
That makes the values independent of the number of threads used to draw them, and
lets a test regenerate one chunk (for example the rows of one compressed entry)
without drawing the whole array.

Stream ids follow a fixed order: lengths, kv, z, q, qI, kI, w, then kv_b and z_b (the
second raw series and its logits of CSA's overlapped compression, drawn only on request).
Normal draws are float32, scaled by an exact power of two where a variance of 1/64
is asked for (std 0.125), then rounded to bf16 by torch's round-to-nearest-even cast.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np
import torch

CHUNK = 1 << 22  # values per counter-addressed chunk

S_LENGTHS, S_KV, S_Z, S_Q, S_QI, S_KI, S_W, S_KV_B, S_Z_B = range(9)
S_EXTRA = 100  # first stream id for ad-hoc test draws


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _rng(seed: int, stream: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, chunk])))


def _fill(seed: int, stream: int, n: int, kind: str, out: np.ndarray | None = None,
          first_chunk: int = 0) -> np.ndarray:
    """Draw ``n`` float32 values of ``kind`` ('normal' | 'uniform') from one stream."""
    if out is None:
        out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def one(c: int) -> None:
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        g = _rng(seed, stream, first_chunk + c)
        if kind == "normal":
            g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        else:
            g.random(hi - lo, dtype=np.float32, out=out[lo:hi])

    if nchunks <= 1:
        for c in range(nchunks):
            one(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(nchunks)))
    return out


def normal_bf16(seed: int, stream: int, shape, std: float = 1.0) -> torch.Tensor:
    """bf16 tensor of N(0, std^2) draws (fp32 draw, exact power-of-two scale, RNE to bf16)."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = torch.empty(n, dtype=torch.bfloat16)
    step = 1 << 26  # convert in slices to bound host memory
    assert step % CHUNK == 0
    for lo in range(0, n, step):
        hi = min(n, lo + step)
        x = _fill(seed, stream, hi - lo, "normal", first_chunk=lo // CHUNK)
        if std != 1.0:
            x *= np.float32(std)
        out[lo:hi] = torch.from_numpy(x).to(torch.bfloat16)
    return out.view(*shape)


def normal_f32(seed: int, stream: int, shape, std: float = 1.0) -> torch.Tensor:
    n = int(np.prod(shape))
    x = _fill(seed, stream, n, "normal")
    if std != 1.0:
        x *= np.float32(std)
    return torch.from_numpy(x).view(*shape)


def uniform_f32(seed: int, stream: int, shape) -> torch.Tensor:
    n = int(np.prod(shape))
    return torch.from_numpy(_fill(seed, stream, n, "uniform")).view(*shape)


def kv_rows_bf16(seed: int, stream: int, row_lo: int, row_hi: int, D: int) -> torch.Tensor:
    """Rows [row_lo, row_hi) of a packed [rows, D] N(0,1) bf16 array drawn by :func:`normal_bf16`.

    Regenerates only the chunks that hold those rows, so a test can look at a few
    compressed entries of a 1M-row context without drawing all of it.
    """
    v_lo, v_hi = row_lo * D, row_hi * D
    c_lo, c_hi = v_lo // CHUNK, (v_hi + CHUNK - 1) // CHUNK
    vals = np.empty((c_hi - c_lo) * CHUNK, dtype=np.float32)
    for c in range(c_lo, c_hi):
        _rng(seed, stream, c).standard_normal(CHUNK, dtype=np.float32,
                                              out=vals[(c - c_lo) * CHUNK:(c - c_lo + 1) * CHUNK])
    sl = vals[v_lo - c_lo * CHUNK: v_hi - c_lo * CHUNK]
    return torch.from_numpy(sl.copy()).to(torch.bfloat16).view(row_hi - row_lo, D)


# --------------------------------------------------------------------------------------
# Workload descriptions
# --------------------------------------------------------------------------------------

@dataclass(frozen=True)
class Lane:
    """One attention lane over a batch of sequences.

    kind:     'csa' (compress m, indexer, top-k, sparse attention) or 'hca' (compress m, dense).
    lengths:  raw KV rows N_b per sequence (packed consecutively in the kv array).
    q_pos:    absolute position of query row 0 of each sequence; row t sits at q_pos + t.
    row_base: index of this lane's first raw row in the packed kv array.
    seq_base: index of this lane's first sequence in the packed q array.
    """
    kind: str
    lengths: tuple
    q_pos: tuple
    T: int
    H: int
    m: int
    W: int = 128
    D: int = 128
    k: int = 0
    HI: int = 0
    CI: int = 64
    kI_fp8: bool = False
    kI_fp4: bool = False         # MXFP4 indexer keys (E2M1 codes, one E8M0 scale per 32 dims)
    scale_group: int = 64
    row_base: int = 0
    seq_base: int = 0

    @property
    def B(self) -> int:
        return len(self.lengths)

    @property
    def entries(self) -> list:
        return [n // self.m for n in self.lengths]

    def kv_off(self) -> list:
        off = [self.row_base]
        for n in self.lengths:
            off.append(off[-1] + n)
        return off

    def ent_off(self) -> list:
        off = [0]
        for e in self.entries:
            off.append(off[-1] + e)
        return off

    def scale_off(self) -> list:
        off = [0]
        for e in self.entries:
            off.append(off[-1] + (e + self.scale_group - 1) // self.scale_group)
        return off


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    lanes: tuple
    desc: str = ""
    z_present: bool = True

    @property
    def total_rows(self) -> int:
        return sum(sum(l.lengths) for l in self.lanes)

    @property
    def total_seqs(self) -> int:
        return sum(l.B for l in self.lanes)


def draw_lengths(seed: int, n: int, lo: int = 1 << 16, hi: int = 1 << 20) -> list:
    """Context lengths drawn log-uniformly in [lo, hi): floor(exp(U*ln(hi/lo) + ln lo))."""
    u = _rng(seed, S_LENGTHS, 0).random(n)  # float64
    return [int(math.floor(math.exp(x * math.log(hi / lo) + math.log(lo)))) for x in u]


def _mixed() -> Workload:
    L = draw_lengths(4, 32)
    csa = Lane("csa", tuple(L[:16]), tuple(L[:16]), T=1, H=64, m=4, k=1024, HI=8, kI_fp8=True,
               row_base=0, seq_base=0)
    hca = Lane("hca", tuple(L[16:]), tuple(L[16:]), T=1, H=64, m=128,
               row_base=sum(L[:16]), seq_base=16)
    return Workload("mixed_decode_b32", 4, (csa, hca),
                    "32 ragged sequences (64K..1M): 16 CSA (m=4, top-1024, fp8 keys) + 16 HCA (m=128)")


WORKLOADS = {
    "csa_decode_4k": Workload(
        "csa_decode_4k", 0,
        (Lane("csa", (4096,), (4096,), T=1, H=16, m=4, k=64, HI=4),),
        "CSA decode, B=1, 4096-token context, 16 heads, top-64 of 1024 entries"),
    "hca_decode_128k": Workload(
        "hca_decode_128k", 1,
        (Lane("hca", (131072,) * 8, (131072,) * 8, T=1, H=64, m=128),),
        "HCA decode, B=8, 131072-token contexts, 64 heads, 1024 entries each"),
    "csa_decode_1m": Workload(
        "csa_decode_1m", 2,
        (Lane("csa", (1 << 20,) * 4, (1 << 20,) * 4, T=1, H=64, m=4, k=1024, HI=8),),
        "CSA decode, B=4, 1M-token contexts, 64 heads, top-1024 of 262144 entries"),
    "csa_prefill_8k_on_128k": Workload(
        "csa_prefill_8k_on_128k", 3,
        (Lane("csa", (131072 + 8192,), (131072,), T=8192, H=64, m=4, k=512, HI=8),),
        "CSA prefill chunk: 8192 query rows on a 131072-token prefix, top-512"),
}
WORKLOADS["mixed_decode_b32"] = _mixed()
CONFIG_ORDER = ["csa_decode_4k", "hca_decode_128k", "csa_decode_1m",
                "csa_prefill_8k_on_128k", "mixed_decode_b32"]


# --------------------------------------------------------------------------------------
# Generation
# --------------------------------------------------------------------------------------

@dataclass
class LaneInputs:
    lane: Lane
    qI: torch.Tensor | None = None        # bf16 [B, T, HI, CI]
    kI: torch.Tensor | None = None        # bf16 [E, CI] or uint8 (e4m3 bytes) [E, CI]
    k_scale: torch.Tensor | None = None   # fp32 [sum ceil(E_b/G)] (fp8 keys only)
    w: torch.Tensor | None = None         # fp32 [B, T, HI]
    kv_off: torch.Tensor = field(default=None)
    ent_off: torch.Tensor = field(default=None)
    scale_off: torch.Tensor = field(default=None)
    q_pos: torch.Tensor = field(default=None)
    q_slice: slice = field(default=None)  # this lane's sequences in the packed q


@dataclass
class Inputs:
    workload: Workload
    kv: torch.Tensor | None      # bf16 [rows, D]
    z: torch.Tensor | None       # bf16 [rows, D]
    q: torch.Tensor | None       # bf16 [S, T, H, D]
    lanes: list
    kv_b: torch.Tensor | None = None   # bf16 [rows, D], series b of overlapped compression
    z_b: torch.Tensor | None = None    # bf16 [rows, D]


def _encode_e4m3(x: torch.Tensor, lengths_e: list, group: int):
    """Per-group fp8 e4m3 (OCP, finite-only) encoding with one fp32 scale per ``group`` entries.

    scale = amax(group tile) / 448, codes = RNE(x / scale) saturated to +-448 (torch cast).
    """
    codes = torch.empty(x.shape, dtype=torch.uint8)
    scales = []
    r = 0
    for e in lengths_e:
        for g0 in range(0, e, group):
            g1 = min(e, g0 + group)
            tile = x[r + g0:r + g1]
            amax = float(tile.abs().max()) if g1 > g0 else 0.0
            s = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
            y = torch.clamp(tile / torch.tensor(s, dtype=torch.float32), -448.0, 448.0)
            codes[r + g0:r + g1] = y.to(torch.float8_e4m3fn).view(torch.uint8)
            scales.append(s)
        r += e
    return codes, torch.tensor(np.array(scales, dtype=np.float32))


def _encode_mxfp4(x: torch.Tensor):
    """OCP MXFP4 encoding of key rows x fp32 [E, C]: per block of 32 consecutive dims, the
    shared scale is 2^X with X = floor(log2(amax)) - 2 (2 = the largest E2M1 exponent),
    clamped to [-127, 127] (an all-zero block takes X = -127); each element is x / 2^X
    rounded to nearest-even on the E2M1 grid {0, 0.5, 1, 1.5, 2, 3, 4, 6} and saturated to
    +-6. Returns packed codes uint8 [E, C/2] (element 2j in the low nibble of byte j) and
    E8M0 scales uint8 [E, C/32]."""
    v = x.numpy().astype(np.float64)
    E, C = v.shape
    blk = v.reshape(E, C // 32, 32)
    amax = np.abs(blk).max(axis=2)
    with np.errstate(divide="ignore"):
        X = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
    X = np.clip(X, -127, 127)
    y = np.abs(blk) / np.exp2(X)[:, :, None]
    # round to nearest even on the grid: steps of 0.5 below 2, 1 in [2, 4), 2 from 4 up
    q = np.where(y < 2, np.rint(y * 2) / 2, np.where(y < 4, np.rint(y), 2 * np.rint(y / 2)))
    q = np.minimum(q, 6.0)
    code = _e2m1_code(q) | np.where(blk < 0, 8, 0).astype(np.uint8)
    code = code.reshape(E, C)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    scales = (X + 127).astype(np.uint8)
    return torch.from_numpy(packed), torch.from_numpy(scales)


def _e2m1_code(q: np.ndarray) -> np.ndarray:
    """E2M1 magnitude code of grid values q in {0, 0.5, 1, 1.5, 2, 3, 4, 6}."""
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    return np.searchsorted(grid, q).astype(np.uint8)


def generate(wl: Workload | str, parts=("kv", "z", "q", "qI", "kI", "w")) -> Inputs:
    """Draw the inputs of a workload (CPU tensors). ``parts`` selects which arrays to draw;
    "kv_b" and "z_b" (series b of overlapped compression, shaped like kv and z) are drawn
    only when listed."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    D = wl.lanes[0].D
    rows = wl.total_rows
    S = wl.total_seqs
    T = max(l.T for l in wl.lanes)
    H = wl.lanes[0].H
    kv = normal_bf16(wl.seed, S_KV, (rows, D)) if "kv" in parts else None
    z = normal_bf16(wl.seed, S_Z, (rows, D)) if ("z" in parts and wl.z_present) else None
    q = normal_bf16(wl.seed, S_Q, (S, T, H, D)) if "q" in parts else None
    lanes = []
    qi_off = ki_off = w_off = 0  # element offsets inside the shared qI / kI / w streams
    csa_lanes = [l for l in wl.lanes if l.kind == "csa"]
    n_qi = sum(l.B * l.T * l.HI * l.CI for l in csa_lanes)
    n_ki = sum(sum(l.entries) * l.CI for l in csa_lanes)
    n_w = sum(l.B * l.T * l.HI for l in csa_lanes)
    qi_all = normal_f32(wl.seed, S_QI, (n_qi,), std=0.125) if ("qI" in parts and n_qi) else None
    ki_all = normal_f32(wl.seed, S_KI, (n_ki,), std=0.125) if ("kI" in parts and n_ki) else None
    w_all = uniform_f32(wl.seed, S_W, (n_w,)) if ("w" in parts and n_w) else None
    for lane in wl.lanes:
        li = LaneInputs(lane)
        li.kv_off = torch.tensor(lane.kv_off(), dtype=torch.int64)
        li.ent_off = torch.tensor(lane.ent_off(), dtype=torch.int64)
        li.q_pos = torch.tensor(lane.q_pos, dtype=torch.int64)
        li.q_slice = slice(lane.seq_base, lane.seq_base + lane.B)
        if lane.kind == "csa":
            nq = lane.B * lane.T * lane.HI * lane.CI
            nk = sum(lane.entries) * lane.CI
            nw = lane.B * lane.T * lane.HI
            if qi_all is not None:
                li.qI = qi_all[qi_off:qi_off + nq].to(torch.bfloat16).view(lane.B, lane.T, lane.HI, lane.CI)
            if ki_all is not None:
                x = ki_all[ki_off:ki_off + nk].view(sum(lane.entries), lane.CI)
                if lane.kI_fp8:
                    li.kI, li.k_scale = _encode_e4m3(x, lane.entries, lane.scale_group)
                    li.scale_off = torch.tensor(lane.scale_off(), dtype=torch.int64)
                elif lane.kI_fp4:
                    li.kI, li.k_scale = _encode_mxfp4(x)
                else:
                    li.kI = x.to(torch.bfloat16)
            if w_all is not None:
                li.w = w_all[w_off:w_off + nw].clone().view(lane.B, lane.T, lane.HI)
            qi_off += nq
            ki_off += nk
            w_off += nw
        lanes.append(li)
    kv_b = normal_bf16(wl.seed, S_KV_B, (rows, D)) if "kv_b" in parts else None
    z_b = normal_bf16(wl.seed, S_Z_B, (rows, D)) if ("z_b" in parts and wl.z_present) else None
    return Inputs(wl, kv, z, q, lanes, kv_b, z_b)


# --------------------------------------------------------------------------------------
# Ad-hoc stage inputs for tests
# --------------------------------------------------------------------------------------

def random_scores(seed: int, rows: int, n: int, levels: int = 0, neg: bool = False) -> torch.Tensor:
    """fp32 [rows, n] scores. ``levels`` > 0 draws from that many distinct values (many ties).

    With ``neg`` the values span both signs and include -0.0 and +0.0.
    """
    g = _rng(seed, S_EXTRA, 0)
    if levels > 0:
        vals = g.standard_normal(levels).astype(np.float32)
        if not neg:
            vals = np.abs(vals)
        x = vals[g.integers(0, levels, size=(rows, n))]
    else:
        x = g.standard_normal((rows, n)).astype(np.float32)
        if not neg:
            x = np.abs(x)
    if neg and n >= 4:
        x[:, ::7] = np.float32(0.0)
        x[:, 3::11] = np.float32(-0.0)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))


def random_selection(seed: int, rows: int, n_entries: list, k: int, fill: float = 1.0) -> torch.Tensor:
    """int32 [rows, k]: per row a random ascending set of distinct entry ids < n_entries[row],
    of size round(fill * min(k, n)), padded with -1."""
    g = _rng(seed, S_EXTRA + 1, 0)
    out = np.full((rows, k), -1, dtype=np.int32)
    for r in range(rows):
        n = n_entries[r]
        c = min(k, n, int(round(fill * min(k, n))))
        if c > 0:
            ids = np.sort(g.choice(n, size=c, replace=False)).astype(np.int32)
            out[r, :c] = ids
    return torch.from_numpy(out)


def with_lanes(wl: Workload, **kw) -> Workload:
    """Copy of a one-lane workload with fields of its lane replaced (for scaled-down tests)."""
    assert len(wl.lanes) == 1
    return replace(wl, lanes=(replace(wl.lanes[0], **kw),))
