"""Device-resident CSA and HCA lanes: buffers plus the call sequence of one attention step.

A lane owns the device copies of its inputs, the compressed cache, the scratch buffers the
calls need (scores, selected ids, workspaces) and the outputs, and chains the C-ABI calls
of one step on the current stream. Everything here is buffer management and argument
marshalling; the arithmetic happens in the HIP kernels.

CSA step ([P2] "Putting It Together"): compress the newest complete chunk(s) into the
cache, score every visible entry with the indexer, keep the top-k, attend to the selected
entries plus the raw window. HCA step: compress the newest chunk(s), attend densely.
"""
from __future__ import annotations

import copy
import math

import torch

from . import (PagedCache, attn_workspace_bytes, compress_kv, compress_kv_overlap, csa_decode_step, hca_attn_decode, hca_decode_step,
               indexer_scores, indexer_topk, sparse_attn_decode,
               topk_select, topk_workspace_bytes)


def _i64(x, device):
    return torch.as_tensor(list(x), dtype=torch.int64).to(device)


class _Lane:
    def __init__(self, lane, kv, z, q, kv_off, ent_off, q_pos, device="cuda"):
        self.lane = lane
        self.device = device
        self.kv, self.z, self.q = kv, z, q
        self.kv_off = kv_off.to(device)
        self.ent_off = ent_off.to(device)
        self.q_pos = q_pos.to(device)
        self.B, self.T, self.H, self.m, self.W = lane.B, lane.T, lane.H, lane.m, lane.W
        E = lane.entries
        self.E_tot = sum(E)
        self.max_entries = max(E) if E else 0
        self.ckv = torch.empty((max(self.E_tot, 1), lane.D), dtype=torch.bfloat16, device=device)
        # entries created by this step: those at or after the first query position, and at
        # least the newest complete chunk (decode appends one chunk every m tokens)
        first = []
        for n_b, e_b, p_b in zip(lane.lengths, E, lane.q_pos):
            first.append(max(0, min(p_b // self.m, e_b - 1)))
        self.first_new = _i64(first, device)
        self.n_new = max([e - f for e, f in zip(E, first)] + [0])
        self.out = torch.empty((self.B, self.T, self.H, lane.D), dtype=torch.float32, device=device)
        self.lse = torch.empty((self.B, self.T, self.H), dtype=torch.float32, device=device)
        self.scale = 1.0 / math.sqrt(lane.D)
        self.ckv_copies = [self.ckv]
        # attention extras ([P1] sections 7 and 8): per-head sink logits (fp32 [H] on the
        # device) and partial RoPE of the query / output; none by default
        self.sink = None
        self.rope_dims = 0
        self.rope_base = 10000.0
        self.paged = None  # PagedCache once the cache moved into the paged layout

    def compress_all(self):
        for c in self.ckv_copies:
            compress_kv(self.kv, self.z, self.kv_off, self.ent_off, self.m, c, max_new_entries=self.max_entries)

    def compress_new(self, r: int = 0):
        if self.n_new:
            compress_kv(self.kv, self.z, self.kv_off, self.ent_off, self.m, self.ckv_copies[r % len(self.ckv_copies)],
                        first_entry=self.first_new, max_new_entries=self.n_new, paged=self.paged)

    def paginate(self, ring_rows: int = 256, block_entries: int | None = None, spare_blocks: int = 5,
                 seed: int = 0, order: str = "random"):
        """Move the lane's compressed cache (and its indexer keys) into a paged pool and its
        raw rows into per-sequence rings ([P2] "KV Cache Management": a classical cache of
        blocks covering lcm(m, m') = 128 raw tokens, 128 / m entries each, and a state cache of
        the newest raw rows). Pool blocks are handed out in a seeded random order (``order`` =
        "random"), or round-robin over the sequences as concurrent growth would allocate them
        ("interleaved"), or each sequence's blocks consecutively ("sequential"), with some spare
        blocks left free, so every lookup goes through the block table. The compressed
        cache must be complete (compress_all) first; afterwards every call reads the paged
        buffers."""
        dev = self.device
        lane = self.lane
        eb = block_entries or max(1, 128 // self.m)
        E = lane.entries
        nblk = [(e + eb - 1) // eb for e in E]
        max_blocks = max(nblk + [1])
        total = sum(nblk) + spare_blocks
        table = torch.zeros((self.B, max_blocks), dtype=torch.int32)
        if order == "random":
            g = torch.Generator().manual_seed(seed)
            perm = torch.randperm(total, generator=g).to(torch.int32)
            used = 0
            for b, n in enumerate(nblk):
                table[b, :n] = perm[used:used + n]
                used += n
        elif order == "sequential":  # each sequence's blocks consecutive, in order
            nxt = 0
            for b, n in enumerate(nblk):
                table[b, :n] = torch.arange(nxt, nxt + n, dtype=torch.int32)
                nxt += n
        else:  # block j of every sequence before block j + 1 of any
            nxt = 0
            for j in range(max_blocks):
                for b, n in enumerate(nblk):
                    if j < n:
                        table[b, j] = nxt
                        nxt += 1
        # pool row of every entry, sequence by sequence (packed entry order)
        rows = []
        for b, e in enumerate(E):
            i = torch.arange(e, dtype=torch.int64)
            rows.append(table[b].to(torch.int64)[i // eb] * eb + i % eb)
        prow = torch.cat(rows).to(dev) if rows else torch.zeros(0, dtype=torch.int64, device=dev)
        pool_rows = total * eb

        def to_pool(x):
            out = torch.zeros((pool_rows,) + tuple(x.shape[1:]), dtype=x.dtype, device=dev)
            if prow.numel():
                out.index_copy_(0, prow, x[:prow.numel()])
            return out

        # ring row of the newest ring_rows raw rows of every sequence (none for ring_rows = 0)
        src, dst = [], []
        offs = lane.kv_off()
        for b, n in enumerate(lane.lengths if ring_rows > 0 else ()):
            r = torch.arange(max(0, n - ring_rows), n, dtype=torch.int64)
            src.append(offs[b] - offs[0] + r)
            dst.append(b * ring_rows + r % ring_rows)
        src = torch.cat(src).to(dev) if src else None
        dst = torch.cat(dst).to(dev) if dst else None
        row0 = offs[0]

        def to_ring(x):
            if x is None:
                return None
            out = torch.zeros((self.B * ring_rows, x.shape[1]), dtype=x.dtype, device=dev)
            out.index_copy_(0, dst, x[row0:].index_select(0, src))
            return out

        self.ckv_copies = [to_pool(c) for c in self.ckv_copies]
        self.ckv = self.ckv_copies[0]
        if ring_rows > 0:  # ring_rows = 0 keeps the raw rows packed as kv_off says
            self.kv, self.z = to_ring(self.kv), to_ring(self.z)
            if getattr(self, "kv_b", None) is not None:
                self.kv_b, self.z_b = to_ring(self.kv_b), to_ring(self.z_b)
        if hasattr(self, "kI_copies"):
            self.kI_copies = [to_pool(c) for c in self.kI_copies]
            self.kI = self.kI_copies[0]
            if self.k_format == "mxfp4":
                self.k_scale_copies = [to_pool(c) for c in self.k_scale_copies]
                self.k_scale = self.k_scale_copies[0]
            elif self.k_scale is not None:
                # fp8 group scales move with the blocks: the scale of pool row r sits at
                # r >> min(log2(group), log2(block)), one per group inside a block or one per
                # block (repeated) when a group spans several blocks
                g = int(self.scale_group)
                assert g > 0 and g & (g - 1) == 0 and eb & (eb - 1) == 0, "power-of-two groups and blocks"
                sh = min(g.bit_length(), eb.bit_length()) - 1
                soff = self.scale_off.cpu()
                sidx = torch.cat([soff[b] + torch.arange(e, dtype=torch.int64) // g for b, e in enumerate(E)]
                                 + [torch.zeros(0, dtype=torch.int64)]).to(dev)
                pool_sc = torch.zeros(max(pool_rows >> sh, 1), dtype=self.k_scale.dtype, device=dev)
                if prow.numel():
                    pool_sc[prow >> sh] = self.k_scale[sidx]
                self.k_scale = pool_sc
                self.k_scale_copies = [pool_sc]
        # row offsets now only count rows: rebase the raw-row prefix sums at 0
        if ring_rows > 0:
            self.kv_off = self.kv_off - self.kv_off[0]
        self.paged = PagedCache(table.to(dev), eb, pool_rows, ring_rows)
        self.pool_rows = pool_rows

    def rotate(self, copies: int):
        """Keep ``copies`` independent copies of the large per-step inputs (compressed cache,
        indexer keys) so that consecutive steps stream different memory: the copies together
        exceed the last-level cache and each step reads from HBM."""
        self.ckv_copies = [self.ckv] + [self.ckv.clone() for _ in range(copies - 1)]

    # per-step outputs and scratch: everything a step writes apart from the cache's newest entries
    _STEP_BUFFERS = ("scores", "idx", "out", "lse", "topk_ws", "attn_ws")

    def micro_batch(self):
        """A lane over the same inputs and cache copies with its own outputs and workspaces,
        so that its steps can run concurrently with this lane's (independent micro-batches in
        flight on parallel streams or graph branches). Concurrent steps must use different
        cache copies: every step rewrites its copy's newest entries."""
        twin = copy.copy(self)
        for name in self._STEP_BUFFERS:
            buf = getattr(self, name, None)
            if buf is not None:
                setattr(twin, name, torch.zeros_like(buf))
        return twin


class CsaLane(_Lane):
    def __init__(self, lane, kv, z, q, li, device="cuda", fused: bool = True, kv_b=None, z_b=None,
                 scoreless: bool = False):
        super().__init__(lane, kv, z, q, li.kv_off, li.ent_off, li.q_pos, device)
        # scoreless: the step selects with the indexer fused with top-k and keeps no score matrix
        self.scoreless = scoreless
        # overlapped compression ([P2] "Deep Dive", dual-series KV compression): series b
        # rows kv_b / z_b, shaped like kv / z; None keeps single-series compression
        self.kv_b, self.z_b = kv_b, z_b
        self.k = lane.k
        self.fused = fused  # the indexer leaves top-k candidate lists for the selection
        self.qI = li.qI.to(device)
        self.w = li.w.to(device)
        self.kI = li.kI.to(device)
        self.k_scale = None if li.k_scale is None else li.k_scale.to(device)
        self.scale_off = None if li.scale_off is None else li.scale_off.to(device)
        self.scale_group = lane.scale_group
        self.k_format = "mxfp4" if getattr(lane, "kI_fp4", False) else None
        self.scores = None if scoreless else torch.empty((self.B, self.T, max(self.max_entries, 1)),
                                                          dtype=torch.float32, device=device)
        self.idx = torch.empty((self.B, self.T, self.k), dtype=torch.int32, device=device)
        nb = topk_workspace_bytes(self.B, self.T, self.max_entries, self.k)
        # workspaces (their contents on entry do not matter; zeroed once at allocation)
        self.topk_ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device=device)
        na = attn_workspace_bytes(self.B, self.T, self.H, lane.D, self.k + self.W)
        self.attn_ws = torch.zeros(max(na, 16), dtype=torch.uint8, device=device)
        self.kI_copies = [self.kI]
        self.k_scale_copies = [self.k_scale]
        # steps keep no scores for rows selected from candidate lists (csl.h, scores_on_demand)
        self.scores_on_demand = False

    def compress_all(self):
        if self.kv_b is None:
            return super().compress_all()
        for c in self.ckv_copies:
            compress_kv_overlap(self.kv, self.z, self.kv_b, self.z_b, self.kv_off, self.ent_off, self.m, c,
                                max_new_entries=self.max_entries)

    def compress_new(self, r: int = 0):
        if self.kv_b is None:
            return super().compress_new(r)
        if self.n_new:
            compress_kv_overlap(self.kv, self.z, self.kv_b, self.z_b, self.kv_off, self.ent_off, self.m,
                                self.ckv_copies[r % len(self.ckv_copies)], first_entry=self.first_new,
                                max_new_entries=self.n_new, paged=self.paged)

    def rotate(self, copies: int):
        super().rotate(copies)
        self.kI_copies = [self.kI] + [self.kI.clone() for _ in range(copies - 1)]
        # per-row MXFP4 scales are as large a stream as the keys' own share: copy them too
        if self.k_format == "mxfp4":
            self.k_scale_copies = [self.k_scale] + [self.k_scale.clone() for _ in range(copies - 1)]

    def index(self, r: int = 0):
        if self.scoreless:  # the selection itself: no score matrix
            indexer_topk(self.qI, self.w, self.kI_copies[r % len(self.kI_copies)], self.ent_off, self.q_pos, self.m,
                         self.k, self.idx, max_entries=self.max_entries,
                         k_scale=self.k_scale_copies[r % len(self.k_scale_copies)], scale_off=self.scale_off,
                         scale_group=self.scale_group, k_format=self.k_format, paged=self.paged)
            return
        indexer_scores(self.qI, self.w, self.kI_copies[r % len(self.kI_copies)], self.ent_off, self.q_pos, self.m,
                       self.scores, max_entries=self.max_entries,
                       k_scale=self.k_scale_copies[r % len(self.k_scale_copies)], scale_off=self.scale_off,
                       scale_group=self.scale_group, topk_ws=self.topk_ws if self.fused else None, topk_k=self.k,
                       k_format=self.k_format, paged=self.paged)

    def select(self):
        if self.scoreless:  # index() already selected
            return
        topk_select(self.scores, self.ent_off, self.q_pos, self.m, self.k, self.idx, ws=self.topk_ws,
                    max_entries=self.max_entries, prepared=self.fused)

    def attend(self, r: int = 0):
        sparse_attn_decode(self.q, self.ckv_copies[r % len(self.ckv_copies)], self.idx, self.kv, self.kv_off,
                           self.ent_off, self.q_pos, self.W, self.out, lse=self.lse, scale=self.scale,
                           ws=self.attn_ws, sink=self.sink, rope_dims=self.rope_dims, rope_base=self.rope_base,
                           paged=self.paged)

    def step(self, r: int = 0, fused: bool = True):
        """One decode step on rotated copy r: one csa_decode_step call, or (fused=False) the
        four entry points one after the other; both give the same result."""
        if not fused:
            self.compress_new(r)
            self.index(r)
            self.select()
            self.attend(r)
            return
        csa_decode_step(self.kv, self.z, self.kv_off, self.ent_off, self.first_new, self.n_new,
                        self.ckv_copies[r % len(self.ckv_copies)], self.qI, self.w,
                        self.kI_copies[r % len(self.kI_copies)], self.scores,
                        self.topk_ws, self.k, self.idx, self.q, self.W, self.out, self.q_pos,
                        self.m, lse=self.lse, scale=self.scale,
                        k_scale=self.k_scale_copies[r % len(self.k_scale_copies)], scale_off=self.scale_off,
                        scale_group=self.scale_group, max_entries=self.max_entries, attn_ws=self.attn_ws,
                        kv_b=self.kv_b, z_b=self.z_b, sink=self.sink, rope_dims=self.rope_dims,
                        rope_base=self.rope_base, k_format=self.k_format, paged=self.paged,
                        scores_on_demand=self.scores_on_demand)


class HcaLane(_Lane):
    def __init__(self, lane, kv, z, q, li, device="cuda"):
        super().__init__(lane, kv, z, q, li.kv_off, li.ent_off, li.q_pos, device)
        na = attn_workspace_bytes(self.B, self.T, self.H, lane.D, self.max_entries + self.W)
        self.attn_ws = torch.zeros(max(na, 16), dtype=torch.uint8, device=device)

    def attend(self, r: int = 0):
        hca_attn_decode(self.q, self.ckv_copies[r % len(self.ckv_copies)], self.kv, self.kv_off, self.ent_off,
                        self.q_pos, self.m, self.W, self.out, lse=self.lse, scale=self.scale,
                        max_entries=self.max_entries, ws=self.attn_ws, sink=self.sink, rope_dims=self.rope_dims,
                        rope_base=self.rope_base, paged=self.paged)

    def step(self, r: int = 0, fused: bool = True):
        """One decode step on rotated copy r: one hca_decode_step call (the newest-entry
        compression inside the attention launch), or (fused=False) compress_kv then
        hca_attn_decode."""
        if not fused:
            self.compress_new(r)
            self.attend(r)
            return
        hca_decode_step(self.kv, self.z, self.kv_off, self.ent_off, self.first_new, self.n_new,
                        self.ckv_copies[r % len(self.ckv_copies)], self.q, self.W, self.out, self.q_pos, self.m,
                        self.max_entries, lse=self.lse, scale=self.scale, attn_ws=self.attn_ws, sink=self.sink,
                        rope_dims=self.rope_dims, rope_base=self.rope_base, paged=self.paged)


def in_flight_graph(chains):
    """Capture one HIP graph whose branches are independent chains of calls (each a list of
    callables that enqueue work on the current stream), for example the steps of several
    micro-batches. Each chain is recorded on its own side stream, forked from the capture
    stream at the start and joined to it at the end, so a replay runs the chains
    concurrently and returns on the stream it was replayed on once all of them are done.
    Chains must not write what another chain reads or writes."""
    side = [torch.cuda.Stream() for _ in chains]  # default priority, like every stream here
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = torch.cuda.current_stream()
        for st, chain in zip(side, chains):
            st.wait_stream(cap)
            with torch.cuda.stream(st):
                for fn in chain:
                    fn()
        for st in side:
            cap.wait_stream(st)
    return g


def build_lanes(inp, device="cuda", scoreless: bool = False):
    """Upload a ``synth.Inputs`` and wrap each of its lanes (``scoreless``: CSA steps select
    with the indexer fused with top-k, keeping no score matrix)."""
    kv = inp.kv.to(device)
    z = None if inp.z is None else inp.z.to(device)
    # series b (if drawn) switches the CSA lanes to overlapped compression; HCA keeps one series
    kv_b = None if getattr(inp, "kv_b", None) is None else inp.kv_b.to(device)
    z_b = None if getattr(inp, "z_b", None) is None else inp.z_b.to(device)
    q_all = inp.q.to(device)
    lanes = []
    for li in inp.lanes:
        q = q_all[li.q_slice].contiguous()
        if li.lane.kind == "csa":
            lanes.append(CsaLane(li.lane, kv, z, q, li, device, kv_b=kv_b, z_b=z_b, scoreless=scoreless))
        else:
            lanes.append(HcaLane(li.lane, kv, z, q, li, device))
    return lanes
