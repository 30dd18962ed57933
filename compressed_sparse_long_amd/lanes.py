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

import math

import torch

from . import (attn_workspace_bytes, compress_kv, compress_kv_overlap, csa_decode_step, hca_attn_decode, indexer_scores, sparse_attn_decode,
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

    def compress_all(self):
        for c in self.ckv_copies:
            compress_kv(self.kv, self.z, self.kv_off, self.ent_off, self.m, c, max_new_entries=self.max_entries)

    def compress_new(self, r: int = 0):
        if self.n_new:
            compress_kv(self.kv, self.z, self.kv_off, self.ent_off, self.m, self.ckv_copies[r % len(self.ckv_copies)],
                        first_entry=self.first_new, max_new_entries=self.n_new)

    def rotate(self, copies: int):
        """Keep ``copies`` independent copies of the large per-step inputs (compressed cache,
        indexer keys) so that consecutive steps stream different memory: the copies together
        exceed the last-level cache and each step reads from HBM."""
        self.ckv_copies = [self.ckv] + [self.ckv.clone() for _ in range(copies - 1)]


class CsaLane(_Lane):
    def __init__(self, lane, kv, z, q, li, device="cuda", fused: bool = True, kv_b=None, z_b=None):
        super().__init__(lane, kv, z, q, li.kv_off, li.ent_off, li.q_pos, device)
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
        self.scores = torch.empty((self.B, self.T, max(self.max_entries, 1)), dtype=torch.float32, device=device)
        self.idx = torch.empty((self.B, self.T, self.k), dtype=torch.int32, device=device)
        nb = topk_workspace_bytes(self.B, self.T, self.max_entries, self.k)
        self.topk_ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=device)  # contents never matter on entry
        na = attn_workspace_bytes(self.B, self.T, self.H, lane.D, self.k + self.W)
        self.attn_ws = torch.empty(max(na, 16), dtype=torch.uint8, device=device)
        self.kI_copies = [self.kI]
        self.k_scale_copies = [self.k_scale]

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
                                max_new_entries=self.n_new)

    def rotate(self, copies: int):
        super().rotate(copies)
        self.kI_copies = [self.kI] + [self.kI.clone() for _ in range(copies - 1)]
        # per-row MXFP4 scales are as large a stream as the keys' own share: copy them too
        if self.k_format == "mxfp4":
            self.k_scale_copies = [self.k_scale] + [self.k_scale.clone() for _ in range(copies - 1)]

    def index(self, r: int = 0):
        indexer_scores(self.qI, self.w, self.kI_copies[r % len(self.kI_copies)], self.ent_off, self.q_pos, self.m,
                       self.scores, max_entries=self.max_entries,
                       k_scale=self.k_scale_copies[r % len(self.k_scale_copies)], scale_off=self.scale_off,
                       scale_group=self.scale_group, topk_ws=self.topk_ws if self.fused else None, topk_k=self.k,
                       k_format=self.k_format)

    def select(self):
        topk_select(self.scores, self.ent_off, self.q_pos, self.m, self.k, self.idx, ws=self.topk_ws,
                    max_entries=self.max_entries, prepared=self.fused)

    def attend(self, r: int = 0):
        sparse_attn_decode(self.q, self.ckv_copies[r % len(self.ckv_copies)], self.idx, self.kv, self.kv_off,
                           self.ent_off, self.q_pos, self.W, self.out, lse=self.lse, scale=self.scale,
                           ws=self.attn_ws, sink=self.sink, rope_dims=self.rope_dims, rope_base=self.rope_base)

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
                        rope_base=self.rope_base, k_format=self.k_format)


class HcaLane(_Lane):
    def __init__(self, lane, kv, z, q, li, device="cuda"):
        super().__init__(lane, kv, z, q, li.kv_off, li.ent_off, li.q_pos, device)
        na = attn_workspace_bytes(self.B, self.T, self.H, lane.D, self.max_entries + self.W)
        self.attn_ws = torch.empty(max(na, 16), dtype=torch.uint8, device=device)

    def attend(self, r: int = 0):
        hca_attn_decode(self.q, self.ckv_copies[r % len(self.ckv_copies)], self.kv, self.kv_off, self.ent_off,
                        self.q_pos, self.m, self.W, self.out, lse=self.lse, scale=self.scale,
                        max_entries=self.max_entries, ws=self.attn_ws, sink=self.sink, rope_dims=self.rope_dims,
                        rope_base=self.rope_base)

    def step(self, r: int = 0):
        self.compress_new(r)
        self.attend(r)


def build_lanes(inp, device="cuda"):
    """Upload a ``synth.Inputs`` and wrap each of its lanes."""
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
            lanes.append(CsaLane(li.lane, kv, z, q, li, device, kv_b=kv_b, z_b=z_b))
        else:
            lanes.append(HcaLane(li.lane, kv, z, q, li, device))
    return lanes
