"""Python binding of libcsl.so, the gfx950 hybrid compressed-attention library.

Argument marshalling only: every function takes torch tensors that already live on the
GPU, passes their device pointers, sizes and torch's current HIP stream to the C ABI
(include/csl.h), and raises on a non-zero status. All computation happens in the HIP
kernels; there is no fallback path. Importing fails if the shared library is not built.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "compress_kv", "compress_kv_overlap", "indexer_scores", "indexer_topk", "indexer_topk_max_k", "topk_select",
    "sparse_attn_decode", "hca_attn_decode", "csa_decode_step", "csa_decode_step_static", "hca_decode_step",
    "topk_workspace_bytes", "attn_workspace_bytes", "PagedCache", "version", "LIB_PATH",
    "EXPORTS", "CslError",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsl.so")

BF16, F32, FP8_E4M3, MXFP4 = 0, 1, 2, 3
EXPORTS = [
    "csl_last_error", "csl_version", "csl_compress_kv", "csl_compress_kv_overlap", "csl_indexer_scores",
    "csl_indexer_topk_max_k", "csl_indexer_topk",
    "csl_topk_workspace_bytes", "csl_topk_select", "csl_attn_workspace_bytes",
    "csl_sparse_attn_decode", "csl_hca_attn_decode", "csl_csa_decode_step", "csl_csa_decode_step_static",
    "csl_hca_decode_step",
]

_P, _I, _L, _F, _S = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class _CsaStep(ctypes.Structure):
    """csl_csa_step (include/csl.h), field for field."""
    _fields_ = [
        ("kv", _P), ("z", _P), ("kv_off", _P), ("ent_off", _P), ("first_entry", _P), ("max_new_entries", _L),
        ("ckv", _P),
        ("q_idx", _P), ("w", _P), ("k_idx", _P), ("k_dtype", _I), ("k_scale", _P), ("scale_off", _P),
        ("scale_group", _I), ("HI", _I), ("CI", _I), ("scores", _P), ("ld", _L), ("topk_ws", _P),
        ("topk_ws_bytes", _S),
        ("k", _I), ("idx", _P),
        ("q", _P), ("H", _I), ("D", _I), ("n_win", _I), ("scale", _F), ("out", _P), ("lse", _P), ("attn_ws", _P),
        ("attn_ws_bytes", _S),
        ("q_pos", _P), ("m", _I), ("B", _I), ("T", _I), ("max_entries", _L),
        ("kv_b", _P), ("z_b", _P),
        ("sink", _P), ("rope_dims", _I), ("rope_base", _F),
        ("paged", _P), ("scores_on_demand", _I),
    ]


class _HcaStep(ctypes.Structure):
    """csl_hca_step (include/csl.h), field for field."""
    _fields_ = [
        ("kv", _P), ("z", _P), ("kv_off", _P), ("ent_off", _P), ("first_entry", _P), ("max_new_entries", _L),
        ("ckv", _P),
        ("q", _P), ("H", _I), ("n_win", _I), ("scale", _F), ("out", _P), ("lse", _P), ("attn_ws", _P),
        ("attn_ws_bytes", _S),
        ("q_pos", _P), ("m", _I), ("B", _I), ("T", _I), ("max_entries", _L),
        ("sink", _P), ("rope_dims", _I), ("rope_base", _F),
        ("paged", _P),
    ]


class _PagedCache(ctypes.Structure):
    """csl_paged_cache (include/csl.h), field for field."""
    _fields_ = [("block_table", _P), ("max_blocks", _I), ("block_entries", _I), ("pool_entries", _L),
                ("ring_rows", _I)]


class _AttnExtras(ctypes.Structure):
    """csl_attn_extras (include/csl.h), field for field."""
    _fields_ = [("sink", _P), ("rope_dims", _I), ("rope_base", _F)]


class CslError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"csl status {status}: {msg}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python compressed_sparse_long_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, L, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "csl_last_error": (ctypes.c_char_p, []),
        "csl_version": (I, []),
        "csl_compress_kv": (I, [P, P, P, P, P, I, I, I, L, P, I, P, P]),
        "csl_compress_kv_overlap": (I, [P, P, P, P, P, P, P, I, I, I, L, P, I, P, P]),
        "csl_indexer_scores": (I, [P, P, P, I, P, P, I, P, P, I, I, I, I, I, L, P, L, P, S, I, P, P]),
        "csl_indexer_topk_max_k": (I, [I]),
        "csl_indexer_topk": (I, [P, P, P, I, P, P, I, P, P, I, I, I, I, I, L, I, P, P, P]),
        "csl_topk_workspace_bytes": (S, [I, I, L, I]),
        "csl_topk_select": (I, [P, L, P, P, I, I, I, I, L, P, P, S, I, P]),
        "csl_attn_workspace_bytes": (S, [I, I, I, I, L]),
        "csl_sparse_attn_decode": (I, [P, P, P, I, P, P, P, P, I, I, I, I, I, F, P, P, P, S,
                                       ctypes.POINTER(_AttnExtras), P, P]),
        "csl_hca_attn_decode": (I, [P, P, P, P, P, P, I, I, I, I, I, I, F, L, P, P, P, S,
                                    ctypes.POINTER(_AttnExtras), P, P]),
        "csl_csa_decode_step": (I, [ctypes.POINTER(_CsaStep), P]),
        "csl_csa_decode_step_static": (I, [ctypes.POINTER(_CsaStep), P]),
        "csl_hca_decode_step": (I, [ctypes.POINTER(_HcaStep), P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def version() -> int:
    return int(_lib.csl_version())


def _check(status: int) -> None:
    if status != 0:
        raise CslError(status, _lib.csl_last_error().decode())


def _ptr(t: torch.Tensor | None, name: str, dtypes=None) -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


class PagedCache:
    """Paged heterogeneous cache ([P2] "KV Cache Management"; csl_paged_cache in csl.h):
    ``block_table`` int32 [B, max_blocks] of pool blocks of ``block_entries`` entries each,
    ``pool_entries`` rows in the entry pool, raw rows in per-sequence rings of ``ring_rows``
    rows (0: packed)."""

    def __init__(self, block_table, block_entries: int, pool_entries: int, ring_rows: int = 0):
        self.block_table = block_table
        self.block_entries = int(block_entries)
        self.pool_entries = int(pool_entries)
        self.ring_rows = int(ring_rows)

    def _struct(self):
        bt = _ptr(self.block_table, "block_table", (torch.int32,))
        return _PagedCache(block_table=bt, max_blocks=int(self.block_table.shape[-1]),
                           block_entries=self.block_entries, pool_entries=self.pool_entries, ring_rows=self.ring_rows)


def _paged(paged):
    return None if paged is None else ctypes.byref(paged._struct())


_I64 = (torch.int64,)
_BF16 = (torch.bfloat16,)
_F32 = (torch.float32,)


def compress_kv(kv, z, kv_off, ent_off, m: int, out, first_entry=None, max_new_entries: int | None = None,
                paged=None, stream=None):
    """Softmax-weighted pooling of every m raw rows into out (fp32 or bf16 [*, D]); see csl.h."""
    B = kv_off.numel() - 1
    D = kv.shape[-1]
    dt = {torch.float32: F32, torch.bfloat16: BF16}.get(out.dtype)
    if dt is None:
        raise ValueError("out must be float32 or bfloat16")
    if max_new_entries is None:
        max_new_entries = out.shape[0]
    _check(_lib.csl_compress_kv(
        _ptr(kv, "kv", _BF16), _ptr(z, "z", _BF16), _ptr(kv_off, "kv_off", _I64), _ptr(ent_off, "ent_off", _I64),
        _ptr(first_entry, "first_entry", _I64), B, D, int(m), int(max_new_entries), _ptr(out, "out"), dt,
        _paged(paged), _stream(stream)))
    return out


def compress_kv_overlap(kv_a, z_a, kv_b, z_b, kv_off, ent_off, m: int, out, first_entry=None,
                        max_new_entries: int | None = None, paged=None, stream=None):
    """CSA's overlapped compression: entry i pools series-a rows [m*i, m*i + m) with series-b
    rows [m*(i-1), m*i) under one softmax per dimension, into out (fp32 or bf16 [*, D]); see csl.h."""
    B = kv_off.numel() - 1
    D = kv_a.shape[-1]
    dt = {torch.float32: F32, torch.bfloat16: BF16}.get(out.dtype)
    if dt is None:
        raise ValueError("out must be float32 or bfloat16")
    if kv_b.shape != kv_a.shape:
        raise ValueError("kv_a and kv_b must have the same shape")
    if max_new_entries is None:
        max_new_entries = out.shape[0]
    _check(_lib.csl_compress_kv_overlap(
        _ptr(kv_a, "kv_a", _BF16), _ptr(z_a, "z_a", _BF16), _ptr(kv_b, "kv_b", _BF16), _ptr(z_b, "z_b", _BF16),
        _ptr(kv_off, "kv_off", _I64), _ptr(ent_off, "ent_off", _I64), _ptr(first_entry, "first_entry", _I64),
        B, D, int(m), int(max_new_entries), _ptr(out, "out"), dt, _paged(paged), _stream(stream)))
    return out


def _key_format(kI, k_format):
    """C key dtype and the accepted k_scale dtypes for indexer keys ``kI``."""
    if k_format == "mxfp4":
        if kI.dtype != torch.uint8:
            raise ValueError("MXFP4 keys are packed uint8 codes [E, CI/2]")
        return MXFP4, (torch.uint8,)
    if kI.dtype == torch.bfloat16:
        return BF16, _F32
    if kI.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3, _F32
    raise ValueError("kI must be bfloat16, fp8 e4m3 (uint8 codes) or, with k_format='mxfp4', packed MXFP4")


def indexer_scores(qI, w, kI, ent_off, q_pos, m: int, scores, max_entries: int | None = None, k_scale=None,
                   scale_off=None, scale_group: int = 64, topk_ws=None, topk_k: int = 0, k_format=None,
                   paged=None, stream=None):
    """Lightning-indexer scores into scores fp32 [B, T, ld]; with ``topk_ws``/``topk_k`` it also
    leaves top-k candidate lists for ``topk_select(..., prepared=True)``. ``k_format='mxfp4'``
    takes packed E2M1 keys with their E8M0 scales in ``k_scale``; see csl.h."""
    B, T, HI, CI = qI.shape
    kd, sdt = _key_format(kI, k_format)
    ld = scores.shape[-1]
    if max_entries is None:
        max_entries = ld
    _check(_lib.csl_indexer_scores(
        _ptr(qI, "qI", _BF16), _ptr(w, "w", _F32), _ptr(kI, "kI"), kd, _ptr(k_scale, "k_scale", sdt),
        _ptr(scale_off, "scale_off", _I64), int(scale_group), _ptr(ent_off, "ent_off", _I64),
        _ptr(q_pos, "q_pos", _I64), int(m), B, T, HI, CI, int(max_entries), _ptr(scores, "scores", _F32), ld,
        _ptr(topk_ws, "topk_ws"), 0 if topk_ws is None else topk_ws.numel() * topk_ws.element_size(), int(topk_k),
        _paged(paged), _stream(stream)))
    return scores


def indexer_topk_max_k(HI: int) -> int:
    return int(_lib.csl_indexer_topk_max_k(int(HI)))


def indexer_topk(qI, w, kI, ent_off, q_pos, m: int, k: int, idx, max_entries: int, k_scale=None, scale_off=None,
                 scale_group: int = 64, k_format=None, paged=None, stream=None):
    """The indexer fused with top-k: ids of the k best visible entries per query row into
    idx int32 [B, T, k] (ascending, -1 padded) without writing scores; see csl.h."""
    B, T, HI, CI = qI.shape
    kd, sdt = _key_format(kI, k_format)
    _check(_lib.csl_indexer_topk(
        _ptr(qI, "qI", _BF16), _ptr(w, "w", _F32), _ptr(kI, "kI"), kd, _ptr(k_scale, "k_scale", sdt),
        _ptr(scale_off, "scale_off", _I64), int(scale_group), _ptr(ent_off, "ent_off", _I64),
        _ptr(q_pos, "q_pos", _I64), int(m), B, T, HI, CI, int(max_entries), int(k),
        _ptr(idx, "idx", (torch.int32,)), _paged(paged), _stream(stream)))
    return idx


def topk_workspace_bytes(B: int, T: int, max_entries: int, k: int) -> int:
    return int(_lib.csl_topk_workspace_bytes(B, T, max_entries, k))


def topk_select(scores, ent_off, q_pos, m: int, k: int, idx, ws=None, max_entries: int | None = None,
                prepared: bool = False, stream=None):
    """Top-k ids per row into idx int32 [B, T, k] (ascending, -1 padded). ``ws`` is a uint8
    device workspace (its contents do not matter); one is allocated if None and needed."""
    B, T, ld = scores.shape
    if max_entries is None:
        max_entries = ld
    need = topk_workspace_bytes(B, T, max_entries, k)
    if ws is None and need > 0:
        ws = torch.zeros(need, dtype=torch.uint8, device=scores.device)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.csl_topk_select(
        _ptr(scores, "scores", _F32), ld, _ptr(ent_off, "ent_off", _I64), _ptr(q_pos, "q_pos", _I64), int(m), B, T,
        int(k), int(max_entries), _ptr(idx, "idx", (torch.int32,)), _ptr(ws, "ws"), ws_bytes, int(bool(prepared)),
        _stream(stream)))
    return idx


def attn_workspace_bytes(B: int, T: int, H: int, D: int, max_keys: int) -> int:
    return int(_lib.csl_attn_workspace_bytes(B, T, H, D, max_keys))


def _attn_ws(ws, B, T, H, D, max_keys, device):
    need = attn_workspace_bytes(B, T, H, D, max_keys)
    if ws is None and need > 0:
        ws = torch.zeros(need, dtype=torch.uint8, device=device)
    return ws, (0 if ws is None else ws.numel() * ws.element_size())


def _extras(sink, rope_dims: int, rope_base: float):
    if sink is None and not rope_dims:
        return None
    return ctypes.byref(_AttnExtras(sink=_ptr(sink, "sink", _F32), rope_dims=int(rope_dims),
                                    rope_base=float(rope_base)))


def sparse_attn_decode(q, ckv, idx, kv, kv_off, ent_off, q_pos, n_win: int, out, lse=None, scale: float | None = None,
                       ws=None, sink=None, rope_dims: int = 0, rope_base: float = 10000.0, paged=None, stream=None):
    """CSA attention over the selected entries plus the raw window; ``sink`` (fp32 [H] logits)
    and ``rope_dims``/``rope_base`` (partial RoPE of q at p, of the output at -p) are the
    optional extras; see csl.h."""
    B, T, H, D = q.shape
    k = idx.shape[-1]
    if scale is None:
        scale = D ** -0.5
    ws, wb = _attn_ws(ws, B, T, H, D, k + n_win, q.device)
    _check(_lib.csl_sparse_attn_decode(
        _ptr(q, "q", _BF16), _ptr(ckv, "ckv", _BF16), _ptr(idx, "idx", (torch.int32,)), k, _ptr(kv, "kv", _BF16),
        _ptr(kv_off, "kv_off", _I64), _ptr(ent_off, "ent_off", _I64), _ptr(q_pos, "q_pos", _I64), int(n_win), B, T, H,
        D, float(scale), _ptr(out, "out", _F32), _ptr(lse, "lse", _F32), _ptr(ws, "ws"), wb,
        _extras(sink, rope_dims, rope_base), _paged(paged), _stream(stream)))
    return out


def hca_attn_decode(q, ckv, kv, kv_off, ent_off, q_pos, m: int, n_win: int, out, lse=None, scale: float | None = None,
                    max_entries: int | None = None, ws=None, sink=None, rope_dims: int = 0, rope_base: float = 10000.0,
                    paged=None, stream=None):
    """HCA dense attention over every visible entry plus the raw window, with the same
    optional extras as sparse_attn_decode; see csl.h."""
    B, T, H, D = q.shape
    if scale is None:
        scale = D ** -0.5
    if max_entries is None:
        max_entries = ckv.shape[0]
    ws, wb = _attn_ws(ws, B, T, H, D, max_entries + n_win, q.device)
    _check(_lib.csl_hca_attn_decode(
        _ptr(q, "q", _BF16), _ptr(ckv, "ckv", _BF16), _ptr(kv, "kv", _BF16), _ptr(kv_off, "kv_off", _I64),
        _ptr(ent_off, "ent_off", _I64), _ptr(q_pos, "q_pos", _I64), int(m), int(n_win), B, T, H, D, float(scale),
        int(max_entries), _ptr(out, "out", _F32), _ptr(lse, "lse", _F32), _ptr(ws, "ws"), wb,
        _extras(sink, rope_dims, rope_base), _paged(paged), _stream(stream)))
    return out


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def csa_decode_step(kv, z, kv_off, ent_off, first_entry, max_new_entries: int, ckv, qI, w, kI, scores, topk_ws,
                    k: int, idx, q, n_win: int, out, q_pos, m: int, lse=None, scale: float | None = None,
                    k_scale=None, scale_off=None, scale_group: int = 64, max_entries: int | None = None,
                    attn_ws=None, kv_b=None, z_b=None, sink=None, rope_dims: int = 0, rope_base: float = 10000.0,
                    k_format=None, paged=None, stream=None, static_scratch: bool = False,
                    scores_on_demand: bool = False):
    """One whole CSA step (compress_kv of the newest entries into ckv, or compress_kv_overlap
    when series b ``kv_b``/``z_b`` is given, indexer_scores with candidate lists, topk_select,
    sparse_attn_decode) in one C call; with ``scores`` None the selection comes from the
    indexer fused with top-k and no score matrix is written; ``scores_on_demand``: rows
    selected from candidate lists keep no scores (see csl.h)."""
    B, T, HI, CI = qI.shape
    H, D = q.shape[2], q.shape[3]
    kd, sdt = _key_format(kI, k_format)
    ld = scores.shape[-1] if scores is not None else 0  # None: the indexer fused with top-k
    if max_entries is None:
        if scores is None:
            raise ValueError("csa_decode_step: max_entries is required without a score buffer")
        max_entries = ld
    if scale is None:
        scale = D ** -0.5
    if static_scratch:  # the library's own scratch array replaces both workspaces
        attn_ws, awb, topk_ws = None, 0, None
    else:
        attn_ws, awb = _attn_ws(attn_ws, B, T, H, D, k + n_win, q.device)
    pstruct = None if paged is None else paged._struct()  # kept alive across the call
    s = _CsaStep(
        kv=_ptr(kv, "kv", _BF16), z=_ptr(z, "z", _BF16), kv_off=_ptr(kv_off, "kv_off", _I64),
        ent_off=_ptr(ent_off, "ent_off", _I64), first_entry=_ptr(first_entry, "first_entry", _I64),
        max_new_entries=int(max_new_entries), ckv=_ptr(ckv, "ckv", _BF16),
        q_idx=_ptr(qI, "qI", _BF16), w=_ptr(w, "w", _F32), k_idx=_ptr(kI, "kI"), k_dtype=kd,
        k_scale=_ptr(k_scale, "k_scale", sdt), scale_off=_ptr(scale_off, "scale_off", _I64),
        scale_group=int(scale_group), HI=HI, CI=CI, scores=_ptr(scores, "scores", _F32), ld=ld,
        topk_ws=_ptr(topk_ws, "topk_ws"), topk_ws_bytes=_nbytes(topk_ws),
        k=int(k), idx=_ptr(idx, "idx", (torch.int32,)),
        q=_ptr(q, "q", _BF16), H=H, D=D, n_win=int(n_win), scale=float(scale), out=_ptr(out, "out", _F32),
        lse=_ptr(lse, "lse", _F32), attn_ws=_ptr(attn_ws, "attn_ws"), attn_ws_bytes=awb,
        kv_b=_ptr(kv_b, "kv_b", _BF16), z_b=_ptr(z_b, "z_b", _BF16),
        sink=_ptr(sink, "sink", _F32), rope_dims=int(rope_dims), rope_base=float(rope_base),
        paged=None if paged is None else ctypes.addressof(pstruct),
        q_pos=_ptr(q_pos, "q_pos", _I64), m=int(m), B=B, T=T, max_entries=int(max_entries),
        scores_on_demand=int(bool(scores_on_demand)))
    fn = _lib.csl_csa_decode_step_static if static_scratch else _lib.csl_csa_decode_step
    _check(fn(ctypes.byref(s), _stream(stream)))
    return out


def hca_decode_step(kv, z, kv_off, ent_off, first_entry, max_new_entries: int, ckv, q, n_win: int, out, q_pos,
                    m: int, max_entries: int, lse=None, scale: float | None = None, attn_ws=None, sink=None,
                    rope_dims: int = 0, rope_base: float = 10000.0, paged=None, stream=None):
    """One whole HCA step (compress_kv of the newest entries into ckv, then hca_attn_decode) in
    one C call, the compression riding in the attention launch where the head count allows;
    see csl.h."""
    B, T, H, D = q.shape
    if scale is None:
        scale = D ** -0.5
    attn_ws, awb = _attn_ws(attn_ws, B, T, H, D, max_entries + n_win, q.device)
    pstruct = None if paged is None else paged._struct()  # kept alive across the call
    s = _HcaStep(
        kv=_ptr(kv, "kv", _BF16), z=_ptr(z, "z", _BF16), kv_off=_ptr(kv_off, "kv_off", _I64),
        ent_off=_ptr(ent_off, "ent_off", _I64), first_entry=_ptr(first_entry, "first_entry", _I64),
        max_new_entries=int(max_new_entries), ckv=_ptr(ckv, "ckv", _BF16),
        q=_ptr(q, "q", _BF16), H=H, n_win=int(n_win), scale=float(scale), out=_ptr(out, "out", _F32),
        lse=_ptr(lse, "lse", _F32), attn_ws=_ptr(attn_ws, "attn_ws"), attn_ws_bytes=awb,
        q_pos=_ptr(q_pos, "q_pos", _I64), m=int(m), B=B, T=T, max_entries=int(max_entries),
        sink=_ptr(sink, "sink", _F32), rope_dims=int(rope_dims), rope_base=float(rope_base),
        paged=None if paged is None else ctypes.addressof(pstruct))
    if D != 128:
        raise ValueError("hca_decode_step: head dim must be 128")
    _check(_lib.csl_hca_decode_step(ctypes.byref(s), _stream(stream)))
    return out


def csa_decode_step_static(kv, z, kv_off, ent_off, first_entry, max_new_entries: int, ckv, qI, w, kI, scores,
                           k: int, idx, q, n_win: int, out, q_pos, m: int, **kw):
    """csa_decode_step without caller workspaces: csl_csa_decode_step_static takes them from
    the library's per-device scratch array (no device allocation anywhere in the call; calls
    overlapping on one device race); see csl.h."""
    kw.pop("topk_ws", None)
    kw.pop("attn_ws", None)
    return csa_decode_step(kv, z, kv_off, ent_off, first_entry, max_new_entries, ckv, qI, w, kI, scores, None, k,
                           idx, q, n_win, out, q_pos, m, static_scratch=True, **kw)
