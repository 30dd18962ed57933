"""The C-ABI library without a GPU: it loads, exports every declared symbol, and rejects bad
host arguments before enqueuing anything (no compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csl.h")
LIB = os.path.join(ROOT, "compressed_sparse_long_amd", "libcsl.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        # build.py by path: importing the package would try to load the missing library
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_csl_build", os.path.join(ROOT, "compressed_sparse_long_amd", "build.py"))
        b = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(b)
        b.build()
    return ctypes.CDLL(LIB)


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csl_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_five_stages():
    syms = declared_symbols()
    for s in ("csl_compress_kv", "csl_indexer_scores", "csl_topk_select", "csl_sparse_attn_decode",
              "csl_hca_attn_decode"):
        assert s in syms


def test_library_exports_every_declared_symbol(lib):
    for s in declared_symbols():
        assert hasattr(lib, s), s
    import compressed_sparse_long_amd as csl
    assert sorted(csl.EXPORTS) == declared_symbols()
    assert csl.version() == 500


P = ctypes.c_void_p
FAKE = P(1 << 20)  # never dereferenced: every call below fails host validation first


def _err(lib):
    lib.csl_last_error.restype = ctypes.c_char_p
    return lib.csl_last_error().decode()


def test_compress_validation(lib):
    f = lib.csl_compress_kv
    f.argtypes = [P, P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64, P, ctypes.c_int, P, P]
    assert f(None, None, FAKE, FAKE, None, 1, 128, 4, 10, FAKE, 1, None, None) == 1
    assert "null" in _err(lib)
    assert f(FAKE, None, FAKE, FAKE, None, 1, 96, 4, 10, FAKE, 1, None, None) == 2
    assert f(FAKE, None, FAKE, FAKE, None, 1, 128, 0, 10, FAKE, 1, None, None) == 1
    assert f(FAKE, None, FAKE, FAKE, None, 1, 128, 4, 10, FAKE, 2, None, None) == 2
    assert f(FAKE, None, FAKE, FAKE, None, -1, 128, 4, 10, FAKE, 1, None, None) == 1
    assert f(P((1 << 20) + 2), None, FAKE, FAKE, None, 1, 128, 4, 10, FAKE, 1, None, None) == 1
    assert "aligned" in _err(lib)
    # nothing to do is a success without touching the device
    assert f(FAKE, None, FAKE, FAKE, None, 0, 128, 4, 10, FAKE, 1, None, None) == 0
    assert _err(lib) == ""


def test_compress_overlap_validation(lib):
    f = lib.csl_compress_kv_overlap
    f.argtypes = [P, P, P, P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64, P, ctypes.c_int, P, P]
    # kv_a, z_a, kv_b, z_b, kv_off, ent_off, first, B, D, m, max_new, out, dtype, stream
    assert f(FAKE, None, None, None, FAKE, FAKE, None, 1, 128, 4, 10, FAKE, 1, None, None) == 1
    assert "kv_b" in _err(lib)
    assert f(FAKE, FAKE, FAKE, None, FAKE, FAKE, None, 1, 128, 4, 10, FAKE, 1, None, None) == 1
    assert "both" in _err(lib)
    assert f(FAKE, None, FAKE, FAKE, FAKE, FAKE, None, 1, 128, 4, 10, FAKE, 1, None, None) == 1
    assert f(FAKE, None, P((1 << 20) + 8), None, FAKE, FAKE, None, 1, 128, 4, 10, FAKE, 1, None, None) == 1
    assert "aligned" in _err(lib)
    assert f(FAKE, None, FAKE, None, FAKE, FAKE, None, 1, 96, 4, 10, FAKE, 1, None, None) == 2
    assert _err(lib).startswith("compress_kv_overlap:")
    assert f(FAKE, None, FAKE, None, FAKE, FAKE, None, 1, 128, 70000, 10, FAKE, 1, None, None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 128, 4, 10, FAKE, 0, None, None) == 0
    assert _err(lib) == ""


def test_indexer_validation(lib):
    f = lib.csl_indexer_scores
    I, L = ctypes.c_int, ctypes.c_int64
    f.argtypes = [P, P, P, I, P, P, I, P, P, I, I, I, I, I, L, P, L, P, ctypes.c_size_t, I, P, P]
    args = [FAKE, FAKE, FAKE, 0, None, None, 64, FAKE, FAKE, 4, 1, 1, 8, 64, 1000, FAKE, 1000, None, 0, 0, None, None]
    bad = list(args); bad[12] = 3
    assert f(*bad) == 2                       # HI
    bad = list(args); bad[13] = 128
    assert f(*bad) == 2                       # CI
    bad = list(args); bad[3] = 2
    assert f(*bad) == 1                       # fp8 without scales
    bad = list(args); bad[16] = 999
    assert f(*bad) == 1                       # ld < max_entries
    bad = list(args); bad[1] = None
    assert f(*bad) == 1
    ok0 = list(args); ok0[11] = 0
    assert f(*ok0) == 0                       # T = 0: nothing to do
    long_rows = list(args); long_rows[14] = 262144; long_rows[16] = 262144
    bad = list(long_rows); bad[17] = FAKE; bad[18] = 100; bad[19] = 1024
    assert f(*bad) == 3                       # top-k workspace too small
    bad = list(long_rows); bad[17] = FAKE; bad[18] = 1 << 30; bad[19] = 0
    assert f(*bad) == 2                       # topk_k out of range
    # fp8 keys in a paged cache: scales per pool block (scale_off unused), power-of-two groups
    import compressed_sparse_long_amd as csl
    pc = csl._PagedCache(FAKE, 8, 32, 1 << 20, 0)
    fp8 = list(args); fp8[3] = 2; fp8[4] = FAKE; fp8[11] = 0; fp8[20] = P(ctypes.addressof(pc))
    assert f(*fp8) == 0, _err(lib)            # scale_off NULL accepted (T = 0: nothing enqueued)
    bad = list(fp8); bad[6] = 48
    assert f(*bad) == 1 and "power-of-two scale_group" in _err(lib)
    bad = list(fp8); bad[20] = None
    assert f(*bad) == 1 and "scale_off" in _err(lib)   # packed: scale_off is needed


def test_topk_validation_and_workspace(lib):
    ws = lib.csl_topk_workspace_bytes
    ws.restype = ctypes.c_size_t
    ws.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int]
    assert ws(1, 1, 1024, 64) == 0            # short rows: one workgroup per row, no workspace
    assert ws(1, 8192, 34816, 512) == 0
    big = ws(4, 1, 262144, 1024)
    assert big > 4 * (2048 * 4 + 1024 * 4)
    f = lib.csl_topk_select
    I, L = ctypes.c_int, ctypes.c_int64
    f.argtypes = [P, L, P, P, I, I, I, I, L, P, P, ctypes.c_size_t, I, P]
    assert f(FAKE, 262144, FAKE, FAKE, 4, 4, 1, 1024, 262144, FAKE, FAKE, big - 1, 0, None) == 3
    assert "workspace" in _err(lib)
    assert f(FAKE, 262144, FAKE, FAKE, 4, 4, 1, 1024, 262144, FAKE, None, 0, 1, None) == 3
    assert f(FAKE, 1024, FAKE, FAKE, 4, 1, 1, 0, 1024, FAKE, None, 0, 0, None) == 2      # k = 0
    assert f(FAKE, 1024, FAKE, FAKE, 4, 1, 1, 5000, 1024, FAKE, None, 0, 0, None) == 2   # k too large
    assert f(FAKE, 100, FAKE, FAKE, 4, 1, 1, 64, 1024, FAKE, None, 0, 0, None) == 1      # ld < max_entries


def test_attention_validation_and_workspace(lib):
    ws = lib.csl_attn_workspace_bytes
    ws.restype = ctypes.c_size_t
    ws.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64]
    assert ws(1, 8192, 64, 128, 640) == 0     # many rows: one split per row
    w3 = ws(4, 1, 64, 128, 1024 + 128)
    # whole (o, lse) partials of 4 rows x 64 heads per split, plus one RoPE table per row
    assert w3 > 0 and (w3 - 4 * 32 * 8) % (4 * 64 * 129 * 4) == 0
    f = lib.csl_sparse_attn_decode
    I = ctypes.c_int
    import compressed_sparse_long_amd as csl
    EX = ctypes.POINTER(csl._AttnExtras)
    f.argtypes = [P, P, P, I, P, P, P, P, I, I, I, I, I, ctypes.c_float, P, P, P, ctypes.c_size_t, EX, P, P]
    base = [FAKE, FAKE, FAKE, 1024, FAKE, FAKE, FAKE, FAKE, 128, 4, 1, 64, 128, 0.088, FAKE, None, FAKE, w3, None, None,
            None]
    bad = list(base); bad[12] = 64
    assert f(*bad) == 2                       # D
    bad = list(base); bad[11] = 24
    assert f(*bad) == 2                       # H not a multiple of 16
    bad = list(base); bad[17] = w3 - 4
    assert f(*bad) == 3
    bad = list(base); bad[2] = None
    assert f(*bad) == 1
    bad = list(base); bad[13] = float("nan")
    assert f(*bad) == 1
    # attention extras: RoPE width and base, sink alignment
    for ex, status in (((None, 48, 10000.0), 2), ((None, -32, 10000.0), 1), ((None, 64, 1.0), 1),
                       ((None, 64, float("nan")), 1), ((P((1 << 20) + 2), 0, 0.0), 1), ((None, 128, 10000.0), 2),
                       ((None, 32, 10000.0), 2)):
        bad = list(base); bad[18] = ctypes.pointer(csl._AttnExtras(*ex))
        assert f(*bad) == status, ex
    assert "rope" in _err(lib) or "sink" in _err(lib)
    g = lib.csl_hca_attn_decode
    L = ctypes.c_int64
    g.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, ctypes.c_float, L, P, P, P, ctypes.c_size_t, EX, P, P]
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 128, 8, 1, 64, 128, 0.088, 1024, FAKE, None, FAKE, 0, None,
             None, None) == 1
    ex = ctypes.pointer(csl._AttnExtras(None, 64, 0.5))
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 128, 128, 8, 1, 64, 128, 0.088, 1024, FAKE, None, FAKE, 1 << 30, ex,
             None, None) == 1
    assert "rope_base" in _err(lib)
    # paged cache descriptor: block size, ring size, id scratch
    PC = csl._PagedCache
    for pc, status in ((PC(None, 4, 32, 1 << 20, 128), 1),          # no table
                       (PC(FAKE, 4, 24, 1 << 20, 128), 1),          # block_entries not a power of two
                       (PC(FAKE, 4, 32, 1 << 20, 96), 1),           # ring not a power of two
                       (PC(FAKE, 4, 32, 1 << 20, 64), 1),           # ring smaller than the window
                       (PC(FAKE, 0, 32, 1 << 20, 128), 1)):         # no blocks
        bad = list(base); bad[19] = P(ctypes.addressof(pc))
        assert f(*bad) == status, _err(lib)
    # the ring must hold the windows of all T query rows: n_win + T - 1 rows
    for T, ring, ok in ((1, 128, True), (2, 128, False), (129, 256, True), (130, 256, False)):
        pc = PC(FAKE, 4, 32, 1 << 20, ring)
        args = list(base); args[10] = T; args[17] = 1 << 30; args[19] = P(ctypes.addressof(pc))
        st = f(*args)
        if ok:
            assert st != 1, _err(lib)       # validation passes (without a GPU the launch itself fails)
        else:
            assert st == 1 and "ring_rows" in _err(lib), (T, ring, _err(lib))
    # ring_rows = 0: the raw rows stay packed, so no ring size applies
    pc = PC(FAKE, 4, 32, 1 << 20, 0)
    args = list(base); args[19] = P(ctypes.addressof(pc))
    assert f(*args) != 1 and "ring" not in _err(lib)
    # scale must be positive: the softmax takes the running maximum of scaled logits
    for sc in (0.0, -0.088, float("inf")):
        bad = list(base); bad[13] = sc
        assert f(*bad) == 1 and "scale" in _err(lib)
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 128, 128, 8, 1, 64, 128, 0.0, 1024, FAKE, None, FAKE, 1 << 30, None,
             None, None) == 1 and "scale" in _err(lib)


def test_step_validation(lib):
    import compressed_sparse_long_amd as csl
    f = lib.csl_csa_decode_step
    f.argtypes = [ctypes.POINTER(csl._CsaStep), P]
    f.restype = ctypes.c_int
    assert f(None, None) == 1
    base = dict(kv=FAKE, kv_off=FAKE, ent_off=FAKE, max_new_entries=1, ckv=FAKE, q_idx=FAKE, w=FAKE, k_idx=FAKE,
                k_dtype=0, scale_group=64, HI=8, CI=64, scores=FAKE, ld=1000, k=64, idx=FAKE, q=FAKE, H=64, D=128,
                n_win=128, scale=0.088, out=FAKE, q_pos=FAKE, m=4, B=1, T=1, max_entries=1000)

    def call(**over):
        s = csl._CsaStep(**{**base, **over})
        return f(ctypes.byref(s), None)
    assert call(HI=3) == 2                      # indexer heads
    assert call(D=64) == 2                      # attention needs D = 128
    assert call(idx=None) == 1
    assert call(ld=999) == 1                    # ld < max_entries
    assert call(k=0) == 2
    assert call(kv=P((1 << 20) + 2)) == 1       # misaligned raw cache
    assert call(m=0) == 1
    assert call(z_b=FAKE) == 1                  # series-b logits without series b
    assert "kv_b" in _err(lib)
    assert call(kv_b=FAKE, z_b=FAKE) == 1       # series-b logits without series-a logits
    assert "z_b" in _err(lib)
    assert call(kv_b=P((1 << 20) + 4)) == 1     # misaligned series b
    assert call(rope_dims=64, rope_base=0.5) == 1   # RoPE base <= 1
    assert call(rope_dims=40, rope_base=1e4) == 2   # RoPE width not a multiple of 32
    assert call(B=0) == 0                       # nothing to do: nothing enqueued
    assert _err(lib) == ""
    # scores on demand is a mode of the same call: validated alike, still needing a score buffer
    assert call(scores_on_demand=1, B=0) == 0
    assert call(scores_on_demand=1, idx=None) == 1
    assert call(scores_on_demand=1, HI=3) == 2
    assert ctypes.sizeof(csl._CsaStep) == csl._CsaStep.scores_on_demand.offset + 8  # the last field, padded
    # without a score buffer: the fused indexer/top-k's limit on k applies instead
    assert call(scores=None, k=1953) == 2
    assert "without scores" in _err(lib)
    assert call(scores=None, idx=None) == 1
    assert call(scores=None, ld=0, B=0) == 0    # ld is ignored without scores
    assert _err(lib) == ""
    # a paged cache: the ring holds the union of the window and the newest compressed chunks
    PC = csl._PagedCache
    def paged_call(ring, **over):
        pc = PC(FAKE, 8, 32, 1 << 20, ring)
        return call(paged=P(ctypes.addressof(pc)), B=0, **over)
    assert paged_call(128) == 0                          # window 128 >= (1 + 1) * 4 - 1 = 7
    assert paged_call(0) == 0                            # raw rows packed: no ring to size
    assert paged_call(64) == 1 and "ring_rows" in _err(lib)        # the window does not fit
    assert paged_call(128, max_new_entries=31) == 0      # (31 + 1) * 4 - 1 = 127 <= 128
    assert paged_call(128, max_new_entries=32) == 1      # (32 + 1) * 4 - 1 = 131 > 128
    assert paged_call(256, max_new_entries=32) == 0
    assert paged_call(128, n_win=0, m=128) == 1          # one HCA chunk plus its tail: 2 * 128 - 1 = 255
    assert paged_call(256, n_win=0, m=128) == 0
    assert paged_call(256, T=129) == 0                   # windows of 129 rows: 128 + 129 - 1 = 256
    assert paged_call(256, T=130) == 1                   # 130 rows: 257 > 256
    # overlapped compression also reads the series-b block before each entry: one more chunk
    assert paged_call(128, kv_b=FAKE, max_new_entries=30) == 0     # (30 + 2) * 4 - 1 = 127
    assert paged_call(128, kv_b=FAKE, max_new_entries=31) == 1     # (31 + 2) * 4 - 1 = 131
    # fp8 indexer keys in the pool: group scales per block, so the group must be a power of two
    assert paged_call(128, k_dtype=2, k_scale=FAKE, scale_group=64) == 0
    assert paged_call(128, k_dtype=2, k_scale=FAKE, scale_group=16, scores=None, ld=0) == 0
    assert paged_call(128, k_dtype=2, k_scale=FAKE, scale_group=96) == 1 and "power-of-two" in _err(lib)
    assert call(k_dtype=2, k_scale=FAKE, B=0) == 1 and "scale_off" in _err(lib)  # packed: scale_off needed


def test_hca_step_validation(lib):
    import compressed_sparse_long_amd as csl
    f = lib.csl_hca_decode_step
    f.argtypes = [ctypes.POINTER(csl._HcaStep), P]
    f.restype = ctypes.c_int
    assert f(None, None) == 1
    base = dict(kv=FAKE, kv_off=FAKE, ent_off=FAKE, max_new_entries=1, ckv=FAKE, q=FAKE, H=64, n_win=128,
                scale=0.088, out=FAKE, attn_ws=FAKE, attn_ws_bytes=1 << 30, q_pos=FAKE, m=128, B=8, T=1,
                max_entries=1024)

    def call(**over):
        s = csl._HcaStep(**{**base, **over})
        return f(ctypes.byref(s), None)
    assert call(m=0) == 1                          # compression ratio
    assert call(H=24) == 2                         # heads not a multiple of 16
    assert call(ckv=None) == 1
    assert call(kv=P((1 << 20) + 2)) == 1          # misaligned raw rows
    assert call(scale=0.0) == 1 and "scale" in _err(lib)
    assert call(max_entries=-1) == 1
    assert call(rope_dims=64, rope_base=0.5) == 1
    assert call(attn_ws=None, attn_ws_bytes=0) == 3  # 9 splits need a workspace
    assert call(B=0) == 0 and _err(lib) == ""      # nothing to do
    # a paged cache: the ring holds the window and the chunk being compressed (2m - 1 rows)
    pc = csl._PagedCache(FAKE, 8, 1, 1 << 20, 128)
    assert call(paged=P(ctypes.addressof(pc)), B=0) == 1 and "ring_rows" in _err(lib)
    pc = csl._PagedCache(FAKE, 8, 1, 1 << 20, 256)
    assert call(paged=P(ctypes.addressof(pc)), B=0) == 0


def test_static_step_rejects_workspaces_beyond_its_scratch(lib):
    """csl_csa_decode_step_static sizes the step's workspaces on the host and refuses, before
    touching a device, a step that needs more than its static scratch array."""
    import compressed_sparse_long_amd as csl
    f = lib.csl_csa_decode_step_static
    f.argtypes = [ctypes.POINTER(csl._CsaStep), P]
    f.restype = ctypes.c_int
    assert f(None, None) == 1
    m = re.search(r"#define CSL_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    limit = int(m.group(1)) << int(m.group(2))
    base = dict(kv=FAKE, kv_off=FAKE, ent_off=FAKE, max_new_entries=1, ckv=FAKE, q_idx=FAKE, w=FAKE, k_idx=FAKE,
                k_dtype=0, scale_group=64, HI=8, CI=64, scores=FAKE, ld=262144, k=1024, idx=FAKE, q=FAKE, H=64,
                D=128, n_win=128, scale=0.088, out=FAKE, q_pos=FAKE, m=4, B=300, T=1, max_entries=262144)
    # 300 rows of 262144 entries: 300 candidate-list workspaces of ~66 KiB, more than the array
    need = lib.csl_topk_workspace_bytes
    need.restype, need.argtypes = ctypes.c_size_t, [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int]
    assert need(300, 1, 262144, 1024) > limit
    s = csl._CsaStep(**base)
    assert f(ctypes.byref(s), None) == 3 and "static scratch" in _err(lib)


def test_indexer_topk_validation(lib):
    f = lib.csl_indexer_topk
    I, L = ctypes.c_int, ctypes.c_int64
    f.argtypes = [P, P, P, I, P, P, I, P, P, I, I, I, I, I, L, I, P, P, P]
    mk = lib.csl_indexer_topk_max_k
    mk.argtypes = [I]
    # a cut must leave room for a 256-key chunk: 2240 - 288 slots with one workgroup per CU (HI = 2,
    # 4, 8 beyond k = 672, and HI = 16); HI = 1 keeps its 960-slot buffer: 672
    assert mk(8) == 1952 and mk(4) == 1952 and mk(2) == 1952 and mk(1) == 672 and mk(16) == 1952 and mk(3) == 0

    def call(idx=FAKE, k=64, HI=8, CI=64, B=1, T=16, me=1000, kd=0, ks=None, m=4):
        # q_idx, w, k_idx, k_dtype, k_scale, scale_off, group, ent_off, q_pos, m, B, T, HI, CI, max_entries, k, idx
        return f(FAKE, FAKE, FAKE, kd, ks, None, 64, FAKE, FAKE, m, B, T, HI, CI, me, k, idx, None, None)

    assert call(idx=None) == 1 and "null" in _err(lib)
    assert call(k=0) == 2 and "k must be in" in _err(lib)
    assert call(k=1953) == 2 and "k must be in" in _err(lib)
    assert call(k=673, HI=1) == 2 and "k must be in" in _err(lib)
    assert call(HI=3) == 2 and "HI" in _err(lib)
    assert call(CI=32) == 2 and "CI" in _err(lib)
    assert call(m=0) == 1
    assert call(B=-1) == 1
    assert call(kd=3) == 1 and "MXFP4" in _err(lib)          # MXFP4 keys need their scales
    assert call(me=1 << 31) == 2 and "max_entries" in _err(lib)
    assert call(idx=P((1 << 20) + 2)) == 1 and "aligned" in _err(lib)
    # nothing to do is a success without touching the device
    assert call(T=0) == 0 and _err(lib) == ""
