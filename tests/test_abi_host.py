"""The C ABI on the host: the library loads, exports every declared entry point,
and rejects every invalid request before any HIP call (so no GPU is needed).

Pointers passed here are fake, 16-byte-aligned addresses: each call below must
fail validation, which happens before anything is enqueued.
"""
import ctypes
import glob
import os
import re

import pytest

import sparse_attention_indexer_lightning_amd as sa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "idxcache.h")
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP, WS, PATTERN, SCRATCH = 0, -1, -2, -3, -4, -5, -6, -7, -9
BF16, FP8, FP32 = 1, 2, 3
FAKE = ctypes.c_void_p(0x10000)       # never dereferenced: validation fails first
FAKE_ODD = ctypes.c_void_p(0x10008)   # 8-byte aligned only


def declared_functions():
    names = set()
    for h in HEADERS:
        src = open(h).read()
        names |= set(re.findall(r"^(?:idxc_status|const char \*|int)\s+(\w+)\s*\(", src, re.M))
    return sorted(names)


def test_every_declared_symbol_is_exported():
    L = sa.lib()
    names = declared_functions()
    assert {"idx_score_topk", "idx_topk", "idx_cache_route", "sparse_mla_attn", "idxc_calib_mfma_rate",
            "idxc_calib_gather_rate"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert L.idxc_abi_version() == 1


def test_status_strings():
    L = sa.lib()
    for code in range(-9, 1):
        assert L.idxc_status_str(code)
    assert L.idxc_status_str(5) == b"unknown status"


def desc(B=1, Lq=128, Lk=128, H=64, D=128, topk=64, qd=FP8, kd=FP8, wd=BF16):
    return sa._IndexerDesc(B, Lq, Lk, H, D, topk, qd, kd, wd)


def score(d, q=FAKE, k=FAKE, w=FAKE, t=FAKE, dbg=None, ws=None, wsb=0):
    return sa.lib().idx_score_topk(ctypes.byref(d) if d is not None else None, q, k, w, t, dbg, ws, wsb, None)


def ws_bytes(d):
    n = ctypes.c_size_t(0)
    st = sa.lib().idx_score_topk_workspace(ctypes.byref(d), ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,code", [
    (dict(qd=9), DTYPE), (dict(wd=0), DTYPE),
    (dict(qd=FP8, kd=BF16), DTYPE), (dict(qd=BF16, kd=BF16, wd=BF16), DTYPE),
    (dict(qd=FP8, kd=FP8, wd=FP32), DTYPE),
    (dict(B=0), SHAPE), (dict(Lq=0), SHAPE), (dict(Lq=200, Lk=100), SHAPE), (dict(H=0), SHAPE),
    (dict(topk=0), SHAPE), (dict(Lk=1 << 24, Lq=1), SHAPE),
    (dict(H=12), UNSUP), (dict(H=128), UNSUP), (dict(topk=2049), UNSUP), (dict(D=64), UNSUP),
    (dict(qd=BF16, kd=BF16, wd=FP32, D=48), UNSUP),
])
def test_indexer_descriptor_rejections(kw, code):
    d = desc(**kw)
    assert score(d) == code
    assert ws_bytes(d)[0] == code


def test_indexer_pointer_and_alignment_rejections():
    d = desc()
    assert score(None) == NULL
    assert score(d, q=None) == NULL
    assert score(d, k=None) == NULL
    assert score(d, w=None) == NULL
    assert score(d, t=None) == NULL
    assert score(d, q=FAKE_ODD) == ALIGN
    assert score(d, k=FAKE_ODD) == ALIGN
    assert score(d, t=FAKE_ODD) == ALIGN
    assert score(d, dbg=FAKE_ODD) == ALIGN
    assert score(d, w=ctypes.c_void_p(0x10002)) == ALIGN


def test_workspace_sizes_and_rejections():
    # prefill-shaped: fused kernel, no workspace
    assert ws_bytes(desc(Lq=8192, Lk=8192, topk=2048)) == (OK, 0)
    assert ws_bytes(desc(Lq=65536, Lk=65536, topk=2048)) == (OK, 0)
    # decode-shaped: one fp32 score row per query (256-byte aligned), then the
    # split row top-k's own workspace
    d = desc(B=32, Lq=1, Lk=200000, topk=2048)
    st, n = ws_bytes(d)
    scores_b = (32 * 200000 * 4 + 255) // 256 * 256
    assert st == OK and n == scores_b + sa.idx_topk_workspace(32, 200000, 2048)
    assert sa.idx_topk_workspace(32, 200000, 2048) >= 32 * 200000 * 8   # (key, index) per score
    assert sa.idx_topk_workspace(4096, 2048, 64) == 0                     # many short rows: not split
    assert score(d) == WS
    assert score(d, ws=FAKE, wsb=n - 1) == WS
    assert score(d, ws=FAKE_ODD, wsb=n) == ALIGN
    # small head counts need more query rows per workgroup than LDS holds at large k
    assert ws_bytes(desc(qd=BF16, kd=BF16, wd=FP32, H=4, D=32, topk=2048, Lq=4096, Lk=4096))[0] == UNSUP
    assert ws_bytes(desc(qd=BF16, kd=BF16, wd=FP32, H=4, D=32, topk=64, Lq=512, Lk=512)) == (OK, 0)


def test_topk_rejections():
    L = sa.lib()
    assert L.idx_topk(FAKE, None, 4, 0, 8, FAKE, None, 0, None) == SHAPE
    assert L.idx_topk(FAKE, None, -1, 10, 8, FAKE, None, 0, None) == SHAPE
    assert L.idx_topk(FAKE, None, 4, 10, 0, FAKE, None, 0, None) == SHAPE
    assert L.idx_topk(FAKE, None, 4, 10, 4096, FAKE, None, 0, None) == UNSUP
    assert L.idx_topk(None, None, 4, 10, 8, FAKE, None, 0, None) == NULL
    # split rows need their workspace
    need = sa.idx_topk_workspace(8, 100000, 2048)
    assert need > 0
    assert L.idx_topk(FAKE, None, 8, 100000, 2048, FAKE, None, 0, None) == WS
    assert L.idx_topk(FAKE, None, 8, 100000, 2048, FAKE, FAKE, need - 1, None) == WS
    assert L.idx_topk(FAKE, None, 8, 100000, 2048, FAKE, FAKE_ODD, need, None) == ALIGN
    assert L.idx_topk(FAKE, None, 4, 10, 8, None, None, 0, None) == NULL
    assert L.idx_topk(ctypes.c_void_p(0x10001), None, 4, 10, 8, FAKE, None, 0, None) == ALIGN
    assert L.idx_topk(FAKE, None, 0, 10, 8, FAKE, None, 0, None) == OK  # nothing to do
    n = ctypes.c_size_t(7)
    assert L.idx_topk_workspace(4, 10, 8, ctypes.byref(n)) == OK and n.value == 0


def route(pattern, layer, d=None, q=FAKE, k=FAKE, w=FAKE, t=FAKE):
    c = ctypes.c_int(-1)
    st = sa.lib().idx_cache_route(pattern, layer, ctypes.byref(d) if d is not None else None,
                                  q, k, w, t, None, 0, None, ctypes.byref(c))
    return st, c.value


def test_router_pattern_rules():
    for pat, layer in ((b"SFFF", 0), (b"SFFF", 1), (b"FSXS", 1), (b"", 0), (b"FS", 2), (b"FS", -1), (b"fS", 0)):
        assert route(pat, layer, desc())[0] == PATTERN, (pat, layer)
    assert route(None, 0, desc())[0] == NULL
    assert route(b"FS", 0, desc(), t=None)[0] == NULL


def test_router_shared_layer_enqueues_nothing():
    # Shared layers need neither inputs nor a descriptor and touch no device state.
    for layer in (1, 2, 3):
        assert route(b"FSSS", layer, None, q=None, k=None, w=None) == (OK, 0)
    assert route(b"FSFS", 3, None, q=None, k=None, w=None) == (OK, 0)


def test_router_full_layer_validates_like_score_topk():
    assert route(b"FSSS", 0, None)[0] == NULL
    assert route(b"FSSS", 0, desc(qd=7))[0] == DTYPE
    assert route(b"FSSS", 0, desc(), q=FAKE_ODD)[0] == ALIGN
    assert route(b"FS", 0, desc(B=32, Lq=1, Lk=200000, topk=2048))[0] == WS


def mla(B=1, Lq=4, Lk=100, Hq=128, Dqk=576, Dv=512, topk=64, scale=0.04, q=FAKE, kv=FAKE, t=FAKE, out=FAKE):
    d = sa._MlaDesc(B, Lq, Lk, Hq, Dqk, Dv, topk)
    return sa.lib().sparse_mla_attn(ctypes.byref(d), q, kv, t, scale, out, None, None, 0, None)


def test_sparse_mla_rejections():
    assert sa.lib().sparse_mla_attn(None, FAKE, FAKE, FAKE, 1.0, FAKE, None, None, 0, None) == NULL
    assert mla(B=0) == SHAPE
    assert mla(Dv=600) == SHAPE
    assert mla(scale=0.0) == SHAPE
    assert mla(scale=float("nan")) == SHAPE
    assert mla(Dqk=128, Dv=128) == UNSUP
    assert mla(Hq=24) == UNSUP
    assert mla(Dqk=32, Dv=32, Hq=6) == UNSUP
    assert mla(topk=4096) == UNSUP
    assert mla(q=None) == NULL
    assert mla(kv=None) == NULL
    assert mla(t=None) == NULL
    assert mla(out=None) == NULL
    assert mla(q=FAKE_ODD) == ALIGN
    assert mla(kv=FAKE_ODD) == ALIGN


def test_overlap_rejections():
    L = sa.lib()
    assert L.idx_overlap(FAKE, FAKE, 0, 8, FAKE, None) == OK        # empty: nothing enqueued
    assert L.idx_overlap(FAKE, FAKE, -1, 8, FAKE, None) == SHAPE
    assert L.idx_overlap(FAKE, FAKE, 4, 0, FAKE, None) == SHAPE
    assert L.idx_overlap(FAKE, FAKE, 4, 4096, FAKE, None) == SHAPE
    assert L.idx_overlap(None, FAKE, 4, 8, FAKE, None) == NULL
    assert L.idx_overlap(FAKE, FAKE, 4, 8, None, None) == NULL
    assert L.idx_overlap(ctypes.c_void_p(0x10002), FAKE, 4, 8, FAKE, None) == ALIGN


# ---------------------------------------------------------------- serving batches over paged caches

def pdesc(num_seqs=2, total_q=3, max_seq_len=1000, num_blocks=40, block_size=64, max_blocks=16, H=64, D=128,
          topk=64, qd=FP8, kd=FP8, wd=BF16):
    return sa._PagedIndexerDesc(num_seqs, total_q, max_seq_len, num_blocks, block_size, max_blocks, H, D, topk, qd,
                                kd, wd)


def pscore(d, ws=FAKE, wsb=1 << 40, **ptrs):
    p = dict(q=FAKE, k=FAKE, bt=FAKE, qs=FAKE, sl=FAKE, w=FAKE, t=FAKE)
    p.update(ptrs)
    return sa.lib().idx_score_topk_paged(ctypes.byref(d) if d is not None else None, p["q"], p["k"], p["bt"],
                                         p["qs"], p["sl"], p["w"], p["t"], ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(block_size=32), SHAPE), (dict(block_size=96), SHAPE), (dict(max_blocks=15), SHAPE),
    (dict(num_seqs=0), SHAPE), (dict(total_q=0), SHAPE), (dict(num_blocks=0), SHAPE),
    (dict(max_seq_len=0), SHAPE), (dict(H=32), UNSUP), (dict(topk=4096), UNSUP), (dict(qd=BF16), DTYPE),
])
def test_paged_indexer_descriptor_rejections(kw, code):
    assert pscore(pdesc(**kw)) == code


def test_paged_indexer_pointers_and_workspace():
    d = pdesc()
    n = ctypes.c_size_t(0)
    assert sa.lib().idx_score_topk_paged_workspace(ctypes.byref(d), ctypes.byref(n)) == OK
    # row metadata, score rows of max_seq_len, the top-k's workspace
    assert n.value >= 3 * 1000 * 4 + 3 * 12
    assert pscore(None) == NULL
    for key in ("q", "k", "bt", "qs", "sl", "w", "t"):
        assert pscore(d, **{key: None}) == NULL, key
    assert pscore(d, q=FAKE_ODD) == ALIGN
    assert pscore(d, ws=None, wsb=0) == WS
    assert pscore(d, wsb=n.value - 1) == WS
    assert pscore(d, ws=ctypes.c_void_p(0x10010), wsb=n.value) == ALIGN


def test_paged_router_pattern_rules_and_shared_layer():
    L = sa.lib()
    d = pdesc()
    done = ctypes.c_int(-1)
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert L.idx_cache_route_paged(b"SF", 0, ctypes.byref(d), *args, ctypes.byref(done)) == PATTERN
    assert L.idx_cache_route_paged(b"FS", 2, ctypes.byref(d), *args, ctypes.byref(done)) == PATTERN
    assert L.idx_cache_route_paged(b"FS", 1, None, None, None, None, None, None, None, FAKE, None, 0, None,
                                   ctypes.byref(done)) == OK
    assert done.value == 0
    bad = pdesc(block_size=48)
    assert L.idx_cache_route_paged(b"FS", 0, ctypes.byref(bad), *args, ctypes.byref(done)) == SHAPE


def test_paged_mla_rejections():
    L = sa.lib()

    def pm(num_seqs=2, total_q=3, num_blocks=10, block_size=16, max_blocks=8, Hq=64, Dqk=576, Dv=512, topk=64,
           ws=FAKE, wsb=1 << 40, **ptrs):
        d = sa._PagedMlaDesc(num_seqs, total_q, num_blocks, block_size, max_blocks, Hq, Dqk, Dv, topk)
        p = dict(q=FAKE, kv=FAKE, bt=FAKE, qs=FAKE, sl=FAKE, t=FAKE, out=FAKE)
        p.update(ptrs)
        return L.sparse_mla_attn_paged(ctypes.byref(d), p["q"], p["kv"], p["bt"], p["qs"], p["sl"], p["t"], 0.1,
                                       p["out"], None, ws, wsb, None)

    assert pm(block_size=24) == SHAPE
    assert pm(total_q=0) == SHAPE
    assert pm(num_blocks=1 << 20, block_size=1 << 12) == SHAPE   # pool rows beyond int32
    assert pm(Hq=24) == UNSUP
    assert pm(Dqk=128, Dv=128) == UNSUP
    assert pm(bt=None) == NULL
    assert pm(q=None) == NULL
    assert pm(out=None) == NULL
    assert pm(kv=FAKE_ODD) == ALIGN
    assert pm(ws=None, wsb=0) == WS
    n = ctypes.c_size_t(0)
    d = sa._PagedMlaDesc(2, 3, 10, 16, 8, 64, 576, 512, 64)
    assert L.sparse_mla_attn_paged_workspace(ctypes.byref(d), ctypes.byref(n)) == OK
    assert n.value >= 3 * 8 + 3 * 64 * 4


# ------------------------------------------------------------ binding checks
#
# The C ABI cannot see tensor sizes, so the binding checks every tensor against
# the descriptor it builds before calling in.  Meta tensors (shape and dtype,
# no storage) run these checks on the CPU; a call whose shapes are all right
# goes on to the device check, which meta tensors fail with TypeError.

import torch  # noqa: E402

F8, B16, F32, I32 = torch.float8_e4m3fn, torch.bfloat16, torch.float32, torch.int32


def m(*shape, dtype):
    return torch.empty(*shape, dtype=dtype, device="meta")


def idx_args(B=1, L=128, H=64, D=128):
    return m(B, L, H, D, dtype=F8), m(B, L, D, dtype=F8), m(B, L, H, dtype=B16)


@pytest.mark.parametrize("bad", ["k_batch", "k_dim", "k_dtype", "w_heads", "w_rows", "t_batch", "t_topk", "t_dtype",
                                 "dbg_short", "dbg_dtype", "q_3d"])
def test_binding_rejects_mismatched_indexer_tensors(bad):
    q, k, w = idx_args()
    kw = {}
    if bad == "k_batch":
        k = m(2, 128, 128, dtype=F8)
    elif bad == "k_dim":
        k = m(1, 128, 64, dtype=F8)
    elif bad == "k_dtype":
        k = m(1, 128, 128, dtype=B16)
    elif bad == "w_heads":
        w = m(1, 128, 32, dtype=B16)
    elif bad == "w_rows":
        w = m(1, 64, 64, dtype=B16)
    elif bad == "t_batch":
        kw["t_out"] = m(2, 128, 64, dtype=I32)
    elif bad == "t_topk":
        kw["t_out"] = m(1, 128, 32, dtype=I32)
    elif bad == "t_dtype":
        kw["t_out"] = m(1, 128, 64, dtype=torch.int64)
    elif bad == "dbg_short":
        kw["scores_dbg"] = m(1, 128, 100, dtype=F32)
    elif bad == "dbg_dtype":
        kw["scores_dbg"] = m(1, 128, 128, dtype=B16)
    elif bad == "q_3d":
        q = m(128, 64, 128, dtype=F8)
    with pytest.raises(ValueError):
        sa.idx_score_topk(q, k, w, 64, **kw)


def test_binding_well_shaped_indexer_call_reaches_the_device_check():
    q, k, w = idx_args()
    with pytest.raises(TypeError):
        sa.idx_score_topk(q, k, w, 64, t_out=m(1, 128, 64, dtype=I32), scores_dbg=m(1, 128, 128, dtype=F32))


def test_binding_rejects_noncontiguous_tensors():
    q, k, w = idx_args()
    k_view = m(1, 128, 128, dtype=F8).transpose(1, 2)   # right shape, strided view
    assert not k_view.is_contiguous()
    with pytest.raises(ValueError):
        sa.idx_score_topk(q, k_view, w, 64)


def test_binding_router_checks_t_cache_against_the_indexer():
    q, k, w = idx_args(B=2)
    with pytest.raises(ValueError):
        sa.idx_cache_route("FS", 0, q, k, w, m(1, 128, 64, dtype=I32))   # cache of a one-sequence batch
    with pytest.raises(ValueError):
        sa.idx_cache_route("FS", 0, q, k, w, m(2, 128, 64, dtype=torch.int64))
    with pytest.raises(TypeError):
        sa.idx_cache_route("FS", 0, q, k, w, m(2, 128, 64, dtype=I32))


@pytest.mark.parametrize("bad", ["scores_dtype", "pos_dtype", "pos_len", "t_shape"])
def test_binding_rejects_mismatched_topk_tensors(bad):
    s = m(8, 500, dtype=F32)
    kw = {}
    if bad == "scores_dtype":
        s = m(8, 500, dtype=torch.float16)
    elif bad == "pos_dtype":
        kw["row_pos"] = m(8, dtype=torch.int64)
    elif bad == "pos_len":
        kw["row_pos"] = m(7, dtype=I32)
    else:
        kw["t_out"] = m(8, 16, dtype=I32)
    with pytest.raises(ValueError):
        sa.idx_topk(s, 32, **kw)


@pytest.mark.parametrize("bad", ["q_dtype", "kv_dtype", "kv_dim", "kv_batch", "t_dtype", "t_rows", "out_dv",
                                 "out_dtype", "lse_shape"])
def test_binding_rejects_mismatched_mla_tensors(bad):
    q, kv, t = m(2, 4, 128, 576, dtype=B16), m(2, 100, 576, dtype=B16), m(2, 4, 64, dtype=I32)
    kw = {}
    if bad == "q_dtype":
        q = m(2, 4, 128, 576, dtype=F32)
    elif bad == "kv_dtype":
        kv = m(2, 100, 576, dtype=F8)
    elif bad == "kv_dim":
        kv = m(2, 100, 512, dtype=B16)
    elif bad == "kv_batch":
        kv = m(1, 100, 576, dtype=B16)
    elif bad == "t_dtype":
        t = m(2, 4, 64, dtype=torch.int64)
    elif bad == "t_rows":
        t = m(2, 3, 64, dtype=I32)
    elif bad == "out_dv":
        kw["out"] = m(2, 4, 128, 576, dtype=B16)
    elif bad == "out_dtype":
        kw["out"] = m(2, 4, 128, 512, dtype=F32)
    else:
        kw["lse"] = m(2, 4, 64, dtype=F32)
    with pytest.raises(ValueError):
        sa.sparse_mla_attn(q, kv, t, 0.04, 512, **kw)


@pytest.mark.parametrize("bad", ["table_rows", "seq_lens_len", "qs_dtype", "k_dim", "w_rows", "t_rows"])
def test_binding_rejects_mismatched_paged_indexer_tensors(bad):
    q, kc, w = m(3, 64, 128, dtype=F8), m(40, 64, 128, dtype=F8), m(3, 64, dtype=B16)
    table, qs, sl = m(2, 16, dtype=I32), m(3, dtype=I32), m(2, dtype=I32)
    kw = {}
    if bad == "table_rows":
        table = m(3, 16, dtype=I32)
    elif bad == "seq_lens_len":
        sl = m(3, dtype=I32)
    elif bad == "qs_dtype":
        qs = m(3, dtype=torch.int64)
    elif bad == "k_dim":
        kc = m(40, 64, 64, dtype=F8)
    elif bad == "w_rows":
        w = m(2, 64, dtype=B16)
    else:
        kw["t_out"] = m(2, 64, dtype=I32)
    with pytest.raises(ValueError):
        sa.idx_score_topk_paged(q, kc, table, qs, sl, w, 64, 1000, **kw)


@pytest.mark.parametrize("bad", ["kv_dim", "t_rows", "table_rows", "out_shape", "lse_shape"])
def test_binding_rejects_mismatched_paged_mla_tensors(bad):
    q, kvc, t = m(3, 128, 576, dtype=B16), m(40, 64, 576, dtype=B16), m(3, 64, dtype=I32)
    table, qs, sl = m(2, 16, dtype=I32), m(3, dtype=I32), m(2, dtype=I32)
    kw = {}
    if bad == "kv_dim":
        kvc = m(40, 64, 512, dtype=B16)
    elif bad == "t_rows":
        t = m(4, 64, dtype=I32)
    elif bad == "table_rows":
        table = m(1, 16, dtype=I32)
    elif bad == "out_shape":
        kw["out"] = m(3, 128, 576, dtype=B16)
    else:
        kw["lse"] = m(3, 64, dtype=F32)
    with pytest.raises(ValueError):
        sa.sparse_mla_attn_paged(q, kvc, table, qs, sl, t, 0.04, 512, **kw)


def noalloc(d, q=FAKE, k=FAKE, w=FAKE, t=FAKE):
    return sa.lib().idx_score_topk_noalloc(ctypes.byref(d) if d is not None else None, q, k, w, t, None)


def test_noalloc_validates_before_any_hip_call():
    d = desc(B=4, Lq=1, Lk=200000, topk=2048)
    assert noalloc(None) == NULL
    assert noalloc(d, q=None) == NULL
    assert noalloc(d, t=FAKE_ODD) == ALIGN
    assert noalloc(desc(H=12)) == UNSUP
    # 64 sequences x 4 queries x 200,000 keys of fp32 scores: more than the
    # 128 MiB static scratch
    assert noalloc(desc(B=64, Lq=4, Lk=200000, topk=2048)) == SCRATCH
    assert sa.lib().idxc_status_str(SCRATCH).startswith(b"request needs more device scratch")


def test_binding_noalloc_requires_t_out():
    q, k, w = idx_args()
    with pytest.raises(ValueError):
        sa.idx_score_topk_noalloc(q, k, w, 64, None)
    with pytest.raises(ValueError):
        sa.idx_score_topk_noalloc(q, k, w, 64, m(1, 128, 32, dtype=I32))


def paged_ws(**kw):
    d = pdesc(**kw)
    n = ctypes.c_size_t(0)
    assert sa.lib().idx_score_topk_paged_workspace(ctypes.byref(d), ctypes.byref(n)) == OK
    return n.value


def test_paged_workspace_by_mode():
    """Prefill-heavy batches (more than 4 rows per sequence, fp8 64 x 128) take the
    fused kernel and need only the row-block prefix; decode batches keep the
    split path's score rows."""
    fused = paged_ws(num_seqs=4, total_q=4800, max_seq_len=200000, num_blocks=4000, block_size=64, max_blocks=3200)
    assert fused <= 256
    split = paged_ws(num_seqs=4, total_q=16, max_seq_len=200000, num_blocks=4000, block_size=64, max_blocks=3200)
    assert split >= 16 * 200000 * 4
    bf16 = paged_ws(num_seqs=4, total_q=4800, max_seq_len=20000, num_blocks=4000, block_size=64, max_blocks=400,
                    qd=BF16, kd=BF16, wd=FP32, D=64)
    assert bf16 >= 4800 * 20000 * 4    # the fused paged form is fp8-only: split path


def test_calib_rejects_before_launch():
    L = sa.lib()
    f = L.idxc_calib_mfma_rate
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert f(0, None, 64, FAKE, 64, 1, 1, FAKE, None) == NULL
    assert f(0, FAKE, 64, FAKE, 64, 1, 1, None, None) == NULL
    assert f(0, FAKE, 8, FAKE, 64, 1, 1, FAKE, None) == SHAPE
    assert f(1, FAKE, 64, FAKE, 64, 0, 1, FAKE, None) == SHAPE
    assert f(1, FAKE, 64, FAKE, 64, 1, 0, FAKE, None) == SHAPE
    assert f(0, FAKE_ODD, 64, FAKE, 64, 1, 1, FAKE, None) == ALIGN
    assert f(2, FAKE, 64, FAKE, 64, 1, 1, FAKE, None) == DTYPE


def test_calib_gather_rejects_before_launch():
    L = sa.lib()
    f = L.idxc_calib_gather_rate
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert f(None, 1152, 10, FAKE, 1, 8, 1, FAKE, None) == NULL
    assert f(FAKE, 1152, 10, None, 1, 8, 1, FAKE, None) == NULL
    assert f(FAKE, 1152, 10, FAKE, 1, 8, 1, None, None) == NULL
    assert f(FAKE, 1100, 10, FAKE, 1, 8, 1, FAKE, None) == SHAPE     # not whole 128-byte lines
    assert f(FAKE, 0, 10, FAKE, 1, 8, 1, FAKE, None) == SHAPE
    assert f(FAKE, 17 * 128, 10, FAKE, 1, 8, 1, FAKE, None) == SHAPE
    assert f(FAKE, 1152, 0, FAKE, 1, 8, 1, FAKE, None) == SHAPE
    assert f(FAKE, 1152, 10, FAKE, 0, 8, 1, FAKE, None) == SHAPE
    assert f(FAKE, 1152, 10, FAKE, 1, 0, 1, FAKE, None) == SHAPE
    assert f(FAKE, 1152, 10, FAKE, 1, 8, 0, FAKE, None) == SHAPE
    assert f(FAKE, 1152, 10, FAKE, 1, 8, (1 << 20) + 1, FAKE, None) == SHAPE
    assert f(FAKE, 1152, 10, FAKE, 1 << 16, 1 << 15, 1, FAKE, None) == SHAPE   # 2^31 entries
    assert f(FAKE_ODD, 1152, 10, FAKE, 1, 8, 1, FAKE, None) == ALIGN
    assert f(FAKE, 1152, 10, FAKE, 1, 8, 1, FAKE_ODD, None) == ALIGN
    assert f(FAKE, 1152, 10, ctypes.c_void_p(0x10002), 1, 8, 1, FAKE, None) == ALIGN
