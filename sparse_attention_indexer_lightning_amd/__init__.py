"""Python binding of libidxcache.so: the lightning indexer with fused top-k, the
IndexCache Full/Shared router and sparse MLA attention on MI355X (gfx950).

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.  The functions carry
the names of the C ABI in ``include/idxcache.h``.  Loading fails loudly when
the library has not been built; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import _build

__all__ = [
    "IdxcError", "lib", "idx_score_topk", "idx_score_topk_workspace", "idx_topk", "idx_topk_workspace",
    "idx_cache_route", "sparse_mla_attn", "sparse_mla_attn_workspace", "indexer_desc", "mla_desc",
    "STATUS", "DTYPE", "idx_overlap", "overlap_matrix",
    "idx_score_topk_paged", "idx_score_topk_paged_workspace", "idx_cache_route_paged",
    "sparse_mla_attn_paged", "sparse_mla_attn_paged_workspace", "paged_indexer_desc", "paged_mla_desc",
    "idx_score_topk_noalloc",
]

STATUS = {0: "IDXC_OK", -1: "IDXC_ERR_NULL", -2: "IDXC_ERR_SHAPE", -3: "IDXC_ERR_DTYPE",
          -4: "IDXC_ERR_ALIGN", -5: "IDXC_ERR_UNSUPPORTED", -6: "IDXC_ERR_WORKSPACE",
          -7: "IDXC_ERR_PATTERN", -8: "IDXC_ERR_HIP", -9: "IDXC_ERR_SCRATCH"}
DTYPE = {torch.bfloat16: 1, torch.float8_e4m3fn: 2, torch.float32: 3}


class IdxcError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().idxc_status_str(status).decode()
        super().__init__(f"{where}: {STATUS.get(status, status)} ({msg})")


class _IndexerDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("B", "Lq", "Lk", "H", "D", "topk", "q_dtype", "k_dtype", "w_dtype")]


class _MlaDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("B", "Lq", "Lk", "Hq", "Dqk", "Dv", "topk")]


class _PagedIndexerDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("num_seqs", "total_q", "max_seq_len", "num_blocks", "block_size",
                                            "max_blocks", "H", "D", "topk", "q_dtype", "k_dtype", "w_dtype")]


class _PagedMlaDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("num_seqs", "total_q", "num_blocks", "block_size", "max_blocks",
                                            "Hq", "Dqk", "Dv", "topk")]


_lib = None


def lib():
    """Load the in-tree libidxcache.so (raises if it has not been built).
    IDXCACHE_LIB names another build of the same library to load instead."""
    global _lib
    if _lib is None:
        path = os.environ.get("IDXCACHE_LIB") or _build.LIB_PATH
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with __graft_entry__.build() "
                              "or python -m sparse_attention_indexer_lightning_amd._build")
        L = ctypes.CDLL(path)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        szp = ctypes.POINTER(ctypes.c_size_t)
        ip = ctypes.POINTER(ctypes.c_int)
        dp = ctypes.POINTER(_IndexerDesc)
        mp = ctypes.POINTER(_MlaDesc)
        L.idxc_abi_version.restype = i32
        L.idxc_abi_version.argtypes = []
        L.idxc_status_str.restype = ctypes.c_char_p
        L.idxc_status_str.argtypes = [i32]
        L.idx_score_topk_workspace.restype = i32
        L.idx_score_topk_workspace.argtypes = [dp, szp]
        L.idx_score_topk.restype = i32
        L.idx_score_topk.argtypes = [dp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.idx_score_topk_noalloc.restype = i32
        L.idx_score_topk_noalloc.argtypes = [dp, vp, vp, vp, vp, vp]
        L.idx_topk_workspace.restype = i32
        L.idx_topk_workspace.argtypes = [i32, i32, i32, szp]
        L.idx_topk.restype = i32
        L.idx_topk.argtypes = [vp, vp, i32, i32, i32, vp, vp, sz, vp]
        L.idx_cache_route.restype = i32
        L.idx_cache_route.argtypes = [ctypes.c_char_p, i32, dp, vp, vp, vp, vp, vp, sz, vp, ip]
        L.sparse_mla_attn_workspace.restype = i32
        L.sparse_mla_attn_workspace.argtypes = [mp, szp]
        L.sparse_mla_attn.restype = i32
        L.sparse_mla_attn.argtypes = [mp, vp, vp, vp, ctypes.c_float, vp, vp, vp, sz, vp]
        L.idx_overlap.restype = i32
        L.idx_overlap.argtypes = [vp, vp, i32, i32, vp, vp]
        pdp = ctypes.POINTER(_PagedIndexerDesc)
        pmp = ctypes.POINTER(_PagedMlaDesc)
        L.idx_score_topk_paged_workspace.restype = i32
        L.idx_score_topk_paged_workspace.argtypes = [pdp, szp]
        L.idx_score_topk_paged.restype = i32
        L.idx_score_topk_paged.argtypes = [pdp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.idx_cache_route_paged.restype = i32
        L.idx_cache_route_paged.argtypes = [ctypes.c_char_p, i32, pdp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, ip]
        L.sparse_mla_attn_paged_workspace.restype = i32
        L.sparse_mla_attn_paged_workspace.argtypes = [pmp, szp]
        L.sparse_mla_attn_paged.restype = i32
        L.sparse_mla_attn_paged.argtypes = [pmp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, sz, vp]
        _lib = L
    return _lib


def _check(status: int, where: str) -> None:
    if status != 0:
        raise IdxcError(status, where)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _cuda_tensor(t, name):
    if not (isinstance(t, torch.Tensor) and t.is_cuda):
        raise TypeError(f"{name} must be a torch tensor on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _want(t, name, shape, dtype=None):
    """Shape and element type of a tensor argument, checked before any call: the
    C ABI sees only pointers and the sizes in the descriptor, so a tensor
    smaller than the descriptor says would be read or written past its end.
    ``shape`` entries of None match any size."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dim() != len(shape) or any(w is not None and int(g) != int(w) for g, w in zip(t.shape, shape)):
        want = tuple("*" if w is None else int(w) for w in shape)
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {want}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_device(*named):
    """Every given tensor is on one GPU; returns that device."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        _cuda_tensor(t, name)
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")
    return dev


def _keep_alive(stream, *tensors):
    """Tensors the binding allocated for a call on a caller-given stream stay
    reserved until that stream's work is done (torch's allocator would otherwise
    hand their memory out again once the Python object dies)."""
    if stream is None:
        return
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(
        stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    for t in tensors:
        if t is not None:
            t.record_stream(s)


def indexer_desc(q, k, w, topk: int) -> _IndexerDesc:
    """Descriptor of an indexer call from q [B,Lq,H,D], k [B,Lk,D], w [B,Lq,H]."""
    B, Lq, H, D = q.shape
    Lk = k.shape[1]
    return _IndexerDesc(B, Lq, Lk, H, D, topk, DTYPE.get(q.dtype, 0), DTYPE.get(k.dtype, 0),
                        DTYPE.get(w.dtype, 0))


def mla_desc(q, kv, t, Dv: int) -> _MlaDesc:
    B, Lq, Hq, Dqk = q.shape
    return _MlaDesc(B, Lq, kv.shape[1], Hq, Dqk, Dv, t.shape[-1])


def _check_indexer(q, k, w, topk, t=None, t_name="t_out", scores_dbg=None):
    if not (isinstance(q, torch.Tensor) and q.dim() == 4):
        raise ValueError("q must be a tensor [B, Lq, H, D]")
    B, Lq, H, D = q.shape
    _want(q, "q", (B, Lq, H, D))
    _want(k, "k", (B, None, D), q.dtype)
    _want(w, "w", (B, Lq, H))
    if t is not None:
        _want(t, t_name, (B, Lq, topk), torch.int32)
    if scores_dbg is not None:
        _want(scores_dbg, "scores_dbg", (B, Lq, k.shape[1]), torch.float32)


def idx_score_topk_workspace(q, k, w, topk: int) -> int:
    _check_indexer(q, k, w, topk)
    d = indexer_desc(q, k, w, topk)
    n = ctypes.c_size_t(0)
    _check(lib().idx_score_topk_workspace(ctypes.byref(d), ctypes.byref(n)), "idx_score_topk_workspace")
    return n.value


def _workspace(nbytes: int, device, ws):
    if nbytes == 0:
        return ws
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def idx_score_topk(q, k, w, topk: int, t_out=None, scores_dbg=None, ws=None, stream=None):
    """Fused indexer score + per-row top-k.  Returns T int32 [B, Lq, topk]."""
    _check_indexer(q, k, w, topk, t_out, "t_out", scores_dbg)
    _same_device(("q", q), ("k", k), ("w", w), ("t_out", t_out), ("scores_dbg", scores_dbg), ("ws", ws))
    B, Lq = q.shape[:2]
    mine = []
    if t_out is None:
        t_out = torch.empty(B, Lq, topk, dtype=torch.int32, device=q.device)
        mine.append(t_out)
    d = indexer_desc(q, k, w, topk)
    ws_in = ws
    ws = _workspace(idx_score_topk_workspace(q, k, w, topk), q.device, ws)
    if ws is not ws_in:
        mine.append(ws)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().idx_score_topk(ctypes.byref(d), _p(q), _p(k), _p(w), _p(t_out), _p(scores_dbg), _p(ws), wsb,
                                _stream(stream, q.device)), "idx_score_topk")
    _keep_alive(stream, *mine)
    return t_out


def idx_score_topk_noalloc(q, k, w, topk: int, t_out, stream=None):
    """idx_score_topk for callers that cannot allocate (graph capture, serving
    loops): the library's static device scratch replaces the workspace, and
    nothing is allocated here either, so the caller passes T.  Calls that may
    overlap on one GPU share that scratch and must not be issued."""
    if t_out is None:
        raise ValueError("t_out is required: this call allocates nothing")
    _check_indexer(q, k, w, topk, t_out, "t_out")
    _same_device(("q", q), ("k", k), ("w", w), ("t_out", t_out))
    d = indexer_desc(q, k, w, topk)
    _check(lib().idx_score_topk_noalloc(ctypes.byref(d), _p(q), _p(k), _p(w), _p(t_out), _stream(stream, q.device)),
           "idx_score_topk_noalloc")
    return t_out


def idx_topk_workspace(R: int, Lk: int, topk: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().idx_topk_workspace(R, Lk, topk, ctypes.byref(n)), "idx_topk_workspace")
    return n.value


def idx_topk(scores, topk: int, row_pos=None, t_out=None, ws=None, stream=None):
    """Row top-k of fp32 scores [R, Lk] (ties to the lower index, ascending, -1 padded)."""
    if not (isinstance(scores, torch.Tensor) and scores.dim() == 2):
        raise ValueError("scores must be a tensor [R, Lk]")
    R, Lk = scores.shape
    _want(scores, "scores", (R, Lk), torch.float32)
    if row_pos is not None:
        _want(row_pos, "row_pos", (R,), torch.int32)
    if t_out is not None:
        _want(t_out, "t_out", (R, topk), torch.int32)
    _same_device(("scores", scores), ("row_pos", row_pos), ("t_out", t_out), ("ws", ws))
    mine = []
    if t_out is None:
        t_out = torch.empty(R, topk, dtype=torch.int32, device=scores.device)
        mine.append(t_out)
    ws_in = ws
    ws = _workspace(idx_topk_workspace(R, Lk, topk), scores.device, ws)
    if ws is not ws_in:
        mine.append(ws)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().idx_topk(_p(scores), _p(row_pos), R, Lk, topk, _p(t_out), _p(ws), wsb,
                          _stream(stream, scores.device)), "idx_topk")
    _keep_alive(stream, *mine)
    return t_out


def idx_cache_route(pattern: str, layer: int, q, k, w, t_cache, topk: int = None, ws=None, stream=None) -> bool:
    """IndexCache router: Full layers overwrite ``t_cache``; Shared layers enqueue nothing.

    Returns True when the layer computed (Full).  On Shared layers q, k, w may be None.
    """
    computed = ctypes.c_int(-1)
    topk = t_cache.shape[-1] if topk is None else topk
    pat = pattern.encode()
    mine = []
    if q is None:
        _same_device(("t_cache", t_cache))
        d_ptr = None
        wsb = 0
        dev = t_cache.device
    else:
        _check_indexer(q, k, w, topk, t_cache, "t_cache")
        _same_device(("q", q), ("k", k), ("w", w), ("t_cache", t_cache), ("ws", ws))
        d = indexer_desc(q, k, w, topk)
        d_ptr = ctypes.byref(d)
        n = ctypes.c_size_t(0)
        st = lib().idx_score_topk_workspace(d_ptr, ctypes.byref(n))
        ws_in = ws
        ws = _workspace(n.value if st == 0 else 0, q.device, ws)
        if ws is not ws_in:
            mine.append(ws)
        wsb = 0 if ws is None else ws.numel() * ws.element_size()
        dev = q.device
    _check(lib().idx_cache_route(pat, layer, d_ptr, _p(q), _p(k), _p(w), _p(t_cache), _p(ws), wsb,
                                 _stream(stream, dev), ctypes.byref(computed)), "idx_cache_route")
    _keep_alive(stream, *mine)
    return computed.value == 1


def _check_mla(q, kv, t, Dv, out=None, lse=None):
    if not (isinstance(q, torch.Tensor) and q.dim() == 4):
        raise ValueError("q must be a tensor [B, Lq, Hq, Dqk]")
    B, Lq, Hq, Dqk = q.shape
    _want(q, "q", (B, Lq, Hq, Dqk), torch.bfloat16)
    _want(kv, "kv", (B, None, Dqk), torch.bfloat16)
    _want(t, "t", (B, Lq, None), torch.int32)
    if out is not None:
        _want(out, "out", (B, Lq, Hq, Dv), torch.bfloat16)
    if lse is not None:
        _want(lse, "lse", (B, Lq, Hq), torch.float32)


def sparse_mla_attn_workspace(q, kv, t, Dv: int) -> int:
    _check_mla(q, kv, t, Dv)
    d = mla_desc(q, kv, t, Dv)
    n = ctypes.c_size_t(0)
    _check(lib().sparse_mla_attn_workspace(ctypes.byref(d), ctypes.byref(n)), "sparse_mla_attn_workspace")
    return n.value


def idx_overlap(t_a, t_b, stream=None):
    """Per-row count of indices present in both index sets (rows ascending, -1 padded)."""
    for name, t in (("t_a", t_a), ("t_b", t_b)):
        _cuda_tensor(t, name)
    if t_a.shape != t_b.shape or t_a.dtype != torch.int32 or t_b.dtype != torch.int32:
        raise ValueError("t_a and t_b must be int32 tensors of one shape [..., topk]")
    topk = t_a.shape[-1]
    R = t_a.numel() // topk
    counts = torch.empty(t_a.shape[:-1], dtype=torch.int32, device=t_a.device)
    _check(lib().idx_overlap(_p(t_a), _p(t_b), R, topk, _p(counts), _stream(stream, t_a.device)), "idx_overlap")
    return counts


def overlap_matrix(ts, stream=None):
    """Layer x layer mean overlap ratio of index sets ts[l] (each [..., topk]):
    entry (i, j) = mean over rows of |T_i & T_j| / (valid entries of T_i).
    The intersections run in the library (idx_overlap); the ratio and the mean
    are a summary of its counts taken here with torch, for reports only."""
    L = len(ts)
    valid = [(t >= 0).sum(dim=-1).clamp(min=1).to(torch.float64) for t in ts]
    m = torch.zeros(L, L, dtype=torch.float64)
    for i in range(L):
        for j in range(L):
            c = idx_overlap(ts[i], ts[j], stream=stream).to(torch.float64)
            m[i, j] = (c / valid[i]).mean().item()
    return m


def sparse_mla_attn(q, kv, t, sm_scale: float, Dv: int, out=None, lse=None, ws=None, stream=None):
    """Sparse MLA attention; returns (out bf16 [B,Lq,Hq,Dv], lse fp32 [B,Lq,Hq] or None)."""
    _check_mla(q, kv, t, Dv, out, lse)
    _same_device(("q", q), ("kv", kv), ("t", t), ("out", out), ("lse", lse), ("ws", ws))
    B, Lq, Hq, _ = q.shape
    mine = []
    if out is None:
        out = torch.empty(B, Lq, Hq, Dv, dtype=torch.bfloat16, device=q.device)
        mine.append(out)
    d = mla_desc(q, kv, t, Dv)
    ws_in = ws
    ws = _workspace(sparse_mla_attn_workspace(q, kv, t, Dv), q.device, ws)
    if ws is not ws_in:
        mine.append(ws)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sparse_mla_attn(ctypes.byref(d), _p(q), _p(kv), _p(t), float(sm_scale), _p(out), _p(lse),
                                 _p(ws), wsb, _stream(stream, q.device)), "sparse_mla_attn")
    _keep_alive(stream, *mine)
    return out, lse


# ------------------------------------------------------------------ serving batches over paged caches
#
# q and w pack the query rows of all sequences ([total_q, H, D], [total_q, H]);
# k_cache / kv_cache are page pools [num_blocks, block_size, row];
# block_table int32 [num_seqs, max_blocks], query_start int32 [num_seqs + 1],
# seq_lens int32 [num_seqs] are device tensors (see include/idxcache.h).


def paged_indexer_desc(q, k_cache, w, block_table, query_start, topk: int, max_seq_len: int) -> _PagedIndexerDesc:
    total_q, H, D = q.shape
    num_blocks, block_size = k_cache.shape[:2]
    return _PagedIndexerDesc(query_start.numel() - 1, total_q, max_seq_len, num_blocks, block_size,
                             block_table.shape[1], H, D, topk, DTYPE.get(q.dtype, 0), DTYPE.get(k_cache.dtype, 0),
                             DTYPE.get(w.dtype, 0))


def paged_mla_desc(q, kv_cache, block_table, query_start, t, Dv: int) -> _PagedMlaDesc:
    total_q, Hq, Dqk = q.shape
    num_blocks, block_size = kv_cache.shape[:2]
    return _PagedMlaDesc(query_start.numel() - 1, total_q, num_blocks, block_size, block_table.shape[1], Hq, Dqk,
                         Dv, t.shape[-1])


def _check_paged_meta(block_table, query_start, seq_lens=None):
    _want(query_start, "query_start", (None,), torch.int32)
    ns = query_start.shape[0] - 1
    if ns < 1:
        raise ValueError("query_start must hold num_seqs + 1 >= 2 entries")
    _want(block_table, "block_table", (ns, None), torch.int32)
    if seq_lens is not None:
        _want(seq_lens, "seq_lens", (ns,), torch.int32)


def _check_paged_indexer(q, k_cache, w, block_table, query_start, topk, seq_lens=None, t=None, t_name="t_out"):
    if not (isinstance(q, torch.Tensor) and q.dim() == 3):
        raise ValueError("q must be a tensor [total_q, H, D]")
    total_q, H, D = q.shape
    _want(q, "q", (total_q, H, D))
    _want(k_cache, "k_cache", (None, None, D), q.dtype)
    _want(w, "w", (total_q, H))
    _check_paged_meta(block_table, query_start, seq_lens)
    if t is not None:
        _want(t, t_name, (total_q, topk), torch.int32)


def idx_score_topk_paged_workspace(q, k_cache, w, block_table, query_start, topk: int, max_seq_len: int) -> int:
    _check_paged_indexer(q, k_cache, w, block_table, query_start, topk)
    d = paged_indexer_desc(q, k_cache, w, block_table, query_start, topk, max_seq_len)
    n = ctypes.c_size_t(0)
    _check(lib().idx_score_topk_paged_workspace(ctypes.byref(d), ctypes.byref(n)), "idx_score_topk_paged_workspace")
    return n.value


def idx_score_topk_paged(q, k_cache, block_table, query_start, seq_lens, w, topk: int, max_seq_len: int,
                         t_out=None, ws=None, stream=None):
    """Indexer score + top-k of every row of a serving batch; returns T int32 [total_q, topk]
    (logical positions of the row's sequence)."""
    _check_paged_indexer(q, k_cache, w, block_table, query_start, topk, seq_lens, t_out)
    _same_device(("q", q), ("k_cache", k_cache), ("w", w), ("block_table", block_table),
                 ("query_start", query_start), ("seq_lens", seq_lens), ("t_out", t_out), ("ws", ws))
    mine = []
    if t_out is None:
        t_out = torch.empty(q.shape[0], topk, dtype=torch.int32, device=q.device)
        mine.append(t_out)
    d = paged_indexer_desc(q, k_cache, w, block_table, query_start, topk, max_seq_len)
    ws_in = ws
    ws = _workspace(idx_score_topk_paged_workspace(q, k_cache, w, block_table, query_start, topk, max_seq_len),
                    q.device, ws)
    if ws is not ws_in:
        mine.append(ws)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().idx_score_topk_paged(ctypes.byref(d), _p(q), _p(k_cache), _p(block_table), _p(query_start),
                                      _p(seq_lens), _p(w), _p(t_out), _p(ws), wsb, _stream(stream, q.device)),
           "idx_score_topk_paged")
    _keep_alive(stream, *mine)
    return t_out


def idx_cache_route_paged(pattern: str, layer: int, q, k_cache, block_table, query_start, seq_lens, w, t_cache,
                          max_seq_len: int, ws=None, stream=None) -> bool:
    """IndexCache router over a serving batch (t_cache int32 [total_q, topk]); True on Full layers."""
    computed = ctypes.c_int(-1)
    topk = t_cache.shape[-1]
    mine = []
    if q is None:
        _same_device(("t_cache", t_cache))
        d_ptr, wsb, dev = None, 0, t_cache.device
    else:
        _check_paged_indexer(q, k_cache, w, block_table, query_start, topk, seq_lens, t_cache, "t_cache")
        _same_device(("q", q), ("k_cache", k_cache), ("w", w), ("block_table", block_table),
                     ("query_start", query_start), ("seq_lens", seq_lens), ("t_cache", t_cache), ("ws", ws))
        d = paged_indexer_desc(q, k_cache, w, block_table, query_start, topk, max_seq_len)
        d_ptr = ctypes.byref(d)
        n = ctypes.c_size_t(0)
        st = lib().idx_score_topk_paged_workspace(d_ptr, ctypes.byref(n))
        ws_in = ws
        ws = _workspace(n.value if st == 0 else 0, q.device, ws)
        if ws is not ws_in:
            mine.append(ws)
        wsb = 0 if ws is None else ws.numel() * ws.element_size()
        dev = q.device
    _check(lib().idx_cache_route_paged(pattern.encode(), layer, d_ptr, _p(q), _p(k_cache), _p(block_table),
                                       _p(query_start), _p(seq_lens), _p(w), _p(t_cache), _p(ws), wsb,
                                       _stream(stream, dev), ctypes.byref(computed)), "idx_cache_route_paged")
    _keep_alive(stream, *mine)
    return computed.value == 1


def _check_paged_mla(q, kv_cache, block_table, query_start, t, Dv, seq_lens=None, out=None, lse=None):
    if not (isinstance(q, torch.Tensor) and q.dim() == 3):
        raise ValueError("q must be a tensor [total_q, Hq, Dqk]")
    total_q, Hq, Dqk = q.shape
    _want(q, "q", (total_q, Hq, Dqk), torch.bfloat16)
    _want(kv_cache, "kv_cache", (None, None, Dqk), torch.bfloat16)
    _want(t, "t", (total_q, None), torch.int32)
    _check_paged_meta(block_table, query_start, seq_lens)
    if out is not None:
        _want(out, "out", (total_q, Hq, Dv), torch.bfloat16)
    if lse is not None:
        _want(lse, "lse", (total_q, Hq), torch.float32)


def sparse_mla_attn_paged_workspace(q, kv_cache, block_table, query_start, t, Dv: int) -> int:
    _check_paged_mla(q, kv_cache, block_table, query_start, t, Dv)
    d = paged_mla_desc(q, kv_cache, block_table, query_start, t, Dv)
    n = ctypes.c_size_t(0)
    _check(lib().sparse_mla_attn_paged_workspace(ctypes.byref(d), ctypes.byref(n)), "sparse_mla_attn_paged_workspace")
    return n.value


def sparse_mla_attn_paged(q, kv_cache, block_table, query_start, seq_lens, t, sm_scale: float, Dv: int, out=None,
                          lse=None, ws=None, stream=None):
    """Sparse MLA attention over a serving batch; returns (out bf16 [total_q, Hq, Dv], lse or None)."""
    _check_paged_mla(q, kv_cache, block_table, query_start, t, Dv, seq_lens, out, lse)
    _same_device(("q", q), ("kv_cache", kv_cache), ("block_table", block_table), ("query_start", query_start),
                 ("seq_lens", seq_lens), ("t", t), ("out", out), ("lse", lse), ("ws", ws))
    total_q, Hq, _ = q.shape
    mine = []
    if out is None:
        out = torch.empty(total_q, Hq, Dv, dtype=torch.bfloat16, device=q.device)
        mine.append(out)
    d = paged_mla_desc(q, kv_cache, block_table, query_start, t, Dv)
    ws_in = ws
    ws = _workspace(sparse_mla_attn_paged_workspace(q, kv_cache, block_table, query_start, t, Dv), q.device, ws)
    if ws is not ws_in:
        mine.append(ws)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sparse_mla_attn_paged(ctypes.byref(d), _p(q), _p(kv_cache), _p(block_table), _p(query_start),
                                       _p(seq_lens), _p(t), float(sm_scale), _p(out), _p(lse), _p(ws), wsb,
                                       _stream(stream, q.device)), "sparse_mla_attn_paged")
    _keep_alive(stream, *mine)
    return out, lse
