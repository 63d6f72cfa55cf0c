"""CPU oracle for the lightning indexer, its top-k, IndexCache routing and sparse MLA.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library and never imports it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, one rounding to the output
type).  This module marshals numpy arrays into it and holds the two pieces that
are control flow rather than arithmetic: the Full/Shared routing rule and the
layer-stack composition.

Sources (page title and section):
  [ITO] itoverdose.com, "IndexCache: Wie DeepSeek O(NL²)-Kosten in Sparse
        Attention um 75% reduziert"
  [PPM] parapluman.nl, Dutch article on IndexCache, section
        "Aandacht cachen met IndexCache"
  [AIB] aiboss88.com, "IndexCache - 清華大学とZhipuが共同開発した、
        スパースアテンション高速化技術。 - AiBoss", section "IndexCacheの技術的原理"
  [SRV] serving batches over paged caches: parapluman.nl, sections
        "Real-world versnellingen op productiemodellen" and "IndexCache in
        productie brengen" (serving engines vLLM, SGLang); setupai.cc,
        "IndexCache 加速長上下文推理 1.82 倍", comparison table (paged memory
        allocation)

Parity status of each function (pins live in tests/test_oracle_*.py):
  indexer_scores   pinned (hand-worked 8-token example; recency / reverse / tie
                   closed forms; a B = 3, Lq < Lk closed form with distinct keys
                   per sequence and scrambled row order; the H = 1 case vs numpy;
                   non-integer scores against the exact rational value rounded
                   to the nearest fp32 by brute force, ties to even)
  topk             pinned (brute force vs full sort and repeated argmax, closed
                   forms, rows with no valid key)
  route            pinned (hand-worked example, invariants)
  sparse_mla       pinned (dense attention via torch SDPA on CPU, closed forms)
  overlap          pinned (hand-worked rows, identical / disjoint / nested sets, symmetry)
  gather_pages     pinned (hand-worked table, identity table = contiguous rows)
  paged_indexer_topk, paged_sparse_mla
                   pinned (one sequence over an identity table = the contiguous
                   oracle; page permutations change nothing; a batch = its
                   sequences taken one at a time)
  stack            pinned (hand-worked two-layer example, Full/Shared second
                   layer x plain/residual FFN, exact integer values).  The way
                   layers compose (per-layer inputs independent of X, residual
                   add of the head-summed attention output, then the seeded FFN
                   stand-in) is a reading of the pages' inference loop; the pin
                   fixes that this code computes that reading.
  codecs           pinned (every fp8 / bf16 code vs torch; bf16 and fp32
                   rounding vs brute-force nearest search)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

DTYPE_CODES = {"bf16": 1, "fp8": 2, "fp32": 3}
_RAW = {"bf16": np.uint16, "fp8": np.uint8, "fp32": np.float32}


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
             "-D_GNU_SOURCE", _SRC, "-o", tmp, "-lpthread", "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64p = ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_int64)
        L.or_decode.restype = ctypes.c_double
        L.or_decode.argtypes = [i32, vp, ctypes.c_size_t]
        L.or_round_f32.restype = ctypes.c_float
        L.or_round_f32.argtypes = [ctypes.c_double]
        L.or_round_bf16.restype = ctypes.c_uint16
        L.or_round_bf16.argtypes = [ctypes.c_double]
        L.or_indexer_scores.restype = i32
        L.or_indexer_scores.argtypes = [i32] * 8 + [vp, vp, vp, i32, i64p, vp, i32]
        L.or_topk.restype = i32
        L.or_topk.argtypes = [i32, i32, vp, vp, i32, vp, i32]
        L.or_sparse_mla.restype = i32
        L.or_sparse_mla.argtypes = [i32] * 7 + [vp, vp, vp, ctypes.c_float, i32, i64p, vp, vp, i32]
        _lib = L
    return _lib


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _raw(a, dtype: str) -> np.ndarray:
    """View an array as the raw element encoding the C oracle reads."""
    a = np.ascontiguousarray(a)
    want = _RAW[dtype]
    if a.dtype != want:
        if a.dtype.itemsize != np.dtype(want).itemsize:
            raise TypeError(f"array of {a.dtype} cannot hold {dtype} elements")
        a = a.view(want)
    return a


# ---------------------------------------------------------------- codecs

def decode(dtype: str, raw: np.ndarray) -> np.ndarray:
    """Exact decode of raw elements to float64 (one C call per element)."""
    raw = _raw(raw, dtype).ravel()
    L = lib()
    code = DTYPE_CODES[dtype]
    return np.array([L.or_decode(code, _ptr(raw), i) for i in range(raw.size)], dtype=np.float64)


def round_bf16(x: float) -> int:
    return int(lib().or_round_bf16(float(x)))


# ---------------------------------------------------------------- indexer

def indexer_scores(q, k, w, dtypes, rows=None, nthreads=None) -> np.ndarray:
    """Scores I[t,s] = sum_h w[t,h] * relu(q[t,h].k[s]) for the listed query rows.

    q [B,Lq,H,D], k [B,Lk,D], w [B,Lq,H]; dtypes = (q_dtype, k_dtype, w_dtype).
    rows: flat query rows b*Lq+i (default all).  Returns fp32 [nrows, Lk] with
    -inf beyond each row's causal position Lk-Lq+i.
    [ITO] § "Wie der Indexer funktioniert und warum MLA entscheidend ist".
    """
    qd, kd, wd = dtypes
    B, Lq, H, D = q.shape
    Lk = k.shape[1]
    assert k.shape == (B, Lk, D) and w.shape == (B, Lq, H)
    rows = np.arange(B * Lq, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, Lk), dtype=np.float32)
    qr, kr, wr = _raw(q, qd), _raw(k, kd), _raw(w, wd)
    rc = lib().or_indexer_scores(B, Lq, Lk, H, D, DTYPE_CODES[qd], DTYPE_CODES[kd], DTYPE_CODES[wd],
                                 _ptr(qr), _ptr(kr), _ptr(wr), rows.size,
                                 rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _ptr(out),
                                 nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"or_indexer_scores failed ({rc})")
    return out


def topk(scores: np.ndarray, pos, k: int, nthreads=None) -> np.ndarray:
    """Row top-k, ties to the lower index, ascending output, -1 padding.

    scores fp32 [R, Lk]; pos[r] = last valid key of row r (None: Lk-1).
    [ITO] § "Einfache Implementierung, enorme Effizienzgewinne".
    """
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    R, Lk = scores.shape
    out = np.empty((R, k), dtype=np.int32)
    posa = None if pos is None else np.ascontiguousarray(pos, dtype=np.int32)
    rc = lib().or_topk(R, Lk, _ptr(scores), None if posa is None else _ptr(posa), k, _ptr(out),
                       nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"or_topk failed ({rc})")
    return out


def row_positions(B: int, Lq: int, Lk: int, rows=None) -> np.ndarray:
    rows = np.arange(B * Lq, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    return (Lk - Lq + rows % Lq).astype(np.int32)


def indexer_topk(q, k, w, dtypes, topk_k: int, rows=None, nthreads=None):
    """Indexer scores followed by the row top-k; returns (T [nrows, k], scores)."""
    B, Lq = q.shape[:2]
    Lk = k.shape[1]
    rows = np.arange(B * Lq, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    s = indexer_scores(q, k, w, dtypes, rows, nthreads)
    return topk(s, row_positions(B, Lq, Lk, rows), topk_k, nthreads), s


# ---------------------------------------------------------------- routing

class PatternError(ValueError):
    pass


def check_pattern(pattern: str, layer: int) -> None:
    """[ITO] § "Der unsichtbare Datenstrom": the first layer must be Full, since it
    fills the cache; every layer is Full or Shared."""
    if not pattern or any(c not in "FS" for c in pattern):
        raise PatternError(f"pattern must be a non-empty string over {{F,S}}: {pattern!r}")
    if pattern[0] != "F":
        raise PatternError("the first layer must be Full")
    if not 0 <= layer < len(pattern):
        raise PatternError(f"layer {layer} outside pattern of {len(pattern)} layers")


def route(pattern: str, layer: int, t_cache: np.ndarray, compute_fn) -> bool:
    """IndexCache routing for one layer.

    [ITO] § "Einfache Implementierung, enorme Effizienzgewinne" and [PPM]
    § "Aandacht cachen met IndexCache": a Full layer runs the indexer and top-k
    and overwrites the single cache buffer; a Shared layer runs nothing and uses
    the cache as left by the nearest preceding Full layer.  Returns True when
    the layer computed.  ``compute_fn()`` returns the layer's index set.
    """
    check_pattern(pattern, layer)
    if pattern[layer] == "F":
        t_cache[...] = compute_fn()
        return True
    return False


# ---------------------------------------------------------------- sparse MLA

def sparse_mla(q, kv, t, sm_scale: float, rows=None, nthreads=None):
    """Sparse MLA attention; q bf16 [B,Lq,Hq,Dqk], kv bf16 [B,Lk,Dqk], t [B,Lq,k].

    Returns (out bf16 bits [nrows,Hq,Dv], lse fp32 [nrows,Hq]) with V = kv[..., :Dv].
    [ITO] introduction and § "Wie der Indexer funktioniert und warum MLA entscheidend ist".
    """
    return _sparse_mla(q, kv, t, sm_scale, None, rows, nthreads)


def _sparse_mla(q, kv, t, sm_scale, Dv, rows, nthreads):
    qr, kvr = _raw(q, "bf16"), _raw(kv, "bf16")
    B, Lq, Hq, Dqk = qr.shape
    Lk = kvr.shape[1]
    Dv = Dqk if Dv is None else Dv
    t = np.ascontiguousarray(t, dtype=np.int32)
    topk_k = t.shape[-1]
    rows = np.arange(B * Lq, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, Hq, Dv), dtype=np.uint16)
    lse = np.empty((rows.size, Hq), dtype=np.float32)
    rc = lib().or_sparse_mla(B, Lq, Lk, Hq, Dqk, Dv, topk_k, _ptr(qr), _ptr(kvr), _ptr(t),
                             float(sm_scale), rows.size,
                             rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                             _ptr(out), _ptr(lse), nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"or_sparse_mla failed ({rc})")
    return out, lse


def sparse_mla_dv(q, kv, t, sm_scale: float, Dv: int, rows=None, nthreads=None):
    """As sparse_mla, with V the first Dv columns of each latent row."""
    return _sparse_mla(q, kv, t, sm_scale, Dv, rows, nthreads)


# ---------------------------------------------------------------- helpers

def overlap(t_a: np.ndarray, t_b: np.ndarray) -> np.ndarray:
    """Per-row size of the intersection of two layers' index sets (entries < 0
    are padding): the cross-layer overlap of [ITO] introduction / "Der
    unsichtbare Datenstrom" and [PPM] "Aandacht cachen met IndexCache",
    written out as a set intersection.  Works on any row order."""
    a = np.asarray(t_a).reshape(-1, np.shape(t_a)[-1])
    b = np.asarray(t_b).reshape(-1, np.shape(t_b)[-1])
    out = np.empty(a.shape[0], np.int64)
    for r in range(a.shape[0]):
        out[r] = len(set(int(x) for x in a[r] if x >= 0) & set(int(x) for x in b[r] if x >= 0))
    return out.reshape(np.shape(t_a)[:-1])


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact: shift into fp32 bits)."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 -> bf16 bits, one rounding, via the C oracle."""
    L = lib()
    flat = np.asarray(x, dtype=np.float64).ravel()
    out = np.fromiter((L.or_round_bf16(float(v)) for v in flat), dtype=np.uint16, count=flat.size)
    return out.reshape(np.shape(x))


def stack_layer(x_bits: np.ndarray, t_cache: np.ndarray, lay, sm_scale: float, Dv: int, residual_ffn: bool,
                rows=None, nthreads=None, detail=False):
    """One layer of the stack after routing (the attention and FFN steps of the
    inference loop in [ITO] § "Einfache Implementierung, enorme
    Effizienzgewinne"), X kept in bf16 between steps:
      O = SparseMLA(q, kv, T) -> X1 = bf16(X + pad(sum_h O))
        -> X = bf16(X1 W)  (plain linear map), or X = bf16(X1 + X1 W)  (``residual_ffn``).
    x_bits bf16 bits [n, Dm] holds the rows listed in ``rows`` (default: all L
    rows, in order); lay["q"] holds the attention queries of those same rows,
    [1, n, Hq, Dqk]; t_cache [1, L, k] is the whole index cache.
    Returns (X bf16 bits [n, Dm], O bf16 bits [n, Hq, Dv]) and, with ``detail``,
    the values each of the two bf16 roundings was applied to (float64 [n, Dm]:
    "pre_x1" = X + pad(sum_h O), "pre_x" = X1 W or X1 + X1 W)."""
    x = bf16_bits_to_f64(x_bits)
    n, Dm = x.shape
    L = t_cache.shape[1]
    rows = np.arange(L, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    assert rows.size == n
    t_rows = np.ascontiguousarray(t_cache.reshape(L, -1)[rows])[None]
    o_bits, _ = sparse_mla_dv(lay["q"], lay["kv"], t_rows, sm_scale, Dv, nthreads=nthreads)
    o = bf16_bits_to_f64(o_bits).reshape(n, -1, Dv).sum(axis=1)
    upd = np.zeros((n, Dm))
    upd[:, :Dv] = o
    pre_x1 = x + upd
    x1 = bf16_bits_to_f64(f64_to_bf16_bits(pre_x1))
    y = x1 @ bf16_bits_to_f64(lay["W"])
    pre_x = x1 + y if residual_ffn else y
    out = (f64_to_bf16_bits(pre_x), o_bits.reshape(n, -1, Dv))
    return out + ({"pre_x1": pre_x1, "pre_x": pre_x},) if detail else out


def stack(pattern: str, x0_bits: np.ndarray, layers, topk_k: int, sm_scale: float, Dv: int,
          residual_ffn: bool, rows=None, nthreads=None, per_layer=False):
    """Layer stack of the inference loop in [ITO] § "Einfache Implementierung, enorme
    Effizienzgewinne" (the composition is a reading; see module docstring).

    layers[l] holds seeded inputs: q_i, k_i, w (indexer, with 'idx_dtypes'),
    q, kv (attention, bf16 bits) and W (FFN stand-in, bf16 bits [Dm, Dm]).
    Per layer: route, then ``stack_layer``.  Per-layer inputs do not depend on
    X, so rows are independent: with ``rows`` given, only those query rows are
    computed; x0_bits and every layer's attention q then hold those rows only,
    in the order of ``rows``, while the indexer inputs stay whole.
    Returns (final X bf16 bits [n, Dm], list of per-layer T [1, L, k]) and,
    with ``per_layer``, also the lists of X after every layer and of every
    layer's attention output O (bf16 bits [n, Hq, Dv])."""
    L = layers[0]["q_i"].shape[1]
    t_cache = np.full((1, L, topk_k), -1, dtype=np.int32)
    rows_a = None if rows is None else np.asarray(rows, dtype=np.int64)
    x = np.asarray(x0_bits)
    ts, xs, os_ = [], [], []
    for li, lay in enumerate(layers):
        def compute(lay=lay):
            full = np.full((1, L, topk_k), -1, dtype=np.int32)
            t, _ = indexer_topk(lay["q_i"], lay["k_i"], lay["w"], lay["idx_dtypes"], topk_k, rows=rows_a,
                                nthreads=nthreads)
            full.reshape(L, topk_k)[slice(None) if rows_a is None else rows_a] = t
            return full

        route(pattern, li, t_cache, compute)
        ts.append(t_cache.copy())
        x, o = stack_layer(x, t_cache, lay, sm_scale, Dv, residual_ffn, rows=rows_a, nthreads=nthreads)
        xs.append(x)
        os_.append(o)
    return (x, ts, xs, os_) if per_layer else (x, ts)


# ---------------------------------------------------------------- serving batches over paged caches

def gather_pages(cache: np.ndarray, table_row, n: int) -> np.ndarray:
    """Rows 0..n-1 of one sequence from a page pool [num_blocks, bs, ...]: row s
    is cache[table_row[s // bs], s % bs] [SRV].  The block-table addressing,
    written out."""
    bs = cache.shape[1]
    s = np.arange(n)
    return cache[np.asarray(table_row, dtype=np.int64)[s // bs], s % bs]


def _batch_rows(query_start, rows):
    """Per sequence: (b, first row, local rows to compute as flat indices)."""
    qs = np.asarray(query_start, dtype=np.int64)
    want = None if rows is None else set(int(r) for r in rows)
    for b in range(qs.size - 1):
        r0, r1 = int(qs[b]), int(qs[b + 1])
        local = [r - r0 for r in range(r0, r1) if want is None or r in want]
        if local:
            yield b, r0, r1, np.asarray(local, dtype=np.int64)


def paged_indexer_topk(q, k_cache, w, block_table, query_start, seq_lens, dtypes, topk_k: int, rows=None,
                       nthreads=None):
    """Index sets of a serving batch [SRV]: sequence b owns rows query_start[b] ..
    query_start[b+1]-1, its last q_len positions; its keys are gathered from the
    pages and the contiguous problem (one sequence, Lq = q_len, Lk = seq_len)
    goes to indexer_topk.  q [total_q,H,D], k_cache [num_blocks,bs,D],
    w [total_q,H] raw arrays.  Returns {row: T row} for the requested rows
    (default all)."""
    out = {}
    for b, r0, r1, local in _batch_rows(query_start, rows):
        L = int(seq_lens[b])
        kb = gather_pages(k_cache, block_table[b], L)[None]
        T, _ = indexer_topk(q[None, r0:r1], kb, w[None, r0:r1], dtypes, topk_k, rows=local, nthreads=nthreads)
        for i, r in enumerate(local):
            out[r0 + int(r)] = T[i]
    return out


def paged_sparse_mla(q, kv_cache, block_table, query_start, seq_lens, t, sm_scale: float, Dv: int, rows=None,
                     nthreads=None):
    """Sparse MLA of a serving batch [SRV]: row r of sequence b attends to the
    latent rows t[r] of b (entries outside [0, seq_len_b) skipped), gathered
    from the pages; the contiguous sparse_mla_dv does the arithmetic.
    Returns {row: (out bf16 bits [Hq, Dv], lse [Hq])}."""
    out = {}
    t = np.asarray(t, dtype=np.int32)
    for b, r0, r1, local in _batch_rows(query_start, rows):
        L = int(seq_lens[b])
        kvb = gather_pages(kv_cache, block_table[b], L)[None]
        tb = t[r0:r1].copy()
        tb[(tb < 0) | (tb >= L)] = -1
        o, lse = sparse_mla_dv(q[None, r0:r1], kvb, tb[None], sm_scale, Dv, rows=local, nthreads=nthreads)
        for i, r in enumerate(local):
            out[r0 + int(r)] = (o[i], lse[i])
    return out
