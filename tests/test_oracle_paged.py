"""Pins of the oracle's serving-batch functions (paged caches, varlen rows)
against the contiguous oracle, which is pinned on its own."""
import numpy as np

import oracle

RNG = np.random.default_rng(7)


def test_gather_pages_hand_example():
    # pool of 3 pages of 2 rows; rows tagged by (page, slot)
    cache = np.array([[[0, 0], [0, 1]], [[1, 0], [1, 1]], [[2, 0], [2, 1]]])
    rows = oracle.gather_pages(cache, [2, 0, 1], 5)
    assert rows.tolist() == [[2, 0], [2, 1], [0, 0], [0, 1], [1, 0]]


def test_gather_pages_identity_is_contiguous():
    flat = RNG.integers(0, 1000, size=(12, 3))
    cache = flat.reshape(3, 4, 3)
    assert np.array_equal(oracle.gather_pages(cache, [0, 1, 2], 10), flat[:10])


def _batch(seq_lens, q_lens, bs, H=4, D=32, dtypes=("bf16", "bf16", "fp32")):
    B = len(seq_lens)
    pages = [(L + bs - 1) // bs for L in seq_lens]
    nblk = sum(pages) + 2
    perm = RNG.permutation(nblk)
    table = np.zeros((B, max(pages)), np.int32)
    o = 0
    for b in range(B):
        table[b, :pages[b]] = perm[o:o + pages[b]]
        o += pages[b]
    qs = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    total = int(qs[-1])
    q = oracle.f64_to_bf16_bits(RNG.normal(0, 1, (total, H, D)))
    k_cache = oracle.f64_to_bf16_bits(RNG.normal(0, 1, (nblk, bs, D)))
    w = RNG.uniform(0, 1, (total, H)).astype(np.float32)
    return q, k_cache, w, table, qs, np.asarray(seq_lens, np.int32), dtypes


def test_paged_indexer_one_sequence_identity_equals_contiguous():
    L, Lq, bs, H, D = 40, 5, 8, 4, 32
    q = oracle.f64_to_bf16_bits(RNG.normal(0, 1, (Lq, H, D)))
    k = oracle.f64_to_bf16_bits(RNG.normal(0, 1, (L, D)))
    w = RNG.uniform(0, 1, (Lq, H)).astype(np.float32)
    k_cache = k.reshape(L // bs, bs, D)
    got = oracle.paged_indexer_topk(q, k_cache, w, np.arange(L // bs)[None], [0, Lq], [L],
                                    ("bf16", "bf16", "fp32"), 16)
    ref, _ = oracle.indexer_topk(q[None], k[None], w[None], ("bf16", "bf16", "fp32"), 16)
    assert np.array_equal(np.stack([got[r] for r in range(Lq)]), ref)


def test_paged_indexer_page_permutation_invariant():
    q, k_cache, w, table, qs, sl, dt = _batch([37, 20], [3, 1], 8)
    a = oracle.paged_indexer_topk(q, k_cache, w, table, qs, sl, dt, 12)
    # move every page to a new slot of a larger pool and rewrite the table
    nblk = k_cache.shape[0]
    perm = RNG.permutation(nblk + 3)[:nblk]
    pool = np.zeros((nblk + 3,) + k_cache.shape[1:], k_cache.dtype)
    pool[perm] = k_cache
    b = oracle.paged_indexer_topk(q, pool, w, perm[table], qs, sl, dt, 12)
    assert all(np.array_equal(a[r], b[r]) for r in a)


def test_paged_indexer_batch_is_its_sequences():
    q, k_cache, w, table, qs, sl, dt = _batch([37, 20, 9], [3, 1, 2], 8)
    full = oracle.paged_indexer_topk(q, k_cache, w, table, qs, sl, dt, 12)
    for b in range(3):
        r0, r1 = qs[b], qs[b + 1]
        one = oracle.paged_indexer_topk(q[r0:r1], k_cache, w[r0:r1], table[b:b + 1], [0, r1 - r0], [sl[b]], dt, 12)
        for i in range(r1 - r0):
            assert np.array_equal(full[r0 + i], one[i])
    # rows sit at the last q_len positions: every index <= seq_len - q_len + i
    for b in range(3):
        for i in range(qs[b + 1] - qs[b]):
            row = full[qs[b] + i]
            v = row[row >= 0]
            assert v.size == min(12, sl[b] - (qs[b + 1] - qs[b]) + i + 1)
            assert v.max() <= sl[b] - (qs[b + 1] - qs[b]) + i


def test_paged_mla_identity_equals_contiguous_and_skips_out_of_range():
    L, Lq, bs, Hq, D = 24, 3, 4, 4, 32
    q = oracle.f64_to_bf16_bits(RNG.normal(0, 1, (Lq, Hq, D)))
    kv = oracle.f64_to_bf16_bits(RNG.normal(0, 1, (L, D)))
    t = RNG.integers(0, L, size=(Lq, 8)).astype(np.int32)
    got = oracle.paged_sparse_mla(q, kv.reshape(L // bs, bs, D), np.arange(L // bs)[None], [0, Lq], [L], t, 0.2, D)
    ref_o, ref_l = oracle.sparse_mla_dv(q[None], kv[None], t[None], 0.2, D)
    for r in range(Lq):
        assert np.array_equal(got[r][0], ref_o[r]) and np.array_equal(got[r][1], ref_l[r])
    # an entry beyond the sequence is skipped exactly like a -1
    t2 = t.copy()
    t2[0, 0] = L + 5
    t3 = t.copy()
    t3[0, 0] = -1
    a = oracle.paged_sparse_mla(q, kv.reshape(L // bs, bs, D), np.arange(L // bs)[None], [0, Lq], [L], t2, 0.2, D)
    b = oracle.paged_sparse_mla(q, kv.reshape(L // bs, bs, D), np.arange(L // bs)[None], [0, Lq], [L], t3, 0.2, D)
    assert np.array_equal(a[0][0], b[0][0])
