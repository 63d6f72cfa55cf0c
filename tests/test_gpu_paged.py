"""GPU parity of the serving-batch entry points (varlen rows over paged caches)
through the C ABI: against the contiguous entry points on the same logical
data (identical results), and against the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_lightning_amd as sa
from parity_util import RTOL, check_index_sets, enc_of, raw

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def make_batch(seq_lens, q_lens, bs, D, dtype, H=64, seed=0, spare_pages=3):
    """Page pool with each sequence's pages at random slots, packed q and w."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    B = len(seq_lens)
    pages = [(L + bs - 1) // bs for L in seq_lens]
    nblk = sum(pages) + spare_pages
    perm = torch.randperm(nblk, generator=g)
    table = torch.zeros(B, max(pages) + 1, dtype=torch.int32)
    o = 0
    for b in range(B):
        table[b, :pages[b]] = perm[o:o + pages[b]]
        o += pages[b]
    qs = torch.tensor([0] + list(np.cumsum(q_lens)), dtype=torch.int32)
    total = int(qs[-1])
    if dtype == torch.float8_e4m3fn:
        q = (torch.randn(total, H, D, generator=g) / math.sqrt(D)).to(dtype)
        k_cache = (torch.randn(nblk, bs, D, generator=g) / math.sqrt(D)).to(dtype)
        w = (torch.randn(total, H, generator=g) * 0.1).to(torch.bfloat16)
    else:
        q = torch.randn(total, H, D, generator=g).to(dtype)
        k_cache = torch.randn(nblk, bs, D, generator=g).to(dtype)
        w = torch.rand(total, H, generator=g)
    sl = torch.tensor(seq_lens, dtype=torch.int32)
    return [x.to(DEV) for x in (q, k_cache, w, table, qs, sl)]


def contiguous_keys(k_cache, table, L):
    bs = k_cache.shape[1]
    s = torch.arange(L, device=k_cache.device)
    return k_cache[table[s // bs].long(), s % bs]


@pytest.mark.parametrize("bs", [64, 256])
def test_paged_decode_equals_contiguous(bs):
    # decode rows (one query per sequence, all of the same length): the paged
    # entry point must return exactly what idx_score_topk returns on the
    # gathered contiguous cache
    L, B, topk = 3000, 4, 256
    q, k_cache, w, table, qs, sl = make_batch([L] * B, [1] * B, bs, 128, torch.float8_e4m3fn, seed=bs)
    kc = torch.stack([contiguous_keys(k_cache, table[b], L) for b in range(B)])
    t_dense = sa.idx_score_topk(q.view(B, 1, 64, 128), kc, w.view(B, 1, 64), topk)
    t_paged = sa.idx_score_topk_paged(q, k_cache, table, qs, sl, w, topk, max_seq_len=L)
    torch.cuda.synchronize()
    assert torch.equal(t_dense.view(B, topk), t_paged)


@pytest.mark.parametrize("enc,D,bs", [("fp8", 128, 64), ("fp8", 128, 128), ("bf16", 64, 64)])
def test_paged_mixed_batch_vs_oracle(enc, D, bs):
    # decode tokens and prefill chunks in one batch, sequences of uneven length
    seq_lens = [2100, 777, 1500, 64, 130]
    q_lens = [1, 5, 1, 3, 0 + 2]
    dtype = torch.float8_e4m3fn if enc == "fp8" else torch.bfloat16
    topk = 512
    q, k_cache, w, table, qs, sl = make_batch(seq_lens, q_lens, bs, D, dtype, seed=len(enc) + D + bs)
    maxL = max(seq_lens) + 37
    t = sa.idx_score_topk_paged(q, k_cache, table, qs, sl, w, topk, max_seq_len=maxL)
    torch.cuda.synchronize()
    tg = t.cpu().numpy()
    qr, kr, wr = raw(q), raw(k_cache), raw(w)
    dts = (enc_of(q), enc_of(k_cache), enc_of(w))
    tb, qsn = table.cpu().numpy(), qs.cpu().numpy()
    for b, L in enumerate(seq_lens):
        r0, r1 = int(qsn[b]), int(qsn[b + 1])
        kb = oracle.gather_pages(kr, tb[b], L)[None]
        to, so = oracle.indexer_topk(qr[None, r0:r1], kb, wr[None, r0:r1], dts, topk)
        pos = oracle.row_positions(1, r1 - r0, L)
        check_index_sets(tg[r0:r1], to, so, pos, topk, RTOL[enc], what=f"seq {b}")
    # the oracle's own serving-batch function agrees with the per-sequence calls
    ob = oracle.paged_indexer_topk(qr, kr, wr, tb, qsn, sl.cpu().numpy(), dts, topk, rows=[0, 1, 6])
    assert set(ob) == {0, 1, 6}


def test_paged_route_full_then_shared():
    q, k_cache, w, table, qs, sl = make_batch([900, 400], [1, 2], 64, 128, torch.float8_e4m3fn, seed=3)
    t_cache = torch.full((3, 128), -7, dtype=torch.int32, device=DEV)
    assert sa.idx_cache_route_paged("FS", 0, q, k_cache, table, qs, sl, w, t_cache, max_seq_len=900)
    torch.cuda.synchronize()
    first = t_cache.clone()
    assert (first != -7).all()
    assert not sa.idx_cache_route_paged("FS", 1, None, None, None, None, None, None, t_cache, max_seq_len=900)
    torch.cuda.synchronize()
    assert torch.equal(first, t_cache)
    ref = sa.idx_score_topk_paged(q, k_cache, table, qs, sl, w, 128, max_seq_len=900)
    torch.cuda.synchronize()
    assert torch.equal(ref, first)


# ---- prefill chunks: the fused kernel with page lookups (more than four rows
# per sequence on average, fp8 with 64 heads of 128)

def test_paged_fused_prefill_equals_contiguous():
    """One sequence whose rows are all its positions, pages at random slots:
    the fused paged path runs the same arithmetic as the contiguous fused
    kernel on the gathered keys, so T is identical."""
    L, topk = 6000, 2048
    q, k_cache, w, table, qs, sl = make_batch([L], [L], 64, 128, torch.float8_e4m3fn, seed=21)
    kc = contiguous_keys(k_cache, table[0], L)[None]
    t_dense = sa.idx_score_topk(q.view(1, L, 64, 128), kc, w.view(1, L, 64), topk)
    t_paged = sa.idx_score_topk_paged(q, k_cache, table, qs, sl, w, topk, max_seq_len=L)
    torch.cuda.synchronize()
    assert torch.equal(t_dense.view(L, topk), t_paged)


def _check_batch_sampled(q, k_cache, w, table, qs, sl, t, seq_lens, topk, n_rows, seed):
    tg = t.cpu().numpy()
    qr, kr, wr = raw(q), raw(k_cache), raw(w)
    dts = (enc_of(q), enc_of(k_cache), enc_of(w))
    tb, qsn = table.cpu().numpy(), qs.cpu().numpy()
    rng = np.random.default_rng(seed)
    for b, L in enumerate(seq_lens):
        r0, r1 = int(qsn[b]), int(qsn[b + 1])
        n = r1 - r0
        if n == 0:
            continue
        local = np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=min(n, n_rows), replace=False)]))
        kb = oracle.gather_pages(kr, tb[b], L)[None]
        to, so = oracle.indexer_topk(qr[None, r0:r1], kb, wr[None, r0:r1], dts, topk, rows=local)
        pos = oracle.row_positions(1, n, L, local)
        check_index_sets(tg[r0 + local], to, so, pos, topk, RTOL["fp8"], what=f"seq {b}")


def test_paged_fused_chunk_4k_vs_oracle():
    """A serving batch with a 4096-query prefill chunk (the last 4096 positions
    of a 20,000-token sequence), a shorter chunk and decode tokens, on
    sampled rows of every sequence."""
    seq_lens, q_lens, topk = [20000, 9000, 5000, 3333], [4096, 700, 1, 3], 2048
    q, k_cache, w, table, qs, sl = make_batch(seq_lens, q_lens, 64, 128, torch.float8_e4m3fn, seed=22)
    t = sa.idx_score_topk_paged(q, k_cache, table, qs, sl, w, topk, max_seq_len=20000)
    torch.cuda.synchronize()
    _check_batch_sampled(q, k_cache, w, table, qs, sl, t, seq_lens, topk, 40, seed=23)


def test_paged_fused_beyond_16bit_keys_vs_oracle():
    """A sequence past 65,536 keys takes the fused kernel's 32-bit index form."""
    seq_lens, q_lens, topk = [70000, 1000], [600, 50], 2048
    q, k_cache, w, table, qs, sl = make_batch(seq_lens, q_lens, 128, 128, torch.float8_e4m3fn, seed=24)
    t = sa.idx_score_topk_paged(q, k_cache, table, qs, sl, w, topk, max_seq_len=70000)
    torch.cuda.synchronize()
    _check_batch_sampled(q, k_cache, w, table, qs, sl, t, seq_lens, topk, 12, seed=25)


@pytest.mark.parametrize("Hq,bs", [(64, 16), (128, 64), (16, 64)])
def test_paged_mla_vs_oracle(Hq, bs):
    seq_lens, q_lens, topk = [1000, 333, 2048], [1, 3, 2], 300
    g = torch.Generator(device="cpu").manual_seed(Hq + bs)
    B = len(seq_lens)
    pages = [(L + bs - 1) // bs for L in seq_lens]
    nblk = sum(pages) + 5
    perm = torch.randperm(nblk, generator=g)
    table = torch.zeros(B, max(pages), dtype=torch.int32)
    o = 0
    for b in range(B):
        table[b, :pages[b]] = perm[o:o + pages[b]]
        o += pages[b]
    qs = torch.tensor([0] + list(np.cumsum(q_lens)), dtype=torch.int32)
    total = int(qs[-1])
    q = torch.randn(total, Hq, 576, generator=g).to(torch.bfloat16)
    kv = torch.randn(nblk, bs, 576, generator=g).to(torch.bfloat16)
    t = torch.empty(total, topk, dtype=torch.int32)
    for b in range(B):
        for r in range(int(qs[b]), int(qs[b + 1])):
            t[r] = torch.randint(0, seq_lens[b], (topk,), generator=g)
    t[0, :5] = -1                      # skipped entries
    t[1, 7] = seq_lens[1] + 3          # beyond the sequence: skipped as well
    sl = torch.tensor(seq_lens, dtype=torch.int32)
    dev = [x.to(DEV) for x in (q, kv, table, qs, sl, t)]
    lse = torch.empty(total, Hq, dtype=torch.float32, device=DEV)
    out, _ = sa.sparse_mla_attn_paged(*dev, 1 / math.sqrt(576), 512, lse=lse)
    torch.cuda.synchronize()
    ref = oracle.paged_sparse_mla(raw(q), raw(kv), table.numpy(), qs.numpy(), sl.numpy(), t.numpy(),
                                  1 / math.sqrt(576), 512)
    go = oracle.bf16_bits_to_f64(raw(out))
    gl = lse.cpu().numpy()
    for r in range(total):
        ro, rl = ref[r]
        err = np.abs(go[r] - oracle.bf16_bits_to_f64(ro)).max()
        assert err <= 2e-2, f"row {r}: max-abs {err}"
        assert np.allclose(gl[r], rl, rtol=1e-4, atol=1e-3)
