"""Pins for the CPU oracle: each test checks it against something other than itself.

Pins used (none retypes the oracle's formula):
  * codecs: every fp8 e4m3fn and bf16 code against torch's own decoders; the
    bf16 rounding against a brute-force nearest-neighbour search.
  * indexer scores: the hand-worked 8-token example (tests/golden), the
    closed-form recency / reverse / tie inputs, and the one-head unit-weight
    case that reduces to numpy inner products.
  * top-k: full sort and an independent repeated-argmax selection on many
    tiny random cases with frequent ties.
  * routing: the hand-worked example's Full/Shared layers and the pattern rules.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_indexer_lightning_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ codecs

def test_fp8_decode_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode("fp8", codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def test_bf16_decode_every_code_matches_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode("bf16", codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def _bf16_value(bits: int) -> float:
    return float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0])


def _nearest_bf16_brute(x: float) -> int:
    """Nearest bf16 to x by exhaustive comparison of the neighbouring codes."""
    f = np.float32(x)
    base = int(np.array([f], dtype=np.float32).view(np.uint32)[0]) >> 16
    best = None
    for b in range(base - 2, base + 3):
        b &= 0xFFFF
        v = _bf16_value(b)
        if math.isnan(v):
            continue
        d = abs(v - x)
        if best is None or d < best[0] or (d == best[0] and (b & 1) == 0 and (best[1] & 1) == 1):
            best = (d, b)
    return best[1]


def test_bf16_round_nearest_even_against_brute_force():
    rng = np.random.default_rng(7)
    xs = list(rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000))
    # exact midpoints between neighbouring bf16 values: ties go to even
    for bits in [0x3F80, 0x3F81, 0x4000, 0x4001, 0xBF85, 0x0001, 0x0080]:
        xs.append((_bf16_value(bits) + _bf16_value(bits + 1)) / 2.0)
    # values just above/below midpoints (only representable in double)
    xs.append((_bf16_value(0x3F80) + _bf16_value(0x3F81)) / 2.0 + 2.0 ** -40)
    xs.append((_bf16_value(0x3F81) + _bf16_value(0x3F82)) / 2.0 - 2.0 ** -40)
    for x in xs:
        assert oracle.round_bf16(x) == _nearest_bf16_brute(float(x)), x


# ------------------------------------------------------------ hand example

def _hand():
    with open(os.path.join(GOLDEN, "hand_example_8tok.json")) as f:
        return json.load(f)


def _hand_layer_inputs(g, layer, dtype="fp32", H=None, D=None):
    L, Hh, Dh = g["L"], g["H"], g["D"]
    H = H or Hh
    D = D or Dh
    k = np.zeros((1, L, D), np.float32)
    k[0, :, :Dh] = np.array(g["keys"], np.float32)
    q = np.zeros((1, L, H, D), np.float32)
    for h in range(Hh):
        q[0, :, h, :Dh] = np.array(g["q_per_row"][h], np.float32)
    w = np.zeros((1, L, H), np.float32)
    ww = g["w_even_odd_by_layer"][str(layer)]
    for t in range(L):
        w[0, t, :Hh] = ww["even"] if t % 2 == 0 else ww["odd"]
    return q, k, w


def test_hand_example_scores_and_topk():
    g = _hand()
    for layer in ("0", "2"):
        q, k, w = _hand_layer_inputs(g, int(layer))
        t, s = oracle.indexer_topk(q, k, w, ("fp32", "fp32", "fp32"), g["topk"])
        exp = g["expected"][layer]
        for row in range(g["L"]):
            assert list(s[row, : row + 1]) == exp["scores"][row], (layer, row)
            assert np.all(np.isneginf(s[row, row + 1:]))
        assert t.tolist() == exp["T"], layer


def test_hand_example_padded_to_native_shape_in_bf16_and_fp8():
    """Zero heads (w = 0) and zero dimensions change nothing; fp8/bf16 hold the values exactly."""
    g = _hand()
    for layer in ("0", "2"):
        for enc, H, D in (("bf16", 4, 32), ("fp8", 64, 128)):
            q, k, w = _hand_layer_inputs(g, int(layer), H=H, D=D)
            tq = torch.from_numpy(q).to(torch.bfloat16 if enc == "bf16" else torch.float8_e4m3fn)
            tk = torch.from_numpy(k).to(tq.dtype)
            tw = torch.from_numpy(w).to(torch.float32 if enc == "bf16" else torch.bfloat16)
            wd = "fp32" if enc == "bf16" else "bf16"
            t, _ = oracle.indexer_topk(tq.view(torch.uint8 if enc == "fp8" else torch.int16).numpy(),
                                       tk.view(torch.uint8 if enc == "fp8" else torch.int16).numpy(),
                                       tw.view(torch.int16).numpy() if wd == "bf16" else tw.numpy(),
                                       (enc, enc, wd), g["topk"])
            assert t.tolist() == g["expected"][layer]["T"], (layer, enc)


def test_hand_example_routing():
    g = _hand()
    L, k = g["L"], g["topk"]
    cache = np.full((L, k), 7777, np.int32)
    seen = []
    for layer in range(len(g["pattern"])):
        q, k_, w = _hand_layer_inputs(g, layer)

        def compute(q=q, k_=k_, w=w):
            return oracle.indexer_topk(q, k_, w, ("fp32",) * 3, k)[0]

        addr = cache.ctypes.data
        did = oracle.route(g["pattern"], layer, cache, compute)
        assert cache.ctypes.data == addr  # the one buffer, never replaced
        assert did == (g["pattern"][layer] == "F")
        seen.append(cache.copy())
        src = g["expected"]["T_by_layer"][str(layer)]
        assert cache.tolist() == g["expected"][src]["T"], layer
    assert np.array_equal(seen[0], seen[1]) and np.array_equal(seen[2], seen[3])


def test_pattern_rules():
    cache = np.zeros((1, 1), np.int32)
    for bad, layer in (("SFFF", 0), ("FSXF", 1), ("", 0), ("FS", 2), ("FS", -1)):
        with pytest.raises(oracle.PatternError):
            oracle.route(bad, layer, cache, lambda: cache)


# ------------------------------------------------------------ closed forms

@pytest.mark.parametrize("enc", ["bf16", "fp8"])
@pytest.mark.parametrize("kind", ["recency", "reverse", "ties", "negzero_ties"])
def test_closed_form_indexer(enc, kind):
    L, H, D, k = 300, 4, 32 if enc == "bf16" else 128, 64
    q, kk, w = inputs.closed_form_indexer(1, L, H, D, enc, kind)
    wd = "fp32" if enc == "bf16" else "bf16"
    rawq = q.view(torch.uint8 if enc == "fp8" else torch.int16).numpy()
    rawk = kk.view(torch.uint8 if enc == "fp8" else torch.int16).numpy()
    raww = w.numpy() if wd == "fp32" else w.view(torch.int16).numpy()
    t, s = oracle.indexer_topk(rawq, rawk, raww, (enc, enc, wd), k)
    for p in range(L):
        if kind == "recency":
            assert np.array_equal(s[p, : p + 1], np.arange(p + 1, dtype=np.float32))
        elif kind == "reverse":
            assert np.array_equal(s[p, : p + 1], -np.arange(p + 1, dtype=np.float32))
        else:
            assert np.all(s[p, : p + 1] == 0.0)
            assert not np.any(np.signbit(s[p, : p + 1]))  # -0 canonicalised
        n = min(k, p + 1)
        if kind == "recency":
            want = list(range(p + 1 - n, p + 1))
        else:
            want = list(range(n))
        assert t[p, :n].tolist() == want and np.all(t[p, n:] == -1), (kind, p)


def test_single_head_unit_weight_is_relu_inner_product():
    """With one head and w = 1 the score is max(0, q.k), an inner product numpy computes."""
    rng = np.random.default_rng(3)
    L, D = 97, 16
    q = rng.integers(-4, 5, (1, L, 1, D)).astype(np.float32)
    k = rng.integers(-4, 5, (1, L, D)).astype(np.float32)
    w = np.ones((1, L, 1), np.float32)
    s = oracle.indexer_scores(q, k, w, ("fp32",) * 3)
    ip = np.maximum(q[0, :, 0, :] @ k[0].T, 0.0)
    for t in range(L):
        assert np.array_equal(s[t, : t + 1], ip[t, : t + 1].astype(np.float32))
    # top-k against numpy's stable argsort of (-score, index)
    kk = 10
    tk = oracle.topk(s, np.arange(L, dtype=np.int32), kk)
    for t in range(kk, L):
        order = np.argsort(-ip[t, : t + 1], kind="stable")[:kk]
        assert tk[t].tolist() == sorted(order.tolist())


def test_linear_in_weights_one_hot_heads():
    """w = e_h picks max(0, q_h.k) out of the sum; negative weights flip it."""
    rng = np.random.default_rng(11)
    L, H, D = 40, 3, 8
    q = rng.integers(-3, 4, (1, L, H, D)).astype(np.float32)
    k = rng.integers(-3, 4, (1, L, D)).astype(np.float32)
    for h in range(H):
        for sign in (1.0, -2.0):
            w = np.zeros((1, L, H), np.float32)
            w[..., h] = sign
            s = oracle.indexer_scores(q, k, w, ("fp32",) * 3)
            ip = sign * np.maximum(q[0, :, h, :] @ k[0].T, 0.0)
            for t in range(L):
                got = s[t, : t + 1]
                assert np.array_equal(got, (ip[t, : t + 1] + 0.0).astype(np.float32))


# ------------------------------------------------------------ top-k brute force

def _topk_sort(s, p, k):
    n = p + 1
    if n <= k:
        return list(range(n)) + [-1] * (k - n)
    order = sorted(range(n), key=lambda j: (-float(s[j]), j))[:k]
    return sorted(order)


def _topk_argmax(s, p, k):
    n = p + 1
    if n <= k:
        return list(range(n)) + [-1] * (k - n)
    taken = np.zeros(n, bool)
    out = []
    for _ in range(k):
        best = -1
        for j in range(n):
            if taken[j]:
                continue
            if best < 0 or s[j] > s[best]:
                best = j
        taken[best] = True
        out.append(best)
    return sorted(out)


def test_topk_brute_force_many_tiny_cases():
    rng = np.random.default_rng(2024)
    for case in range(3000):
        L = int(rng.integers(1, 40))
        k = int(rng.integers(1, 12))
        vals = rng.integers(-3, 4, (L, L)).astype(np.float32)
        if case % 5 == 0:
            vals[vals == 0] = -0.0  # negative zero must tie with +0
        pos = np.arange(L, dtype=np.int32)
        got = oracle.topk(vals, pos, k, nthreads=1)
        for r in range(L):
            want = _topk_sort(vals[r], r, k)
            assert got[r].tolist() == want, (case, r)
            if case % 10 == 0:
                assert _topk_argmax(vals[r], r, k) == want


def test_topk_invariants_random_rows():
    rng = np.random.default_rng(5)
    R, Lk, k = 64, 500, 37
    s = rng.standard_normal((R, Lk)).astype(np.float32)
    pos = rng.integers(0, Lk, R).astype(np.int32)
    t = oracle.topk(s, pos, k)
    for r in range(R):
        n = min(k, pos[r] + 1)
        row = t[r]
        assert np.all(row[n:] == -1) and np.all(row[:n] >= 0) and np.all(row[:n] <= pos[r])
        assert np.all(np.diff(row[:n]) > 0)
        if pos[r] + 1 > k:
            chosen = s[r, row]
            rest = np.delete(s[r, : pos[r] + 1], row)
            assert chosen.min() >= rest.max()


def test_topk_row_with_no_valid_key():
    """pos = -1 means the row has no key: the index set is empty, all padding."""
    s = np.array([[3.0, 1.0, 2.0], [3.0, 1.0, 2.0], [3.0, 1.0, 2.0]], np.float32)
    pos = np.array([-1, 0, 2], np.int32)
    t = oracle.topk(s, pos, 2)
    assert t.tolist() == [[-1, -1], [0, -1], [0, 2]]


# ------------------------------------------------------------ batches, Lq < Lk

def _batched_closed_form(enc):
    """B = 3 sequences of Lk = 40 keys, Lq = 5 queries each (positions 35..39).
    Keys of sequence b hold the base-8 digits of v = s + 100 b; head 0 of query
    (b, i) is a*(1, 8, 64) on digits 0-2, head 1 is a*(1, 8, 64) on digits 3-5,
    a = 1 + (b + i) mod 3.  Head weights (1, 512) (sequence 1: (-1, -512)).
    Then q_0.k = a (v mod 512), q_1.k = a (v div 512), both >= 0, so
    I[(b, i), s] = +-a (s + 100 b) exactly for s <= 35 + i."""
    B, Lq, Lk, H, D = 3, 5, 40, 2, 8
    q = np.zeros((B, Lq, H, D), np.float32)
    k = np.zeros((B, Lk, D), np.float32)
    w = np.zeros((B, Lq, H), np.float32)
    a = np.zeros((B, Lq))
    for b in range(B):
        for s in range(Lk):
            v = s + 100 * b
            for j in range(6):
                k[b, s, j] = (v >> (3 * j)) & 7
        for i in range(Lq):
            a[b, i] = 1 + (b + i) % 3
            q[b, i, 0, :3] = a[b, i] * np.array([1, 8, 64])
            q[b, i, 1, 3:6] = a[b, i] * np.array([1, 8, 64])
            w[b, i] = (-1.0, -512.0) if b == 1 else (1.0, 512.0)
    if enc == "fp32":
        return (q, k, w), ("fp32",) * 3, a
    tq = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    tk = torch.from_numpy(k).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    tw = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy()
    return (tq, tk, tw), ("fp8", "fp8", "bf16"), a


@pytest.mark.parametrize("enc", ["fp32", "fp8"])
def test_batched_rows_and_offset_positions(enc):
    (q, k, w), dts, a = _batched_closed_form(enc)
    B, Lq, Lk, topk = 3, 5, 40, 4
    # every flat row, in a scrambled order, to pin row -> (b, i) as well
    rows = np.array([7, 0, 14, 3, 10, 5, 12, 1, 9, 2, 13, 6, 11, 4, 8], np.int64)
    t, s = oracle.indexer_topk(q, k, w, dts, topk, rows=rows)
    for r, flat in enumerate(rows):
        b, i = divmod(int(flat), Lq)
        p = Lk - Lq + i
        sign = -1.0 if b == 1 else 1.0
        want = sign * a[b, i] * (np.arange(p + 1) + 100 * b)
        assert np.array_equal(s[r, : p + 1], want.astype(np.float32)), (b, i)
        assert np.all(np.isneginf(s[r, p + 1:])), (b, i)
        exp_t = list(range(topk)) if b == 1 else list(range(p + 1 - topk, p + 1))
        assert t[r].tolist() == exp_t, (b, i)


# ------------------------------------------------------------ fp32 rounding

def _f32_from_bits(u: int) -> float:
    return float(np.array([u], dtype=np.uint32).view(np.float32)[0])


def _nearest_f32_brute(x) -> float:
    """Nearest fp32 to the exact rational x (ties to the even code), by
    comparing exact distances to the neighbouring codes of a first guess."""
    from fractions import Fraction
    x = Fraction(x)
    if x == 0:
        return 0.0
    guess = np.float32(float(x))
    base = int(np.array([guess], dtype=np.float32).view(np.uint32)[0])
    best = None
    for u in range(base - 3, base + 4):
        u &= 0xFFFFFFFF
        v = _f32_from_bits(u)
        if not math.isfinite(v):
            continue
        d = abs(Fraction(v) - x)
        if best is None or d < best[0] or (d == best[0] and (u & 1) == 0 and (best[1] & 1) == 1):
            best = (d, u)
    return _f32_from_bits(best[1])


def test_round_f32_nearest_even_against_brute_force():
    rng = np.random.default_rng(17)
    L = oracle.lib()
    xs = list(rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 38, 2000))
    xs += list(rng.uniform(-4, 4, 500))                       # non-integer, mantissa bits beyond fp32
    for u in [0x3F800000, 0x3F800001, 0x40490FDB, 0x00000001, 0x00800000, 0x7F7FFFFE, 0xBF800003]:
        lo, hi = _f32_from_bits(u), _f32_from_bits(u + 1)
        mid = (lo + hi) / 2.0                                  # exact in double: a tie
        xs += [mid, mid + abs(mid) * 2.0 ** -40, mid - abs(mid) * 2.0 ** -40]
    for x in xs:
        got = L.or_round_f32(float(x))
        want = _nearest_f32_brute(float(x))
        assert np.float32(got).tobytes() == np.float32(want).tobytes(), x


def test_scores_round_once_to_nearest_even():
    """Non-integer scores: the exact value of sum_h w * max(0, q.k) (Python
    fractions) rounded to the nearest fp32 by brute force.  Inputs have at
    most 12 significant bits, so the exact score has at most ~40 and every
    rounding direction (down, up, tie to even) occurs."""
    from fractions import Fraction
    rng = np.random.default_rng(23)
    Lq, H, D = 24, 4, 6
    q = (rng.integers(-2047, 2048, (1, Lq, H, D)) / 64.0).astype(np.float32)
    k = (rng.integers(-2047, 2048, (1, Lq, D)) / 128.0).astype(np.float32)
    w = (rng.integers(-2047, 2048, (1, Lq, H)) / 1024.0).astype(np.float32)
    # crafted rows: q.k = 1 + 2^-11 + 2^-24 (a tie: even rounds down) and
    # q.k = 1 + 2^-11 + 2^-23 + 2^-24 + 2^-35 (above the tie: rounds up)
    q[0, 0] = 0.0; w[0, 0] = 0.0; q[0, 0, 0, 0] = 1 + 2.0 ** -12; w[0, 0, 0] = 1.0
    q[0, 1] = 0.0; w[0, 1] = 0.0; q[0, 1, 0, 0] = 1 + 2.0 ** -12; w[0, 1, 0] = 1.0
    k[0, 0] = 0.0; k[0, 0, 0] = 1 + 2.0 ** -12
    k[0, 1] = 0.0; k[0, 1, 0] = 1 + 2.0 ** -12 + 2.0 ** -23
    s = oracle.indexer_scores(q, k, w, ("fp32",) * 3)
    assert s[0, 0] == np.float32(1 + 2.0 ** -11)
    assert s[1, 1] == np.float32(1 + 2.0 ** -11 + 2.0 ** -22)
    inexact = 0
    for t in range(Lq):
        for j in range(t + 1):
            exact = Fraction(0)
            for h in range(H):
                dot = sum(Fraction(float(q[0, t, h, d])) * Fraction(float(k[0, j, d])) for d in range(D))
                exact += Fraction(float(w[0, t, h])) * max(dot, Fraction(0))
            want = _nearest_f32_brute(exact)
            inexact += Fraction(want) != exact
            assert np.float32(s[t, j]).tobytes() == np.float32(want).tobytes(), (t, j, float(exact))
    assert inexact > 100   # the pin exercises rounding, not just exact sums
