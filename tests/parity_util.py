"""Shared helpers of the GPU parity tests: raw views for the oracle, the score
tolerance, and the index-set comparison rules.

Score tolerance (fp32 accumulation on both sides of an identical-input sum):
    |g - o| <= rtol * (|o| + 0.01 * max_s |o[t, s]|)
with rtol = 1e-2 for fp8 inputs and 2e-3 for bf16 inputs.  The floor term keeps
scores that cancel to nearly zero from demanding a relative match.

Index sets: identical where both sides agree on every score's order; where the
fused kernel's fp32 scores and the oracle's differ, disagreements must lie
within the score tolerance of the oracle's k-th score (theta), and the overlap
must be >= 99.9 %.
"""
import numpy as np
import torch

import oracle

RTOL = {"fp8": 1e-2, "bf16": 2e-3}


def enc_of(t: torch.Tensor) -> str:
    return {torch.float8_e4m3fn: "fp8", torch.bfloat16: "bf16", torch.float32: "fp32"}[t.dtype]


def raw(t: torch.Tensor) -> np.ndarray:
    """Host copy of a tensor's bytes in the oracle's element encoding."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def indexer_oracle(q, k, w, topk, rows=None):
    """Oracle (T, scores) for the listed flat rows of a device problem."""
    return oracle.indexer_topk(raw(q), raw(k), raw(w), (enc_of(q), enc_of(k), enc_of(w)), topk, rows=rows)


def score_tol(o_row: np.ndarray, rtol: float) -> np.ndarray:
    finite = np.isfinite(o_row)
    mx = np.abs(o_row[finite]).max() if finite.any() else 0.0
    return rtol * (np.abs(o_row) + 0.01 * mx)


def check_scores(g: np.ndarray, o: np.ndarray, rtol: float, what=""):
    """Row-wise tolerance; -inf must match exactly."""
    assert g.shape == o.shape
    for r in range(o.shape[0]):
        fin = np.isfinite(o[r])
        assert np.array_equal(np.isneginf(g[r]), np.isneginf(o[r])), f"{what} row {r}: mask differs"
        tol = score_tol(o[r], rtol)
        err = np.abs(g[r][fin].astype(np.float64) - o[r][fin])
        bad = err > tol[fin]
        assert not bad.any(), (f"{what} row {r}: {bad.sum()} scores out of tolerance, worst "
                               f"{err.max():.3g} (tol {tol[fin][np.argmax(err)]:.3g})")


def check_index_sets(tg: np.ndarray, to: np.ndarray, o_scores: np.ndarray, pos: np.ndarray, k: int,
                     rtol: float, what="", min_overlap=0.999):
    """Set comparison of T rows under the rules in the module docstring."""
    inter = 0
    total = 0
    for r in range(to.shape[0]):
        n = min(k, int(pos[r]) + 1)
        gv = tg[r, :n]
        assert np.all(tg[r, n:] == -1), f"{what} row {r}: bad padding"
        assert np.all(np.diff(gv) > 0), f"{what} row {r}: not ascending/unique"
        assert gv[0] >= 0 and gv[-1] <= pos[r], f"{what} row {r}: index outside [0, p]"
        sg, so = set(gv.tolist()), set(to[r, :n].tolist())
        inter += len(sg & so)
        total += n
        diff = sg ^ so
        if diff:
            row = o_scores[r, : pos[r] + 1].astype(np.float64)
            theta = np.sort(row)[::-1][n - 1]
            tol = rtol * (abs(theta) + 0.01 * np.abs(row).max())
            for s in diff:
                assert abs(row[s] - theta) <= tol, (f"{what} row {r}: key {s} differs with score {row[s]} "
                                                    f"far from theta {theta}")
    overlap = inter / max(total, 1)
    assert overlap >= min_overlap, f"{what}: overlap {overlap:.5f}"
    return overlap


def check_t_invariants_gpu(t: torch.Tensor, Lq: int, Lk: int, k: int):
    """Invariants of every row of T, checked on the GPU for large outputs."""
    R = t.shape[0] * t.shape[1] if t.dim() == 3 else t.shape[0]
    t2 = t.reshape(R, k)
    i = torch.arange(R, device=t.device) % Lq
    pos = (Lk - Lq + i).to(torch.int64)
    n = torch.clamp(pos + 1, max=k)
    col = torch.arange(k, device=t.device)[None, :]
    valid = col < n[:, None]
    assert bool(((t2 >= 0) == valid).all()), "valid entries and -1 padding disagree with min(k, p+1)"
    assert bool((t2[valid] <= pos[:, None].expand(-1, k)[valid]).all()), "index beyond the query position"
    if k > 1:
        inc = (t2[:, 1:] > t2[:, :-1]) | ~valid[:, 1:]
        assert bool(inc.all()), "indices not strictly ascending"


def sample_rows(L: int, k: int, n_random: int, seed: int):
    rng = np.random.default_rng(seed)
    fixed = {0, 1, min(L - 1, k - 1), min(L - 1, k), min(L - 1, k + 1), L // 2, L - 2 if L > 1 else 0, L - 1}
    rand = set(rng.choice(L, size=min(L, n_random), replace=False).tolist())
    return np.array(sorted(fixed | rand), dtype=np.int64)


# ------------------------------------------------------------ stack X bounds

U_F32 = 2.0 ** -24    # unit roundoff of fp32


def _bf16_round(v):
    """bf16 round-to-nearest-even of float64 values, by the oracle's pinned rounding."""
    return oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(v))


def _round_spread(v, d):
    """max |R(a) - R(v)| over |a - v| <= d, R = bf16 rounding: R is monotone, so
    the extremes are R(v - d) and R(v + d).  Zero wherever no rounding boundary
    lies within d of v."""
    r = _bf16_round(v)
    return np.maximum(np.abs(_bf16_round(v + d) - r), np.abs(_bf16_round(v - d) - r))


def stack_layer_bound(e_in, det, o_heads, x1_o, W, d_o, residual):
    """Element-wise bound on |X_gpu - X_oracle| after one stack layer.

    The layer computes X1 = bf16(X + pad(sum_h O)), then X = bf16(X1 W) or
    bf16(X1 + X1 W); the GPU harness sums in fp32, the oracle in fp64, and both
    round to bf16 at those two points.  Arguments:
      e_in     bound on |X_gpu - X_oracle| entering the layer (0: same input),
      det      the oracle's unrounded values at the two roundings
               (stack_layer(..., detail=True)): pre_x1, pre_x,
      o_heads  the oracle's attention output (float64 [n, Hq, Dv]),
      x1_o     the oracle's X1 (= bf16(pre_x1)),
      d_o      max |O_gpu - O_oracle| of this layer, a scalar or one value per row.
    Each rounding is bounded by the spread of R over an interval around the
    oracle's unrounded value (exact, see _round_spread):
      d1 = e_in + Hq d_o + gamma_Hq sum_h |O_h| + u32 |pre_x1|   (O terms: first Dv columns)
      e1 = spread(pre_x1, d1)
      dY = (e1 + gamma_Dm (|X1| + e1)) |W|  [+ e1 + u32 |pre_x| when residual]
      e  = spread(pre_x, dY).
    """
    n, Dm = det["pre_x1"].shape
    Hq, Dv = o_heads.shape[1:]
    d1 = np.array(e_in, dtype=np.float64) * np.ones((n, Dm))
    d_o = np.broadcast_to(np.asarray(d_o, dtype=np.float64).reshape(-1, 1), (n, 1))
    d1[:, :Dv] += Hq * d_o + Hq * U_F32 * np.abs(o_heads).sum(axis=1)
    d1 += U_F32 * np.abs(det["pre_x1"])          # the harness's fp32 add
    e1 = _round_spread(det["pre_x1"], d1)
    dy = (e1 + Dm * U_F32 * (np.abs(x1_o) + e1)) @ np.abs(W)
    if residual:
        dy = dy + e1 + U_F32 * np.abs(det["pre_x"])
    return _round_spread(det["pre_x"], dy)


def harness_layer(x, o, W, residual, torch):
    """The GPU side of one stack layer's composition (harness arithmetic, not the
    library): X1 = bf16(X + sum_h O) in fp32, then the FFN stand-in in fp32,
    rounded once to bf16.  x bf16 [n, Dm], o bf16 [n, Hq, Dv], W bf16 [Dm, Dm]."""
    Dv = o.shape[-1]
    s = torch.zeros_like(x, dtype=torch.float32)
    s[:, :Dv] = torch.sum(o, dim=1, dtype=torch.float32)
    x1 = (x.float() + s).to(torch.bfloat16).float()
    y = x1 @ W.float()
    return ((x1 + y) if residual else y).to(torch.bfloat16)
