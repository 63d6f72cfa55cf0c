"""Training-free greedy choice of Full / Shared layers.

The search of itoverdose.com, "IndexCache: Wie DeepSeek O(NL²)-Kosten in
Sparse Attention um 75% reduziert", section "Training-freie Optimierung:
Greedy-Suche mit minimalem Verlust" (also parapluman.nl, "Aandacht cachen met
IndexCache"): start with every layer Full and, one step at a time, turn into
a Shared layer the Full layer whose conversion raises the loss on calibration
data the least, until the wanted number of Full layers remains.  Each step
evaluates every remaining candidate once, so a search to few Full layers
costs O(N^2) loss evaluations.

The loss is a callback: on real models it runs the network on calibration
data; any function of the pattern string works here.  Layer 0 always stays
Full (it fills the index cache).
"""
from __future__ import annotations

from typing import Callable, List, Tuple


def greedy_pattern(n_layers: int, loss_fn: Callable[[str], float], n_full: int = 1
                   ) -> List[Tuple[str, float]]:
    """Returns the search path [(pattern, loss), ...] from all-Full down to
    ``n_full`` Full layers.  Ties between candidates go to the lower layer."""
    if n_layers < 1:
        raise ValueError("n_layers must be >= 1")
    if not 1 <= n_full <= n_layers:
        raise ValueError("n_full must lie in [1, n_layers]")
    pattern = ["F"] * n_layers
    path = [("".join(pattern), float(loss_fn("".join(pattern))))]
    while pattern.count("F") > n_full:
        best = None
        for layer in range(1, n_layers):
            if pattern[layer] != "F":
                continue
            cand = pattern.copy()
            cand[layer] = "S"
            c = "".join(cand)
            loss = float(loss_fn(c))
            if best is None or loss < best[1]:
                best = (c, loss)
        pattern = list(best[0])
        path.append(best)
    return path


def stack_deviation_loss(stack):
    """Loss for ``greedy_pattern`` from a layer stack run through the library
    (``stack.Stack``): the relative deviation of a pattern's final X from the
    all-Full stack's final X.  Without calibration data or trained weights this
    is the one loss the synthetic stack offers: how much the model's output
    moves when layers reuse the cached index set.  Evaluations are memoised per
    pattern."""
    from .stack import relative_deviation

    n = len(stack.layers)
    ref = stack.run("F" * n).clone()
    memo = {}

    def loss(pattern: str) -> float:
        if pattern not in memo:
            memo[pattern] = relative_deviation(stack.run(pattern), ref)
        return memo[pattern]

    loss.memo = memo
    return loss
