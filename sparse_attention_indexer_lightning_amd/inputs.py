"""Seeded synthetic workloads for the indexer, IndexCache routing and sparse MLA.

This module only draws random tensors of the right shapes, distributions and
encodings.  It holds none of the method's arithmetic and is the one module that
both the HIP path's callers and the oracle's callers share.

Recipe (the same on every device):
  * Every tensor is drawn from its own ``torch.Generator`` seeded with
    ``mix(seed, layer, tensor_id)``; on a GPU the draw runs on the GPU
    (Philox), on the CPU it runs on the CPU.  Values are drawn in fp32 and cast
    once to the stored encoding (fp8 e4m3fn, bf16 or fp32).
  * Indexer: q, k ~ N(0,1) scaled by 1/sqrt(d_I) in fp8 (or N(0,1) in bf16 for
    the tiny stack), head weights w ~ N(0, 0.1^2) in bf16 (or U(0,1) in fp32).
  * Attention: q and the latent KV rows ~ N(0,1) in bf16.
  * FFN stand-in: W ~ N(0,1)/sqrt(D) in bf16; X0 ~ N(0,1) in bf16.
  * Closed-form inputs (recency / reverse / ties) build scores with a known
    order; see ``closed_form_indexer``.

The oracle never depends on the generator: it reads back the exact bytes the
kernels consumed.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

FP8 = torch.float8_e4m3fn


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Lq: int
    Lk: int
    H: int          # indexer heads
    D: int          # indexer head dim
    topk: int
    idx_dtype: str  # "fp8" or "bf16" for q and k
    w_dtype: str    # "bf16" or "fp32"
    seed: int
    layers: int = 1
    pattern: str = "F"
    Hq: int = 0     # attention heads (0: no attention in this workload)
    Dqk: int = 0
    Dv: int = 0
    Dm: int = 0     # model width of the stack (0: no stack)
    residual_ffn: bool = False
    notes: str = field(default="", compare=False)


WORKLOADS = {
    "tiny_stack": Workload("tiny_stack", 1, 512, 512, 4, 32, 64, "bf16", "fp32", 0, layers=4,
                           pattern="FSSS", Hq=4, Dqk=32, Dv=32, Dm=32, residual_ffn=False),
    "prefill_8k": Workload("prefill_8k", 1, 8192, 8192, 64, 128, 2048, "fp8", "bf16", 1),
    "prefill_64k": Workload("prefill_64k", 1, 65536, 65536, 64, 128, 2048, "fp8", "bf16", 2),
    "decode_200k": Workload("decode_200k", 32, 1, 200000, 64, 128, 2048, "fp8", "bf16", 3,
                            Hq=128, Dqk=576, Dv=512),
    "stack_32k": Workload("stack_32k", 1, 32768, 32768, 64, 128, 2048, "fp8", "bf16", 4, layers=16,
                          pattern="FSSS" * 4, Hq=128, Dqk=576, Dv=512, Dm=7168, residual_ffn=True),
}

# tensor ids inside one (seed, layer)
T_Q_IDX, T_K_IDX, T_W_IDX, T_Q_ATT, T_KV_ATT, T_W_FFN, T_X0 = range(7)


def mix(seed: int, layer: int, tensor_id: int) -> int:
    """A 63-bit seed for one tensor of one layer (splitmix64 finaliser)."""
    z = (seed * 0x9E3779B97F4A7C15 + layer * 0xBF58476D1CE4E5B9 + tensor_id * 0x94D049BB133111EB + 1)
    z &= (1 << 64) - 1
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & ((1 << 64) - 1)
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & ((1 << 64) - 1)
    return (z ^ (z >> 31)) & ((1 << 63) - 1)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


_CHUNK = 1 << 26  # elements drawn per chunk, bounds fp32 temporaries to 256 MB


def normal(shape, std: float, out_dtype, device, seed: int) -> torch.Tensor:
    """N(0, std^2) drawn in fp32 chunks, cast once to ``out_dtype``."""
    n = math.prod(shape)
    out = torch.empty(n, dtype=out_dtype, device=device)
    g = _gen(device, seed)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        x = torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        out[s:e] = x.to(out_dtype)
    return out.view(shape)


def uniform(shape, out_dtype, device, seed: int) -> torch.Tensor:
    g = _gen(device, seed)
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32).to(out_dtype)


def _torch_dtype(name: str):
    return {"fp8": FP8, "bf16": torch.bfloat16, "fp32": torch.float32}[name]


def indexer_inputs(wl: Workload, layer: int = 0, device="cpu"):
    """(q [B,Lq,H,D], k [B,Lk,D], w [B,Lq,H]) for one layer of a workload."""
    dt = _torch_dtype(wl.idx_dtype)
    std = 1.0 / math.sqrt(wl.D) if wl.idx_dtype == "fp8" else 1.0
    q = normal((wl.B, wl.Lq, wl.H, wl.D), std, dt, device, mix(wl.seed, layer, T_Q_IDX))
    k = normal((wl.B, wl.Lk, wl.D), std, dt, device, mix(wl.seed, layer, T_K_IDX))
    if wl.w_dtype == "fp32":
        w = uniform((wl.B, wl.Lq, wl.H), torch.float32, device, mix(wl.seed, layer, T_W_IDX))
    else:
        w = normal((wl.B, wl.Lq, wl.H), 0.1, _torch_dtype(wl.w_dtype), device,
                   mix(wl.seed, layer, T_W_IDX))
    return q, k, w


def attention_inputs(wl: Workload, layer: int = 0, device="cpu"):
    """(q [B,Lq,Hq,Dqk], kv [B,Lk,Dqk]) in bf16 for one layer of a workload."""
    q = normal((wl.B, wl.Lq, wl.Hq, wl.Dqk), 1.0, torch.bfloat16, device,
               mix(wl.seed, layer, T_Q_ATT))
    kv = normal((wl.B, wl.Lk, wl.Dqk), 1.0, torch.bfloat16, device, mix(wl.seed, layer, T_KV_ATT))
    return q, kv


def ffn_weight(wl: Workload, layer: int, device="cpu") -> torch.Tensor:
    return normal((wl.Dm, wl.Dm), 1.0 / math.sqrt(wl.Dm), torch.bfloat16, device,
                  mix(wl.seed, layer, T_W_FFN))


def stack_x0(wl: Workload, device="cpu") -> torch.Tensor:
    return normal((wl.Lq, wl.Dm), 1.0, torch.bfloat16, device, mix(wl.seed, 0, T_X0))


def closed_form_indexer(B: int, L: int, H: int, D: int, dtype: str, kind: str, device="cpu"):
    """Indexer inputs whose scores have a closed form (exact in fp8, bf16 and fp32).

    Keys hold the base-8 digits of their index s in d = 0..5 (s < 2^18), head 0
    has q = (1, 8, 64, 0, 0, 0) and head 1 has q = (0, 0, 0, 1, 8, 64), every
    other head and dimension is zero.  Then q_0.k[s] = s mod 512 and
    q_1.k[s] = s div 512, so with w = (1, 512) the score is exactly s
    ("recency"), with w = (-1, -512) it is exactly -s ("reverse"), and with
    w = 0 or w = -0 every score is zero ("ties", "negzero_ties").
    """
    assert H >= 2 and D >= 6 and L <= (1 << 18)
    dt = _torch_dtype(dtype)
    s = torch.arange(L, dtype=torch.int64)
    kf = torch.zeros(B, L, D, dtype=torch.float32)
    for j in range(6):
        kf[:, :, j] = ((s >> (3 * j)) & 7).to(torch.float32)
    qf = torch.zeros(B, L, H, D, dtype=torch.float32)
    qf[:, :, 0, 0], qf[:, :, 0, 1], qf[:, :, 0, 2] = 1.0, 8.0, 64.0
    qf[:, :, 1, 3], qf[:, :, 1, 4], qf[:, :, 1, 5] = 1.0, 8.0, 64.0
    wf = torch.zeros(B, L, H, dtype=torch.float32)
    if kind == "recency":
        wf[:, :, 0], wf[:, :, 1] = 1.0, 512.0
    elif kind == "reverse":
        wf[:, :, 0], wf[:, :, 1] = -1.0, -512.0
    elif kind == "ties":
        pass
    elif kind == "negzero_ties":
        wf.fill_(-0.0)
    else:
        raise ValueError(kind)
    wdt = torch.float32 if dtype == "bf16" else torch.bfloat16
    return qf.to(dt).to(device), kf.to(dt).to(device), wf.to(wdt).to(device)
