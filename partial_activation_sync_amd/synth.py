"""Seeded synthetic inputs, shared by the tests, the benchmark and the oracle's callers.

This module holds none of the sublayer's arithmetic: it only draws seeded normal
tensors on the CPU and rounds them (round-to-nearest-even) to the storage dtype.
The oracle never imports it; callers pass its tensors to both sides.

Each tensor comes from its own ``torch.Generator`` seeded by (base seed, tensor id),
so a tensor's values do not depend on which other tensors were drawn, or in which
order.  Values: N(mean, std^2) in float32, then cast to the dtype.
"""
import torch

BASE_SEED = 20250624

# Tensor ids: one stream per named input.
X, W1, W2, CTX, WO, X0, GAMMA, BETA, PARTIALS, RESID = 1, 2, 3, 4, 5, 6, 7, 8, 9, 10
# Upstream gradients for the backward: dL/d out and dL/d out_resid.
DOUT, DRES = 11, 12
# The full block: QKV projection weights, and QKV activations for the attention core alone.
WQKV, QKV = 13, 14


def _generator(seed: int, tensor_id: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed((int(seed) * 1_000_003 + int(tensor_id) * 7919) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def normal(shape, tensor_id: int, *, std: float = 1.0, mean: float = 0.0,
           dtype=torch.bfloat16, seed: int = BASE_SEED) -> torch.Tensor:
    """A CPU tensor of the given shape with N(mean, std^2) entries, rounded to dtype."""
    t = torch.randn(tuple(shape), generator=_generator(seed, tensor_id), dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(dtype)


def replicated(shape_one_rank, P: int, tensor_id: int, **kw) -> torch.Tensor:
    """One [T, h] draw copied to every rank: [P, T, h] (an input replicated per rank)."""
    one = normal(shape_one_rank, tensor_id, **kw)
    return one.unsqueeze(0).expand(P, *one.shape).contiguous()


def sample_rows(T: int, n: int, seed: int = BASE_SEED) -> torch.Tensor:
    """Sorted distinct token indices: 0, T-1 and n-2 seeded others (all of them if T <= n)."""
    if T <= n:
        return torch.arange(T)
    g = _generator(seed, 1000 + T)
    inner = torch.randperm(T - 2, generator=g)[: n - 2] + 1
    rows = torch.cat([torch.tensor([0, T - 1]), inner])
    return torch.sort(rows).values
