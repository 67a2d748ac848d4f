"""Seeded synthetic inputs and the named workloads they are drawn for.

This module holds no arithmetic of the method (no padding, no offsets, no
reduce, no optimizer): only parameter shapes, random draws and seeds. Both
the HIP path and the CPU oracle consume the tensors it produces.

Workloads (the pages name no dataset; all inputs are synthetic):
  fp32_1000x1003_nd4      one fp32 1000x1003 weight, N_d = 4, 3 Adam steps
  llama7b_layer_nd8       one Llama-7B-shaped layer (d = 4096, FFN 11008),
                          bf16 parameters, N_d = 8
  llama7b_rank_local_nd64 one rank's shard of a 7B-shaped model (32 such
                          layers + 32000x4096 embedding and LM head), N_d = 64,
                          64 shard-layout gradient chunks
  small_tensors_10k_nd8   10,000 tensors, numel log-uniform in [64, 65536]
  mlp8192x28672_accum_nd16  8192x28672 (x2) and 28672x8192 bf16, N_d = 16,
                          8 micro-batches accumulated before Adam
"""
import hashlib
import math
from dataclasses import dataclass, field
from typing import List

import numpy as np
import torch


def derive_seed(*parts) -> int:
    """Stable 63-bit seed from any printable parts (workload, kind, rank, ...)."""
    h = hashlib.sha256("/".join(str(p) for p in parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(n: int, sigma: float, dtype: torch.dtype, seed: int, device="cpu",
           chunk: int = 1 << 27) -> torch.Tensor:
    """n draws of N(0, sigma^2) in `dtype` (drawn in fp32, then converted)."""
    out = torch.empty(n, dtype=dtype, device=device)
    g = generator(seed, device)
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        x = torch.randn(hi - lo, generator=g, device=device, dtype=torch.float32)
        x.mul_(sigma)
        out[lo:hi].copy_(x)
    return out


@dataclass
class Workload:
    name: str
    numel: List[int]
    n_d: int
    param_dtype: torch.dtype
    grad_dtype: torch.dtype
    param_sigma: float
    grad_sigma: float
    ones: List[int] = field(default_factory=list)  # tensors initialised to 1.0
    steps: int = 1
    micro_batches: int = 1
    rank_local: int = -1     # >= 0: only this rank's shard is resident
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    seed: int = 0


def _llama_layer(d=4096, f=11008):
    # Wq, Wk, Wv, Wo, W1, W3, W2, attention-norm, ffn-norm
    return [d * d] * 4 + [d * f] * 3 + [d] * 2


def llama_stack(n_layers=32, n_d=8) -> Workload:
    """n_layers Llama-7B decoder layers (the shapes of _llama_layer), bf16,
    every rank resident: the model a per-layer gather schedule walks."""
    layer = _llama_layer()
    return Workload(
        f"llama7b_{n_layers}layers_nd{n_d}", layer * n_layers, n_d, torch.bfloat16,
        torch.bfloat16, 0.02, 1e-3,
        ones=[9 * i + 7 for i in range(n_layers)] + [9 * i + 8 for i in range(n_layers)])


def small_tensor_sizes(count=10_000, lo=64, hi=65536, seed=0) -> List[int]:
    """numel = round(exp(U(ln lo, ln hi))) for `count` tensors, seeded."""
    rng = np.random.default_rng(derive_seed("small_tensor_sizes", seed))
    x = rng.uniform(math.log(lo), math.log(hi), size=count)
    return [int(round(math.exp(v))) for v in x]


def workloads():
    layer = _llama_layer()
    return {
        "fp32_1000x1003_nd4": Workload(
            "fp32_1000x1003_nd4", [1000 * 1003], 4, torch.float32, torch.float32,
            0.02, 1e-2, steps=3),
        "llama7b_layer_nd8": Workload(
            "llama7b_layer_nd8", layer, 8, torch.bfloat16, torch.bfloat16, 0.02, 1e-3,
            ones=[7, 8]),
        "llama7b_rank_local_nd64": Workload(
            "llama7b_rank_local_nd64", layer * 32 + [32000 * 4096] * 2, 64, torch.bfloat16,
            torch.bfloat16, 0.02, 1e-3,
            ones=[9 * i + 7 for i in range(32)] + [9 * i + 8 for i in range(32)],
            rank_local=0),
        "small_tensors_10k_nd8": Workload(
            "small_tensors_10k_nd8", small_tensor_sizes(), 8, torch.bfloat16, torch.bfloat16,
            0.02, 1e-2),
        "mlp8192x28672_accum_nd16": Workload(
            "mlp8192x28672_accum_nd16", [8192 * 28672, 8192 * 28672, 28672 * 8192], 16,
            torch.bfloat16, torch.bfloat16, 0.02, 1e-3, micro_batches=8),
    }


def flat_params(w: Workload, device="cpu", scale_numel=None) -> torch.Tensor:
    """All parameters of `w`, unpadded, back to back, in w.param_dtype.
    Parameters listed in w.ones (norm weights) are 1.0."""
    numel = scale_numel or w.numel
    total = int(sum(numel))
    x = normal(total, w.param_sigma, w.param_dtype, derive_seed(w.name, w.seed, "params"),
               device)
    if w.ones:
        off = np.concatenate([[0], np.cumsum(numel)])
        for t in w.ones:
            if t < len(numel):
                x[int(off[t]):int(off[t + 1])] = 1.0
    return x


def grad_buffer(w: Workload, n: int, rank: int, step: int = 1, micro_batch: int = 0,
                device="cpu") -> torch.Tensor:
    """Rank `rank`'s gradient buffer of n elements for a step / micro-batch."""
    return normal(n, w.grad_sigma, w.grad_dtype,
                  derive_seed(w.name, w.seed, "grad", rank, step, micro_batch), device)
