"""Seeded synthetic workloads for the fused LM-head linear + cross-entropy.

This module is shared by the CPU oracle and the GPU path.  It only draws random
numbers and shapes them into inputs; it contains none of the loss arithmetic.

Every workload is an LM head: hidden states X [N, H], the head weight W [V, H]
(row-major, the `lm_head.weight` orientation: the AI-infra knowledge-base page
M011, §01, writes the weight as W[V, D] with logits Z = H Wᵀ), and pre-shifted
next-token labels [N] int64 where `ignore_index` (-100) marks positions that
carry no target (Unsloth fused-CE chapter, §4 and §7; M011 §07).

Recipe (identical for every config, only the shapes and label law differ):
  * three CPU `torch.Generator` streams: X from `seed`, W from
    `seed + 1000000`, labels and ignored positions (in that order) from
    `seed + 2000000` (so no two configs share a stream);
  * X ~ N(0, 1) and W ~ N(0, 0.02²) sampled in fp32, then rounded to bf16 by
    round-to-nearest-even (`Tensor.to(torch.bfloat16)`);
  * labels: uniform over [0, V), or Zipf(s) over ranks 1..V — P(k) ∝ k^-s
    normalised over V, sampled by fp64 inverse CDF, token id = k - 1;
  * ignored positions: either floor(f·N) rows drawn without replacement, or
    every position i with i % period == period - 1 (the last token of each
    packed sequence, whose next token belongs to another sample).
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np
import torch

IGNORE_INDEX = -100
BASE_SEED = 20261202
W_STREAM = 1_000_000
LABEL_STREAM = 2_000_000


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    N: int                      # tokens (rows of X)
    H: int                      # hidden size
    V: int                      # vocabulary size
    labels: str = "uniform"     # "uniform" or "zipf"
    zipf_s: float = 1.1
    ignore_frac: float = 0.0    # fraction of rows set to IGNORE_INDEX
    ignore_period: int = 0      # >0: positions i % period == period-1 ignored
    softcap: float = 0.0        # logit tanh softcap; <= 0 means off
    seed: int = BASE_SEED
    x_std: float = 1.0
    w_std: float = 0.02

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def flops_fwd_bwd(self) -> int:
        """Dense multiply-add work of one forward + backward: four N·H·V
        contractions (forward logits, recomputed logits, dX, dW), 2 flops each."""
        return 8 * self.N * self.H * self.V


# The five workloads the measurements are quoted on (index = seed offset).
WORKLOADS = {
    "tiny": Workload("tiny", N=256, H=64, V=1000, labels="uniform",
                     ignore_frac=0.10, seed=BASE_SEED + 0),
    # Liger's chunking example shape (16384 tokens, H 4096, V 32000).
    "liger": Workload("liger", N=16384, H=4096, V=32000, labels="uniform",
                      ignore_frac=0.05, seed=BASE_SEED + 1),
    # Llama-3-8B head: batch 2 x seq 4096.
    "llama3_8b": Workload("llama3_8b", N=8192, H=4096, V=128256, labels="zipf",
                          ignore_frac=0.10, seed=BASE_SEED + 2),
    # Gemma-2 2B head with the tanh logit softcap of 30.
    "gemma2_2b": Workload("gemma2_2b", N=8192, H=2304, V=256128, labels="zipf",
                          ignore_frac=0.10, softcap=30.0, seed=BASE_SEED + 3),
    # Long-sequence Qwen2.5-style head: batch 4 x seq 8192, packed sequences of
    # 2048 tokens whose boundary positions carry no target.
    "qwen25_long": Workload("qwen25_long", N=32768, H=3584, V=152064,
                            labels="uniform", ignore_period=2048,
                            seed=BASE_SEED + 4),
}

WORKLOAD_ORDER = ["tiny", "liger", "llama3_8b", "gemma2_2b", "qwen25_long"]


def zipf_ranks_inverse_cdf(u: torch.Tensor, V: int, s: float) -> torch.Tensor:
    """Map uniforms u in [0,1) to ranks 1..V with P(k) ∝ k^-s (fp64 inverse CDF)."""
    k = np.arange(1, V + 1, dtype=np.float64)
    w = k ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    idx = np.searchsorted(cdf, u.numpy(), side="right")
    idx = np.minimum(idx, V - 1)
    return torch.from_numpy(idx.astype(np.int64) + 1)


def make_inputs(w: Workload, device: Optional[str] = None):
    """Return (X bf16 [N,H], W bf16 [V,H], labels int64 [N]) on `device`
    (CPU tensors when device is None).  Bitwise reproducible for a given w."""
    X = make_x(w)
    W = make_w(w)
    labels = make_labels(w)
    if device is not None:
        X, W, labels = X.to(device), W.to(device), labels.to(device)
    return X, W, labels


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def make_x(w: Workload) -> torch.Tensor:
    g = _gen(w.seed)
    return (torch.randn(w.N, w.H, generator=g, dtype=torch.float32) * w.x_std).to(torch.bfloat16)


def make_w(w: Workload) -> torch.Tensor:
    g = _gen(w.seed + W_STREAM)
    return (torch.randn(w.V, w.H, generator=g, dtype=torch.float32) * w.w_std).to(torch.bfloat16)


def make_labels(w: Workload) -> torch.Tensor:
    g = _gen(w.seed + LABEL_STREAM)
    if w.labels == "uniform":
        labels = torch.randint(0, w.V, (w.N,), generator=g, dtype=torch.int64)
    elif w.labels == "zipf":
        u = torch.rand(w.N, generator=g, dtype=torch.float64)
        labels = zipf_ranks_inverse_cdf(u, w.V, w.zipf_s) - 1
    else:
        raise ValueError(f"unknown label law {w.labels!r}")
    if w.ignore_frac > 0:
        n_ign = int(np.floor(w.ignore_frac * w.N))
        perm = torch.randperm(w.N, generator=g)
        labels[perm[:n_ign]] = IGNORE_INDEX
    if w.ignore_period > 0:
        pos = torch.arange(w.N)
        labels[(pos % w.ignore_period) == (w.ignore_period - 1)] = IGNORE_INDEX
    return labels


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a bf16/fp32 CPU tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def fingerprint(*tensors: torch.Tensor) -> str:
    """sha256 over the raw bytes of CPU tensors (bf16 viewed as int16)."""
    h = hashlib.sha256()
    for t in tensors:
        t = t.detach().to("cpu").contiguous()
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16)
        h.update(t.numpy().tobytes())
    return h.hexdigest()


def row_sample(N: int, count: int, seed: int) -> np.ndarray:
    """Seeded sorted sample of distinct row indices (always includes 0, N-1)."""
    rng = np.random.default_rng(seed)
    count = min(count, N)
    pick = set(rng.choice(N, size=max(0, count - 2), replace=False).tolist())
    pick.update({0, N - 1})
    return np.array(sorted(pick), dtype=np.int64)
