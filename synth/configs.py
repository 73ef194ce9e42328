"""Workload shapes for the synthetic FFN layer stacks.

Five workloads, each a stack of FFN layers of one transformer shape with a
ReLU or ReGLU activation:

* ``tiny``     -- one ReLU layer, d=512, ffn=2048, fp32 weights, no predictor
                  (the mask is the true sign of the pre-activation); 16 tokens.
* ``opt6.7b``  -- 32 ReLU layers, d=4096, ffn=16384, fp16, rank-1024 predictor;
                  128 decode tokens at batch 1.
* ``falcon40b``-- 60 ReLU layers, d=8192, ffn=32768, fp16; per-layer mean active
                  fraction drawn from U[3%, 12%]; predictor rank 512 where that
                  mean is below 5%, else 1024; hot neurons permuted to the front.
* ``llama70b`` -- 80 ReGLU layers, d=8192, ffn=28672, fp16 gate/up/down, the
                  predictor and the mask on the gate; batch 64 and batch 1.
* ``opt175b``  -- 96 ReLU layers, d=12288, ffn=49152, Q4_0 weights, rank-1024
                  fp16 predictor; batch 1 and batch 8.

The activation-frequency profile is a power law over a seeded neuron order.
Where a workload is "tuned so the top X% of neurons carry 80% of activation
mass" (PowerInfer's profiling statistic for OPT-30B and Llama-2-70B, page
"PowerInfer: Fast Large Language Model Serving with a Consumer-grade GPU",
section «Метод»), the exponent ``alpha`` is the one that reaches that share; it
is solved in :mod:`synth.gen` and pinned by the generator tests.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

# Variance of the predictor's logit error (logit = pre-activation + noise).
NOISE_VAR = 0.3
# Clip range of the per-neuron activation probability.
P_MIN, P_MAX = 0.005, 0.95


@dataclass(frozen=True)
class StackConfig:
    name: str
    index: int                 # seed namespace of this workload
    layers: int
    d: int
    ffn: int
    wtype: str                 # "f32" | "f16" | "q4_0"
    act: str                   # "relu" | "reglu" | "sqrelu"
    rank: Optional[int]        # None: no predictor (true mask); -1: adaptive per layer
    mean_active: Tuple[float, float]   # (lo, hi); lo == hi for a fixed mean
    alpha: Optional[float]     # None: solve for the mass share below
    mass_share: Optional[Tuple[float, float]] = None  # (top fraction, share)
    tokens: int = 16
    batches: Tuple[int, ...] = (1,)
    hot_first: bool = False
    noise_var: float = NOISE_VAR
    notes: str = field(default="", compare=False)

    @property
    def has_predictor(self) -> bool:
        return self.rank is not None

    def layer_rank(self, mean: float) -> int:
        """Predictor rank of a layer: fixed, or 512 for sparse layers (<5% active) else 1024."""
        if self.rank is None:
            return 0
        if self.rank == -1:
            return 512 if mean < 0.05 else 1024
        return self.rank


CONFIGS = {
    "tiny": StackConfig("tiny", 0, 1, 512, 2048, "f32", "relu", None, (0.10, 0.10), 1.0,
                        tokens=16, batches=(1,)),
    "opt6.7b": StackConfig("opt6.7b", 1, 32, 4096, 16384, "f16", "relu", 1024, (0.10, 0.10), None,
                           mass_share=(0.26, 0.80), tokens=128, batches=(1,)),
    "falcon40b": StackConfig("falcon40b", 2, 60, 8192, 32768, "f16", "relu", -1, (0.03, 0.12), 1.0,
                             tokens=128, batches=(1,), hot_first=True),
    "llama70b": StackConfig("llama70b", 3, 80, 8192, 28672, "f16", "reglu", 1024, (0.10, 0.10), None,
                            mass_share=(0.43, 0.80), tokens=64, batches=(64, 1)),
    "opt175b": StackConfig("opt175b", 4, 96, 12288, 49152, "q4_0", "relu", 1024, (0.08, 0.08), 1.0,
                           tokens=64, batches=(1, 8)),
}
ORDER = ["tiny", "opt6.7b", "falcon40b", "llama70b", "opt175b"]


def scaled(cfg: StackConfig, *, layers=None, d=None, ffn=None, rank=None, tokens=None, name=None) -> StackConfig:
    """A copy of ``cfg`` with smaller sizes (for tests that must finish in seconds)."""
    from dataclasses import replace
    kw = {}
    if layers is not None:
        kw["layers"] = layers
    if d is not None:
        kw["d"] = d
    if ffn is not None:
        kw["ffn"] = ffn
    if rank is not None:
        kw["rank"] = rank
    if tokens is not None:
        kw["tokens"] = tokens
    if name is not None:
        kw["name"] = name
    return replace(cfg, **kw)
