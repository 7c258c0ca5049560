"""Named synthetic workloads (shapes, dtypes, length mixes, threshold).

Each workload is an attention+MLP denoiser tower standing in for the pages' hybrid
tower: RMSNorm, one joint softmax over the prefix K/V plus the in-block keys, a GELU
MLP of width 4*d, an untied LM head, and the block/threshold operating point
(block 16, gamma 0.8) of dzen.guru "NVIDIA Nemotron 70B генерирует текст…",
section "Как попробовать?".

Towers are keyed by name, so workloads that share a tower (the three d=2048
workloads) also share its weights bit for bit.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    tower: str            # key of the weight streams
    n: int                # sequences in the batch
    plen: Tuple           # ("fixed", P) or ("uniform", lo, hi), both bounds inclusive
    B: int                # block size
    d: int                # d_model
    H: int                # query heads
    Hkv: int              # key/value heads
    hd: int               # head dim
    L: int                # denoiser layers
    F: int                # MLP width
    V: int                # vocabulary (the [MASK] id is V)
    dtype: str            # "f32" or "bf16": storage type of weights and prefix K/V
    gamma: float = 0.8
    tau_range: Tuple[float, float] = (1.0, 64.0)   # per-position logit inverse temperature
    weight_std: float = 0.02
    kv_std: float = 1.0
    seed: int = 0
    rms_eps: float = 1e-6
    batch_key: str = ""   # key of the prefix-length / prefix-K/V streams ("" = the workload name)
    # Mixture-of-experts MLP in every denoiser layer: (experts, top_k, shared experts,
    # expert width); () = the dense MLP of width F.
    moe: Tuple = ()

    @property
    def batch(self) -> str:
        return self.batch_key or self.name

    @property
    def G(self) -> int:
        return self.H // self.Hkv

    @property
    def qkv_dim(self) -> int:
        return (self.H + 2 * self.Hkv) * self.hd

    @property
    def M(self) -> int:
        return self.n * self.B

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def weight_params(self, active_experts: float = 0.0) -> int:
        """Parameters streamed once per step (layer GEMMs + LM head; the embedding is a gather).

        With a mixture of experts: the router plus `active_experts` experts (routed and
        shared) per layer, the experts that hold at least one row."""
        mlp = 2 * self.F * self.d
        if self.moe:
            E, _, _, de = self.moe
            mlp = E * self.d + int(round(active_experts * 2 * de * self.d))
        per_layer = self.qkv_dim * self.d + self.d * self.H * self.hd + mlp
        return self.L * per_layer + self.V * self.d


_D2048 = dict(tower="d2048", d=2048, H=16, Hkv=16, hd=128, L=8, F=8192, V=131072, dtype="bf16")

WORKLOADS = {
    # Tiny fp32 tower: parity at 1e-4; everything fits in cache.
    "tiny_fp32": Workload(name="tiny_fp32", tower="tiny", n=1, plen=("fixed", 128), B=16, d=256, H=4,
                          Hkv=4, hd=64, L=2, F=1024, V=4096, dtype="f32"),
    # bf16 tower at batch 1, prefix 4096: batch-1 weight streaming.
    "b1_p4096": Workload(name="b1_p4096", n=1, plen=("fixed", 4096), B=16, **_D2048),
    # Ragged batch of 32 prefixes in [512, 8192], per-sequence commit loops.
    "ragged32": Workload(name="ragged32", n=32, plen=("uniform", 512, 8192), B=16, **_D2048),
    # Long-context grouped-query attention: 32 query heads over 2 K/V heads, prefix 65536.
    "gqa_long": Workload(name="gqa_long", tower="d4096", n=4, plen=("fixed", 65536), B=16, d=4096, H=32,
                         Hkv=2, hd=128, L=4, F=16384, V=131072, dtype="bf16"),
    # Throughput sweep: batch 64, prefixes in [1024, 4096]; B and gamma vary per run.
    "sweep64_b8": Workload(name="sweep64_b8", batch_key="sweep64", n=64, plen=("uniform", 1024, 4096), B=8,
                           **_D2048),
    "sweep64_b16": Workload(name="sweep64_b16", batch_key="sweep64", n=64, plen=("uniform", 1024, 4096), B=16,
                            **_D2048),
    "sweep64_b32": Workload(name="sweep64_b32", batch_key="sweep64", n=64, plen=("uniform", 1024, 4096), B=32,
                            **_D2048),
    # The batch-1 tower with each MLP a mixture of 128 experts, 6 routed + 2 shared per token
    # (the counts of the pages' MoE layers), expert width 1024: the eight active experts
    # together are as wide as the dense MLP (F = 8192).
    "moe_b1_p4096": Workload(name="moe_b1_p4096", batch_key="b1_p4096", n=1, plen=("fixed", 4096), B=16,
                             moe=(128, 6, 2, 1024), **_D2048),
}

SWEEP_GAMMAS = (0.5, 0.8, 0.95)


def get_workload(name: str, *, gamma: Optional[float] = None, **overrides) -> Workload:
    w = WORKLOADS[name]
    if gamma is not None:
        overrides["gamma"] = gamma
    return w.with_(**overrides) if overrides else w
