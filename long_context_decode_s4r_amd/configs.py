"""The five workloads the path is built and measured on.

Shapes follow the low-rank compressed-KV (S4R) setting: per-layer bases of
rank r over D' = n_kv_heads * head_dim concatenated channels, s exact sink
tokens, a T'-row SVD sample, a W-step query-coefficient window, top-k
selection and an exact recent window.  Value distributions are described in
synth.py.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    n_layers: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    rank: int
    n_sink: int
    n_sample: int
    q_window: int
    top_k: int
    n_recent: int
    pool_kernel: int
    L: int
    storage: str            # "f32" or "bf16"
    decode_steps: int
    model: str              # "factor" (exact low rank + noise) or "power" (decaying spectrum)
    factor_rank: int = 0
    exponents: Tuple[float, ...] = (0.8,)   # power model: sigma_i = i^-e, one per layer
    noise: float = 0.01
    sink_scale: float = 1.0
    planted_frac: float = 0.0
    planted_scale: float = 1.0
    planted_run: int = 64
    seed: int = 0
    sample_recent_num: int = 7
    sample_recent_den: int = 10
    rank_v: int = 0            # value rank; 0 = the key rank
    local_window: int = 0      # 0: exact recent window, 1: rebuilt from coefficients
    eig_max_sweeps: int = 0    # 0: the library default

    @property
    def D(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def G(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_units(self) -> int:
        return self.n_layers * self.batch

    def exponent(self, layer: int) -> float:
        if len(self.exponents) == 1:
            return self.exponents[0]
        return self.exponents[layer]

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _qwen_exponents(n_layers: int = 28) -> Tuple[float, ...]:
    return tuple(0.5 + 0.7 * l / (n_layers - 1) for l in range(n_layers))


# single layer, single head, fp32; exact rank-16 states plus N(0, 0.01^2) noise,
# sink rows 10x; 64 decode steps; seed 0
TINY_F32 = Workload(
    name="tiny_f32_L1024", n_layers=1, batch=1, n_q_heads=1, n_kv_heads=1, head_dim=64,
    rank=16, n_sink=4, n_sample=128, q_window=8, top_k=32, n_recent=16, pool_kernel=7,
    L=1024, storage="f32", decode_steps=64, model="factor", factor_rank=16, noise=0.01,
    sink_scale=10.0, seed=0)

# one Llama-3-8B-shaped attention layer at 32K context, batch 16, bf16
LLAMA8B_32K = Workload(
    name="llama3_8b_layer_32k_b16", n_layers=1, batch=16, n_q_heads=32, n_kv_heads=8,
    head_dim=128, rank=256, n_sink=4, n_sample=2048, q_window=16, top_k=512, n_recent=64,
    pool_kernel=7, L=32768, storage="bf16", decode_steps=64, model="power",
    exponents=(0.8,), noise=0.01, seed=1)

# same layer at 128K, batch 4, r = 192, k = 1024, 2% planted rows with 4x norms
LLAMA8B_128K = LLAMA8B_32K.with_(
    name="llama3_8b_layer_128k_b4", batch=4, L=131072, rank=192, top_k=1024,
    planted_frac=0.02, planted_scale=4.0, seed=2)

# prefill only: bases and projection of one sequence at 64K
PREFILL_64K = LLAMA8B_32K.with_(
    name="prefill_d1024_64k", batch=1, L=65536, n_sample=4096, rank=256, decode_steps=0,
    seed=3)

# 28-layer Qwen-2.5-7B-shaped decode at 64K, batch 8, per-layer spectra
QWEN7B_64K = Workload(
    name="qwen2.5_7b_28l_64k_b8", n_layers=28, batch=8, n_q_heads=28, n_kv_heads=4,
    head_dim=128, rank=128, n_sink=4, n_sample=2048, q_window=16, top_k=512, n_recent=64,
    pool_kernel=7, L=65536, storage="bf16", decode_steps=64, model="power",
    exponents=_qwen_exponents(28), noise=0.01, seed=4)

ALL = (TINY_F32, LLAMA8B_32K, LLAMA8B_128K, PREFILL_64K, QWEN7B_64K)


def by_name(name: str) -> Optional[Workload]:
    for w in ALL:
        if w.name == name:
            return w
    return None
