"""Seeded synthetic inputs for the compressed-KV path.

This module only draws numbers: it holds none of the method's arithmetic and
is shared by the tests, the bench and the smoke check, on both sides of every
parity comparison.  All draws come from torch generators seeded from
(workload seed, layer, sequence, stream), so a case can be regenerated on the
CPU or on a GPU (values differ between the two devices; each comparison uses
one device's draws, copied where both sides need them).

State models (one per layer and per K|V):
  * "factor": X = A F + noise, A [L x q], F [q x D'] ~ N(0, 1), noise std
    ``noise`` (exactly rank q without noise);
  * "power":  X = Z diag(sigma) Q^T + noise with sigma_i = i^-e scaled so
    sum sigma_i^2 = D' (per-element RMS about 1), Q a random orthogonal
    matrix, Z ~ N(0, 1); noise std ``noise`` (1% of the RMS).
Sink rows are multiplied by ``sink_scale``.  Planted rows (128K workload):
floor(frac * L) positions in runs of ``planted_run`` tokens placed at seeded,
non-overlapping run-aligned offsets inside [L/4, 3L/4), K and V rows scaled.
Decode queries are N(0, 1); decode keys/values come from the same state
model as the prompt.  Everything is rounded to the storage type at the end.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional

import torch

from .configs import Workload

_STREAM_K, _STREAM_V, _STREAM_Q, _STREAM_MODEL, _STREAM_PLANT = 1, 2, 3, 4, 5


def storage_dtype(storage: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[storage]


def _gen(device, *key: int) -> torch.Generator:
    """Generator seeded from a tuple of small integers (a fixed mixing of the
    key; the exact constant only has to be stable)."""
    h = 0x9E3779B97F4A7C15
    for k in key:
        h = (h ^ (int(k) + 0x632BE59BD9B4E019 + ((h << 6) & (2**64 - 1)) + (h >> 2))) & (2**64 - 1)
    g = torch.Generator(device=device)
    g.manual_seed(h & (2**63 - 1))
    return g


def power_spectrum(D: int, exponent: float, device="cpu") -> torch.Tensor:
    i = torch.arange(1, D + 1, dtype=torch.float64, device=device)
    s = i.pow(-exponent)
    s = s * math.sqrt(D / float((s * s).sum()))
    return s.to(torch.float32)


def random_orthogonal(D: int, gen: torch.Generator, device) -> torch.Tensor:
    A = torch.randn(D, D, generator=gen, device=device, dtype=torch.float32)
    if device != "cpu" and torch.device(device).type != "cpu":
        Q, R = torch.linalg.qr(A.cpu().double())
        Q = Q * torch.sign(torch.diagonal(R)).unsqueeze(0)
        return Q.to(device=device, dtype=torch.float32)
    Q, R = torch.linalg.qr(A.double())
    Q = Q * torch.sign(torch.diagonal(R)).unsqueeze(0)
    return Q.to(torch.float32)


@dataclass
class StateModel:
    """Draws rows of one layer's K or V states."""
    kind: str
    D: int
    noise: float
    sigma: Optional[torch.Tensor] = None   # power
    Q: Optional[torch.Tensor] = None       # power
    F: Optional[torch.Tensor] = None       # factor

    def rows(self, n: int, gen: torch.Generator, device) -> torch.Tensor:
        if self.kind == "factor":
            A = torch.randn(n, self.F.shape[0], generator=gen, device=device)
            X = A @ self.F
        else:
            Z = torch.randn(n, self.D, generator=gen, device=device) * self.sigma
            X = Z @ self.Q.T
        if self.noise > 0:
            X = X + self.noise * torch.randn(n, self.D, generator=gen, device=device)
        return X


def state_model(w: Workload, layer: int, kind: int, device) -> StateModel:
    g = _gen(device, w.seed, _STREAM_MODEL, layer, kind)
    if w.model == "factor":
        F = torch.randn(w.factor_rank, w.D, generator=g, device=device)
        return StateModel("factor", w.D, w.noise, F=F)
    sigma = power_spectrum(w.D, w.exponent(layer), device)
    Q = random_orthogonal(w.D, g, device)
    return StateModel("power", w.D, w.noise, sigma=sigma, Q=Q)


def planted_positions(w: Workload, seq: int, L: int) -> torch.Tensor:
    n = int(math.floor(w.planted_frac * L))
    if n == 0:
        return torch.zeros(0, dtype=torch.int64)
    run = w.planted_run
    lo, hi = L // 4, (3 * L) // 4
    n_slots = (hi - lo) // run
    n_runs = -(-n // run)
    g = _gen("cpu", w.seed, _STREAM_PLANT, seq)
    slots = torch.randperm(n_slots, generator=g)[:n_runs].sort().values
    pos = (lo + slots.unsqueeze(1) * run + torch.arange(run).unsqueeze(0)).reshape(-1)
    return pos[:n]


@dataclass
class Prompt:
    K: torch.Tensor          # [U][L][D'] storage dtype
    V: torch.Tensor
    models: List[StateModel]  # per (layer, kind): index 2*layer + {0: K, 1: V}


def make_prompt(w: Workload, device="cpu", L: Optional[int] = None,
                batch: Optional[int] = None, n_layers: Optional[int] = None,
                first_layer: int = 0) -> Prompt:
    """Prompt K, V for every (layer, sequence) unit, unit = layer*batch + seq,
    for layers [first_layer, first_layer + n_layers) (unit numbering starts
    at the first of them; a layer's draws do not depend on which others are
    generated with it)."""
    L = w.L if L is None else L
    batch = w.batch if batch is None else batch
    n_layers = w.n_layers - first_layer if n_layers is None else n_layers
    dt = storage_dtype(w.storage)
    U = n_layers * batch
    K = torch.empty(U, L, w.D, dtype=dt, device=device)
    V = torch.empty(U, L, w.D, dtype=dt, device=device)
    models = []
    for li in range(n_layers):
        layer = first_layer + li
        mk = state_model(w, layer, _STREAM_K, device)
        mv = state_model(w, layer, _STREAM_V, device)
        models += [mk, mv]
        for b in range(batch):
            u = li * batch + b
            plant = planted_positions(w, b, L).to(device)
            for kind, m, out in ((_STREAM_K, mk, K), (_STREAM_V, mv, V)):
                g = _gen(device, w.seed, kind, layer, b)
                X = m.rows(L, g, device)
                if w.sink_scale != 1.0:
                    X[: w.n_sink] *= w.sink_scale
                if plant.numel():
                    X[plant] *= w.planted_scale
                out[u] = X.to(dt)
    return Prompt(K, V, models)


@dataclass
class DecodeInputs:
    q: torch.Tensor      # [steps][U][H_q][d_h]
    k: torch.Tensor      # [steps][U][H_kv][d_h]
    v: torch.Tensor


def make_decode_inputs(w: Workload, prompt: Prompt, steps: int, device="cpu",
                       batch: Optional[int] = None, n_layers: Optional[int] = None,
                       first_layer: int = 0) -> DecodeInputs:
    """Decode-step queries, keys and values for the layers of `prompt`
    (generated with the same first_layer and n_layers)."""
    batch = w.batch if batch is None else batch
    n_layers = len(prompt.models) // 2 if n_layers is None else n_layers
    dt = storage_dtype(w.storage)
    U = n_layers * batch
    q = torch.empty(steps, U, w.n_q_heads, w.head_dim, dtype=dt, device=device)
    k = torch.empty(steps, U, w.n_kv_heads, w.head_dim, dtype=dt, device=device)
    v = torch.empty(steps, U, w.n_kv_heads, w.head_dim, dtype=dt, device=device)
    for li in range(n_layers):
        layer = first_layer + li
        mk, mv = prompt.models[2 * li], prompt.models[2 * li + 1]
        for b in range(batch):
            u = li * batch + b
            gq = _gen(device, w.seed, _STREAM_Q, layer, b)
            q[:, u] = torch.randn(steps, w.n_q_heads, w.head_dim, generator=gq,
                                  device=device).to(dt)
            gk = _gen(device, w.seed, _STREAM_K + 16, layer, b)
            gv = _gen(device, w.seed, _STREAM_V + 16, layer, b)
            k[:, u] = mk.rows(steps, gk, device).reshape(steps, w.n_kv_heads, w.head_dim).to(dt)
            v[:, u] = mv.rows(steps, gv, device).reshape(steps, w.n_kv_heads, w.head_dim).to(dt)
    return DecodeInputs(q, k, v)
