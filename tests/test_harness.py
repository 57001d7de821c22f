"""Host checks of the GPU parity harness itself (no GPU): the latent-score
bound the parity tests assert covers the arithmetic the kernels use (query
coefficients split into bf16 hi + lo parts, bf16 key coefficients, fp32
accumulation and fp32 softmax), emulated here with torch on the CPU."""
import math

import numpy as np
import pytest
import torch

from oracle import s4r

from gpu_helpers import score_bound


def emulated_scores(o: s4r.Cache, J):
    """Scores as the bf16 scorer forms them: base-2 logits from hi + lo bf16
    query parts times bf16 coefficients, accumulated in fp32, then an fp32
    softmax per row and an fp32 sum over rows."""
    rows = torch.from_numpy(o.window_rows()).float()
    ck = torch.from_numpy(o.CK[J]).float()          # bf16 values, exact in fp32
    qs = rows * (math.log2(math.e) / math.sqrt(o.rank))
    hi = qs.to(torch.bfloat16).float()
    lo = (qs - hi).to(torch.bfloat16).float()
    z = hi @ ck.T + lo @ ck.T                         # fp32 sums
    m = z.max(dim=1, keepdim=True).values
    p = torch.exp2(z - m)
    p = p / p.sum(dim=1, keepdim=True)
    return p.sum(dim=0).double().numpy()


@pytest.mark.parametrize("seed,r,planted", [(0, 64, False), (1, 128, True), (2, 256, False)])
def test_score_bound_covers_bf16_scorer(seed, r, planted):
    rng = np.random.default_rng(seed)
    H_q, H_kv, d, W = 8, 2, 128, 8
    D = H_kv * d
    L = 3000
    sig = np.arange(1, D + 1) ** -0.8
    sig *= math.sqrt(D / np.sum(sig ** 2))
    Q = np.linalg.qr(rng.standard_normal((D, D)))[0]
    K = (rng.standard_normal((L, D)) * sig) @ Q.T
    V = (rng.standard_normal((L, D)) * sig) @ Q.T
    if planted:
        K[1000:1060] *= 4.0
    K, V = s4r.rnd(K, "bf16"), s4r.rnd(V, "bf16")
    o, _ = s4r.prefill(K, V, n_q_heads=H_q, n_kv_heads=H_kv, head_dim=d, rank=r, n_sink=4,
                       n_sample=512, q_window=W, top_k=64, n_recent=16, pool_kernel=7,
                       storage="bf16", L_max=L + W + 2)
    for t in range(W + 1):
        q = s4r.rnd(rng.standard_normal((H_q, d)), "bf16")
        kv = s4r.rnd(rng.standard_normal((H_kv, d)), "bf16")
        s4r.decode_step(o, q, kv, kv)
    J = o.candidates()
    ref = o.last["score"]
    got = emulated_scores(o, J)
    bound = score_bound(o, J)
    assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) / bound))
    # the bound is not vacuous: it stays far below the scores that matter
    assert np.max(bound / ref) < 1e-3
