"""Pins of the float64 oracle against things other than itself.

Each test ties a step of the oracle to what the S4R review page or the
mathematics fixes: exact reconstruction of exactly-low-rank states,
equality with plain full-cache attention when r = D' and top-k covers every
candidate, the latent identity at r = D', library SVD, closed-form softmax
values, score invariants, pure-Python brute force on tiny inputs, sampling
counts, invariances and the closed-form memory ratio.  The last block plants
plausible mistakes in (a copy of) the oracle and checks that a pin fails.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import s4r

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------- #
# independent reference routines (plain loops / textbook definitions)
# --------------------------------------------------------------------------- #
def full_attention_plain(q, K_all, V_all, n_kv_heads):
    """Textbook multi-head attention with grouped KV heads, written with
    explicit loops: out_a = sum_j softmax_j(q_a . k_j,h / sqrt(d)) v_j,h."""
    H_q, d = q.shape
    G = H_q // n_kv_heads
    out = np.zeros((H_q, d))
    for a in range(H_q):
        h = a // G
        logits = []
        for j in range(K_all.shape[0]):
            kj = K_all[j, h * d:(h + 1) * d]
            logits.append(sum(float(q[a, i]) * float(kj[i]) for i in range(d)) / math.sqrt(d))
        m = max(logits)
        w = [math.exp(x - m) for x in logits]
        s = sum(w)
        for j in range(K_all.shape[0]):
            out[a] += (w[j] / s) * V_all[j, h * d:(h + 1) * d]
    return out


def latent_scores_plain(CK_J, rows, r):
    n = len(CK_J)
    score = [0.0] * n
    for row in rows:
        z = [sum(float(row[i]) * float(c[i]) for i in range(len(row))) / math.sqrt(r) for c in CK_J]
        m = max(z)
        e = [math.exp(x - m) for x in z]
        s = sum(e)
        for j in range(n):
            score[j] += e[j] / s
    return np.array(score)


def pool_plain(score, kappa):
    n = len(score)
    h = kappa // 2
    return np.array([max(score[max(0, j - h):min(n, j + h + 1)]) for j in range(n)])


def topk_plain(pooled, k):
    idx = list(range(len(pooled)))
    idx.sort(key=lambda j: (-pooled[j], j))
    return sorted(idx[:min(k, len(pooled))])


def small_cache(seed=0, *, H_q=4, H_kv=2, d=4, r=None, L=40, s=2, n_rec=4, W=3, k=6,
                kappa=3, T=16, storage="f64", L_max=None, lowrank=None, noise=0.0):
    rng = _rng(seed)
    D = H_kv * d
    r = D if r is None else r
    if lowrank:
        F = rng.standard_normal((lowrank, D))
        K = rng.standard_normal((L, lowrank)) @ F + noise * rng.standard_normal((L, D))
        F2 = rng.standard_normal((lowrank, D))
        V = rng.standard_normal((L, lowrank)) @ F2 + noise * rng.standard_normal((L, D))
    else:
        K = rng.standard_normal((L, D))
        V = rng.standard_normal((L, D))
    K = s4r.rnd(K, storage)
    V = s4r.rnd(V, storage)
    cache, info = s4r.prefill(K, V, n_q_heads=H_q, n_kv_heads=H_kv, head_dim=d, rank=r,
                              n_sink=s, n_sample=T, q_window=W, top_k=k, n_recent=n_rec,
                              pool_kernel=kappa, storage=storage,
                              L_max=L_max if L_max else L + 16)
    return cache, K, V, rng


# --------------------------------------------------------------------------- #
# P1: exact rank -> exact reconstruction
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_exact_rank_reconstruction(seed):
    rng = _rng(seed)
    L, D, r, s, T = 200, 32, 8, 4, 24
    X = rng.standard_normal((L, r)) @ rng.standard_normal((r, D))
    X[:s] *= 10.0
    B, lam, S, pos = s4r.build_basis(X, s, T, r, "f64")
    C = s4r.project(X[s:], B, "f64")
    rel = np.linalg.norm(C @ B.T - X[s:]) / np.linalg.norm(X[s:])
    assert rel < 1e-12
    # B is orthonormal and the (r+1)-th eigenvalue of the sample Gram vanishes
    assert np.allclose(B.T @ B, np.eye(r), atol=1e-12)
    assert lam[r] < 1e-10 * lam[0]


# --------------------------------------------------------------------------- #
# P2: r = D' and k >= |J| -> full-cache attention
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("seed,H_q,H_kv", [(0, 4, 2), (1, 2, 2), (2, 6, 2), (3, 3, 1)])
def test_full_rank_all_selected_equals_full_attention(seed, H_q, H_kv):
    d, L, s, n_rec = 4, 30, 2, 4
    cache, K, V, rng = small_cache(seed, H_q=H_q, H_kv=H_kv, d=d, L=L, s=s, n_rec=n_rec,
                                   k=10_000, T=16, W=3, kappa=3)
    K_all, V_all = K.copy(), V.copy()
    for step in range(5):
        q = rng.standard_normal((H_q, d))
        kn = rng.standard_normal((H_kv, d))
        vn = rng.standard_normal((H_kv, d))
        out = s4r.decode_step(cache, q, kn, vn)
        K_all = np.vstack([K_all, kn.reshape(1, -1)])
        V_all = np.vstack([V_all, vn.reshape(1, -1)])
        ref = full_attention_plain(q, K_all, V_all, H_kv)
        assert np.max(np.abs(out - ref)) < 1e-12 * max(1.0, np.max(np.abs(ref)))
        # every candidate selected, ascending
        J = cache.candidates()
        assert np.array_equal(cache.last["positions"], J)


# --------------------------------------------------------------------------- #
# P3: latent identity at r = D'
# --------------------------------------------------------------------------- #
def test_query_concat_layout():
    # H_q = 6, H_kv = 2 -> G = 3; vector g concatenates heads g and 3 + g
    q = np.arange(6 * 2, dtype=float).reshape(6, 2)
    qc = s4r.query_concat(q, 2)
    assert qc.shape == (3, 4)
    for g in range(3):
        assert np.array_equal(qc[g], np.concatenate([q[g], q[3 + g]]))


def test_latent_identity_full_rank():
    rng = _rng(5)
    H_q, H_kv, d = 6, 2, 4
    D = H_kv * d
    B, *_ = s4r.build_basis(rng.standard_normal((50, D)), 2, 20, D, "f64")
    q = rng.standard_normal((H_q, d))
    k = rng.standard_normal((H_kv, d))
    cq = s4r.query_concat(q, H_kv) @ B
    ck = k.reshape(-1) @ B
    G = H_q // H_kv
    for g in range(G):
        direct = sum(q[h * G + g] @ k[h] for h in range(H_kv))
        assert abs(cq[g] @ ck - direct) < 1e-12 * (1 + abs(direct))


# --------------------------------------------------------------------------- #
# P4: Gram eigendecomposition vs library SVD
# --------------------------------------------------------------------------- #
def test_gram_eigen_matches_svd():
    rng = _rng(7)
    X = rng.standard_normal((300, 24)) * (np.arange(1, 25) ** -0.8)
    B, lam, S, _ = s4r.build_basis(X, 4, 64, 6, "f64")
    sv = np.linalg.svd(S, compute_uv=False)
    assert np.allclose(lam, sv ** 2, rtol=0, atol=1e-10 * lam[0])
    _, _, Vt = np.linalg.svd(S)
    P_lib = Vt[:6].T @ Vt[:6]
    assert np.max(np.abs(B @ B.T - P_lib)) < 1e-9


# --------------------------------------------------------------------------- #
# closed-form latent softmax and selection cases
# --------------------------------------------------------------------------- #
def test_latent_scores_closed_form():
    # r = 4, one row c_q = (2,0,0,0); candidates (1,0,0,0), 0, (-1,0,0,0):
    # z = (2/2, 0, -2/2) = (1, 0, -1) -> softmax (e, 1, 1/e) / (e + 1 + 1/e)
    CK = np.array([[1.0, 0, 0, 0], [0, 0, 0, 0], [-1.0, 0, 0, 0]])
    row = np.array([[2.0, 0, 0, 0]])
    e = math.e
    want = np.array([e, 1.0, 1.0 / e]) / (e + 1.0 + 1.0 / e)
    assert np.allclose(s4r.latent_scores(CK, row, 4), want, atol=1e-15)
    # two rows sum: second row (0, 0, 0, 0) gives the uniform 1/3
    rows = np.array([[2.0, 0, 0, 0], [0, 0, 0, 0]])
    assert np.allclose(s4r.latent_scores(CK, rows, 4), want + 1.0 / 3.0, atol=1e-15)


def test_pool_and_topk_closed_form():
    score = np.array([0.1, 0.5, 0.2, 0.2, 0.0, 0.9, 0.3])
    assert np.array_equal(s4r.max_pool(score, 1), score)
    assert np.allclose(s4r.max_pool(score, 3), [0.5, 0.5, 0.5, 0.2, 0.9, 0.9, 0.9])
    assert np.allclose(s4r.max_pool(score, 5), [0.5, 0.5, 0.5, 0.9, 0.9, 0.9, 0.9])
    # ties -> lower index first; output ascending
    p = np.array([0.3, 0.7, 0.7, 0.1, 0.7, 0.3])
    assert list(s4r.select_topk(p, 2)) == [1, 2]
    assert list(s4r.select_topk(p, 4)) == [0, 1, 2, 4]
    assert list(s4r.select_topk(p, 100)) == [0, 1, 2, 3, 4, 5]
    assert list(s4r.select_topk(p, 0)) == []


# --------------------------------------------------------------------------- #
# P5: score invariants
# --------------------------------------------------------------------------- #
def test_score_invariants():
    cache, K, V, rng = small_cache(11, H_q=4, H_kv=2, d=4, r=5, L=60, k=8, W=3, kappa=5)
    for step in range(6):
        s4r.decode_step(cache, rng.standard_normal((4, 4)), rng.standard_normal((2, 4)),
                        rng.standard_normal((2, 4)))
        sc, po = cache.last["score"], cache.last["pooled"]
        w_eff = min(cache.steps, cache.q_window)
        assert abs(sc.sum() - w_eff * cache.G) < 1e-12
        assert np.all(sc >= 0) and np.all(po >= sc)
        assert len(cache.last["positions"]) == min(cache.top_k, len(cache.candidates()))


# --------------------------------------------------------------------------- #
# P6: pure-Python brute force on tiny inputs
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_bruteforce_tiny(seed):
    cache, K, V, rng = small_cache(seed, H_q=4, H_kv=2, d=3, r=4, L=48, s=3, n_rec=5,
                                   k=7, W=3, kappa=3, T=20, storage="f64")
    for step in range(5):
        q = rng.standard_normal((4, 3))
        kn = rng.standard_normal((2, 3))
        vn = rng.standard_normal((2, 3))
        out = s4r.decode_step(cache, q, kn, vn)
        J = cache.candidates()
        rows = cache.window_rows()
        sc = latent_scores_plain(cache.CK[J], rows, cache.rank)
        assert np.allclose(sc, cache.last["score"], atol=1e-12)
        po = pool_plain(list(sc), cache.pool_kernel)
        assert np.allclose(po, cache.last["pooled"], atol=1e-12)
        sel = topk_plain(list(cache.last["pooled"]), cache.top_k)
        assert list(J[sel]) == list(cache.last["positions"])
        # reconstruction + attention by loops
        pos = J[sel]
        K_hat = [[sum(cache.CK[p, i] * cache.BK[c, i] for i in range(cache.rank))
                  for c in range(6)] for p in pos]
        V_hat = [[sum(cache.CV[p, i] * cache.BV[c, i] for i in range(cache.rank))
                  for c in range(6)] for p in pos]
        K_all = np.vstack([cache.sink_k, cache.ring_k, np.array(K_hat)])
        V_all = np.vstack([cache.sink_v, cache.ring_v, np.array(V_hat)])
        ref = full_attention_plain(q, K_all, V_all, 2)
        assert np.max(np.abs(ref - out)) < 1e-12


# --------------------------------------------------------------------------- #
# P7: sampling counts
# --------------------------------------------------------------------------- #
def test_sample_positions_hand_case():
    # L = 20, s = 2, T' = 10 -> 7 recent (13..19), 3 uniform over [2, 13):
    # span 11 -> offsets 0, 3, 7 -> 2, 5, 9
    pos = s4r.sample_positions(20, 2, 10)
    assert list(pos) == [2, 5, 9, 13, 14, 15, 16, 17, 18, 19]


@pytest.mark.parametrize("L,s,T", [(1024, 4, 128), (32768, 4, 2048), (65536, 4, 4096),
                                   (100, 4, 96), (50, 0, 10), (17, 4, 3)])
def test_sample_positions_counts(L, s, T):
    pos = s4r.sample_positions(L, s, T)
    n_r = (7 * T) // 10
    assert len(pos) == T and len(set(pos.tolist())) == T
    assert pos.min() >= s and pos.max() < L
    assert np.array_equal(np.sort(pos)[-n_r:] if n_r else np.array([], int),
                          np.arange(L - n_r, L))


def test_sample_positions_rejects_oversized():
    with pytest.raises(ValueError):
        s4r.sample_positions(20, 4, 17)


# --------------------------------------------------------------------------- #
# P8: invariances of the basis construction
# --------------------------------------------------------------------------- #
def test_basis_invariances():
    rng = _rng(9)
    L, D, s, T, r = 120, 16, 4, 40, 5
    X = rng.standard_normal((L, D)) * (np.arange(1, D + 1) ** -1.0)
    B, lam, S, pos = s4r.build_basis(X, s, T, r, "f64")
    X2 = X.copy()
    X2[pos] *= rng.uniform(0.1, 10.0, size=(len(pos), 1))
    B2, lam2, S2, _ = s4r.build_basis(X2, s, T, r, "f64")
    assert np.max(np.abs(B @ B.T - B2 @ B2.T)) < 1e-10
    perm = rng.permutation(len(pos))
    assert np.allclose(s4r.gram(S[perm]), s4r.gram(S), atol=1e-13)


# --------------------------------------------------------------------------- #
# bf16 rounding vs the library conversion (round to nearest even)
# --------------------------------------------------------------------------- #
def test_bf16_rounding_matches_library():
    torch = pytest.importorskip("torch")
    rng = _rng(3)
    x32 = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -5 * (1 + 5 * 2 ** -9),
                     0.0, -0.0, 255.5, 1.0 - 2 ** -9], dtype=np.float32)
    x32 = np.concatenate([x32, ties])
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    got = s4r.rnd(x32.astype(np.float64), "bf16")
    assert np.array_equal(got, ref)
    assert s4r.rnd(np.array([1 + 2 ** -8]), "bf16")[0] == 1.0        # tie -> even
    assert s4r.rnd(np.array([1 + 3 * 2 ** -8]), "bf16")[0] == 1 + 2 ** -6


# --------------------------------------------------------------------------- #
# P10: closed-form memory ratio
# --------------------------------------------------------------------------- #
def test_memory_ratio():
    D, r, s, n_rec = 1024, 256, 4, 64
    ratios = [s4r.persistent_bytes(L, D, r, s, n_rec, 2) / s4r.full_cache_bytes(L, D, 2)
              for L in (1 << 12, 1 << 15, 1 << 20, 1 << 26)]
    assert all(a > b for a, b in zip(ratios, ratios[1:]))
    assert abs(ratios[-1] - r / D) < 1e-4
    # closed form at 32K: ((s + n_rec) D + (L - s) r + D r) / (L D)
    L = 32768
    want = ((s + n_rec) * D + (L - s) * r + D * r) / (L * D)
    assert abs(ratios[1] - want) < 1e-15


def test_defaults_match_pages():
    with open(os.path.join(GOLDEN, "s4r_defaults.json")) as f:
        d = json.load(f)
    # the 7:3 split in the sampler
    pos = s4r.sample_positions(1000, d["n_sink"]["value"], 100)
    recent = np.sum(pos >= 1000 - 70)
    num, den = d["sample_split_recent_to_uniform"]["value"]
    assert recent == 100 * num // (num + d["sample_split_recent_to_uniform"]["value"][1]) == 70
    # latent scale 1/sqrt(r): one candidate pair, one row
    CK = np.array([[1.0] + [0.0] * 15, [0.0] * 16])
    row = np.array([[4.0] + [0.0] * 15])
    sc = s4r.latent_scores(CK, row, 16)
    z = 4.0 / math.sqrt(16)
    assert abs(sc[0] - math.exp(z) / (math.exp(z) + 1)) < 1e-15


# --------------------------------------------------------------------------- #
# planted mistakes: each must make a pin fail
# --------------------------------------------------------------------------- #
def _mutant_no_scale(CK_J, rows, rank):
    Z = np.asarray(rows) @ np.asarray(CK_J).T
    Z = Z - Z.max(axis=1, keepdims=True)
    P = np.exp(Z)
    P /= P.sum(axis=1, keepdims=True)
    return P.sum(axis=0)


def _mutant_concat(q, n_kv_heads):
    q = np.asarray(q, np.float64)
    H_q, d = q.shape
    G = H_q // n_kv_heads
    return q.reshape(G, n_kv_heads, d).reshape(G, n_kv_heads * d)


def _mutant_topk_high_index(pooled, k):
    n = len(pooled)
    order = np.lexsort((-np.arange(n), -np.asarray(pooled)))
    return np.sort(order[:min(k, n)])


def _mutant_gqa(q, keys_exact, values_exact, CK_sel, CV_sel, BK, BV, n_kv_heads):
    q = np.asarray(q)
    H_q, d = q.shape
    K_hat = CK_sel @ BK.T
    V_hat = CV_sel @ BV.T
    keys = np.concatenate([keys_exact, K_hat])
    vals = np.concatenate([values_exact, V_hat])
    out = np.zeros((H_q, d))
    for a in range(H_q):
        h = a % n_kv_heads  # interleaved instead of contiguous groups
        sl = slice(h * d, (h + 1) * d)
        out[a] = s4r.softmax_attention(q[a], keys[:, sl], vals[:, sl])
    return out


def _mutant_no_normalize(Y):
    return np.asarray(Y, np.float64)


@pytest.mark.parametrize("target,mutant,pins", [
    ("latent_scores", _mutant_no_scale, [test_latent_scores_closed_form]),
    ("query_concat", _mutant_concat, [test_query_concat_layout]),
    ("select_topk", _mutant_topk_high_index, [test_pool_and_topk_closed_form]),
    ("sparse_attention", _mutant_gqa,
     [lambda: test_full_rank_all_selected_equals_full_attention(0, 4, 2)]),
    ("normalize_rows", _mutant_no_normalize, [test_basis_invariances]),
])
def test_planted_mistake_is_caught(monkeypatch, target, mutant, pins):
    monkeypatch.setattr(s4r, target, mutant)
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()
