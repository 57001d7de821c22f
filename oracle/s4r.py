"""Float64 CPU oracle for S4R-style low-rank compressed-KV attention.

TEST INFRASTRUCTURE ONLY.  This module is the checker, not the product: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP path and imports
nothing from it.

Source of the method: the machine review of "S^4R: Selective Sampling,
Subspaces, and Sparse Reconstruction for Compressed Long-Context KV Caching"
(pith.science/paper/2608.00528, arXiv 2608.00528).  The review prints one
formula (the latent score Z = C_Q C_K^T / sqrt(r), 'Referee Report', major
comment 2, and 'Assumptions & free parameters') and describes the other steps
in prose ('What carries the argument', 'Core claim', 'Referee Report' summary,
'Assumptions & free parameters').  Each function below names the passage it
follows.  Where the review is silent the plainest reading is taken and named
in the docstring (readings R1..R14 are listed in the design notes).

Everything is float64.  Inputs are read as stored (fp32 or bf16 values,
widened).  ``rnd(x, storage)`` rounds to the storage type (round to nearest,
ties to even) and is applied only where the method *stores* a tensor: the
normalised SVD sample, the bases, the coefficient caches and the fp32 query
window.  ``storage == "f64"`` disables rounding (used by the exactness pins).

Parity pins (tests/test_oracle_pins.py) tie every function here to something
other than itself: exact-rank reconstruction (also with separate key and
value ranks, and for a basis shared by several layers), equality with full
attention at r = D' and k >= |J| (also with the recent window rebuilt from
coefficients), the latent identity at r = D', library SVD (also of the
stacked samples of a layer window), closed-form softmax cases, a hand-built
window ring (with and without prompt-tail queries), score invariants,
pure-Python brute force on tiny inputs with the test's own query window,
sampling counts (7:3, 10:0 and the full prompt), the closed-form memory
ratio and the rank it gives for a retention target.  A table of planted
mistakes checks that each pin catches the error it is meant to catch.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

STORAGES = ("f64", "f32", "bf16")


# --------------------------------------------------------------------------- #
# rounding to the storage type
# --------------------------------------------------------------------------- #
def rnd(x, storage: str) -> np.ndarray:
    """Round float64 values to the storage type and widen back to float64.

    bf16 keeps 8 significant bits (1 implicit + 7 stored); the rounding is to
    nearest with ties to even, done on the float64 value directly so there is
    no double rounding through fp32.  Values outside the normal bf16 range are
    not produced by the workloads and are not treated specially.
    """
    x = np.asarray(x, dtype=np.float64)
    if storage == "f64":
        return x.copy()
    if storage == "f32":
        return x.astype(np.float32).astype(np.float64)
    if storage == "bf16":
        m, e = np.frexp(x)  # x = m * 2**e, 0.5 <= |m| < 1
        q = np.rint(m * 256.0)  # 8 significant bits, ties to even
        return np.ldexp(q / 256.0, e)
    raise ValueError(f"unknown storage {storage!r}")


# --------------------------------------------------------------------------- #
# prefill: sinks, sampling, normalisation, bases, projection
# --------------------------------------------------------------------------- #
def sample_positions(L: int, n_sink: int, n_sample: int,
                     recent_num: int = 7, recent_den: int = 10) -> np.ndarray:
    """Positions of the SVD sample ('Core claim' and 'Load-bearing premise':
    T' non-sink prompt tokens, seven tenths of them taken from the end of the
    prompt and the remainder spread over the rest; the ratio is a free
    parameter in 'Assumptions & free parameters', and 'If this is right'
    compares it with an all-recent 10:0 sample).

    Reading R2: n_r = floor(num T' / den) positions ending at the last prompt
    token; the other n_u = T' - n_r are evenly spaced (no RNG) over the
    non-sink positions before them, [s, L - n_r).  num = den gives the
    all-recent sample (n_u = 0).  Returned uniform part first, then the
    recent run; all distinct.
    """
    n_r = (recent_num * n_sample) // recent_den
    n_u = n_sample - n_r
    span = L - n_r - n_sink
    if n_sample < 0 or n_r > L - n_sink or span < n_u:
        raise ValueError("sample does not fit in the non-sink prompt")
    uniform = n_sink + (np.arange(n_u, dtype=np.int64) * span) // max(n_u, 1)
    recent = np.arange(L - n_r, L, dtype=np.int64)
    return np.concatenate([uniform[:n_u], recent])


def normalize_rows(Y: np.ndarray) -> np.ndarray:
    """Per-token normalisation of the sampled states before the SVD ('What
    carries the argument', Eqs. 1-2; 'Core claim').  Each row is divided by
    its Euclidean norm; an all-zero row stays zero."""
    Y = np.asarray(Y, dtype=np.float64)
    n = np.sqrt(np.sum(Y * Y, axis=1, keepdims=True))
    out = np.zeros_like(Y)
    nz = n[:, 0] > 0
    out[nz] = Y[nz] / n[nz]
    return out


def gram(S: np.ndarray) -> np.ndarray:
    """A = S^T S; its eigenvectors are the right singular vectors of S
    (Eqs. 1-2 as summarised in 'What carries the argument')."""
    S = np.asarray(S, dtype=np.float64)
    return S.T @ S


def eig_desc(A: np.ndarray):
    """Eigenpairs of the symmetric matrix A, eigenvalues descending."""
    lam, U = np.linalg.eigh(np.asarray(A, dtype=np.float64))
    order = np.argsort(-lam, kind="stable")
    return lam[order], U[:, order]


def build_basis(X: np.ndarray, n_sink: int, n_sample: int, rank: int,
                storage: str, recent_num: int = 7, recent_den: int = 10):
    """Basis B (D' x r) of one state matrix X (L x D') of one layer and one
    sequence ('What carries the argument', Eqs. 1-2: B holds the r leading
    right singular vectors of the normalised sample, i.e. the r leading
    eigenvectors of its Gram matrix).

    Returns (B, eigenvalues descending, S, positions).  S is the stored
    (rounded) normalised sample; B is rounded to the storage type.
    """
    X = np.asarray(X, dtype=np.float64)
    L = X.shape[0]
    pos = sample_positions(L, n_sink, n_sample, recent_num, recent_den)
    S = rnd(normalize_rows(X[pos]), storage)
    lam, U = eig_desc(gram(S))
    B = rnd(U[:, :rank], storage)
    return B, lam, S, pos


def build_basis_shared(Xs, n_sink: int, n_sample: int, rank: int, storage: str,
                       recent_num: int = 7, recent_den: int = 10):
    """One basis for a window of neighbouring layers (DepthWeave-KV page,
    'Core claim' and Eq. 1: low-rank channel bases shared across a window of
    adjacent layers, each layer keeping its own coefficients on the shared
    basis; the learned router and residuals are not part of this).

    Reading: the shared basis is the rank-r truncated SVD of the layers'
    normalised samples stacked row-wise, i.e. the r leading eigenvectors of
    the sum of the per-layer Gram matrices.  Xs: the window's state matrices
    (each L x D', same sequence).  Returns (B, eigenvalues, [S per layer])."""
    Ss = []
    for X in Xs:
        X = np.asarray(X, dtype=np.float64)
        pos = sample_positions(X.shape[0], n_sink, n_sample, recent_num, recent_den)
        Ss.append(rnd(normalize_rows(X[pos]), storage))
    A = sum(gram(S) for S in Ss)
    lam, U = eig_desc(A)
    return rnd(U[:, :rank], storage), lam, Ss


def project(X: np.ndarray, B: np.ndarray, storage: str) -> np.ndarray:
    """Coefficients c = x . B of every row of X (Eq. 3 as summarised in 'What
    carries the argument': every non-sink token is stored as c = s.B).
    Reading R1: the stored rows are projected raw (no normalisation)."""
    return rnd(np.asarray(X, np.float64) @ np.asarray(B, np.float64), storage)


# --------------------------------------------------------------------------- #
# decode
# --------------------------------------------------------------------------- #
def query_concat(q: np.ndarray, n_kv_heads: int) -> np.ndarray:
    """Latent-query inputs (reading R5): with G = H_q / H_kv, vector g is the
    concatenation over KV heads h of query head h*G + g, so that its dot
    product with a concatenated key sums the G-th member's per-head logits.
    q: [H_q][d_h] -> [G][D']."""
    q = np.asarray(q, np.float64)
    H_q, d_h = q.shape
    G = H_q // n_kv_heads
    return q.reshape(n_kv_heads, G, d_h).transpose(1, 0, 2).reshape(G, n_kv_heads * d_h)


def latent_scores(CK_J: np.ndarray, rows: np.ndarray, rank: int) -> np.ndarray:
    """Latent relevance score of every candidate ('Referee Report' major
    comment 2: Z = C_Q C_K^T / sqrt(r); 'What carries the argument': softmax
    attention between the window of query coefficients and the cached key
    coefficients, Eqs. 8-10).

    rows: the W_eff*G query-coefficient rows; CK_J: the candidates' key
    coefficients.  Each row's softmax runs over the candidates (reading R4),
    and the per-candidate score is the sum of the rows' probabilities
    (reading R6).  Returns score[|J|]."""
    CK_J = np.asarray(CK_J, np.float64)
    rows = np.asarray(rows, np.float64)
    if CK_J.shape[0] == 0 or rows.shape[0] == 0:
        return np.zeros(CK_J.shape[0])
    Z = rows @ CK_J.T / math.sqrt(rank)
    Z = Z - Z.max(axis=1, keepdims=True)
    P = np.exp(Z)
    P /= P.sum(axis=1, keepdims=True)
    return P.sum(axis=0)


def max_pool(score: np.ndarray, kappa: int) -> np.ndarray:
    """Pooling of the scores before selection ('Assumptions & free
    parameters': pooling kernel 7, taken from SnapKV).  Reading R7: max
    pooling, stride 1, window clipped at the candidate edges; kappa = 1 is
    the identity."""
    score = np.asarray(score, np.float64)
    if kappa % 2 != 1:
        raise ValueError("pool width must be odd")
    h = kappa // 2
    n = score.shape[0]
    out = score.copy()
    for d in range(1, h + 1):
        if d >= n:
            break
        out[:-d] = np.maximum(out[:-d], score[d:])
        out[d:] = np.maximum(out[d:], score[:-d])
    return out


def select_topk(pooled: np.ndarray, k: int) -> np.ndarray:
    """Top-k candidate selection ('Core claim': only the local window plus
    the top-k global positions are reconstructed; Eqs. 13-15).  Reading R8:
    larger score first, equal scores -> lower index first; the first
    min(k, n) are returned in ascending index order."""
    pooled = np.asarray(pooled, np.float64)
    n = pooled.shape[0]
    kk = min(max(k, 0), n)
    order = np.lexsort((np.arange(n), -pooled))  # primary -pooled, then index
    return np.sort(order[:kk])


def softmax_attention(qh: np.ndarray, Kh: np.ndarray, Vh: np.ndarray) -> np.ndarray:
    """softmax(q K^T / sqrt(d_h)) V for one query head (exact attention,
    Eqs. 16-18; reading R10 for the 1/sqrt(d_h) scale)."""
    qh = np.asarray(qh, np.float64)
    logits = np.asarray(Kh, np.float64) @ qh / math.sqrt(qh.shape[0])
    logits -= logits.max()
    p = np.exp(logits)
    p /= p.sum()
    return p @ np.asarray(Vh, np.float64)


def sparse_attention(q, keys_exact, values_exact, CK_sel, CV_sel, BK, BV,
                     n_kv_heads: int) -> np.ndarray:
    """Sparse reconstruction then exact attention ('What carries the
    argument': only the selected positions are rebuilt, Eq. 16, before exact
    attention with the uncompressed sink tokens; the exact recent window is
    reading R3).

    keys_exact/values_exact: [n_exact][D'] uncompressed rows (sinks + recent
    ring); CK_sel/CV_sel: [k][r] coefficients of the selected positions.
    Query head a uses KV head a // G (reading R11).  Returns [H_q][d_h]."""
    q = np.asarray(q, np.float64)
    H_q, d_h = q.shape
    G = H_q // n_kv_heads
    K_hat = np.asarray(CK_sel, np.float64) @ np.asarray(BK, np.float64).T
    V_hat = np.asarray(CV_sel, np.float64) @ np.asarray(BV, np.float64).T
    keys = np.concatenate([np.asarray(keys_exact, np.float64), K_hat], axis=0)
    vals = np.concatenate([np.asarray(values_exact, np.float64), V_hat], axis=0)
    out = np.zeros((H_q, d_h))
    for a in range(H_q):
        h = a // G
        sl = slice(h * d_h, (h + 1) * d_h)
        out[a] = softmax_attention(q[a], keys[:, sl], vals[:, sl])
    return out


# --------------------------------------------------------------------------- #
# the persistent compressed cache of one (layer, sequence)
# --------------------------------------------------------------------------- #
@dataclass
class Cache:
    """Per-(layer, sequence) state ('What carries the argument': sinks kept
    exact, every other token as coefficients; 'If this is right': persistent
    size about r/D' of the full cache).

    Coefficient rows are indexed by absolute position (rows < n_sink unused).
    The recent ring holds the last n_recent tokens exactly; slot = pos mod
    n_recent.  qwin holds the last W query-coefficient blocks; the block
    pushed as number p (counting from 0) sits in slot p mod W, and
    ``pushes`` counts the blocks pushed so far (prompt-tail queries, if the
    window was initialised from them, then one per decode step).

    rank is the key rank r_K (latent scores use 1/sqrt(rank)); rank_v the
    value rank r_V (defaults to rank; 'Reading between the lines' mentions a
    1:1.5 key-to-value rank split).  local_exact False is the variant in
    which the recent window is rebuilt from coefficients like the top-k rows
    ('Core claim': only the local window and the top-k positions are
    reconstructed) instead of being read from the exact ring."""
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    rank: int
    n_sink: int
    q_window: int
    top_k: int
    n_recent: int
    pool_kernel: int
    storage: str
    sink_k: np.ndarray
    sink_v: np.ndarray
    ring_k: np.ndarray
    ring_v: np.ndarray
    CK: np.ndarray
    CV: np.ndarray
    BK: np.ndarray
    BV: np.ndarray
    qwin: np.ndarray
    L: int
    pushes: int = 0
    rank_v: int = 0
    local_exact: bool = True
    last: dict = field(default_factory=dict)

    def __post_init__(self):
        if not self.rank_v:
            self.rank_v = self.rank

    @property
    def G(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def window_rows(self) -> np.ndarray:
        """The W_eff * G valid query-coefficient rows, newest block first,
        W_eff = min(pushes, W) (reading R9: without prompt-tail queries the
        window starts empty and always includes the current query)."""
        w_eff = min(self.pushes, self.q_window)
        slots = [(self.pushes - 1 - i) % self.q_window for i in range(w_eff)]
        if not slots:
            return np.zeros((0, self.rank))
        return np.concatenate([self.qwin[s] for s in slots], axis=0)

    def candidates(self) -> np.ndarray:
        """Compressed candidate positions J = [s, L_t - n_recent)."""
        return np.arange(self.n_sink, max(self.L - self.n_recent, self.n_sink))

    def local_positions(self) -> np.ndarray:
        """The recent window [L_t - n_recent, L_t) (never below the sinks)."""
        return np.arange(max(self.L - self.n_recent, self.n_sink), self.L)


def push_query(cache: Cache, q) -> np.ndarray:
    """Project one token's queries into the key subspace ('Core claim':
    queries are mapped onto the key basis) and push the G coefficient
    vectors into the window ('What carries the argument': the window of
    query coefficients).  The window is stored in fp32 (reading R13).
    Returns the pushed block [G][r_K]."""
    cq = rnd(query_concat(q, cache.n_kv_heads) @ cache.BK, "f32")
    cache.qwin[cache.pushes % cache.q_window] = cq
    cache.pushes += 1
    return cq


def prefill(K: np.ndarray, V: np.ndarray, *, n_q_heads: int, n_kv_heads: int,
            head_dim: int, rank: int, n_sink: int, n_sample: int, q_window: int,
            top_k: int, n_recent: int, pool_kernel: int, storage: str,
            L_max: int | None = None, recent_num: int = 7, recent_den: int = 10,
            rank_v: int | None = None, tail_q=None, local_exact: bool = True,
            BK=None, BV=None):
    """Prefill of one (layer, sequence): sinks and recent ring kept exact,
    bases from the sample, coefficients of every row in [s, L).
    K, V: [L][D'] as stored.  rank_v: value rank (default: rank).
    tail_q: optional [n][H_q][d_h] queries of the last n prompt tokens (oldest
    first, n <= W): the window starts with their coefficients (the variant
    that seeds the window from the prompt's last queries; reading R9 is the
    default, an empty window).  BK, BV: bases to use instead of building
    them (a depth-shared basis).  Returns (Cache, info)."""
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    L, Dp = K.shape
    rank_v = rank if rank_v is None else rank_v
    if Dp != n_kv_heads * head_dim:
        raise ValueError("D' must equal n_kv_heads * head_dim")
    if L < n_sink + n_recent:
        raise ValueError("prompt shorter than sinks + recent window")
    L_max = L if L_max is None else L_max
    info = dict(positions=sample_positions(L, n_sink, n_sample, recent_num, recent_den))
    if BK is None:
        BK, info["lam_k"], info["S_k"], _ = build_basis(K, n_sink, n_sample, rank, storage,
                                                        recent_num, recent_den)
    if BV is None:
        BV, info["lam_v"], info["S_v"], _ = build_basis(V, n_sink, n_sample, rank_v, storage,
                                                        recent_num, recent_den)
    CK = np.zeros((L_max, rank))
    CV = np.zeros((L_max, rank_v))
    CK[n_sink:L] = project(K[n_sink:L], BK, storage)
    CV[n_sink:L] = project(V[n_sink:L], BV, storage)
    ring_k = np.zeros((n_recent, Dp))
    ring_v = np.zeros((n_recent, Dp))
    for p in range(L - n_recent, L):
        ring_k[p % n_recent] = K[p]
        ring_v[p % n_recent] = V[p]
    G = n_q_heads // n_kv_heads
    cache = Cache(n_q_heads, n_kv_heads, head_dim, rank, n_sink, q_window, top_k,
                  n_recent, pool_kernel, storage, K[:n_sink].copy(), V[:n_sink].copy(),
                  ring_k, ring_v, CK, CV, BK, BV, np.zeros((q_window, G, rank)), L, 0,
                  rank_v, local_exact)
    if tail_q is not None:
        if len(tail_q) > q_window:
            raise ValueError("more prompt-tail queries than the window holds")
        for qt in tail_q:
            push_query(cache, qt)
    return cache, info


def decode_append(cache: Cache, q, k_new, v_new):
    """First stage of a decode step: store the new token and its query.

    The new token's key/value coefficients are appended (Eq. 3 applied to the
    new token), its exact key/value enter the recent ring (evicting the
    oldest, which then becomes a compressed candidate), and its queries go
    through push_query.  Mutates cache; returns the pushed block [G][r_K]."""
    k_cat = np.asarray(k_new, np.float64).reshape(-1)
    v_cat = np.asarray(v_new, np.float64).reshape(-1)
    p = cache.L
    if p >= cache.CK.shape[0]:
        raise ValueError("coefficient cache is full")
    cache.CK[p] = rnd(k_cat @ cache.BK, cache.storage)
    cache.CV[p] = rnd(v_cat @ cache.BV, cache.storage)
    cache.ring_k[p % cache.n_recent] = k_cat
    cache.ring_v[p % cache.n_recent] = v_cat
    cache.L = p + 1
    return push_query(cache, q)


def decode_select(cache: Cache):
    """Latent scoring, pooling and top-k over the current candidates.
    Returns (positions selected ascending, score, pooled)."""
    J = cache.candidates()
    score = latent_scores(cache.CK[J], cache.window_rows(), cache.rank)
    pooled = max_pool(score, cache.pool_kernel)
    sel = select_topk(pooled, cache.top_k)
    return J[sel], score, pooled


def decode_attend(cache: Cache, q, positions) -> np.ndarray:
    """Reconstruction of the selected positions and exact attention over the
    sinks, the recent window and the reconstructed rows.  The recent window
    comes from the exact ring, or, with local_exact False, is rebuilt from
    its coefficients together with the selected rows."""
    positions = np.asarray(positions, dtype=np.int64)
    if cache.local_exact:
        keys_exact = np.concatenate([cache.sink_k, cache.ring_k], axis=0)
        vals_exact = np.concatenate([cache.sink_v, cache.ring_v], axis=0)
        rebuilt = positions
    else:
        keys_exact, vals_exact = cache.sink_k, cache.sink_v
        rebuilt = np.concatenate([positions, cache.local_positions()])
    return sparse_attention(q, keys_exact, vals_exact, cache.CK[rebuilt],
                            cache.CV[rebuilt], cache.BK, cache.BV, cache.n_kv_heads)


def decode_step(cache: Cache, q, k_new, v_new) -> np.ndarray:
    """One decode step for one (layer, sequence), in the order the 'Referee
    Report' summary gives: the query coefficients enter the window and score
    the candidates (Eqs. 8-10), the recent window and the k best candidates
    are chosen (Eqs. 13-15), and the chosen rows are rebuilt and attended
    exactly (Eqs. 16-18).  q: [H_q][d_h], k_new/v_new: [H_kv][d_h].  Returns
    out [H_q][d_h]; cache.last holds positions, score and pooled."""
    decode_append(cache, q, k_new, v_new)
    positions, score, pooled = decode_select(cache)
    out = decode_attend(cache, q, positions)
    cache.last = dict(positions=positions, score=score, pooled=pooled)
    return out


# --------------------------------------------------------------------------- #
# accounting
# --------------------------------------------------------------------------- #
def persistent_bytes(L: int, D: int, rank: int, n_sink: int, n_recent: int,
                     elem_bytes: int, rank_v: int | None = None) -> int:
    """Persistent cache bytes of one layer and sequence for K and V: exact
    sinks + exact recent ring + coefficients of the other tokens + bases
    ('If this is right': the persistent cache per layer tends to r/D' of the
    full cache for long contexts; memory analysis Eqs. 19-24)."""
    rank_v = rank if rank_v is None else rank_v
    n_coef = max(L - n_sink, 0)
    return elem_bytes * (2 * (n_sink + n_recent) * D + (n_coef + D) * (rank + rank_v))


def full_cache_bytes(L: int, D: int, elem_bytes: int) -> int:
    return 2 * elem_bytes * L * D


def rank_for_ratio(eta: float, L: int, D: int, n_sink: int, n_recent: int,
                   v_to_k: tuple = (1, 1), multiple: int = 8):
    """Ranks (r_K, r_V) for a target retention ratio eta ('Referee Report'
    major comment 3 and 'Assumptions & free parameters': r is solved from
    the memory equation, Eq. 21, for a target eta).  The page does not print
    Eq. 21; the accounting used here is persistent_bytes / full_cache_bytes
    <= eta.  r_V / r_K = v_to_k[1] / v_to_k[0]; both are multiples of
    ``multiple``.  Returns the largest such pair that meets the target (the
    ratio is increasing in the ranks), or (0, 0) if even rank 0 exceeds it."""
    a, b = v_to_k
    best = (0, 0)
    t = 1
    while True:
        rk, rv = a * t * multiple, b * t * multiple
        if rk > D or rv > D:
            break
        if persistent_bytes(L, D, rk, n_sink, n_recent, 1, rv) > eta * full_cache_bytes(L, D, 1):
            break
        best = (rk, rv)
        t += 1
    return best
