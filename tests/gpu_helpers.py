"""Stage-wise GPU-vs-oracle comparison helpers for the parity tests.

Protocol: every decode step is checked on identical stored bits.  The oracle
takes the GPU's state from before the step, runs the append stage itself and
compares the appended rows; it then adopts the GPU's appended rows and window
row, runs scoring + pooling + top-k and compares the scores and the selected
set (equal except near-ties); finally it evaluates the attention output on
the GPU's selected set and compares it with the GPU output.
"""
from __future__ import annotations

import copy
import math
from dataclasses import dataclass, field
from typing import List

import numpy as np
import torch

from oracle import s4r

# Tolerances.
#  - selection: symmetric difference only at near-ties of the oracle's
#    pooled score (|score - tau| < 1e-6, tau = the k-th pooled score);
#  - attention output: relative L2 per (unit, head) <= 1e-5 (fp32 storage) or
#    2e-3 (bf16 storage, fp32 accumulation);
#  - coefficient rows (projection and appended): the GPU rounds an fp32 sum
#    of D' products, the oracle an exact one, so they may differ by the fp32
#    summation error (bounded here by 2^-18 * sum|x_i b_i|, i.e. 64 fp32
#    unit roundoffs of the absolute terms) plus one storage ulp of the result;
#  - query coefficients: fp32 sums of D' products, |diff| <= 1e-5 * sum|terms|.
TIE_GAP = 1e-6
OUT_TOL = {"f32": 1e-5, "bf16": 2e-3}


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float32 if t.dtype == torch.bfloat16 else t.dtype).double().numpy() \
        if t.is_floating_point() else t.detach().cpu().numpy()


def snapshot(kc, u: int, w) -> s4r.Cache:
    """Oracle cache holding the GPU state of unit u (float64 widening)."""
    lens = kc.lens[u].cpu().numpy()
    G = w.n_q_heads // w.n_kv_heads
    return s4r.Cache(
        w.n_q_heads, w.n_kv_heads, w.head_dim, w.rank, w.n_sink, w.q_window, w.top_k,
        w.n_recent, w.pool_kernel, w.storage,
        np64(kc.sink_k[u]), np64(kc.sink_v[u]), np64(kc.ring_k[u]), np64(kc.ring_v[u]),
        np64(kc.coef_k[u]), np64(kc.coef_v[u]), np64(kc.basis_k[u]), np64(kc.basis_v[u]),
        np64(kc.qwin[u]).reshape(w.q_window, G, w.rank), int(lens[0]), int(lens[1]),
        w.rank_v or w.rank, w.local_window == 0)


def bf16_ulps(a: np.ndarray, b: np.ndarray) -> int:
    """Max distance in bf16 steps between two arrays of bf16-representable values."""
    ta = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).int()
    tb = torch.from_numpy(np.ascontiguousarray(b, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).int()
    # map sign-magnitude to a monotone integer line
    ma = torch.where(ta < 0, -(ta & 0x7FFF), ta)
    mb = torch.where(tb < 0, -(tb & 0x7FFF), tb)
    return int((ma - mb).abs().max()) if ma.numel() else 0


def storage_ulp(x: np.ndarray, storage: str) -> np.ndarray:
    bits = 8 if storage == "bf16" else 24
    e = np.floor(np.log2(np.maximum(np.abs(x), 1e-30)))
    return np.exp2(e - (bits - 1))


def check_rows(gpu: np.ndarray, ref: np.ndarray, storage: str, what: str, mag: np.ndarray):
    """gpu, ref: rounded coefficient rows; mag: sum_i |x_i| |b_i| per entry."""
    err = np.abs(gpu - ref)
    bound = storage_ulp(ref, storage) + 2.0 ** -18 * mag
    bad = err > bound
    assert not np.any(bad), f"{what}: {int(bad.sum())} entries beyond the bound, " \
        f"worst ratio {float(np.max(err / bound)):.3g}"


def topk_ok(sel_gpu: np.ndarray, sel_ref: np.ndarray, pooled_ref: np.ndarray, J: np.ndarray,
            k: int):
    """Selected sets equal except for positions at a near-tie of the oracle's
    k-th pooled score.  Returns (ok, n_diff, worst_gap)."""
    a = set(int(x) for x in sel_gpu)
    b = set(int(x) for x in sel_ref)
    if len(a) != len(b):
        return False, -1, float("inf")
    diff = a ^ b
    if not diff:
        return True, 0, 0.0
    kk = min(k, len(J))
    tau = np.sort(pooled_ref)[::-1][kk - 1]
    worst = max(abs(pooled_ref[int(p) - J[0]] - tau) for p in diff)
    return worst < TIE_GAP, len(diff), worst


@dataclass
class StepStats:
    n_checked: int = 0
    topk_diffs: int = 0
    worst_gap: float = 0.0
    max_out_err: float = 0.0
    max_score_err: float = 0.0
    max_score_ratio: float = 0.0      # worst |error| / bound of the latent scores
    max_score_err_near_tau: float = 0.0  # worst error within 1e-4 of the k-th pooled score
    notes: List[str] = field(default_factory=list)


# Latent-score error bound.  bf16 storage: the GPU forms each base-2 logit
# from the query coefficients as a bf16 hi + lo pair (hi = bf16(x), lo =
# bf16(x - hi): together within 2^-18 of x, relative) times the stored
# coefficients, accumulated by 2 r / 32 MFMAs into fp32 (each adds at most
# 2^-24 of the sum of |terms|): |dz| <= (2^-18 + r/16 * 2^-24) A <= 2^-17 A
# for r <= 256, A = sum_i |c_q,i c_k,i| log2(e)/sqrt(r).  fp32 storage: a
# plain fp32 dot product, |dz| <= (r + 1) 2^-24 A.  A softmax probability
# p = 2^(z - m) / S then moves by at most p (dz_j + max_j' dz_j') ln 2 (the
# second term from the normaliser), and the score by the sum of that over
# the window rows; 1.5x margin, plus 1e-6 relative and 1e-9 absolute for the
# fp32 exp2 and sums.
def score_bound(o: s4r.Cache, J: np.ndarray) -> np.ndarray:
    rows = o.window_rows()
    CK = o.CK[J]
    scale = 1.0 / math.sqrt(o.rank)
    Z = rows @ CK.T * scale
    P = np.exp(Z - Z.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    A = np.abs(rows) @ np.abs(CK).T * scale * math.log2(math.e)
    rel = 2.0 ** -17 if o.storage == "bf16" else (o.rank + 1) * 2.0 ** -24
    dz = rel * A
    per_row = P * (dz + dz.max(axis=1, keepdims=True)) * math.log(2.0)
    score = P.sum(axis=0)
    return 1.5 * per_row.sum(axis=0) + 1e-6 * score + 1e-9


def check_decode_step(kc, w, u: int, pre: s4r.Cache, post: s4r.Cache, q, k, v, out_gpu,
                      topk_gpu, scores_gpu, stats: StepStats):
    """Stage-wise comparison of one unit's decode step (see module doc)."""
    storage = w.storage
    o = copy.deepcopy(pre)
    qn, kn, vn = np64(q), np64(k), np64(v)
    s4r.decode_append(o, qn, kn, vn)
    p = o.L - 1
    check_rows(post.CK[p], o.CK[p], storage, f"unit {u} appended c^K",
               np.abs(kn.reshape(-1)) @ np.abs(o.BK))
    check_rows(post.CV[p], o.CV[p], storage, f"unit {u} appended c^V",
               np.abs(vn.reshape(-1)) @ np.abs(o.BV))
    slot = (o.pushes - 1) % o.q_window
    qcat = s4r.query_concat(qn, w.n_kv_heads)
    scale = np.abs(qcat) @ np.abs(o.BK)
    assert np.all(np.abs(post.qwin[slot] - o.qwin[slot]) <= 1e-5 * scale + 1e-30), \
        f"unit {u}: query coefficients differ"
    assert np.array_equal(post.ring_k[p % o.n_recent], o.ring_k[p % o.n_recent])
    assert np.array_equal(post.ring_v[p % o.n_recent], o.ring_v[p % o.n_recent])
    assert post.L == o.L and post.pushes == o.pushes
    # adopt the GPU's stored rows (stage isolation)
    o.CK[p] = post.CK[p]
    o.CV[p] = post.CV[p]
    o.qwin[slot] = post.qwin[slot]
    pos_ref, score_ref, pooled_ref = s4r.decode_select(o)
    J = o.candidates()
    if scores_gpu is not None and len(J):
        sg = np64(scores_gpu)[J]
        err = np.abs(sg - score_ref)
        bound = score_bound(o, J)
        ratio = float(np.max(err / bound))
        stats.max_score_err = max(stats.max_score_err, float(np.max(err)))
        stats.max_score_ratio = max(stats.max_score_ratio, ratio)
        kk = min(w.top_k, len(J))
        if kk > 0:
            tau = np.sort(pooled_ref)[::-1][kk - 1]
            near = np.abs(score_ref - tau) < 1e-4
            if np.any(near):
                stats.max_score_err_near_tau = max(stats.max_score_err_near_tau,
                                                   float(np.max(err[near])))
        assert ratio <= 1.0, (f"unit {u}: latent score error {float(np.max(err)):.3g} exceeds its "
                              f"bound (worst ratio {ratio:.3g})")
    kk = min(w.top_k, len(J))
    sel = np64(topk_gpu)[:kk].astype(np.int64)
    assert np.all(np64(topk_gpu)[kk:] == -1)
    assert np.all(np.diff(sel) > 0), "selected positions must be ascending"
    ok, nd, gap = topk_ok(sel, pos_ref, pooled_ref, J, w.top_k)
    assert ok, f"unit {u}: top-k sets differ by {nd} beyond near-ties (worst gap {gap:.3g})"
    stats.topk_diffs += max(nd, 0)
    stats.worst_gap = max(stats.worst_gap, gap)
    ref = s4r.decode_attend(o, qn, sel)
    og = np64(out_gpu)
    for a in range(w.n_q_heads):
        e = np.linalg.norm(og[a] - ref[a]) / max(np.linalg.norm(ref[a]), 1e-30)
        stats.max_out_err = max(stats.max_out_err, e)
        assert e <= OUT_TOL[storage], f"unit {u} head {a}: rel err {e:.3g}"
    stats.n_checked += 1


def check_bases(w, K_u: np.ndarray, B_gpu: np.ndarray, eig_gpu: np.ndarray, what: str):
    """Bases of one unit and kind vs the oracle's: eigenvalues within
    1e-4 * lambda_1, captured sample energy of the GPU subspace within the
    rounding bound of its storage, orthonormal columns."""
    B_ref, lam, S, _ = s4r.build_basis(K_u, w.n_sink, w.n_sample, B_gpu.shape[1], w.storage,
                                       w.sample_recent_num, w.sample_recent_den)
    assert np.max(np.abs(eig_gpu - lam)) <= 1e-4 * lam[0], f"{what}: eigenvalues"
    Q, _ = np.linalg.qr(B_gpu)
    e_gpu = float(np.sum((S @ Q) ** 2))
    rank = B_gpu.shape[1]
    e_ref = float(np.sum(lam[:rank]))
    # bf16 rounding turns the subspace by O(2^-8); the energy it loses is
    # second order, below 4 * 2^-16 of the captured energy
    tol = 6e-5 if w.storage == "bf16" else 1e-6
    assert abs(e_gpu - e_ref) <= tol * e_ref, f"{what}: energy {e_gpu} vs {e_ref}"
    ortho = np.max(np.abs(B_gpu.T @ B_gpu - np.eye(rank)))
    assert ortho <= (0.05 if w.storage == "bf16" else 1e-5), f"{what}: orthonormality {ortho}"
    return B_ref, lam


def run_prefill(kvlr, w, prompt, L_max, eig=True, build_ws=None):
    """Bases (convergence checked) and projection of a prompt.  build_ws: an
    optional caller workspace for the basis build (its first bytes then hold
    the normalised sample)."""
    cfg = kvlr.config_of(w)
    U, L = prompt.K.shape[0], prompt.K.shape[1]
    kc = kvlr.KVCache.allocate(cfg, U, L_max)
    D = w.n_kv_heads * w.head_dim
    ek = torch.zeros(U, D, device="cuda") if eig else None
    ev = torch.zeros(U, D, device="cuda") if eig else None
    K, V = prompt.K.cuda(), prompt.V.cuda()
    kvlr.build_bases(kc, K, V, ek, ev, ws=build_ws, check_converged=True)
    kvlr.project(kc, K, V)
    torch.cuda.synchronize()
    return kc, K, V, ek, ev


def sample_of_workspace(ws: torch.Tensor, w, U: int) -> torch.Tensor:
    """The normalised sample the basis build leaves at the start of its
    workspace: [U][2 (K, V)][T'][D'] in the storage type."""
    dt = torch.bfloat16 if w.storage == "bf16" else torch.float32
    n = U * 2 * w.n_sample * w.D
    return ws[: n * (2 if w.storage == "bf16" else 4)].view(dt).view(U, 2, w.n_sample, w.D)


def check_sample_bits(w, X_u: np.ndarray, S_gpu: torch.Tensor, what: str):
    """The GPU's stored sample against rnd(normalize_rows(X[positions])):
    bit-exact in bf16 (both sides round the fp64 quotient once).  In fp32 an
    entry may differ by one fp32 step only where the fp64 quotient lies
    within 2^-40 (relative) of an fp32 rounding midpoint, since the two
    sides sum the squared norm in different orders."""
    pos = s4r.sample_positions(X_u.shape[0], w.n_sink, w.n_sample, w.sample_recent_num,
                               w.sample_recent_den)
    exact = s4r.normalize_rows(X_u[pos])
    ref = s4r.rnd(exact, w.storage)
    got = np64(S_gpu)
    if w.storage == "bf16":
        bad = got != ref
        assert not np.any(bad), f"{what}: {int(bad.sum())} sample entries differ from the oracle's"
    else:
        bad = got != ref
        if np.any(bad):
            ulp = np.spacing(np.abs(ref[bad]).astype(np.float32)).astype(np.float64)
            assert np.all(np.abs(got[bad] - ref[bad]) <= ulp), what
            f32 = exact[bad].astype(np.float32).astype(np.float64)
            mid = (f32 + np.where(exact[bad] > f32, ulp, -ulp) / 2)
            assert np.all(np.abs(exact[bad] - mid) <= 2.0 ** -40 * np.abs(exact[bad])), what


def run_checked_steps(kvlr, w, kc, dec, steps: int, units=None, check_every: int = 1,
                      ws_fill=None):
    """Run `steps` decode steps on the GPU, checking the listed units stage
    by stage.  ws_fill(t, ws) may overwrite the decode workspace before step
    t (its contents between calls must never change a result).  Returns
    StepStats."""
    U = kc.n_units
    units = list(range(U)) if units is None else units
    out = torch.empty(U, w.n_q_heads, w.head_dim, device="cuda")
    topk = torch.empty(U, w.top_k, dtype=torch.int32, device="cuda")
    scores = torch.zeros(U, kc.L_max, device="cuda")
    ws = kvlr.decode_workspace(kc)
    stats = StepStats()
    for t in range(steps):
        chk = (t % check_every == 0) or t == steps - 1
        pre = [snapshot(kc, u, w) for u in units] if chk else None
        q, k, v = dec.q[t].cuda(), dec.k[t].cuda(), dec.v[t].cuda()
        print(f"  step {t}", flush=True)
        if ws_fill is not None:
            ws_fill(t, ws)
        kvlr.decode_step(kc, q, k, v, out, topk, scores, ws)
        torch.cuda.synchronize()
        if chk:
            for i, u in enumerate(units):
                post = snapshot(kc, u, w)
                check_decode_step(kc, w, u, pre[i], post, q[u], k[u], v[u], out[u], topk[u],
                                  scores[u], stats)
    return stats
