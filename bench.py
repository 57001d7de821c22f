"""Throughput of the compressed-KV decode step on one MI355X.

Default workload: one Llama-3-8B-shaped attention layer (32 query heads, 8 KV
heads, head dim 128, D' = 1024), context 32K, batch 16 sequences, bf16
storage, rank 256, 4 sinks, 2048-row SVD sample, query window 16, top-k 512,
exact recent window 64.  A step is one full decode step of every sequence:
append + query coefficients, latent scoring, pooled top-k, reconstruction and
exact attention, merge.  Inputs (caches, bases, queries) are resident in HBM
before timing.  The caches rotate over several instances with identical
contents (as the layers of a model would), enough that what one instance's
step reads through the caches (bases, gathered rows, exact rows) totals twice
the 256 MB Infinity Cache over a rotation: a step cannot be served from what
the same instance's previous step left there.  (The scan itself is read
non-temporally and leaves nothing behind.)

Other workloads (``--workload``): the same layer at 128K context and batch 4
(planted atypical norms); the 28-layer Qwen-2.5-7B-shaped model at 64K, batch
8, a step being 28 per-layer calls captured in one HIP graph; the tiny fp32
single-head case (microseconds per step).  ``--probe`` measures the read
bandwidth and MFMA ceilings only.

Prints one JSON line.  ``--gpus`` above 1 is refused: the path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from long_context_decode_s4r_amd import configs, kvlr, profiling, synth  # noqa: E402

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, vendor figure
MALL_BYTES = 256 << 20       # MI355X Infinity Cache
METRIC = "decode steps/sec/GPU at 32K ctx (HBM GB/s % of peak); prefill tokens/sec"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(w, U: int, n_cand: float):
    """Bytes the method must move per decode step of U units (per launch for
    the scan).  scan: every candidate's key coefficients once, plus the query
    window (fp32) and its row statistics; rest: gathered coefficient rows (k
    per unit, K and V), both bases, exact sink + recent rows, and q / k / v /
    out."""
    G, r, rv, D = w.G, w.rank, w.rank_v or w.rank, w.D
    eb = 2 if w.storage == "bf16" else 4
    scan = U * n_cand * r * eb + U * w.q_window * G * (r * 4 + 8)
    gathered = U * w.top_k * (r + rv) * eb
    bases = U * D * (r + rv) * eb
    exact = U * (w.n_sink + w.n_recent) * D * eb * 2
    io = U * (w.n_q_heads * w.head_dim * (eb + 4) + 2 * D * eb + (r + rv) * eb + G * r * 4)
    return scan, scan + gathered + bases + exact + io


def stored_traffic(kernel: str, workload: str):
    """HBM traffic per launch measured with rocprofv3 counters, if it was taken
    on the current kernel sources (profiles/traffic.json)."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
        e = d[kernel][workload]
        if e.get("source_sha") != profiling.source_sha():
            return None
        return float(e["bytes_per_launch"])
    except Exception:
        return None


# --------------------------------------------------------------------------- #
# measured ceilings
# --------------------------------------------------------------------------- #
def _probe_lib():
    import ctypes
    lib = kvlr.load()
    lib.kvlr_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.kvlr_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p]
    return lib


def run_probes(full: bool = True):
    """Measured ceilings (include/kvlr_probe.h): streaming-read bandwidth over
    a 4 GiB buffer (16x the Infinity Cache) through the register path and the
    direct global->LDS path (plain and non-temporal, the latter being the
    latent scan's loads), and the dense bf16 MFMA rate.  Each
    configuration: one untimed launch, then the best of 5 timed launches (HIP
    events on the launch stream).  full=False runs only the configurations
    that were best on this GPU."""
    lib = _probe_lib()
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best_ms(launch, reps=5):
        launch()
        best = float("inf")
        for _ in range(reps):
            e0.record(st)
            launch()
            e1.record(st)
            e1.synchronize()
            best = min(best, e0.elapsed_time(e1))
        return best

    if full:
        cfgs = [(0, b, dp) for b in (256, 512, 1024, 2048, 4096) for dp in (2, 4, 8, 16)] + [(1, 256, 0), (2, 256, 0)]
        cfgs += [(m, 256, ch) for m in (3, 4) for ch in (64, 128, 256, 512, 2048)]
    else:
        cfgs = [(0, 256, 8), (0, 512, 4), (1, 256, 0), (2, 256, 0)]
    reads = []
    for method, blocks, depth in cfgs:
        def launch():
            rc = lib.kvlr_probe_read(buf.data_ptr(), nbytes, method, blocks, depth, sink.data_ptr(),
                                     st.cuda_stream)
            assert rc == 0, rc
        ms = best_ms(launch)
        reads.append({"method": ["register", "global_to_lds", "global_to_lds_nt", "lds_row_slabs",
                                 "lds_row_slabs_nt"][method], "blocks": blocks,
                      "depth": depth, "gbps": round(nbytes / (ms / 1e3) / 1e9, 1)})
    del buf
    # the ceiling is the best contiguous stream; the row-slab reads (the
    # access pattern of the prefill projection: rows of 2048 B read in
    # column slabs of `depth` bytes) are reported beside it
    rows = [r for r in reads if r["method"].startswith("lds_row_slabs")]
    reads = [r for r in reads if not r["method"].startswith("lds_row_slabs")]
    mfma = []
    for shape, fl in ((0, 16384), (1, 32768)):
        blocks, iters = 2048, 4000
        def launch():
            rc = lib.kvlr_probe_mfma(shape, iters, blocks, sink.data_ptr(), st.cuda_stream)
            assert rc == 0, rc
        ms = best_ms(launch)
        flops = blocks * 4 * iters * 8 * fl
        mfma.append({"shape": ["16x16x32_bf16", "32x32x16_bf16"][shape],
                     "tflops": round(flops / (ms / 1e3) / 1e12, 1)})
    best_read = max(reads, key=lambda r: r["gbps"])
    torch.cuda.empty_cache()
    return {"read": reads, "row_slab_read": rows, "best_read_gbps": best_read["gbps"],
            "best_read_config": {k: best_read[k] for k in ("method", "blocks", "depth")},
            "mfma": mfma, "best_mfma_tflops": max(m["tflops"] for m in mfma)}


COPY_PROBE_BYTES = 1 << 30


def copy_probe():
    """Five copies of a 1 GiB device buffer (reads and writes 1 GiB each): the
    reference for scaling rocprofv3's FETCH_SIZE / WRITE_SIZE counters."""
    a = torch.ones(COPY_PROBE_BYTES // 4, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": COPY_PROBE_BYTES, "copies": 5}), flush=True)


# --------------------------------------------------------------------------- #
# CPU baseline: the float64 oracle on the host cores
# --------------------------------------------------------------------------- #
def oracle_cache_of(kc, u, w, extra_rows: int):
    """Float64 oracle state of one unit of a GPU cache, with room for
    extra_rows more tokens."""
    import numpy as np
    from oracle import s4r
    f = lambda t: t.detach().float().cpu().double().numpy()
    lens = kc.lens[u].cpu().tolist()
    grow = lambda a: np.concatenate([a, np.zeros((extra_rows, a.shape[1]))])
    return s4r.Cache(w.n_q_heads, w.n_kv_heads, w.head_dim, w.rank, w.n_sink, w.q_window,
                     w.top_k, w.n_recent, w.pool_kernel, w.storage, f(kc.sink_k[u]),
                     f(kc.sink_v[u]), f(kc.ring_k[u]), f(kc.ring_v[u]), grow(f(kc.coef_k[u])),
                     grow(f(kc.coef_v[u])), f(kc.basis_k[u]), f(kc.basis_v[u]),
                     f(kc.qwin[u]).reshape(w.q_window, w.G, w.rank), lens[0], lens[1],
                     w.rank_v or w.rank, w.local_window == 0)


def cpu_baseline(kc, dec, w, U, budget_s: float, u: int = 0, scale_note: str = ""):
    """Oracle decode steps of one unit on the host cores for about budget_s
    seconds, scaled to the U units of a step.  The BLAS threads are set to
    the cores this process may run on."""
    from oracle import s4r
    cores = len(os.sched_getaffinity(0))
    limiter = None
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:
        pass
    o = oracle_cache_of(kc, u, w, extra_rows=4096)
    L0 = o.L
    qs = [dec.q[t][u].float().cpu().double().numpy() for t in range(dec.q.shape[0])]
    ks = [dec.k[t][u].float().cpu().double().numpy() for t in range(dec.q.shape[0])]
    vs = [dec.v[t][u].float().cpu().double().numpy() for t in range(dec.q.shape[0])]
    n, t0 = 0, time.perf_counter()
    while True:
        t = n % len(qs)
        s4r.decode_step(o, qs[t], ks[t], vs[t])
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 4096:
            break
    if limiter is not None and hasattr(limiter, "restore_original_limits"):
        limiter.restore_original_limits()
    per_unit_step = el / n
    return {"value": round(1.0 / (per_unit_step * U), 4), "unit": "steps/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{n} float64 oracle decode steps of one unit (context {L0} to {o.L}), "
                      f"{el:.1f} s on {cores} cores, scaled x{U} to the {U} units of a step"
                      + scale_note}


# --------------------------------------------------------------------------- #
# prefill legs
# --------------------------------------------------------------------------- #
def _time_ms(fn, reps):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(reps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def run_prefill_leg():
    """Prefill of one 64K-token sequence (D' = 1024, r = 256, T' = 4096):
    bases (sample, Gram, eigensolve) + projection of K and V, prefill
    tokens/s = L / (basis build + projection).  Two prompts (two seeds)
    alternate in the timed loops, so a call never finds the previous call's
    prompt in the Infinity Cache.  The full-prompt basis build (T' = L - s,
    the full-prompt SVD baseline) is timed beside it."""
    w = configs.PREFILL_64K
    cfg = kvlr.config_of(w)
    prompts = [synth.make_prompt(w.with_(seed=w.seed + i), device="cuda") for i in range(2)]
    kc = kvlr.KVCache.allocate(cfg, 1, w.L)
    ws = torch.empty(kvlr.workspace_bytes(cfg, kvlr.OP_BUILD_BASES, 1, w.L), dtype=torch.uint8,
                     device="cuda")
    pws_n = kvlr.workspace_bytes(cfg, kvlr.OP_PROJECT, 1, w.L)
    pws = torch.empty(max(pws_n, 1), dtype=torch.uint8, device="cuda") if pws_n > 0 else None
    sw = torch.zeros(1, 2, dtype=torch.int32, device="cuda")
    for p in prompts:  # warm-up
        kvlr.build_bases(kc, p.K, p.V, ws=ws, sweeps=sw)
        kvlr.project(kc, p.K, p.V, ws=pws)
    torch.cuda.synchronize()
    t_b = _time_ms(lambda i: kvlr.build_bases(kc, prompts[i % 2].K, prompts[i % 2].V, ws=ws, sweeps=sw), 4)
    sweeps = sw.cpu().tolist()[0]
    t_p = _time_ms(lambda i: kvlr.project(kc, prompts[i % 2].K, prompts[i % 2].V, ws=pws), 20)
    n_proj = 2 * (w.L - w.n_sink)
    flops = 2.0 * n_proj * w.D * w.rank
    # the projection's attainable ceiling: it reads the states and writes the
    # coefficients (bf16), so below the ridge it is bound by HBM at its
    # arithmetic intensity, min(MFMA peak, intensity x 8 TB/s)
    proj_bytes = 2.0 * n_proj * (w.D + w.rank)
    attainable = min(BF16_PEAK_TFLOPS, flops / proj_bytes * HBM_PEAK_GBPS / 1e3)
    tflops = flops / (t_p / 1e3) / 1e12
    leg = {"workload": w.name, "tokens_per_s": round(w.L / ((t_b + t_p) / 1e3), 1),
           "build_bases_ms": round(t_b, 3), "project_ms": round(t_p, 4),
           "eig_sweeps_kv": sweeps,
           "project_tflops": round(tflops, 1),
           "project_mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4),
           "project_attainable_tflops": round(attainable, 1),
           "project_frac_of_attainable": round(tflops / attainable, 4),
           "timing": "HIP events around 4 builds / 20 projections, two prompts alternating"}
    # For reference only: the vendor library's GEMM (torch.matmul, hipBLASLt)
    # on the same two products, x[s:] . B for K and V, bf16 out, same
    # alternation.  Not part of the path.
    outs = [torch.empty(w.L - w.n_sink, w.rank, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    bk, bv = kc.basis_k[0].contiguous(), kc.basis_v[0].contiguous()

    def lib_gemm(i):
        p = prompts[i % 2]
        torch.matmul(p.K[0, w.n_sink:], bk, out=outs[0])
        torch.matmul(p.V[0, w.n_sink:], bv, out=outs[1])
    lib_gemm(0)
    t_l = _time_ms(lib_gemm, 20)
    leg["library_gemm_ms"] = round(t_l, 4)
    leg["library_gemm_tflops"] = round(flops / (t_l / 1e3) / 1e12, 1)
    del outs
    # For reference only: the vendor eigensolver (torch.linalg.eigh, fp32,
    # both D' x D' Grams in one batched call) on Grams of the same size and
    # spectrum (the last T' rows, each divided by its norm).  Not part of the
    # path; compare with build_bases_ms, which the eigensolve dominates.
    grams = []
    for X in (prompts[0].K[0], prompts[0].V[0]):
        S = X[w.L - w.n_sample:].float()
        S = S / S.norm(dim=1, keepdim=True)
        grams.append(S.T @ S)
    grams = torch.stack(grams)
    torch.linalg.eigh(grams)
    t_e = _time_ms(lambda i: torch.linalg.eigh(grams), 2)
    leg["library_eigh_ms"] = round(t_e, 3)
    del grams, S
    del ws
    torch.cuda.empty_cache()
    # the full-prompt baseline: every non-sink token in the Gram
    wf = w.with_(n_sample=w.L - w.n_sink)
    cff = kvlr.config_of(wf)
    wsf = torch.empty(kvlr.workspace_bytes(cff, kvlr.OP_BUILD_BASES, 1, w.L), dtype=torch.uint8,
                      device="cuda")
    kf = kvlr.KVCache.allocate(cff, 1, w.L)
    kvlr.build_bases(kf, prompts[0].K, prompts[0].V, ws=wsf, sweeps=sw)
    torch.cuda.synchronize()
    t_f = _time_ms(lambda i: kvlr.build_bases(kf, prompts[i % 2].K, prompts[i % 2].V, ws=wsf, sweeps=sw), 2)
    leg["full_prompt"] = {"n_sample": wf.n_sample, "build_bases_ms": round(t_f, 3),
                          "tokens_per_s": round(w.L / ((t_f + t_p) / 1e3), 1),
                          "gram_gflop": round(2 * 2.0 * wf.n_sample * w.D * w.D / 1e9, 1),
                          "eig_sweeps_kv": sw.cpu().tolist()[0]}
    del wsf, kf, kc, prompts
    torch.cuda.empty_cache()
    # The same prefill for a batch of 8 sequences in one call: the eigensolve
    # is bound by the latency of its rounds on 32 CUs at one sequence, so a
    # batch fills the GPU for about the same wall time.  Reported beside the
    # single-sequence line, which is the workload's own.
    B = 8
    wb = w.with_(batch=B)
    cfb = kvlr.config_of(wb)
    pb = synth.make_prompt(wb, device="cuda")
    kb = kvlr.KVCache.allocate(cfb, B, w.L)
    wsb = torch.empty(kvlr.workspace_bytes(cfb, kvlr.OP_BUILD_BASES, B, w.L), dtype=torch.uint8,
                      device="cuda")
    pwb_n = kvlr.workspace_bytes(cfb, kvlr.OP_PROJECT, B, w.L)
    pwb = torch.empty(max(pwb_n, 1), dtype=torch.uint8, device="cuda")
    swb = torch.zeros(B, 2, dtype=torch.int32, device="cuda")
    kvlr.build_bases(kb, pb.K, pb.V, ws=wsb, sweeps=swb)
    kvlr.project(kb, pb.K, pb.V, ws=pwb)
    t_bb = _time_ms(lambda i: kvlr.build_bases(kb, pb.K, pb.V, ws=wsb, sweeps=swb), 2)
    t_pb = _time_ms(lambda i: kvlr.project(kb, pb.K, pb.V, ws=pwb), 4)
    sw_b = swb.cpu().tolist()
    leg["batch_8"] = {"sequences": B, "build_bases_ms": round(t_bb, 3), "project_ms": round(t_pb, 4),
                      "tokens_per_s": round(B * w.L / ((t_bb + t_pb) / 1e3), 1),
                      "eig_sweeps": sorted({v for x in sw_b for v in x})}
    del pb, kb, wsb, pwb
    torch.cuda.empty_cache()
    return leg


# --------------------------------------------------------------------------- #
# decode legs
# --------------------------------------------------------------------------- #
def _timed_eager_and_graph(step, steps, graph_steps, log_name):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, n):
        torch.cuda.synchronize()
        e0.record()
        fn(n)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    log(f"[bench] {log_name}: timing {steps} eager steps")
    ms_eager = timed(lambda n: [step(i) for i in range(n)], steps)
    ms_graph = None
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(graph_steps):
                step(i)
        g.replay()
        torch.cuda.synchronize()
        reps = max(1, steps // graph_steps)
        log(f"[bench] {log_name}: timing {reps * graph_steps} graph-replayed steps")
        ms_graph = timed(lambda n: [g.replay() for _ in range(n)], reps) / graph_steps
    except Exception as ex:  # graph capture unavailable: eager numbers only
        log(f"[bench] graph capture failed: {ex}")
    return ms_eager, ms_graph


def _stage_profile(step, steps):
    kvlr.profile_enable(True)
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    stage_ms, n_prof = kvlr.profile_read()
    kvlr.profile_enable(False)
    return {k: v / max(n_prof, 1) for k, v in stage_ms.items()}


def scorer_kernel(w):
    """The latent-scoring kernel the library launches for this shape (its
    dispatch rule: the MFMA 32x32x16 scorer for 65..128 window rows and key
    rank <= 192 in bf16, else k_score_bf16; fp32 storage: k_score_f32)."""
    if w.storage != "bf16":
        return "k_score_f32"
    rows = w.q_window * w.G
    return "k_score_mfma32" if 64 < rows <= 128 and w.rank <= 192 else "k_score_bf16"


def _roofline(scan_bytes, score_ms, w, ceiling):
    achieved = scan_bytes / (score_ms / 1e3) / 1e9
    kern = scorer_kernel(w)
    r = {"bound": "hbm", "kernel": f"{kern} (latent scoring)", "achieved": round(achieved, 1),
         "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
         "traffic": stored_traffic(kern, w.name)}
    if ceiling:
        r["measured_read_ceiling"] = ceiling
        r["frac_of_measured_ceiling"] = round(achieved / ceiling, 4)
    return r


def _config_of(w, n_inst):
    c = {"workload": w.name, "layers": w.n_layers, "batch": w.batch, "context": w.L,
         "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
         "rank": w.rank, "top_k": w.top_k, "q_window": w.q_window, "n_recent": w.n_recent,
         "n_sink": w.n_sink, "n_sample": w.n_sample, "storage": w.storage,
         "cache_instances": n_inst}
    if w.planted_frac:
        c["planted"] = {"fraction": w.planted_frac, "scale": w.planted_scale}
    return c


def _result(w, args, ms, ms_eager, ms_graph, stage_ms, scan_bytes, step_bytes, ceiling, n_inst,
            timing_note=""):
    use_graph = ms_graph is not None and ms_graph <= ms_eager
    return {
        "metric": METRIC, "value": round(1e3 / ms, 2), "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "us_per_step": round(ms * 1e3, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.storage,
        "data": "synthetic",
        "config": _config_of(w, n_inst),
        "roofline": _roofline(scan_bytes, stage_ms["score"], w, ceiling),
        "step_hbm_gbps": round(step_bytes / (ms / 1e3) / 1e9, 1),
        "step_hbm_frac": round(step_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
        "stage_us": {k: round(v * 1e3, 2) for k, v in stage_ms.items()},
        "ms_per_step_eager": round(ms_eager, 5),
        "ms_per_step_graph": None if ms_graph is None else round(ms_graph, 5),
        "timing": ("hip_graph_replay" if use_graph else "eager") + timing_note,
        "algorithmic_bytes": {"scan": int(scan_bytes), "step": int(step_bytes)},
    }


def run_layer_decode(w, args, ceiling):
    """Decode of one layer's batch (the 32K and 128K workloads, and the tiny
    fp32 case): units = the batch's sequences of one layer."""
    U = w.n_units
    cfg = kvlr.config_of(w)
    el = 2 if w.storage == "bf16" else 4
    rv = w.rank_v or w.rank
    # bytes a step reads with cached loads: B^K (its transposed copy), B^V,
    # the gathered coefficient rows and the exact rows
    reread = U * el * ((w.rank + rv) * w.D + w.top_k * (w.rank + rv)
                       + 2 * (w.n_sink + w.n_recent) * w.D)
    n_inst = args.instances or max(3, min(32, math.ceil(2 * MALL_BYTES / reread)))
    per_inst = w.q_window + math.ceil((args.warmup + 3 * args.steps + 6 * n_inst) / n_inst) + 8
    L_max = w.L + per_inst
    log(f"[bench] workload {w.name}: generating prompt on the GPU")
    t0 = time.time()
    prompt = synth.make_prompt(w, device="cuda")
    n_dec = 64
    dec = synth.make_decode_inputs(w, prompt, n_dec, device="cuda")
    base = kvlr.KVCache.allocate(cfg, U, L_max)
    kvlr.build_bases(base, prompt.K, prompt.V, check_converged=True)
    kvlr.project(base, prompt.K, prompt.V)
    torch.cuda.synchronize()
    log(f"[bench] prompt + prefill ready ({time.time() - t0:.1f} s); {n_inst} cache instances")
    del prompt
    torch.cuda.empty_cache()
    caches = [base] + [base.clone() for _ in range(n_inst - 1)]
    out = torch.empty(U, w.n_q_heads, w.head_dim, device="cuda")
    decs = [kvlr.Decoder(c, out) for c in caches]

    def step(i):
        t = i % n_dec
        decs[i % n_inst].step(dec.q[t], dec.k[t], dec.v[t])

    for i in range(w.q_window * n_inst + args.warmup):  # fill every window, then warm up
        step(i)
    torch.cuda.synchronize()
    ms_eager, ms_graph = _timed_eager_and_graph(step, args.steps, 6 * n_inst, w.name)
    ms = min(ms_eager, ms_graph) if ms_graph is not None else ms_eager
    stage_ms = _stage_profile(step, args.steps)
    lens = caches[0].lens[0, 0].item()
    n_cand = lens - w.n_sink - w.n_recent
    scan_bytes, step_bytes = algorithmic_bytes(w, U, n_cand)
    result = _result(w, args, ms, ms_eager, ms_graph, stage_ms, scan_bytes, step_bytes, ceiling, n_inst)
    del decs, caches, base
    torch.cuda.empty_cache()
    return result, dec


def run_model_decode(w, args, ceiling):
    """Decode of the 28-layer workload: a step is one call per layer (that
    layer's batch of units), the layers in order as a model issues them; the
    calls of several steps are captured in one HIP graph and replayed.  One
    step scans 3.75 GB, far beyond the Infinity Cache, so one cache instance."""
    cfg = kvlr.config_of(w)
    B, NL = w.batch, w.n_layers
    L_max = w.L + w.q_window + args.warmup + 3 * args.steps + 16
    kc = kvlr.KVCache.allocate(cfg, NL * B, L_max)
    n_dec = 32
    q = torch.empty(n_dec, NL * B, w.n_q_heads, w.head_dim, dtype=torch.bfloat16, device="cuda")
    kn = torch.empty(n_dec, NL * B, w.n_kv_heads, w.head_dim, dtype=torch.bfloat16, device="cuda")
    vn = torch.empty_like(kn)
    log(f"[bench] workload {w.name}: {NL} layers, prefill one layer at a time")
    t0 = time.time()
    for l in range(NL):
        p = synth.make_prompt(w, device="cuda", n_layers=1, first_layer=l)
        d = synth.make_decode_inputs(w, p, n_dec, device="cuda", first_layer=l)
        view = kc.units(l * B, B)
        kvlr.build_bases(view, p.K, p.V, check_converged=True)
        kvlr.project(view, p.K, p.V)
        q[:, l * B:(l + 1) * B] = d.q
        kn[:, l * B:(l + 1) * B] = d.k
        vn[:, l * B:(l + 1) * B] = d.v
        del p, d
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log(f"[bench] prefill of {NL} layers done ({time.time() - t0:.1f} s)")
    out = torch.empty(NL * B, w.n_q_heads, w.head_dim, device="cuda")
    decs = [kvlr.Decoder(kc.units(l * B, B), out[l * B:(l + 1) * B]) for l in range(NL)]
    qs = [[q[t, l * B:(l + 1) * B] for l in range(NL)] for t in range(n_dec)]
    ks = [[kn[t, l * B:(l + 1) * B] for l in range(NL)] for t in range(n_dec)]
    vs = [[vn[t, l * B:(l + 1) * B] for l in range(NL)] for t in range(n_dec)]

    def step(i):
        t = i % n_dec
        for l in range(NL):
            decs[l].step(qs[t][l], ks[t][l], vs[t][l])

    for i in range(w.q_window + args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms_eager, ms_graph = _timed_eager_and_graph(step, args.steps, 4, w.name)
    ms = min(ms_eager, ms_graph) if ms_graph is not None else ms_eager
    stage_ms = _stage_profile(step, max(8, args.steps // 4))
    stage_ms = {k: v * NL for k, v in stage_ms.items()}  # per layer call -> per step
    lens = kc.lens[0, 0].item()
    n_cand = lens - w.n_sink - w.n_recent
    scan_bytes, step_bytes = algorithmic_bytes(w, NL * B, n_cand)
    result = _result(w, args, ms, ms_eager, ms_graph, stage_ms, scan_bytes, step_bytes, ceiling, 1,
                     f" ({NL} per-layer calls per step)")
    result["unit"] = f"steps/s (all {NL} layers)"
    dec = synth.DecodeInputs(q, kn, vn)
    return result, dec, kc


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=600)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--workload", default=configs.LLAMA8B_32K.name,
                    help="one of: " + ", ".join(w.name for w in configs.ALL if w.decode_steps))
    ap.add_argument("--instances", type=int, default=0, help="cache instances (0 = auto)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain device copy of known size (HBM counter calibration)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only run the prefill leg (basis build + projection of one 64K sequence)")
    ap.add_argument("--probe", action="store_true",
                    help="only run the measured-ceiling probes (read bandwidth, bf16 MFMA rate)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the compressed-KV path has no multi-GPU part "
              "(units shard across GPUs without exchange); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    kvlr.load()
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe()
        return
    if args.probe:
        print(json.dumps({"probe": run_probes(full=True)}), flush=True)
        return
    if args.prefill_only:
        print(json.dumps({"prefill": run_prefill_leg()}), flush=True)
        return
    w = configs.by_name(args.workload)
    if w is None or not w.decode_steps:
        sys.exit(f"unknown decode workload {args.workload}")
    ceiling = probe = None
    if not args.no_probe:
        log("[bench] read-bandwidth probe")
        probe = run_probes(full=False)
        ceiling = probe["best_read_gbps"]
    if w.n_layers > 1:
        result, dec, kc = run_model_decode(w, args, ceiling)
    else:
        result, dec = run_layer_decode(w, args, ceiling)
        kc = None
    if probe:
        result["probe"] = {"best_read_gbps": probe["best_read_gbps"],
                           "best_read_config": probe["best_read_config"],
                           "best_mfma_tflops": probe["best_mfma_tflops"]}
    if not args.no_prefill and w.name == configs.LLAMA8B_32K.name:
        log("[bench] prefill leg (64K tokens, D' = 1024, r = 256)")
        result["prefill"] = run_prefill_leg()
    if not args.no_cpu:
        log("[bench] oracle CPU baseline")
        if kc is None:
            # a fresh single-unit prefill of the same workload for the oracle's state
            prompt = synth.make_prompt(w, device="cuda", batch=1)
            kc1 = kvlr.KVCache.allocate(kvlr.config_of(w), 1, w.L + w.q_window + 8)
            kvlr.build_bases(kc1, prompt.K, prompt.V)
            kvlr.project(kc1, prompt.K, prompt.V)
            d1 = kvlr.Decoder(kc1, torch.empty(1, w.n_q_heads, w.head_dim, device="cuda"))
            for i in range(w.q_window):
                d1.step(dec.q[i][:1].contiguous(), dec.k[i][:1].contiguous(), dec.v[i][:1].contiguous())
            torch.cuda.synchronize()
            result["cpu_baseline"] = cpu_baseline(kc1, dec, w, w.n_units, args.cpu_budget)
        else:
            result["cpu_baseline"] = cpu_baseline(kc, dec, w, w.n_units, args.cpu_budget,
                                                  scale_note=" (layer 0, sequence 0; the units "
                                                  "differ only in their spectra)")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
