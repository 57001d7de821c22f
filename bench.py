"""Throughput of the compressed-KV decode step on one MI355X.

Workload (default): one Llama-3-8B-shaped attention layer (32 query heads,
8 KV heads, head dim 128, D' = 1024), context 32K, batch 16 sequences, bf16
storage, rank 256, 4 sinks, 2048-row SVD sample, query window 16, top-k 512,
exact recent window 64.  A step is one full decode step of every sequence:
append + query coefficients, latent scoring, pooled top-k, reconstruction and
exact attention, merge.  Inputs (caches, bases, queries) are resident in HBM
before timing.  The caches rotate over several instances with identical
contents, so the scan of one instance cannot be served from the 256 MB
Infinity Cache left by the previous step.

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
METRIC = "decode steps/sec/GPU at 32K ctx (HBM GB/s % of peak); prefill tokens/sec"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(w, U: int, n_cand: float):
    """Bytes the method must move per decode step (per launch for the scan).
    scan: every candidate's key coefficients once; rest: gathered coefficient
    rows (k per unit, K and V), both bases, exact sink + recent rows, the
    query window, and q / k / v / out."""
    G, r, D = w.G, w.rank, w.D
    scan = U * n_cand * r * 2 + U * w.q_window * G * r * 4 + U * w.q_window * G * 8
    gathered = U * w.top_k * r * 2 * 2
    bases = U * D * r * 2 * 2
    exact = U * (w.n_sink + w.n_recent) * D * 2 * 2
    io = U * (w.n_q_heads * w.head_dim * (2 + 4) + 2 * D * 2 + 2 * r * 2 + G * r * 4)
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


def oracle_cache_of(kc, u, w):
    """Float64 oracle state of one unit of a GPU cache (for the CPU baseline)."""
    from oracle import s4r
    f = lambda t: t.detach().float().cpu().double().numpy()
    lens = kc.lens[u].cpu().tolist()
    return s4r.Cache(w.n_q_heads, w.n_kv_heads, w.head_dim, w.rank, w.n_sink, w.q_window,
                     w.top_k, w.n_recent, w.pool_kernel, w.storage, f(kc.sink_k[u]),
                     f(kc.sink_v[u]), f(kc.ring_k[u]), f(kc.ring_v[u]), f(kc.coef_k[u]),
                     f(kc.coef_v[u]), f(kc.basis_k[u]), f(kc.basis_v[u]),
                     f(kc.qwin[u]).reshape(w.q_window, w.G, w.rank), lens[0], lens[1],
                     w.rank_v or w.rank, w.local_window == 0)


def cpu_baseline(kc, dec, w, U, budget_s: float):
    """Oracle decode steps on host cores for one unit, scaled to the batch."""
    from oracle import s4r
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    o = oracle_cache_of(kc, 0, w)
    room = kc.L_max - o.L  # steps the copied cache can still take
    qs = [dec.q[t][0].float().cpu().double().numpy() for t in range(dec.q.shape[0])]
    ks = [dec.k[t][0].float().cpu().double().numpy() for t in range(dec.q.shape[0])]
    vs = [dec.v[t][0].float().cpu().double().numpy() for t in range(dec.q.shape[0])]
    n, t0 = 0, time.perf_counter()
    while True:
        t = n % len(qs)
        s4r.decode_step(o, qs[t], ks[t], vs[t])
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= room:
            break
    per_unit_step = el / n
    return {"value": 1.0 / (per_unit_step * U), "unit": "steps/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n} float64 oracle decode steps of one of the {U} sequences "
                      f"(unit 0, context {o.L - n}), {el:.1f} s, scaled x{U} to the batch"}


def run_prefill_leg(args):
    """Prefill of one 64K sequence: bases (sample, Gram, eigensolve) + projection."""
    w = configs.PREFILL_64K
    cfg = kvlr.config_of(w)
    prompt = synth.make_prompt(w, device="cuda")
    K, V = prompt.K, prompt.V
    kc = kvlr.KVCache.allocate(cfg, 1, w.L)
    ws = torch.empty(kvlr.workspace_bytes(cfg, kvlr.OP_BUILD_BASES, 1, w.L), dtype=torch.uint8,
                     device="cuda")
    pws_n = kvlr.workspace_bytes(cfg, kvlr.OP_PROJECT, 1, w.L)
    pws = torch.empty(max(pws_n, 1), dtype=torch.uint8, device="cuda") if pws_n > 0 else None
    kvlr.build_bases(kc, K, V, ws=ws)  # warm-up
    kvlr.project(kc, K, V, ws=pws)
    torch.cuda.synchronize()
    reps = 2
    t_b = 0.0
    e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
    for _ in range(reps):
        e0.record()
        kvlr.build_bases(kc, K, V, ws=ws)
        e1.record()
        torch.cuda.synchronize()
        t_b += e0.elapsed_time(e1) / reps
    # the projection alone, back to back (inputs resident, workspace allocated once)
    p_reps = 20
    e0.record()
    for _ in range(p_reps):
        kvlr.project(kc, K, V, ws=pws)
    e1.record()
    torch.cuda.synchronize()
    t_p = e0.elapsed_time(e1) / p_reps
    n_proj = 2 * (w.L - w.n_sink)
    flops = 2.0 * n_proj * w.D * w.rank
    return {"workload": w.name, "tokens_per_s": w.L / ((t_b + t_p) / 1e3),
            "build_bases_ms": t_b, "project_ms": t_p,
            "project_tflops": flops / (t_p / 1e3) / 1e12,
            "project_mfma_frac": flops / (t_p / 1e3) / 1e12 / BF16_PEAK_TFLOPS}


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
    a 4 GiB buffer (16x the 256 MB Infinity Cache) through the register path
    and the direct global->LDS path, and the dense bf16 MFMA rate.  Each
    configuration: one untimed launch, then the best of 5 timed launches
    (HIP events on the launch stream)."""
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

    reads = []
    configs_ = [(0, b, dpt) for b in ((1024, 2048) if not full else (256, 512, 1024, 2048, 4096))
                for dpt in ((8,) if not full else (2, 4, 8, 16))] + [(1, 256, 0)]
    for method, blocks, depth in configs_:
        def launch():
            rc = lib.kvlr_probe_read(buf.data_ptr(), nbytes, method, blocks, depth, sink.data_ptr(),
                                     st.cuda_stream)
            assert rc == 0, rc
        ms = best_ms(launch)
        reads.append({"method": ["register", "global_to_lds"][method], "blocks": blocks,
                      "depth": depth, "gbps": round(nbytes / (ms / 1e3) / 1e9, 1)})
    del buf
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
    return {"read": reads, "best_read_gbps": best_read["gbps"],
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=600)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--workload", default=configs.LLAMA8B_32K.name)
    ap.add_argument("--instances", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
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
    if args.copy_probe:
        copy_probe()
        return
    if args.probe:
        kvlr.load()
        torch.cuda.set_device(0)
        print(json.dumps({"probe": run_probes(full=True)}), flush=True)
        return
    if args.prefill_only:
        kvlr.load()
        torch.cuda.set_device(0)
        print(json.dumps({"prefill": run_prefill_leg(args)}), flush=True)
        return
    w = configs.by_name(args.workload)
    if w is None:
        sys.exit(f"unknown workload {args.workload}")
    kvlr.load()
    torch.cuda.set_device(0)
    U = w.n_units
    n_inst = max(1, args.instances)
    per_inst = w.q_window + math.ceil((args.warmup + 3 * args.steps + 6 * n_inst) / n_inst) + 8
    L_max = w.L + per_inst
    cfg = kvlr.config_of(w)

    log(f"[bench] workload {w.name}: generating prompt on the GPU")
    t0 = time.time()
    prompt = synth.make_prompt(w, device="cuda")
    n_dec = 64
    dec = synth.make_decode_inputs(w, prompt, n_dec, device="cuda")
    torch.cuda.synchronize()
    log(f"[bench] prompt ready ({time.time() - t0:.1f} s); building bases + projecting")
    base = kvlr.KVCache.allocate(cfg, U, L_max)
    t0 = time.time()
    kvlr.build_bases(base, prompt.K, prompt.V)
    kvlr.project(base, prompt.K, prompt.V)
    torch.cuda.synchronize()
    log(f"[bench] prefill done ({time.time() - t0:.1f} s)")
    del prompt
    torch.cuda.empty_cache()
    caches = [base] + [base.clone() for _ in range(n_inst - 1)]
    out = torch.empty(U, w.n_q_heads, w.head_dim, device="cuda")
    decs = [kvlr.Decoder(c, out) for c in caches]

    def step(i):
        t = i % n_dec
        decs[i % n_inst].step(dec.q[t], dec.k[t], dec.v[t])

    # fill every instance's query window, then warm up
    for i in range(w.q_window * n_inst):
        step(i)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, n):
        torch.cuda.synchronize()
        e0.record()
        fn(n)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # (a) eager launches
    log(f"[bench] timing {args.steps} eager steps over {n_inst} cache instances")
    ms_eager = timed(lambda n: [step(i) for i in range(n)], args.steps)
    # (b) HIP graph: a fixed run of steps captured once and replayed
    ms_graph = None
    graph_steps = 6 * n_inst
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(graph_steps):
                step(i)
        g.replay()
        torch.cuda.synchronize()
        reps = max(1, args.steps // graph_steps)
        log(f"[bench] timing {reps * graph_steps} graph-replayed steps")
        ms_graph = timed(lambda n: [g.replay() for _ in range(n)], reps) / graph_steps
    except Exception as ex:  # graph capture unavailable: eager numbers only
        log(f"[bench] graph capture failed: {ex}")
    # the faster of the two launch modes is the step time (both are reported);
    # on this ROCm a replayed graph leaves ~5 us between kernel nodes
    use_graph = ms_graph is not None and ms_graph < ms_eager
    ms = ms_graph if use_graph else ms_eager
    # (c) stage timing: HIP events recorded by the library between its launches
    kvlr.profile_enable(True)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    stage_ms, n_prof = kvlr.profile_read()
    kvlr.profile_enable(False)
    stage_ms = {k: v / max(n_prof, 1) for k, v in stage_ms.items()}
    lens = caches[0].lens[0, 0].item()
    n_cand = lens - w.n_sink - w.n_recent
    scan_bytes, step_bytes = algorithmic_bytes(w, U, n_cand)
    score_ms = stage_ms["score"]
    achieved = scan_bytes / (score_ms / 1e3) / 1e9
    roofline = {"bound": "hbm", "kernel": "k_score_bf16 (latent scoring)",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": stored_traffic("k_score_bf16", w.name)}
    result = {
        "metric": METRIC, "value": round(1e3 / ms, 2), "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "context": w.L, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "rank": w.rank,
                   "top_k": w.top_k, "q_window": w.q_window, "n_recent": w.n_recent,
                   "n_sink": w.n_sink, "n_sample": w.n_sample, "cache_instances": n_inst},
        "roofline": roofline,
        "step_hbm_gbps": round(step_bytes / (ms / 1e3) / 1e9, 1),
        "step_hbm_frac": round(step_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
        "stage_us": {k: round(v * 1e3, 2) for k, v in stage_ms.items()},
        "ms_per_step_eager": round(ms_eager, 5),
        "ms_per_step_graph": None if ms_graph is None else round(ms_graph, 5),
        "timing": "hip_graph_replay" if use_graph else "eager",
        "algorithmic_bytes": {"scan_per_launch": int(scan_bytes), "step": int(step_bytes)},
    }
    if not args.no_prefill:
        del caches, decs, base
        torch.cuda.empty_cache()
        log("[bench] prefill leg (64K tokens, D' = 1024, r = 256)")
        result["prefill"] = run_prefill_leg(args)
    if not args.no_cpu:
        log("[bench] oracle CPU baseline")
        # a fresh single-unit prefill for the oracle's state (same workload)
        prompt = synth.make_prompt(w, device="cuda", batch=1)
        kc1 = kvlr.KVCache.allocate(cfg, 1, L_max)
        kvlr.build_bases(kc1, prompt.K, prompt.V)
        kvlr.project(kc1, prompt.K, prompt.V)
        d1 = kvlr.Decoder(kc1, torch.empty(1, w.n_q_heads, w.head_dim, device="cuda"))
        for i in range(w.q_window):
            d1.step(dec.q[i][:1].contiguous(), dec.k[i][:1].contiguous(), dec.v[i][:1].contiguous())
        torch.cuda.synchronize()
        result["cpu_baseline"] = cpu_baseline(kc1, dec, w, U, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
