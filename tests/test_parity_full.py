"""GPU parity at the sizes the benchmark runs, and prefill edge paths.

The decode cases use the workloads' own shapes, so every kernel runs in the
launch configuration the benchmark times: at 32K context and batch 16 each
scoring block scans about 32 position tiles with three segment flushes in the
middle of its scan, and from the second step on the top-k takes its hint
path.  Two units are checked stage by stage on every step (tests/gpu_helpers.py
holds the protocol), including the latent scores against their error bound.
"""
import numpy as np
import pytest
import torch

from long_context_decode_s4r_amd import configs, synth
from oracle import s4r

from gpu_helpers import (check_bases, check_rows, check_sample_bits, np64, run_checked_steps,
                         run_prefill, sample_of_workspace, snapshot)

pytestmark = pytest.mark.gpu


def _kvlr():
    from long_context_decode_s4r_amd import kvlr
    kvlr.load()
    return kvlr


def _prefill_checked(w, prompt, units, L_max, proj_rows=None):
    """Prefill on the GPU, then bases, sample bits and projection rows of the
    listed units against the oracle (projection: all rows, or every
    proj_rows-th row)."""
    kvlr = _kvlr()
    cfg = kvlr.config_of(w)
    U, L = prompt.K.shape[0], prompt.K.shape[1]
    ws = torch.empty(kvlr.workspace_bytes(cfg, kvlr.OP_BUILD_BASES, U, L), dtype=torch.uint8,
                     device="cuda")
    kc, K, V, ek, ev = run_prefill(kvlr, w, prompt, L_max, build_ws=ws)
    S = sample_of_workspace(ws, w, U)
    for u in units:
        print(f"  prefill checks unit {u}", flush=True)
        Ku, Vu = np64(prompt.K[u]), np64(prompt.V[u])
        check_sample_bits(w, Ku, S[u, 0], f"unit {u} K sample")
        check_sample_bits(w, Vu, S[u, 1], f"unit {u} V sample")
        check_bases(w, Ku, np64(kc.basis_k[u]), np64(ek[u]), f"unit {u} K basis")
        check_bases(w, Vu, np64(kc.basis_v[u]), np64(ev[u]), f"unit {u} V basis")
        rows = np.arange(w.n_sink, L)[::proj_rows or 1]
        for X, B, C, what in ((Ku, kc.basis_k[u], kc.coef_k[u], "C^K"), (Vu, kc.basis_v[u], kc.coef_v[u], "C^V")):
            Bn = np64(B)
            ref = s4r.project(X[rows], Bn, w.storage)
            check_rows(np64(C)[rows], ref, w.storage, f"unit {u} {what}", np.abs(X[rows]) @ np.abs(Bn))
        snap = snapshot(kc, u, w)
        assert np.array_equal(snap.sink_k, Ku[:w.n_sink]) and np.array_equal(snap.sink_v, Vu[:w.n_sink])
        assert snap.L == L and snap.pushes == 0
    return kc


def _decode_checked(w, prompt, kc, steps, units):
    dec = synth.make_decode_inputs(w, prompt, steps, device="cuda")
    st = run_checked_steps(_kvlr(), w, kc, dec, steps, units=units)
    print(f"  checked={st.n_checked} topk_near_tie_diffs={st.topk_diffs} worst_gap={st.worst_gap:.3g} "
          f"max_out_err={st.max_out_err:.3g} max_score_err={st.max_score_err:.3g} "
          f"score_err/bound={st.max_score_ratio:.3g} "
          f"score_err_near_tau={st.max_score_err_near_tau:.3g}", flush=True)
    return st


@pytest.mark.timeout(900)
def test_llama_32k_b16_bench_size(gpu_lib):
    """The headline decode workload at full size: 16 sequences of 32 768
    tokens, D' = 1024, r = 256, T' = 2048, W = 16, k = 512; units 0 and 15
    checked on each of 24 steps."""
    w = configs.LLAMA8B_32K
    print(f"case {w.name} full size", flush=True)
    prompt = synth.make_prompt(w, device="cuda")
    steps = 24
    kc = _prefill_checked(w, prompt, [0, 15], w.L + steps + 8, proj_rows=7)
    st = _decode_checked(w, prompt, kc, steps, [0, 15])
    assert st.n_checked == 2 * steps


@pytest.mark.timeout(900)
def test_prefill_d1024_64k_full(gpu_lib):
    """The prefill workload at full size: L = 65 536, T' = 4096, a full-rank
    1024 x 1024 Gram, r = 256; bases, sample bits and every projection row."""
    w = configs.PREFILL_64K
    print(f"case {w.name} full size", flush=True)
    prompt = synth.make_prompt(w, device="cuda")
    _prefill_checked(w, prompt, [0], w.L)


@pytest.mark.timeout(900)
def test_llama_128k_b4_planted(gpu_lib):
    """128K context, batch 4, r = 192, k = 1024, with 2% of the positions
    planted at 4x norm in mid-prompt runs; units 0 and 3 checked."""
    w = configs.LLAMA8B_128K
    print(f"case {w.name} full size", flush=True)
    prompt = synth.make_prompt(w, device="cuda")
    steps = 6
    kc = _prefill_checked(w, prompt, [0, 3], w.L + steps + 8, proj_rows=13)
    st = _decode_checked(w, prompt, kc, steps, [0, 3])
    assert st.n_checked == 2 * steps


@pytest.mark.timeout(900)
def test_qwen_layer_64k_b8(gpu_lib):
    """One layer of the 28-layer Qwen-shaped workload at full size: 64K
    context, batch 8, G = 7 (112 window rows), D' = 512, r = 128."""
    w = configs.QWEN7B_64K.with_(n_layers=1, exponents=(0.5 + 0.7 * 13 / 27,))
    print(f"case {w.name} layer 13 full size", flush=True)
    prompt = synth.make_prompt(w, device="cuda")
    steps = 20
    kc = _prefill_checked(w, prompt, [0, 7], w.L + steps + 8, proj_rows=5)
    st = _decode_checked(w, prompt, kc, steps, [0, 7])
    assert st.n_checked == 2 * steps


@pytest.mark.parametrize("storage", ["f32", "bf16"])
def test_single_token_recent_window(gpu_lib, storage):
    """n_recent = 1: the exact ring holds only the new token, which enters
    the candidates one step later (its c^V is first read then)."""
    if storage == "f32":
        w = configs.TINY_F32.with_(n_q_heads=4, n_kv_heads=2, head_dim=32, rank=16, q_window=4,
                                   top_k=24, n_recent=1, n_sample=64)
    else:
        w = configs.LLAMA8B_32K.with_(n_q_heads=8, n_kv_heads=2, head_dim=128, rank=64,
                                      q_window=8, top_k=64, n_recent=1, n_sample=256,
                                      model="power", exponents=(0.8,))
    print(f"case n_recent=1 {storage}", flush=True)
    prompt = synth.make_prompt(w, L=2000, batch=2)
    steps = 10
    kc = _prefill_checked(w, prompt, [0, 1], 2000 + steps + 4)
    dec = synth.make_decode_inputs(w, prompt, steps, batch=2)
    st = run_checked_steps(_kvlr(), w, kc, dec, steps)
    assert st.n_checked == 2 * steps


@pytest.mark.parametrize("storage,D", [("f32", 64), ("bf16", 1024)])
def test_eigensolve_sweep_report(gpu_lib, storage, D):
    """The sweep counts come back on the device: positive when the Jacobi
    iteration converged, -1 when eig_max_sweeps cut it short (and the
    binding's check then raises)."""
    kvlr = _kvlr()
    if storage == "f32":
        w = configs.TINY_F32
    else:
        w = configs.LLAMA8B_32K.with_(batch=1, n_sample=1024)
    prompt = synth.make_prompt(w, L=4096, batch=1)
    K, V = prompt.K.cuda(), prompt.V.cuda()
    for limit, converged in ((0, True), (1, False)):
        print(f"  eig_max_sweeps={limit}", flush=True)
        cfg = kvlr.config_of(w.with_(eig_max_sweeps=limit))
        kc = kvlr.KVCache.allocate(cfg, 1, 4096)
        sw = torch.full((1, 2), 99, dtype=torch.int32, device="cuda")
        kvlr.build_bases(kc, K, V, sweeps=sw)
        torch.cuda.synchronize()
        got = sw.cpu().tolist()[0]
        if converged:
            assert all(2 <= x <= 24 for x in got), got
        else:
            assert got == [-1, -1], got
            with pytest.raises(kvlr.KvlrError):
                kvlr.build_bases(kc, K, V, check_converged=True)


@pytest.mark.parametrize("storage", ["f32", "bf16"])
def test_decode_graph_replay(gpu_lib, storage):
    """Three kvlr_decode_step calls captured in one HIP graph and replayed four
    times, with eager work and synchronisations between the replays: after
    every replay the output, the top-k picks and every cache buffer equal, bit
    for bit, those of the same three steps run eagerly on an identical cache
    (the step records no memset node and keeps no host state across calls)."""
    kvlr = _kvlr()
    if storage == "f32":
        w = configs.TINY_F32.with_(n_q_heads=4, n_kv_heads=2, head_dim=64, rank=32, q_window=4,
                                   top_k=32, n_recent=8, n_sample=256)
    else:
        w = configs.LLAMA8B_32K.with_(batch=2, n_sample=512, top_k=128)
    L, steps, reps = 4000, 3, 4
    prompt = synth.make_prompt(w, L=L, batch=2)
    dec = synth.make_decode_inputs(w, prompt, steps, batch=2)
    q = [dec.q[t].cuda() for t in range(steps)]
    kn = [dec.k[t].cuda() for t in range(steps)]
    vn = [dec.v[t].cuda() for t in range(steps)]
    ref, *_ = run_prefill(kvlr, w, prompt, L + steps * (reps + 1) + 8, eig=False)
    kc, warm = ref.clone(), ref.clone()
    shape = (2, w.n_q_heads, w.head_dim)
    out_r, out_g, out_w = (torch.empty(shape, device="cuda") for _ in range(3))
    tk_r, tk_g, tk_w = (torch.empty(2, w.top_k, dtype=torch.int32, device="cuda") for _ in range(3))
    d_ref, d_g = kvlr.Decoder(ref, out_r, tk_r), kvlr.Decoder(kc, out_g, tk_g)
    kvlr.Decoder(warm, out_w, tk_w).step(q[0], kn[0], vn[0])  # the library's one-time set-up, eagerly
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(steps):
            d_g.step(q[t], kn[t], vn[t])
    for rep in range(reps):
        print(f"  replay {rep}", flush=True)
        for t in range(steps):
            d_ref.step(q[t], kn[t], vn[t])
        out_w.fill_(float(rep))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_r), rep
        assert torch.equal(tk_g, tk_r), rep
        for name in kvlr.BUFFERS:
            assert torch.equal(getattr(kc, name), getattr(ref, name)), (rep, name)


@pytest.mark.parametrize("storage", ["f32", "bf16"])
def test_prefill_graph_replay(gpu_lib, storage):
    """kvlr_build_bases and kvlr_project captured in one HIP graph: every
    replay (with eager work and synchronisations between replays) gives
    bit-identical bases, coefficients and state to the eager calls."""
    kvlr = _kvlr()
    if storage == "f32":
        w = configs.TINY_F32.with_(n_q_heads=4, n_kv_heads=2, head_dim=64, rank=32, q_window=4,
                                   top_k=32, n_recent=8, n_sample=256)
    else:
        w = configs.LLAMA8B_32K.with_(batch=2, n_sample=512, top_k=128)
    L = 3000
    prompt = synth.make_prompt(w, L=L, batch=2)
    cfg = kvlr.config_of(w)
    K, V = prompt.K.cuda(), prompt.V.cuda()
    ws = torch.empty(kvlr.workspace_bytes(cfg, kvlr.OP_BUILD_BASES, 2, L), dtype=torch.uint8,
                     device="cuda")
    pn = kvlr.workspace_bytes(cfg, kvlr.OP_PROJECT, 2, L)
    pws = torch.empty(pn, dtype=torch.uint8, device="cuda") if pn else None
    sw = torch.zeros(2, 2, dtype=torch.int32, device="cuda")
    ref = kvlr.KVCache.allocate(cfg, 2, L + 8)
    kvlr.build_bases(ref, K, V, ws=ws, sweeps=sw)
    kvlr.project(ref, K, V, ws=pws)
    torch.cuda.synchronize()
    kc = kvlr.KVCache.allocate(cfg, 2, L + 8)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kvlr.build_bases(kc, K, V, ws=ws, sweeps=sw)
        kvlr.project(kc, K, V, ws=pws)
    for rep in range(3):
        print(f"  replay {rep}", flush=True)
        for name in kvlr.BUFFERS:  # eager work between replays
            getattr(kc, name).zero_()
        ws.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name in kvlr.BUFFERS:
            assert torch.equal(getattr(kc, name), getattr(ref, name)), (rep, name)
        assert bool((sw > 0).all())
