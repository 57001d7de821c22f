"""Thin ctypes binding of libkvlr.so (include/kvlr.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Tensors are torch tensors used as device memory; work goes on the
current torch stream.  ``load()`` raises when the library has not been built
(there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvlr.so")

F32, BF16 = 0, 1
OK, EINVAL, EWORKSPACE, EDEVICE, ELAUNCH = 0, 1, 2, 3, 4
OP_BUILD_BASES, OP_PROJECT, OP_DECODE, OP_INIT_WINDOW = 0, 1, 2, 3
BUFFERS = ("sink_k", "sink_v", "ring_k", "ring_v", "coef_k", "coef_v", "basis_k", "basis_v",
           "qwin", "lens", "state")
LOCAL_EXACT, LOCAL_RECONSTRUCTED = 0, 1
STAGES = ("prologue", "score", "pool", "topk", "attend", "merge")


class KvlrError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"kvlr status {status}: {msg}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_q_heads", "n_kv_heads", "head_dim", "rank_k", "rank_v", "n_sink", "n_sample",
        "sample_recent_num", "sample_recent_den", "q_window", "top_k", "n_recent",
        "pool_kernel", "local_window", "eig_max_sweeps", "dtype")]


class CacheStruct(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in BUFFERS] + [("L_max", ctypes.c_int64)]


_lib = None


def load():
    """Load libkvlr.so (built by long_context_decode_s4r_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i64, i32, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    cfgp, cachep = ctypes.POINTER(Config), ctypes.POINTER(CacheStruct)
    sig = {
        "kvlr_check_config": (i32, [cfgp]),
        "kvlr_cache_bytes": (i32, [cfgp, i64, i64, ctypes.POINTER(sz)]),
        "kvlr_workspace_bytes": (i32, [cfgp, i32, i64, i64, ctypes.POINTER(sz)]),
        "kvlr_build_bases": (i32, [cfgp, i64, i64, P, P, cachep, P, P, P, P, sz, P]),
        "kvlr_build_bases_shared": (i32, [cfgp, i64, i64, i32, i64, P, P, cachep, P, P, P, P, sz, P]),
        "kvlr_init_window": (i32, [cfgp, i64, i32, P, cachep, P, sz, P]),
        "kvlr_project": (i32, [cfgp, i64, i64, P, P, cachep, P, sz, P]),
        "kvlr_decode_step": (i32, [cfgp, i64, P, P, P, cachep, P, P, P, P, sz, P]),
        "kvlr_decode_step_noalloc": (i32, [cfgp, i64, P, P, P, cachep, P, P, P, P]),
        "kvlr_rank_for_ratio": (i32, [ctypes.c_double, i64, i32, i32, i32, i32, i32, i32,
                                      ctypes.POINTER(i32), ctypes.POINTER(i32)]),
        "kvlr_last_error": (ctypes.c_char_p, []),
        "kvlr_abi_version": (i32, []),
        "kvlr_build_info": (ctypes.c_char_p, []),
        "kvlr_profile_enable": (i32, [i32]),
        "kvlr_profile_read": (i32, [ctypes.POINTER(ctypes.c_float), i32, ctypes.POINTER(i32)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != OK:
        raise KvlrError(status, load().kvlr_last_error().decode())


def make_config(n_q_heads, n_kv_heads, head_dim, rank, n_sink, n_sample, q_window, top_k,
                n_recent, pool_kernel, storage, sample_recent_num=7, sample_recent_den=10,
                rank_v=None, local_window=LOCAL_EXACT, eig_max_sweeps=0) -> Config:
    """rank is the key rank r_K; rank_v defaults to it."""
    return Config(n_q_heads, n_kv_heads, head_dim, rank, rank if rank_v is None else rank_v,
                  n_sink, n_sample, sample_recent_num, sample_recent_den, q_window, top_k,
                  n_recent, pool_kernel, local_window, eig_max_sweeps,
                  {"f32": F32, "bf16": BF16}[storage])


def config_of(w) -> Config:
    """Config of a configs.Workload."""
    return make_config(w.n_q_heads, w.n_kv_heads, w.head_dim, w.rank, w.n_sink, w.n_sample,
                       w.q_window, w.top_k, w.n_recent, w.pool_kernel, w.storage,
                       w.sample_recent_num, w.sample_recent_den, w.rank_v or w.rank,
                       w.local_window, w.eig_max_sweeps)


def rank_for_ratio(eta: float, L: int, d_kv: int, n_sink: int, n_recent: int,
                   k_parts: int = 1, v_parts: int = 1, multiple: int = 8):
    """(r_K, r_V) for a retention target eta (host-side helper of the library)."""
    rk, rv = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(load().kvlr_rank_for_ratio(eta, L, d_kv, n_sink, n_recent, k_parts, v_parts, multiple,
                                      ctypes.byref(rk), ctypes.byref(rv)))
    return rk.value, rv.value


def storage_of(cfg: Config) -> torch.dtype:
    return torch.bfloat16 if cfg.dtype == BF16 else torch.float32


def check_config(cfg: Config) -> None:
    _check(load().kvlr_check_config(ctypes.byref(cfg)))


def cache_bytes(cfg: Config, n_units: int, L_max: int):
    arr = (ctypes.c_size_t * len(BUFFERS))()
    _check(load().kvlr_cache_bytes(ctypes.byref(cfg), n_units, L_max, arr))
    return dict(zip(BUFFERS, list(arr)))


def workspace_bytes(cfg: Config, op: int, n_units: int, L: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load().kvlr_workspace_bytes(ctypes.byref(cfg), op, n_units, L, ctypes.byref(out)))
    return out.value


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None or t.numel() == 0 else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


@dataclass
class KVCache:
    """Caller-owned persistent state of n_units (layer, sequence) units."""
    cfg: Config
    n_units: int
    L_max: int
    sink_k: torch.Tensor
    sink_v: torch.Tensor
    ring_k: torch.Tensor
    ring_v: torch.Tensor
    coef_k: torch.Tensor
    coef_v: torch.Tensor
    basis_k: torch.Tensor
    basis_v: torch.Tensor
    qwin: torch.Tensor
    lens: torch.Tensor
    state: torch.Tensor      # [U][bytes] opaque decode state of the library

    @staticmethod
    def allocate(cfg: Config, n_units: int, L_max: int, device="cuda") -> "KVCache":
        check_config(cfg)
        dt = storage_of(cfg)
        D = cfg.n_kv_heads * cfg.head_dim
        G = cfg.n_q_heads // cfg.n_kv_heads
        U, rk, rv = n_units, cfg.rank_k, cfg.rank_v
        sizes = cache_bytes(cfg, U, L_max)
        z = lambda *shape, dtype=dt: torch.zeros(*shape, dtype=dtype, device=device)
        c = KVCache(cfg, U, L_max,
                    z(U, cfg.n_sink, D), z(U, cfg.n_sink, D),
                    z(U, cfg.n_recent, D), z(U, cfg.n_recent, D),
                    z(U, L_max, rk), z(U, L_max, rv), z(U, D, rk), z(U, D, rv),
                    z(U, cfg.q_window, G, rk, dtype=torch.float32),
                    z(U, 2, dtype=torch.int32),
                    z(U, sizes["state"] // U, dtype=torch.uint8))
        for name in BUFFERS:
            t = getattr(c, name)
            assert t.numel() * t.element_size() == sizes[name], name
        return c

    def units(self, start: int, count: int) -> "KVCache":
        """View of units [start, start + count) sharing storage."""
        sl = slice(start, start + count)
        return KVCache(self.cfg, count, self.L_max,
                       *[getattr(self, n)[sl] for n in BUFFERS])

    def clone(self) -> "KVCache":
        return KVCache(self.cfg, self.n_units, self.L_max,
                       *[getattr(self, n).clone() for n in BUFFERS])

    def struct(self) -> CacheStruct:
        s = CacheStruct()
        for n in BUFFERS:
            t = getattr(self, n)
            assert t.is_contiguous(), n
            setattr(s, n, t.data_ptr() if t.numel() else None)
        s.L_max = self.L_max
        return s


def _check_tensor(t: torch.Tensor, name: str, dtype: torch.dtype, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def build_bases(cache: KVCache, K: torch.Tensor, V: torch.Tensor, eig_k=None, eig_v=None,
                ws: Optional[torch.Tensor] = None, stream=None, sweeps=None,
                check_converged: bool = False) -> None:
    """Enqueue the basis build.  sweeps: optional [U][2] int32 device tensor
    for the eigensolves' sweep counts (-1 = not converged).  check_converged
    (a convenience for callers that can wait) fills such a tensor, waits for
    the stream and raises if any eigensolve did not converge."""
    cfg = cache.cfg
    U, L = K.shape[0], K.shape[1]
    D = cfg.n_kv_heads * cfg.head_dim
    _check_tensor(K, "K", storage_of(cfg), (cache.n_units, L, D))
    _check_tensor(V, "V", storage_of(cfg), (cache.n_units, L, D))
    for name, e in (("eig_k", eig_k), ("eig_v", eig_v)):
        if e is not None:
            _check_tensor(e, name, torch.float32, (U, D))
    if sweeps is not None:
        _check_tensor(sweeps, "sweeps", torch.int32, (U, 2))
    elif check_converged:
        sweeps = torch.empty(U, 2, dtype=torch.int32, device=K.device)
    need = workspace_bytes(cfg, OP_BUILD_BASES, U, L)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=K.device)
    st = cache.struct()
    _check(load().kvlr_build_bases(ctypes.byref(cfg), U, L, _ptr(K), _ptr(V), ctypes.byref(st),
                                   _ptr(eig_k), _ptr(eig_v), _ptr(sweeps), _ptr(ws), ws.numel(),
                                   _stream(stream)))
    if check_converged:
        torch.cuda.current_stream().synchronize() if stream is None else stream.synchronize()
        bad = (sweeps < 0).nonzero().tolist()
        if bad:
            raise KvlrError(EDEVICE, f"eigensolve did not converge within the sweep limit for "
                                     f"(unit, K=0|V=1) {bad}")


def build_bases_shared(cache: KVCache, n_layers: int, depth_window: int, K: torch.Tensor,
                       V: torch.Tensor, eig_k=None, eig_v=None, ws: Optional[torch.Tensor] = None,
                       stream=None, sweeps=None) -> None:
    """Bases shared over windows of depth_window neighbouring layers (units
    layer-major: unit = layer * batch + sequence)."""
    cfg = cache.cfg
    U, L = K.shape[0], K.shape[1]
    if U % n_layers:
        raise ValueError("n_units must be n_layers * batch")
    D = cfg.n_kv_heads * cfg.head_dim
    _check_tensor(K, "K", storage_of(cfg), (cache.n_units, L, D))
    _check_tensor(V, "V", storage_of(cfg), (cache.n_units, L, D))
    for name, e in (("eig_k", eig_k), ("eig_v", eig_v)):
        if e is not None:
            _check_tensor(e, name, torch.float32, (U, D))
    if sweeps is not None:
        _check_tensor(sweeps, "sweeps", torch.int32, (U, 2))
    if ws is None:
        ws = torch.empty(workspace_bytes(cfg, OP_BUILD_BASES, U, L), dtype=torch.uint8, device=K.device)
    st = cache.struct()
    _check(load().kvlr_build_bases_shared(ctypes.byref(cfg), n_layers, U // n_layers, depth_window, L,
                                          _ptr(K), _ptr(V), ctypes.byref(st), _ptr(eig_k), _ptr(eig_v),
                                          _ptr(sweeps), _ptr(ws), ws.numel(), _stream(stream)))


def init_window(cache: KVCache, q_tail: torch.Tensor, ws: Optional[torch.Tensor] = None,
                stream=None) -> None:
    """Seed the query window with the prompt's last queries, q_tail
    [U][n_tail][H_q][d_h] (oldest first); call after project()."""
    cfg = cache.cfg
    U = cache.n_units
    if q_tail.dim() != 4:
        raise ValueError("q_tail must be [U][n_tail][H_q][d_h]")
    n_tail = q_tail.shape[1]
    _check_tensor(q_tail, "q_tail", storage_of(cfg), (U, n_tail, cfg.n_q_heads, cfg.head_dim))
    if ws is None:
        ws = torch.empty(max(workspace_bytes(cfg, OP_INIT_WINDOW, U, cache.L_max), 1),
                         dtype=torch.uint8, device=q_tail.device)
    st = cache.struct()
    _check(load().kvlr_init_window(ctypes.byref(cfg), U, n_tail, _ptr(q_tail), ctypes.byref(st),
                                   _ptr(ws), ws.numel(), _stream(stream)))


def project(cache: KVCache, K: torch.Tensor, V: torch.Tensor, ws: Optional[torch.Tensor] = None,
            stream=None) -> None:
    cfg = cache.cfg
    U, L = K.shape[0], K.shape[1]
    D = cfg.n_kv_heads * cfg.head_dim
    _check_tensor(K, "K", storage_of(cfg), (cache.n_units, L, D))
    _check_tensor(V, "V", storage_of(cfg), (cache.n_units, L, D))
    if ws is None:
        need = workspace_bytes(cfg, OP_PROJECT, U, L)
        ws = torch.empty(need, dtype=torch.uint8, device=K.device) if need > 0 else None
    st = cache.struct()
    _check(load().kvlr_project(ctypes.byref(cfg), U, L, _ptr(K), _ptr(V), ctypes.byref(st), _ptr(ws),
                               0 if ws is None else ws.numel(), _stream(stream)))


def decode_workspace(cache: KVCache) -> torch.Tensor:
    need = workspace_bytes(cache.cfg, OP_DECODE, cache.n_units, cache.L_max)
    return torch.empty(need, dtype=torch.uint8, device=cache.coef_k.device)


def decode_step(cache: KVCache, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                out: torch.Tensor, topk: Optional[torch.Tensor] = None,
                scores: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                stream=None, check: bool = True) -> None:
    cfg = cache.cfg
    U = cache.n_units
    if check:
        dt = storage_of(cfg)
        _check_tensor(q, "q", dt, (U, cfg.n_q_heads, cfg.head_dim))
        _check_tensor(k_new, "k_new", dt, (U, cfg.n_kv_heads, cfg.head_dim))
        _check_tensor(v_new, "v_new", dt, (U, cfg.n_kv_heads, cfg.head_dim))
        _check_tensor(out, "out", torch.float32, (U, cfg.n_q_heads, cfg.head_dim))
        if topk is not None:
            _check_tensor(topk, "topk", torch.int32, (U, cfg.top_k))
        if scores is not None:
            _check_tensor(scores, "scores", torch.float32, (U, cache.L_max))
    if ws is None:
        ws = decode_workspace(cache)
    st = cache.struct()
    _check(load().kvlr_decode_step(ctypes.byref(cfg), U, _ptr(q), _ptr(k_new), _ptr(v_new),
                                   ctypes.byref(st), _ptr(out), _ptr(topk), _ptr(scores), _ptr(ws),
                                   ws.numel(), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 32 << 20  # KVLR_NOALLOC_SCRATCH_BYTES


def decode_step_noalloc(cache: KVCache, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                        out: torch.Tensor, topk: Optional[torch.Tensor] = None,
                        scores: Optional[torch.Tensor] = None, stream=None) -> None:
    """decode_step without a workspace: the library's fixed per-GPU scratch
    is used instead (kvlr_decode_step_noalloc)."""
    cfg = cache.cfg
    U = cache.n_units
    dt = storage_of(cfg)
    _check_tensor(q, "q", dt, (U, cfg.n_q_heads, cfg.head_dim))
    _check_tensor(k_new, "k_new", dt, (U, cfg.n_kv_heads, cfg.head_dim))
    _check_tensor(v_new, "v_new", dt, (U, cfg.n_kv_heads, cfg.head_dim))
    _check_tensor(out, "out", torch.float32, (U, cfg.n_q_heads, cfg.head_dim))
    if topk is not None:
        _check_tensor(topk, "topk", torch.int32, (U, cfg.top_k))
    if scores is not None:
        _check_tensor(scores, "scores", torch.float32, (U, cache.L_max))
    st = cache.struct()
    _check(load().kvlr_decode_step_noalloc(ctypes.byref(cfg), U, _ptr(q), _ptr(k_new), _ptr(v_new),
                                           ctypes.byref(st), _ptr(out), _ptr(topk), _ptr(scores),
                                           _stream(stream)))


def profile_enable(on: bool) -> None:
    _check(load().kvlr_profile_enable(1 if on else 0))


def profile_read():
    ms = (ctypes.c_float * len(STAGES))()
    steps = ctypes.c_int(0)
    _check(load().kvlr_profile_read(ms, len(STAGES), ctypes.byref(steps)))
    return dict(zip(STAGES, list(ms))), steps.value


class Decoder:
    """Repeated decode steps on one cache with the ctypes arguments prepared
    once (no per-call validation beyond the library's own)."""

    def __init__(self, cache: KVCache, out: torch.Tensor, topk: Optional[torch.Tensor] = None,
                 scores: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
        self.cache = cache
        self.lib = load()
        self.cfg = cache.cfg
        self.U = cache.n_units
        self.ws = decode_workspace(cache) if ws is None else ws
        self.out, self.topk, self.scores = out, topk, scores
        self._st = cache.struct()
        self._args_tail = (_ptr(out), _ptr(topk), _ptr(scores), _ptr(self.ws), self.ws.numel())

    def step(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, stream=None):
        st = self.lib.kvlr_decode_step(ctypes.byref(self.cfg), self.U, q.data_ptr(),
                                       k_new.data_ptr(), v_new.data_ptr(), ctypes.byref(self._st),
                                       *self._args_tail, _stream(stream))
        if st != OK:
            _check(st)
