"""Host-only checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching a device."""
import ctypes
import os
import re

import pytest

from long_context_decode_s4r_amd import configs, kvlr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kvlr.LIB_PATH):
        pytest.skip("libkvlr.so not built")
    return kvlr.load()


def header_functions():
    src = open(os.path.join(ROOT, "include", "kvlr.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvlr_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert lib.kvlr_abi_version() == 1
    assert b"gfx950" in lib.kvlr_build_info()


def test_struct_layout_matches_header():
    assert ctypes.sizeof(kvlr.Config) == 14 * 4
    assert ctypes.sizeof(kvlr.CacheStruct) == 12 * 8 + 8


@pytest.mark.parametrize("w", configs.ALL, ids=lambda w: w.name)
def test_workload_configs_valid(lib, w):
    kvlr.check_config(kvlr.config_of(w))


def _cfg(**kw):
    base = dict(n_q_heads=32, n_kv_heads=8, head_dim=128, rank=256, n_sink=4, n_sample=2048,
                q_window=16, top_k=512, n_recent=64, pool_kernel=7, storage="bf16")
    base.update(kw)
    return kvlr.make_config(**base)


@pytest.mark.parametrize("kw,msg", [
    (dict(n_q_heads=30), "multiple"),
    (dict(n_q_heads=80, n_kv_heads=8), "G = 10"),
    (dict(rank=100), "rank"),
    (dict(rank=2048), "rank"),
    (dict(pool_kernel=4), "odd"),
    (dict(n_recent=0), "n_recent"),
    (dict(top_k=-1), "top_k"),
    (dict(head_dim=44), "head_dim"),
    (dict(q_window=64), "q_window"),
    (dict(n_sample=0), "n_sample"),
    (dict(storage="f32", rank=256, q_window=16), "8192"),
])
def test_config_rejected(lib, kw, msg):
    with pytest.raises(kvlr.KvlrError) as e:
        kvlr.check_config(_cfg(**kw))
    assert e.value.status == kvlr.EINVAL and msg in str(e.value)


def test_reserved_and_dtype(lib):
    c = _cfg()
    c.reserved = 1
    assert lib.kvlr_check_config(ctypes.byref(c)) == kvlr.EINVAL
    c = _cfg()
    c.dtype = 7
    assert lib.kvlr_check_config(ctypes.byref(c)) == kvlr.EINVAL
    assert lib.kvlr_check_config(None) == kvlr.EINVAL


def test_cache_and_workspace_sizes(lib):
    w = configs.LLAMA8B_32K
    cfg = kvlr.config_of(w)
    b = kvlr.cache_bytes(cfg, 16, 34000)
    assert b["coef_k"] == 16 * 34000 * 256 * 2
    assert b["basis_v"] == 16 * 1024 * 256 * 2
    assert b["qwin"] == 16 * 16 * 4 * 256 * 4
    assert b["rowstat"] == 16 * 16 * 4 * 2 * 4
    assert b["lens"] == 16 * 2 * 4
    assert b["sink_k"] == 16 * 4 * 1024 * 2 and b["ring_v"] == 16 * 64 * 1024 * 2
    ws = kvlr.workspace_bytes(cfg, kvlr.OP_DECODE, 16, 34000)
    assert ws > 16 * 34000 * (4 + 4 * 4)
    wb = kvlr.workspace_bytes(cfg, kvlr.OP_BUILD_BASES, 16, 32768)
    assert wb > 4 * 32 * 1024 * 1024 * 8
    # projection: the two bases of every unit, transposed, in bf16
    assert kvlr.workspace_bytes(cfg, kvlr.OP_PROJECT, 16, 32768) == 16 * 2 * 256 * 1024 * 2
    with pytest.raises(kvlr.KvlrError):
        kvlr.workspace_bytes(cfg, 9, 16, 100)


def test_calls_reject_bad_arguments_without_device(lib):
    cfg = _cfg()
    cache = kvlr.CacheStruct()
    # null inputs
    st = lib.kvlr_build_bases(ctypes.byref(cfg), 1, 32768, None, None, ctypes.byref(cache),
                              None, None, None, 0, None)
    assert st == kvlr.EINVAL
    # sample does not fit (needs 2048 rows in 100 tokens)
    st = lib.kvlr_build_bases(ctypes.byref(cfg), 1, 100, ctypes.c_void_p(16), ctypes.c_void_p(16),
                              ctypes.byref(cache), None, None, None, 0, None)
    assert st == kvlr.EINVAL and b"does not fit" in lib.kvlr_last_error()
    # prompt shorter than sinks + recent window
    st = lib.kvlr_project(ctypes.byref(cfg), 1, 10, ctypes.c_void_p(16), ctypes.c_void_p(16),
                          ctypes.byref(cache), None, 0, None)
    assert st == kvlr.EINVAL
    # decode: null cache buffers
    st = lib.kvlr_decode_step(ctypes.byref(cfg), 1, ctypes.c_void_p(16), ctypes.c_void_p(16),
                              ctypes.c_void_p(16), ctypes.byref(cache), ctypes.c_void_p(16), None,
                              None, None, 0, None)
    assert st == kvlr.EINVAL
    # decode: workspace too small (all cache pointers set to a dummy non-null value)
    for name in kvlr.BUFFERS:
        setattr(cache, name, 4096)
    cache.L_max = 40000
    st = lib.kvlr_decode_step(ctypes.byref(cfg), 1, ctypes.c_void_p(16), ctypes.c_void_p(16),
                              ctypes.c_void_p(16), ctypes.byref(cache), ctypes.c_void_p(16), None,
                              None, ctypes.c_void_p(16), 100, None)
    assert st == kvlr.EWORKSPACE and b"workspace" in lib.kvlr_last_error()
    # project: prompt longer than the cache
    st = lib.kvlr_project(ctypes.byref(cfg), 1, 50000, ctypes.c_void_p(16), ctypes.c_void_p(16),
                          ctypes.byref(cache), None, 0, None)
    assert st == kvlr.EINVAL and b"L_max" in lib.kvlr_last_error()


def test_profile_read_bad_args(lib):
    assert lib.kvlr_profile_read(None, 5, None) == kvlr.EINVAL
