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


def header_functions(header="kvlr.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvlr_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert lib.kvlr_abi_version() == 2
    probes = header_functions("kvlr_probe.h")
    assert probes == ["kvlr_probe_mfma", "kvlr_probe_read"]
    for n in probes:
        assert hasattr(lib, n), n
    assert b"gfx950" in lib.kvlr_build_info()


def header_struct_fields(name):
    """Field names of a struct in include/kvlr.h, in order."""
    src = open(os.path.join(ROOT, "include", "kvlr.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    body = re.search(r"typedef struct %s \{(.*?)\}" % name, src, flags=re.S).group(1)
    return re.findall(r"\b(\w+)\s*;", body)


def test_struct_layout_matches_header():
    assert [n for n, _ in kvlr.Config._fields_] == header_struct_fields("kvlr_config")
    assert [n for n, _ in kvlr.CacheStruct._fields_] == header_struct_fields("kvlr_cache")
    assert ctypes.sizeof(kvlr.Config) == 16 * 4
    assert ctypes.sizeof(kvlr.CacheStruct) == 11 * 8 + 8


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


def test_enum_fields_and_dtype(lib):
    c = _cfg()
    c.local_window = 5
    assert lib.kvlr_check_config(ctypes.byref(c)) == kvlr.EINVAL
    c = _cfg()
    c.eig_max_sweeps = -1
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
    # opaque decode state: at least the scorer's bf16 window copy and the row statistics
    assert b["state"] >= 16 * (16 * 4 * 2 * 256 * 2 + 16 * 4 * 2 * 4) and b["state"] % (16 * 256) == 0
    assert b["lens"] == 16 * 2 * 4
    assert b["sink_k"] == 16 * 4 * 1024 * 2 and b["ring_v"] == 16 * 64 * 1024 * 2
    ws = kvlr.workspace_bytes(cfg, kvlr.OP_DECODE, 16, 34000)
    assert ws > 16 * 34000 * (4 + 4 * 4)
    wb = kvlr.workspace_bytes(cfg, kvlr.OP_BUILD_BASES, 16, 32768)
    assert wb > 4 * 32 * 1024 * 1024 * 8
    # projection: the two bases of every unit, transposed, in bf16
    # the value basis transposed (the key basis transposed lives in the state)
    assert kvlr.workspace_bytes(cfg, kvlr.OP_PROJECT, 16, 32768) == 16 * 256 * 1024 * 2
    with pytest.raises(kvlr.KvlrError):
        kvlr.workspace_bytes(cfg, 9, 16, 100)


def test_calls_reject_bad_arguments_without_device(lib):
    cfg = _cfg()
    cache = kvlr.CacheStruct()
    # null inputs
    st = lib.kvlr_build_bases(ctypes.byref(cfg), 1, 32768, None, None, ctypes.byref(cache),
                              None, None, None, None, 0, None)
    assert st == kvlr.EINVAL
    # sample does not fit (needs 2048 rows in 100 tokens)
    st = lib.kvlr_build_bases(ctypes.byref(cfg), 1, 100, ctypes.c_void_p(16), ctypes.c_void_p(16),
                              ctypes.byref(cache), None, None, None, None, 0, None)
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


def test_calls_reject_device_pointers_off_16_byte_boundaries(lib):
    # the kernels move rows in 16-byte pieces; every case is refused before any launch
    cfg = _cfg()
    cache = kvlr.CacheStruct()
    for name in kvlr.BUFFERS:
        setattr(cache, name, 4096)
    cache.L_max = 40000
    big = 1 << 40
    v = ctypes.c_void_p

    def decode(q=16, out=16, ws=16):
        return lib.kvlr_decode_step(ctypes.byref(cfg), 1, v(q), v(16), v(16), ctypes.byref(cache), v(out),
                                    None, None, v(ws), big, None)
    for st in (decode(q=24), decode(out=8), decode(ws=20)):
        assert st == kvlr.EINVAL and b"16-byte" in lib.kvlr_last_error()
    cache.coef_k = 4104
    assert decode() == kvlr.EINVAL and b"16-byte" in lib.kvlr_last_error()
    cache.coef_k = 4096
    st = lib.kvlr_project(ctypes.byref(cfg), 1, 30000, v(8), v(16), ctypes.byref(cache), None, 0, None)
    assert st == kvlr.EINVAL and b"16-byte" in lib.kvlr_last_error()
    st = lib.kvlr_build_bases(ctypes.byref(cfg), 1, 32768, v(16), v(18), ctypes.byref(cache),
                              None, None, None, v(16), big, None)
    assert st == kvlr.EINVAL and b"16-byte" in lib.kvlr_last_error()


def test_profile_read_bad_args(lib):
    assert lib.kvlr_profile_read(None, 5, None) == kvlr.EINVAL


@pytest.mark.parametrize("eta,L,D,s,n_rec,parts", [
    (0.2, 32768, 1024, 4, 64, (1, 1)), (0.3, 65536, 512, 4, 64, (1, 1)),
    (0.25, 131072, 1024, 4, 64, (2, 3)), (0.05, 4096, 1024, 4, 64, (1, 1)),
    (0.5, 1024, 64, 4, 16, (1, 1)), (0.01, 100, 64, 4, 16, (1, 1))])
def test_rank_for_ratio_matches_oracle(lib, eta, L, D, s, n_rec, parts):
    """The library's host helper against the oracle's accounting."""
    from oracle import s4r
    assert kvlr.rank_for_ratio(eta, L, D, s, n_rec, *parts) == s4r.rank_for_ratio(
        eta, L, D, s, n_rec, parts)


def test_rank_for_ratio_rejects(lib):
    with pytest.raises(kvlr.KvlrError):
        kvlr.rank_for_ratio(0.0, 1000, 64, 4, 16)
    with pytest.raises(kvlr.KvlrError):
        kvlr.rank_for_ratio(0.2, 1000, 64, 4, 16, 0, 1)


def test_probe_argument_errors(lib):
    """Probe calls reject bad arguments before any launch."""
    lib.kvlr_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.kvlr_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p]
    assert lib.kvlr_probe_read(None, 1 << 20, 0, 256, 4, 16, None) == 1
    assert lib.kvlr_probe_read(16, 1000, 0, 256, 4, 16, None) == 1       # not a multiple of 16 KiB
    assert lib.kvlr_probe_read(16, 1 << 20, 0, 256, 3, 16, None) == 1    # unsupported depth
    assert lib.kvlr_probe_read(16, 1 << 20, 5, 256, 4, 16, None) == 1    # unknown method
    assert lib.kvlr_probe_read(16, 1 << 20, 3, 256, 96, 16, None) == 1   # row slabs: unsupported width
    assert lib.kvlr_probe_read(16, 1 << 19, 4, 256, 64, 16, None) == 1   # row slabs: not whole 1 MiB tiles
    assert lib.kvlr_probe_read(16, 1 << 14, 2, 256, 4, 16, None) == 1    # LDS paths: whole 32 KiB stages
    assert lib.kvlr_probe_mfma(2, 10, 256, 16, None) == 1
    assert lib.kvlr_probe_mfma(0, 0, 256, 16, None) == 1
