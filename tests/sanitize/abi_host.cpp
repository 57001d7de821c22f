// Host-side checks of libkvlr's C ABI, built together with a host-only copy
// of the library under AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_host_sanitizer.py).  Everything here runs without a GPU: config
// validation, buffer and workspace sizes, the rank helper, and every
// argument check that must fail before a device is touched.  Any sanitizer
// report aborts the process; a failed expectation exits with status 1.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "kvlr.h"
#include "kvlr_probe.h"

static int g_fail = 0;

#define EXPECT(cond)                                                      \
  do {                                                                    \
    if (!(cond)) {                                                        \
      std::fprintf(stderr, "%s:%d: expected %s (last error: %s)\n",       \
                   __FILE__, __LINE__, #cond, kvlr_last_error());         \
      ++g_fail;                                                           \
    }                                                                     \
  } while (0)

static kvlr_config llama_layer() {
  kvlr_config c{};
  c.n_q_heads = 32;
  c.n_kv_heads = 8;
  c.head_dim = 128;
  c.rank_k = 256;
  c.rank_v = 256;
  c.n_sink = 4;
  c.n_sample = 2048;
  c.sample_recent_num = 7;
  c.sample_recent_den = 10;
  c.q_window = 16;
  c.top_k = 512;
  c.n_recent = 64;
  c.pool_kernel = 7;
  c.local_window = KVLR_LOCAL_EXACT;
  c.eig_max_sweeps = 0;
  c.dtype = KVLR_BF16;
  return c;
}

static kvlr_config qwen_layer() {
  kvlr_config c = llama_layer();
  c.n_q_heads = 28;
  c.n_kv_heads = 4;
  c.rank_k = 128;
  c.rank_v = 192;
  c.q_window = 32;
  return c;
}

static kvlr_config tiny_f32() {
  kvlr_config c = llama_layer();
  c.n_q_heads = 4;
  c.n_kv_heads = 2;
  c.head_dim = 32;
  c.rank_k = 16;
  c.rank_v = 24;
  c.n_sample = 64;
  c.q_window = 4;
  c.top_k = 24;
  c.n_recent = 8;
  c.dtype = KVLR_F32;
  return c;
}

static void check_configs() {
  const kvlr_config good[] = {llama_layer(), qwen_layer(), tiny_f32()};
  for (const auto& c : good) EXPECT(kvlr_check_config(&c) == KVLR_OK);
  EXPECT(kvlr_check_config(nullptr) == KVLR_EINVAL);
  EXPECT(std::strlen(kvlr_last_error()) > 0);

  // one bad field at a time
  struct Bad {
    int32_t kvlr_config::*field;
    int32_t value;
  };
  const Bad bad[] = {
      {&kvlr_config::n_q_heads, 30},     {&kvlr_config::n_kv_heads, 0},
      {&kvlr_config::head_dim, 44},      {&kvlr_config::rank_k, 100},
      {&kvlr_config::rank_k, 2048},      {&kvlr_config::rank_v, -1},
      {&kvlr_config::n_sink, -1},        {&kvlr_config::n_sample, 0},
      {&kvlr_config::sample_recent_num, 11}, {&kvlr_config::sample_recent_den, 0},
      {&kvlr_config::q_window, 0},       {&kvlr_config::q_window, 64},
      {&kvlr_config::top_k, -1},         {&kvlr_config::n_recent, 0},
      {&kvlr_config::pool_kernel, 4},    {&kvlr_config::local_window, 5},
      {&kvlr_config::eig_max_sweeps, -1}, {&kvlr_config::dtype, 7},
  };
  for (const auto& b : bad) {
    kvlr_config c = llama_layer();
    c.*(b.field) = b.value;
    EXPECT(kvlr_check_config(&c) == KVLR_EINVAL);
    EXPECT(std::strlen(kvlr_last_error()) > 0);
  }
}

static void check_sizes() {
  const kvlr_config c = llama_layer();
  size_t b[KVLR_BUF_COUNT];
  EXPECT(kvlr_cache_bytes(&c, 16, 34000, b) == KVLR_OK);
  EXPECT(b[KVLR_BUF_COEF_K] == (size_t)16 * 34000 * 256 * 2);
  EXPECT(b[KVLR_BUF_BASIS_V] == (size_t)16 * 1024 * 256 * 2);
  EXPECT(b[KVLR_BUF_LENS] == (size_t)16 * 2 * 4);
  EXPECT(kvlr_cache_bytes(&c, 0, 34000, b) == KVLR_EINVAL);
  EXPECT(kvlr_cache_bytes(&c, 16, -5, b) == KVLR_EINVAL);
  EXPECT(kvlr_cache_bytes(&c, 16, 34000, nullptr) == KVLR_EINVAL);
  EXPECT(kvlr_cache_bytes(nullptr, 16, 34000, b) == KVLR_EINVAL);

  const kvlr_config q = qwen_layer();
  EXPECT(kvlr_cache_bytes(&q, 8, 70000, b) == KVLR_OK);
  EXPECT(b[KVLR_BUF_COEF_V] == (size_t)8 * 70000 * 192 * 2);

  for (int op = KVLR_OP_BUILD_BASES; op <= KVLR_OP_INIT_WINDOW; ++op) {
    size_t ws = 0;
    EXPECT(kvlr_workspace_bytes(&c, op, 16, 34000, &ws) == KVLR_OK);
    EXPECT(op == KVLR_OP_PROJECT || ws > 0);
  }
  size_t ws = 0;
  EXPECT(kvlr_workspace_bytes(&c, 9, 16, 34000, &ws) == KVLR_EINVAL);
  EXPECT(kvlr_workspace_bytes(&c, KVLR_OP_DECODE, 16, 34000, nullptr) == KVLR_EINVAL);
}

static void check_rank_helper() {
  int32_t rk = -1, rv = -1;
  EXPECT(kvlr_rank_for_ratio(0.2, 32768, 1024, 4, 64, 1, 1, 32, &rk, &rv) == KVLR_OK);
  EXPECT(rk > 0 && rk == rv && rk % 32 == 0);
  EXPECT(kvlr_rank_for_ratio(0.25, 131072, 1024, 4, 64, 2, 3, 32, &rk, &rv) == KVLR_OK);
  EXPECT(rk > 0 && rk * 3 == rv * 2);
  EXPECT(kvlr_rank_for_ratio(1e-6, 100, 64, 4, 16, 1, 1, 8, &rk, &rv) == KVLR_OK);
  EXPECT(rk == 0 && rv == 0);
  EXPECT(kvlr_rank_for_ratio(0.0, 1000, 64, 4, 16, 1, 1, 8, &rk, &rv) == KVLR_EINVAL);
  EXPECT(kvlr_rank_for_ratio(0.2, 1000, 64, 4, 16, 0, 1, 8, &rk, &rv) == KVLR_EINVAL);
  EXPECT(kvlr_rank_for_ratio(0.2, 1000, 64, 4, 16, 1, 1, 8, nullptr, &rv) == KVLR_EINVAL);
  // a sweep over targets: ranks grow with eta and stay within D'
  int32_t last = 0;
  for (int i = 1; i <= 100; ++i) {
    EXPECT(kvlr_rank_for_ratio(0.01 * i, 65536, 512, 4, 64, 1, 1, 16, &rk, &rv) == KVLR_OK);
    EXPECT(rk >= last && rk <= 512);
    last = rk;
  }
}

static void check_call_arguments() {
  // dummy, never dereferenced: every call below must fail on its arguments
  void* const p = reinterpret_cast<void*>(4096);
  kvlr_config c = llama_layer();
  kvlr_cache cache{};
  EXPECT(kvlr_build_bases(&c, 1, 32768, nullptr, nullptr, &cache, nullptr, nullptr, nullptr,
                          nullptr, 0, nullptr) == KVLR_EINVAL);
  EXPECT(kvlr_build_bases(&c, 1, 100, p, p, &cache, nullptr, nullptr, nullptr, nullptr, 0,
                          nullptr) == KVLR_EINVAL);
  EXPECT(std::strstr(kvlr_last_error(), "does not fit") != nullptr);
  EXPECT(kvlr_build_bases_shared(&c, 4, 2, 0, 32768, p, p, &cache, nullptr, nullptr, nullptr,
                                 nullptr, 0, nullptr) == KVLR_EINVAL);
  EXPECT(kvlr_project(&c, 1, 10, p, p, &cache, nullptr, 0, nullptr) == KVLR_EINVAL);
  EXPECT(kvlr_decode_step(&c, 1, p, p, p, &cache, (float*)p, nullptr, nullptr, nullptr, 0,
                          nullptr) == KVLR_EINVAL);
  EXPECT(kvlr_init_window(&c, 1, 0, p, &cache, nullptr, 0, nullptr) == KVLR_EINVAL);

  // every cache buffer set (to the dummy): workspace and capacity checks
  cache.sink_k = cache.sink_v = cache.ring_k = cache.ring_v = p;
  cache.coef_k = cache.coef_v = cache.basis_k = cache.basis_v = p;
  cache.qwin = (float*)p;
  cache.lens = (int32_t*)p;
  cache.state = p;
  cache.L_max = 40000;
  EXPECT(kvlr_decode_step(&c, 1, p, p, p, &cache, (float*)p, nullptr, nullptr, p, 100,
                          nullptr) == KVLR_EWORKSPACE);
  EXPECT(std::strstr(kvlr_last_error(), "workspace") != nullptr);
  EXPECT(kvlr_project(&c, 1, 50000, p, p, &cache, nullptr, 0, nullptr) == KVLR_EINVAL);
  EXPECT(std::strstr(kvlr_last_error(), "L_max") != nullptr);
  EXPECT(kvlr_init_window(&c, 1, 17, p, &cache, p, 1 << 20, nullptr) == KVLR_EINVAL);

  // the allocation-free step: too large for the fixed scratch
  cache.L_max = 1 << 24;
  EXPECT(kvlr_decode_step_noalloc(&c, 64, p, p, p, &cache, (float*)p, nullptr, nullptr,
                                  nullptr) == KVLR_EWORKSPACE);
  EXPECT(kvlr_decode_step_noalloc(nullptr, 1, p, p, p, &cache, (float*)p, nullptr, nullptr,
                                  nullptr) == KVLR_EINVAL);

  // probes and profiling
  EXPECT(kvlr_probe_read(nullptr, 1 << 20, 0, 256, 2, (uint32_t*)p, nullptr) != 0);
  EXPECT(kvlr_probe_read(p, 1000, 0, 256, 2, (uint32_t*)p, nullptr) != 0);
  EXPECT(kvlr_probe_read(p, 1 << 20, 0, 256, 3, (uint32_t*)p, nullptr) != 0);
  EXPECT(kvlr_probe_mfma(5, 10, 1, (float*)p, nullptr) != 0);
  EXPECT(kvlr_profile_read(nullptr, 5, nullptr) == KVLR_EINVAL);
  float ms[6];
  int steps = 0;
  EXPECT(kvlr_profile_read(ms, 9, &steps) == KVLR_EINVAL);
}

int main() {
  EXPECT(kvlr_abi_version() == KVLR_ABI_VERSION);
  EXPECT(std::strstr(kvlr_build_info(), "gfx950") != nullptr);
  check_configs();
  check_sizes();
  check_rank_helper();
  check_call_arguments();
  if (g_fail) {
    std::fprintf(stderr, "%d host ABI expectation(s) failed\n", g_fail);
    return 1;
  }
  std::printf("host ABI checks passed\n");
  return 0;
}
