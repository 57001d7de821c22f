// C ABI of the kvlr library: argument validation, workspace carving and the
// launch sequence of each call.  Every function validates its arguments and
// returns KVLR_EINVAL before touching the device.
#include "../../include/kvlr.h"
#include "common.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

using namespace kvlr;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return KVLR_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(KVLR_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

size_t elem_bytes(const kvlr_config* c) { return c->dtype == KVLR_BF16 ? 2 : 4; }

bool rank_supported_bf16(int r) { return r == 32 || r == 64 || r == 128 || r == 192 || r == 256; }

Dims dims_of(const kvlr_config* c) {
  Dims d;
  d.Hq = c->n_q_heads;
  d.Hkv = c->n_kv_heads;
  d.dh = c->head_dim;
  d.D = c->n_kv_heads * c->head_dim;
  d.r = c->rank;
  d.G = c->n_q_heads / c->n_kv_heads;
  d.s = c->n_sink;
  d.T = c->n_sample;
  d.rnum = c->sample_recent_num;
  d.rden = c->sample_recent_den;
  d.W = c->q_window;
  d.k = c->top_k;
  d.nrec = c->n_recent;
  d.kappa = c->pool_kernel;
  d.dtype = c->dtype;
  return d;
}

int check_cfg(const kvlr_config* c) {
  if (!c) return fail(KVLR_EINVAL, "config is NULL");
  if (c->reserved != 0) return fail(KVLR_EINVAL, "config.reserved must be 0");
  if (c->dtype != KVLR_F32 && c->dtype != KVLR_BF16) return fail(KVLR_EINVAL, "unknown dtype %d", c->dtype);
  if (c->n_q_heads < 1 || c->n_kv_heads < 1 || c->head_dim < 1)
    return fail(KVLR_EINVAL, "head counts and head_dim must be >= 1");
  if (c->n_q_heads % c->n_kv_heads != 0)
    return fail(KVLR_EINVAL, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", c->n_q_heads, c->n_kv_heads);
  const int G = c->n_q_heads / c->n_kv_heads;
  if (G > 8) return fail(KVLR_EINVAL, "query heads per KV head G = %d > 8 is not supported", G);
  if (c->head_dim > 256) return fail(KVLR_EINVAL, "head_dim %d > 256 is not supported", c->head_dim);
  const int64_t D = (int64_t)c->n_kv_heads * c->head_dim;
  if (D % 2 != 0 || D > 4096) return fail(KVLR_EINVAL, "D' = %lld must be even and <= 4096", (long long)D);
  if ((1 + G) * D > 12288) return fail(KVLR_EINVAL, "(1 + G) * D' = %lld exceeds 12288", (long long)((1 + G) * D));
  if ((int64_t)G * c->head_dim > 1024) return fail(KVLR_EINVAL, "G * head_dim must be <= 1024");
  if (c->rank < 1 || c->rank > D) return fail(KVLR_EINVAL, "rank %d must be in [1, D' = %lld]", c->rank, (long long)D);
  if (c->rank % 8 != 0) return fail(KVLR_EINVAL, "rank %d must be a multiple of 8", c->rank);
  if (c->head_dim % 8 != 0) return fail(KVLR_EINVAL, "head_dim %d must be a multiple of 8", c->head_dim);
  if (c->n_sink < 0) return fail(KVLR_EINVAL, "n_sink must be >= 0");
  if (c->n_sample < 1) return fail(KVLR_EINVAL, "n_sample must be >= 1");
  if (c->sample_recent_den < 1 || c->sample_recent_num < 0 || c->sample_recent_num > c->sample_recent_den)
    return fail(KVLR_EINVAL, "sample recent share must be num/den with 0 <= num <= den, den >= 1");
  if (c->q_window < 1) return fail(KVLR_EINVAL, "q_window must be >= 1");
  if (c->top_k < 0) return fail(KVLR_EINVAL, "top_k must be >= 0");
  if (c->n_recent < 1) return fail(KVLR_EINVAL, "n_recent must be >= 1 (the new token is held exactly)");
  if (c->pool_kernel < 1 || c->pool_kernel % 2 == 0 || c->pool_kernel > 255)
    return fail(KVLR_EINVAL, "pool_kernel must be odd and in [1, 255]");
  if (c->dtype == KVLR_BF16) {
    if (!rank_supported_bf16(c->rank)) return fail(KVLR_EINVAL, "bf16 storage needs rank in {32, 64, 128, 192, 256}");
    if (c->q_window * G > 128) return fail(KVLR_EINVAL, "bf16 storage needs q_window * G <= 128");
  } else {
    if ((int64_t)c->q_window * G * c->rank > 8192)
      return fail(KVLR_EINVAL, "fp32 storage needs q_window * G * rank <= 8192");
  }
  if (attend_lds_bytes(dims_of(c)) == 0)
    return fail(KVLR_EINVAL, "rank / head shape too large for the attention tile (160 KB LDS)");
  return KVLR_OK;
}


int check_sample_fits(const kvlr_config* c, int64_t L) {
  if (L < (int64_t)c->n_sink + c->n_recent)
    return fail(KVLR_EINVAL, "prompt length %lld < n_sink + n_recent", (long long)L);
  const int64_t n_r = ((int64_t)c->sample_recent_num * c->n_sample) / c->sample_recent_den;
  const int64_t n_u = c->n_sample - n_r;
  if (n_r > L - c->n_sink || L - n_r - c->n_sink < n_u)
    return fail(KVLR_EINVAL, "sample of %d rows does not fit in %lld non-sink tokens", c->n_sample,
                (long long)(L - c->n_sink));
  return KVLR_OK;
}

// ---- workspace layouts ------------------------------------------------------
struct BuildLayout {
  size_t S, A0, A1, V0, V1, part, frozen, final_buf, counter, total;
  int nchunk;
};

BuildLayout build_layout(const kvlr_config* c, int64_t U) {
  BuildLayout b;
  const int64_t D = (int64_t)c->n_kv_heads * c->head_dim;
  const int64_t nmat = 2 * U;
  b.nchunk = (int)((D + 15) / 16);
  size_t off = 0;
  b.S = off;
  off = align_up(off + (size_t)nmat * c->n_sample * D * elem_bytes(c));
  const size_t mat = (size_t)nmat * D * D * sizeof(double);
  b.A0 = off;
  off = align_up(off + mat);
  b.A1 = off;
  off = align_up(off + mat);
  b.V0 = off;
  off = align_up(off + mat);
  b.V1 = off;
  off = align_up(off + mat);
  b.part = off;
  off = align_up(off + (size_t)nmat * b.nchunk * 2 * sizeof(double));
  b.frozen = off;
  off = align_up(off + (size_t)nmat * sizeof(int));
  b.final_buf = off;
  off = align_up(off + (size_t)nmat * sizeof(int));
  b.counter = off;
  off = align_up(off + sizeof(int));
  b.total = off;
  return b;
}

struct DecodeLayout {
  size_t stepinfo, partial, spill, tilestat, keys, topk, qlat, ylat, yex, astat, gmax, cslot,
      tkpcnt, tkhint, total;
  DecodeWs t;  // tiling fields
};

DecodeLayout decode_layout(const kvlr_config* c, int64_t U, int64_t Lmax) {
  DecodeLayout L;
  Dims d = dims_of(c);
  decode_tiling(d, U, Lmax, &L.t);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.stepinfo = take((size_t)U * 4 * sizeof(int32_t));
  L.partial = take((size_t)U * L.t.Lc_cap * sizeof(float));
  L.spill = take((size_t)U * d.G * L.t.Lc_cap * sizeof(float));
  L.tilestat = take((size_t)U * L.t.nsplit * d.G * 2 * sizeof(float));
  L.keys = take((size_t)U * L.t.Lc_cap * sizeof(uint32_t));
  L.topk = take((size_t)U * (c->top_k > 0 ? c->top_k : 1) * sizeof(int32_t));
  L.qlat = take((size_t)U * d.Hq * d.r * sizeof(float));
  L.ylat = take((size_t)U * (L.t.nsl > 0 ? L.t.nsl : 1) * d.Hq * d.r * sizeof(float));
  L.yex = take((size_t)U * L.t.nse * d.Hq * d.dh * sizeof(float));
  L.astat = take((size_t)U * (L.t.nsl + L.t.nse) * d.Hq * 2 * sizeof(float));
  L.gmax = take((size_t)U * (L.t.Lc_cap / 8) * sizeof(uint32_t));
  L.cslot = take((size_t)U * L.t.Lc_cap * 8);
  L.tkpcnt = take((size_t)U * L.t.tk_nbp * sizeof(int));
  L.tkhint = take((size_t)U * sizeof(uint32_t));
  L.total = off;
  return L;
}

int check_cache(const kvlr_cache* cache, bool need_state, int n_sink) {
  if (!cache) return fail(KVLR_EINVAL, "cache is NULL");
  if (!cache->basis_k || !cache->basis_v) return fail(KVLR_EINVAL, "cache bases are NULL");
  if (need_state) {
    if (n_sink > 0 && (!cache->sink_k || !cache->sink_v))
      return fail(KVLR_EINVAL, "sink buffers are NULL");
    if (!cache->ring_k || !cache->ring_v || !cache->coef_k ||
        !cache->coef_v || !cache->qwin || !cache->rowstat || !cache->lens || !cache->qsplit)
      return fail(KVLR_EINVAL, "a cache buffer is NULL");
    if (cache->L_max < 1) return fail(KVLR_EINVAL, "cache L_max must be >= 1");
  }
  return KVLR_OK;
}

CachePtrs cache_ptrs(const kvlr_cache* c) {
  CachePtrs p;
  p.sink_k = c->sink_k;
  p.sink_v = c->sink_v;
  p.ring_k = c->ring_k;
  p.ring_v = c->ring_v;
  p.coef_k = c->coef_k;
  p.coef_v = c->coef_v;
  p.basis_k = c->basis_k;
  p.basis_v = c->basis_v;
  p.qwin = c->qwin;
  p.qsplit = (uint16_t*)c->qsplit;
  p.rowstat = c->rowstat;
  p.lens = c->lens;
  p.Lmax = c->L_max;
  return p;
}

// ---- stage timing -------------------------------------------------------------
constexpr int kStages = 6;
constexpr int kMaxProfiled = 8192;
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<hipEvent_t> g_prof_events;  // kMaxProfiled * (kStages + 1)
int g_prof_steps = 0;

}  // namespace

extern "C" {

int kvlr_check_config(const kvlr_config* cfg) {
  const int e = check_cfg(cfg);
  return e == KVLR_OK ? ok() : e;
}

int kvlr_cache_bytes(const kvlr_config* cfg, int64_t n_units, int64_t L_max, size_t* bytes) {
  int e = check_cfg(cfg);
  if (e) return e;
  if (!bytes) return fail(KVLR_EINVAL, "bytes is NULL");
  if (n_units < 1 || L_max < 1) return fail(KVLR_EINVAL, "n_units and L_max must be >= 1");
  const size_t eb = elem_bytes(cfg);
  const int64_t D = (int64_t)cfg->n_kv_heads * cfg->head_dim;
  const int64_t G = cfg->n_q_heads / cfg->n_kv_heads;
  bytes[KVLR_BUF_SINK_K] = bytes[KVLR_BUF_SINK_V] = (size_t)n_units * cfg->n_sink * D * eb;
  bytes[KVLR_BUF_RING_K] = bytes[KVLR_BUF_RING_V] = (size_t)n_units * cfg->n_recent * D * eb;
  bytes[KVLR_BUF_COEF_K] = bytes[KVLR_BUF_COEF_V] = (size_t)n_units * L_max * cfg->rank * eb;
  bytes[KVLR_BUF_BASIS_K] = bytes[KVLR_BUF_BASIS_V] = (size_t)n_units * D * cfg->rank * eb;
  bytes[KVLR_BUF_QWIN] = (size_t)n_units * cfg->q_window * G * cfg->rank * sizeof(float);
  bytes[KVLR_BUF_ROWSTAT] = (size_t)n_units * cfg->q_window * G * 2 * sizeof(float);
  bytes[KVLR_BUF_LENS] = (size_t)n_units * 2 * sizeof(int32_t);
  bytes[KVLR_BUF_QSPLIT] = (size_t)n_units * cfg->q_window * G * 2 * cfg->rank * sizeof(uint16_t);
  return ok();
}

int kvlr_workspace_bytes(const kvlr_config* cfg, int op, int64_t n_units, int64_t L, size_t* bytes) {
  int e = check_cfg(cfg);
  if (e) return e;
  if (!bytes) return fail(KVLR_EINVAL, "bytes is NULL");
  if (n_units < 1 || L < 1) return fail(KVLR_EINVAL, "n_units and L must be >= 1");
  switch (op) {
    case KVLR_OP_BUILD_BASES: *bytes = build_layout(cfg, n_units).total; break;
    case KVLR_OP_PROJECT: *bytes = project_ws_bytes(dims_of(cfg), n_units); break;
    case KVLR_OP_DECODE: *bytes = decode_layout(cfg, n_units, L).total; break;
    default: return fail(KVLR_EINVAL, "unknown op %d", op);
  }
  return ok();
}

int kvlr_build_bases(const kvlr_config* cfg, int64_t n_units, int64_t L, const void* K,
                     const void* V, kvlr_cache* cache, float* eigvals_k, float* eigvals_v,
                     void* ws, size_t ws_bytes, void* stream) {
  int e = check_cfg(cfg);
  if (e) return e;
  if (n_units < 1 || n_units > (1 << 20)) return fail(KVLR_EINVAL, "n_units out of range");
  if ((e = check_sample_fits(cfg, L))) return e;
  if (!K || !V) return fail(KVLR_EINVAL, "K or V is NULL");
  if ((e = check_cache(cache, false, cfg->n_sink))) return e;
  const BuildLayout bl = build_layout(cfg, n_units);
  if (!ws || ws_bytes < bl.total)
    return fail(KVLR_EWORKSPACE, "workspace of %zu bytes needed, %zu given", bl.total, ws_bytes);
  hipStream_t st = (hipStream_t)stream;
  const Dims d = dims_of(cfg);
  const int nmat = (int)(2 * n_units);
  char* w = (char*)ws;
  double* A[2] = {(double*)(w + bl.A0), (double*)(w + bl.A1)};
  double* Vm[2] = {(double*)(w + bl.V0), (double*)(w + bl.V1)};
  double* part = (double*)(w + bl.part);
  int* frozen = (int*)(w + bl.frozen);
  int* final_buf = (int*)(w + bl.final_buf);
  int* counter = (int*)(w + bl.counter);
  hipError_t he;
  if ((he = launch_sample_normalize(d, (int)n_units, L, K, V, w + bl.S, st)) != hipSuccess)
    return hip_fail(he, "sample/normalise");
  if ((he = launch_gram(d, nmat, w + bl.S, A[0], Vm[0], st)) != hipSuccess) return hip_fail(he, "gram");
  if ((he = hipMemsetAsync(frozen, 0, (size_t)nmat * sizeof(int), st)) != hipSuccess)
    return hip_fail(he, "memset");
  if ((he = hipMemsetAsync(final_buf, 0, (size_t)nmat * sizeof(int), st)) != hipSuccess)
    return hip_fail(he, "memset");
  const int n = d.D;
  const int max_sweeps = 30;
  const double tol = 1e-13;
  int cur = 0;
  if (bjac_supported(n)) {
    // block Jacobi, in place in A[0] and V[0]; A[1] holds the rounds' Q blocks
    const int nb = n / 32;
    for (int sweep = 0; sweep < max_sweeps; ++sweep) {
      for (int rd = -1; rd < nb - 1; ++rd)  // the self round, then the cross rounds
        if ((he = launch_bjac_round(n, nmat, A[0], Vm[0], A[1], frozen, rd, st)) != hipSuccess)
          return hip_fail(he, "block jacobi round");
      if ((he = launch_jacobi_check(n, nmat, A[0], part, frozen, final_buf, 0, counter, tol, st)) != hipSuccess)
        return hip_fail(he, "jacobi check");
      int active = -1;
      if ((he = hipMemcpyAsync(&active, counter, sizeof(int), hipMemcpyDeviceToHost, st)) != hipSuccess)
        return hip_fail(he, "memcpy");
      if ((he = hipStreamSynchronize(st)) != hipSuccess) return fail(KVLR_EDEVICE, "sync: %s", hipGetErrorString(he));
      if (active == 0) break;
    }
  } else
  for (int sweep = 0; sweep < max_sweeps; ++sweep) {
    for (int rd = 0; rd < n - 1; ++rd) {
      if ((he = launch_jacobi_round(n, nmat, A[cur], A[cur ^ 1], Vm[cur], Vm[cur ^ 1], frozen, st)) != hipSuccess)
        return hip_fail(he, "jacobi round");
      cur ^= 1;
    }
    if (n <= 2) break;
    if (sweep >= 2) {
      if ((he = launch_jacobi_check(n, nmat, A[cur], part, frozen, final_buf, cur, counter, tol, st)) != hipSuccess)
        return hip_fail(he, "jacobi check");
      int active = -1;
      if ((he = hipMemcpyAsync(&active, counter, sizeof(int), hipMemcpyDeviceToHost, st)) != hipSuccess)
        return hip_fail(he, "memcpy");
      if ((he = hipStreamSynchronize(st)) != hipSuccess) return fail(KVLR_EDEVICE, "sync: %s", hipGetErrorString(he));
      if (active == 0) break;
    }
  }
  if ((he = launch_extract(d, nmat, A[0], A[1], Vm[0], Vm[1], frozen, final_buf, cur, cache->basis_k,
                           cache->basis_v, eigvals_k, eigvals_v, st)) != hipSuccess)
    return hip_fail(he, "extract");
  if ((he = hipStreamSynchronize(st)) != hipSuccess) return fail(KVLR_EDEVICE, "sync: %s", hipGetErrorString(he));
  return ok();
}

int kvlr_project(const kvlr_config* cfg, int64_t n_units, int64_t L, const void* K, const void* V,
                 kvlr_cache* cache, void* ws, size_t ws_bytes, void* stream) {
  int e = check_cfg(cfg);
  if (e) return e;
  if (n_units < 1 || n_units > (1 << 20)) return fail(KVLR_EINVAL, "n_units out of range");
  if (!K || !V) return fail(KVLR_EINVAL, "K or V is NULL");
  if ((e = check_cache(cache, true, cfg->n_sink))) return e;
  if (L < (int64_t)cfg->n_sink + cfg->n_recent)
    return fail(KVLR_EINVAL, "prompt length %lld < n_sink + n_recent", (long long)L);
  if (L > cache->L_max) return fail(KVLR_EINVAL, "prompt length %lld > cache L_max %lld", (long long)L, (long long)cache->L_max);
  if (L > INT32_MAX - 1) return fail(KVLR_EINVAL, "prompt too long");
  hipStream_t st = (hipStream_t)stream;
  const Dims d = dims_of(cfg);
  const size_t need = project_ws_bytes(d, n_units);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(KVLR_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  hipError_t he;
  if ((he = launch_project(d, (int)n_units, L, cache->L_max, K, V, cache->basis_k, cache->basis_v,
                           cache->coef_k, cache->coef_v, ws, st)) != hipSuccess)
    return hip_fail(he, "project");
  if ((he = launch_exact_and_reset(d, (int)n_units, L, K, V, cache->sink_k, cache->sink_v, cache->ring_k,
                                   cache->ring_v, cache->qwin, cache->rowstat, cache->lens,
                                   (uint16_t*)cache->qsplit, st)) != hipSuccess)
    return hip_fail(he, "exact/reset");
  return ok();
}

int kvlr_decode_step(const kvlr_config* cfg, int64_t n_units, const void* q, const void* k_new,
                     const void* v_new, kvlr_cache* cache, float* out, int32_t* topk_idx,
                     float* scores, void* ws, size_t ws_bytes, void* stream) {
  int e = check_cfg(cfg);
  if (e) return e;
  if (n_units < 1 || n_units > 65535) return fail(KVLR_EINVAL, "n_units must be in [1, 65535]");
  if (!q || !k_new || !v_new || !out) return fail(KVLR_EINVAL, "q, k_new, v_new or out is NULL");
  if ((e = check_cache(cache, true, cfg->n_sink))) return e;
  if (cache->L_max > INT32_MAX - 1) return fail(KVLR_EINVAL, "L_max too large");
  const DecodeLayout dl = decode_layout(cfg, n_units, cache->L_max);
  if (!ws || ws_bytes < dl.total)
    return fail(KVLR_EWORKSPACE, "workspace of %zu bytes needed, %zu given", dl.total, ws_bytes);
  hipStream_t st = (hipStream_t)stream;
  const Dims d = dims_of(cfg);
  char* w = (char*)ws;
  DecodeWs dw = dl.t;
  dw.stepinfo = (int32_t*)(w + dl.stepinfo);
  dw.partial = (float*)(w + dl.partial);
  dw.spill = (float*)(w + dl.spill);
  dw.tilestat = (float*)(w + dl.tilestat);
  dw.keys = (uint32_t*)(w + dl.keys);
  dw.topk = (int32_t*)(w + dl.topk);
  dw.qlat = (float*)(w + dl.qlat);
  dw.ylat = (float*)(w + dl.ylat);
  dw.yex = (float*)(w + dl.yex);
  dw.astat = (float*)(w + dl.astat);
  dw.gmax = (uint32_t*)(w + dl.gmax);
  dw.cslot = (uint2*)(w + dl.cslot);
  dw.tkpcnt = (int*)(w + dl.tkpcnt);
  dw.tkhint = (uint32_t*)(w + dl.tkhint);
  const CachePtrs cp = cache_ptrs(cache);
  const int U = (int)n_units;

  hipEvent_t* ev = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (g_prof_on && g_prof_steps < kMaxProfiled) {
      ev = &g_prof_events[(size_t)g_prof_steps * (kStages + 1)];
      ++g_prof_steps;
    }
  }
  hipError_t he;
  if (ev) (void)hipEventRecord(ev[0], st);
  if ((he = launch_prologue(d, U, q, k_new, v_new, cp, dw, st)) != hipSuccess) return hip_fail(he, "prologue");
  if (ev) (void)hipEventRecord(ev[1], st);
  if ((he = launch_score(d, U, cp, dw, st)) != hipSuccess) return hip_fail(he, "score");
  if (ev) (void)hipEventRecord(ev[2], st);
  if ((he = launch_pool(d, U, cp, dw, scores, st)) != hipSuccess) return hip_fail(he, "pool");
  if (ev) (void)hipEventRecord(ev[3], st);
  if ((he = launch_topk(d, U, cp, dw, v_new, topk_idx, out, st)) != hipSuccess) return hip_fail(he, "topk");
  if (ev) (void)hipEventRecord(ev[4], st);
  if ((he = launch_attend(d, U, q, cp, dw, st)) != hipSuccess) return hip_fail(he, "attend");
  if (ev) (void)hipEventRecord(ev[5], st);
  if ((he = launch_merge(d, U, cp, dw, out, st)) != hipSuccess) return hip_fail(he, "merge");
  if (ev) (void)hipEventRecord(ev[6], st);
  return ok();
}

const char* kvlr_last_error(void) { return g_err; }

int kvlr_abi_version(void) { return KVLR_ABI_VERSION; }

const char* kvlr_build_info(void) {
  return "kvlr gfx950 (HIP " __DATE__ " " __TIME__ ")";
}

int kvlr_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (on && g_prof_events.empty()) {
    g_prof_events.resize((size_t)kMaxProfiled * (kStages + 1));
    for (auto& e : g_prof_events) {
      hipError_t he = hipEventCreate(&e);
      if (he != hipSuccess) {
        g_prof_events.clear();
        return fail(KVLR_EDEVICE, "hipEventCreate: %s", hipGetErrorString(he));
      }
    }
  }
  g_prof_on = on != 0;
  if (on) g_prof_steps = 0;
  return ok();
}

int kvlr_profile_read(float* ms, int n, int* steps) {
  if (!ms || n < 0 || n > kStages) return fail(KVLR_EINVAL, "ms must hold 0..%d entries", kStages);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (int i = 0; i < n; ++i) ms[i] = 0.f;
  for (int sidx = 0; sidx < g_prof_steps; ++sidx) {
    hipEvent_t* ev = &g_prof_events[(size_t)sidx * (kStages + 1)];
    hipError_t he = hipEventSynchronize(ev[kStages]);
    if (he != hipSuccess) return fail(KVLR_EDEVICE, "event sync: %s", hipGetErrorString(he));
    for (int i = 0; i < n; ++i) {
      float t = 0.f;
      he = hipEventElapsedTime(&t, ev[i], ev[i + 1]);
      if (he != hipSuccess) return fail(KVLR_EDEVICE, "elapsed: %s", hipGetErrorString(he));
      ms[i] += t;
    }
  }
  if (steps) *steps = g_prof_steps;
  g_prof_steps = 0;
  return ok();
}

}  // extern "C"
