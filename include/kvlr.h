/*
 * kvlr.h -- C ABI of the low-rank compressed-KV (S4R-style) attention path
 * for AMD MI355X (gfx950).
 *
 * Method: "S^4R: Selective Sampling, Subspaces, and Sparse Reconstruction for
 * Compressed Long-Context KV Caching", as described by its machine review at
 * pith.science/paper/2608.00528 (sections 'What carries the argument',
 * 'Core claim', 'Referee Report', 'Assumptions & free parameters').
 *
 * Three calls carry the path:
 *   kvlr_build_bases  prefill, bases B^K, B^V of rank r from a 7:3 sample of
 *                     token-wise normalised non-sink states (Eqs. 1-2);
 *   kvlr_project      prefill, every non-sink token stored as c = x.B (Eq. 3),
 *                     sinks and the recent window kept exact;
 *   kvlr_decode_step  one decode step: new token appended, latent scoring
 *                     Z = C_Q C_K^T / sqrt(r) + softmax over a window of query
 *                     coefficients (Eqs. 8-10), pooled top-k selection
 *                     (Eqs. 13-15), sparse reconstruction c.B^T of the selected
 *                     rows (Eq. 16) and exact attention over sinks + recent
 *                     window + reconstructed rows (Eqs. 16-18).
 *
 * Conventions shared by every call
 *   - Every pointer argument named as device memory is a device pointer owned
 *     by the caller; the library never allocates, frees or keeps pointers
 *     after a call returns.  Host-memory arguments are named as such.
 *   - A "unit" is one (layer, sequence) pair; every per-unit buffer is
 *     unit-major ([n_units][...]), units are independent.
 *   - D' = n_kv_heads * head_dim (KV heads concatenated, head-major: channel
 *     h*head_dim + j); G = n_q_heads / n_kv_heads.
 *   - "storage" tensors (K, V, q, k_new, v_new, sinks, ring, coefficients,
 *     bases) have the element type cfg->dtype (fp32 or bf16, row-major);
 *     the query window, row statistics, outputs and scores are fp32.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*, NULL =
 *     the null stream) and the call returns without waiting, except
 *     kvlr_build_bases, which synchronises `stream` between eigensolver
 *     sweeps to test convergence.  Asynchronous device faults surface at the
 *     caller's next synchronisation.
 *   - Return value: KVLR_OK, or an error status with no work enqueued for
 *     argument errors; kvlr_last_error() then returns a message (thread-
 *     local, valid until the next call on the same thread).
 */
#ifndef KVLR_H
#define KVLR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVLR_ABI_VERSION 1

typedef enum { KVLR_F32 = 0, KVLR_BF16 = 1 } kvlr_dtype;

typedef enum {
  KVLR_OK = 0,
  KVLR_EINVAL = 1,      /* bad shape / parameter / null pointer            */
  KVLR_EWORKSPACE = 2,  /* workspace smaller than kvlr_workspace_bytes()   */
  KVLR_EDEVICE = 3,     /* HIP runtime error (no device, sync failure ...) */
  KVLR_ELAUNCH = 4      /* a kernel launch failed                          */
} kvlr_status;

/* Shape of one attention layer plus the method's parameters
 * ('Assumptions & free parameters': s, W, kappa, 7:3 split, rank r). */
typedef struct kvlr_config {
  int32_t n_q_heads;          /* H_q                                           */
  int32_t n_kv_heads;         /* H_kv, divides H_q                             */
  int32_t head_dim;           /* d_h                                           */
  int32_t rank;               /* r <= D'                                       */
  int32_t n_sink;             /* s: exact sink tokens                          */
  int32_t n_sample;           /* T': rows of the SVD sample                    */
  int32_t sample_recent_num;  /* recent share of the sample = num/den (7/10)   */
  int32_t sample_recent_den;
  int32_t q_window;           /* W: query-coefficient window (decode steps)    */
  int32_t top_k;              /* k: reconstructed positions per step           */
  int32_t n_recent;           /* exact recent window (includes the new token)  */
  int32_t pool_kernel;        /* kappa: odd max-pool width, 1 = no pooling     */
  int32_t dtype;              /* kvlr_dtype of the storage tensors             */
  int32_t reserved;           /* must be 0                                     */
} kvlr_config;

/* Persistent per-unit state, all device memory owned by the caller.  Sizes in
 * bytes come from kvlr_cache_bytes(); index order of kvlr_buffer. */
typedef struct kvlr_cache {
  void* sink_k;     /* [U][s][D']          storage  exact sink keys          */
  void* sink_v;     /* [U][s][D']          storage                           */
  void* ring_k;     /* [U][n_recent][D']   storage  slot = position % n_rec  */
  void* ring_v;     /* [U][n_recent][D']   storage                           */
  void* coef_k;     /* [U][L_max][r]       storage  row = absolute position  */
  void* coef_v;     /* [U][L_max][r]       storage  (rows < s unused)        */
  void* basis_k;    /* [U][D'][r]          storage  B^K, orthonormal columns */
  void* basis_v;    /* [U][D'][r]          storage  B^V                      */
  float* qwin;      /* [U][W][G][r]        fp32     slot = step % W          */
  float* rowstat;   /* [U][W][G][2]        fp32     per window row: running
                                                    max and sum of its latent
                                                    softmax (base-2 domain)  */
  int32_t* lens;    /* [U][2]              int32    {tokens cached, decode
                                                    steps taken}             */
  void* qsplit;     /* [U][W][G][2][r]     bf16     qwin * log2(e)/sqrt(r)
                                                    as hi + lo bf16 parts
                                                    (MFMA operands of the
                                                    latent scoring)          */
  int64_t L_max;    /* capacity in tokens (prompt + decode steps)           */
} kvlr_cache;

enum {
  KVLR_BUF_SINK_K = 0, KVLR_BUF_SINK_V, KVLR_BUF_RING_K, KVLR_BUF_RING_V,
  KVLR_BUF_COEF_K, KVLR_BUF_COEF_V, KVLR_BUF_BASIS_K, KVLR_BUF_BASIS_V,
  KVLR_BUF_QWIN, KVLR_BUF_ROWSTAT, KVLR_BUF_LENS, KVLR_BUF_QSPLIT, KVLR_BUF_COUNT
};

enum { KVLR_OP_BUILD_BASES = 0, KVLR_OP_PROJECT = 1, KVLR_OP_DECODE = 2 };

/* Validate cfg.  Returns KVLR_OK or KVLR_EINVAL (message in last_error). */
int kvlr_check_config(const kvlr_config* cfg);

/* Byte sizes of the kvlr_cache buffers for n_units units of capacity L_max
 * tokens.  bytes: host array of KVLR_BUF_COUNT entries, written on success. */
int kvlr_cache_bytes(const kvlr_config* cfg, int64_t n_units, int64_t L_max,
                     size_t* bytes);

/* Device workspace needed by one call of `op` (KVLR_OP_*) on n_units units;
 * L = prompt length for the prefill ops, the cache capacity L_max for
 * KVLR_OP_DECODE.  *bytes (host) is written on success.  The workspace holds
 * only scratch (sample, Gram/eigensolver matrices, transposed bases, partial
 * scores, spilled logits, attention partials) and, for decode, a top-k speed
 * hint; its contents between calls are unspecified and never change a
 * result. */
int kvlr_workspace_bytes(const kvlr_config* cfg, int op, int64_t n_units,
                         int64_t L, size_t* bytes);

/* Prefill part 1: bases ('What carries the argument': truncated SVD over the
 * sampled, token-wise-normalised non-sink states; 'Core claim': 7:3
 * recent-to-uniform sample of T' tokens).
 *   K, V      device, [U][L][D'] storage: the prompt's keys and values.
 *   cache     basis_k / basis_v are written ([U][D'][r], top-r eigenvectors
 *             of S^T S, S = the rounded, row-normalised sample); other
 *             buffers untouched.
 *   eigvals_k, eigvals_v  device, optional (NULL = skip), [U][D'] fp32: all
 *             eigenvalues of S^T S, descending.
 *   ws        device workspace of ws_bytes >= kvlr_workspace_bytes(BUILD).
 * Sample positions: floor(T'*num/den) most recent prompt positions plus
 * T' - that many evenly spaced over [s, L - recent); requires L >= s +
 * n_recent and that the sample fits.  Synchronises `stream`. */
int kvlr_build_bases(const kvlr_config* cfg, int64_t n_units, int64_t L,
                     const void* K, const void* V, kvlr_cache* cache,
                     float* eigvals_k, float* eigvals_v,
                     void* ws, size_t ws_bytes, void* stream);

/* Prefill part 2: coefficients and exact buffers (Eq. 3: every non-sink token
 * stored as c = x.B; sinks kept exact, 'Core claim').
 *   K, V      device, [U][L][D'] storage (same prompt as kvlr_build_bases).
 *   cache     reads basis_k/v; writes coef_k/v rows [s, L), sink_k/v, ring
 *             (positions [L - n_recent, L)), zeroes qwin, qsplit and rowstat, sets
 *             lens = {L, 0}.  Requires L <= cache->L_max.
 *   ws        device workspace, ws_bytes >= kvlr_workspace_bytes(PROJECT): the
 *             bases transposed ([U][2][r][D'] storage) for the MFMA kernel; the
 *             size is 0 (ws may be NULL) for fp32 storage or r % 64 != 0. */
int kvlr_project(const kvlr_config* cfg, int64_t n_units, int64_t L,
                 const void* K, const void* V, kvlr_cache* cache,
                 void* ws, size_t ws_bytes, void* stream);

/* One decode step for every unit ('Referee Report' summary: sliding window of
 * query coefficients, latent scoring Eqs. 8-10, local window plus top-k
 * selection Eqs. 13-15, sparse reconstruction and exact attention Eqs. 16-18).
 *   q         device, [U][H_q][d_h] storage: the new token's queries.
 *   k_new     device, [U][H_kv][d_h] storage: its key; v_new likewise.
 *   cache     read and advanced: the token is appended at position L_t - 1
 *             (coefficient rows and exact ring), its query coefficients enter
 *             the window, lens advance by one token and one step.  Requires
 *             lens[u][0] < L_max for every unit (device-side: a full unit is
 *             left unchanged and its output rows are set to zero).
 *   out       device, [U][H_q][d_h] fp32: attention output.
 *   topk_idx  device, optional, [U][top_k] int32: selected absolute positions,
 *             ascending; unused tail entries (fewer candidates than top_k) = -1.
 *   scores    device, optional, [U][L_max] fp32: latent score of candidate
 *             position j at index j (before pooling); other entries untouched.
 *   ws        device workspace, ws_bytes >= kvlr_workspace_bytes(DECODE, L_max).
 *             Reusing the same workspace for consecutive steps of the same
 *             cache lets the top-k start from the previous step's threshold
 *             (a speed hint only: any workspace content gives the same
 *             result).
 * Candidates are positions [s, L_t - n_recent); ties in the pooled score go to
 * the lower position. */
int kvlr_decode_step(const kvlr_config* cfg, int64_t n_units,
                     const void* q, const void* k_new, const void* v_new,
                     kvlr_cache* cache, float* out, int32_t* topk_idx,
                     float* scores, void* ws, size_t ws_bytes, void* stream);

/* Message for the last non-OK status on this thread ("" if none). */
const char* kvlr_last_error(void);

/* ABI version (KVLR_ABI_VERSION) and build string (host memory, static). */
int kvlr_abi_version(void);
const char* kvlr_build_info(void);

/* Stage timing for measurement.  kvlr_profile_enable(1) makes every following
 * kvlr_decode_step record HIP events between its stages on its stream
 * (stages: 0 prologue, 1 latent scoring, 2 score finalisation + pooling,
 * 3 top-k selection, 4 reconstruction + attention, 5 split merge);
 * kvlr_profile_enable(0) stops.  kvlr_profile_read
 * waits for the recorded events, writes the summed milliseconds per stage to
 * ms (host, n entries, n <= 6) and the number of profiled steps to *steps,
 * then clears the record.  Records at most 8192 steps. */
int kvlr_profile_enable(int on);
int kvlr_profile_read(float* ms, int n, int* steps);

#ifdef __cplusplus
}
#endif
#endif /* KVLR_H */
