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
 *   kvlr_build_bases  prefill: bases B^K (rank r_K) and B^V (rank r_V) from a
 *                     sample of the prompt's non-sink states, each state row
 *                     scaled to unit length (Eqs. 1-2);
 *   kvlr_project      prefill: every non-sink token kept as its coefficients
 *                     c = x.B (Eq. 3); the sinks and the recent window stay
 *                     exact;
 *   kvlr_decode_step  one decode step: the new token is appended; the latent
 *                     scores Z = C_Q C_K^T / sqrt(r_K) of the last W steps'
 *                     query coefficients go through a softmax over the cached
 *                     positions (Eqs. 8-10); a pooled top-k picks positions
 *                     (Eqs. 13-15); the picked rows are rebuilt from their
 *                     coefficients (Eq. 16) and attended exactly together with
 *                     the sinks and the recent window (Eqs. 16-18).
 *
 * Conventions shared by every call
 *   - Every pointer argument named as device memory is a device pointer owned
 *     by the caller; the library never allocates, frees or keeps pointers
 *     after a call returns.  Host-memory arguments are named as such.
 *   - Device buffers start on a 16-byte boundary (hipMalloc and torch
 *     allocations start on 256): the kernels move rows in 16-byte pieces.  A
 *     call given a device pointer that does not returns KVLR_EINVAL.
 *   - A "unit" is one (layer, sequence) pair; every per-unit buffer is
 *     unit-major ([n_units][...]).  Where layers matter (depth-shared bases)
 *     units are layer-major: unit = layer * batch + sequence.
 *   - D' = n_kv_heads * head_dim (KV heads concatenated, head-major: channel
 *     h*head_dim + j); G = n_q_heads / n_kv_heads.
 *   - "storage" tensors (K, V, q, k_new, v_new, sinks, ring, coefficients,
 *     bases) have the element type cfg->dtype (fp32 or bf16, row-major);
 *     the query window, outputs and scores are fp32.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*, NULL =
 *     the null stream) and every call returns without waiting for it; no
 *     call copies to or from the host or synchronises, so every call can be
 *     captured in a HIP graph.  Asynchronous device faults surface at the
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

#define KVLR_ABI_VERSION 2

typedef enum { KVLR_F32 = 0, KVLR_BF16 = 1 } kvlr_dtype;

/* How the recent window (the last n_recent tokens) enters the attention. */
typedef enum {
  KVLR_LOCAL_EXACT = 0,         /* exact rows from the ring buffer            */
  KVLR_LOCAL_RECONSTRUCTED = 1  /* rebuilt from their coefficients like the
                                   top-k rows ('Core claim': only the local
                                   window and the top-k positions are rebuilt) */
} kvlr_local_window;

typedef enum {
  KVLR_OK = 0,
  KVLR_EINVAL = 1,      /* bad shape / parameter / null pointer            */
  KVLR_EWORKSPACE = 2,  /* workspace smaller than kvlr_workspace_bytes()   */
  KVLR_EDEVICE = 3,     /* HIP runtime error (no device ...)               */
  KVLR_ELAUNCH = 4      /* a kernel launch failed                          */
} kvlr_status;

/* Shape of one attention layer plus the method's parameters
 * ('Assumptions & free parameters': s, W, kappa, the 7:3 sample split and the
 * rank; 'Reading between the lines': a key-to-value rank split). */
typedef struct kvlr_config {
  int32_t n_q_heads;          /* H_q                                           */
  int32_t n_kv_heads;         /* H_kv, divides H_q                             */
  int32_t head_dim;           /* d_h                                           */
  int32_t rank_k;             /* r_K <= D': key rank (latent scale 1/sqrt(r_K)) */
  int32_t rank_v;             /* r_V <= D': value rank                         */
  int32_t n_sink;             /* s: exact sink tokens                          */
  int32_t n_sample;           /* T': rows of the SVD sample                    */
  int32_t sample_recent_num;  /* recent share of the sample = num/den (7/10;
                                 num = den: all-recent 10:0 sample)           */
  int32_t sample_recent_den;
  int32_t q_window;           /* W: query-coefficient window (blocks)          */
  int32_t top_k;              /* k: reconstructed positions per step           */
  int32_t n_recent;           /* recent window (includes the new token)        */
  int32_t pool_kernel;        /* kappa: odd max-pool width, 1 = no pooling     */
  int32_t local_window;       /* kvlr_local_window                             */
  int32_t eig_max_sweeps;     /* Jacobi sweeps enqueued by kvlr_build_bases;
                                 0 = the default (16 for the fp32
                                 eigensolve of bf16 storage, else 24)          */
  int32_t dtype;              /* kvlr_dtype of the storage tensors             */
} kvlr_config;

/* Persistent per-unit state, all device memory owned by the caller.  Sizes in
 * bytes come from kvlr_cache_bytes(), in the order of the KVLR_BUF_* enum. */
typedef struct kvlr_cache {
  void* sink_k;     /* [U][s][D']          storage  exact sink keys          */
  void* sink_v;     /* [U][s][D']          storage                           */
  void* ring_k;     /* [U][n_recent][D']   storage  slot = position % n_rec  */
  void* ring_v;     /* [U][n_recent][D']   storage                           */
  void* coef_k;     /* [U][L_max][r_K]     storage  row = absolute position  */
  void* coef_v;     /* [U][L_max][r_V]     storage  (rows < s unused)        */
  void* basis_k;    /* [U][D'][r_K]        storage  B^K, orthonormal columns */
  void* basis_v;    /* [U][D'][r_V]        storage  B^V                      */
  float* qwin;      /* [U][W][G][r_K]      fp32     query coefficients; the
                                                    block pushed as number p
                                                    (from 0) is in slot p % W */
  int32_t* lens;    /* [U][2]              int32    {tokens cached, query
                                                    blocks pushed}           */
  void* state;      /* [U][state bytes]    opaque   the library's own per-unit
                                                    decode state (running
                                                    softmax statistics of the
                                                    window rows and the
                                                    scorer's operand copy of
                                                    the window); written by
                                                    kvlr_project, advanced by
                                                    kvlr_decode_step         */
  int64_t L_max;    /* capacity in tokens (prompt + decode steps)           */
} kvlr_cache;

enum {
  KVLR_BUF_SINK_K = 0, KVLR_BUF_SINK_V, KVLR_BUF_RING_K, KVLR_BUF_RING_V,
  KVLR_BUF_COEF_K, KVLR_BUF_COEF_V, KVLR_BUF_BASIS_K, KVLR_BUF_BASIS_V,
  KVLR_BUF_QWIN, KVLR_BUF_LENS, KVLR_BUF_STATE, KVLR_BUF_COUNT
};

enum { KVLR_OP_BUILD_BASES = 0, KVLR_OP_PROJECT = 1, KVLR_OP_DECODE = 2, KVLR_OP_INIT_WINDOW = 3 };

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
 * hint; its contents between calls never change a result.  One documented
 * exception, for checking: after kvlr_build_bases the first bytes of its
 * workspace hold the normalised sample, [U][2 (K, V)][T'][D'] storage. */
int kvlr_workspace_bytes(const kvlr_config* cfg, int op, int64_t n_units,
                         int64_t L, size_t* bytes);

/* Prefill part 1: bases ('What carries the argument', Eqs. 1-2: leading right
 * singular vectors of the per-token normalised sample of non-sink states;
 * 'Core claim': the T'-token sample takes 7 parts from the end of the prompt
 * to 3 parts spread evenly over the rest).
 *   K, V      device, [U][L][D'] storage: the prompt's keys and values.
 *   cache     basis_k ([U][D'][r_K]) and basis_v ([U][D'][r_V]) are written:
 *             the leading eigenvectors of S^T S, S = the sample with every
 *             row divided by its norm and rounded once to the storage type;
 *             other buffers untouched.
 *   eigvals_k, eigvals_v  device, optional (NULL = skip), [U][D'] fp32: all
 *             eigenvalues of S^T S, descending.
 *   sweeps    device, optional (NULL = skip), [U][2] int32: Jacobi sweeps
 *             the K and V eigensolves took to reach off(A)_F <= tol tr(A),
 *             or -1 if they had not within cfg->eig_max_sweeps (the bases are
 *             then the current, unconverged iterate).  The eigensolve runs in
 *             fp32 with tol = 1e-5 for bf16 storage and D' a multiple of 64
 *             (>= 128): eigenvalues to ~1e-5 of the largest, far inside the
 *             bf16 rounding of the stored basis; otherwise in fp64 with
 *             tol = 1e-13.
 *             The call cannot return this as a status without synchronising;
 *             read it after the stream has reached the call.
 *   ws        device workspace of ws_bytes >= kvlr_workspace_bytes(BUILD).
 * Sample positions: floor(T'*num/den) most recent prompt positions plus
 * T' - that many evenly spaced over [s, L - recent); requires L >= s +
 * n_recent and that the sample fits. */
int kvlr_build_bases(const kvlr_config* cfg, int64_t n_units, int64_t L,
                     const void* K, const void* V, kvlr_cache* cache,
                     float* eigvals_k, float* eigvals_v, int32_t* sweeps,
                     void* ws, size_t ws_bytes, void* stream);

/* kvlr_build_bases with one basis per window of neighbouring layers
 * (DepthWeave-KV page, 'Core claim' and Eq. 1: low-rank channel bases shared
 * across a window of adjacent layers, each layer keeping its own coefficients;
 * the router and residuals of that page are not part of this).
 *   n_layers, batch  units are layer-major, unit = layer * batch + sequence;
 *   depth_window     layers [w d, w d + d) share a basis (the last window may
 *                    be shorter); 1 gives per-layer bases.
 * The shared basis of a window and sequence is the rank-r truncated SVD of the
 * layers' normalised samples stacked row-wise: the leading eigenvectors of
 * the sum of their Gram matrices.  It is written to basis_k / basis_v of
 * every unit of the window (copies, so the decode step is unchanged);
 * eigvals and sweeps (optional) hold the window's values for every unit.
 * Workspace: kvlr_workspace_bytes(BUILD, n_layers * batch, L).  Other
 * arguments and errors as for kvlr_build_bases. */
int kvlr_build_bases_shared(const kvlr_config* cfg, int64_t n_layers, int64_t batch,
                            int32_t depth_window, int64_t L, const void* K, const void* V,
                            kvlr_cache* cache, float* eigvals_k, float* eigvals_v,
                            int32_t* sweeps, void* ws, size_t ws_bytes, void* stream);

/* Prefill part 2: coefficients and exact buffers (Eq. 3: every non-sink token
 * kept as c = x.B; the sinks stay exact, 'Core claim').
 *   K, V      device, [U][L][D'] storage (same prompt as kvlr_build_bases).
 *   cache     reads basis_k/v; writes coef_k/v rows [s, L), sink_k/v, ring
 *             (positions [L - n_recent, L)), zeroes qwin and state, sets
 *             lens = {L, 0}.  Requires L <= cache->L_max.
 *   ws        device workspace, ws_bytes >= kvlr_workspace_bytes(PROJECT): the
 *             value basis transposed for the MFMA kernel (the key basis
 *             transposed is kept in the cache's state, where decoding reads
 *             it too); the size is 0 (ws may be NULL) for fp32 storage or
 *             ranks not a multiple of 64. */
int kvlr_project(const kvlr_config* cfg, int64_t n_units, int64_t L,
                 const void* K, const void* V, kvlr_cache* cache,
                 void* ws, size_t ws_bytes, void* stream);

/* Seed the query-coefficient window with the queries of the prompt's last
 * n_tail tokens (a variant of the window's start: by default it starts empty
 * and the first decode step scores with its own query only).  Call after
 * kvlr_project, before the first decode step.
 *   n_tail    1 <= n_tail <= W.
 *   q_tail    device, [U][n_tail][H_q][d_h] storage, oldest token first.
 *   cache     each tail query's coefficients c_q[g] = q_cat[g].B^K are pushed
 *             into qwin as a decode step would push them (lens[1] advances by
 *             n_tail), and the pushed rows' softmax statistics over the
 *             current candidates [s, L - n_recent) go into state.
 *   ws        device workspace of ws_bytes >= kvlr_workspace_bytes(INIT_WINDOW,
 *             U, L_max) (sized for n_tail = W). */
int kvlr_init_window(const kvlr_config* cfg, int64_t n_units, int32_t n_tail,
                     const void* q_tail, kvlr_cache* cache, void* ws, size_t ws_bytes,
                     void* stream);

/* One decode step for every unit ('Referee Report' summary: a window of the
 * last W steps' query coefficients, latent scoring Eqs. 8-10, selection of the
 * recent window and the top-k positions Eqs. 13-15, rebuilding of the chosen
 * rows and exact attention Eqs. 16-18).
 *   q         device, [U][H_q][d_h] storage: the new token's queries.
 *   k_new     device, [U][H_kv][d_h] storage: its key; v_new likewise.
 *   cache     read and advanced: the token is appended at position L_t - 1
 *             (coefficient rows and exact ring), its query coefficients are
 *             pushed into the window, lens advance by one token and one
 *             block.  Requires lens[u][0] < L_max for every unit (device-side:
 *             a full unit is left unchanged and its output rows are zero).
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

/* kvlr_decode_step for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step and the same results, with the workspace taken from a fixed scratch
 * array of KVLR_NOALLOC_SCRATCH_BYTES that the library keeps in device memory,
 * one copy per GPU, for the life of the process.  The call allocates nothing.
 * Arguments as for kvlr_decode_step, without ws / ws_bytes.
 * Errors: KVLR_EWORKSPACE if kvlr_workspace_bytes(DECODE) for this call
 * exceeds the scratch (the message gives both sizes); KVLR_EDEVICE if the
 * scratch of the current device cannot be located.
 * Every call on one GPU shares that GPU's scratch, and the scratch keeps the
 * last call's contents (only a speed hint of the top-k, which never changes a
 * result): calls that overlap on one GPU (concurrent streams or threads)
 * race and must be ordered by the caller. */
#define KVLR_NOALLOC_SCRATCH_BYTES (32 << 20)
int kvlr_decode_step_noalloc(const kvlr_config* cfg, int64_t n_units,
                             const void* q, const void* k_new, const void* v_new,
                             kvlr_cache* cache, float* out, int32_t* topk_idx,
                             float* scores, void* stream);

/* Ranks for a target retention ratio eta ('Referee Report' major comment 3 and
 * 'Assumptions & free parameters': the rank is solved from the memory
 * equation, Eq. 21, for a target eta; the page does not print Eq. 21, so the
 * accounting is this library's persistent bytes over the full cache's:
 * (2 (s + n_recent) D' + (L - s + D') (r_K + r_V)) / (2 L D') <= eta).
 * Host only.  r_K : r_V = k_parts : v_parts, both multiples of `multiple`;
 * *rank_k, *rank_v (host) get the largest such pair within the target, or 0
 * if none.  Returns KVLR_EINVAL for non-positive sizes or parts. */
int kvlr_rank_for_ratio(double eta, int64_t L, int32_t d_kv, int32_t n_sink,
                        int32_t n_recent, int32_t k_parts, int32_t v_parts,
                        int32_t multiple, int32_t* rank_k, int32_t* rank_v);

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
 * then clears the record.  Records at most 8192 steps.  Measurement only: a
 * profiled step records events, so it is not meant for graph capture. */
int kvlr_profile_enable(int on);
int kvlr_profile_read(float* ms, int n, int* steps);

#ifdef __cplusplus
}
#endif
#endif /* KVLR_H */
