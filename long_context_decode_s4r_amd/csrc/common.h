// Internal helpers shared by the kvlr HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace kvlr {

// ---- vector types used by the bf16 MFMA builtins ---------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---- bf16 <-> fp32 (storage type for bf16 is uint16_t) ----------------------
__device__ __forceinline__ float bf2f(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

// round to nearest, ties to even; NaN stays NaN
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp64 -> bf16, round to nearest, ties to even, in one step (no rounding
// through fp32 first, which can land on a bf16 tie and round again).
// Finite values in the normal bf16 range are handled on the bits; zeros keep
// their sign; anything else (NaN, inf, subnormal or overflowing results) goes
// through fp32, whose double rounding cannot matter there.
__device__ __forceinline__ uint16_t d2bf(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint64_t sign = (u >> 63) << 15;
  const uint64_t mag = u & 0x7fffffffffffffffull;
  if (mag == 0) return (uint16_t)sign;
  const int eb = (int)(mag >> 52) - 1023 + 127;  // bf16 biased exponent
  if (eb <= 0 || eb >= 255) return f2bf((float)x);
  // exponent and 52 fraction bits, rebiased; drop the low 45 fraction bits
  const uint64_t t = ((uint64_t)eb << 52) | (mag & 0x000fffffffffffffull);
  const uint64_t r = (t + 0x00000fffffffffffull + ((t >> 45) & 1ull)) >> 45;
  return (uint16_t)(sign | r);  // a carry into the exponent is the right result
}

// storage element access, T = float (fp32) or uint16_t (bf16)
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float ld(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void st(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float ld(const uint16_t* p, size_t i) { return bf2f(p[i]); }
  static __device__ __forceinline__ void st(uint16_t* p, size_t i, float v) { p[i] = f2bf(v); }
};

// 8 consecutive bf16 (16 bytes, 16-byte aligned) as an MFMA operand
__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) {
  u16x8 v = *reinterpret_cast<const u16x8*>(p);
  return __builtin_bit_cast(bf16x8, v);
}

// LDS byte offset of a pointer into __shared__ memory
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Eight 16-byte LDS reads issued back to back; the asm waits for all of
// them before it ends, so no read is left in flight past the statement.
// Kept opaque so the compiler's tracking of direct global->LDS loads does
// not add waits for other LDS buffers in front of it.
__device__ __forceinline__ void lds_read8(const uint32_t a[8], bf16x8 out[8]) {
  u16x8 o0, o1, o2, o3, o4, o5, o6, o7;
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %9\n\t"
      "ds_read_b128 %2, %10\n\t"
      "ds_read_b128 %3, %11\n\t"
      "ds_read_b128 %4, %12\n\t"
      "ds_read_b128 %5, %13\n\t"
      "ds_read_b128 %6, %14\n\t"
      "ds_read_b128 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o0), "=&v"(o1), "=&v"(o2), "=&v"(o3), "=&v"(o4), "=&v"(o5), "=&v"(o6), "=&v"(o7)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
  out[0] = __builtin_bit_cast(bf16x8, o0);
  out[1] = __builtin_bit_cast(bf16x8, o1);
  out[2] = __builtin_bit_cast(bf16x8, o2);
  out[3] = __builtin_bit_cast(bf16x8, o3);
  out[4] = __builtin_bit_cast(bf16x8, o4);
  out[5] = __builtin_bit_cast(bf16x8, o5);
  out[6] = __builtin_bit_cast(bf16x8, o6);
  out[7] = __builtin_bit_cast(bf16x8, o7);
}

// Four 16-byte LDS reads, same contract as lds_read8.
__device__ __forceinline__ void lds_read4(const uint32_t a[4], bf16x8 out[4]) {
  u16x8 o0, o1, o2, o3;
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o0), "=&v"(o1), "=&v"(o2), "=&v"(o3)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
  out[0] = __builtin_bit_cast(bf16x8, o0);
  out[1] = __builtin_bit_cast(bf16x8, o1);
  out[2] = __builtin_bit_cast(bf16x8, o2);
  out[3] = __builtin_bit_cast(bf16x8, o3);
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row (M index) held by accumulator register i of lane l for the 32x32 MFMA
// result; the column (N index) is l % 32.
__device__ __forceinline__ int acc_row32(int i, int l) { return 8 * (i >> 2) + 4 * (l >> 5) + (i & 3); }

__device__ __forceinline__ float warp_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float warp_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Reductions over the 64 lanes of a wave without LDS round trips: four DPP
// steps inside each row of 16 lanes (quad xor 1, quad xor 2, half-row mirror,
// row mirror) leave every lane of a row holding the row's value (bit-identical
// across the row), then the four rows are combined from v_readlane results,
// so every lane returns the same wave value.  N independent values are
// reduced together to overlap their latencies.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
template <int N>
__device__ __forceinline__ void wave_sum_n(float* v) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_f<0xB1>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_f<0x4E>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_f<0x141>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_f<0x140>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i)
    v[i] = (lane_f(v[i], 0) + lane_f(v[i], 16)) + (lane_f(v[i], 32) + lane_f(v[i], 48));
}
template <int N>
__device__ __forceinline__ void wave_max_n(float* v) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], dpp_f<0xB1>(v[i]));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], dpp_f<0x4E>(v[i]));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], dpp_f<0x141>(v[i]));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], dpp_f<0x140>(v[i]));
#pragma unroll
  for (int i = 0; i < N; ++i)
    v[i] = fmaxf(fmaxf(lane_f(v[i], 0), lane_f(v[i], 16)), fmaxf(lane_f(v[i], 32), lane_f(v[i], 48)));
}

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace kvlr

// ---- launchers (defined in prefill.hip / decode.hip, called by api.hip) ------
namespace kvlr {

struct Dims {
  int Hq, Hkv, dh, D;
  int r;       // key rank r_K (the latent scores, the query window)
  int rv;      // value rank r_V
  int G, s, T, rnum, rden, W, k, nrec, kappa, dtype;
  int local;   // recent window: 0 exact ring, 1 rebuilt from coefficients
};

// prefill
hipError_t launch_sample_normalize(const Dims& d, int U, int64_t L, const void* K, const void* V,
                                   void* S, hipStream_t st);
// gws: device workspace of gram_nt_ws_bytes(d, nmat) bytes for the bf16 GEMM
// form (D' a multiple of 128); null (or 0 bytes needed) selects the direct kernel
size_t gram_nt_ws_bytes(const Dims& d, int nmat);
hipError_t launch_gram(const Dims& d, int nmat, const void* S, double* A, double* Vm, void* gws,
                       hipStream_t st);
hipError_t launch_jacobi_round(int n, int nmat, const double* A_src, double* A_dst,
                               const double* V_src, double* V_dst, const int* frozen,
                               hipStream_t st);
// block Jacobi (n a multiple of 64, n >= 128): round k of a sweep (k = -1:
// rotations inside blocks; k = 0 .. n/32 - 2: between the blocks the circle
// schedule pairs); Qbuf holds bjac_q_bytes(n, nmat)
bool bjac_supported(int n);
size_t bjac_q_bytes(int n, int nmat);
// (T = double, or float for the fp32 eigensolve of bf16 storage)
template <typename T>
hipError_t launch_bjac_round(int n, int nmat, T* A, T* V, T* Qbuf, const int* frozen, int k,
                             hipStream_t st);
// fp32 eigensolve: round k's subproblems (into Q; skipped when !do_eig) with V's
// update of round kv of sweep vs (vs < 0: none) from Qv in one launch, then
// A's update of round k; Q and Qv each hold bjac_q_bytes(n, nmat) / 2
hipError_t launch_bjac_round_f32(int n, int nmat, float* A, float* V, float* Q, const float* Qv,
                                 const int* frozen, const int* done_sweeps, int k, int do_eig, int kv,
                                 int vs, hipStream_t st);
// the Gram matrices rounded to fp32 and V32 = I (start of the fp32 eigensolve)
hipError_t launch_to_f32(int n, int nmat, const double* A64, float* A32, float* V32, hipStream_t st);
// convergence bookkeeping of the eigensolves, per matrix: frozen (converged,
// later rounds skip it), final_buf (buffer holding its result, scalar path),
// done_sweeps (sweep count at convergence, 0 = not yet)
hipError_t launch_jacobi_init(int nmat, int* frozen, int* final_buf, int* done_sweeps, hipStream_t st);
template <typename T>
hipError_t launch_jacobi_check(int n, int nmat, const T* A, double* part, int* frozen,
                               int* final_buf, int* done_sweeps, int cur, int sweep, double tol,
                               hipStream_t st);
template <typename S>
hipError_t launch_extract(const Dims& d, int nmat, const S* A0, const S* A1, const S* V0, const S* V1,
                          const int* frozen, const int* final_buf, const int* done_sweeps, int cur,
                          void* basis_k, void* basis_v, float* eig_k, float* eig_v, int32_t* sweeps,
                          int batch, int depth, int* eidx, hipStream_t st);
// bases shared over windows of `depth` layers: Grams summed into each
// window's first layer, the other layers' matrices frozen
hipError_t launch_gram_window_sum(int n, int n_layers, int batch, int depth, double* A, int* frozen,
                                  hipStream_t st);
// workspace bytes of launch_project_call (B^V transposed; 0 when not used)
size_t project_ws_bytes(const Dims& d, int64_t U);

// decode
constexpr int kHistBins = 4096;  // selection histogram over the top 12 key bits
constexpr int kPoolChunk = 2048; // candidates per block of the pooling kernel
constexpr int kTopkGroupCap = 8192;  // group maxima per unit read by the top-k kernel

struct DecodeWs {
  int32_t* stepinfo;  // [U][4]     {tokens cached, steps taken, unit full, -}
  float* partial;     // [U][Lc_cap] score contribution of the older window rows
  float* spill;       // [U][G][Lc_cap] base-2 logits of the current rows
  float* tilestat;    // [U][nsplit][G][2] per-split (max, sum) of the current rows
  uint32_t* keys;     // [U][Lc_cap] pooled scores as ordered bit patterns
  int32_t* topk;      // [U][ktot] rebuilt rows: the picks ascending, then the
                      //            recent window's positions if it is rebuilt
  float* qlat;        // [U][Hq][r] query heads projected onto their KV head's
                      //            slice of B^K, times log2(e)/sqrt(d_h)
  float* ylat;        // [U][nsl][Hq][r] per split: sum_j p_j c^V_j (latent)
  float* yex;         // [U][nse][Hq][dh] per split: sum_j p_j v_j (exact rows)
  float* astat;       // [U][nsl + nse][Hq][2] per split: (max, sum) of the
                      //            base-2 attention logits
  uint32_t* gmax;     // [U][Lc_cap / 8] largest key of each group of 8 << gsh candidates
  uint2* cslot;       // [U][Lc_cap] top-k scratch: (key, position) candidates
  int* tkpcnt;        // [U][tk_nbp] keys >= the hint per pooling block
  uint32_t* tkhint;   // [U] selection hint carried from the previous step (any value is valid)
  // tiling (decode_tiling)
  int Lc_cap, nsplit, chunk;  // scoring: candidate capacity, splits, split length
  int gsh;                    // top-k: groups of 8 << gsh candidates, at most kTopkGroupCap
  int tk_nbp;                 // pooling blocks per unit, ceil(Lc_cap / kPoolChunk)
  int nsl, nhg, hb, rsl;      // attention over selected rows: row splits, head
                              // groups, heads per group, rows per split
  int nse, rse;               // attention over exact rows: splits, rows per split
  int ktot;                   // length of the rebuilt-row list (k, + n_rec if rebuilt)
  int attend_lds;             // dynamic LDS of the attention kernel (bytes)
};

struct CachePtrs {
  void *sink_k, *sink_v, *ring_k, *ring_v, *coef_k, *coef_v, *basis_k, *basis_v;
  float* qwin;
  int32_t* lens;
  // per-unit opaque decode state, state_stride bytes per unit:
  //   [W][G][2][r] bf16  hi / lo parts of qwin * log2(e)/sqrt(r) (scorer operands)
  //   [W][G][2]    fp32  running (max, sum) of each window row's latent softmax
  //   (bf16 storage) [r][D'] bf16  B^K transposed, one contiguous row per
  //                  column of B^K (the prologue's operand; written by the
  //                  projection call, not part of the window state)
  uint8_t* state;
  int64_t state_stride, rowstat_off, bkt_off;
  int64_t Lmax;
};
__host__ __device__ inline uint16_t* qsplit_of(const CachePtrs& c, int64_t u) {
  return reinterpret_cast<uint16_t*>(c.state + u * c.state_stride);
}
__host__ __device__ inline float* rowstat_of(const CachePtrs& c, int64_t u) {
  return reinterpret_cast<float*>(c.state + u * c.state_stride + c.rowstat_off);
}
__host__ __device__ inline uint16_t* bkt_of(const CachePtrs& c, int64_t u) {
  return reinterpret_cast<uint16_t*>(c.state + u * c.state_stride + c.bkt_off);
}
// state layout of one unit (bytes): the bf16 window operands, then the row
// statistics (together the window state, cleared by the projection call),
// then for bf16 storage B^K transposed; 256-byte aligned parts
inline int64_t state_rowstat_off(const Dims& d) {
  return ((int64_t)d.W * d.G * 2 * d.r * 2 + 15) / 16 * 16;
}
inline int64_t state_bkt_off(const Dims& d) {
  return (state_rowstat_off(d) + (int64_t)d.W * d.G * 2 * 4 + 255) / 256 * 256;
}
inline int64_t state_unit_bytes(const Dims& d) {
  return state_bkt_off(d) + (d.dtype != 0 ? ((int64_t)d.r * d.D * 2 + 255) / 256 * 256 : 0);
}

// prefill: the window seeded with the prompt's last n_tail queries
size_t window_init_ws_bytes(const Dims& d, int64_t U, int64_t L, int n_tail);
hipError_t launch_window_init(const Dims& d, int U, int64_t L, int n_tail, const void* q_tail,
                              const CachePtrs& c, void* ws, hipStream_t st);

// prefill: exact sinks and ring, window and decode state cleared, lens = {L, 0},
// (bf16) B^K transposed into the unit state
// the whole projection call: coefficients, exact rows, window reset and the
// transposed B^K of the decode state
hipError_t launch_project_call(const Dims& d, int U, int64_t L, const void* K, const void* V,
                               const CachePtrs& c, void* ws, hipStream_t st);
hipError_t launch_exact_and_reset(const Dims& d, int U, int64_t L, const void* K, const void* V,
                                  const CachePtrs& c, hipStream_t st);

hipError_t launch_prologue(const Dims& d, int U, const void* q, const void* k_new,
                           const void* v_new, const CachePtrs& c, const DecodeWs& w,
                           hipStream_t st);
hipError_t launch_score(const Dims& d, int U, const CachePtrs& c, const DecodeWs& w,
                        hipStream_t st);
hipError_t launch_pool(const Dims& d, int U, const CachePtrs& c, const DecodeWs& w,
                       float* scores_user, hipStream_t st);
hipError_t launch_topk(const Dims& d, int U, const CachePtrs& c, const DecodeWs& w, const void* v_new,
                       int32_t* topk_user, float* out, hipStream_t st);
hipError_t launch_attend(const Dims& d, int U, const void* q, const CachePtrs& c,
                         const DecodeWs& w, hipStream_t st);
hipError_t launch_merge(const Dims& d, int U, const CachePtrs& c, const DecodeWs& w, float* out,
                        hipStream_t st);

// decode tiling decisions shared by the workspace sizing and the launches:
// fills the int fields of *w (pointers untouched)
void decode_tiling(const Dims& d, int64_t U, int64_t Lmax, DecodeWs* w);
// dynamic LDS bytes of the attention kernel for this shape (0 if it cannot fit)
size_t attend_lds_bytes(const Dims& d);
// bf16 storage: (key rank, value rank) pairs the attention kernel is built for
bool attend_ranks_supported(int r, int rv);

}  // namespace kvlr
