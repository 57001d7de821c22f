// Decode-step kernels: prologue (append + query coefficients + window),
// latent scoring, pooled top-k selection (two kernels), sparse reconstruction
// + exact attention (split over rows, splits merged by the last block).
//
// Method: S^4R review (pith.science/paper/2608.00528): 'What carries the
// argument' (relevance of every cached position from a softmax of the last W
// steps' query coefficients against its key coefficients, Eqs. 8-10; only
// the chosen positions are rebuilt from their coefficients, Eqs. 13-16, and
// attended exactly together with the exact sink tokens), 'Core claim' (the
// queries are mapped onto the key basis), 'Referee Report' major comment 2
// (Z = C_Q C_K^T / sqrt(r)).
//
// Latent softmax bookkeeping.  Each window row (one query coefficient vector
// of one earlier step) keeps the running max m and sum S of its softmax over
// the candidates in base 2 (rowstat).  Candidates only grow, by one position
// per step (the token leaving the exact recent window), so a row's (m, S) is
// updated with that one logit in the prologue and stays exact.  Only the G
// rows of the current step need a full pass: the scoring kernel writes their
// logits to a spill buffer together with per-split (m, S) partials, and the
// pooling kernel merges them before adding their probabilities.  The key
// coefficients are therefore read once per step.
//
// Per-step flow of the unit state: the prologue reads lens and snapshots it
// in stepinfo; every later kernel reads stepinfo; the top-k kernel (one
// block per unit) advances lens.
#include "common.h"

#include <float.h>
#include <math.h>

namespace kvlr {

static inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Attention tile over the selected rows: hb query heads (multiple of 8) and
// rsl rows (multiple of 4, <= 64) per block.  LDS: projected queries
// [hb][r + 4] fp32, logits [hb][rsl + 1] fp32, probabilities [rsl][hb] fp32,
// coefficient rows of K
// and V [rsl][r] storage type with 16 bytes of padding per row.
static size_t latent_lds(const Dims& d, int hb, int rsl) {
  const size_t el = d.dtype == 0 ? 4 : 2;
  return (size_t)hb * (d.r + 4) * 4 + (size_t)hb * (rsl + 1) * 4 + 16 + (size_t)rsl * hb * 4 +
         (size_t)rsl * (d.r * el + 16) + (size_t)rsl * (d.rv * el + 16);
}
// exact rows, per wave: queries [G][dh] fp32, probabilities [32][8] fp32,
// value rows [32][dh + 16 bytes] storage type
__host__ __device__ inline int exact_wave_floats(int G, int dh, int el) {
  return G * dh + 32 * 8 + 8 * (dh * el + 16);
}
static size_t exact_lds(const Dims& d) {
  return (size_t)4 * exact_wave_floats(d.G, d.dh, d.dtype == 0 ? 4 : 2) * 4;
}
static int attn_tile_bytes(int r, int rv);
static void attend_tile(const Dims& d, int* hb, int* rsl) {
  if (d.dtype != 0) {  // bf16: MFMA tiles of 64 rows x 32 heads
    *hb = 32;
    *rsl = 64;
    return;
  }
  int h = (int)round_up(d.Hq, 8);
  if (h > 32) h = 32;
  int rs = 32;
  while (latent_lds(d, h, rs) > 96 * 1024 && rs > 8) rs /= 2;
  while (latent_lds(d, h, rs) > 96 * 1024 && h > 8) h /= 2;
  *hb = h;
  *rsl = rs;
}

size_t attend_lds_bytes(const Dims& d) {
  int hb, rsl;
  attend_tile(d, &hb, &rsl);
  size_t a = d.dtype != 0 ? (size_t)attn_tile_bytes(d.r, d.rv) : latent_lds(d, hb, rsl);
  size_t b = exact_lds(d);
  a = a > b ? a : b;
  return a <= 160 * 1024 ? a : 0;
}

void decode_tiling(const Dims& d, int64_t U, int64_t Lmax, DecodeWs* w) {
  int64_t lc = Lmax - d.s - d.nrec;
  if (lc < 1) lc = 1;
  lc = round_up(lc, 64);
  w->Lc_cap = (int)lc;
  // scoring: one round of blocks (the kernel holds one block per CU)
  int64_t target = (256 + U - 1) / U;
  if (target < 1) target = 1;
  int64_t maxsplit = lc / 256;
  if (maxsplit < 1) maxsplit = 1;
  int64_t ns = target < maxsplit ? target : maxsplit;
  int64_t ch = round_up((lc + ns - 1) / ns, 64);
  ns = (lc + ch - 1) / ch;
  w->nsplit = (int)ns;
  w->chunk = (int)ch;
  // attention: selected rows in splits of rsl rows x hb heads, exact rows in
  // splits of at most 32 rows
  attend_tile(d, &w->hb, &w->rsl);
  // top-k floor: at most kTopkGroupCap group maxima per unit
  w->gsh = 0;
  while (((lc + (8 << w->gsh) - 1) >> (3 + w->gsh)) > kTopkGroupCap) ++w->gsh;
  w->tk_nbp = (int)((lc + kPoolChunk - 1) / kPoolChunk);
  w->nhg = (d.Hq + w->hb - 1) / w->hb;
  // rebuilt rows: the top-k picks, then (reconstructed local window) the
  // recent window's positions; exact rows: the sinks, then (exact local
  // window) the recent ring
  w->ktot = d.k + (d.local ? d.nrec : 0);
  w->nsl = (w->ktot + w->rsl - 1) / w->rsl;
  const int nex = d.s + (d.local ? 0 : d.nrec);
  w->nse = (nex + 31) / 32;
  w->rse = w->nse > 0 ? (nex + w->nse - 1) / w->nse : 0;
  w->attend_lds = (int)attend_lds_bytes(d);
}

__device__ __forceinline__ int wrap_slot(int x, int W) { return ((x % W) + W) % W; }

// rows rebuilt from coefficients in this step (token count before the
// append = Lcur): the min(k, |J|) picks, plus the recent window when it is
// reconstructed rather than exact
__device__ __forceinline__ int n_rebuilt(const Dims& d, int Lcur) {
  const int kk = max(0, min(d.k, Lcur + 1 - d.nrec - d.s));
  return kk + (d.local ? min(d.nrec, Lcur + 1 - d.s) : 0);
}
// exact rows: the sinks, plus the recent ring when it is attended exactly
__host__ __device__ __forceinline__ int n_exact_rows(const Dims& d) { return d.s + (d.local ? 0 : d.nrec); }

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Kernels that may need more than the default 64 KB of dynamic LDS get the
// limit raised once (gfx950 has 160 KB of LDS per CU).
template <typename K>
static hipError_t allow_lds(K kernel, size_t lds, size_t* done) {
  if (lds <= 65536 || lds <= *done) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e == hipSuccess) *done = lds;
  return e;
}

__device__ __forceinline__ int wv_of(int tid) { return __builtin_amdgcn_readfirstlane(tid >> 6); }
__device__ __forceinline__ int l_of(int tid) { return tid & 63; }

// 16 bytes of storage elements -> fp32
template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void ld(const float* p, float* o) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(p);
    o[0] = v[0]; o[1] = v[1]; o[2] = v[2]; o[3] = v[3];
  }
};
template <> struct Vec16<uint16_t> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void ld(const uint16_t* p, float* o) {
    const u16x8 v = *reinterpret_cast<const u16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = bf2f(v[e]);
  }
};

// --------------------------------------------------------------------------
// prologue: grid (2 * ncb + 1 + H_kv, U), 256 threads.
//   blocks [0, ncb):      c^K(new) = k_cat . B^K and c_q[g] = q_cat[g] . B^K
//                         (window push) for 4*VEC basis columns each;
//   blocks [ncb, 2 ncb):  c^V(new) = v_cat . B^V;
//   block 2 ncb:          exact ring push of k and v; the older window rows'
//                         (m, S) updated with the candidate entering this
//                         step;
//   block 2 ncb + 1 + h:  the G query heads of KV head h projected onto the
//                         rows of B^K that belong to head h, for attention in
//                         the coefficient space.
// GEMV layout: thread (row group rg = tid / 4, column group cg = tid % 4)
// reads 16 bytes of a basis row per iteration (rows rg, rg + 64, ...);
// partial sums are reduced over row groups with lane shuffles and LDS.
// --------------------------------------------------------------------------
// state block of the prologue: exact ring push of k and v; the older window
// rows' (m, S) updated with the candidate entering the compressed set
template <typename T>
__device__ __forceinline__ void prologue_state(const Dims& d, const CachePtrs& c, const T* __restrict__ kn,
                                               const T* __restrict__ vn, const DecodeWs& w, float qscale,
                                               int u, int tid, int32_t Lcur, int32_t steps, float* sm) {
  constexpr int VEC = Vec16<T>::N;
  const int D = d.D, r = d.r, G = d.G, W = d.W;
  const int64_t p = Lcur;
  {  // exact ring push, 16-byte pieces, loads before stores
    const int rs = (int)(p % d.nrec);
    constexpr int NP = (4096 / VEC + 255) / 256;  // D <= 4096
    u16x8 bk[NP], bv[NP];
    const int np = D / VEC;
    const u16x8* sk = reinterpret_cast<const u16x8*>(kn + (int64_t)u * D);
    const u16x8* sv = reinterpret_cast<const u16x8*>(vn + (int64_t)u * D);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int pc = min(tid + 256 * i, np - 1);
      bk[i] = sk[pc];
      bv[i] = sv[pc];
    }
    u16x8* dk = reinterpret_cast<u16x8*>((T*)c.ring_k + ((int64_t)u * d.nrec + rs) * D);
    u16x8* dv = reinterpret_cast<u16x8*>((T*)c.ring_v + ((int64_t)u * d.nrec + rs) * D);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int pc = tid + 256 * i;
      if (pc < np) {
        dk[pc] = bk[i];
        dv[pc] = bv[i];
      }
    }
  }
  const int weff = min(steps + 1, W);
  const int nold = (weff - 1) * G;
  if (nold <= 0) return;
  float* ce = sm;  // [r]
  const int64_t pe = (int64_t)Lcur - d.nrec;  // candidate entering the compressed set
  const T* cep = (const T*)c.coef_k + ((int64_t)u * c.Lmax + pe) * r;
  for (int i = tid; i < r; i += 256) ce[i] = Elem<T>::ld(cep, i);
  __syncthreads();
  for (int o0 = 0; o0 < nold; o0 += 64) {
    const int o = o0 + (tid >> 2), part = tid & 3;
    float z = 0.f;
    int sl = 0, g = 0;
    if (o < nold) {
      const int i = 1 + o / G;
      g = o % G;
      sl = wrap_slot(steps - i, W);
      const float* qr = c.qwin + (((int64_t)u * W + sl) * G + g) * r;
#pragma unroll 16
      for (int kk = part; kk < r; kk += 4) z += qr[kk] * ce[kk];
    }
    z += __shfl_xor(z, 1);
    z += __shfl_xor(z, 2);
    if (o < nold && part == 0) {
      z *= qscale;
      float* rsp = rowstat_of(c, u) + (sl * G + g) * 2;
      const float m = rsp[0], S = rsp[1];
      const float mn = fmaxf(m, z);
      rsp[0] = mn;
      rsp[1] = S * exp2f(m - mn) + exp2f(z - mn);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_prologue(Dims d, CachePtrs c, const T* __restrict__ q,
                                                  const T* __restrict__ kn,
                                                  const T* __restrict__ vn, DecodeWs w,
                                                  float qscale, float ascale, int ncb, int ncbv) {
  constexpr int VEC = Vec16<T>::N;
  constexpr int NVMAX = 9;  // 1 + G, G <= 8
  const int b = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  const int D = d.D, G = d.G, W = d.W;
  const int nkv = ncb + ncbv;  // K column blocks, then V column blocks
  const int r = b >= ncb && b < nkv ? d.rv : d.r;  // rank of this block's basis
  const int32_t Lcur = c.lens[2 * u], steps = c.lens[2 * u + 1];
  // basis pieces of this thread are requested together with the unit state:
  // GEMV blocks rows rg + 64 i of their column slice, projected-query blocks
  // rows rg + 8 i of head h's slice (first column pass)
  constexpr int PF = 16;
  u16x8 bpre[PF];
  if (b < nkv) {
    const T* B = (const T*)(b >= ncb ? c.basis_v : c.basis_k) + (int64_t)u * D * r;
    const int col = min((b >= ncb ? b - ncb : b) * 4 * VEC + (tid & 3) * VEC, r - VEC);
#pragma unroll
    for (int i = 0; i < PF; ++i)
      bpre[i] = *reinterpret_cast<const u16x8*>(B + (int64_t)min((tid >> 2) + 64 * i, D - 1) * r + col);
  } else if (b > nkv) {
    const int h = b - nkv - 1;
    const T* B = (const T*)c.basis_k + ((int64_t)u * D + (int64_t)h * d.dh) * r;
    const int col = min((tid & 31) * VEC, r - VEC);
#pragma unroll
    for (int i = 0; i < PF; ++i)
      bpre[i] = *reinterpret_cast<const u16x8*>(B + (int64_t)min((tid >> 5) + 8 * i, d.dh - 1) * r + col);
  }
  const bool full = (int64_t)Lcur >= c.Lmax;
  if (b == 0 && tid == 0) {
    w.stepinfo[4 * u + 0] = Lcur;
    w.stepinfo[4 * u + 1] = steps;
    w.stepinfo[4 * u + 2] = full ? 1 : 0;
    w.stepinfo[4 * u + 3] = 0;
  }
  if (full) return;
  const int64_t p = Lcur;
  extern __shared__ float sm[];
  if (b < nkv) {
    const int kind = b >= ncb ? 1 : 0;
    const int cb = kind ? b - ncb : b;
    const int nvec = kind == 0 ? 1 + G : 1;
    float* xs = sm;                         // [nvec][D]
    float* red = xs + nvec * D;             // [16 lane rows][nvec][4 * VEC]
    // stage x_0 (k or v) and the G concatenated query vectors as fp32; every
    // thread owns 16-byte pieces, all loads are issued before the stores
    {
      const T* x0 = (kind == 0 ? kn : vn) + (int64_t)u * D;
      const T* qu = q + (int64_t)u * d.Hq * d.dh;
      const int nx = D / VEC, nq = kind == 0 ? d.Hq * d.dh / VEC : 0;
      constexpr int NP = (12288 / VEC + 255) / 256;  // (1 + G) * D <= 12288
      float buf[NP][VEC];
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int pc = tid + 256 * i;
        const T* src = pc < nx ? x0 + pc * VEC : qu + min(pc - nx, max(nq - 1, 0)) * VEC;
        Vec16<T>::ld(src, buf[i]);  // pieces past the end re-read a valid one
      }
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int pc = tid + 256 * i;
        if (pc < nx) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) xs[pc * VEC + e] = buf[i][e];
        } else if (pc < nx + nq) {
          // query element (head a = h * G + g, j) -> vector g, channel h * dh + j
          const int qe = (pc - nx) * VEC, a = qe / d.dh, j = qe % d.dh;
          const int h = a / G, g = a % G;
#pragma unroll
          for (int e = 0; e < VEC; ++e) xs[(1 + g) * D + h * d.dh + j + e] = buf[i][e];
        }
      }
    }
    __syncthreads();
    const T* B = (const T*)(kind == 0 ? c.basis_k : c.basis_v) + (int64_t)u * D * r;
    const int cg = tid & 3, rg = tid >> 2;
    const int col = cb * 4 * VEC + cg * VEC;
    float acc[NVMAX][VEC];
#pragma unroll
    for (int v = 0; v < NVMAX; ++v)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[v][e] = 0.f;
    if (col < r) {
      for (int kk0 = rg; kk0 < D; kk0 += 64 * PF) {
        u16x8 braw[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) {
          if (kk0 == rg) {
            braw[i] = bpre[i];
          } else {
            const int kk = min(kk0 + 64 * i, D - 1);  // rows past D are read, then skipped
            braw[i] = *reinterpret_cast<const u16x8*>(B + (int64_t)kk * r + col);
          }
        }
#pragma unroll
        for (int i = 0; i < PF; ++i) {
          const int kk = kk0 + 64 * i;
          if (kk < D) {
            const T* bv = reinterpret_cast<const T*>(&braw[i]);
#pragma unroll
            for (int v = 0; v < NVMAX; ++v) {
              if (v < nvec) {
                const float x = xs[v * D + kk];
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[v][e] += x * Elem<T>::ld(bv, e);
              }
            }
          }
        }
      }
    }
    // reduce over the row groups: DPP rotations by 4 and 8 inside each row of
    // 16 lanes leave lanes 0..3 of the row holding the sum of its 4 row
    // groups (per column group); the 16 rows of the block meet in LDS
    const int lane = tid & 63, wv = tid >> 6;
    const int prow = wv * 4 + (lane >> 4);
#pragma unroll
    for (int v = 0; v < NVMAX; ++v) {
      if (v < nvec) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          float x = acc[v][e];
          x += dpp_f<0x124>(x);  // row_ror:4
          x += dpp_f<0x128>(x);  // row_ror:8
          if ((lane & 15) < 4) red[(prow * nvec + v) * 4 * VEC + (lane & 3) * VEC + e] = x;
        }
      }
    }
    __syncthreads();
    for (int t = tid; t < nvec * 4 * VEC; t += 256) {
      const int v = t / (4 * VEC), cc = t % (4 * VEC);
      const int cl = cb * 4 * VEC + cc;
      if (cl >= r) continue;
      float sum = 0.f;
#pragma unroll
      for (int q2 = 0; q2 < 16; ++q2) sum += red[(q2 * nvec + v) * 4 * VEC + cc];
      if (v == 0) {
        T* C = (T*)(kind == 0 ? c.coef_k : c.coef_v);
        Elem<T>::st(C, ((int64_t)u * c.Lmax + p) * r + cl, sum);
      } else {
        const int64_t row = ((int64_t)u * W + steps % W) * G + (v - 1);
        c.qwin[row * r + cl] = sum;
        const float x = sum * qscale;  // MFMA operands of the latent scoring
        const uint16_t hb = f2bf(x);
        uint16_t* qs = qsplit_of(c, u) + ((steps % W) * G + (v - 1)) * 2 * r;
        qs[cl] = hb;
        qs[r + cl] = f2bf(x - bf2f(hb));
      }
    }
    return;
  }
  if (b > nkv) {
    // qlat[h G + g] = ascale * q[h G + g] . B^K[h dh : (h + 1) dh, :]
    // (fp32 storage: fp32 rows; bf16 storage: bf16 hi and lo rows)
    const int h = b - nkv - 1, dh = d.dh;
    float* qs = sm;                 // [G][dh]
    float* red = qs + G * dh;       // [4 waves][G][32 * VEC]
    const T* qh = q + ((int64_t)u * d.Hq + h * G) * dh;
    for (int e = tid; e < G * dh; e += 256) qs[e] = Elem<T>::ld(qh, e) * ascale;
    __syncthreads();
    const T* B = (const T*)c.basis_k + ((int64_t)u * D + (int64_t)h * dh) * r;
    const int cg = tid & 31, rg = tid >> 5, lane = tid & 63, wv = tid >> 6;
    for (int c0 = 0; c0 < r; c0 += 32 * VEC) {
      const int colc = min(c0 + cg * VEC, r - VEC);  // columns past r: computed, not stored
      float acc[8][VEC];
#pragma unroll
      for (int g = 0; g < 8; ++g)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[g][e] = 0.f;
      for (int j0 = rg; j0 < dh; j0 += 8 * PF) {
        u16x8 braw[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) {
          if (c0 == 0 && j0 == rg)
            braw[i] = bpre[i];
          else
            braw[i] = *reinterpret_cast<const u16x8*>(B + (int64_t)min(j0 + 8 * i, dh - 1) * r + colc);
        }
#pragma unroll
        for (int i = 0; i < PF; ++i) {
          const int j = j0 + 8 * i;
          if (j < dh) {
            const T* bv = reinterpret_cast<const T*>(&braw[i]);
#pragma unroll
            for (int g = 0; g < 8; ++g) {
              if (g < G) {
                const float x = qs[g * dh + j];
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[g][e] += x * Elem<T>::ld(bv, e);
              }
            }
          }
        }
      }
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        if (g < G) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const float x = acc[g][e] + __shfl_xor(acc[g][e], 32);
            if (lane < 32) red[(wv * G + g) * 32 * VEC + cg * VEC + e] = x;
          }
        }
      }
      __syncthreads();
      for (int t = tid; t < G * 32 * VEC; t += 256) {
        const int g = t / (32 * VEC), cc = t % (32 * VEC);
        if (c0 + cc < r) {
          const int o = g * 32 * VEC + cc, st = G * 32 * VEC;
          const float x = (red[o] + red[o + st]) + (red[o + 2 * st] + red[o + 3 * st]);
          const int64_t a = (int64_t)u * d.Hq + h * G + g;
          if constexpr (sizeof(T) == 4) {
            w.qlat[a * r + c0 + cc] = x;
          } else {  // MFMA operands: bf16 hi and lo rows
            uint16_t* ql = reinterpret_cast<uint16_t*>(w.qlat) + a * 2 * r + c0 + cc;
            const uint16_t hb = f2bf(x);
            ql[0] = hb;
            ql[r] = f2bf(x - bf2f(hb));
          }
        }
      }
      __syncthreads();
    }
    return;
  }
  prologue_state<T>(d, c, kn, vn, w, qscale, u, tid, Lcur, steps, sm);
}

// --------------------------------------------------------------------------
// prologue for bf16 storage when d_h divides 256: grid (r_K / 16 + 1, U),
// 256 threads, products on MFMA 16x16x32.
//   blocks [0, r_K / 16):  16 columns of B^K each, read from the transposed
//     copy in the unit state (one contiguous D'-element row per column, so
//     a block's operand slab is a few whole rows: 32 KB at D' = 1024),
//     straight into the B operands; A = up to 16 input vectors straight
//     from memory (row 0: k, row 1 + g: query head g of every KV head,
//     concatenated; K = channel).  Wave w takes the channels
//     [256 w, 256 w + 256) of every 1024, whole heads since d_h divides
//     256.  After a head's last k-step its accumulator holds the head's
//     partial products: for row 1 + g that is the projected query
//     q[h G + g] . B^K_h of the attention in coefficient space; the sums
//     over heads (in the wave, then over the waves in LDS) give c^K(new)
//     (row 0) and the window query latents (rows 1 .. G).  B^K is read once
//     for all three.
//   block r_K / 16:  exact ring push of k and v; the older window rows'
//     (m, S) updated with the candidate entering the compressed set.
// c^V(new) is first read when the new position leaves the exact ring, at
// least one step later, so its GEMV runs beside the top-k selection (the
// extra blocks of that launch), off this step's critical path.
// --------------------------------------------------------------------------
__host__ __device__ inline bool prologue_fused(const Dims& d) {
  return d.dtype != 0 && d.dh % 32 == 0 && 256 % d.dh == 0 && d.G + 1 <= 16;
}

// state block, bf16 storage: every load (the new k and v, the entering
// candidate's key coefficients, the window rows' query latents and their
// (m, S)) is requested before the first use, so the block costs about one
// memory round trip.  Wave w takes window rows w, w + 4, ...; lane l holds
// columns 4 l .. 4 l + 3 (rank <= 256).
__device__ __forceinline__ void prologue_state_bf16(const Dims& d, const CachePtrs& c, const uint16_t* __restrict__ kn,
                                                    const uint16_t* __restrict__ vn, float qscale, int u, int tid,
                                                    int32_t Lcur, int32_t steps) {
  const int D = d.D, r = d.r, G = d.G, W = d.W;
  const int l = tid & 63, wv = tid >> 6;
  const int64_t p = Lcur;
  const int rs = (int)(p % d.nrec);
  constexpr int NP = (4096 / 8 + 255) / 256;  // D <= 4096
  const int np = D / 8;
  u16x8 bk[NP], bv[NP];
  const u16x8* sk = reinterpret_cast<const u16x8*>(kn + (int64_t)u * D);
  const u16x8* sv = reinterpret_cast<const u16x8*>(vn + (int64_t)u * D);
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int pc = min(tid + 256 * i, np - 1);
    bk[i] = sk[pc];
    bv[i] = sv[pc];
  }
  const int weff = min(steps + 1, W);
  const int nold = (weff - 1) * G;
  const int c4 = min(4 * l, r - 4);
  const bool cok = 4 * l < r;
  const int64_t pe = (int64_t)Lcur - d.nrec;  // candidate entering the compressed set
  const uint16_t* cep = (const uint16_t*)c.coef_k + ((int64_t)u * c.Lmax + max(pe, (int64_t)0)) * r + c4;
  const uint2 cer = *reinterpret_cast<const uint2*>(cep);
  constexpr int RB = 16;  // window rows per wave and batch
  f32x4 qv[RB];
  float2 st = make_float2(0.f, 0.f);
  auto row_of = [&](int o, int* sl, int* g) {
    const int i = 1 + o / G;
    *g = o % G;
    *sl = wrap_slot(steps - i, W);
  };
  auto issue = [&](int m0) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      int sl, g;
      row_of(min(wv + 4 * (m0 + i), max(nold - 1, 0)), &sl, &g);
      qv[i] = *reinterpret_cast<const f32x4*>(c.qwin + (((int64_t)u * W + sl) * G + g) * r + c4);
    }
    int sl, g;
    row_of(min(wv + 4 * (m0 + (l & (RB - 1))), max(nold - 1, 0)), &sl, &g);
    st = *reinterpret_cast<const float2*>(rowstat_of(c, u) + (sl * G + g) * 2);
  };
  if (nold > 0) issue(0);
  u16x8* dk = reinterpret_cast<u16x8*>((uint16_t*)c.ring_k + ((int64_t)u * d.nrec + rs) * D);
  u16x8* dv = reinterpret_cast<u16x8*>((uint16_t*)c.ring_v + ((int64_t)u * d.nrec + rs) * D);
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int pc = tid + 256 * i;
    if (pc < np) {
      dk[pc] = bk[i];
      dv[pc] = bv[i];
    }
  }
  if (nold <= 0) return;
  const float ce0 = cok ? bf2f((uint16_t)(cer.x & 0xffffu)) : 0.f, ce1 = cok ? bf2f((uint16_t)(cer.x >> 16)) : 0.f;
  const float ce2 = cok ? bf2f((uint16_t)(cer.y & 0xffffu)) : 0.f, ce3 = cok ? bf2f((uint16_t)(cer.y >> 16)) : 0.f;
  for (int m0 = 0; wv + 4 * m0 < nold; m0 += RB) {
    if (m0 > 0) issue(m0);
    float zl = 0.f;
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      float z = (qv[i][0] * ce0 + qv[i][1] * ce1) + (qv[i][2] * ce2 + qv[i][3] * ce3);
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) z += __shfl_xor(z, m);
      if (l == i) zl = z;
    }
    const int o = wv + 4 * (m0 + l);
    if (l < RB && o < nold) {
      int sl, g;
      row_of(o, &sl, &g);
      const float z = zl * qscale;
      const float mn = fmaxf(st.x, z);
      *reinterpret_cast<float2*>(rowstat_of(c, u) + (sl * G + g) * 2) =
          make_float2(mn, st.y * exp2f(st.x - mn) + exp2f(z - mn));
    }
  }
}

__global__ __launch_bounds__(256) void k_prologue_mfma(Dims d, CachePtrs c, const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ kn,
                                                       const uint16_t* __restrict__ vn, DecodeWs w,
                                                       float qscale, float ascale, int ncb) {
  const int b = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  const int l = tid & 63, wv = tid >> 6, n16 = l & 15, kq = l >> 4;
  const int D = d.D, r = d.r, G = d.G, W = d.W, dh = d.dh, Hq = d.Hq;
  const int32_t Lcur = c.lens[2 * u], steps = c.lens[2 * u + 1];
  const bool live = (int64_t)Lcur < c.Lmax;
  if (b == 0 && tid == 0) {
    w.stepinfo[4 * u + 0] = Lcur;
    w.stepinfo[4 * u + 1] = steps;
    w.stepinfo[4 * u + 2] = live ? 0 : 1;
    w.stepinfo[4 * u + 3] = 0;
  }
  if (b == ncb) {
    if (live) prologue_state_bf16(d, c, kn, vn, qscale, u, tid, Lcur, steps);
    return;
  }
  __shared__ float red[4][16][17];  // the waves' sums over their heads
  constexpr int KSW = 8;            // k-steps of 32 channels per wave and round
  const bf16x8 zero8 = __builtin_bit_cast(bf16x8, u16x8{});
  const int col = 16 * b + n16;     // < r (r is a multiple of 32)
  const uint16_t* bt = bkt_of(c, u) + (int64_t)col * D;
  const int g1 = min(max(n16 - 1, 0), G - 1);  // query of A row n16 (rows past G: zero)
  f32x4 run = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 256 * wv; c0 < D; c0 += 1024) {
    bf16x8 xa[KSW], xb[KSW];
#pragma unroll
    for (int ks = 0; ks < KSW; ++ks) {
      const int kk = c0 + 32 * ks + 8 * kq;
      const int kc = kk < D ? kk : 0;  // k-steps past D' are skipped below
      xb[ks] = ld_bf16x8(bt + kc);
      const uint16_t* src = n16 == 0 ? kn + (int64_t)u * D + kc
                                     : q + ((int64_t)u * Hq + (kc / dh) * G + g1) * dh + kc % dh;
      xa[ks] = ld_bf16x8(src);
    }
    if (n16 > G) {
#pragma unroll
      for (int ks = 0; ks < KSW; ++ks) xa[ks] = zero8;
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSW; ++ks) {
      if (c0 + 32 * ks >= D) break;
      acc = mfma16x16x32(xa[ks], xb[ks], acc);
      if ((32 * (ks + 1)) % dh == 0) {  // last k-step of head (c0 + 32 ks) / dh (c0 % d_h == 0)
        // lane: rows 4 kq + i, column col; rows 1 .. G are the head's projected queries
        if (live) {
          const int h = (c0 + 32 * ks) / dh;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int v = 4 * kq + i;
            if (v >= 1 && v <= G) {
              const float x = acc[i] * ascale;
              uint16_t* ql = reinterpret_cast<uint16_t*>(w.qlat) + ((int64_t)u * Hq + h * G + v - 1) * 2 * r + col;
              const uint16_t hb = f2bf(x);
              ql[0] = hb;
              ql[r] = f2bf(x - bf2f(hb));
            }
          }
        }
        run += acc;
        acc = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wv][4 * kq + i][n16] = run[i];
  __syncthreads();
  if (!live || tid >= (1 + G) * 16) return;
  // thread: row v, column cl
  const int v = tid >> 4, cc = tid & 15, cl = 16 * b + cc;
  const float sum = (red[0][v][cc] + red[1][v][cc]) + (red[2][v][cc] + red[3][v][cc]);
  if (v == 0) {
    ((uint16_t*)c.coef_k)[((int64_t)u * c.Lmax + Lcur) * r + cl] = f2bf(sum);
  } else {
    const int64_t row = ((int64_t)u * W + steps % W) * G + (v - 1);
    c.qwin[row * r + cl] = sum;
    const float x = sum * qscale;  // MFMA operands of the latent scoring
    const uint16_t hb = f2bf(x);
    uint16_t* qs = qsplit_of(c, u) + ((steps % W) * G + (v - 1)) * 2 * r;
    qs[cl] = hb;
    qs[r + cl] = f2bf(x - bf2f(hb));
  }
}

// c^V(new) = v_cat . B^V, 32 columns per block of 1024 threads: thread
// (row group tid / 4, column octet tid % 4) takes rows rg, rg + 256, ...;
// row-group sums meet over lanes, then over the 16 waves in LDS.  Blocks
// of the top-k launch (see the prologue).
__device__ __forceinline__ void value_coef_block(const Dims& d, const CachePtrs& c, const DecodeWs& w,
                                                 const uint16_t* __restrict__ vn, int u, int vb, int tid) {
  __shared__ float vred[16 * 32];
  const int32_t* si = w.stepinfo + 4 * u;
  if (si[2]) return;  // no append
  const int64_t p = si[0];
  const int D = d.D, r = d.rv;
  const int cq = tid & 3, rg = tid >> 2;
  const int col = min(32 * vb + 8 * cq, r - 8);
  const uint16_t* B = (const uint16_t*)c.basis_v + (int64_t)u * D * r;
  const uint16_t* x = vn + (int64_t)u * D;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int r0 = 0; r0 < D; r0 += 1024) {
    u16x8 bw[4];
    float xv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = r0 + rg + 256 * i;
      bw[i] = *reinterpret_cast<const u16x8*>(B + (int64_t)min(row, D - 1) * r + col);
      xv[i] = row < D ? bf2f(x[row]) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(xv[i], bf2f(bw[i][e]), acc[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int m = 4; m < 64; m <<= 1) acc[e] += __shfl_xor(acc[e], m);
  const int l = tid & 63, wv = tid >> 6;
  if (l < 4)
#pragma unroll
    for (int e = 0; e < 8; ++e) vred[wv * 32 + 8 * l + e] = acc[e];
  __syncthreads();
  if (tid < 32) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += vred[i * 32 + tid];
    const int cl = 32 * vb + tid;
    if (cl < r) ((uint16_t*)c.coef_v)[((int64_t)u * c.Lmax + p) * r + cl] = f2bf(s);
  }
}

hipError_t launch_prologue(const Dims& d, int U, const void* q, const void* k_new,
                           const void* v_new, const CachePtrs& c, const DecodeWs& w,
                           hipStream_t st) {
  const int vec = d.dtype == 0 ? 4 : 8;
  const int ncb = (d.r + 4 * vec - 1) / (4 * vec);
  const int ncbv = (d.rv + 4 * vec - 1) / (4 * vec);
  const int nvec = 1 + d.G;
  size_t lds = ((size_t)nvec * d.D + 16 * nvec * 4 * vec) * sizeof(float);
  if (lds < (size_t)d.r * sizeof(float)) lds = (size_t)d.r * sizeof(float);
  if (lds < (size_t)d.rv * sizeof(float)) lds = (size_t)d.rv * sizeof(float);
  const size_t lq = ((size_t)d.G * d.dh + (size_t)4 * d.G * 32 * vec) * sizeof(float);
  if (lds < lq) lds = lq;
  dim3 grid(ncb + ncbv + 1 + d.Hkv, U);
  const float qscale = kLog2e / sqrtf((float)d.r);
  const float ascale = kLog2e / sqrtf((float)d.dh);
  if (d.dtype == 0) {
    hipLaunchKernelGGL(k_prologue<float>, grid, dim3(256), lds, st, d, c, (const float*)q,
                       (const float*)k_new, (const float*)v_new, w, qscale, ascale, ncb, ncbv);
  } else if (prologue_fused(d)) {
    const int ncb16 = d.r / 16;
    hipLaunchKernelGGL(k_prologue_mfma, dim3(ncb16 + 1, U), dim3(256), 0, st, d, c, (const uint16_t*)q,
                       (const uint16_t*)k_new, (const uint16_t*)v_new, w, qscale, ascale, ncb16);
  } else {
    hipLaunchKernelGGL(k_prologue<uint16_t>, grid, dim3(256), lds, st, d, c, (const uint16_t*)q,
                       (const uint16_t*)k_new, (const uint16_t*)v_new, w, qscale, ascale, ncb, ncbv);
  }
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// latent scoring, bf16 storage: grid (nsplit, U), 512 threads (8 waves, two
// per SIMD).  A unit's 64-position tiles are dealt round-robin over its
// nsplit blocks.
//
// Key coefficients stream through a 4-stage LDS ring, 64 positions per tile,
// filled by direct global->LDS loads (global_load_lds_dwordx4), three tiles
// ahead, without spending registers on them.  One block barrier per tile: a
// wave waits (vmcnt) for its own pieces of tile t, and after the barrier
// every piece of t has landed and every wave is done with tile t-1, whose
// stage then takes the request for tile t+3.  The stages are distinct LDS
// objects and the waits are asm statements with a memory clobber, so the
// compiler's own LDS-DMA tracking adds no full wait; the MFMA operand reads
// are inline asm (lds_read8) for the same reason.  Within a position row the
// 16-byte chunks are XOR-swizzled by the position index, so the operand
// reads of 16 consecutive positions hit distinct banks.
//
// Work units: MFMA 16x16x32 tiles of (16 window rows, 16 tile positions).
// Window rows are in "age order" (row rho = i*G + g is query head-group g of
// the step i steps ago; rows 0..G-1 are the current step), in NRB blocks of
// 16.  The row blocks form NG groups of RBW; wave w owns group w % NG (its A
// operands stay in registers: the fp32 query coefficients, scaled by
// log2(e)/sqrt(r), as bf16 hi + lo parts, two MFMAs per step, ~16 mantissa
// bits) and the column blocks w / NG + (8 / NG) j of every tile.  The
// K-index permutation gives lane (n, kq) of both operands the chunks
// 4 ks + kq.  Per position, a group's probability sum over its rows lands in
// an LDS segment buffer; every 8 tiles the block sums the groups and stores
// the segment, together with the current rows' logits.
// --------------------------------------------------------------------------
// cache policy of the scan's direct global->LDS loads: non-temporal.  The
// key coefficients are read once per step; streamed this way they run
// faster (7.0 against 6.4 TB/s measured on a plain 1 GiB stream) and do not
// evict the step's other data (bases, gathered rows, partial scores) from
// the L2 and Infinity Cache, which the kernels after the scan then hit.
constexpr int kScanPolicy = 2;   // the instruction's nt bit
constexpr int kScoreTP = 64;     // positions per tile
constexpr int kScoreSeg = 512;   // positions per output segment (buffered in LDS)
constexpr int kScoreNST = 4;     // LDS ring stages (3 tiles in flight)
constexpr int kScoreWaves = 8;

template <int KS>
struct ScoreStage {
  __attribute__((aligned(16))) uint8_t b[kScoreTP * KS * 32];  // 64 rows x r bf16
};

// sum over the four 16-lane rows of a wave, result in every lane
__device__ __forceinline__ float sum_lane_rows(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int KS, int NG, int RBW>
__global__ __launch_bounds__(512) void k_score_bf16(Dims d, CachePtrs c, DecodeWs w) {
  constexpr int r = KS * 16;
  constexpr int ROWB = r * 2;                  // bytes per coefficient row
  constexpr int TILEB = kScoreTP * ROWB;
  constexpr int NCH = r / 8;                   // 16-byte chunks per row
  constexpr int SWZ = (NCH % 16 == 0) ? 15 : (NCH % 8 == 0) ? 7 : (NCH % 4 == 0) ? 3 : 0;
  constexpr int DW = TILEB / 1024 < kScoreWaves ? TILEB / 1024 : kScoreWaves;  // DMA waves
  constexpr int PW = TILEB / (DW * 1024);      // DMA instructions per DMA wave per tile
  constexpr int SEGT = kScoreSeg / kScoreTP;   // tiles per segment
  constexpr int NKS = r / 32;                  // MFMA K steps
  constexpr int WPG = kScoreWaves / NG;        // waves per row-block group
  constexpr int NUW = WPG >= 4 ? 1 : 4 / WPG;  // column blocks per wave and tile
  constexpr int KB = (RBW == 2 && NKS > 6) ? 4 : 8;  // operand reads per batch (register budget)
  static_assert(TILEB % (DW * 1024) == 0, "tile must split into 1 KB pieces per wave");
  static_assert(NCH % 4 == 0, "rank must be a multiple of 32");
  static_assert(kScoreSeg % 256 == 0, "flush: 4 positions per lane");
  __shared__ ScoreStage<KS> st0, st1, st2, st3;
  __shared__ __attribute__((aligned(16))) float segred[NG][kScoreSeg];   // per group partial scores
  __shared__ __attribute__((aligned(16))) float segspill[8][kScoreSeg];  // current rows' logits

  const int split = blockIdx.x, u = blockIdx.y;
  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, n16 = l & 15, kq = l >> 4;
  const int32_t* si = w.stepinfo + 4 * u;
  if (si[2]) return;
  const int Lcur = si[0], steps = si[1];
  const int G = d.G, W = d.W, s = d.s;
  const int weff = min(steps + 1, W);
  const int nrows = weff * G;
  const int nrb = (W * G + 15) / 16;
  const int ngr = (nrb + RBW - 1) / RBW;       // groups holding row blocks
  const int64_t cend = (int64_t)Lcur + 1 - d.nrec;
  // the unit's candidate tiles dealt round-robin over the splits: tile t of
  // this block is the unit's tile t * nsplit + split, so at any moment the
  // unit's blocks stream neighbouring tiles
  const int64_t ntu = (max(cend - s, (int64_t)0) + kScoreTP - 1) / kScoreTP;
  const int ntl = ntu > split ? (int)((ntu - split + w.nsplit - 1) / w.nsplit) : 0;

  // ---- DMA of one tile into a stage ----------------------------------------
  // Piece q of this lane: LDS row pl, slot sl holds global chunk sl ^ (pl & SWZ);
  // the lane offsets are the same for every tile, only the tile base moves.
  const uint8_t* cbase = reinterpret_cast<const uint8_t*>(
      (const uint16_t*)c.coef_k + (int64_t)u * c.Lmax * r);
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  uint32_t qoff[PW];
#pragma unroll
  for (int q = 0; q < PW; ++q) {
    const int Q = (wvu * PW + q) * 64 + l;
    const int pl = Q / NCH, slot = Q % NCH;
    qoff[q] = (uint32_t)(pl * ROWB + ((slot ^ (pl & SWZ)) << 4));
  }
  auto issue = [&](int64_t p0, uint8_t* stage) {
    if (DW < kScoreWaves && wvu >= DW) return;
    const uint8_t* tb = cbase + p0 * ROWB;
    if (p0 + kScoreTP <= c.Lmax) {
#pragma unroll
      for (int q = 0; q < PW; ++q)
        __builtin_amdgcn_global_load_lds(
            (const void*)(tb + qoff[q]),
            (__attribute__((address_space(3))) void*)(stage + (wvu * PW + q) * 1024), 16, 0, kScanPolicy);
    } else {  // last tile of the buffer: clamp rows
#pragma unroll
      for (int q = 0; q < PW; ++q) {
        const int pl = ((wvu * PW + q) * 64 + l) / NCH;
        const int64_t pos = min(p0 + pl, c.Lmax - 1);
        __builtin_amdgcn_global_load_lds(
            (const void*)(cbase + pos * ROWB + (qoff[q] - pl * ROWB)),
            (__attribute__((address_space(3))) void*)(stage + (wvu * PW + q) * 1024), 16, 0, kScanPolicy);
      }
    }
  };
  // the block's tiles: t covers positions tp(t) + [0, TP); requests past the
  // last tile re-read it (harmless, keeps the ring's count uniform)
  auto tp = [&](int t) {
    return (int64_t)s + ((int64_t)min(t, max(ntl - 1, 0)) * w.nsplit + split) * kScoreTP;
  };
  if (ntl > 0) {  // prime the ring before the operand loads below
    issue(tp(0), st0.b);
    issue(tp(1), st1.b);
    issue(tp(2), st2.b);
  }

  // ---- this wave's row blocks and column blocks ----------------------------
  const int rg = wv % NG, cw = wv / NG;
  const bool wact = rg < ngr && cw < 4;
  // A fragments: row rho = 16 (RBW rg + b) + n16 of the window (rows past it -> 0)
  bf16x8 ahi[RBW][NKS], alo[RBW][NKS];
  // older rows' log-normaliser m + log2(S) for this lane's accumulator rows
  // 16 rb + 4 kq + i; current and invalid rows get +huge (probability 0)
  float mrow[RBW][4];
#pragma unroll
  for (int b = 0; b < RBW; ++b) {
    const int rb = RBW * rg + b;
    const int rho = 16 * rb + n16;
    const bool valid = wact && rho < nrows;
    const int rv = valid ? rho : 0;
    const int i = rv / G, g = rv % G;
    const int sl = wrap_slot(steps - i, W);
    const uint16_t* qh = qsplit_of(c, u) + ((sl * G + g) * 2) * r;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 h = ld_bf16x8(qh + (4 * ks + kq) * 8);
      const bf16x8 lo = ld_bf16x8(qh + r + (4 * ks + kq) * 8);
      ahi[b][ks] = valid ? h : __builtin_bit_cast(bf16x8, u16x8{});
      alo[b][ks] = valid ? lo : __builtin_bit_cast(bf16x8, u16x8{});
    }
    float2 stv[4];
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) {
      const int rr = 16 * rb + 4 * kq + i2;
      const int rv2 = rr < nrows ? rr : 0;
      const int ii = rv2 / G, g2 = rv2 % G;
      const int sl2 = wrap_slot(steps - ii, W);
      stv[i2] = *reinterpret_cast<const float2*>(rowstat_of(c, u) + (sl2 * G + g2) * 2);
    }
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) {
      const int rr = 16 * rb + 4 * kq + i2;
      const bool old_row = wact && rr >= G && rr < nrows;
      mrow[b][i2] = old_row ? stv[i2].x + log2f(stv[i2].y) : FLT_MAX;
    }
  }
  // current row g = wave index (g < G): running (max, sum) over the
  // positions this lane flushes
  float nm = -INFINITY, ns = 0.f;

  // tile t of the block (positions tp(t) + pl; segment slot (t % SEGT)*TP + pl)
  auto compute = [&](int t, const uint8_t* stage) {
    if (!wact) return;
    const uint32_t sbase = lds_offset(stage);
#pragma unroll 1
    for (int j = 0; j < NUW; ++j) {
      const int cb = cw + WPG * j;  // < 4: cw < min(WPG, 4) and WPG * NUW = 4 or NUW = 1
      const int pl = 16 * cb + n16;  // position row of this lane's B operand
      const uint32_t rbase = sbase + pl * ROWB;
      const int sw = pl & SWZ;
      f32x4 acc[RBW];
#pragma unroll
      for (int b = 0; b < RBW; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < NKS; k0 += KB) {
        uint32_t ad[KB];
        bf16x8 bb[KB];
#pragma unroll
        for (int kk = 0; kk < KB; ++kk)
          ad[kk] = rbase + (((4 * min(k0 + kk, NKS - 1) + kq) ^ sw) << 4);
        if constexpr (KB == 8)
          lds_read8(ad, bb);
        else
          lds_read4(ad, bb);
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
          if (k0 + kk < NKS) {
#pragma unroll
            for (int b = 0; b < RBW; ++b) acc[b] = mfma16(ahi[b][k0 + kk], bb[kk], acc[b]);
#pragma unroll
            for (int b = 0; b < RBW; ++b) acc[b] = mfma16(alo[b][k0 + kk], bb[kk], acc[b]);
          }
        }
      }
      // arguments are <= 0 (or -huge for excluded rows): the hardware exp2
      // is exact enough and its flush of tiny results is harmless here
      float ps = 0.f;
#pragma unroll
      for (int b = 0; b < RBW; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) ps += __builtin_amdgcn_exp2f(acc[b][i] - mrow[b][i]);
      ps = sum_lane_rows(ps);
      const int sp = (t % SEGT) * kScoreTP + pl;  // position within the segment
      if (l < 16) segred[rg][sp] = ps;
      if (rg == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * kq + i < G) segspill[4 * kq + i][sp] = acc[0][i];
      }
    }
  };

  float* partial = w.partial + (int64_t)u * w.Lc_cap - s;           // [position]
  float* spill = w.spill + (int64_t)u * G * w.Lc_cap - s;            // [row][position]
  // flush of segment sg (the block's tiles SEGT sg ..), four positions per
  // lane and one 16-byte store per wave: the last wave stores the group sums,
  // wave g < G the current row g's logits (and folds them into its running
  // max and sum); positions from cend on are not stored
  auto flush = [&](int sg) {
#pragma unroll
    for (int e0 = 4 * l; e0 < kScoreSeg; e0 += 256) {
    const int t = sg * SEGT + e0 / kScoreTP;
    const int64_t pos = tp(t) + e0 % kScoreTP;
    const int ne = t < ntl ? (int)min((int64_t)4, cend - pos) : 0;
    if (wv == kScoreWaves - 1 && ne > 0) {
      f32x4 sum = *reinterpret_cast<const f32x4*>(&segred[0][e0]);
      for (int q2 = 1; q2 < ngr; ++q2) sum += *reinterpret_cast<const f32x4*>(&segred[q2][e0]);
      if (ne == 4) {
        *reinterpret_cast<f32x4*>(partial + pos) = sum;
      } else {
        for (int e = 0; e < ne; ++e) partial[pos + e] = sum[e];
      }
    }
    if (wv < G && ne > 0) {
      const f32x4 z = *reinterpret_cast<const f32x4*>(&segspill[wv][e0]);
      float* dst = spill + (int64_t)wv * w.Lc_cap + pos;
      if (ne == 4) {
        *reinterpret_cast<f32x4*>(dst) = z;
      } else {
        for (int e = 0; e < ne; ++e) dst[e] = z[e];
      }
      float mx = nm;
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = e < ne ? fmaxf(mx, z[e]) : mx;
      float acc = ns * __builtin_amdgcn_exp2f(nm - mx);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc += e < ne ? __builtin_amdgcn_exp2f(z[e] - mx) : 0.f;
      nm = mx;
      ns = acc;
    }
    }
  };
  // tile t lives in stage t % 4.  At the wait of step t the wave's requests
  // issued after tile t are exactly tiles t+1 and t+2 (flush stores go out
  // before the next request), so vmcnt(2 PW) means tile t has landed.
  constexpr int kWaitN = (kScoreNST - 2) * PW;
  for (int t = 0; t < ntl; t += kScoreNST) {
#define KVLR_SCORE_STEP(k, SREAD, SNEXT)                                                    \
    if (t + k >= ntl) break;                                                                \
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kWaitN) : "memory");  \
    if ((t + k) % SEGT == 0 && t + k > 0) {                                                 \
      flush((t + k) / SEGT - 1);                                                            \
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");                       \
    }                                                                                       \
    issue(tp(t + k + 3), SNEXT);                                                            \
    compute(t + k, SREAD);
    KVLR_SCORE_STEP(0, st0.b, st3.b)
    KVLR_SCORE_STEP(1, st1.b, st0.b)
    KVLR_SCORE_STEP(2, st2.b, st1.b)
    KVLR_SCORE_STEP(3, st3.b, st2.b)
#undef KVLR_SCORE_STEP
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (ntl > 0) flush((ntl - 1) / SEGT);

  // current row g's (max, sum) over this split, from the lanes of wave g
  if (wv < G) {
    float m = nm, sm = ns;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(sm, o);
      const float mx = fmaxf(m, m2);
      const float a = (m == -INFINITY) ? 0.f : sm * exp2f(m - mx);
      const float b2 = (m2 == -INFINITY) ? 0.f : s2 * exp2f(m2 - mx);
      sm = a + b2;
      m = mx;
    }
    if (l == 0) {
      float* tst = w.tilestat + ((int64_t)u * w.nsplit + split) * G * 2;
      tst[wv * 2 + 0] = m;
      tst[wv * 2 + 1] = sm;
    }
  }
}

// --------------------------------------------------------------------------
// latent scoring, bf16 storage, products on MFMA 32x32x16 (on gfx950 this
// shape runs at the full bf16 rate, twice the flops per cycle of 16x16x32).
// grid (nsplit, U), 512 threads (8 waves, two per SIMD); the unit's tiles,
// the 4-stage LDS ring and its direct global->LDS loads, the waits and the
// one barrier per tile are those of k_score_bf16 above.
//
// Work of a tile (64 positions): combos (row block rb of 32 window rows,
// column block cb of 32 positions), 2 NRB of them (6 or 8), one per wave.  A
// wave keeps its row block's query operands for all k-steps in registers
// (bf16 hi + lo, ~16 mantissa bits) and reads the B operands (the
// positions' key coefficients, K-contiguous 16-byte chunks of the swizzled
// rows) from the tile's stage.  Lane l's accumulator i holds row
// 8 (i / 4) + 4 (l / 32) + i % 4 of the row block for position l % 32.  The
// wave turns the older rows into probabilities with their running
// (max, sum), sums them over its rows (the lane halves meet through a
// permlane32 swap) into the segment buffer, and, for row block 0, writes
// the current rows' logits to the spill buffer.  Every kScoreSeg positions
// the block adds the row blocks' sums, stores the segment and folds the
// current rows' logits into their running (max, sum).
//
// Splitting the rank of a combo over several waves (for W G <= 64) was
// measured slower than k_score_bf16, and with a full-rank share per wave
// r = 256 spills; the dispatch below takes this kernel only for 3 or 4 row
// blocks and r <= 192.
// --------------------------------------------------------------------------
template <int NKS, int NRB, int GM>
__global__ __launch_bounds__(512) void k_score_mfma32(Dims d, CachePtrs c, DecodeWs w) {
  constexpr int r = NKS * 16;
  constexpr int ROWB = r * 2;
  constexpr int TILEB = kScoreTP * ROWB;
  constexpr int NCH = r / 8;
  constexpr int SWZ = (NCH % 16 == 0) ? 15 : (NCH % 8 == 0) ? 7 : (NCH % 4 == 0) ? 3 : 1;
  constexpr int DW = TILEB / 1024 < kScoreWaves ? TILEB / 1024 : kScoreWaves;
  constexpr int PW = TILEB / (DW * 1024);
  constexpr int SEGT = kScoreSeg / kScoreTP;
  constexpr int COMBOS = 2 * NRB;
  constexpr int KB = NKS % 4 == 0 ? 4 : NKS % 2 == 0 ? 2 : 1;
  static_assert(TILEB % (DW * 1024) == 0, "tile must split into 1 KB pieces per wave");
  static_assert(COMBOS <= kScoreWaves, "one combo per wave");
  __shared__ ScoreStage<NKS> st0, st1, st2, st3;
  __shared__ __attribute__((aligned(16))) float segred[NRB][kScoreSeg];   // row blocks' partial scores
  __shared__ __attribute__((aligned(16))) float segspill[GM][kScoreSeg];  // current rows' logits
  static_assert(sizeof(ScoreStage<NKS>) == TILEB, "stage size");

  const int split = blockIdx.x, u = blockIdx.y;
  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63;
  const int32_t* si = w.stepinfo + 4 * u;
  if (si[2]) return;
  const int Lcur = si[0], steps = si[1];
  const int G = d.G, W = d.W, s = d.s;
  const int weff = min(steps + 1, W);
  const int nrows = weff * G;
  const int64_t cend = (int64_t)Lcur + 1 - d.nrec;
  const int64_t ntu = (max(cend - s, (int64_t)0) + kScoreTP - 1) / kScoreTP;
  const int ntl = ntu > split ? (int)((ntu - split + w.nsplit - 1) / w.nsplit) : 0;

  // ---- DMA of one tile into a stage (as in k_score_bf16)
  const uint8_t* cbase = reinterpret_cast<const uint8_t*>(
      (const uint16_t*)c.coef_k + (int64_t)u * c.Lmax * r);
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  uint32_t qoff[PW];
#pragma unroll
  for (int q = 0; q < PW; ++q) {
    const int Q = (wvu * PW + q) * 64 + l;
    const int pl = Q / NCH, slot = Q % NCH;
    qoff[q] = (uint32_t)(pl * ROWB + ((slot ^ (pl & SWZ)) << 4));
  }
  auto issue = [&](int64_t p0, uint8_t* stage) {
    if (DW < kScoreWaves && wvu >= DW) return;
    const uint8_t* tb = cbase + p0 * ROWB;
    if (p0 + kScoreTP <= c.Lmax) {
#pragma unroll
      for (int q = 0; q < PW; ++q)
        __builtin_amdgcn_global_load_lds(
            (const void*)(tb + qoff[q]),
            (__attribute__((address_space(3))) void*)(stage + (wvu * PW + q) * 1024), 16, 0, kScanPolicy);
    } else {  // last tile of the buffer: clamp rows
#pragma unroll
      for (int q = 0; q < PW; ++q) {
        const int pl = ((wvu * PW + q) * 64 + l) / NCH;
        const int64_t pos = min(p0 + pl, c.Lmax - 1);
        __builtin_amdgcn_global_load_lds(
            (const void*)(cbase + pos * ROWB + (qoff[q] - pl * ROWB)),
            (__attribute__((address_space(3))) void*)(stage + (wvu * PW + q) * 1024), 16, 0, kScanPolicy);
      }
    }
  };
  auto tp = [&](int t) {
    return (int64_t)s + ((int64_t)min(t, max(ntl - 1, 0)) * w.nsplit + split) * kScoreTP;
  };
  if (ntl > 0) {
    issue(tp(0), st0.b);
    issue(tp(1), st1.b);
    issue(tp(2), st2.b);
  }

  // ---- this wave's combo
  const int combo = wv;
  const bool wact = wv < COMBOS;
  const int rb = combo >> 1, cb = combo & 1;
  const int p = l & 31, hk = l >> 5;
  bf16x8 ahi[NKS], alo[NKS];
  float mrow[16];
  {
    const int rho = 32 * rb + p;
    const bool valid = wact && rho < nrows;
    const int rv = valid ? rho : 0;
    const int sl = wrap_slot(steps - rv / G, W);
    const uint16_t* qh = qsplit_of(c, u) + ((sl * G + rv % G) * 2) * r;
#pragma unroll
    for (int k = 0; k < NKS; ++k) {
      const bf16x8 h = ld_bf16x8(qh + 16 * k + 8 * hk);
      const bf16x8 lo = ld_bf16x8(qh + r + 16 * k + 8 * hk);
      ahi[k] = valid ? h : __builtin_bit_cast(bf16x8, u16x8{});
      alo[k] = valid ? lo : __builtin_bit_cast(bf16x8, u16x8{});
    }
    const float* rst = rowstat_of(c, u);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rr = 32 * rb + acc_row32(i, l);
      const bool old_row = wact && rr >= G && rr < nrows;
      const int r2 = old_row ? rr : G;
      const float2 stv = *reinterpret_cast<const float2*>(rst + (wrap_slot(steps - r2 / G, W) * G + r2 % G) * 2);
      mrow[i] = old_row ? stv.x + log2f(stv.y) : FLT_MAX;
    }
  }
  // current row g (< G <= GM): accumulator g % 4 of the lanes with hk = g / 4
  // in the waves of row block 0; wave g < G keeps the row's running
  // (max, sum) over the positions it flushes
  float nm = -INFINITY, ns = 0.f;
  float* partial = w.partial + (int64_t)u * w.Lc_cap - s;
  float* spill = w.spill + (int64_t)u * G * w.Lc_cap - s;

  auto compute = [&](int t, const uint8_t* stage) {
    f32x16 acc = f32x16{};
    if (wact) {
      const uint32_t rbase = lds_offset(stage) + (32 * cb + p) * ROWB;
      const int sw = (32 * cb + p) & SWZ;
#pragma unroll
      for (int k0 = 0; k0 < NKS; k0 += KB) {
        uint32_t ad[4];
        bf16x8 bb[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          ad[kk] = rbase + (((2 * min(k0 + kk, NKS - 1) + hk) ^ sw) << 4);
        lds_read4(ad, bb);
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
          acc = mfma32x32x16(ahi[k0 + kk], bb[kk], acc);
          acc = mfma32x32x16(alo[k0 + kk], bb[kk], acc);
        }
      }
    }
    if (!wact) return;
    // arguments are <= 0 (or -huge for excluded rows): the hardware exp2
    // is exact enough and its flush of tiny results is harmless here
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) ps += __builtin_amdgcn_exp2f(acc[i] - mrow[i]);
    {
      const auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(ps), __float_as_uint(ps), false, false);
      ps = __uint_as_float(sw2[0]) + __uint_as_float(sw2[1]);
    }
    const int sp = (t % SEGT) * kScoreTP + 32 * cb + p;  // position within the segment
    if (hk == 0) segred[rb][sp] = ps;
    if (rb == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * hk + i < G) segspill[4 * hk + i][sp] = acc[i];
    }
  };

  // flush of segment sg, four positions per lane and one 16-byte store per
  // wave: the last wave stores the row blocks' summed scores, wave g < G the
  // current row g's logits (and folds them into its running max and sum);
  // positions from cend on are not stored
  auto flush = [&](int sg) {
#pragma unroll
    for (int e0 = 4 * l; e0 < kScoreSeg; e0 += 256) {
      const int t = sg * SEGT + e0 / kScoreTP;
      const int64_t pos = tp(t) + e0 % kScoreTP;
      const int ne = t < ntl ? (int)min((int64_t)4, cend - pos) : 0;
      if (wv == kScoreWaves - 1 && ne > 0) {
        f32x4 sum = *reinterpret_cast<const f32x4*>(&segred[0][e0]);
#pragma unroll
        for (int q2 = 1; q2 < NRB; ++q2) sum += *reinterpret_cast<const f32x4*>(&segred[q2][e0]);
        if (ne == 4) {
          *reinterpret_cast<f32x4*>(partial + pos) = sum;
        } else {
          for (int e = 0; e < ne; ++e) partial[pos + e] = sum[e];
        }
      }
      if (wv < G && ne > 0) {
        const f32x4 z = *reinterpret_cast<const f32x4*>(&segspill[wv][e0]);
        float* dst = spill + (int64_t)wv * w.Lc_cap + pos;
        if (ne == 4) {
          *reinterpret_cast<f32x4*>(dst) = z;
        } else {
          for (int e = 0; e < ne; ++e) dst[e] = z[e];
        }
        float mx = nm;
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = e < ne ? fmaxf(mx, z[e]) : mx;
        float acc = ns * __builtin_amdgcn_exp2f(nm - mx);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc += e < ne ? __builtin_amdgcn_exp2f(z[e] - mx) : 0.f;
        nm = mx;
        ns = acc;
      }
    }
  };
  constexpr int kWaitN = (kScoreNST - 2) * PW;
  for (int t = 0; t < ntl; t += kScoreNST) {
#define KVLR_SCORE32_STEP(k, SREAD, SNEXT)                                                  \
    if (t + k >= ntl) break;                                                                \
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kWaitN) : "memory");  \
    if ((t + k) % SEGT == 0 && t + k > 0) {                                                 \
      flush((t + k) / SEGT - 1);                                                            \
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");                       \
    }                                                                                       \
    issue(tp(t + k + 3), SNEXT);                                                            \
    compute(t + k, SREAD);
    KVLR_SCORE32_STEP(0, st0.b, st3.b)
    KVLR_SCORE32_STEP(1, st1.b, st0.b)
    KVLR_SCORE32_STEP(2, st2.b, st1.b)
    KVLR_SCORE32_STEP(3, st3.b, st2.b)
#undef KVLR_SCORE32_STEP
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (ntl > 0) flush((ntl - 1) / SEGT);

  // current row g's (max, sum) over this split, from the lanes of wave g
  if (wv < G) {
    float m = nm, sm = ns;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(sm, o);
      const float mx = fmaxf(m, m2);
      const float a = (m == -INFINITY) ? 0.f : sm * exp2f(m - mx);
      const float b2 = (m2 == -INFINITY) ? 0.f : s2 * exp2f(m2 - mx);
      sm = a + b2;
      m = mx;
    }
    if (l == 0) {
      float* tst = w.tilestat + ((int64_t)u * w.nsplit + split) * G * 2;
      tst[wv * 2 + 0] = m;
      tst[wv * 2 + 1] = sm;
    }
  }
}

// latent scoring, fp32 storage: plain fp32 dot products, one position per
// thread.  The window rows (scaled) sit in LDS; the block's positions are
// taken in runs of P, each run's key-coefficient rows first copied into LDS
// with coalesced loads (rows padded by one float), so every product reads
// LDS.  The G current rows keep their running (max, sum) in registers; the
// block combines them with wave shuffles and one LDS exchange (ms_combine:
// a (max, sum) pair of base-2 softmax statistics merged into (m, s); pairs
// with no mass are skipped).
__device__ __forceinline__ void ms_combine(float& m, float& s, float m2, float s2) {
  if (!(s2 > 0.f)) return;
  if (!(s > 0.f)) {
    m = m2;
    s = s2;
    return;
  }
  const float mx = fmaxf(m, m2);
  s = s * exp2f(m - mx) + s2 * exp2f(m2 - mx);
  m = mx;
}

__global__ __launch_bounds__(256) void k_score_f32(Dims d, CachePtrs c, DecodeWs w, float qscale, int P) {
  const int split = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  const int32_t* si = w.stepinfo + 4 * u;
  if (si[2]) return;
  const int Lcur = si[0], steps = si[1];
  const int G = d.G, W = d.W, s = d.s, r = d.r;
  const int weff = min(steps + 1, W);
  const int nrows = weff * G;
  const int64_t cend = (int64_t)Lcur + 1 - d.nrec;
  const int64_t j0 = s + (int64_t)split * w.chunk;
  const int64_t j1 = min(j0 + (int64_t)w.chunk, cend);
  extern __shared__ float sm[];
  float* qs = sm;                   // [nrows][r]
  float* rm = qs + W * G * r;       // [nrows] max
  float* ri = rm + W * G;           // [nrows] 1/S
  float* red = ri + W * G;          // [4 waves][8 rows][2]
  float* cs = red + 64;             // [P][r + 1] key-coefficient rows of a run
  for (int e = tid; e < nrows * r; e += blockDim.x) {
    const int rho = e / r, k = e % r, i = rho / G, g = rho % G;
    const int sl = wrap_slot(steps - i, W);
    qs[e] = c.qwin[(((int64_t)u * W + sl) * G + g) * r + k] * qscale;
  }
  for (int rho = tid; rho < nrows; rho += blockDim.x) {
    const int i = rho / G, g = rho % G;
    const int sl = wrap_slot(steps - i, W);
    const float* rs = rowstat_of(c, u) + (sl * G + g) * 2;
    rm[rho] = rs[0];
    ri[rho] = rho < G ? 0.f : 1.f / rs[1];
  }
  float nm[8], ns[8];
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    nm[g] = -INFINITY;
    ns[g] = 0.f;
  }
  const float* CK = (const float*)c.coef_k + (int64_t)u * c.Lmax * r;
  const int ld = r + 1;
  for (int64_t p0 = j0; p0 < j1; p0 += P) {
    const int np = (int)min((int64_t)P, j1 - p0);
    __syncthreads();  // the previous run's rows are done (and, first, qs / rm / ri are written)
    for (int e = tid; e < np * r; e += blockDim.x) cs[(e / r) * ld + e % r] = CK[p0 * r + e];
    __syncthreads();
    if (tid < np) {
      const int64_t j = p0 + tid;
      const float* cj = cs + tid * ld;
#pragma unroll
      for (int g = 0; g < 8; ++g) {  // current rows: logits spilled, running (max, sum)
        if (g < G) {
          float z = 0.f;
          for (int k = 0; k < r; ++k) z += qs[g * r + k] * cj[k];
          w.spill[((int64_t)u * G + g) * w.Lc_cap + (j - s)] = z;
          const float mx = fmaxf(nm[g], z);
          ns[g] = ns[g] * exp2f(nm[g] - mx) + exp2f(z - mx);
          nm[g] = mx;
        }
      }
      float ps = 0.f;
      for (int rho = G; rho < nrows; ++rho) {
        float z = 0.f;
        for (int k = 0; k < r; ++k) z += qs[rho * r + k] * cj[k];
        ps += exp2f(z - rm[rho]) * ri[rho];
      }
      w.partial[(int64_t)u * w.Lc_cap + (j - s)] = ps;
    }
  }
  // current rows' (max, sum) over the block: waves by shuffles, then LDS
  const int lane = tid & 63, wv = tid >> 6;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    if (g < G) {
      for (int o = 1; o < 64; o <<= 1) {
        const float m2 = __shfl_xor(nm[g], o), s2 = __shfl_xor(ns[g], o);
        ms_combine(nm[g], ns[g], m2, s2);
      }
      if (lane == 0) {
        red[(wv * 8 + g) * 2] = nm[g];
        red[(wv * 8 + g) * 2 + 1] = ns[g];
      }
    }
  }
  __syncthreads();
  if (tid < G) {
    float m = -INFINITY, S = 0.f;
    for (int x = 0; x < 4; ++x) ms_combine(m, S, red[(x * 8 + tid) * 2], red[(x * 8 + tid) * 2 + 1]);
    float* tst = w.tilestat + ((int64_t)u * w.nsplit + split) * G * 2;
    tst[tid * 2] = m;
    tst[tid * 2 + 1] = S;
  }
}

// LDS of k_score_mfma32<NKS, NRB, GM> (4 stages, segment buffers)
constexpr size_t score32_lds(int nks, int nrb, int gm) {
  return (size_t)4 * kScoreTP * nks * 32 + (size_t)(nrb + gm) * kScoreSeg * 4;
}
// the MFMA 32x32x16 scorer is used for 3 or 4 row blocks of 32 when its LDS
// fits and a wave's query operands (bf16 hi + lo) stay within 12 k-steps
// (96 registers; 16 k-steps spill)
constexpr bool score32_ok(int nks, int nrb, int gm) {
  return nrb >= 3 && nrb <= 4 && nks <= 12 && score32_lds(nks, nrb, gm) <= 160 * 1024;
}

template <int NKS, int NRB, int GM>
static hipError_t launch_score32(const Dims& d, int U, const CachePtrs& c, const DecodeWs& w, hipStream_t st) {
  if constexpr (score32_ok(NKS, NRB, GM)) {
    hipLaunchKernelGGL((k_score_mfma32<NKS, NRB, GM>), dim3(w.nsplit, U), dim3(512), 0, st, d, c, w);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

// MFMA 32x32x16 scorer where it is the faster one (W G in 65..128, r <= 192)
template <int KS>
static bool try_score32(const Dims& d, int U, const CachePtrs& c, const DecodeWs& w, hipStream_t st,
                        hipError_t* e) {
  const int nrb = (d.W * d.G + 31) / 32;
  const int gm = d.G <= 4 ? 4 : 8;
#define KVLR_S32(NRB, GM)                                              \
  if (nrb == NRB && gm == GM && score32_ok(KS, NRB, GM)) {               \
    *e = launch_score32<KS, NRB, GM>(d, U, c, w, st);                   \
    return true;                                                        \
  }
  KVLR_S32(3, 4) KVLR_S32(3, 8) KVLR_S32(4, 4) KVLR_S32(4, 8)
#undef KVLR_S32
  return false;
}

template <int KS>
static hipError_t launch_score_bf16(const Dims& d, int U, const CachePtrs& c, const DecodeWs& w,
                                    hipStream_t st) {
  hipError_t e;
  if (try_score32<KS>(d, U, c, w, st, &e)) return e;
  const int nrb = (d.W * d.G + 15) / 16;
  dim3 grid(w.nsplit, U);
  if (nrb <= 1)
    hipLaunchKernelGGL((k_score_bf16<KS, 1, 1>), grid, dim3(512), 0, st, d, c, w);
  else if (nrb <= 2)
    hipLaunchKernelGGL((k_score_bf16<KS, 2, 1>), grid, dim3(512), 0, st, d, c, w);
  else if (nrb <= 4 && KS == 16)  // r = 256: one row block and two column blocks per wave
    // (measured faster than two row blocks per wave there; slower at r = 192)
    hipLaunchKernelGGL((k_score_bf16<KS, 4, 1>), grid, dim3(512), 0, st, d, c, w);
  else if (nrb <= 4)
    hipLaunchKernelGGL((k_score_bf16<KS, 2, 2>), grid, dim3(512), 0, st, d, c, w);
  else if (nrb <= 8)
    hipLaunchKernelGGL((k_score_bf16<KS, 4, 2>), grid, dim3(512), 0, st, d, c, w);
  else if constexpr (KS <= 8)  // up to 256 window rows: four row blocks per group
    hipLaunchKernelGGL((k_score_bf16<KS, 4, 4>), grid, dim3(512), 0, st, d, c, w);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_score(const Dims& d, int U, const CachePtrs& c, const DecodeWs& w,
                        hipStream_t st) {
  const float qscale = kLog2e / sqrtf((float)d.r);
  if (d.dtype == 0) {
    dim3 grid(w.nsplit, U);
    // runs of P positions: up to 256 (one per thread), within 96 KB of rows
    int P = (int)((96 * 1024 / sizeof(float)) / (d.r + 1));
    P = P > 256 ? 256 : (P < 1 ? 1 : P);
    const size_t lds = ((size_t)d.W * d.G * d.r + 2 * d.W * d.G + 64 + (size_t)P * (d.r + 1)) * sizeof(float);
    static size_t done = 0;
    hipError_t e = allow_lds(&k_score_f32, lds, &done);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_score_f32, grid, dim3(256), lds, st, d, c, w, qscale, P);
    return hipGetLastError();
  }
  switch (d.r) {
    case 128: return launch_score_bf16<8>(d, U, c, w, st);
    case 192: return launch_score_bf16<12>(d, U, c, w, st);
    case 256: return launch_score_bf16<16>(d, U, c, w, st);
    case 64: return launch_score_bf16<4>(d, U, c, w, st);
    case 32: return launch_score_bf16<2>(d, U, c, w, st);
    default: return hipErrorInvalidValue;
  }
}


// --------------------------------------------------------------------------
// pooling: grid (ceil(Lc_cap / kPoolChunk), U), 256 threads.
//   1. merge the current rows' per-split (m, S) (every block; block 0 stores
//      them in rowstat at this step's window slot);
//   2. score[j] = partial[j] + sum_g exp2(z_g[j] - m_g) / S_g for the block's
//      candidates plus a halo of kappa/2 on each side;
//   3. pooled key = max over |d| <= kappa/2 inside the candidates, stored as
//      the float's bit pattern (scores are >= 0, so bits order like values).
// --------------------------------------------------------------------------
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, false);
}
// inclusive prefix sum over the wave: row_shr 1, 2, 4, 8 within rows of 16,
// then row_bcast:15 (rows 1, 3) and row_bcast:31 (rows 2, 3)
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp_i<0x111, 0xF>(x);
  x += dpp_i<0x112, 0xF>(x);
  x += dpp_i<0x114, 0xF>(x);
  x += dpp_i<0x118, 0xF>(x);
  x += dpp_i<0x142, 0xA>(x);
  x += dpp_i<0x143, 0xC>(x);
  return x;
}

// min and max over the wave (xor-pattern DPP, then the four rows), in every lane
__device__ __forceinline__ void wave_minmax_u(unsigned int& mn, unsigned int& mx) {
#define KVLR_MM(CTRL)                                                                          \
  mn = min(mn, (unsigned int)__builtin_amdgcn_update_dpp(0, (int)mn, CTRL, 0xF, 0xF, false)); \
  mx = max(mx, (unsigned int)__builtin_amdgcn_update_dpp(0, (int)mx, CTRL, 0xF, 0xF, false));
  KVLR_MM(0xB1)
  KVLR_MM(0x4E)
  KVLR_MM(0x141)
  KVLR_MM(0x140)
#undef KVLR_MM
  mn = min(min((unsigned int)__builtin_amdgcn_readlane((int)mn, 0), (unsigned int)__builtin_amdgcn_readlane((int)mn, 16)),
           min((unsigned int)__builtin_amdgcn_readlane((int)mn, 32), (unsigned int)__builtin_amdgcn_readlane((int)mn, 48)));
  mx = max(max((unsigned int)__builtin_amdgcn_readlane((int)mx, 0), (unsigned int)__builtin_amdgcn_readlane((int)mx, 16)),
           max((unsigned int)__builtin_amdgcn_readlane((int)mx, 32), (unsigned int)__builtin_amdgcn_readlane((int)mx, 48)));
}

__global__ __launch_bounds__(256) void k_pool(Dims d, CachePtrs c, DecodeWs w,
                                              float* __restrict__ scores_user) {
  const int blk = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  const int G = d.G, s = d.s;
  const int h = d.kappa >> 1;
  const int c0 = blk * kPoolChunk;
  // scores are computed in groups of 8 positions over the chunk plus the
  // pooling halo, rounded out to whole groups: [base, base + 8 ng)
  const int hg = (h + 7) >> 3;
  const int base = c0 - 8 * hg, ng = kPoolChunk / 8 + 2 * hg;
  __shared__ float Mg[8], Ig[8];
  __shared__ float wm[4][8], wsum[4][8];
  __shared__ __attribute__((aligned(16))) float sc[kPoolChunk + 256];
  const int lane = tid & 63, wv = tid >> 6;
  // the split statistics of the current rows and this thread's first group
  // of score inputs (16-byte loads, clamped to the buffer; the candidate
  // count only masks them afterwards) go out before the unit state is read
  const int32_t* si = w.stepinfo + 4 * u;
  const float* tp = w.tilestat + (int64_t)u * w.nsplit * G * 2;
  float2 tv[8];
  {
    const int sp = min(tid, w.nsplit - 1);
#pragma unroll
    for (int g = 0; g < 8; ++g)
      tv[g] = *reinterpret_cast<const float2*>(tp + (sp * G + min(g, G - 1)) * 2);
  }
  const float* part = w.partial + (int64_t)u * w.Lc_cap;
  const float* spill = w.spill + (int64_t)u * G * w.Lc_cap;
  auto gstart = [&](int gi) { return min(max(base + 8 * gi, 0), w.Lc_cap - 8); };
  f32x4 pv[2], sv[8][2];
  {
    const int j = gstart(tid);
    pv[0] = *reinterpret_cast<const f32x4*>(part + j);
    pv[1] = *reinterpret_cast<const f32x4*>(part + j + 4);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      if (g < G) {
        sv[g][0] = *reinterpret_cast<const f32x4*>(spill + (int64_t)g * w.Lc_cap + j);
        sv[g][1] = *reinterpret_cast<const f32x4*>(spill + (int64_t)g * w.Lc_cap + j + 4);
      }
    }
  }
  if (si[2]) return;
  const int Lcur = si[0], steps = si[1];
  const int nc = Lcur + 1 - d.nrec - s;
  if (c0 >= nc && blk != 0) return;
  const int c1 = min(c0 + kPoolChunk, nc);
  {  // 1. current rows' softmax statistics over all splits: max, then the
     //    rescaled sums (splits past nsplit contribute nothing)
    const bool ok = tid < w.nsplit;
    float m[8], sm[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) m[g] = ok && tv[g].y > 0.f ? tv[g].x : -INFINITY;
    wave_max_n<8>(m);
    if (lane == 0)
#pragma unroll
      for (int g = 0; g < 8; ++g) wm[wv][g] = m[g];
    __syncthreads();
    float M[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      M[g] = fmaxf(fmaxf(wm[0][g], wm[1][g]), fmaxf(wm[2][g], wm[3][g]));
      sm[g] = ok && tv[g].y > 0.f ? tv[g].y * __builtin_amdgcn_exp2f(tv[g].x - M[g]) : 0.f;
    }
    wave_sum_n<8>(sm);
    if (lane == 0)
#pragma unroll
      for (int g = 0; g < 8; ++g) wsum[wv][g] = sm[g];
    __syncthreads();
    if (tid < G) {
      const float mm = M[tid];
      const float ss = (wsum[0][tid] + wsum[1][tid]) + (wsum[2][tid] + wsum[3][tid]);
      Mg[tid] = mm;
      Ig[tid] = 1.f / ss;
      if (blk == 0) {
        float* rs = rowstat_of(c, u) + ((steps % d.W) * G + tid) * 2;
        rs[0] = mm;
        rs[1] = ss;
      }
    }
    __syncthreads();
  }
  if (c0 >= nc) return;
  // 2. scores of group gi -> sc[8 gi ..]; positions outside [0, nc) are
  //    never read as candidates
  auto score_group = [&](int gi, const f32x4 (&p2)[2], const f32x4 (&s2)[8][2]) {
    const int j0 = base + 8 * gi;
    const int shift = j0 - gstart(gi);  // 0 except where the load was clamped
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = e < 4 ? p2[0][e] : p2[1][e - 4];
#pragma unroll
      for (int g = 0; g < 8; ++g)
        if (g < G) x += __builtin_amdgcn_exp2f((e < 4 ? s2[g][0][e] : s2[g][1][e - 4]) - Mg[g]) * Ig[g];
      v[e] = x;
    }
    if (shift == 0) {
      *reinterpret_cast<f32x4*>(sc + 8 * gi) = f32x4{v[0], v[1], v[2], v[3]};
      *reinterpret_cast<f32x4*>(sc + 8 * gi + 4) = f32x4{v[4], v[5], v[6], v[7]};
    }
    if (scores_user && shift == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (j0 + e >= c0 && j0 + e < c1) scores_user[(int64_t)u * c.Lmax + s + j0 + e] = v[e];
    }
  };
  score_group(tid, pv, sv);
  for (int gi = tid + 256; gi < ng; gi += 256) {  // the halo groups past 256
    const int j = gstart(gi);
    f32x4 p2[2], s2[8][2];
    p2[0] = *reinterpret_cast<const f32x4*>(part + j);
    p2[1] = *reinterpret_cast<const f32x4*>(part + j + 4);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      if (g < G) {
        s2[g][0] = *reinterpret_cast<const f32x4*>(spill + (int64_t)g * w.Lc_cap + j);
        s2[g][1] = *reinterpret_cast<const f32x4*>(spill + (int64_t)g * w.Lc_cap + j + 4);
      }
    }
    score_group(gi, p2, s2);
  }
  __syncthreads();
  uint32_t* keys = w.keys + (int64_t)u * w.Lc_cap;
  // 3. thread t: candidates c0 + 8t .. c0 + 8t + 7 (kPoolChunk = 8 * 256);
  //    sc index of position j is j - base
  const int jb = c0 + 8 * tid;
  unsigned int tmx = 0u;  // the largest of this thread's keys
  uint32_t kv[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  if (jb < c1) {
    if (h <= 4) {
      float win[16];  // scores at jb - 4 .. jb + 11, -inf outside the candidates
      const int i0 = jb - 4 - base;  // = 8 tid + 8 hg - 4: a multiple of 4
      if (i0 >= 0) {                 // four 16-byte reads
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const f32x4 v4 = *reinterpret_cast<const f32x4*>(sc + i0 + 4 * x);
#pragma unroll
          for (int y = 0; y < 4; ++y) win[4 * x + y] = v4[y];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) win[e] = sc[max(i0 + e, 0)];
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int j = jb - 4 + e;
        win[e] = (j >= 0 && j < nc) ? win[e] : -INFINITY;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float mx = win[e + 4];
#pragma unroll
        for (int dd = 1; dd <= 4; ++dd)
          if (dd <= h) mx = fmaxf(mx, fmaxf(win[e + 4 - dd], win[e + 4 + dd]));
        kv[e] = __float_as_uint(mx);
        if (jb + e < c1) {
          tmx = max(tmx, kv[e]);
        }
      }
      if (jb + 8 <= c1) {
        *reinterpret_cast<uint4*>(keys + jb) = make_uint4(kv[0], kv[1], kv[2], kv[3]);
        *reinterpret_cast<uint4*>(keys + jb + 4) = make_uint4(kv[4], kv[5], kv[6], kv[7]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (jb + e < c1) keys[jb + e] = kv[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = jb + e;
        if (j >= c1) break;
        float mx = sc[j - base];
        for (int dd = 1; dd <= h; ++dd) {
          if (j - dd >= 0) mx = fmaxf(mx, sc[j - dd - base]);
          if (j + dd < nc) mx = fmaxf(mx, sc[j + dd - base]);
        }
        kv[e] = __float_as_uint(mx);
        keys[j] = kv[e];
        tmx = max(tmx, kv[e]);
      }
    }
  }
  // 4. the maximum of each group of 8 << gsh candidates (2^gsh neighbouring
  //    threads; c0 is a multiple of the group size), for the top-k floor
  for (int o = 1; o < (1 << w.gsh); o <<= 1) tmx = max(tmx, (unsigned int)__shfl_xor((int)tmx, o));
  if (jb < c1 && (tid & ((1 << w.gsh) - 1)) == 0)
    w.gmax[(int64_t)u * (w.Lc_cap >> 3) + (jb >> (3 + w.gsh))] = tmx;
  // 5. the keys >= the selection hint (the previous top-k threshold with a
  //    margin; any value is valid, the top-k kernel checks the count), as
  //    (key, position) in position order into this block's stretch of the
  //    top-k slot buffer, their count into tkpcnt
  const uint32_t hint = w.tkhint[u];
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) cnt += (jb + e < c1 && kv[e] >= hint) ? 1 : 0;
  const int incl = wave_incl_scan(cnt);
  __shared__ int ptot[4];
  if (lane == 63) ptot[wv] = incl;
  __syncthreads();
  int off = incl - cnt, tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    off += i < wv ? ptot[i] : 0;
    tot += ptot[i];
  }
  uint2* dst = w.cslot + (int64_t)u * w.Lc_cap + c0;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (jb + e < c1 && kv[e] >= hint) dst[off++] = make_uint2(kv[e], (unsigned int)(jb + e));
  if (tid == 0) w.tkpcnt[(int64_t)u * w.tk_nbp + blk] = tot;
}

hipError_t launch_pool(const Dims& d, int U, const CachePtrs& c, const DecodeWs& w,
                       float* scores_user, hipStream_t st) {
  dim3 grid((w.Lc_cap + kPoolChunk - 1) / kPoolChunk, U);
  hipLaunchKernelGGL(k_pool, grid, dim3(256), 0, st, d, c, w, scores_user);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// top-k: one 1024-thread block per unit.
//   Keys are pooled scores as ordered bit patterns.  Wave w owns a
//   contiguous stretch of whole 256-key tiles (split by the capacity), read
//   with coalesced 16-byte loads, the first tiles and the group maxima
//   requested before the unit state arrives.
//   1. Floor: the pool kernel leaves the maximum of each group of 8
//      candidates.  Sets of disjoint groups have maxima too; if kk of them
//      are >= x, so is the kk-th largest key.  Each wave bounds the m_w-th
//      largest of its values from below by a bitwise search (wave ballots
//      only), with sum_w m_w >= kk; the floor is the least of the bounds.
//   2. The keys >= floor (candidates) are compacted per wave, in position
//      order (one ballot per key slot of a tile), into the wave's LDS list,
//      entries past kTopkWaveCap into the workspace; every later pass runs
//      over those short lists with full, mostly conflict-free LDS atomics.
//   3. Threshold T = the kk-th largest key, by a radix select over
//      [floor, max]: 2^12-bin histograms of (key - floor) >> shift, refined
//      until the selected bin is one key value (also when the bin turns out
//      to hold a single value) or is taken whole.
//   4. Ordered compaction: every key above the threshold bin, and the first
//      (kk - #above) keys of that bin in position order (ties -> lower
//      position), in ascending position order; one block scan of (#above,
//      #in-bin) per thread gives both offsets.  The picks leave through LDS
//      in one coalesced pass.
//   Also advances lens and writes the outputs of units whose cache is full
//   (topk = -1, out = 0).
// --------------------------------------------------------------------------
constexpr int kTopkThreads = 1024; // 16 waves; <= 128 VGPRs per thread
constexpr int kTopkTileRegs = 12;  // key tiles per wave held in registers (+4 VGPRs each)
constexpr int kTopkGroupRegs = kTopkGroupCap / kTopkThreads;  // group maxima per thread
constexpr int kTopkBinBits = 12;   // histogram digits per pass
constexpr int kTopkBins = 1 << kTopkBinBits;
constexpr int kTopkWaveCap = 512;  // candidates per wave kept in LDS
constexpr int kTopkCap = 16 * kTopkWaveCap;  // hint path: candidate list capacity
constexpr float kTopkHintMargin = 0.85f;     // hint = this x the previous threshold

// exclusive block prefix sums of two counters (a, b); totals in *ta, *tb
__device__ __forceinline__ int2 block_excl_scan2(int a, int b, int2* wtot, int* ta, int* tb) {
  constexpr int NW = kTopkThreads / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int ia = wave_incl_scan(a), ib = wave_incl_scan(b);
  if (lane == 63) wtot[wid] = make_int2(ia, ib);
  __syncthreads();
  int ba = 0, bb = 0, sa = 0, sb = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int2 t = wtot[i];
    if (i < wid) {
      ba += t.x;
      bb += t.y;
    }
    sa += t.x;
    sb += t.y;
  }
  __syncthreads();
  *ta = sa;
  *tb = sb;
  return make_int2(ba + ia - a, bb + ib - b);
}

// The bin holding the r-th largest of the counts in hs[0, nb) (bins above
// it hold fewer than r keys): thread t owns bins [16 t, 16 t + 16); the
// owner of the crossing bin writes its index, the remaining rank inside it
// and its count.  Ends with a block barrier.
__device__ __forceinline__ void topk_find_bin(const unsigned int* hs, int nb, int r, int2* wtot,
                                              unsigned int* sh_bin, int* sh_rem, int* sh_cnt) {
  constexpr int BPT = kTopkBins / kTopkThreads;
  const int b0 = BPT * threadIdx.x;
  unsigned int hv[BPT];
#pragma unroll
  for (int i = 0; i < BPT; i += 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(&hs[b0 + i]);
    hv[i] = b0 + i < nb ? v.x : 0u;
    hv[i + 1] = b0 + i + 1 < nb ? v.y : 0u;
    hv[i + 2] = b0 + i + 2 < nb ? v.z : 0u;
    hv[i + 3] = b0 + i + 3 < nb ? v.w : 0u;
  }
  int local = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) local += (int)hv[i];
  int tot, dummy;
  const int excl = block_excl_scan2(local, 0, wtot, &tot, &dummy).x;
  int above = tot - excl - local;  // keys in higher bins
  if (above < r && above + local >= r) {
    bool found = false;
#pragma unroll
    for (int i = BPT - 1; i >= 0; --i) {
      if (!found && above + (int)hv[i] >= r) {
        *sh_bin = (unsigned int)(b0 + i);
        *sh_rem = r - above;
        *sh_cnt = (int)hv[i];
        found = true;
      }
      above += (int)hv[i];
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kTopkThreads) void k_topk(Dims d, CachePtrs c, DecodeWs w,
                                               const uint16_t* __restrict__ vn,
                                               int32_t* __restrict__ topk_user,
                                               float* __restrict__ out) {
  const int u = blockIdx.y, tid = threadIdx.x;
  if (blockIdx.x > 0) {
    value_coef_block(d, c, w, vn, u, blockIdx.x - 1, tid);
    return;
  }
  const int lane = tid & 63, wid = tid >> 6;
  constexpr int NW = kTopkThreads / 64;
  const uint32_t* keys = w.keys + (int64_t)u * w.Lc_cap;
  const uint32_t* gmx = w.gmax + (int64_t)u * (w.Lc_cap >> 3);
  const int ncap = w.Lc_cap;
  // 0. the hint path: the pooling blocks left their keys >= the hint in
  //    position order; when at least kk and at most kTopkCap keys passed,
  //    the kk-th largest key is >= the hint and those keys are the whole
  //    candidate list.  Otherwise the full scan below runs.
  const int nbp = w.tk_nbp;
  const int pc = w.tkpcnt[(int64_t)u * nbp + min(tid, nbp - 1)];
  const uint32_t hint = w.tkhint[u];
  const int32_t* si = w.stepinfo + 4 * u;
  const int k = d.k;
  if (si[2]) {
    if (topk_user)
      for (int i = tid; i < k; i += kTopkThreads) topk_user[(int64_t)u * k + i] = -1;
    for (int i = tid; i < d.Hq * d.dh; i += kTopkThreads) out[(int64_t)u * d.Hq * d.dh + i] = 0.f;
    return;
  }
  const int Lcur = si[0], steps = si[1];
  const int s = d.s;
  const int nc = Lcur + 1 - d.nrec - s;
  const int kk = min(k, nc);
  // (lens and the unused top-k slots are written at the end)
  // reconstructed local window: its positions follow the picks in the
  // rebuilt-row list
  const int nloc = d.local ? min(d.nrec, Lcur + 1 - s) : 0;
  int32_t* sel = w.topk + (int64_t)u * w.ktot;
  for (int i = tid; i < nloc; i += kTopkThreads) sel[max(kk, 0) + i] = Lcur + 1 - nloc + i;
  if (kk <= 0) {
    if (tid == 0) {
      c.lens[2 * u] = Lcur + 1;
      c.lens[2 * u + 1] = steps + 1;
    }
    if (topk_user)
      for (int i = tid; i < k; i += kTopkThreads) topk_user[(int64_t)u * k + i] = -1;
    return;
  }
  __shared__ __attribute__((aligned(16))) unsigned int hs[kTopkBins];
  __shared__ uint2 cand[NW * kTopkWaveCap];  // candidates (key, position), position order
  __shared__ int roff[kTopkThreads + 1];     // hint path: the pooling blocks' list offsets
  __shared__ int2 wtot[NW];
  __shared__ unsigned int wlo[NW], whi[NW];
  __shared__ unsigned int sh_bin, sh_kmin, sh_kmax;
  __shared__ int sh_rem, sh_cnt;
  for (int i = tid; i < kTopkBins; i += kTopkThreads) hs[i] = 0u;
  if (tid == 0) {
    sh_kmin = 0xFFFFFFFFu;
    sh_kmax = 0u;
  }
  const int nbu = (nc + kPoolChunk - 1) / kPoolChunk;  // pooling blocks that ran
  int ptot, pdummy;
  const int poff = block_excl_scan2(tid < nbu && nbu <= kTopkThreads ? pc : 0, 0, wtot, &ptot, &pdummy).x;
  const bool fast = nbu <= kTopkThreads && ptot >= kk && ptot <= kTopkCap;  // block-uniform
  auto range_shift = [](unsigned int base, unsigned int top) {
    const unsigned int rg = top - base;
    const int bits = rg == 0u ? 0 : 32 - __clz((int)rg);
    return max(bits - kTopkBinBits, 0);
  };
  unsigned int lo, hi;
  // full scan: wave wid's stretch of tiles and its candidate list
  const int ntc = (ncap + 255) / 256;
  const int tpw = (ntc + NW - 1) / NW;
  const int t0 = wid * tpw;
  const int t1 = min(t0 + tpw, ntc);
  uint2* wlist = cand + wid * kTopkWaveCap;
  uint2* wslot = w.cslot + (int64_t)u * ncap + (int64_t)t0 * 256;
  int wcount = 0;  // wave-uniform
  if (fast) {
    if (tid < nbu) roff[tid] = poff;
    if (tid == 0) roff[nbu] = ptot;
    __syncthreads();
    // list entry i comes from pooling block r (roff[r] <= i < roff[r + 1]);
    // four entries per thread and round, requested together
    auto block_of = [&](int i) {
      int a = 0, z = nbu;
      while (z - a > 1) {
        const int m = (a + z) >> 1;
        if (roff[m] <= i) a = m; else z = m;
      }
      return a;
    };
    const uint2* src = w.cslot + (int64_t)u * ncap;
    unsigned int mx = 0u, mn = 0xFFFFFFFFu;
    for (int i0 = 0; i0 < ptot; i0 += 4 * kTopkThreads) {
      uint2 e[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = i0 + q * kTopkThreads + tid;
        if (i < ptot) {
          const int r = block_of(i);
          e[q] = src[(int64_t)r * kPoolChunk + (i - roff[r])];
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = i0 + q * kTopkThreads + tid;
        if (i < ptot) {
          cand[i] = e[q];
          mx = max(mx, e[q].x);
        }
      }
    }
    wave_minmax_u(mn, mx);
    if (lane == 0) whi[wid] = mx;
    __syncthreads();
    lo = hint;
    hi = whi[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) hi = max(hi, whi[i]);
  } else {
    // Wave wid scans tiles [t0, t1) of 256 keys (lane l: keys 4 l .. 4 l + 3
    // of a tile, one 16-byte load); the group maxima are requested first.
    // Unconditional loads at clamped addresses (reads stay below Lc_cap;
    // entries past the unit's candidates are masked later).
    const int gsz = 8 << w.gsh;
    const int ngcap = (ncap + gsz - 1) / gsz;  // <= kTopkThreads * kTopkGroupRegs
    uint32_t gv[kTopkGroupRegs];
#pragma unroll
    for (int i = 0; i < kTopkGroupRegs; ++i) gv[i] = gmx[min(tid + kTopkThreads * i, ngcap - 1)];
    uint4 kt[kTopkTileRegs];
#pragma unroll
    for (int i = 0; i < kTopkTileRegs; ++i)
      kt[i] = *reinterpret_cast<const uint4*>(keys + min((t0 + i) * 256 + 4 * lane, ncap - 4));
    // 1. floor.  The pool kernel leaves the maximum of every group of 8 << gsh
    //    candidates (at most kTopkGroupCap groups); register slot i of thread t
    //    holds group t + 1024 i.  Wave w searches its own values for x_w, a lower bound (on a
    //    grid of 2^-12 of its range) of their m_w-th largest, m_w =
    //    ceil(kk n_w / n) for its n_w of the n values: every wave then holds
    //    m_w values >= x_w, together >= kk values from disjoint key sets, so
    //    floor = min_w x_w is at most the kk-th largest key.  (n < kk: no
    //    floor.)  The values' maximum is also the keys' maximum.
    const int ng = (nc + gsz - 1) / gsz;
    const int nval = ng;
    {
      bool gok[kTopkGroupRegs];
  #pragma unroll
      for (int i = 0; i < kTopkGroupRegs; ++i) gok[i] = tid + kTopkThreads * i < ng;
      unsigned int mn = 0xFFFFFFFFu, mx = 0u;
      int nw = 0;  // wave-uniform
  #pragma unroll
      for (int i = 0; i < kTopkGroupRegs; ++i) {
        if (gok[i]) {
          mn = min(mn, gv[i]);
          mx = max(mx, gv[i]);
        }
        nw += __popcll(__ballot(gok[i]));
      }
      wave_minmax_u(mn, mx);
      unsigned int xw = 0xFFFFFFFFu;  // no values: no bound from this wave
      if (nw > 0 && nval >= kk) {
        const int mw = (int)(((int64_t)kk * nw + nval - 1) / nval);
        const unsigned int rg = mx - mn;
        const int top = rg == 0u ? -1 : 31 - __clz((int)rg);
        const int sh = max(top + 1 - 12, 0);
        unsigned int dv[kTopkGroupRegs];  // offsets above mn; 0 (never counted) for no value
  #pragma unroll
        for (int i = 0; i < kTopkGroupRegs; ++i) dv[i] = gok[i] ? gv[i] - mn : 0u;
        unsigned int t = 0u;  // offset above mn with >= mw values at or above it
        for (int bit = top; bit >= sh; --bit) {
          const unsigned int cand_t = t | (1u << bit);  // >= 1
          int cnt = 0;
  #pragma unroll
          for (int i = 0; i < kTopkGroupRegs; ++i)  // lanes with dv[i] >= cand_t (35: unsigned >=)
            cnt += __popcll(__builtin_amdgcn_uicmp(dv[i], cand_t, 35));
          if (cnt >= mw) t = cand_t;
        }
        xw = mn + t;
      }
      if (lane == 0) {
        wlo[wid] = xw;
        whi[wid] = mx;
      }
    }
    __syncthreads();
    lo = wlo[0];
    hi = whi[0];
  #pragma unroll
    for (int i = 1; i < NW; ++i) {
      lo = min(lo, wlo[i]);
      hi = max(hi, whi[i]);
    }
    if (nval < kk) lo = 0u;  // fewer values than picks: every key is a candidate
    // 2. candidates: keys >= lo, compacted per wave in position order (ballot
    //    counts): the wave's first kTopkWaveCap go to its stretch of the LDS
    //    list, any further ones to the wave's region of the unit's slot
    //    buffer (indexed like the list, starting at the wave's first position,
    //    so it never overflows).
    auto take_tile = [&](const uint4& kv, int t) {
      const int j = t * 256 + 4 * lane;
      const uint32_t kx[4] = {kv.x, kv.y, kv.z, kv.w};
      bool p[4];
      uint64_t bl[4];
      int before = 0, tot = 0;
  #pragma unroll
      for (int e = 0; e < 4; ++e) {  // lane masks of j + e < nc (36: unsigned <) and key >= lo (35: >=)
        bl[e] = __builtin_amdgcn_uicmp((unsigned int)(j + e), (unsigned int)nc, 36) &
                __builtin_amdgcn_uicmp(kx[e], lo, 35);
        p[e] = (bl[e] >> lane) & 1u;
        before += __builtin_amdgcn_mbcnt_hi((uint32_t)(bl[e] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bl[e], 0u));
        tot += __popcll(bl[e]);
      }
      int o = wcount + before;
  #pragma unroll
      for (int e = 0; e < 4; ++e)
        if (p[e]) {
          const uint2 v = make_uint2(kx[e], (unsigned int)(j + e));
          if (o < kTopkWaveCap)
            wlist[o] = v;
          else
            wslot[o] = v;
          ++o;
        }
      wcount += tot;
    };
    for (int r0 = 0; t0 + r0 < t1; r0 += kTopkTileRegs) {
      if (r0 > 0) {
  #pragma unroll
        for (int i = 0; i < kTopkTileRegs; ++i) {
          const int j = (t0 + r0 + i) * 256 + 4 * lane;
          kt[i] = *reinterpret_cast<const uint4*>(keys + min(j, ncap - 4));
        }
      }
  #pragma unroll
      for (int i = 0; i < kTopkTileRegs; ++i)
        if (t0 + r0 + i < t1 && (t0 + r0 + i) * 256 < nc) take_tile(kt[i], t0 + r0 + i);
    }
    if (wcount > kTopkWaveCap) {
      // the slot entries are read back by other lanes of the same wave
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
  }
  // candidates of this thread in position order: a contiguous share of the
  // list (hint path) or of its wave's list (neighbouring lanes hold
  // different stretches, so the equal keys of a pooled run do not collide in
  // one atomic)
  const int cpt = fast ? (ptot + kTopkThreads - 1) / kTopkThreads : (wcount + 63) / 64;
  const int nlist = fast ? ptot : wcount;
  const int a0 = min((fast ? tid : lane) * cpt, nlist), a1 = min(a0 + cpt, nlist);
  auto visit_ordered = [&](auto&& f) {
    for (int i = a0; i < a1; ++i) {
      const uint2 e = fast ? cand[i] : (i < kTopkWaveCap ? wlist[i] : wslot[i]);
      f(e.x, (int)e.y);
    }
  };
  // histogram of f(key) over the thread's candidates with pred(key); equal
  // consecutive bins cost one atomic
  auto histo = [&](auto&& pred, auto&& binof) {
    unsigned int pb = 0xFFFFFFFFu, pc = 0u;
    visit_ordered([&](uint32_t key, int) {
      if (!pred(key)) return;
      const unsigned int bn = binof(key);
      if (bn != pb) {
        if (pc) atomicAdd(&hs[pb], pc);
        pb = bn;
        pc = 0u;
      }
      ++pc;
    });
    if (pc) atomicAdd(&hs[pb], pc);
  };
  // 3. threshold
  int shift = range_shift(lo, hi);
  histo([](uint32_t) { return true; }, [&](uint32_t key) { return (key - lo) >> shift; });
  __syncthreads();
  topk_find_bin(hs, kTopkBins, kk, wtot, &sh_bin, &sh_rem, &sh_cnt);
  unsigned int bin = sh_bin;
  int rem = sh_rem, cnt_bin = sh_cnt;
  while (shift > 0 && rem < cnt_bin) {
    const int nsh = max(shift - kTopkBinBits, 0);
    const unsigned int nb = 1u << (shift - nsh);
    for (int i = tid; i < (int)nb; i += kTopkThreads) hs[i] = 0u;
    __syncthreads();
    unsigned int bmin = 0xFFFFFFFFu, bmax = 0u;
    histo(
        [&](uint32_t key) {
          const bool in = ((key - lo) >> shift) == bin;
          if (in) {
            bmin = min(bmin, key);
            bmax = max(bmax, key);
          }
          return in;
        },
        [&](uint32_t key) { return ((key - lo) >> nsh) & (nb - 1u); });
    wave_minmax_u(bmin, bmax);
    if (lane == 0) {
      if (bmin != 0xFFFFFFFFu) atomicMin(&sh_kmin, bmin);
      if (bmax != 0u) atomicMax(&sh_kmax, bmax);
    }
    __syncthreads();
    if (sh_kmin == sh_kmax) {  // one value: it is the threshold
      bin = sh_kmin - lo;
      shift = 0;
      break;
    }
    topk_find_bin(hs, (int)nb, rem, wtot, &sh_bin, &sh_rem, &sh_cnt);
    const unsigned int sub = sh_bin;
    rem = sh_rem;
    cnt_bin = sh_cnt;
    bin = (bin << (shift - nsh)) | sub;
    shift = nsh;
    if (tid == 0) {
      sh_kmin = 0xFFFFFFFFu;
      sh_kmax = 0u;
    }
    __syncthreads();
  }
  if (tid == 0) {  // the next step's hint: this threshold's bin edge, with a margin
    const unsigned int edge = lo + (bin << shift);
    w.tkhint[u] = __float_as_uint(__uint_as_float(edge) * kTopkHintMargin);
  }
  // 4. compaction in position order: keys with (key - lo) >> shift above
  // `bin`, then the first `rem` keys of the bin; the in-bin keys taken
  // before thread t number min(rem, in-bin keys before t)
  int c_gt = 0, c_eq = 0;
  visit_ordered([&](uint32_t key, int) {
    const unsigned int bn = (key - lo) >> shift;
    c_gt += bn > bin;
    c_eq += bn == bin;
  });
  int tgt, teq;
  const int2 base = block_excl_scan2(c_gt, c_eq, wtot, &tgt, &teq);
  const int take_eq = max(0, min(rem - base.y, c_eq));
  int off = base.x + min(rem, base.y);
  // the picks go through LDS (the histogram is free now) and leave in one
  // coalesced pass; units with more than kTopkBins picks write directly
  const bool stage = kk <= kTopkBins;
  int seen = 0;
  visit_ordered([&](uint32_t key, int j) {
    const unsigned int bn = (key - lo) >> shift;
    bool take = bn > bin;
    if (bn == bin) {
      take = seen < take_eq;
      ++seen;
    }
    if (take) {
      if (stage) {
        hs[off] = (unsigned int)(s + j);
      } else {
        sel[off] = s + j;
        if (topk_user) topk_user[(int64_t)u * k + off] = s + j;
      }
      ++off;
    }
  });
  if (stage) {
    __syncthreads();
    for (int i = tid; i < kk; i += kTopkThreads) {
      const int v = (int)hs[i];
      sel[i] = v;
      if (topk_user) topk_user[(int64_t)u * k + i] = v;
    }
  }
  if (tid == 0) {
    c.lens[2 * u] = Lcur + 1;
    c.lens[2 * u + 1] = steps + 1;
  }
  if (topk_user)
    for (int i = kk + tid; i < k; i += kTopkThreads) topk_user[(int64_t)u * k + i] = -1;
}

hipError_t launch_topk(const Dims& d, int U, const CachePtrs& c, const DecodeWs& w, const void* v_new,
                       int32_t* topk_user, float* out, hipStream_t st) {
  const int nvb = prologue_fused(d) ? d.rv / 32 : 0;  // c^V(new) blocks, see the prologue
  hipLaunchKernelGGL(k_topk, dim3(1 + nvb, U), dim3(kTopkThreads), 0, st, d, c, w,
                     (const uint16_t*)v_new, topk_user, out);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// Sparse reconstruction + exact attention, evaluated in coefficient space.
//
// For a selected position j of KV head h, the reconstructed key is
// k_hat = B^K_h c^K_j (B^K_h: the d_h rows of B^K that belong to head h), so
// q . k_hat = (B^K_h^T q) . c^K_j, and sum_j p_j v_hat_j = B^V_h (sum_j p_j
// c^V_j).  The prologue writes qlat = B^K_h^T q (times log2(e)/sqrt(d_h));
// here every block scores rows against all query heads at once, which reads
// each selected coefficient row once per step instead of once per KV head,
// and the merge applies B^V_h once per head.  The algebra is exact; only the
// fp32 summation order differs from rebuilding the keys and values first.
//
// grid (nsl * nhg + nse * ceil(H_kv / 4), U), 256 threads (4 waves):
//   block (split, hg) < nsl * nhg: selected rows [split * rsl, +rsl) of the
//     top-k list, heads [hg * hb, +hb): logits c^K_j . qlat[a], a split-local
//     softmax, ylat[a] = sum_j p_j c^V_j;
//   then block (e, hq): exact rows [e * rse, +rse) of (sinks, recent ring),
//     wave w takes KV head 4 hq + w; lane = row for the logits, lane =
//     channel for the values; yex[a] = sum_j p_j v_j.
// Every split stores its (max, sum) per head; k_merge combines them.
// --------------------------------------------------------------------------
template <typename T> struct Quad;  // 4 storage elements
template <> struct Quad<float> {
  typedef f32x4 V;
  static __device__ __forceinline__ f32x4 f(V v) { return v; }
};
template <> struct Quad<uint16_t> {
  typedef unsigned short V __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ f32x4 f(V v) {
    return f32x4{bf2f(v[0]), bf2f(v[1]), bf2f(v[2]), bf2f(v[3])};
  }
};

// Exact rows (sinks, then the recent ring) of one block: block index be
// among the exact blocks; needs no unit state (a full unit's results are
// never read).
template <typename T>
__device__ __forceinline__ void attend_exact(const Dims& d, const CachePtrs& c, const DecodeWs& w,
                                             const T* __restrict__ q, float ascale, int be, int u,
                                             int tid, float* smf) {
  const int wv = tid >> 6, l = tid & 63, Hq = d.Hq;
  // block (e, hq): rows [e * rse, +rse) (rse <= 32), KV head h = 4 hq + wave.
  // Lane l < nrow loads row l's K and V slices of head h in one phase (V goes
  // to LDS), scores it against the G query heads, and after the softmax the
  // lanes switch to channels (c = l + 64 i) to sum the values from LDS.
  const int nhq = (d.Hkv + 3) >> 2;
  const int e = be / nhq, h = (be % nhq) * 4 + wv;
  const int s = d.s, nrec = d.nrec, G = d.G, dh = d.dh, D = d.D;
  const int row0 = e * w.rse;
  const int nrow = min(w.rse, n_exact_rows(d) - row0);
  if (nrow <= 0 || h >= d.Hkv) return;  // no block-wide barrier below
  constexpr int VEC = Vec16<T>::N;
  const int ldv = dh + VEC;                        // padded LDS row (storage elements)
  float* qs = smf + wv * exact_wave_floats(G, dh, (int)sizeof(T));  // [G][dh] queries, times ascale
  float* pw = qs + G * dh;                          // [32][8] probabilities
  T* vs = reinterpret_cast<T*>(pw + 32 * 8);        // [32][ldv] value rows
  const bool live = l < nrow;
  const int row = row0 + min(l, nrow - 1);  // lanes past nrow repeat the last row
  const int64_t roff = row < s ? ((int64_t)u * s + row) * D : ((int64_t)u * nrec + (row - s)) * D;
  const T* krow = (row < s ? (const T*)c.sink_k : (const T*)c.ring_k) + roff + (int64_t)h * dh;
  const T* vrow = (row < s ? (const T*)c.sink_v : (const T*)c.ring_v) + roff + (int64_t)h * dh;
  const T* qh = q + ((int64_t)u * Hq + h * G) * dh;
  const int npc = dh / VEC;  // 16-byte pieces per row slice
  float z[8];
#pragma unroll
  for (int g = 0; g < 8; ++g) z[g] = 0.f;
  for (int p0 = 0; p0 < npc; p0 += 16) {
    u16x8 kr[16], vr[16], qr[4];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int pc = min(p0 + t, npc - 1);
      kr[t] = *reinterpret_cast<const u16x8*>(krow + pc * VEC);
      vr[t] = *reinterpret_cast<const u16x8*>(vrow + pc * VEC);
    }
    if (p0 == 0) {  // the G query rows: G * dh / VEC pieces over 64 lanes
#pragma unroll
      for (int t = 0; t < 4; ++t)  // G * dh <= 1024: at most 256 pieces
        qr[t] = *reinterpret_cast<const u16x8*>(qh + min(l + 64 * t, G * npc - 1) * VEC);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int pc = l + 64 * t;
        if (pc < G * npc) {
          const T* qv = reinterpret_cast<const T*>(&qr[t]);
#pragma unroll
          for (int x = 0; x < VEC; x += 4)
            *reinterpret_cast<f32x4*>(qs + pc * VEC + x) =
                f32x4{Elem<T>::ld(qv, x), Elem<T>::ld(qv, x + 1), Elem<T>::ld(qv, x + 2),
                      Elem<T>::ld(qv, x + 3)} * ascale;
        }
      }
    }
#pragma unroll
    for (int t = 0; t < 16; ++t)
      if (live && p0 + t < npc) *reinterpret_cast<u16x8*>(vs + l * ldv + (p0 + t) * VEC) = vr[t];
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      if (p0 + t < npc) {
        const T* kv = reinterpret_cast<const T*>(&kr[t]);
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          if (g < G) {
            const float* qg = qs + g * dh + (p0 + t) * VEC;
#pragma unroll
            for (int x = 0; x < VEC; x += 4) {
              const f32x4 q4 = *reinterpret_cast<const f32x4*>(qg + x);
              z[g] += q4[0] * Elem<T>::ld(kv, x) + q4[1] * Elem<T>::ld(kv, x + 1) +
                      q4[2] * Elem<T>::ld(kv, x + 2) + q4[3] * Elem<T>::ld(kv, x + 3);
            }
          }
        }
      }
    }
  }
  float m[8], S[8];
#pragma unroll
  for (int g = 0; g < 8; ++g) m[g] = live ? z[g] : -INFINITY;
  wave_max_n<8>(m);
#pragma unroll
  for (int g = 0; g < 8; ++g) S[g] = live ? __builtin_amdgcn_exp2f(z[g] - m[g]) : 0.f;
  if (l < 32) {  // pw[row][g], g padded to 8
    *reinterpret_cast<f32x4*>(pw + l * 8) = f32x4{S[0], S[1], S[2], S[3]};
    *reinterpret_cast<f32x4*>(pw + l * 8 + 4) = f32x4{S[4], S[5], S[6], S[7]};
  }
  wave_sum_n<8>(S);
  __builtin_amdgcn_wave_barrier();
  // values: lane l holds channel pairs c = 2 l + 128 i, i < 2 (d_h <= 256)
  float o[8][4];
#pragma unroll
  for (int g = 0; g < 8; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) o[g][i] = 0.f;
  const int c0 = min(2 * l, dh - 2), c1 = min(2 * l + 128, dh - 2);
#pragma unroll 4
  for (int j = 0; j < nrow; ++j) {
    const T* vj = vs + j * ldv;
    const float v0 = Elem<T>::ld(vj, c0), v1 = Elem<T>::ld(vj, c0 + 1);
    const float v2 = Elem<T>::ld(vj, c1), v3 = Elem<T>::ld(vj, c1 + 1);
    const f32x4 pa = *reinterpret_cast<const f32x4*>(pw + j * 8);
    const f32x4 pb = G > 4 ? *reinterpret_cast<const f32x4*>(pw + j * 8 + 4) : f32x4{};
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const float p = g < 4 ? pa[g] : pb[g - 4];
      o[g][0] += p * v0;
      o[g][1] += p * v1;
      o[g][2] += p * v2;
      o[g][3] += p * v3;
    }
  }
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    if (g < G) {
      const int a = h * G + g;
      float* yo = w.yex + (((int64_t)u * w.nse + e) * Hq + a) * dh;
      if (2 * l < dh) {
        yo[2 * l] = o[g][0];
        yo[2 * l + 1] = o[g][1];
      }
      if (2 * l + 128 < dh) {
        yo[2 * l + 128] = o[g][2];
        yo[2 * l + 129] = o[g][3];
      }
      if (l == 0) {
        float* stp = w.astat + (((int64_t)u * (w.nsl + w.nse) + w.nsl + e) * Hq + a) * 2;
        stp[0] = m[g];
        stp[1] = S[g];
      }
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_attend(Dims d, CachePtrs c, DecodeWs w,
                                                const T* __restrict__ q, float ascale) {
  typedef typename Quad<T>::V QV;
  const int b = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  extern __shared__ __attribute__((aligned(16))) float smf[];
  if (b >= w.nsl * w.nhg) {
    attend_exact<T>(d, c, w, q, ascale, b - w.nsl * w.nhg, u, tid, smf);
    return;
  }
  const int32_t* si = w.stepinfo + 4 * u;
  if (si[2]) return;  // full unit: the top-k kernel wrote zeros
  const int Lcur = si[0];
  const int r = d.r, rv = d.rv, Hq = d.Hq;  // key rank (logits), value rank (values)
  const int kk = n_rebuilt(d, Lcur);
  const int wv = tid >> 6, l = tid & 63;

  {
    // ---------------- selected rows, coefficient space (fp32 VALU) ----------------
    const int split = b / w.nhg, hg = b % w.nhg;
    const int row0 = split * w.rsl;
    const int nrow = min(w.rsl, kk - row0);
    if (nrow <= 0) return;
    const int hb = w.hb, a0 = hg * hb, na = min(hb, Hq - a0);
    constexpr int E = 16 / sizeof(T);                 // elements per 16-byte piece
    const int ldq = r + 4, ldz = w.rsl + 1, ldc = r + E, r4 = r / 4, rE = r / E;
    const int ldcv = rv + E, rv4 = rv / 4, rvE = rv / E;
    float* qt = smf;                                  // [hb][ldq]
    float* zs = qt + hb * ldq;                        // [hb][ldz]
    T* ck = reinterpret_cast<T*>(zs + ((hb * ldz + 3) & ~3) + w.rsl * hb);  // [rsl][ldc]
    T* cv = ck + w.rsl * ldc;                         // [rsl][ldcv]
    const int32_t* sel = w.topk + (int64_t)u * w.ktot + row0;
    {
      // every thread issues its loads (8 pieces of K and of V per round)
      // before it stores any of them
      const T* cks = (const T*)c.coef_k + (int64_t)u * c.Lmax * r;
      const T* cvs = (const T*)c.coef_v + (int64_t)u * c.Lmax * rv;
      const int npk = nrow * rE, npv = nrow * rvE, npc = npk > npv ? npk : npv;
      for (int e0 = 0; e0 < npc; e0 += 256 * 8) {
        u16x8 xk[8], xv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int ek = min(e0 + tid + 256 * i, npk - 1), ev = min(e0 + tid + 256 * i, npv - 1);
          const int64_t pk = min(max((int64_t)sel[ek / rE], (int64_t)0), c.Lmax - 1);
          const int64_t pv = min(max((int64_t)sel[ev / rvE], (int64_t)0), c.Lmax - 1);
          xk[i] = *reinterpret_cast<const u16x8*>(cks + pk * r + (ek % rE) * E);
          xv[i] = *reinterpret_cast<const u16x8*>(cvs + pv * rv + (ev % rvE) * E);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int e = e0 + tid + 256 * i;
          if (e < npk) *reinterpret_cast<u16x8*>(ck + (e / rE) * ldc + (e % rE) * E) = xk[i];
          if (e < npv) *reinterpret_cast<u16x8*>(cv + (e / rvE) * ldcv + (e % rvE) * E) = xv[i];
        }
      }
      const float* qsrc = w.qlat + ((int64_t)u * Hq + a0) * r;
      const int nq = na * r4;
      for (int e0 = 0; e0 < nq; e0 += 256 * 8) {
        f32x4 x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int e = min(e0 + tid + 256 * i, nq - 1);
          x[i] = *reinterpret_cast<const f32x4*>(qsrc + (int64_t)(e / r4) * r + 4 * (e % r4));
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int e = e0 + tid + 256 * i;
          if (e < nq) *reinterpret_cast<f32x4*>(qt + (e / r4) * ldq + 4 * (e % r4)) = x[i];
        }
      }
    }
    __syncthreads();
    // logits: item (a, row group of 4); rows past nrow are computed from
    // stale LDS and discarded
    const int ngj = (nrow + 3) >> 2;
    for (int e = tid; e < na * ngj; e += 256) {
      const int a = e / ngj, jg = e % ngj;
      const float* qa = qt + a * ldq;
      const T* c0 = ck + 4 * jg * ldc;
      f32x4 acc[4] = {};
#pragma unroll 4
      for (int i = 0; i < r; i += 4) {
        const f32x4 q4 = *reinterpret_cast<const f32x4*>(qa + i);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          acc[jj] += q4 * Quad<T>::f(*reinterpret_cast<const QV*>(c0 + jj * ldc + i));
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        if (4 * jg + jj < nrow)
          zs[a * ldz + 4 * jg + jj] = (acc[jj][0] + acc[jj][1]) + (acc[jj][2] + acc[jj][3]);
    }
    __syncthreads();
    // split-local softmax: a wave takes 8 heads at a time, a lane per row;
    // probabilities go to pT[row][head]
    float* pT = zs + hb * ldz;  // [rsl][hb]
    for (int ab = wv * 8; ab < na; ab += 32) {
      float z[8], m[8], p[8], S[8];
#pragma unroll
      for (int aa = 0; aa < 8; ++aa) {
        const bool ok = l < nrow && ab + aa < na;
        z[aa] = ok ? zs[(ab + aa) * ldz + l] : -INFINITY;
        m[aa] = z[aa];
      }
      wave_max_n<8>(m);
#pragma unroll
      for (int aa = 0; aa < 8; ++aa) {
        p[aa] = z[aa] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z[aa] - m[aa]);
        S[aa] = p[aa];
      }
      wave_sum_n<8>(S);
      if (l < nrow) {
        *reinterpret_cast<f32x4*>(pT + l * hb + ab) = f32x4{p[0], p[1], p[2], p[3]};
        *reinterpret_cast<f32x4*>(pT + l * hb + ab + 4) = f32x4{p[4], p[5], p[6], p[7]};
      }
      if (l < 8 && ab + l < na) {
        float mm = m[0], ss = S[0];
#pragma unroll
        for (int aa = 1; aa < 8; ++aa) {
          mm = l == aa ? m[aa] : mm;
          ss = l == aa ? S[aa] : ss;
        }
        float* stp = w.astat + (((int64_t)u * (w.nsl + w.nse) + split) * Hq + a0 + ab + l) * 2;
        stp[0] = mm;
        stp[1] = ss;
      }
    }
    __syncthreads();
    // ylat[a] = sum_j p[a][j] c^V_j: item (8 heads, 4 coefficients)
    const int nag = (na + 7) >> 3;
    for (int e = tid; e < nag * rv4; e += 256) {
      const int ag = e / rv4, i4 = e % rv4;
      f32x4 acc[8] = {};
#pragma unroll 4
      for (int j = 0; j < nrow; ++j) {
        const f32x4 v4 = Quad<T>::f(*reinterpret_cast<const QV*>(cv + j * ldcv + 4 * i4));
        const f32x4 pa = *reinterpret_cast<const f32x4*>(pT + j * hb + 8 * ag);
        const f32x4 pb = *reinterpret_cast<const f32x4*>(pT + j * hb + 8 * ag + 4);
        acc[0] += pa[0] * v4;
        acc[1] += pa[1] * v4;
        acc[2] += pa[2] * v4;
        acc[3] += pa[3] * v4;
        acc[4] += pb[0] * v4;
        acc[5] += pb[1] * v4;
        acc[6] += pb[2] * v4;
        acc[7] += pb[3] * v4;
      }
#pragma unroll
      for (int aa = 0; aa < 8; ++aa) {
        const int a = 8 * ag + aa;
        if (a < na)
          *reinterpret_cast<f32x4*>(w.ylat + (((int64_t)u * w.nsl + split) * Hq + a0 + a) * rv +
                                    4 * i4) = acc[aa];
      }
    }
    return;
  }
}

// --------------------------------------------------------------------------
// Selected rows for bf16 storage with MFMA (16x16x32, bf16 in, fp32 out):
// block (split, hg): 64 rows x 32 heads.  The projected queries and the
// probabilities enter as bf16 hi + lo pairs (two MFMAs each), so products
// carry about 16 mantissa bits; the coefficients are exact bf16.
//   logits: wave w -> head tile w / 2, row tiles 2 (w % 2) + {0, 1}, K = r;
//   softmax as in the fp32 kernel (a lane per row), probabilities to LDS;
//   values: wave w -> head tile w % 2, half of the r / 16 coefficient tiles,
//     K = the 64 rows; the V rows are staged transposed ([coefficient][row])
//     so every MFMA operand is one 16-byte LDS read.
// Loads that do not depend on the unit state (top-k entries, query
// fragments) are issued together with it.
// --------------------------------------------------------------------------
constexpr int kAttnRows = 64;
template <int R, int RV>
struct AttnTile {
  static constexpr int KC = R / 8;                 // 16-byte chunks per key coefficient row
  static constexpr int CKB = R * 2 + 16;           // bytes per staged K row
  static constexpr int CVB = kAttnRows * 2 + 16;   // bytes per transposed V row
  static constexpr int ZLD = kAttnRows + 1, PLD = kAttnRows + 4;  // fp32 strides
  // the logits and probabilities reuse the K rows' space once the logit
  // MFMAs are done (a block barrier separates them), so two blocks fit a CU
  static constexpr int ck = 0;
  static constexpr int zs = 0;
  static constexpr int pz = zs + ((32 * ZLD * 4 + 15) & ~15);
  static constexpr int kz = kAttnRows * CKB > pz + 32 * PLD * 4 ? kAttnRows * CKB : pz + 32 * PLD * 4;
  static constexpr int cv = (kz + 15) & ~15;
  static constexpr int bytes = cv + RV * CVB;      // V rows transposed: RV coefficient rows
};
static int attn_tile_bytes(int r, int rv) {
  const int kb = kAttnRows * (r * 2 + 16);
  const int zp = ((32 * (kAttnRows + 1) * 4 + 15) & ~15) + 32 * (kAttnRows + 4) * 4;
  return ((kb > zp ? kb : zp) + 15) / 16 * 16 + rv * (kAttnRows * 2 + 16);
}


// bf16 hi / lo pair of 8 fp32 values as MFMA operands
__device__ __forceinline__ void split8(f32x4 p0, f32x4 p1, bf16x8* hi, bf16x8* lo) {
  u16x8 ph, pl;
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    const float pv = x < 4 ? p0[x] : p1[x - 4];
    const uint16_t hb = f2bf(pv);
    ph[x] = hb;
    pl[x] = f2bf(pv - bf2f(hb));
  }
  *hi = __builtin_bit_cast(bf16x8, ph);
  *lo = __builtin_bit_cast(bf16x8, pl);
}

// Exact rows for bf16 storage: the logits on MFMA 16x16x32 (A = the G
// query rows of KV head h, bf16 and exact, zero past G; B = the K rows,
// K = channels, read straight from memory; D = heads x rows), the softmax
// reduced over each 16-lane row of the wave, the values as in attend_exact.
__device__ __forceinline__ void attend_exact_mfma(const Dims& d, const CachePtrs& c, const DecodeWs& w,
                                                  const uint16_t* __restrict__ q, float ascale, int be,
                                                  int u, int tid, float* smf) {
  const int wv = tid >> 6, l = tid & 63, Hq = d.Hq;
  const int n16 = l & 15, kq = l >> 4;
  const int nhq = (d.Hkv + 3) >> 2;
  const int e = be / nhq, h = (be % nhq) * 4 + wv;
  const int s = d.s, nrec = d.nrec, G = d.G, dh = d.dh, D = d.D;
  const int row0 = e * w.rse;
  const int nrow = min(w.rse, n_exact_rows(d) - row0);
  if (nrow <= 0 || h >= d.Hkv) return;  // no block-wide barrier below
  constexpr int VEC = 8;
  const int ldv = dh + VEC;                        // padded LDS row (storage elements)
  float* pw = smf + wv * exact_wave_floats(G, dh, 2) + G * dh;  // [32][8] probabilities
  uint16_t* vs = reinterpret_cast<uint16_t*>(pw + 32 * 8);       // [32][ldv] value rows
  auto rowptr = [&](const void* sink, const void* ring, int rr) {
    const int64_t roff = rr < s ? ((int64_t)u * s + rr) * D : ((int64_t)u * nrec + (rr - s)) * D;
    return (rr < s ? (const uint16_t*)sink : (const uint16_t*)ring) + roff + (int64_t)h * dh;
  };
  const int nks = dh / 32;  // head_dim multiple of 32 here
  // B: K row 16 t + n16 (clamped to the last row), channels 32 ks + 8 kq
  bf16x8 kb[2][8];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint16_t* kr = rowptr(c.sink_k, c.ring_k, row0 + min(16 * t + n16, nrow - 1));
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      if (ks < nks) kb[t][ks] = ld_bf16x8(kr + 32 * ks + 8 * kq);
  }
  // A: query head h G + n16 (zero past G)
  bf16x8 qa[8];
  {
    const uint16_t* qh = q + ((int64_t)u * Hq + h * G + min(n16, G - 1)) * dh;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      if (ks < nks) qa[ks] = n16 < G ? ld_bf16x8(qh + 32 * ks + 8 * kq) : __builtin_bit_cast(bf16x8, u16x8{});
  }
  // V rows to LDS: piece x = l + 64 i of (row, 16-byte chunk); all loads
  // first (clamped), then the stores (rows <= 32, d_h <= 256: <= 16 each)
  const int npc = dh / VEC;
  u16x8 vp[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int x = min(l + 64 * i, nrow * npc - 1);
    vp[i] = *reinterpret_cast<const u16x8*>(rowptr(c.sink_v, c.ring_v, row0 + x / npc) + (x % npc) * VEC);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int x = l + 64 * i;
    if (x < nrow * npc) *reinterpret_cast<u16x8*>(vs + (x / npc) * ldv + (x % npc) * VEC) = vp[i];
  }
  // logits: lane holds heads 4 kq + i, rows 16 t + n16
  f32x4 z[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    z[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      if (ks < nks) z[t] = mfma16x16x32(qa[ks], kb[t][ks], z[t]);
  }
  float m[4], S[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float z0 = n16 < nrow ? z[0][i] * ascale : -INFINITY;
    const float z1 = 16 + n16 < nrow ? z[1][i] * ascale : -INFINITY;
    float mx = fmaxf(z0, z1);
    mx = fmaxf(mx, dpp_f<0xB1>(mx));
    mx = fmaxf(mx, dpp_f<0x4E>(mx));
    mx = fmaxf(mx, dpp_f<0x141>(mx));
    mx = fmaxf(mx, dpp_f<0x140>(mx));
    m[i] = mx;
    const float p0 = n16 < nrow ? __builtin_amdgcn_exp2f(z0 - mx) : 0.f;
    const float p1 = 16 + n16 < nrow ? __builtin_amdgcn_exp2f(z1 - mx) : 0.f;
    if (kq < 2) {
      pw[n16 * 8 + 4 * kq + i] = p0;
      pw[(16 + n16) * 8 + 4 * kq + i] = p1;
    }
    float sm = p0 + p1;
    sm += dpp_f<0xB1>(sm);
    sm += dpp_f<0x4E>(sm);
    sm += dpp_f<0x141>(sm);
    sm += dpp_f<0x140>(sm);
    S[i] = sm;
  }
  __builtin_amdgcn_s_waitcnt(0);  // V rows and probabilities are in LDS
  __builtin_amdgcn_wave_barrier();
  // values: lane l holds channel pairs c = 2 l + 128 i, i < 2 (d_h <= 256)
  float o[8][4];
#pragma unroll
  for (int g = 0; g < 8; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) o[g][i] = 0.f;
  const int c0 = min(2 * l, dh - 2), c1 = min(2 * l + 128, dh - 2);
#pragma unroll 4
  for (int j = 0; j < nrow; ++j) {
    const uint16_t* vj = vs + j * ldv;
    const float v0 = bf2f(vj[c0]), v1 = bf2f(vj[c0 + 1]);
    const float v2 = bf2f(vj[c1]), v3 = bf2f(vj[c1 + 1]);
    const f32x4 pa = *reinterpret_cast<const f32x4*>(pw + j * 8);
    const f32x4 pb = G > 4 ? *reinterpret_cast<const f32x4*>(pw + j * 8 + 4) : f32x4{};
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const float p = g < 4 ? pa[g] : pb[g - 4];
      o[g][0] += p * v0;
      o[g][1] += p * v1;
      o[g][2] += p * v2;
      o[g][3] += p * v3;
    }
  }
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    if (g < G) {
      const int a = h * G + g;
      float* yo = w.yex + (((int64_t)u * w.nse + e) * Hq + a) * dh;
      if (2 * l < dh) {
        yo[2 * l] = o[g][0];
        yo[2 * l + 1] = o[g][1];
      }
      if (2 * l + 128 < dh) {
        yo[2 * l + 128] = o[g][2];
        yo[2 * l + 129] = o[g][3];
      }
    }
  }
  // statistics: lane (n16 = 0, kq) holds heads 4 kq + i
  if (n16 == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = 4 * kq + i;
      if (g < G) {
        float* stp = w.astat + (((int64_t)u * (w.nsl + w.nse) + w.nsl + e) * Hq + h * G + g) * 2;
        stp[0] = m[i];
        stp[1] = S[i];
      }
    }
  }
}

template <int R, int RV>
__global__ __launch_bounds__(256) void k_attend_mfma(Dims d, CachePtrs c, DecodeWs w,
                                                     const uint16_t* __restrict__ q, float ascale) {
  typedef AttnTile<R, RV> Lay;
  constexpr int NR = kAttnRows;
  constexpr int KC = Lay::KC, KS = KC / 4, NT = RV / 16, KCV = RV / 8;
  constexpr int NPC = NR * KC;                 // pieces per staged K matrix
  constexpr int NP = (NPC + 255) / 256;        // pieces per thread
  static_assert(KC % 4 == 0 && NT % 2 == 0, "ranks must be multiples of 32");
  const int b = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  extern __shared__ __attribute__((aligned(16))) float smf[];
  if (b >= w.nsl * w.nhg) {
    if (d.dh % 32 == 0)
      attend_exact_mfma(d, c, w, q, ascale, b - w.nsl * w.nhg, u, tid, smf);
    else
      attend_exact<uint16_t>(d, c, w, q, ascale, b - w.nsl * w.nhg, u, tid, smf);
    return;
  }
  uint8_t* lds = reinterpret_cast<uint8_t*>(smf);
  const int wv = tid >> 6, l = tid & 63, n16 = l & 15, kg = l >> 4;
  const int Hq = d.Hq;
  const int split = b / w.nhg, hg = b % w.nhg;
  const int row0 = split * NR, a0 = hg * 32;
  // ---- unit state, this split's top-k entries and the query fragments
  const int32_t* si = w.stepinfo + 4 * u;
  const int full = si[2], Lcur = si[0];
  int selv[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int j = min(tid + 256 * i, NPC - 1) / KC;
    selv[i] = w.topk[(int64_t)u * w.ktot + min(row0 + j, w.ktot - 1)];
  }
  // V pieces: lane l of wave wv takes rows 4 (l % 16) + {0..3} and chunks
  // 4 wv + l / 16 + 16 p, so the transposed stores below are 8-byte writes
  // of four rows that spread over the banks
  const int vjg = l & 15, vcl = l >> 4;
  int selr[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) selr[q] = w.topk[(int64_t)u * w.ktot + min(row0 + 4 * vjg + q, w.ktot - 1)];
  const int ht = wv >> 1, rt0 = 2 * (wv & 1);
  const int ah = min(a0 + 16 * ht + n16, Hq - 1);  // heads past H_q repeat the last one
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(w.qlat) + ((int64_t)u * Hq + ah) * 2 * R;
  bf16x8 ahi[KS], alo[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    ahi[ks] = ld_bf16x8(qp + (4 * ks + kg) * 8);
    alo[ks] = ld_bf16x8(qp + R + (4 * ks + kg) * 8);
  }
  if (full) return;  // the top-k kernel wrote zeros
  const int kk = n_rebuilt(d, Lcur);
  const int nrow = min(NR, kk - row0);
  if (nrow <= 0) return;
  // ---- gather the rows: K row-major, V transposed (rows past nrow: V zeroed)
  {
    const uint16_t* cks = (const uint16_t*)c.coef_k + (int64_t)u * c.Lmax * R;
    const uint16_t* cvs = (const uint16_t*)c.coef_v + (int64_t)u * c.Lmax * RV;
    constexpr int NVP = (KCV + 15) / 16;  // V chunk passes
    u16x8 xk[NP], xv[NVP][4];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int e = min(tid + 256 * i, NPC - 1);
      const int cc = e % KC;
      const int64_t pos = min(max((int64_t)selv[i], (int64_t)0), c.Lmax - 1);
      xk[i] = *reinterpret_cast<const u16x8*>(cks + pos * R + cc * 8);
    }
#pragma unroll
    for (int p = 0; p < NVP; ++p) {
      const int cc = min(4 * wv + vcl + 16 * p, KCV - 1);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t pos = min(max((int64_t)selr[q], (int64_t)0), c.Lmax - 1);
        xv[p][q] = *reinterpret_cast<const u16x8*>(cvs + pos * RV + cc * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int e = tid + 256 * i;
      if (e < NPC) {
        const int j = e / KC, cc = e % KC;
        *reinterpret_cast<u16x8*>(lds + Lay::ck + j * Lay::CKB + cc * 16) = xk[i];
      }
    }
#pragma unroll
    for (int p = 0; p < NVP; ++p) {
      const int cc = 4 * wv + vcl + 16 * p;
      if (cc < KCV) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (4 * vjg + q >= nrow) xv[p][q] = u16x8{};
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const uint32_t lo = (uint32_t)xv[p][0][x] | ((uint32_t)xv[p][1][x] << 16);
          const uint32_t hi = (uint32_t)xv[p][2][x] | ((uint32_t)xv[p][3][x] << 16);
          *reinterpret_cast<uint2*>(lds + Lay::cv + (cc * 8 + x) * Lay::CVB + 8 * vjg) = make_uint2(lo, hi);
        }
      }
    }
  }
  __syncthreads();
  // ---- logits: 16 heads x 32 rows per wave (two 16 x 16 tiles)
  float* zs = reinterpret_cast<float*>(lds + Lay::zs);
  {
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    const uint8_t* k0 = lds + Lay::ck + (16 * rt0 + n16) * Lay::CKB;
    const uint8_t* k1 = k0 + 16 * Lay::CKB;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(k0 + (4 * ks + kg) * 16);
      const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(k1 + (4 * ks + kg) * 16);
      acc0 = mfma16x16x32(ahi[ks], b0, acc0);
      acc1 = mfma16x16x32(ahi[ks], b1, acc1);
      acc0 = mfma16x16x32(alo[ks], b0, acc0);
      acc1 = mfma16x16x32(alo[ks], b1, acc1);
    }
    __syncthreads();  // every wave is done with the K rows: zs takes their space
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      zs[(16 * ht + 4 * kg + i) * Lay::ZLD + 16 * rt0 + n16] = acc0[i];
      zs[(16 * ht + 4 * kg + i) * Lay::ZLD + 16 * rt0 + 16 + n16] = acc1[i];
    }
  }
  __syncthreads();
  // ---- split-local softmax: wave w takes heads [8w, 8w + 8), lane = row
  float* pz = reinterpret_cast<float*>(lds + Lay::pz);
  {
    const int ab = 8 * wv;
    float z[8], m[8], S[8];
#pragma unroll
    for (int aa = 0; aa < 8; ++aa) {
      z[aa] = l < nrow ? zs[(ab + aa) * Lay::ZLD + l] : -INFINITY;
      m[aa] = z[aa];
    }
    wave_max_n<8>(m);
#pragma unroll
    for (int aa = 0; aa < 8; ++aa) {
      S[aa] = l < nrow ? __builtin_amdgcn_exp2f(z[aa] - m[aa]) : 0.f;
      pz[(ab + aa) * Lay::PLD + l] = S[aa];
    }
    wave_sum_n<8>(S);
    if (l < 8 && a0 + ab + l < Hq) {
      float mm = m[0], ss = S[0];
#pragma unroll
      for (int aa = 1; aa < 8; ++aa) {
        mm = l == aa ? m[aa] : mm;
        ss = l == aa ? S[aa] : ss;
      }
      float* stp = w.astat + (((int64_t)u * (w.nsl + w.nse) + split) * Hq + a0 + ab + l) * 2;
      stp[0] = mm;
      stp[1] = ss;
    }
  }
  __syncthreads();
  // ---- values: ylat[head][i] = sum_rows p[head][row] c^V[row][i], K = 64 rows
  {
    const int ht2 = wv & 1;
    const float* prow = pz + (16 * ht2 + n16) * Lay::PLD + 8 * kg;
    bf16x8 ph0, pl0, ph1, pl1;
    split8(*reinterpret_cast<const f32x4*>(prow), *reinterpret_cast<const f32x4*>(prow + 4), &ph0, &pl0);
    split8(*reinterpret_cast<const f32x4*>(prow + 32), *reinterpret_cast<const f32x4*>(prow + 36), &ph1,
           &pl1);
    const int hd = a0 + 16 * ht2 + 4 * kg;
    float* yb = w.ylat + ((int64_t)u * w.nsl + split) * Hq * RV;
#pragma unroll
    for (int t = 0; t < NT / 2; ++t) {
      const int it = (wv >> 1) * (NT / 2) + t;
      const uint8_t* vr = lds + Lay::cv + (16 * it + n16) * Lay::CVB + kg * 16;
      const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(vr);
      const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(vr + 64);
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
      y = mfma16x16x32(ph0, b0, y);
      y = mfma16x16x32(ph1, b1, y);
      y = mfma16x16x32(pl0, b0, y);
      y = mfma16x16x32(pl1, b1, y);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (hd + i < Hq) yb[(int64_t)(hd + i) * RV + 16 * it + n16] = y[i];
    }
  }
}

// --------------------------------------------------------------------------
// merge: grid (H_kv, U), 256 threads.  For the G query heads a of KV head h:
// M = max over splits, weights f = 2^(m_split - M), L = sum f S_split;
//   out[a] = (sum_exact f yex + B^V_h (sum_selected f ylat)) / L.
// --------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_merge(Dims d, CachePtrs c, DecodeWs w,
                                               float* __restrict__ out) {
  const int h = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  const int l = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = d.rv, Hq = d.Hq, G = d.G, dh = d.dh;  // everything here has the value rank
  const int nst = w.nsl + w.nse;
  extern __shared__ __attribute__((aligned(16))) float smf[];
  float* ys = smf;                 // [G][r]
  float* oe = ys + G * r;          // [G][dh] exact-row part of the output
  float* fs = oe + G * dh;         // [G][nst]
  float* Lg = fs + G * nst;        // [8]
  float* stl = Lg + 8;             // [G][nst][2]
  // ---- every load that does not need the unit state goes out first: the
  // state itself, this thread's B^V row pieces, split statistics, the first
  // 8 selected-row partials of column tid and 4 exact partials per item
  const int32_t* si = w.stepinfo + 4 * u;
  const int full = si[2], Lcur = si[0];
  constexpr int VEC = Vec16<T>::N;
  const int hf = tid & 1;
  const int rh = (r / VEC + 1) / 2 * VEC;
  const int i0 = hf ? rh : 0, i1 = hf ? r : rh;
  const T* bbase = (const T*)c.basis_v + ((int64_t)u * d.D + (int64_t)h * dh) * r;
  u16x8 br[16];
  auto load_b = [&](int cb, int ib) {
    const T* brow = bbase + (int64_t)min(cb + (tid >> 1), dh - 1) * r;
#pragma unroll
    for (int t = 0; t < 16; ++t)
      br[t] = *reinterpret_cast<const u16x8*>(brow + max(min(ib + t * VEC, i1 - VEC), 0));
  };
  load_b(0, i0);
  const float* stb = w.astat + ((int64_t)u * nst * Hq + h * G) * 2;
  float2 stv[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int x = min(tid + 256 * t, G * nst - 1);
    stv[t] = *reinterpret_cast<const float2*>(stb + ((int64_t)(x % nst) * Hq + x / nst) * 2);
  }
  const int icol = min(tid, r - 1);
  const float* ylb = w.ylat + ((int64_t)u * w.nsl * Hq + h * G) * r + icol;
  const int nsl1 = max(w.nsl, 1);
  float yv[8][8];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int g = 0; g < 8; ++g) yv[t][g] = ylb[((int64_t)min(t, nsl1 - 1) * Hq + min(g, G - 1)) * r];
  const float* yeb = w.yex + ((int64_t)u * w.nse * Hq + h * G) * dh;
  float ev[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int x = min(tid + 256 * m, G * dh - 1);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      ev[m][e] = w.nse > 0 ? yeb[((int64_t)min(e, w.nse - 1) * Hq + x / dh) * dh + x % dh] : 0.f;
  }
  if (full) return;  // the top-k kernel wrote zeros
  const int kk = n_rebuilt(d, Lcur);
  const int nl = (kk + w.rsl - 1) / w.rsl;  // selected-row splits that ran
  for (int t = 0; t * 256 < G * nst; ++t) {
    const int x = tid + 256 * t;
    if (x < G * nst) {
      const int sp = x % nst;
      const bool ran = sp < nl || sp >= w.nsl;
      float2 v = t < 2 ? stv[t] : *reinterpret_cast<const float2*>(stb + ((int64_t)sp * Hq + x / nst) * 2);
      stl[2 * ((x / nst) * nst + sp)] = ran ? v.x : -INFINITY;
      stl[2 * ((x / nst) * nst + sp) + 1] = ran ? v.y : 0.f;
    }
  }
  __syncthreads();
  // per head (a wave each): M = max over splits, f = 2^(m - M), L = sum f S
  for (int g = wv; g < G; g += 4) {
    float mx[1] = {-INFINITY};
    for (int sp = l; sp < nst; sp += 64) mx[0] = fmaxf(mx[0], stl[2 * (g * nst + sp)]);
    wave_max_n<1>(mx);
    float L[1] = {0.f};
    for (int sp = l; sp < nst; sp += 64) {
      const float m = stl[2 * (g * nst + sp)];
      const float f = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mx[0]);
      fs[g * nst + sp] = f;
      L[0] += f * stl[2 * (g * nst + sp) + 1];
    }
    wave_sum_n<1>(L);
    if (l == 0) Lg[g] = L[0];
  }
  __syncthreads();
  // selected-row part: ys[g][i] = sum over splits of f * ylat; column tid's
  // first 8 splits come from the registers loaded above
  for (int i = tid; i < r; i += 256) {
    float acc[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) acc[g] = 0.f;
    int sp0 = 0;
    if (i == tid) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (t < nl)
#pragma unroll
          for (int g = 0; g < 8; ++g)
            if (g < G) acc[g] += fs[g * nst + t] * yv[t][g];
      sp0 = 8;
    }
    const float* yp = w.ylat + ((int64_t)u * w.nsl * Hq + h * G) * r + i;
    for (; sp0 < nl; sp0 += 8) {
      float v[8][8];
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int g = 0; g < 8; ++g)
          v[t][g] = yp[((int64_t)min(sp0 + t, nl - 1) * Hq + min(g, G - 1)) * r];
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (sp0 + t < nl)
#pragma unroll
          for (int g = 0; g < 8; ++g)
            if (g < G) acc[g] += fs[g * nst + sp0 + t] * v[t][g];
    }
#pragma unroll
    for (int g = 0; g < 8; ++g)
      if (g < G) ys[g * r + i] = acc[g];
  }
  // exact-row part: oe[g][ch] = sum over exact splits of f * yex; the first
  // 4 splits of this thread's first 4 items come from registers
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int x = tid + 256 * m;
    if (x < G * dh) {
      const int g = x / dh;
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (e < w.nse) acc += fs[g * nst + w.nsl + e] * ev[m][e];
      for (int e = 4; e < w.nse; ++e)
        acc += fs[g * nst + w.nsl + e] * yeb[((int64_t)e * Hq + g) * dh + x % dh];
      oe[x] = acc;
    }
  }
  for (int x = tid + 1024; x < G * dh; x += 256) {
    const int g = x / dh;
    float acc = 0.f;
    for (int e = 0; e < w.nse; ++e)
      acc += fs[g * nst + w.nsl + e] * yeb[((int64_t)e * Hq + g) * dh + x % dh];
    oe[x] = acc;
  }
  __syncthreads();
  // out: thread (channel ch = tid / 2 + 128 m, half hf) dots half [i0, i1)
  // of B^V row h dh + ch with ys[g]; halves combined by a lane shuffle
  for (int cb = 0; cb < dh; cb += 128) {
    const int ch = cb + (tid >> 1);
    float acc[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) acc[g] = 0.f;
    for (int ib = i0; ib < i1; ib += 16 * VEC) {
      if (cb > 0 || ib > i0) load_b(cb, ib);
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        if (ib + t * VEC < i1) {
          const T* bv = reinterpret_cast<const T*>(&br[t]);
#pragma unroll
          for (int g = 0; g < 8; ++g) {
            if (g < G) {
              const float* yg = ys + g * r + ib + t * VEC;
#pragma unroll
              for (int x = 0; x < VEC; x += 4) {
                const f32x4 y4 = *reinterpret_cast<const f32x4*>(yg + x);
                acc[g] += Elem<T>::ld(bv, x) * y4[0] + Elem<T>::ld(bv, x + 1) * y4[1] +
                          Elem<T>::ld(bv, x + 2) * y4[2] + Elem<T>::ld(bv, x + 3) * y4[3];
              }
            }
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < 8; ++g) acc[g] += __shfl_xor(acc[g], 1);
    if (ch < dh) {
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        if (g < G && (g & 1) == hf) {  // the two lanes of a channel share the stores
          const int a = h * G + g;
          out[((int64_t)u * Hq + a) * dh + ch] = (acc[g] + oe[g * dh + ch]) / Lg[g];
        }
      }
    }
  }
}

// --------------------------------------------------------------------------
// merge for bf16 storage: grid (nparts H_kv, U), 256 threads; block
// (h, part) writes the part-th share of head h's channel tiles (every part
// forms the split combination itself).  Same combination as
// k_merge; the selected-row partials are read as 16-byte vectors (thread t:
// coefficients 4 (t % 64) .. + 3 of heads t / 64 and t / 64 + 4), and
// B^V_h (sum_sel f ylat) runs on MFMA 16x16x32: A = 16 channels of B^V_h
// straight from memory (K = coefficient index), B = the G head vectors as
// bf16 hi + lo pairs (two MFMAs, ~16 mantissa bits), D = channels x heads.
// Wave w takes the part's channel tiles w, w + 4, ...
// --------------------------------------------------------------------------
constexpr int kMergeCT = 4;  // channel tiles per wave (head_dim <= 256)
__global__ __launch_bounds__(256) void k_merge_mfma(Dims d, CachePtrs c, DecodeWs w, int nparts,
                                                    float* __restrict__ out) {
  const int h = blockIdx.x / nparts, part = blockIdx.x % nparts, u = blockIdx.y, tid = threadIdx.x;
  const int l = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = l & 15, kq = l >> 4;
  const int r = d.rv, Hq = d.Hq, G = d.G, dh = d.dh;  // everything here has the value rank
  const int nst = w.nsl + w.nse;
  const int nks = r / 32, nct = (dh + 15) / 16;
  const int ctper = (nct + nparts - 1) / nparts;  // channel tiles of this block: part * ctper + ...
  extern __shared__ __attribute__((aligned(16))) float smf[];
  const int ldy = r + 4;           // ys row stride: the heads' rows start 4 banks apart
  float* ys = smf;                 // [G][ldy]
  float* oe = ys + G * ldy;        // [G][dh] exact-row part of the output
  float* fs = oe + G * dh;         // [G][nst]
  float* Lg = fs + G * nst;        // [8]
  float* stl = Lg + 8;             // [G][nst][2]
  // ---- loads that do not need the unit state go out first
  const int32_t* si = w.stepinfo + 4 * u;
  const int full = si[2], Lcur = si[0];
  const float* stb = w.astat + ((int64_t)u * nst * Hq + h * G) * 2;
  float2 stv[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int x = min(tid + 256 * t, G * nst - 1);
    stv[t] = *reinterpret_cast<const float2*>(stb + ((int64_t)(x % nst) * Hq + x / nst) * 2);
  }
  // selected-row partials: coefficients i4 .. i4 + 3 of heads gq and gq + 4,
  // first 8 splits
  const int i4 = min(4 * l, r - 4), gq = tid >> 6;
  const float* ylb = w.ylat + ((int64_t)u * w.nsl * Hq + h * G) * r + i4;
  const int nsl1 = max(w.nsl, 1);
  f32x4 yv[8][2];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int e = 0; e < 2; ++e)
      yv[t][e] = *reinterpret_cast<const f32x4*>(
          ylb + ((int64_t)min(t, nsl1 - 1) * Hq + min(gq + 4 * e, G - 1)) * r);
  const float* yeb = w.yex + ((int64_t)u * w.nse * Hq + h * G) * dh;
  float ev[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int x = min(tid + 256 * m, G * dh - 1);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      ev[m][e] = w.nse > 0 ? yeb[((int64_t)min(e, w.nse - 1) * Hq + x / dh) * dh + x % dh] : 0.f;
  }
  // B^V_h fragments: channel tile ct = part * ctper + wv + 4 m, rows clamped into the head
  const uint16_t* bbase = (const uint16_t*)c.basis_v + ((int64_t)u * d.D + (int64_t)h * dh) * r;
  bf16x8 bfr[kMergeCT][8];
#pragma unroll
  for (int m = 0; m < kMergeCT; ++m) {
    const int ctm = part * ctper + wv + 4 * m;
    const int ch = min(ctm * 16 + n16, dh - 1);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      if (wv + 4 * m < ctper && ctm < nct && ks < nks)
        bfr[m][ks] = ld_bf16x8(bbase + (int64_t)ch * r + 32 * ks + 8 * kq);
  }
  if (full) return;  // the top-k kernel wrote zeros
  const int kk = n_rebuilt(d, Lcur);
  const int nl = (kk + w.rsl - 1) / w.rsl;  // selected-row splits that ran
  for (int t = 0; t * 256 < G * nst; ++t) {
    const int x = tid + 256 * t;
    if (x < G * nst) {
      const int sp = x % nst;
      const bool ran = sp < nl || sp >= w.nsl;
      float2 v = t < 2 ? stv[t] : *reinterpret_cast<const float2*>(stb + ((int64_t)sp * Hq + x / nst) * 2);
      stl[2 * ((x / nst) * nst + sp)] = ran ? v.x : -INFINITY;
      stl[2 * ((x / nst) * nst + sp) + 1] = ran ? v.y : 0.f;
    }
  }
  __syncthreads();
  // per head (a wave each): M = max over splits, f = 2^(m - M), L = sum f S
  for (int g = wv; g < G; g += 4) {
    float mx[1] = {-INFINITY};
    for (int sp = l; sp < nst; sp += 64) mx[0] = fmaxf(mx[0], stl[2 * (g * nst + sp)]);
    wave_max_n<1>(mx);
    float L[1] = {0.f};
    for (int sp = l; sp < nst; sp += 64) {
      const float m = stl[2 * (g * nst + sp)];
      const float f = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mx[0]);
      fs[g * nst + sp] = f;
      L[0] += f * stl[2 * (g * nst + sp) + 1];
    }
    wave_sum_n<1>(L);
    if (l == 0) Lg[g] = L[0];
  }
  __syncthreads();
  // selected-row part: ys[g][i] = sum over splits of f * ylat (coefficient
  // groups past 64 * 4 loop; splits past 8 are read here)
  for (int ib = 4 * l; ib < r; ib += 256) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int g = gq + 4 * e;
      if (g >= G) continue;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const float* yp = w.ylat + ((int64_t)u * w.nsl * Hq + h * G + g) * r + ib;
      int sp0 = 0;
      if (ib == 4 * l && ib == i4) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if (t < nl) acc += fs[g * nst + t] * yv[t][e];
        sp0 = 8;
      }
      for (int sp = sp0; sp < nl; ++sp)
        acc += fs[g * nst + sp] * *reinterpret_cast<const f32x4*>(yp + (int64_t)sp * Hq * r);
      *reinterpret_cast<f32x4*>(ys + g * ldy + ib) = acc;
    }
  }
  // exact-row part: oe[g][ch] = sum over exact splits of f * yex
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int x = tid + 256 * m;
    if (x < G * dh) {
      const int g = x / dh;
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (e < w.nse) acc += fs[g * nst + w.nsl + e] * ev[m][e];
      for (int e = 4; e < w.nse; ++e)
        acc += fs[g * nst + w.nsl + e] * yeb[((int64_t)e * Hq + g) * dh + x % dh];
      oe[x] = acc;
    }
  }
  for (int x = tid + 1024; x < G * dh; x += 256) {
    const int g = x / dh;
    float acc = 0.f;
    for (int e = 0; e < w.nse; ++e)
      acc += fs[g * nst + w.nsl + e] * yeb[((int64_t)e * Hq + g) * dh + x % dh];
    oe[x] = acc;
  }
  __syncthreads();
  // B operands (shared by the wave's channel tiles): head n16's coefficients
  // 32 ks + 8 kq .. + 7 as bf16 hi / lo
  bf16x8 bh[8], bl[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    if (ks < nks && n16 < G) {
      const float* yr = ys + n16 * ldy + 32 * ks + 8 * kq;
      split8(*reinterpret_cast<const f32x4*>(yr), *reinterpret_cast<const f32x4*>(yr + 4), &bh[ks], &bl[ks]);
    } else {
      bh[ks] = __builtin_bit_cast(bf16x8, u16x8{});
      bl[ks] = bh[ks];
    }
  }
#pragma unroll
  for (int m = 0; m < kMergeCT; ++m) {
    const int ct = part * ctper + wv + 4 * m;
    if (wv + 4 * m >= ctper || ct >= nct) break;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ks < nks) {
        acc = mfma16x16x32(bfr[m][ks], bh[ks], acc);
        acc = mfma16x16x32(bfr[m][ks], bl[ks], acc);
      }
    }
    // lane: channels ct * 16 + 4 kq + i, head n16
    const int ch0 = ct * 16 + 4 * kq;
    if (n16 < G && ch0 < dh) {
      const float inv = 1.f / Lg[n16];
      f32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = (acc[i] + oe[n16 * dh + ch0 + i]) * inv;
      float* op = out + ((int64_t)u * Hq + h * G + n16) * dh + ch0;
      if (ch0 + 4 <= dh) {
        *reinterpret_cast<f32x4*>(op) = o;
      } else {
        for (int i = 0; i < dh - ch0; ++i) op[i] = o[i];
      }
    }
  }
}

static size_t merge_lds(const Dims& d, const DecodeWs& w) {  // (k_merge_mfma pads ys rows by 4)
  return ((size_t)d.G * (d.rv + 4 + d.dh) + (size_t)3 * d.G * (w.nsl + w.nse) + 8) * sizeof(float);
}


template <typename T>
static hipError_t launch_attend_t(const Dims& d, int U, const void* q, const CachePtrs& c,
                                  const DecodeWs& w, hipStream_t st) {
  static size_t done = 0;
  if (w.attend_lds <= 0) return hipErrorInvalidValue;
  hipError_t e = allow_lds(&k_attend<T>, (size_t)w.attend_lds, &done);
  if (e != hipSuccess) return e;
  const float ascale = kLog2e / sqrtf((float)d.dh);
  hipLaunchKernelGGL(k_attend<T>, dim3(w.nsl * w.nhg + w.nse * ((d.Hkv + 3) / 4), U), dim3(256),
                     w.attend_lds, st, d,
                     c, w, (const T*)q, ascale);
  return hipGetLastError();
}

template <int R, int RV>
static hipError_t launch_attend_mfma(const Dims& d, int U, const void* q, const CachePtrs& c,
                                     const DecodeWs& w, hipStream_t st) {
  static size_t done = 0;
  if (w.attend_lds <= 0) return hipErrorInvalidValue;
  hipError_t e = allow_lds(&k_attend_mfma<R, RV>, (size_t)w.attend_lds, &done);
  if (e != hipSuccess) return e;
  const float ascale = kLog2e / sqrtf((float)d.dh);
  hipLaunchKernelGGL((k_attend_mfma<R, RV>), dim3(w.nsl * w.nhg + w.nse * ((d.Hkv + 3) / 4), U),
                     dim3(256), w.attend_lds, st, d, c, w, (const uint16_t*)q, ascale);
  return hipGetLastError();
}

// bf16 rank pairs with a kernel: equal ranks, and values at 1.5x the keys
// (the key-to-value split the review mentions) where that rank exists
bool attend_ranks_supported(int r, int rv) {
  if (r == rv) return r == 32 || r == 64 || r == 128 || r == 192 || r == 256;
  return (r == 128 && rv == 192) || (r == 64 && rv == 96);
}

hipError_t launch_attend(const Dims& d, int U, const void* q, const CachePtrs& c,
                         const DecodeWs& w, hipStream_t st) {
  if (d.dtype == 0) return launch_attend_t<float>(d, U, q, c, w, st);
  if (d.r == d.rv) {
    switch (d.r) {
      case 32: return launch_attend_mfma<32, 32>(d, U, q, c, w, st);
      case 64: return launch_attend_mfma<64, 64>(d, U, q, c, w, st);
      case 128: return launch_attend_mfma<128, 128>(d, U, q, c, w, st);
      case 192: return launch_attend_mfma<192, 192>(d, U, q, c, w, st);
      case 256: return launch_attend_mfma<256, 256>(d, U, q, c, w, st);
      default: return hipErrorInvalidValue;
    }
  }
  if (d.r == 128 && d.rv == 192) return launch_attend_mfma<128, 192>(d, U, q, c, w, st);
  if (d.r == 64 && d.rv == 96) return launch_attend_mfma<64, 96>(d, U, q, c, w, st);
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_merge_t(const Dims& d, int U, const CachePtrs& c, const DecodeWs& w,
                                 float* out, hipStream_t st) {
  static size_t done = 0;
  const size_t lds = merge_lds(d, w);
  hipError_t e = allow_lds(&k_merge<T>, lds, &done);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_merge<T>, dim3(d.Hkv, U), dim3(256), lds, st, d, c, w, out);
  return hipGetLastError();
}

hipError_t launch_merge(const Dims& d, int U, const CachePtrs& c, const DecodeWs& w, float* out,
                        hipStream_t st) {
  if (d.dtype == 0) return launch_merge_t<float>(d, U, c, w, out, st);
  static size_t done = 0;
  const size_t lds = merge_lds(d, w);
  hipError_t e = allow_lds(&k_merge_mfma, lds, &done);
  if (e != hipSuccess) return e;
  // two blocks per KV head (halves of its channel tiles): twice the blocks
  // in flight for the same loads of the split partials
  const int nparts = (d.dh + 15) / 16 >= 2 ? 2 : 1;
  hipLaunchKernelGGL(k_merge_mfma, dim3(nparts * d.Hkv, U), dim3(256), lds, st, d, c, w, nparts, out);
  return hipGetLastError();
}

}  // namespace kvlr
