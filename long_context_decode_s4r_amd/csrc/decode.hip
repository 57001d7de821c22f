// Decode-step kernels: prologue (append + query coefficients + window),
// latent scoring, pooled top-k selection, sparse reconstruction + exact
// attention (split over rows), merge of the splits.
//
// Method: S^4R review (pith.science/paper/2608.00528): 'What carries the
// argument' (latent-space relevance scoring between a sliding window of query
// coefficients and the cached key coefficients, Eqs. 8-10; sparse
// reconstruction of the selected positions, Eqs. 13-16; exact attention with
// the uncompressed sinks), 'Core claim' (queries projected into the key
// subspace), 'Referee Report' major comment 2 (Z = C_Q C_K^T / sqrt(r)).
//
// Latent softmax bookkeeping.  Each window row (one query coefficient vector
// of one earlier step) keeps the running max m and sum S of its softmax over
// the candidates in base 2 (rowstat).  Candidates only grow, by one position
// per step (the token leaving the exact recent window), so a row's (m, S) is
// updated with that one logit in the prologue and stays exact.  Only the G
// rows of the current step need a full pass: the scoring kernel writes their
// logits to a spill buffer together with per-split (m, S) partials, and the
// selection kernel merges them before adding their probabilities.  The key
// coefficients are therefore read once per step.
#include "common.h"

#include <float.h>
#include <math.h>

namespace kvlr {

static inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

void decode_tiling(const Dims& d, int64_t U, int64_t Lmax, int* Lc_cap, int* nsplit, int* chunk,
                   int* nsa) {
  int64_t lc = Lmax - d.s - d.nrec;
  if (lc < 1) lc = 1;
  lc = round_up(lc, 64);
  *Lc_cap = (int)lc;
  int64_t target = (1024 + U - 1) / U;
  if (target < 1) target = 1;
  int64_t maxsplit = lc / 256;
  if (maxsplit < 1) maxsplit = 1;
  int64_t ns = target < maxsplit ? target : maxsplit;
  int64_t ch = round_up((lc + ns - 1) / ns, 32);
  ns = (lc + ch - 1) / ch;
  *nsplit = (int)ns;
  *chunk = (int)ch;
  *nsa = (d.s + d.nrec + d.k + 63) / 64;
}

__device__ __forceinline__ int wrap_slot(int x, int W) { return ((x % W) + W) % W; }

// --------------------------------------------------------------------------
// prologue: grid (ceil(r/64), U, 2 {K, V}), 256 threads
//   K part: c^K(new) = k_cat . B^K, c_q[g] = q_cat[g] . B^K (window push),
//           old window rows' (m, S) updated with the entering candidate.
//   V part: c^V(new) = v_cat . B^V.
//   chunk 0 of each part pushes the exact k / v into the recent ring.
// --------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_prologue(Dims d, CachePtrs c, const T* __restrict__ q,
                                                  const T* __restrict__ kn,
                                                  const T* __restrict__ vn,
                                                  int32_t* __restrict__ stepinfo, float qscale) {
  const int chunk = blockIdx.x, u = blockIdx.y, kind = blockIdx.z;
  const int tid = threadIdx.x;
  const int D = d.D, r = d.r, G = d.G, W = d.W;
  const int32_t Lcur = c.lens[2 * u], steps = c.lens[2 * u + 1];
  const bool full = (int64_t)Lcur >= c.Lmax;
  if (chunk == 0 && kind == 0 && tid == 0) {
    stepinfo[4 * u + 0] = Lcur;
    stepinfo[4 * u + 1] = steps;
    stepinfo[4 * u + 2] = full ? 1 : 0;
    stepinfo[4 * u + 3] = 0;
  }
  if (full) return;
  const int64_t p = Lcur;
  const int slot = steps % W;
  const int nvec = kind == 0 ? 1 + G : 1;
  extern __shared__ float sm[];
  float* xs = sm;                    // [nvec][D]
  float* red = xs + nvec * D;        // [4][nvec][64]
  float* ce = red + 4 * nvec * 64;   // [r]
  const T* x0 = (kind == 0 ? kn : vn) + (int64_t)u * D;
  for (int i = tid; i < D; i += 256) xs[i] = Elem<T>::ld(x0, i);
  if (kind == 0) {
    const T* qu = q + (int64_t)u * d.Hq * d.dh;
    for (int i = tid; i < G * D; i += 256) {
      const int g = i / D, idx = i % D, h = idx / d.dh, j = idx % d.dh;
      xs[(1 + g) * D + idx] = Elem<T>::ld(qu, (int64_t)(h * G + g) * d.dh + j);
    }
  }
  __syncthreads();
  const T* B = (const T*)(kind == 0 ? c.basis_k : c.basis_v) + (int64_t)u * D * r;
  const int col = chunk * 64 + (tid & 63), rg = tid >> 6;
  float acc[9];
#pragma unroll
  for (int v = 0; v < 9; ++v) acc[v] = 0.f;
  if (col < r) {
    for (int kk = rg; kk < D; kk += 4) {
      const float b = Elem<T>::ld(B, (int64_t)kk * r + col);
#pragma unroll
      for (int v = 0; v < 9; ++v)
        if (v < nvec) acc[v] += xs[v * D + kk] * b;
    }
  }
#pragma unroll
  for (int v = 0; v < 9; ++v)
    if (v < nvec) red[(rg * nvec + v) * 64 + (tid & 63)] = acc[v];
  __syncthreads();
  if (rg == 0 && col < r) {
    for (int v = 0; v < nvec; ++v) {
      const float sum = red[(0 * nvec + v) * 64 + tid] + red[(1 * nvec + v) * 64 + tid] +
                        red[(2 * nvec + v) * 64 + tid] + red[(3 * nvec + v) * 64 + tid];
      if (v == 0) {
        T* C = (T*)(kind == 0 ? c.coef_k : c.coef_v);
        Elem<T>::st(C, ((int64_t)u * c.Lmax + p) * r + col, sum);
      } else {
        c.qwin[(((int64_t)u * W + slot) * G + (v - 1)) * r + col] = sum;
      }
    }
  }
  if (chunk != 0) return;
  {  // exact ring push
    T* ring = (T*)(kind == 0 ? c.ring_k : c.ring_v);
    const int rs = (int)(p % d.nrec);
    for (int i = tid; i < D; i += 256) ring[((int64_t)u * d.nrec + rs) * D + i] = x0[i];
  }
  if (kind != 0) return;
  // old rows: add the candidate entering the compressed set this step
  const int weff = min(steps + 1, W);
  const int nold = (weff - 1) * G;
  if (nold <= 0) return;
  const int64_t pe = (int64_t)Lcur - d.nrec;
  const T* cep = (const T*)c.coef_k + ((int64_t)u * c.Lmax + pe) * r;
  for (int i = tid; i < r; i += 256) ce[i] = Elem<T>::ld(cep, i);
  __syncthreads();
  for (int o = tid; o < nold; o += 256) {
    const int i = 1 + o / G, g = o % G;
    const int sl = wrap_slot(steps - i, W);
    const float* qr = c.qwin + (((int64_t)u * W + sl) * G + g) * r;
    float z = 0.f;
    for (int kk = 0; kk < r; ++kk) z += qr[kk] * ce[kk];
    z *= qscale;
    float* rs = c.rowstat + (((int64_t)u * W + sl) * G + g) * 2;
    const float m = rs[0], S = rs[1];
    const float mn = fmaxf(m, z);
    rs[0] = mn;
    rs[1] = S * exp2f(m - mn) + exp2f(z - mn);
  }
}

hipError_t launch_prologue(const Dims& d, int U, const void* q, const void* k_new,
                           const void* v_new, const CachePtrs& c, const DecodeWs& w,
                           hipStream_t st) {
  const int nvec = 1 + d.G;
  const size_t lds = ((size_t)nvec * d.D + 4 * nvec * 64 + d.r) * sizeof(float);
  dim3 grid((d.r + 63) / 64, U, 2);
  const float qscale = kLog2e / sqrtf((float)d.r);
  if (d.dtype == 0)
    hipLaunchKernelGGL(k_prologue<float>, grid, dim3(256), lds, st, d, c, (const float*)q,
                       (const float*)k_new, (const float*)v_new, w.stepinfo, qscale);
  else
    hipLaunchKernelGGL(k_prologue<uint16_t>, grid, dim3(256), lds, st, d, c, (const uint16_t*)q,
                       (const uint16_t*)k_new, (const uint16_t*)v_new, w.stepinfo, qscale);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// latent scoring, bf16 storage: grid (nsplit, U), 64 * ceil(W*G/32) threads.
// Wave w owns window rows [32w, 32w + 32) in "age order" (row rho = i*G + g is
// query head-group g of the step i steps ago; rows 0..G-1 are the current
// step).  The fp32 query coefficients (scaled by log2(e)/sqrt(r)) are split
// into bf16 hi + lo parts held in registers for the whole block; key
// coefficients stream through registers, 32 positions per MFMA tile.
// K-index permutation: lane (n, kg) of the B operand holds, for k-step ks, the
// 8 coefficients kg*r/2 + 8*ks + [0, 8) of position n (a contiguous run per
// lane); the A operand uses the same permutation.
// --------------------------------------------------------------------------
template <int KS>
__global__ __launch_bounds__(256) void k_score_bf16(Dims d, CachePtrs c, DecodeWs w,
                                                    float qscale) {
  constexpr int r = KS * 16, half = KS * 8;
  const int split = blockIdx.x, u = blockIdx.y;
  const int wv = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int nw = blockDim.x >> 6;
  const int32_t* si = w.stepinfo + 4 * u;
  if (si[2]) return;
  const int Lcur = si[0], steps = si[1];
  const int G = d.G, W = d.W, s = d.s;
  const int weff = min(steps + 1, W);
  const int nrows = weff * G;
  const int64_t cend = (int64_t)Lcur + 1 - d.nrec;
  const int64_t j0 = s + (int64_t)split * w.chunk;
  const int64_t j1 = min(j0 + (int64_t)w.chunk, cend);
  float* tst = w.tilestat + ((int64_t)u * w.nsplit + split) * G * 2;
  extern __shared__ float red[];  // [nw][chunk]

  const int mm = l & 31, kg = l >> 5;
  bf16x8 ahi[KS], alo[KS];
  {
    const int rho = 32 * wv + mm;
    const float* qr = nullptr;
    if (rho < nrows) {
      const int i = rho / G, g = rho % G;
      const int sl = wrap_slot(steps - i, W);
      qr = c.qwin + (((int64_t)u * W + sl) * G + g) * r + kg * half;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u16x8 hv, lv;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = qr ? qr[8 * ks + e] * qscale : 0.f;
        const uint16_t hb = f2bf(x);
        hv[e] = hb;
        lv[e] = f2bf(x - bf2f(hb));
      }
      ahi[ks] = __builtin_bit_cast(bf16x8, hv);
      alo[ks] = __builtin_bit_cast(bf16x8, lv);
    }
  }
  float mrow[16], irow[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int rr = 32 * wv + acc_row32(i, l);
    if (rr < G || rr >= nrows) {
      mrow[i] = FLT_MAX;
      irow[i] = 0.f;
    } else {
      const int ii = rr / G, g = rr % G;
      const int sl = wrap_slot(steps - ii, W);
      const float* rs = c.rowstat + (((int64_t)u * W + sl) * G + g) * 2;
      mrow[i] = rs[0];
      irow[i] = 1.f / rs[1];
    }
  }
  float nm[4], ns[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    nm[i] = -INFINITY;
    ns[i] = 0.f;
  }
  const uint16_t* base = (const uint16_t*)c.coef_k + (int64_t)u * c.Lmax * r + kg * half;
  float* spill = w.spill + (int64_t)u * G * w.Lc_cap;
  for (int64_t p0 = j0; p0 < j1; p0 += 32) {
    const int64_t jn = p0 + mm;
    const bool pv = jn < j1;
    const uint16_t* src = base + (pv ? jn : j0) * r;
    bf16x8 b[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) b[ks] = ld_bf16x8(src + 8 * ks);
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      acc = mfma32x32x16(ahi[ks], b[ks], acc);
      acc = mfma32x32x16(alo[ks], b[ks], acc);
    }
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) ps += exp2f(acc[i] - mrow[i]) * irow[i];
    ps += __shfl_xor(ps, 32);
    if (l < 32) red[wv * w.chunk + (int)(p0 - j0) + mm] = ps;
    if (wv == 0 && pv) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * kg + i;
        if (row < G) {
          const float z = acc[i];
          spill[(int64_t)row * w.Lc_cap + (jn - s)] = z;
          const float mx = fmaxf(nm[i], z);
          ns[i] = ns[i] * exp2f(nm[i] - mx) + exp2f(z - mx);
          nm[i] = mx;
        }
      }
    }
  }
  __syncthreads();
  float* partial = w.partial + (int64_t)u * w.Lc_cap + (j0 - s);
  for (int t = threadIdx.x; t < (int)(j1 - j0); t += blockDim.x) {
    float sum = 0.f;
    for (int q2 = 0; q2 < nw; ++q2) sum += red[q2 * w.chunk + t];
    partial[t] = sum;
  }
  if (wv == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float m = nm[i], sm = ns[i];
      for (int o = 1; o < 32; o <<= 1) {
        const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(sm, o);
        const float mx = fmaxf(m, m2);
        const float a = (m == -INFINITY) ? 0.f : sm * exp2f(m - mx);
        const float b2 = (m2 == -INFINITY) ? 0.f : s2 * exp2f(m2 - mx);
        sm = a + b2;
        m = mx;
      }
      const int row = 4 * kg + i;
      if (mm == 0 && row < G) {
        tst[row * 2 + 0] = m;
        tst[row * 2 + 1] = sm;
      }
    }
  }
}

// latent scoring, fp32 storage: plain fp32 dot products, one position per
// thread, window rows staged in LDS.
__global__ __launch_bounds__(256) void k_score_f32(Dims d, CachePtrs c, DecodeWs w, float qscale) {
  const int split = blockIdx.x, u = blockIdx.y;
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
  float* red = ri + W * G;          // [256][2] for the new-row stats
  for (int e = threadIdx.x; e < nrows * r; e += blockDim.x) {
    const int rho = e / r, k = e % r, i = rho / G, g = rho % G;
    const int sl = wrap_slot(steps - i, W);
    qs[e] = c.qwin[(((int64_t)u * W + sl) * G + g) * r + k] * qscale;
  }
  for (int rho = threadIdx.x; rho < nrows; rho += blockDim.x) {
    const int i = rho / G, g = rho % G;
    const int sl = wrap_slot(steps - i, W);
    const float* rs = c.rowstat + (((int64_t)u * W + sl) * G + g) * 2;
    rm[rho] = rs[0];
    ri[rho] = rho < G ? 0.f : 1.f / rs[1];
  }
  __syncthreads();
  float nm[8], ns[8];
  for (int g = 0; g < 8; ++g) {
    nm[g] = -INFINITY;
    ns[g] = 0.f;
  }
  const float* CK = (const float*)c.coef_k + (int64_t)u * c.Lmax * r;
  for (int64_t j = j0 + threadIdx.x; j < j1; j += blockDim.x) {
    const float* cj = CK + j * r;
    float ps = 0.f;
    for (int rho = 0; rho < nrows; ++rho) {
      float z = 0.f;
      for (int k = 0; k < r; ++k) z += qs[rho * r + k] * cj[k];
      if (rho < G) {
        w.spill[((int64_t)u * G + rho) * w.Lc_cap + (j - s)] = z;
        const float mx = fmaxf(nm[rho], z);
        ns[rho] = ns[rho] * exp2f(nm[rho] - mx) + exp2f(z - mx);
        nm[rho] = mx;
      } else {
        ps += exp2f(z - rm[rho]) * ri[rho];
      }
    }
    w.partial[(int64_t)u * w.Lc_cap + (j - s)] = ps;
  }
  // new-row statistics: block reduction per row (fixed order)
  float* tst = w.tilestat + ((int64_t)u * w.nsplit + split) * G * 2;
  for (int g = 0; g < G; ++g) {
    red[threadIdx.x * 2] = nm[g];
    red[threadIdx.x * 2 + 1] = ns[g];
    __syncthreads();
    if (threadIdx.x == 0) {
      float m = -INFINITY, S = 0.f;
      for (int t = 0; t < blockDim.x; ++t) {
        const float m2 = red[2 * t], s2 = red[2 * t + 1];
        if (s2 == 0.f) continue;
        const float mx = fmaxf(m, m2);
        S = (m == -INFINITY ? 0.f : S * exp2f(m - mx)) + s2 * exp2f(m2 - mx);
        m = mx;
      }
      tst[g * 2] = m;
      tst[g * 2 + 1] = S;
    }
    __syncthreads();
  }
}

hipError_t launch_score(const Dims& d, int U, const CachePtrs& c, const DecodeWs& w,
                        hipStream_t st) {
  const float qscale = kLog2e / sqrtf((float)d.r);
  dim3 grid(w.nsplit, U);
  if (d.dtype == 0) {
    const size_t lds = ((size_t)d.W * d.G * d.r + 2 * d.W * d.G + 512) * sizeof(float);
    hipLaunchKernelGGL(k_score_f32, grid, dim3(256), lds, st, d, c, w, qscale);
    return hipGetLastError();
  }
  const int nw = (d.W * d.G + 31) / 32;
  const size_t lds = (size_t)nw * w.chunk * sizeof(float);
  switch (d.r) {
    case 128: hipLaunchKernelGGL(k_score_bf16<8>, grid, dim3(64 * nw), lds, st, d, c, w, qscale); break;
    case 192: hipLaunchKernelGGL(k_score_bf16<12>, grid, dim3(64 * nw), lds, st, d, c, w, qscale); break;
    case 256: hipLaunchKernelGGL(k_score_bf16<16>, grid, dim3(64 * nw), lds, st, d, c, w, qscale); break;
    case 64: hipLaunchKernelGGL(k_score_bf16<4>, grid, dim3(64 * nw), lds, st, d, c, w, qscale); break;
    case 32: hipLaunchKernelGGL(k_score_bf16<2>, grid, dim3(64 * nw), lds, st, d, c, w, qscale); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// selection: one 1024-thread block per unit.
//   1. merge the current rows' split statistics -> rowstat of this slot
//   2. score[j] = partial[j] + sum_g exp2(z_g[j] - m_g) / S_g
//   3. pooled key = max over |d| <= kappa/2 inside the candidates (bits of a
//      non-negative float order like the float)
//   4. radix select (4 x 8 bits, most significant first) of the k-th key T
//   5. ordered compaction: keys > T, then keys == T in index order until k
// --------------------------------------------------------------------------
__device__ __forceinline__ int block_excl_scan_flag(bool f, int* wsum, int* total) {
  // 1024 threads = 16 waves; wsum: 16 ints of LDS
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const unsigned long long bal = __ballot(f);
  const int within = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) wsum[wid] = __popcll(bal);
  __syncthreads();
  int before = 0, tot = 0;
  for (int i = 0; i < 16; ++i) {
    const int v = wsum[i];
    if (i < wid) before += v;
    tot += v;
  }
  __syncthreads();
  *total = tot;
  return before + within;
}

__global__ __launch_bounds__(1024) void k_select(Dims d, CachePtrs c, DecodeWs w,
                                                 int32_t* __restrict__ topk_user,
                                                 float* __restrict__ scores_user) {
  const int u = blockIdx.x, tid = threadIdx.x;
  const int32_t* si = w.stepinfo + 4 * u;
  const int G = d.G, W = d.W, s = d.s, k = d.k;
  if (si[2]) {
    if (topk_user)
      for (int i = tid; i < k; i += blockDim.x) topk_user[(int64_t)u * k + i] = -1;
    return;
  }
  const int Lcur = si[0], steps = si[1];
  const int slot = steps % W;
  const int nc = Lcur + 1 - d.nrec - s;
  __shared__ float Mg[8], Ig[8];
  __shared__ unsigned int hist[256];
  __shared__ int wsum[16];
  __shared__ unsigned int sh_prefix;
  __shared__ int sh_remaining;
  if (tid < G) {
    float M = -INFINITY, S = 0.f;
    const float* tp = w.tilestat + (int64_t)u * w.nsplit * G * 2;
    for (int sp = 0; sp < w.nsplit; ++sp) {
      const float m2 = tp[(sp * G + tid) * 2], s2 = tp[(sp * G + tid) * 2 + 1];
      if (!(s2 > 0.f)) continue;
      const float mx = fmaxf(M, m2);
      S = (M == -INFINITY ? 0.f : S * exp2f(M - mx)) + s2 * exp2f(m2 - mx);
      M = mx;
    }
    Mg[tid] = M;
    Ig[tid] = 1.f / S;
    float* rs = c.rowstat + (((int64_t)u * W + slot) * G + tid) * 2;
    rs[0] = M;
    rs[1] = S;
  }
  __syncthreads();
  const float* part = w.partial + (int64_t)u * w.Lc_cap;
  const float* spill = w.spill + (int64_t)u * G * w.Lc_cap;
  float* score = w.score + (int64_t)u * w.Lc_cap;
  for (int j = tid; j < nc; j += blockDim.x) {
    float sc = part[j];
    for (int g = 0; g < G; ++g) sc += exp2f(spill[(int64_t)g * w.Lc_cap + j] - Mg[g]) * Ig[g];
    score[j] = sc;
    if (scores_user) scores_user[(int64_t)u * c.Lmax + s + j] = sc;
  }
  __threadfence_block();
  __syncthreads();
  uint32_t* keys = w.keys + (int64_t)u * w.Lc_cap;
  const int hk = d.kappa >> 1;
  for (int j = tid; j < nc; j += blockDim.x) {
    float mx = score[j];
    for (int dd = 1; dd <= hk; ++dd) {
      if (j - dd >= 0) mx = fmaxf(mx, score[j - dd]);
      if (j + dd < nc) mx = fmaxf(mx, score[j + dd]);
    }
    keys[j] = __float_as_uint(mx);
  }
  __threadfence_block();
  __syncthreads();
  const int kk = min(k, nc);
  int32_t* out = w.topk + (int64_t)u * k;
  if (kk > 0) {
    unsigned int prefix = 0, mask = 0;
    int remaining = kk;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int j = tid; j < nc; j += blockDim.x) {
        const unsigned int key = keys[j];
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        int cum = 0, sel = 0;
        for (int b = 255; b >= 0; --b) {
          const int h = (int)hist[b];
          if (cum + h >= remaining) {
            sel = b;
            break;
          }
          cum += h;
        }
        sh_prefix = prefix | ((unsigned int)sel << shift);
        sh_remaining = remaining - cum;
      }
      __syncthreads();
      prefix = sh_prefix;
      remaining = sh_remaining;
      mask |= 255u << shift;
    }
    const unsigned int T = prefix;
    const int need_eq = remaining;
    int base = 0, eq_base = 0;
    for (int c0 = 0; c0 < nc; c0 += blockDim.x) {
      const int j = c0 + tid;
      const unsigned int key = j < nc ? keys[j] : 0u;
      const bool gt = j < nc && key > T;
      const bool eq = j < nc && key == T;
      int eq_tot, sel_tot;
      const int eq_rank = eq_base + block_excl_scan_flag(eq, wsum, &eq_tot);
      const bool take = gt || (eq && eq_rank < need_eq);
      const int pos = base + block_excl_scan_flag(take, wsum, &sel_tot);
      if (take) {
        out[pos] = s + j;
        if (topk_user) topk_user[(int64_t)u * k + pos] = s + j;
      }
      base += sel_tot;
      eq_base += eq_tot;
    }
  }
  if (topk_user)
    for (int i = kk + tid; i < k; i += blockDim.x) topk_user[(int64_t)u * k + i] = -1;
}

hipError_t launch_select(const Dims& d, int U, const CachePtrs& c, const DecodeWs& w,
                         int32_t* topk_user, float* scores_user, hipStream_t st) {
  hipLaunchKernelGGL(k_select, dim3(U), dim3(1024), 0, st, d, c, w, topk_user, scores_user);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// sparse reconstruction + exact attention: grid (nsa, H_kv, U), 256 threads.
// Split `split` owns rows [64 split, 64 split + 64) of the row list
//   [0, s)            sinks (exact)
//   [s, s + nrec)     recent ring (exact)
//   [s + nrec, R)     selected positions, reconstructed as c . B^T
// For bf16 the reconstruction is an MFMA 32x32x16 product [rows x r] x
// [r x d_h] per KV head (the basis rows of head h are contiguous in r);
// fp32 storage uses plain dot products.  Then for the G query heads of this
// KV head: logits, split-local softmax (max, sum) and sum p.V into part.
// --------------------------------------------------------------------------
template <typename T, int KS>
__global__ __launch_bounds__(256) void k_attend(Dims d, CachePtrs c, DecodeWs w,
                                                const T* __restrict__ q, float sm_scale) {
  const int split = blockIdx.x, h = blockIdx.y, u = blockIdx.z;
  const int tid = threadIdx.x;
  const int32_t* si = w.stepinfo + 4 * u;
  if (si[2]) return;
  const int Lcur = si[0];
  const int s = d.s, nrec = d.nrec, dh = d.dh, G = d.G, D = d.D, r = d.r;
  const int nc = Lcur + 1 - nrec - s;
  const int kk = min(d.k, nc);
  const int R = s + nrec + kk;
  const int row0 = split * 64;
  const int ldk = dh + 1;
  float* part = w.part + (int64_t)u * d.Hq * w.nsa * (dh + 2);
  if (row0 >= R) {
    for (int e = tid; e < G * (dh + 2); e += blockDim.x) {
      const int g = e / (dh + 2), j = e % (dh + 2);
      part[((int64_t)(h * G + g) * w.nsa + split) * (dh + 2) + j] = (j == 0) ? -INFINITY : 0.f;
    }
    return;
  }
  extern __shared__ float sm[];
  float* Kh = sm;                 // [64][dh + 1]
  float* Vh = Kh + 64 * ldk;      // [64][dh + 1]
  float* qs = Vh + 64 * ldk;      // [G][dh]
  float* pl = qs + G * dh;        // [G][64]
  float* hs = pl + G * 64;        // [G][2]
  for (int e = tid; e < G * dh; e += blockDim.x) {
    const int g = e / dh, j = e % dh;
    qs[e] = Elem<T>::ld(q, ((int64_t)u * d.Hq + h * G + g) * dh + j);
  }
  const int32_t* sel = w.topk + (int64_t)u * d.k;
  if constexpr (KS > 0) {
    constexpr int half = KS * 8;
    const int wv = tid >> 6, l = tid & 63, mm = l & 31, kg = l >> 5;
    const int ncb = dh / 32;
    for (int kind = 0; kind < 2; ++kind) {
      const uint16_t* Cb = (const uint16_t*)(kind ? c.coef_v : c.coef_k);
      const uint16_t* Bb = (const uint16_t*)(kind ? c.basis_v : c.basis_k);
      float* dst = kind ? Vh : Kh;
      for (int mb = 0; mb < 2; ++mb) {
        const int row = row0 + 32 * mb + mm;
        const bool rec = row >= s + nrec && row < R;
        const int64_t pos = rec ? sel[row - s - nrec] : 0;
        const uint16_t* asrc = Cb + ((int64_t)u * c.Lmax + pos) * (KS * 16) + kg * half;
        bf16x8 a[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (rec)
            a[ks] = ld_bf16x8(asrc + 8 * ks);
          else
            a[ks] = __builtin_bit_cast(bf16x8, u16x8{});
        }
        for (int cb = wv; cb < ncb; cb += 4) {
          const int ch = h * dh + 32 * cb + mm;
          const uint16_t* bsrc = Bb + ((int64_t)u * D + ch) * (KS * 16) + kg * half;
          f32x16 acc = {};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) acc = mfma32x32x16(a[ks], ld_bf16x8(bsrc + 8 * ks), acc);
#pragma unroll
          for (int i = 0; i < 16; ++i) dst[(32 * mb + acc_row32(i, l)) * ldk + 32 * cb + mm] = acc[i];
        }
      }
    }
  } else {
    for (int e = tid; e < 64 * dh; e += blockDim.x) {
      const int rr = e / dh, j = e % dh;
      const int row = row0 + rr;
      float kv = 0.f, vv = 0.f;
      if (row >= s + nrec && row < R) {
        const int64_t pos = sel[row - s - nrec];
        const T* ck = (const T*)c.coef_k + ((int64_t)u * c.Lmax + pos) * r;
        const T* cv = (const T*)c.coef_v + ((int64_t)u * c.Lmax + pos) * r;
        const T* bk = (const T*)c.basis_k + ((int64_t)u * D + h * dh + j) * r;
        const T* bv = (const T*)c.basis_v + ((int64_t)u * D + h * dh + j) * r;
        for (int i = 0; i < r; ++i) {
          kv += Elem<T>::ld(ck, i) * Elem<T>::ld(bk, i);
          vv += Elem<T>::ld(cv, i) * Elem<T>::ld(bv, i);
        }
      }
      Kh[rr * ldk + j] = kv;
      Vh[rr * ldk + j] = vv;
    }
  }
  __syncthreads();
  // exact rows
  for (int e = tid; e < 64 * dh; e += blockDim.x) {
    const int rr = e / dh, j = e % dh;
    const int row = row0 + rr;
    if (row < s) {
      Kh[rr * ldk + j] = Elem<T>::ld((const T*)c.sink_k, ((int64_t)u * s + row) * D + h * dh + j);
      Vh[rr * ldk + j] = Elem<T>::ld((const T*)c.sink_v, ((int64_t)u * s + row) * D + h * dh + j);
    } else if (row < s + nrec) {
      const int slot = row - s;
      Kh[rr * ldk + j] = Elem<T>::ld((const T*)c.ring_k, ((int64_t)u * nrec + slot) * D + h * dh + j);
      Vh[rr * ldk + j] = Elem<T>::ld((const T*)c.ring_v, ((int64_t)u * nrec + slot) * D + h * dh + j);
    }
  }
  __syncthreads();
  for (int e = tid; e < G * 64; e += blockDim.x) {
    const int g = e >> 6, rr = e & 63;
    float z = -INFINITY;
    if (row0 + rr < R) {
      float dot = 0.f;
      for (int j = 0; j < dh; ++j) dot += qs[g * dh + j] * Kh[rr * ldk + j];
      z = dot * sm_scale;
    }
    pl[e] = z;
  }
  __syncthreads();
  {
    const int wv = tid >> 6, l = tid & 63;
    for (int g = wv; g < G; g += 4) {
      const float z = pl[g * 64 + l];
      const float m = warp_max(z);
      const float e = (z == -INFINITY) ? 0.f : exp2f(z - m);
      const float ls = warp_sum(e);
      pl[g * 64 + l] = e;
      if (l == 0) {
        hs[2 * g] = m;
        hs[2 * g + 1] = ls;
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < G * (dh + 2); e += blockDim.x) {
    const int g = e / (dh + 2), j = e % (dh + 2);
    float v;
    if (j < 2) {
      v = hs[2 * g + j];
    } else {
      v = 0.f;
      for (int rr = 0; rr < 64; ++rr) v += pl[g * 64 + rr] * Vh[rr * ldk + (j - 2)];
    }
    part[((int64_t)(h * G + g) * w.nsa + split) * (dh + 2) + j] = v;
  }
}

// The attention tile can exceed the default 64 KB dynamic LDS limit; raise it
// once per kernel instantiation (gfx950 has 160 KB of LDS per CU).
template <typename T, int KS>
static hipError_t allow_lds(size_t lds) {
  static size_t done = 0;
  if (lds <= 65536 || lds <= done) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attend<T, KS>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e == hipSuccess) done = lds;
  return e;
}

hipError_t launch_attend(const Dims& d, int U, const void* q, const CachePtrs& c,
                         const DecodeWs& w, hipStream_t st) {
  dim3 grid(w.nsa, d.Hkv, U);
  const size_t lds = ((size_t)2 * 64 * (d.dh + 1) + d.G * d.dh + d.G * 64 + 2 * d.G) * sizeof(float);
  const float sm_scale = kLog2e / sqrtf((float)d.dh);
  hipError_t e = hipSuccess;
  if (d.dtype == 0) {
    if ((e = allow_lds<float, 0>(lds)) != hipSuccess) return e;
    hipLaunchKernelGGL((k_attend<float, 0>), grid, dim3(256), lds, st, d, c, w, (const float*)q, sm_scale);
    return hipGetLastError();
  }
  const uint16_t* qb = (const uint16_t*)q;
  switch (d.r) {
    case 128:
      if ((e = allow_lds<uint16_t, 8>(lds)) != hipSuccess) return e;
      hipLaunchKernelGGL((k_attend<uint16_t, 8>), grid, dim3(256), lds, st, d, c, w, qb, sm_scale); break;
    case 192:
      if ((e = allow_lds<uint16_t, 12>(lds)) != hipSuccess) return e;
      hipLaunchKernelGGL((k_attend<uint16_t, 12>), grid, dim3(256), lds, st, d, c, w, qb, sm_scale); break;
    case 256:
      if ((e = allow_lds<uint16_t, 16>(lds)) != hipSuccess) return e;
      hipLaunchKernelGGL((k_attend<uint16_t, 16>), grid, dim3(256), lds, st, d, c, w, qb, sm_scale); break;
    case 64:
      if ((e = allow_lds<uint16_t, 4>(lds)) != hipSuccess) return e;
      hipLaunchKernelGGL((k_attend<uint16_t, 4>), grid, dim3(256), lds, st, d, c, w, qb, sm_scale); break;
    case 32:
      if ((e = allow_lds<uint16_t, 2>(lds)) != hipSuccess) return e;
      hipLaunchKernelGGL((k_attend<uint16_t, 2>), grid, dim3(256), lds, st, d, c, w, qb, sm_scale); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// merge of the row splits (online-softmax combination) + advance lens
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_merge(Dims d, CachePtrs c, DecodeWs w,
                                               float* __restrict__ out) {
  const int a = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  const int dh = d.dh;
  const int32_t* si = w.stepinfo + 4 * u;
  float* o = out + ((int64_t)u * d.Hq + a) * dh;
  if (si[2]) {
    for (int j = tid; j < dh; j += blockDim.x) o[j] = 0.f;
    return;
  }
  const float* pp = w.part + ((int64_t)u * d.Hq + a) * w.nsa * (dh + 2);
  float M = -INFINITY;
  for (int sp = 0; sp < w.nsa; ++sp) M = fmaxf(M, pp[sp * (dh + 2)]);
  float Lsum = 0.f;
  for (int sp = 0; sp < w.nsa; ++sp) {
    const float m = pp[sp * (dh + 2)];
    if (m != -INFINITY) Lsum += pp[sp * (dh + 2) + 1] * exp2f(m - M);
  }
  for (int j = tid; j < dh; j += blockDim.x) {
    float acc = 0.f;
    for (int sp = 0; sp < w.nsa; ++sp) {
      const float m = pp[sp * (dh + 2)];
      if (m != -INFINITY) acc += pp[sp * (dh + 2) + 2 + j] * exp2f(m - M);
    }
    o[j] = acc / Lsum;
  }
  if (a == 0 && tid == 0) {
    c.lens[2 * u] = si[0] + 1;
    c.lens[2 * u + 1] = si[1] + 1;
  }
}

hipError_t launch_merge(const Dims& d, int U, const CachePtrs& c, const DecodeWs& w, float* out,
                        hipStream_t st) {
  hipLaunchKernelGGL(k_merge, dim3(d.Hq, U), dim3(256), 0, st, d, c, w, out);
  return hipGetLastError();
}

}  // namespace kvlr
