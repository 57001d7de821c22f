// Prefill kernels: sample + token-wise normalisation, Gram matrix S^T S,
// parallel cyclic Jacobi eigensolver, top-r basis extraction, projection of
// every non-sink token onto the bases, exact sink / recent-window copies.
//
// Method: S^4R review (pith.science/paper/2608.00528), 'What carries the
// argument' (bases = leading right singular vectors of the per-token
// normalised sample, Eqs. 1-2; every non-sink token kept as its coefficients
// on the basis, Eq. 3) and 'Core claim' (the first s tokens stay exact; the
// T'-token sample takes 7 parts from the end of the prompt to 3 parts spread
// evenly over the rest).
#include "common.h"

#include <math.h>

namespace kvlr {

// --------------------------------------------------------------------------
// 1. sample + normalise: S[m][i][:] = rnd(x_p / ||x_p||), m = 2u + (0 K | 1 V),
//    the quotient in fp64 and rounded once to the storage type
//    sample position p(i): the first n_u entries are evenly spaced over
//    [s, L - n_r), the last n_r are the most recent prompt positions.
// --------------------------------------------------------------------------
__device__ __forceinline__ int64_t sample_pos(int i, int nT, int64_t L, int s, int rnum, int rden) {
  const int64_t n_r = ((int64_t)rnum * nT) / rden;
  const int64_t n_u = nT - n_r;
  if (i < n_u) return s + ((int64_t)i * (L - n_r - s)) / n_u;
  return L - n_r + (i - n_u);
}

template <typename T>
__global__ __launch_bounds__(256) void k_sample_normalize(const T* __restrict__ K,
                                                          const T* __restrict__ V,
                                                          T* __restrict__ S, int64_t L, int D,
                                                          int nT, int s, int rnum, int rden) {
  const int i = blockIdx.x;
  const int m = blockIdx.y;
  const int u = m >> 1;
  const T* X = (m & 1) ? V : K;
  const int64_t p = sample_pos(i, nT, L, s, rnum, rden);
  const T* row = X + ((int64_t)u * L + p) * D;
  // the row in registers (D' <= 4096: at most 16 elements per thread), every
  // element requested before the first is used; the norm's sum in fp64, over
  // the lanes of a wave, then the four waves
  constexpr int NPT = 4096 / 256;
  float xv[NPT];
#pragma unroll
  for (int c = 0; c < NPT; ++c) {
    const int j = threadIdx.x + 256 * c;
    const float v = Elem<T>::ld(row, min(j, D - 1));  // in bounds; elements past D' are zeroed
    xv[c] = j < D ? v : 0.f;
  }
  double ss = 0.0;
#pragma unroll
  for (int c = 0; c < NPT; ++c) ss += (double)xv[c] * (double)xv[c];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  __shared__ double red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const double nrm = sqrt((red[0] + red[1]) + (red[2] + red[3]));
  T* out = S + ((int64_t)m * nT + i) * D;
  // x / ||x|| in fp64, rounded once to the storage type (a zero row stays 0)
#pragma unroll
  for (int c = 0; c < NPT; ++c) {
    const int j = threadIdx.x + 256 * c;
    if (j < D) {
      const double x = nrm > 0.0 ? (double)xv[c] / nrm : 0.0;
      if constexpr (sizeof(T) == 2)
        out[j] = d2bf(x);
      else
        out[j] = (float)x;
    }
  }
}

// bf16 rows with D' a multiple of 8: a wave per sampled row, moved in
// 16-byte pieces (the rows then start on 16-byte boundaries), the norm's sum
// in fp64 over the wave's lanes; the same quotient and rounding as above
__global__ __launch_bounds__(256) void k_sample_normalize_v8(const uint16_t* __restrict__ K,
                                                             const uint16_t* __restrict__ V,
                                                             uint16_t* __restrict__ S, int64_t L, int D,
                                                             int nT, int s, int rnum, int rden) {
  const int l = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int m = blockIdx.y, u = m >> 1;
  if (i >= nT) return;  // whole waves; no block barrier below
  const uint16_t* row = ((m & 1) ? V : K) + ((int64_t)u * L + sample_pos(i, nT, L, s, rnum, rden)) * D;
  constexpr int NC = 4096 / 512;  // pieces of 8 per lane (D' <= 4096)
  const int n8 = D / 8;
  u16x8 xv[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)  // every piece requested first (past the row: its last piece again)
    xv[c] = *reinterpret_cast<const u16x8*>(row + 8 * min(l + 64 * c, n8 - 1));
  double ss = 0.0;
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (l + 64 * c < n8)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double x = bf2f(xv[c][e]);
        ss += x * x;
      }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  const double nrm = sqrt(ss);
  uint16_t* out = S + ((int64_t)m * nT + i) * D;
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (l + 64 * c < n8) {
      u16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = d2bf(nrm > 0.0 ? (double)bf2f(xv[c][e]) / nrm : 0.0);
      *reinterpret_cast<u16x8*>(out + 8 * (l + 64 * c)) = o;
    }
}

hipError_t launch_sample_normalize(const Dims& d, int U, int64_t L, const void* K, const void* V,
                                   void* S, hipStream_t st) {
  if (d.dtype != 0 && d.D % 8 == 0) {
    hipLaunchKernelGGL(k_sample_normalize_v8, dim3((d.T + 3) / 4, 2 * U), dim3(256), 0, st,
                       (const uint16_t*)K, (const uint16_t*)V, (uint16_t*)S, L, d.D, d.T, d.s, d.rnum,
                       d.rden);
    return hipGetLastError();
  }
  dim3 grid(d.T, 2 * U);
  if (d.dtype == 0)
    hipLaunchKernelGGL(k_sample_normalize<float>, grid, dim3(256), 0, st, (const float*)K,
                       (const float*)V, (float*)S, L, d.D, d.T, d.s, d.rnum, d.rden);
  else
    hipLaunchKernelGGL(k_sample_normalize<uint16_t>, grid, dim3(256), 0, st,
                       (const uint16_t*)K, (const uint16_t*)V, (uint16_t*)S, L, d.D, d.T, d.s,
                       d.rnum, d.rden);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// 2. Gram A = S^T S (fp64 out) and V = I
// --------------------------------------------------------------------------
// bf16: MFMA 32x32x16, fp32 accumulation; one 64x64 output tile per block,
// upper-triangle tile pairs only, mirrored on store.
__global__ __launch_bounds__(256) void k_gram_bf16(const uint16_t* __restrict__ S,
                                                   double* __restrict__ A, int nT, int D,
                                                   int nt) {
  const int m = blockIdx.y;
  // tile pair index -> (ti, tj), ti <= tj
  int idx = blockIdx.x, ti = 0;
  while (idx >= nt - ti) {
    idx -= nt - ti;
    ++ti;
  }
  const int tj = ti + idx;
  __shared__ uint16_t Si[32][72];
  __shared__ uint16_t Sj[32][72];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int wi = w >> 1, wj = w & 1;
  const uint16_t* Sm = S + (int64_t)m * nT * D;
  f32x16 acc = {};
  const int lr = tid >> 3, cg = tid & 7;
  for (int t0 = 0; t0 < nT; t0 += 32) {
    {
      const int t = t0 + lr;
      const int ci = ti * 64 + 8 * cg, cj = tj * 64 + 8 * cg;
      u16x8 vi = {}, vj = {};
      if (t < nT && ci < D) vi = *reinterpret_cast<const u16x8*>(Sm + (int64_t)t * D + ci);
      if (t < nT && cj < D) vj = *reinterpret_cast<const u16x8*>(Sm + (int64_t)t * D + cj);
      *reinterpret_cast<u16x8*>(&Si[lr][8 * cg]) = vi;
      *reinterpret_cast<u16x8*>(&Sj[lr][8 * cg]) = vj;
    }
    __syncthreads();
    const int mm = l & 31, kg = l >> 5;
#pragma unroll
    for (int kk = 0; kk < 32; kk += 16) {
      u16x8 a, b;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a[e] = Si[kk + 8 * kg + e][32 * wi + mm];
        b[e] = Sj[kk + 8 * kg + e][32 * wj + mm];
      }
      acc = mfma32x32x16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc);
    }
    __syncthreads();
  }
  double* Am = A + (int64_t)m * D * D;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = ti * 64 + 32 * wi + acc_row32(i, l);
    const int col = tj * 64 + 32 * wj + (l & 31);
    if (row < D && col < D) {
      Am[(int64_t)row * D + col] = (double)acc[i];
      if (ti != tj) Am[(int64_t)col * D + row] = (double)acc[i];
    }
  }
}

// bf16, D' a multiple of 128: the Gram as a GEMM whose operands are both
// K-contiguous.  The sample is first copied channel-major (k_sample_t: S^T
// [D'][Tp], Tp = T' rounded up to 64, zero-padded; 64 x 64 tiles through
// LDS, coalesced reads and writes).  k_gram_nt: a block owns one 128 x 128
// tile pair (ti <= tj) of one matrix and one of `nsp` equal stretches of the
// tokens; 4 waves, wave w the 64 x 64 quadrant (w / 2, w % 2) as 2 x 2 MFMA
// 32x32x16 tiles (fp32 accumulation).  Per 64-token chunk the block stages
// the two 128-row operand slabs (16 KB each, rows padded to 144 bytes so the
// operand reads of 8 consecutive rows hit distinct banks) through a 2-stage
// LDS buffer, the next chunk's slabs loaded into registers during the
// current one's products.  Each block stores its fp32 partial tile;
// k_gram_reduce sums the stretches in fixed order in fp64 and writes A and
// its mirror, so the result does not depend on scheduling.
constexpr int kGT = 128;      // output tile edge
constexpr int kGK = 64;       // tokens per chunk
constexpr int kGLd = kGK + 8; // LDS row stride (bf16)

__global__ __launch_bounds__(256) void k_sample_t(const uint16_t* __restrict__ S,
                                                  uint16_t* __restrict__ ST, int nT, int Tp, int D) {
  __shared__ uint16_t t[64][65];
  const int m = blockIdx.z, t0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const uint16_t* Sm = S + (int64_t)m * nT * D;
  uint16_t* STm = ST + (int64_t)m * D * Tp;
  uint16_t v[64 * 64 / 256];  // every load of the thread in flight before the first store
#pragma unroll
  for (int k = 0; k < 64 * 64 / 256; ++k) {
    const int e = threadIdx.x + 256 * k, r = e >> 6, c = e & 63;  // token t0 + r, channel c0 + c
    const uint16_t x = Sm[(int64_t)min(t0 + r, nT - 1) * D + c0 + c];  // rows past nT: zero
    v[k] = t0 + r < nT ? x : (uint16_t)0;
  }
#pragma unroll
  for (int k = 0; k < 64 * 64 / 256; ++k) {
    const int e = threadIdx.x + 256 * k;
    t[e >> 6][e & 63] = v[k];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int c = e >> 6, r = e & 63;  // channel c0 + c, token t0 + r
    STm[(int64_t)(c0 + c) * Tp + t0 + r] = t[r][c];
  }
}

__global__ __launch_bounds__(256) void k_gram_nt(const uint16_t* __restrict__ ST,
                                                 float* __restrict__ part, int Tp, int D, int nt,
                                                 int nsp) {
  const int m = blockIdx.y;
  const int npair = nt * (nt + 1) / 2;
  const int pr = blockIdx.x / nsp, sp = blockIdx.x % nsp;
  int idx = pr, ti = 0;
  while (idx >= nt - ti) {
    idx -= nt - ti;
    ++ti;
  }
  const int tj = ti + idx;
  // this block's tokens: whole chunks [c0, c1)
  const int nch = Tp / kGK;
  const int c0 = (int)((int64_t)nch * sp / nsp), c1 = (int)((int64_t)nch * (sp + 1) / nsp);
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][kGT * kGLd];  // [stage][A | B]
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, mm = l & 31, kg = l >> 5;
  const uint16_t* STm = ST + (int64_t)m * D * Tp;
  const uint16_t* rowA = STm + (int64_t)(ti * kGT) * Tp;
  const uint16_t* rowB = STm + (int64_t)(tj * kGT) * Tp;
  // loads of a chunk: 2 slabs x 128 rows x 8 pieces of 16 bytes; thread tid
  // takes pieces tid + 256 q, q < 4, of each slab (row p / 8, piece p % 8)
  u16x8 ra[4], rb[4];
  auto load = [&](int ch) {
    const int64_t tk = (int64_t)ch * kGK;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int p = tid + 256 * q, r = p >> 3, pc = p & 7;
      ra[q] = *reinterpret_cast<const u16x8*>(rowA + (int64_t)r * Tp + tk + 8 * pc);
      rb[q] = *reinterpret_cast<const u16x8*>(rowB + (int64_t)r * Tp + tk + 8 * pc);
    }
  };
  auto store = [&](int stg) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int p = tid + 256 * q, r = p >> 3, pc = p & 7;
      *reinterpret_cast<u16x8*>(&lds[stg][0][r * kGLd + 8 * pc]) = ra[q];
      *reinterpret_cast<u16x8*>(&lds[stg][1][r * kGLd + 8 * pc]) = rb[q];
    }
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = f32x16{};
  const int wr = 64 * (w >> 1), wc = 64 * (w & 1);
  if (c0 < c1) {
    load(c0);
    store(0);
    __syncthreads();
    for (int ch = c0; ch < c1; ++ch) {
      const int stg = (ch - c0) & 1;
      if (ch + 1 < c1) load(ch + 1);
#pragma unroll
      for (int kk = 0; kk < kGK / 16; ++kk) {
        bf16x8 a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          a[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(
                                                &lds[stg][0][(wr + 32 * i + mm) * kGLd + 16 * kk + 8 * kg]));
          b[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(
                                                &lds[stg][1][(wc + 32 * i + mm) * kGLd + 16 * kk + 8 * kg]));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
      }
      if (ch + 1 < c1) store(stg ^ 1);
      __syncthreads();
    }
  }
  float* pt = part + (((int64_t)m * npair + pr) * nsp + sp) * kGT * kGT;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        pt[(wr + 32 * i + acc_row32(v, l)) * kGT + wc + 32 * j + mm] = acc[i][j][v];
}

// A[i][j] (and A[j][i]) = sum over the stretches of tile pair (ti <= tj), in order
__global__ __launch_bounds__(256) void k_gram_reduce(const float* __restrict__ part,
                                                     double* __restrict__ A, int D, int nt, int nsp) {
  const int m = blockIdx.y;
  const int npair = nt * (nt + 1) / 2;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)npair * kGT * kGT) return;
  const int pr = (int)(e / (kGT * kGT)), x = (int)(e % (kGT * kGT));
  int idx = pr, ti = 0;
  while (idx >= nt - ti) {
    idx -= nt - ti;
    ++ti;
  }
  const int tj = ti + idx;
  if (ti == tj && x / kGT > x % kGT) return;  // a diagonal tile: its upper triangle, mirrored
  const float* pt = part + ((int64_t)m * npair + pr) * nsp * kGT * kGT + x;
  double sum = 0.0;
  for (int s0 = 0; s0 < nsp; s0 += 8) {  // eight stretches requested together, summed in order
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = pt[(int64_t)min(s0 + q, nsp - 1) * kGT * kGT];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (s0 + q < nsp) sum += (double)v[q];
  }
  const int row = ti * kGT + x / kGT, col = tj * kGT + x % kGT;
  double* Am = A + (int64_t)m * D * D;
  Am[(int64_t)row * D + col] = sum;
  Am[(int64_t)col * D + row] = sum;
}

bool gram_nt_supported(const Dims& d) { return d.dtype != 0 && d.D % kGT == 0; }

// token stretches per tile pair: about 320 blocks in all, each with at least
// 4 chunks of 64 tokens
int gram_nt_splits(const Dims& d, int nmat) {
  const int nt = d.D / kGT, npair = nt * (nt + 1) / 2;
  const int nch = (d.T + kGK - 1) / kGK;
  int nsp = (320 + npair * nmat - 1) / (npair * nmat);
  nsp = nsp > nch / 4 ? nch / 4 : nsp;
  return nsp < 1 ? 1 : (nsp > 64 ? 64 : nsp);
}

size_t gram_nt_ws_bytes(const Dims& d, int nmat) {
  if (!gram_nt_supported(d)) return 0;
  const int64_t Tp = (d.T + kGK - 1) / kGK * kGK;
  const int nt = d.D / kGT, npair = nt * (nt + 1) / 2;
  const size_t st = (size_t)nmat * d.D * Tp * 2;
  const size_t pa = (size_t)nmat * npair * gram_nt_splits(d, nmat) * kGT * kGT * 4;
  return (st + 255) / 256 * 256 + pa;
}

// fp32: plain fp64 accumulation, one output entry per thread
__global__ __launch_bounds__(256) void k_gram_f32(const float* __restrict__ S,
                                                  double* __restrict__ A, int nT, int D) {
  const int m = blockIdx.y;
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)D * D) return;
  const int i = (int)(e / D), j = (int)(e % D);
  const float* Sm = S + (int64_t)m * nT * D;
  double acc = 0.0;
  for (int t = 0; t < nT; ++t) acc += (double)Sm[(int64_t)t * D + i] * (double)Sm[(int64_t)t * D + j];
  A[(int64_t)m * D * D + e] = acc;
}

__global__ void k_eye(double* __restrict__ Vm, int D) {
  const int m = blockIdx.y;
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)D * D) return;
  Vm[(int64_t)m * D * D + e] = (e / D == e % D) ? 1.0 : 0.0;
}

hipError_t launch_gram(const Dims& d, int nmat, const void* S, double* A, double* Vm, void* gws,
                       hipStream_t st) {
  const int D = d.D;
  const int64_t n2 = (int64_t)D * D;
  if (gram_nt_supported(d) && gws) {
    const int Tp = (d.T + kGK - 1) / kGK * kGK;
    const int nt = D / kGT, npair = nt * (nt + 1) / 2, nsp = gram_nt_splits(d, nmat);
    uint16_t* ST = (uint16_t*)gws;
    float* part = (float*)((char*)gws + ((size_t)nmat * D * Tp * 2 + 255) / 256 * 256);
    hipLaunchKernelGGL(k_sample_t, dim3(Tp / 64, D / 64, nmat), dim3(256), 0, st, (const uint16_t*)S, ST,
                       d.T, Tp, D);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_gram_nt, dim3(npair * nsp, nmat), dim3(256), 0, st, ST, part, Tp, D, nt, nsp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_gram_reduce, dim3((unsigned)((npair * kGT * kGT + 255) / 256), nmat), dim3(256), 0,
                       st, part, A, D, nt, nsp);
  } else if (d.dtype == 0) {
    hipLaunchKernelGGL(k_gram_f32, dim3((unsigned)((n2 + 255) / 256), nmat), dim3(256), 0, st,
                       (const float*)S, A, d.T, D);
  } else {
    const int nt = (D + 63) / 64;
    hipLaunchKernelGGL(k_gram_bf16, dim3(nt * (nt + 1) / 2, nmat), dim3(256), 0, st,
                       (const uint16_t*)S, A, d.T, D, nt);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_eye, dim3((unsigned)((n2 + 255) / 256), nmat), dim3(256), 0, st, Vm, D);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// 3. parallel cyclic Jacobi (two-sided rotations, fp64).
//
// Storage is kept in "pair order": in every round the disjoint rotation pairs
// are the slot pairs (2a, 2a+1).  After a round every slot's content moves to
// dest(slot), the round-robin (circle) move that keeps slot 0 fixed and
// rotates the other n-1 slots by one place, so n-1 consecutive rounds meet
// every index pair once (one sweep).  A thread owns one 2x2 block, reads it
// (and the two diagonal blocks that define its rotations) from the source
// buffer and writes the rotated block to the permuted places of the
// destination buffer; V accumulates the rotations with the same moves.
// Rotation: textbook symmetric Schur 2x2 (Golub & Van Loan), zeroing A[p][q].
// --------------------------------------------------------------------------
__device__ __forceinline__ int jac_dest(int slot, int n) {
  if (n <= 2 || slot == 0) return slot;
  if (slot == 1) return 2;
  const int k = slot >> 1;
  if ((slot & 1) == 0) return (k <= (n >> 1) - 2) ? slot + 2 : n - 1;
  return slot - 2;
}

__device__ __forceinline__ void jac_rot(const double* A, int n, int a, double* c, double* s,
                                        double* t) {
  const double app = A[(int64_t)(2 * a) * n + 2 * a];
  const double aqq = A[(int64_t)(2 * a + 1) * n + 2 * a + 1];
  const double apq = A[(int64_t)(2 * a) * n + 2 * a + 1];
  if (apq == 0.0) {
    *c = 1.0;
    *s = 0.0;
    *t = 0.0;
    return;
  }
  const double tau = (aqq - app) / (2.0 * apq);
  double tt;
  if (fabs(tau) > 1e150) {
    tt = 0.5 / tau;
  } else {
    tt = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
  }
  const double cc = 1.0 / sqrt(1.0 + tt * tt);
  *c = cc;
  *s = tt * cc;
  *t = tt;
}

__global__ __launch_bounds__(256) void k_jacobi_round(const double* __restrict__ Asrc,
                                                      double* __restrict__ Adst,
                                                      const double* __restrict__ Vsrc,
                                                      double* __restrict__ Vdst,
                                                      const int* __restrict__ frozen, int n) {
  const int m = blockIdx.y;
  if (frozen[m]) return;
  const int h = n >> 1;
  const int64_t nA = (int64_t)h * h, nV = (int64_t)n * h;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= nA + nV) return;
  const int64_t off = (int64_t)m * n * n;
  const double* A = Asrc + off;
  if (t < nA) {
    const int a = (int)(t / h), b = (int)(t % h);
    double ca, sa, ta, cb, sb, tb;
    jac_rot(A, n, a, &ca, &sa, &ta);
    double* Ad = Adst + off;
    const int pa = jac_dest(2 * a, n), qa = jac_dest(2 * a + 1, n);
    if (a == b) {
      const double app = A[(int64_t)(2 * a) * n + 2 * a];
      const double aqq = A[(int64_t)(2 * a + 1) * n + 2 * a + 1];
      const double apq = A[(int64_t)(2 * a) * n + 2 * a + 1];
      Ad[(int64_t)pa * n + pa] = app - ta * apq;
      Ad[(int64_t)qa * n + qa] = aqq + ta * apq;
      Ad[(int64_t)pa * n + qa] = 0.0;
      Ad[(int64_t)qa * n + pa] = 0.0;
      return;
    }
    jac_rot(A, n, b, &cb, &sb, &tb);
    const double m00 = A[(int64_t)(2 * a) * n + 2 * b], m01 = A[(int64_t)(2 * a) * n + 2 * b + 1];
    const double m10 = A[(int64_t)(2 * a + 1) * n + 2 * b],
                 m11 = A[(int64_t)(2 * a + 1) * n + 2 * b + 1];
    // rows: J_a^T M
    const double r00 = ca * m00 - sa * m10, r01 = ca * m01 - sa * m11;
    const double r10 = sa * m00 + ca * m10, r11 = sa * m01 + ca * m11;
    // columns: (J_a^T M) J_b
    const double n00 = cb * r00 - sb * r01, n01 = sb * r00 + cb * r01;
    const double n10 = cb * r10 - sb * r11, n11 = sb * r10 + cb * r11;
    const int pb = jac_dest(2 * b, n), qb = jac_dest(2 * b + 1, n);
    Ad[(int64_t)pa * n + pb] = n00;
    Ad[(int64_t)pa * n + qb] = n01;
    Ad[(int64_t)qa * n + pb] = n10;
    Ad[(int64_t)qa * n + qb] = n11;
  } else {
    const int64_t tv = t - nA;
    const int i = (int)(tv / h), b = (int)(tv % h);
    double cb, sb, tb;
    jac_rot(A, n, b, &cb, &sb, &tb);
    const double* Vr = Vsrc + off + (int64_t)i * n;
    const double v0 = Vr[2 * b], v1 = Vr[2 * b + 1];
    double* Vd = Vdst + off + (int64_t)i * n;
    Vd[jac_dest(2 * b, n)] = cb * v0 - sb * v1;
    Vd[jac_dest(2 * b + 1, n)] = sb * v0 + cb * v1;
  }
}

hipError_t launch_jacobi_round(int n, int nmat, const double* A_src, double* A_dst,
                               const double* V_src, double* V_dst, const int* frozen,
                               hipStream_t st) {
  const int64_t h = n / 2;
  const int64_t tot = h * h + (int64_t)n * h;
  hipLaunchKernelGGL(k_jacobi_round, dim3((unsigned)((tot + 255) / 256), nmat), dim3(256), 0, st,
                     A_src, A_dst, V_src, V_dst, frozen, n);
  return hipGetLastError();
}

// convergence test: off(A)_F <= tol * trace(A); partial sums per row chunk,
// then one thread per matrix sums them in a fixed order
constexpr int kJacRowsPerBlock = 4;

template <typename T>
__global__ __launch_bounds__(256) void k_offnorm(const T* __restrict__ A,
                                                 const int* __restrict__ frozen,
                                                 double* __restrict__ part, int n, int nchunk) {
  const int m = blockIdx.y;
  if (frozen[m]) return;
  const T* Am = A + (int64_t)m * n * n;
  const int r0 = blockIdx.x * kJacRowsPerBlock;
  double off = 0.0, tr = 0.0;
  // the block's rows and the thread's columns c = tid + 256 j: for D' <= 1024
  // every load of the thread is issued before the first sum
#pragma unroll
  for (int dr = 0; dr < kJacRowsPerBlock; ++dr) {
    const int r = r0 + dr;
    if (r >= n) break;
#pragma unroll 4
    for (int c = threadIdx.x; c < n; c += blockDim.x) {
      const double x = (double)Am[(int64_t)r * n + c];
      if (c == r)
        tr += x;
      else
        off += x * x;
    }
  }
  __shared__ double so[256], st[256];
  so[threadIdx.x] = off;
  st[threadIdx.x] = tr;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      so[threadIdx.x] += so[threadIdx.x + o];
      st[threadIdx.x] += st[threadIdx.x + o];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    part[((int64_t)m * nchunk + blockIdx.x) * 2 + 0] = so[0];
    part[((int64_t)m * nchunk + blockIdx.x) * 2 + 1] = st[0];
  }
}

__global__ void k_jacobi_check(const double* __restrict__ part, int* __restrict__ frozen,
                               int* __restrict__ final_buf, int* __restrict__ done_sweeps, int nmat,
                               int nchunk, int cur, int sweep, double tol) {
  // a wave per matrix: lanes sum strided partials, then the wave's sum
  const int lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  for (int m = threadIdx.x >> 6; m < nmat; m += nw) {
    if (frozen[m]) continue;
    double off = 0.0, tr = 0.0;
    for (int c = lane; c < nchunk; c += 64) {
      off += part[((int64_t)m * nchunk + c) * 2 + 0];
      tr += part[((int64_t)m * nchunk + c) * 2 + 1];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      off += __shfl_xor(off, o);
      tr += __shfl_xor(tr, o);
    }
    if (lane == 0 && (sqrt(off) <= tol * fabs(tr) || off == 0.0)) {
      frozen[m] = 1;
      final_buf[m] = cur;
      done_sweeps[m] = sweep + 1;
    }
  }
}

// matrices whose eigensolve reached the tolerance are frozen: every later
// round and check kernel returns at once for them, so a fixed number of
// sweeps can be enqueued without reading anything back
__global__ void k_jacobi_init(int* __restrict__ frozen, int* __restrict__ final_buf,
                              int* __restrict__ done_sweeps, int nmat) {
  for (int m = threadIdx.x; m < nmat; m += blockDim.x) {
    frozen[m] = 0;
    final_buf[m] = 0;
    done_sweeps[m] = 0;
  }
}

hipError_t launch_jacobi_init(int nmat, int* frozen, int* final_buf, int* done_sweeps,
                              hipStream_t st) {
  hipLaunchKernelGGL(k_jacobi_init, dim3(1), dim3(256), 0, st, frozen, final_buf, done_sweeps, nmat);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_jacobi_check(int n, int nmat, const T* A, double* part, int* frozen,
                               int* final_buf, int* done_sweeps, int cur, int sweep, double tol,
                               hipStream_t st) {
  const int nchunk = (n + kJacRowsPerBlock - 1) / kJacRowsPerBlock;
  hipLaunchKernelGGL(k_offnorm<T>, dim3(nchunk, nmat), dim3(256), 0, st, A, frozen, part, n, nchunk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_jacobi_check, dim3(1), dim3(256), 0, st, part, frozen, final_buf, done_sweeps,
                     nmat, nchunk, cur, sweep, tol);
  return hipGetLastError();
}
template hipError_t launch_jacobi_check<double>(int, int, const double*, double*, int*, int*, int*,
                                                int, int, double, hipStream_t);
template hipError_t launch_jacobi_check<float>(int, int, const float*, double*, int*, int*, int*,
                                               int, int, double, hipStream_t);

// --------------------------------------------------------------------------
// 3b. block Jacobi (two-sided, fp64), for n a multiple of 64 and >= 128.
//
// The n indices form nb = n / 32 blocks of 32.  A sweep is one "self" round
// (k = -1: subproblem p = blocks (2p, 2p + 1), whose rotations pair indices
// inside the same block) and nb - 1 "cross" rounds k = 0 .. nb - 2 (blocks
// paired by the circle method, block 0 fixed and the others rotating by one
// place per round; the rotations pair an index of I with one of J), so every
// index pair is rotated once per sweep, as in scalar cyclic Jacobi.  For
// subproblem p = (I, J) the 64 x 64 submatrix S = A[I u J, I u J] is rotated
// in LDS (the 2x2 Schur rotation above; 31 self or 32 cross inner rounds of
// 32 disjoint pairs) and Q_p accumulates the rotations.  Then, with Q the
// block diagonal of the Q_p, A <- Q^T A Q and V <- V Q: tile (P, P') of A
// becomes Q_P^T A[P, P'] Q_P' and row tile R of V's pair columns P becomes
// V[R, P] Q_P.  Every tile reads only itself, so the update is in place.
// --------------------------------------------------------------------------
constexpr int kBJ = 32;       // indices per block
constexpr int kBJ2 = 2 * kBJ; // indices per pair (one subproblem)

__device__ __forceinline__ int bj_block(int slot, int k, int nb) {
  return slot == 0 ? 0 : 1 + (slot - 1 + k) % (nb - 1);
}
// blocks (I, J) of subproblem p in round k (k < 0: the self round)
__device__ __forceinline__ void bj_pair(int p, int k, int nb, int* I, int* J) {
  if (k < 0) {
    *I = 2 * p;
    *J = 2 * p + 1;
  } else {
    *I = bj_block(p, k, nb);
    *J = bj_block(nb - 1 - p, k, nb);
  }
}
// global index of local index li (< 64) of pair (I, J)
__device__ __forceinline__ int bj_index(int li, int I, int J) {
  return li < kBJ ? I * kBJ + li : J * kBJ + (li - kBJ);
}

// grid (nb / 2, nmat), kBJEigThreads threads: Q_p of every subproblem of
// round k.  Inner round kr rotates the local index pairs (pi[kr][a],
// qi[kr][a]), a < 32, tabulated in LDS once: self rounds pair indices inside
// each half by the circle method over 32, cross rounds pair a with
// 32 + (a + kr) % 32.  Thread t updates 2x2 block t of S and two entry pairs
// of Q.
constexpr int kBJEigThreads = 1024;
__device__ __forceinline__ double bj_sqrt(double x) { return sqrt(x); }
__device__ __forceinline__ float bj_sqrt(float x) { return sqrtf(x); }
__device__ __forceinline__ double bj_rsqrt(double x) { return rsqrt(x); }
__device__ __forceinline__ float bj_rsqrt(float x) { return rsqrtf(x); }
// subproblem p of matrix m (called by all kBJEigThreads threads of a block)
template <typename T>
__device__ __forceinline__ void bjac_eig_block(const T* __restrict__ Aall, T* __restrict__ Qall, int n,
                                               int k, int m, int p) {
  constexpr int NT = kBJEigThreads, NP = kBJ2 / 2;
  static_assert(NP * NP == NT && kBJ2 * NP == 2 * NT, "one 2x2 block and two Q pairs per thread");
  static_assert((kBJ & (kBJ - 1)) == 0, "cross-round pairs use a power-of-two block");
  const int nb = n / kBJ, tid = threadIdx.x;
  int I, J;
  bj_pair(p, k, nb, &I, &J);
  const T* A = Aall + (int64_t)m * n * n;
  __shared__ T S[kBJ2][kBJ2 + 1];
  __shared__ T Q[kBJ2][kBJ2 + 1];
  __shared__ T rc[NP], rs[NP], rt[NP];
  __shared__ uint8_t pi[kBJ][NP], qi[kBJ][NP];
  {  // S = A[I u J, I u J]: every load of the thread in flight before the first store
    constexpr int NIT = kBJ2 * kBJ2 / NT;
    static_assert(NIT * NT == kBJ2 * kBJ2, "S splits evenly over the threads");
    T sv[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int e = tid + NT * it, i = e / kBJ2, j = e % kBJ2;
      sv[it] = A[(int64_t)bj_index(i, I, J) * n + bj_index(j, I, J)];
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int e = tid + NT * it, i = e / kBJ2, j = e % kBJ2;
      S[i][j] = sv[it];
      Q[i][j] = i == j ? T(1) : T(0);
    }
  }
  const int nround = k < 0 ? kBJ - 1 : kBJ;
  for (int e = tid; e < kBJ * NP; e += NT) {
    const int kr = e / NP, a = e % NP;
    int x, y;
    if (k < 0) {  // circle method over the 32 indices of each half
      const int h = a / (NP / 2), c = a % (NP / 2);
      auto cs = [&](int z) { return z == 0 ? 0 : 1 + (z - 1 + kr) % (kBJ - 1); };
      x = kBJ * h + cs(c);
      y = kBJ * h + cs(kBJ - 1 - c);
    } else {
      x = a;
      y = kBJ + (a + kr) % kBJ;
    }
    pi[kr][a] = (uint8_t)x;
    qi[kr][a] = (uint8_t)y;
  }
  __syncthreads();
  const int a = tid / NP, b = tid % NP;          // this thread's 2x2 block of S
  const int qrow = tid / NP, qb = tid % NP;      // Q rows qrow and qrow + 32, pair qb
  // cross rounds keep Q in registers: pair qb of round kr is (qb, 32 + (qb +
  // kr) % 32), so this thread holds x = Q[row][qb] and y = Q[row][32 + (qb +
  // kr) % 32] for its two rows, and after each round takes y from the lane of
  // pair qb + 1 (mod 32) of the same half-wave; self rounds use Q in LDS
  const bool qreg = k >= 0;
  T x0 = qrow == qb ? T(1) : T(0), y0 = T(0), x1 = T(0), y1 = x0;
  const int ysrc = (tid & 32) | ((tid + 1) & 31);
  {
    for (int kr = 0; kr < nround; ++kr) {
      if (tid < NP) {
        const int ip = qreg ? tid : pi[kr][tid], iq = qreg ? kBJ + ((tid + kr) & (kBJ - 1)) : qi[kr][tid];
        const T app = S[ip][ip], aqq = S[iq][iq], apq = S[ip][iq];
        T c = T(1), sn = T(0), t = T(0);
        if (apq != T(0)) {
          // the rotation above with tau = d / (2 apq) multiplied through by
          // |2 apq|: t = sgn(tau) 2|apq| / (|d| + sqrt(d^2 + 4 apq^2)), one
          // square root and one division (the entries are Gram sums of unit
          // vectors, far from overflow)
          const T d = aqq - app, a2 = T(2) * fabs(apq);
          const bool neg = (d < T(0)) != (apq < T(0)) && d != T(0);
          t = a2 / (fabs(d) + bj_sqrt(d * d + a2 * a2));
          t = neg ? -t : t;
          c = bj_rsqrt(T(1) + t * t);
          sn = t * c;
        }
        rc[tid] = c;
        rs[tid] = sn;
        rt[tid] = t;
      }
      __syncthreads();
      // S <- J^T S J on block (a, b); Q <- Q J on its two entry pairs (the
      // blocks and pairs are disjoint, so no thread reads another's stores)
      int pa, qa, pb, qbb, pq, qq;  // cross rounds: the pairs by arithmetic, no table reads
      if (qreg) {
        pa = a;
        qa = kBJ + ((a + kr) & (kBJ - 1));
        pb = b;
        qbb = kBJ + ((b + kr) & (kBJ - 1));
        pq = pb;
        qq = qbb;
      } else {
        pa = pi[kr][a];
        qa = qi[kr][a];
        pb = pi[kr][b];
        qbb = qi[kr][b];
        pq = pi[kr][qb];
        qq = qi[kr][qb];
      }
      const T m00 = S[pa][pb], m01 = S[pa][qbb], m10 = S[qa][pb], m11 = S[qa][qbb];
      const T cq = rc[qb], sq = rs[qb];
      if (a == b) {
        const T ta = rt[a];
        S[pa][pa] = m00 - ta * m01;
        S[qa][qa] = m11 + ta * m01;
        S[pa][qa] = T(0);
        S[qa][pa] = T(0);
      } else {
        const T ca = rc[a], sa = rs[a], cb = rc[b], sb = rs[b];
        const T r00 = ca * m00 - sa * m10, r01 = ca * m01 - sa * m11;
        const T r10 = sa * m00 + ca * m10, r11 = sa * m01 + ca * m11;
        S[pa][pb] = cb * r00 - sb * r01;
        S[pa][qbb] = sb * r00 + cb * r01;
        S[qa][pb] = cb * r10 - sb * r11;
        S[qa][qbb] = sb * r10 + cb * r11;
      }
      if (qreg) {
        const T n0 = sq * x0 + cq * y0, n1 = sq * x1 + cq * y1;
        x0 = cq * x0 - sq * y0;
        x1 = cq * x1 - sq * y1;
        y0 = kr + 1 < nround ? __shfl(n0, ysrc) : n0;
        y1 = kr + 1 < nround ? __shfl(n1, ysrc) : n1;
      } else {
        const T v00 = Q[qrow][pq], v01 = Q[qrow][qq];
        const T v10 = Q[qrow + NP][pq], v11 = Q[qrow + NP][qq];
        Q[qrow][pq] = cq * v00 - sq * v01;
        Q[qrow][qq] = sq * v00 + cq * v01;
        Q[qrow + NP][pq] = cq * v10 - sq * v11;
        Q[qrow + NP][qq] = sq * v10 + cq * v11;
      }
      __syncthreads();
    }
  }
  T* Qo = Qall + ((int64_t)m * (nb / 2) + p) * kBJ2 * kBJ2;
  if (qreg) {
    const int yc = kBJ + ((qb + nround - 1) & (kBJ - 1));
    Qo[qrow * kBJ2 + qb] = x0;
    Qo[qrow * kBJ2 + yc] = y0;
    Qo[(qrow + NP) * kBJ2 + qb] = x1;
    Qo[(qrow + NP) * kBJ2 + yc] = y1;
  } else {
    for (int e = tid; e < kBJ2 * kBJ2; e += NT) Qo[e] = Q[e / kBJ2][e % kBJ2];
  }
}

template <typename T>
__global__ __launch_bounds__(kBJEigThreads) void k_bjac_eig(const T* __restrict__ Aall,
                                                            T* __restrict__ Qall,
                                                            const int* __restrict__ frozen, int n,
                                                            int k) {
  const int m = blockIdx.y;
  if (frozen[m]) return;
  bjac_eig_block<T>(Aall, Qall, n, k, m, blockIdx.x);
}


// grid ((nb/2)^2 + (n/64)(nb/2), nmat), 256 threads: the in-place update of
// A's tiles (P, P') and V's tiles (row tile R, pair P) of outer round k.
// The 64 x 64 x 64 products run on fp64 MFMA 16x16x4 (lane l: A[l % 16][l / 16],
// B[l / 16][l % 16]; D element v at row l / 16 + 4 v, column l % 16); wave w
// computes the 32 x 32 quadrant (w / 2, w % 2), four 16 x 16 tiles; the
// tile operand is read from LDS (row stride 65 doubles: the transposed
// stores of 16 lanes land in distinct banks), the Q operands from memory.
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int kBJLd = kBJ2 + 1;

// the 16x16x4 MFMA of the scalar type: fp64 (D element v of lane l at row
// l / 16 + 4 v) or fp32 (row 4 (l / 16) + v); operands as above for both
template <typename T> struct BjMfma;
template <> struct BjMfma<double> {
  typedef f64x4 acc;
  typedef double2 pair;
  static __device__ __forceinline__ acc mma(double a, double b, acc c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ int row(int r4, int v) { return r4 + 4 * v; }
};
template <> struct BjMfma<float> {
  typedef f32x4 acc;
  typedef float2 pair;
  static __device__ __forceinline__ acc mma(float a, float b, acc c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ int row(int r4, int v) { return 4 * r4 + v; }
};

// tile `tile` of matrix m, by the 256 threads tid = 0..255 of a group that
// owns the LDS tile X (the group's block barriers: A tiles 3, V tiles 1;
// `active` false runs the barriers only)
// A's update covers the upper triangle of subproblem pairs, P <= P2 (A is
// symmetric: the tile of (P2, P) is the transpose of that of (P, P2) and is
// written from it), so np (np + 1) / 2 A tiles; V's tiles follow them
__host__ __device__ __forceinline__ int bj_natile(int np) { return np * (np + 1) / 2; }
constexpr int kBJTileIt = kBJ2 * kBJ2 / 2 / 256;  // column pairs of a tile per thread of a group

template <typename T>
__device__ __forceinline__ void bjac_apply_tile(T* __restrict__ Aall, T* __restrict__ Vall,
                                                const T* __restrict__ Qall, int n, int k, int m,
                                                int tile, int tid, bool active, T (*X)[kBJLd]) {
  typedef BjMfma<T> Mf;
  const int nb = n / kBJ, np = nb / 2;
  const int l = tid & 63, w = tid >> 6, qi = w >> 1, qj = w & 1, c16 = l & 15, r4 = l >> 4;
  constexpr int NKS = kBJ2 / 4;  // MFMA k-steps
  const T* Qm = Qall + (int64_t)m * np * kBJ2 * kBJ2;
  typename Mf::acc acc[2][2];
  // the Q factors' MFMA operands come straight from memory (L2) into
  // registers: lane (r4, c16) of k-step ks needs Q[4 ks + r4][col + c16]
  auto qfrag = [&](const T* Qp, int col, T (&f0)[NKS], T (&f1)[NKS]) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      f0[ks] = active ? Qp[(4 * ks + r4) * kBJ2 + col + c16] : T(0);
      f1[ks] = active ? Qp[(4 * ks + r4) * kBJ2 + col + 16 + c16] : T(0);
    }
  };
  auto zero = [&]() {
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int tj = 0; tj < 2; ++tj) acc[ti][tj] = typename Mf::acc{T(0), T(0), T(0), T(0)};
  };
  // acc[ti][tj][v] = sum_k A'[k][32 qi + 16 ti + r4 + 4 v] B'[k][32 qj + 16 tj + c16]
  // with A' from registers (a0, a1) and B' = X, or A' = X and B' from registers
  auto gemm_ra = [&](const T (&a0)[NKS], const T (&a1)[NKS]) {
    zero();
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int kr = 4 * ks + r4;
      const T b0 = X[kr][32 * qj + c16], b1 = X[kr][32 * qj + 16 + c16];
      acc[0][0] = Mf::mma(a0[ks], b0, acc[0][0]);
      acc[0][1] = Mf::mma(a0[ks], b1, acc[0][1]);
      acc[1][0] = Mf::mma(a1[ks], b0, acc[1][0]);
      acc[1][1] = Mf::mma(a1[ks], b1, acc[1][1]);
    }
  };
  auto gemm_rb = [&](const T (&b0)[NKS], const T (&b1)[NKS]) {
    zero();
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int kr = 4 * ks + r4;
      const T a0 = X[kr][32 * qi + c16], a1 = X[kr][32 * qi + 16 + c16];
      acc[0][0] = Mf::mma(a0, b0[ks], acc[0][0]);
      acc[0][1] = Mf::mma(a0, b1[ks], acc[0][1]);
      acc[1][0] = Mf::mma(a1, b0[ks], acc[1][0]);
      acc[1][1] = Mf::mma(a1, b1[ks], acc[1][1]);
    }
  };
  // output element (ti, tj, v) of this lane: row orow(ti, v), column ocol(tj)
  auto orow = [&](int ti, int v) { return 32 * qi + 16 * ti + Mf::row(r4, v); };
  auto ocol = [&](int tj) { return 32 * qj + 16 * tj + c16; };
  if (tile < bj_natile(np)) {
    int P = 0, rem = tile;  // tile -> (P, P2), P <= P2
    while (rem >= np - P) {
      rem -= np - P;
      ++P;
    }
    const int P2 = P + rem;
    int I, J, I2, J2;
    bj_pair(P, k, nb, &I, &J);
    bj_pair(P2, k, nb, &I2, &J2);
    T* A = Aall + (int64_t)m * n * n;
    T qa0[NKS], qa1[NKS];
    qfrag(Qm + (int64_t)P * kBJ2 * kBJ2, 32 * qi, qa0, qa1);  // A' = Q_P (rows of Q_P^T)
    if (active) {  // pairs of columns, 8- or 16-byte loads, all in flight before the first store
      typename Mf::pair xs[kBJTileIt];
#pragma unroll
      for (int it = 0; it < kBJTileIt; ++it) {
        const int e = tid + 256 * it, i = e / (kBJ2 / 2), j = 2 * (e % (kBJ2 / 2));
        xs[it] = *reinterpret_cast<const typename Mf::pair*>(A + (int64_t)bj_index(i, I, J) * n + bj_index(j, I2, J2));
      }
#pragma unroll
      for (int it = 0; it < kBJTileIt; ++it) {
        const int e = tid + 256 * it, i = e / (kBJ2 / 2), j = 2 * (e % (kBJ2 / 2));
        X[i][j] = xs[it].x;
        X[i][j + 1] = xs[it].y;
      }
    }
    __syncthreads();
    gemm_ra(qa0, qa1);  // T = Q_P^T X
    T qb0[NKS], qb1[NKS];
    qfrag(Qm + (int64_t)P2 * kBJ2 * kBJ2, 32 * qj, qb0, qb1);  // B' = Q_P2
    __syncthreads();
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int tj = 0; tj < 2; ++tj)
#pragma unroll
        for (int v = 0; v < 4; ++v) X[ocol(tj)][orow(ti, v)] = acc[ti][tj][v];  // X <- T^T
    __syncthreads();
    gemm_rb(qb0, qb1);  // T Q_P2
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int tj = 0; tj < 2; ++tj)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (active) A[(int64_t)bj_index(orow(ti, v), I, J) * n + bj_index(ocol(tj), I2, J2)] = acc[ti][tj][v];
    if (P != P2) {  // the mirrored tile A[P2, P], through LDS for row-contiguous stores
      __syncthreads();
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int tj = 0; tj < 2; ++tj)
#pragma unroll
          for (int v = 0; v < 4; ++v) X[ocol(tj)][orow(ti, v)] = acc[ti][tj][v];
      __syncthreads();
      for (int e = tid; active && e < kBJ2 * kBJ2 / 2; e += 256) {
        const int i = e / (kBJ2 / 2), j = 2 * (e % (kBJ2 / 2));  // row i of P2, columns j, j + 1 of P
        typename Mf::pair x;
        x.x = X[i][j];
        x.y = X[i][j + 1];
        *reinterpret_cast<typename Mf::pair*>(A + (int64_t)bj_index(i, I2, J2) * n + bj_index(j, I, J)) = x;
      }
    }
  } else {
    const int t2 = tile - bj_natile(np), R = t2 / np, P = t2 % np;
    int I, J;
    bj_pair(P, k, nb, &I, &J);
    T* V = Vall + (int64_t)m * n * n;
    T qb0[NKS], qb1[NKS];
    qfrag(Qm + (int64_t)P * kBJ2 * kBJ2, 32 * qj, qb0, qb1);  // B' = Q_P
    if (active) {
      typename Mf::pair xs[kBJTileIt];
#pragma unroll
      for (int it = 0; it < kBJTileIt; ++it) {
        const int e = tid + 256 * it, i = e / (kBJ2 / 2), j = 2 * (e % (kBJ2 / 2));
        xs[it] = *reinterpret_cast<const typename Mf::pair*>(V + (int64_t)(kBJ2 * R + i) * n + bj_index(j, I, J));
      }
#pragma unroll
      for (int it = 0; it < kBJTileIt; ++it) {
        const int e = tid + 256 * it, i = e / (kBJ2 / 2), j = 2 * (e % (kBJ2 / 2));
        X[j][i] = xs[it].x;
        X[j + 1][i] = xs[it].y;
      }
    }
    __syncthreads();
    gemm_rb(qb0, qb1);  // V[R, P] Q_P
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int tj = 0; tj < 2; ++tj)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (active) V[(int64_t)(kBJ2 * R + orow(ti, v)) * n + bj_index(ocol(tj), I, J)] = acc[ti][tj][v];
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_bjac_apply(T* __restrict__ Aall,
                                                    T* __restrict__ Vall,
                                                    const T* __restrict__ Qall,
                                                    const int* __restrict__ frozen, int n, int k) {
  const int m = blockIdx.y;
  if (frozen[m]) return;
  __shared__ __attribute__((aligned(16))) T X[kBJ2][kBJLd];  // the tile (V: transposed)
  bjac_apply_tile<T>(Aall, Vall, Qall, n, k, m, blockIdx.x, threadIdx.x, true, X);
}

// fp32 eigensolve: round k's subproblems (blocks [0, nb/2), when do_eig) and,
// in the same launch, V's update of the previous round kv with its Q blocks
// Qv (blocks past nb/2, four V tiles each): the V update is not on the path
// to the next round, so it runs on the CUs the subproblems leave idle.  The
// V round belongs to sweep vs (-1: none) and runs for a matrix that was
// still being solved in that sweep (not frozen, or frozen by that sweep's
// check).
template <typename T>
__global__ __launch_bounds__(kBJEigThreads) void k_bjac_eigv(T* __restrict__ Aall, T* __restrict__ Qall,
                                                             T* __restrict__ Vall, const T* __restrict__ Qv,
                                                             const int* __restrict__ frozen,
                                                             const int* __restrict__ done_sweeps, int n,
                                                             int k, int do_eig, int kv, int vs) {
  const int m = blockIdx.y, np = n / kBJ2;
  if ((int)blockIdx.x < np) {
    if (!do_eig || frozen[m]) return;
    bjac_eig_block<T>(Aall, Qall, n, k, m, blockIdx.x);
    return;
  }
  if (vs < 0 || (frozen[m] && done_sweeps[m] != vs + 1)) return;
  constexpr int G = kBJEigThreads / 256;
  __shared__ __attribute__((aligned(16))) T X[G][kBJ2][kBJLd];
  const int grp = threadIdx.x >> 8;
  const int tile = bj_natile(np) + ((int)blockIdx.x - np) * G + grp;
  const bool active = tile < bj_natile(np) + (n / kBJ2) * np;
  bjac_apply_tile<T>(Aall, Vall, Qv, n, kv, m, tile, threadIdx.x & 255, active, X[grp]);
}

bool bjac_supported(int n) { return n >= 2 * kBJ2 && n % kBJ2 == 0; }

size_t bjac_q_bytes(int n, int nmat) { return (size_t)nmat * (n / kBJ2) * kBJ2 * kBJ2 * sizeof(double); }

template <typename T>
hipError_t launch_bjac_round(int n, int nmat, T* A, T* V, T* Qbuf, const int* frozen, int k,
                             hipStream_t st) {
  const int nb = n / kBJ, np = nb / 2;
  hipLaunchKernelGGL(k_bjac_eig<T>, dim3(np, nmat), dim3(kBJEigThreads), 0, st, A, Qbuf, frozen, n, k);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_bjac_apply<T>, dim3(bj_natile(np) + (n / kBJ2) * np, nmat), dim3(256), 0, st, A, V, Qbuf,
                     frozen, n, k);
  return hipGetLastError();
}
// fp32 path: round k's subproblems with V's update of round kv (sweep vs,
// Q blocks Qv) in one launch, then A's update of round k alone
hipError_t launch_bjac_round_f32(int n, int nmat, float* A, float* V, float* Q, const float* Qv,
                                 const int* frozen, const int* done_sweeps, int k, int do_eig, int kv,
                                 int vs, hipStream_t st) {
  const int np = n / kBJ2;
  const int nvt = (n / kBJ2) * np;                       // V tiles
  const int G = kBJEigThreads / 256;
  hipLaunchKernelGGL(k_bjac_eigv<float>, dim3(np + (nvt + G - 1) / G, nmat), dim3(kBJEigThreads), 0, st,
                     A, Q, V, Qv, frozen, done_sweeps, n, k, do_eig, kv, vs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !do_eig) return e;
  hipLaunchKernelGGL(k_bjac_apply<float>, dim3(bj_natile(np), nmat), dim3(256), 0, st, A, V, Q, frozen, n, k);
  return hipGetLastError();
}

template hipError_t launch_bjac_round<double>(int, int, double*, double*, double*, const int*, int,
                                              hipStream_t);
template hipError_t launch_bjac_round<float>(int, int, float*, float*, float*, const int*, int,
                                             hipStream_t);

// the Gram matrices rounded to fp32 (A32) and V32 = I: the start of the fp32
// eigensolve
__global__ void k_to_f32(const double* __restrict__ A64, float* __restrict__ A32,
                         float* __restrict__ V32, int D) {
  const int m = blockIdx.y;
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)D * D) return;
  A32[(int64_t)m * D * D + e] = (float)A64[(int64_t)m * D * D + e];
  V32[(int64_t)m * D * D + e] = (e / D == e % D) ? 1.f : 0.f;
}

hipError_t launch_to_f32(int n, int nmat, const double* A64, float* A32, float* V32, hipStream_t st) {
  const int64_t n2 = (int64_t)n * n;
  hipLaunchKernelGGL(k_to_f32, dim3((unsigned)((n2 + 255) / 256), nmat), dim3(256), 0, st, A64, A32, V32, n);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// 4. eigenvalues descending (bitonic sort of (lambda, slot) in LDS, one block
//    per output matrix; the sorted slots go to the workspace), basis = the
//    first r eigenvector columns, rounded to storage (k_extract_gather, rows
//    of V spread over many blocks).
// --------------------------------------------------------------------------
// the matrix whose eigensolve serves output m (= 2 unit + kind): its own, or,
// with bases shared over a window of `depth` layers (units layer-major,
// `batch` sequences per layer), the window's first layer's
__device__ __forceinline__ int extract_source(int m, int batch, int depth) {
  const int u = m >> 1, kind = m & 1;
  const int layer = u / batch, seq = u % batch;
  return 2 * ((layer - layer % depth) * batch + seq) + kind;
}

template <typename T, typename S>
__global__ __launch_bounds__(256) void k_extract_gather(const S* __restrict__ V0,
                                                        const S* __restrict__ V1,
                                                        const int* __restrict__ frozen,
                                                        const int* __restrict__ final_buf, int cur,
                                                        const int* __restrict__ eidx, int n, int rk,
                                                        int rv, T* __restrict__ BK, T* __restrict__ BV,
                                                        int batch, int depth) {
  const int m = blockIdx.y, u = m >> 1, kind = m & 1;
  const int r = kind ? rv : rk;
  const int ms = extract_source(m, batch, depth);
  const int buf = frozen[ms] ? final_buf[ms] : cur;
  const S* Vm = (buf ? V1 : V0) + (int64_t)ms * n * n;
  const int* idx = eidx + (int64_t)m * n;
  T* B = (kind ? BV : BK) + (int64_t)u * n * r;
  // rows [4 bx, 4 bx + 4) of the basis; thread t: columns t, t + 256, ...
  for (int c = threadIdx.x; c < r; c += 256) {
    const int col = idx[c];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = 4 * blockIdx.x + q;
      if (i < n) {
        const double x = (double)Vm[(int64_t)i * n + col];
        if constexpr (sizeof(T) == 2)
          B[(int64_t)i * r + c] = d2bf(x);
        else
          B[(int64_t)i * r + c] = (float)x;
      }
    }
  }
}

template <typename T, typename S>
__global__ __launch_bounds__(1024) void k_extract(const S* __restrict__ A0,
                                                  const S* __restrict__ A1,
                                                  const S* __restrict__ V0,
                                                  const S* __restrict__ V1,
                                                  const int* __restrict__ frozen,
                                                  const int* __restrict__ final_buf,
                                                  const int* __restrict__ done_sweeps, int cur,
                                                  int n, int rk, int rv, T* __restrict__ BK,
                                                  T* __restrict__ BV, float* __restrict__ eigK,
                                                  float* __restrict__ eigV,
                                                  int32_t* __restrict__ sweeps, int batch, int depth,
                                                  int* __restrict__ eidx) {
  extern __shared__ unsigned char smem_raw[];
  const int m = blockIdx.x, u = m >> 1, kind = m & 1;
  const int ms = extract_source(m, batch, depth);
  const int buf = frozen[ms] ? final_buf[ms] : cur;
  const S* A = (buf ? A1 : A0) + (int64_t)ms * n * n;
  if (sweeps && threadIdx.x == 0) sweeps[m] = done_sweeps[ms] > 0 ? done_sweeps[ms] : -1;
  int np2 = 1;
  while (np2 < n) np2 <<= 1;
  double* key = reinterpret_cast<double*>(smem_raw);
  int* idx = reinterpret_cast<int*>(key + np2);
  for (int i = threadIdx.x; i < np2; i += blockDim.x) {
    key[i] = i < n ? (double)A[(int64_t)i * n + i] : -INFINITY;
    idx[i] = i;
  }
  __syncthreads();
  // sort descending by key, ties by ascending slot
  for (int size = 2; size <= np2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < np2; i += blockDim.x) {
        const int j = i ^ stride;
        if (j > i) {
          const bool desc = (i & size) == 0;
          const double ki = key[i], kj = key[j];
          const int ii = idx[i], ij = idx[j];
          // "i before j" in descending order with ascending tie-break
          const bool i_first = (ki > kj) || (ki == kj && ii < ij);
          if (i_first != desc) {
            key[i] = kj;
            key[j] = ki;
            idx[i] = ij;
            idx[j] = ii;
          }
        }
      }
      __syncthreads();
    }
  }
  float* eig = kind ? eigV : eigK;
  if (eig)
    for (int i = threadIdx.x; i < n; i += blockDim.x) eig[(int64_t)u * n + i] = (float)key[i];
  for (int i = threadIdx.x; i < n; i += blockDim.x) eidx[(int64_t)m * n + i] = idx[i];
}

template <typename S>
hipError_t launch_extract(const Dims& d, int nmat, const S* A0, const S* A1, const S* V0, const S* V1,
                          const int* frozen, const int* final_buf, const int* done_sweeps, int cur,
                          void* basis_k, void* basis_v, float* eig_k, float* eig_v, int32_t* sweeps,
                          int batch, int depth, int* eidx, hipStream_t st) {
  int np2 = 1;
  while (np2 < d.D) np2 <<= 1;
  const size_t lds = (size_t)np2 * (sizeof(double) + sizeof(int));
  const dim3 gg((unsigned)((d.D + 3) / 4), nmat);
  if (d.dtype == 0) {
    hipLaunchKernelGGL((k_extract<float, S>), dim3(nmat), dim3(1024), lds, st, A0, A1, V0, V1, frozen,
                       final_buf, done_sweeps, cur, d.D, d.r, d.rv, (float*)basis_k,
                       (float*)basis_v, eig_k, eig_v, sweeps, batch, depth, eidx);
    hipLaunchKernelGGL((k_extract_gather<float, S>), gg, dim3(256), 0, st, V0, V1, frozen, final_buf, cur, eidx,
                       d.D, d.r, d.rv, (float*)basis_k, (float*)basis_v, batch, depth);
  } else {
    hipLaunchKernelGGL((k_extract<uint16_t, S>), dim3(nmat), dim3(1024), lds, st, A0, A1, V0, V1,
                       frozen, final_buf, done_sweeps, cur, d.D, d.r, d.rv, (uint16_t*)basis_k,
                       (uint16_t*)basis_v, eig_k, eig_v, sweeps, batch, depth, eidx);
    hipLaunchKernelGGL((k_extract_gather<uint16_t, S>), gg, dim3(256), 0, st, V0, V1, frozen, final_buf, cur,
                       eidx, d.D, d.r, d.rv, (uint16_t*)basis_k, (uint16_t*)basis_v, batch, depth);
  }
  return hipGetLastError();
}
template hipError_t launch_extract<double>(const Dims&, int, const double*, const double*, const double*,
                                           const double*, const int*, const int*, const int*, int, void*,
                                           void*, float*, float*, int32_t*, int, int, int*, hipStream_t);
template hipError_t launch_extract<float>(const Dims&, int, const float*, const float*, const float*,
                                          const float*, const int*, const int*, const int*, int, void*,
                                          void*, float*, float*, int32_t*, int, int, int*, hipStream_t);

// --------------------------------------------------------------------------
// 5. projection C[j] = rnd(X[j] . B) for j in [s, L)
// --------------------------------------------------------------------------
// bf16: block = 64 rows x all r columns (r % 32 == 0, r <= 256), K-loop over
// D' in chunks of 32 staged through LDS; MFMA 32x32x16, fp32 accumulation.
__global__ __launch_bounds__(256) void k_project_bf16(const uint16_t* __restrict__ K,
                                                      const uint16_t* __restrict__ V,
                                                      const uint16_t* __restrict__ BK,
                                                      const uint16_t* __restrict__ BV,
                                                      uint16_t* __restrict__ CK,
                                                      uint16_t* __restrict__ CV, int64_t L,
                                                      int64_t Lmax, int D, int rk, int rv, int s) {
  const int u = blockIdx.y >> 1, kind = blockIdx.y & 1;
  const int r = kind ? rv : rk;
  const uint16_t* X = (kind ? V : K) + (int64_t)u * L * D;
  const uint16_t* B = (kind ? BV : BK) + (int64_t)u * D * r;
  uint16_t* C = (kind ? CV : CK) + (int64_t)u * Lmax * r;
  const int64_t row0 = s + (int64_t)blockIdx.x * 64;
  __shared__ uint16_t Xs[64][40];
  __shared__ uint16_t Bt[256][40];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int ntile = 2 * (r / 32);  // (row block, col block) pairs
  f32x16 acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = f32x16{};
  for (int k0 = 0; k0 < D; k0 += 32) {
    {  // X tile: 64 rows x 32 cols, one 16-byte group per thread
      const int rr = tid >> 2, cg = tid & 3;
      const int64_t row = row0 + rr;
      u16x8 v = {};
      if (row < L && k0 + 8 * cg < D) v = *reinterpret_cast<const u16x8*>(X + row * D + k0 + 8 * cg);
      *reinterpret_cast<u16x8*>(&Xs[rr][8 * cg]) = v;
    }
    // B tile: 32 rows (k) x r cols, stored transposed
    for (int g = tid; g < 32 * (r / 8); g += 256) {
      const int kr = g / (r / 8), cg = g % (r / 8);
      u16x8 v = {};
      if (k0 + kr < D) v = *reinterpret_cast<const u16x8*>(B + (int64_t)(k0 + kr) * r + 8 * cg);
#pragma unroll
      for (int e = 0; e < 8; ++e) Bt[8 * cg + e][kr] = v[e];
    }
    __syncthreads();
    const int mm = l & 31, kg = l >> 5;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int tile = w + 4 * q;
      if (tile < ntile) {
        const int rb = tile & 1, cb = tile >> 1;
#pragma unroll
        for (int kk = 0; kk < 32; kk += 16) {
          bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(&Xs[32 * rb + mm][kk + 8 * kg]));
          bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(&Bt[32 * cb + mm][kk + 8 * kg]));
          acc[q] = mfma32x32x16(a, b, acc[q]);
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int tile = w + 4 * q;
    if (tile < ntile) {
      const int rb = tile & 1, cb = tile >> 1;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t row = row0 + 32 * rb + acc_row32(i, l);
        const int col = 32 * cb + (l & 31);
        if (row < L) C[row * r + col] = f2bf(acc[q][i]);
      }
    }
  }
}

// bf16, r a multiple of 64: the bases are first transposed (B^T[n][k]) into
// the call's workspace so that every MFMA operand is one K-contiguous
// 16-byte read.  Block: 256 rows x all r columns of one (unit, K | V); 8
// waves (two per SIMD), wave w owns rows [32 w, 32 w + 32) and every column
// block (accumulators in AGPRs).  The K loop advances 64 channels per step:
//   - the wave's X fragments (lane (m, kg): row m, channels 8 kg + 16 kk)
//     stream from global memory straight into registers three steps ahead;
//   - the B^T tile of a step (r rows x 128 bytes) is loaded into registers
//     two steps ahead and stored to the free half of a 2-stage LDS buffer
//     one step ahead, before the step's barrier; within a row the 16-byte
//     chunk c sits in slot c ^ ((n >> 1) & 7), so the operand reads of 16
//     consecutive rows hit distinct banks.
constexpr int kProjRows = 256;   // rows per block
constexpr int kProjWaves = 8;    // waves per block
constexpr int kProjK = 64;       // channels per K step
constexpr int kProjRing = 4;     // X fragment ring depth (steps)

__device__ __forceinline__ void transpose_tile(const uint16_t* __restrict__ B, uint16_t* __restrict__ T,
                                               int D, int r, int k0, int n0);

// NS = D' / 64 steps when known at compile time (the loop then unrolls), 0 =
// runtime
template <int R, int NS>
__global__ __launch_bounds__(kProjWaves * 64) void k_project_mfma(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ BTK, int64_t sk, const uint16_t* __restrict__ BTV, int64_t sv,
    uint16_t* __restrict__ CK, uint16_t* __restrict__ CV,
    int64_t L, int64_t Lmax, int D, int s, int kind_only) {
  constexpr int NT = kProjWaves * 64;
  constexpr int NCB = R / 32;
  constexpr int SB = R * kProjK * 2;         // stage bytes
  constexpr int NPB = SB / 16 / NT;          // 16-byte B^T pieces per thread per step
  constexpr int AR = kProjRing;
  static_assert(SB % (16 * NT) == 0, "rank must be a multiple of 64");
  __shared__ __attribute__((aligned(16))) uint8_t stg[2 * SB];
  // kind_only < 0: grid.y = 2 U (K and V share the rank R); else grid.y = U
  const int u = kind_only < 0 ? blockIdx.y >> 1 : blockIdx.y;
  const int kind = kind_only < 0 ? blockIdx.y & 1 : kind_only;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, mm = l & 31, kg = l >> 5;
  const uint16_t* X = (kind ? V : K) + (int64_t)u * L * D;
  const uint16_t* Bt = kind ? BTV + (int64_t)u * sv : BTK + (int64_t)u * sk;
  uint16_t* C = (kind ? CV : CK) + (int64_t)u * Lmax * R;
  const int64_t row0 = s + (int64_t)blockIdx.x * kProjRows;
  const int nsteps = NS > 0 ? NS : D / kProjK;
  // this lane's X row (rows past L re-read the last one; their results are not stored)
  const uint16_t* xr = X + min(row0 + 32 * w + mm, L - 1) * D + 8 * kg;
  // B^T pieces of this thread: piece p = tid + NT i -> row n = p / 8, chunk p % 8
  uint32_t bsrc[NPB], bdst[NPB];
#pragma unroll
  for (int i = 0; i < NPB; ++i) {
    const int p = tid + NT * i, n = p >> 3, c = p & 7;
    bsrc[i] = (uint32_t)(n * D + 8 * c);
    bdst[i] = (uint32_t)(n * (kProjK * 2) + ((c ^ ((n >> 1) & 7)) << 4));
  }
  auto load_b = [&](int step, u16x8* br) {
    const uint16_t* src = Bt + (int64_t)min(step, nsteps - 1) * kProjK;
#pragma unroll
    for (int i = 0; i < NPB; ++i) br[i] = *reinterpret_cast<const u16x8*>(src + bsrc[i]);
  };
  auto store_b = [&](int step, const u16x8* br) {
    uint8_t* stage = stg + (step & 1) * SB;
#pragma unroll
    for (int i = 0; i < NPB; ++i) *reinterpret_cast<u16x8*>(stage + bdst[i]) = br[i];
  };
  auto load_a = [&](int step, bf16x8* a) {
    const uint16_t* p = xr + (int64_t)min(step, nsteps - 1) * kProjK;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) a[kk] = ld_bf16x8(p + 16 * kk);
  };
  f32x16 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x16{};
  // lane (n = mm, kg) reads chunk 2 kk + kg of B^T row 32 cb + n
  const int sw = (mm >> 1) & 7;  // (n >> 1) & 7, the same for every column block
  auto compute = [&](int step, const bf16x8* a) {
    const uint8_t* stage = stg + (step & 1) * SB + mm * (kProjK * 2);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int co = ((2 * kk + kg) ^ sw) << 4;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const bf16x8 bb = *reinterpret_cast<const bf16x8*>(stage + 32 * cb * (kProjK * 2) + co);
        acc[cb] = mfma32x32x16(a[kk], bb, acc[cb]);
      }
    }
  };
  // A ring of AR steps (AR - 1 ahead) and B^T 2 steps ahead in registers;
  // D' is a multiple of AR steps, so the loop has a single exit
  bf16x8 ar[AR][4];
  u16x8 bA[NPB], bB[NPB];
  load_b(0, bA);
  load_b(1, bB);
#pragma unroll
  for (int i = 0; i < AR - 1; ++i) load_a(i, ar[i]);
  store_b(0, bA);
  __syncthreads();
#pragma unroll
  for (int t = 0; t < nsteps; t += AR) {
#pragma unroll
    for (int k = 0; k < AR; ++k) {
      load_b(t + k + 2, (k & 1) ? bB : bA);
      load_a(t + k + AR - 1, ar[(k + AR - 1) % AR]);
      compute(t + k, ar[k]);
      store_b(t + k + 1, (k & 1) ? bA : bB);
      __syncthreads();
    }
  }
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t row = row0 + 32 * w + acc_row32(i, l);
      if (row < L) C[row * R + 32 * cb + mm] = f2bf(acc[cb][i]);
    }
  }
}

__global__ __launch_bounds__(256) void k_project_f32(const float* __restrict__ K,
                                                     const float* __restrict__ V,
                                                     const float* __restrict__ BK,
                                                     const float* __restrict__ BV,
                                                     float* __restrict__ CK, float* __restrict__ CV,
                                                     int64_t L, int64_t Lmax, int D, int rk, int rv,
                                                     int s) {
  const int u = blockIdx.y >> 1, kind = blockIdx.y & 1;
  const int r = kind ? rv : rk;
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nrow = L - s;
  if (e >= nrow * r) return;
  const int64_t row = s + e / r;
  const int c = (int)(e % r);
  const float* X = (kind ? V : K) + ((int64_t)u * L + row) * D;
  const float* B = (kind ? BV : BK) + (int64_t)u * D * r;
  double acc = 0.0;  // fp64 accumulation, rounded once to fp32
  for (int k = 0; k < D; ++k) acc += (double)X[k] * (double)B[(int64_t)k * r + c];
  (kind ? CV : CK)[((int64_t)u * Lmax + row) * r + c] = (float)acc;
}

// B^K and B^V transposed: BTK / BTV, unit strides sk / sv (elements)
struct BasisT {
  const uint16_t *k, *v;
  int64_t sk, sv;
};

template <int R>
static hipError_t launch_project_mfma(const Dims& d, int U, int64_t L, int64_t Lmax, const void* K,
                                      const void* V, void* CK, void* CV, const BasisT& bt,
                                      int kind_only, hipStream_t st) {
  const int64_t nrow = L - d.s;
  const dim3 grid((unsigned)((nrow + kProjRows - 1) / kProjRows), kind_only < 0 ? 2 * U : U);
#define KVLR_PROJ_LAUNCH(NS)                                                                     \
  hipLaunchKernelGGL((k_project_mfma<R, NS>), grid, dim3(kProjWaves * 64), 0, st,               \
                     (const uint16_t*)K, (const uint16_t*)V, bt.k, bt.sk, bt.v, bt.sv,         \
                     (uint16_t*)CK, (uint16_t*)CV, L, Lmax, d.D, d.s, kind_only)
  switch (d.D / kProjK) {
    case 8: KVLR_PROJ_LAUNCH(8); break;
    case 16: KVLR_PROJ_LAUNCH(16); break;
    default: KVLR_PROJ_LAUNCH(0); break;
  }
#undef KVLR_PROJ_LAUNCH
  return hipGetLastError();
}

static hipError_t launch_project_rank(int R, const Dims& d, int U, int64_t L, int64_t Lmax,
                                      const void* K, const void* V, void* CK, void* CV,
                                      const BasisT& bt, int kind_only, hipStream_t st) {
  switch (R) {
    case 64: return launch_project_mfma<64>(d, U, L, Lmax, K, V, CK, CV, bt, kind_only, st);
    case 128: return launch_project_mfma<128>(d, U, L, Lmax, K, V, CK, CV, bt, kind_only, st);
    case 192: return launch_project_mfma<192>(d, U, L, Lmax, K, V, CK, CV, bt, kind_only, st);
    case 256: return launch_project_mfma<256>(d, U, L, Lmax, K, V, CK, CV, bt, kind_only, st);
    default: return hipErrorInvalidValue;
  }
}

static bool project_mfma_ok(const Dims& d) {
  auto ok = [](int r) { return r == 64 || r == 128 || r == 192 || r == 256; };
  return d.dtype != 0 && ok(d.r) && ok(d.rv) && d.D % (kProjRing * kProjK) == 0;
}

size_t project_ws_bytes(const Dims& d, int64_t U) {
  if (!project_mfma_ok(d)) return 0;
  return (size_t)U * d.rv * d.D * sizeof(uint16_t);  // B^V transposed
}

// the projection kernels without MFMA (fp32 storage, other ranks)
static hipError_t launch_project_plain(const Dims& d, int U, int64_t L, int64_t Lmax, const void* K,
                                       const void* V, const void* BK, const void* BV, void* CK,
                                       void* CV, hipStream_t st) {
  const int64_t nrow = L - d.s;
  if (nrow <= 0) return hipSuccess;
  if (d.dtype == 0) {
    const int64_t tot = nrow * (d.r > d.rv ? d.r : d.rv);
    hipLaunchKernelGGL(k_project_f32, dim3((unsigned)((tot + 255) / 256), 2 * U), dim3(256), 0, st,
                       (const float*)K, (const float*)V, (const float*)BK, (const float*)BV,
                       (float*)CK, (float*)CV, L, Lmax, d.D, d.r, d.rv, d.s);
  } else {
    hipLaunchKernelGGL(k_project_bf16, dim3((unsigned)((nrow + 63) / 64), 2 * U), dim3(256), 0,
                       st, (const uint16_t*)K, (const uint16_t*)V, (const uint16_t*)BK,
                       (const uint16_t*)BV, (uint16_t*)CK, (uint16_t*)CV, L, Lmax, d.D, d.r, d.rv,
                       d.s);
  }
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// 6. exact sinks + recent ring, window / statistics reset, lens = {L, 0}
// --------------------------------------------------------------------------
// block `row` of unit u: [0, s + nrec) exact rows, then one block for the reset
template <typename T>
__device__ __forceinline__ void exact_reset_block(const T* __restrict__ K, const T* __restrict__ V,
                                                  const CachePtrs& c, int64_t L, int D, int s, int nrec,
                                                  int qw_per_unit, int u, int row) {
  T* sk = (T*)c.sink_k;
  T* sv = (T*)c.sink_v;
  T* rk = (T*)c.ring_k;
  T* rv = (T*)c.ring_v;
  if (row < s) {
    const T* src = K + ((int64_t)u * L + row) * D;
    const T* srcv = V + ((int64_t)u * L + row) * D;
    for (int j = threadIdx.x; j < D; j += blockDim.x) {
      sk[((int64_t)u * s + row) * D + j] = src[j];
      sv[((int64_t)u * s + row) * D + j] = srcv[j];
    }
  } else if (row < s + nrec) {
    const int64_t p = L - nrec + (row - s);
    const int slot = (int)(p % nrec);
    const T* src = K + ((int64_t)u * L + p) * D;
    const T* srcv = V + ((int64_t)u * L + p) * D;
    for (int j = threadIdx.x; j < D; j += blockDim.x) {
      rk[((int64_t)u * nrec + slot) * D + j] = src[j];
      rv[((int64_t)u * nrec + slot) * D + j] = srcv[j];
    }
  } else {
    for (int j = threadIdx.x; j < qw_per_unit; j += blockDim.x) c.qwin[(int64_t)u * qw_per_unit + j] = 0.f;
    uint32_t* st = reinterpret_cast<uint32_t*>(c.state + u * c.state_stride);
    for (int64_t j = threadIdx.x; j < c.bkt_off / 4; j += blockDim.x) st[j] = 0u;  // window state
    if (threadIdx.x == 0) {
      c.lens[2 * u] = (int32_t)L;
      c.lens[2 * u + 1] = 0;
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_exact_reset(const T* __restrict__ K,
                                                     const T* __restrict__ V, CachePtrs c,
                                                     int64_t L, int D, int s, int nrec,
                                                     int qw_per_unit) {
  exact_reset_block<T>(K, V, c, L, D, s, nrec, qw_per_unit, blockIdx.y, blockIdx.x);
}

// One 32 x 32 tile of B [D][r] transposed into T [r][D] (T[n][k] = B[k][n]).
__device__ __forceinline__ void transpose_tile(const uint16_t* __restrict__ B, uint16_t* __restrict__ T,
                                               int D, int r, int k0, int n0) {
  __shared__ uint16_t t[32][33];
  for (int e = threadIdx.x; e < 1024; e += 256) {
    const int kk = e >> 5, nn = e & 31;
    if (k0 + kk < D && n0 + nn < r) t[kk][nn] = B[(int64_t)(k0 + kk) * r + n0 + nn];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 1024; e += 256) {
    const int nn = e >> 5, kk = e & 31;
    if (k0 + kk < D && n0 + nn < r) T[(int64_t)(n0 + nn) * D + k0 + kk] = t[kk][nn];
  }
}

// Everything the bf16 MFMA projection call does besides the products, in one
// launch (grid.y = unit): blocks [0, s + nrec] the exact rows and the window
// reset, then the tiles of B^K transposed into the unit state (the decode
// prologue's operand, which the projection reads too), then the tiles of B^V
// transposed into the call's workspace.
__global__ __launch_bounds__(256) void k_project_prep(const uint16_t* __restrict__ K,
                                                      const uint16_t* __restrict__ V, CachePtrs c,
                                                      uint16_t* __restrict__ BTV, int64_t L, int D,
                                                      int s, int nrec, int qw_per_unit, int rk, int rv) {
  const int u = blockIdx.y, nE = s + nrec + 1, nkx = (D + 31) / 32;
  const int x = blockIdx.x;
  if (x < nE) {
    exact_reset_block<uint16_t>(K, V, c, L, D, s, nrec, qw_per_unit, u, x);
    return;
  }
  const int tk = x - nE, ntk = nkx * ((rk + 31) / 32);
  if (tk < ntk) {
    transpose_tile((const uint16_t*)c.basis_k + (int64_t)u * D * rk, bkt_of(c, u), D, rk, (tk % nkx) * 32,
                   (tk / nkx) * 32);
  } else {
    const int tv = tk - ntk;
    transpose_tile((const uint16_t*)c.basis_v + (int64_t)u * D * rv, BTV + (int64_t)u * rv * D, D, rv,
                   (tv % nkx) * 32, (tv / nkx) * 32);
  }
}

// B^K transposed into the unit state (bf16): tile of 32 channels x 32 columns
__global__ __launch_bounds__(256) void k_basis_kt_state(CachePtrs c, int D, int r) {
  const int u = blockIdx.z;
  transpose_tile((const uint16_t*)c.basis_k + (int64_t)u * D * r, bkt_of(c, u), D, r, blockIdx.x * 32,
                 blockIdx.y * 32);
}

hipError_t launch_exact_and_reset(const Dims& d, int U, int64_t L, const void* K, const void* V,
                                  const CachePtrs& c, hipStream_t st) {
  dim3 grid(d.s + d.nrec + 1, U);
  const int qw = d.W * d.G * d.r;
  if (d.dtype == 0) {
    hipLaunchKernelGGL(k_exact_reset<float>, grid, dim3(256), 0, st, (const float*)K,
                       (const float*)V, c, L, d.D, d.s, d.nrec, qw);
  } else {
    hipLaunchKernelGGL(k_exact_reset<uint16_t>, grid, dim3(256), 0, st, (const uint16_t*)K,
                       (const uint16_t*)V, c, L, d.D, d.s, d.nrec, qw);
    hipLaunchKernelGGL(k_basis_kt_state, dim3((d.D + 31) / 32, (d.r + 31) / 32, U), dim3(256), 0,
                       st, c, d.D, d.r);
  }
  return hipGetLastError();
}

hipError_t launch_project_call(const Dims& d, int U, int64_t L, const void* K, const void* V,
                               const CachePtrs& c, void* ws, hipStream_t st) {
  if (!project_mfma_ok(d)) {
    hipError_t e = launch_project_plain(d, U, L, c.Lmax, K, V, c.basis_k, c.basis_v, c.coef_k, c.coef_v, st);
    if (e != hipSuccess) return e;
    return launch_exact_and_reset(d, U, L, K, V, c, st);
  }
  uint16_t* BTV = (uint16_t*)ws;
  const int nkx = (d.D + 31) / 32;
  const int nb = d.s + d.nrec + 1 + nkx * ((d.r + 31) / 32) + nkx * ((d.rv + 31) / 32);
  hipLaunchKernelGGL(k_project_prep, dim3(nb, U), dim3(256), 0, st, (const uint16_t*)K,
                     (const uint16_t*)V, c, BTV, L, d.D, d.s, d.nrec, d.W * d.G * d.r, d.r, d.rv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || L <= d.s) return e;
  const BasisT bt = {bkt_of(c, 0), BTV, c.state_stride / (int64_t)sizeof(uint16_t), (int64_t)d.rv * d.D};
  if (d.r == d.rv) return launch_project_rank(d.r, d, U, L, c.Lmax, K, V, c.coef_k, c.coef_v, bt, -1, st);
  e = launch_project_rank(d.r, d, U, L, c.Lmax, K, V, c.coef_k, c.coef_v, bt, 0, st);
  if (e != hipSuccess) return e;
  return launch_project_rank(d.rv, d, U, L, c.Lmax, K, V, c.coef_k, c.coef_v, bt, 1, st);
}

// --------------------------------------------------------------------------
// 7. window seeded with the prompt's last queries (the variant that starts
//    decoding with a full query-coefficient window): every tail query's
//    coefficients are pushed like a decode step's, and the pushed rows'
//    running softmax statistics are computed over the current candidates
//    [s, L - n_rec), so the first decode step scores with them as with rows
//    of earlier steps.
// --------------------------------------------------------------------------
// grid (n_tail, U), 256 threads: c_q[g] = q_cat[g] . B^K for tail query j
template <typename T>
__global__ __launch_bounds__(256) void k_window_push(Dims d, CachePtrs c, const T* __restrict__ qt,
                                                     int n_tail, float qscale) {
  const int j = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  const int D = d.D, r = d.r, G = d.G, W = d.W, dh = d.dh;
  extern __shared__ float xs[];  // [G][D'] concatenated queries
  const T* qj = qt + ((int64_t)u * n_tail + j) * d.Hq * dh;
  for (int e = tid; e < d.Hq * dh; e += 256) {
    const int a = e / dh, i = e % dh, h = a / G, g = a % G;
    xs[g * D + h * dh + i] = Elem<T>::ld(qj, e);
  }
  __syncthreads();
  const int slot = (c.lens[2 * u + 1] + j) % W;
  const T* B = (const T*)c.basis_k + (int64_t)u * D * r;
  uint16_t* qs = qsplit_of(c, u);
  for (int col = tid; col < r; col += 256) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < D; ++k) {
      const float b = Elem<T>::ld(B, (int64_t)k * r + col);
#pragma unroll
      for (int g = 0; g < 8; ++g)
        if (g < G) acc[g] += xs[g * D + k] * b;
    }
    for (int g = 0; g < G; ++g) {
      const int row = slot * G + g;
      c.qwin[((int64_t)u * W * G + row) * r + col] = acc[g];
      const float x = acc[g] * qscale;  // the scorer's operands: bf16 hi + lo
      const uint16_t hb = f2bf(x);
      qs[(row * 2 + 0) * r + col] = hb;
      qs[(row * 2 + 1) * r + col] = f2bf(x - bf2f(hb));
    }
  }
}

constexpr int kWinRows = 8;      // window rows per block of the statistics pass
constexpr int kWinTile = 256;    // candidates per block

// grid (ntile, ceil(nrows / 8), U), 256 threads: partial (max, sum) of the
// base-2 logits of 8 pushed rows over one tile of candidates; thread (row
// tid / 32, lane tid % 32) takes candidates lane, lane + 32, ...
template <typename T>
__global__ __launch_bounds__(256) void k_window_stats(Dims d, CachePtrs c, int n_tail, float qscale,
                                                      float2* __restrict__ part, int ntile) {
  const int tile = blockIdx.x, rg = blockIdx.y, u = blockIdx.z, tid = threadIdx.x;
  const int r = d.r, G = d.G, W = d.W;
  const int nrows = n_tail * G;
  const int row = rg * kWinRows + tid / 32, lane = tid % 32;
  extern __shared__ float qrow[];  // [8][r] window rows, scaled to base 2
  const int pushed0 = c.lens[2 * u + 1];
  for (int e = tid; e < kWinRows * r; e += 256) {
    const int rr = rg * kWinRows + e / r;
    float v = 0.f;
    if (rr < nrows) {
      const int slot = (pushed0 + rr / G) % W;
      v = c.qwin[(((int64_t)u * W + slot) * G + rr % G) * r + e % r] * qscale;
    }
    qrow[e] = v;
  }
  __syncthreads();
  const int64_t L = c.lens[2 * u];
  const int64_t j0 = d.s, j1 = L - d.nrec;  // candidates
  const T* CK = (const T*)c.coef_k + (int64_t)u * c.Lmax * r;
  float m = -INFINITY, S = 0.f;
  if (row < nrows) {
    for (int t = lane; t < kWinTile; t += 32) {
      const int64_t j = j0 + (int64_t)tile * kWinTile + t;
      if (j >= j1) break;
      const T* cj = CK + j * r;
      float z = 0.f;
      for (int i = 0; i < r; ++i) z += qrow[(tid / 32) * r + i] * Elem<T>::ld(cj, i);
      const float mn = fmaxf(m, z);
      S = (m == -INFINITY ? 0.f : S * exp2f(m - mn)) + exp2f(z - mn);
      m = mn;
    }
  }
  // combine the 32 lanes of the row (fixed order)
  for (int o = 1; o < 32; o <<= 1) {
    const float m2 = __shfl_xor(m, o), S2 = __shfl_xor(S, o);
    const float mn = fmaxf(m, m2);
    const float a = m == -INFINITY ? 0.f : S * exp2f(m - mn);
    const float b = m2 == -INFINITY ? 0.f : S2 * exp2f(m2 - mn);
    S = a + b;
    m = mn;
  }
  if (lane == 0 && row < nrows) part[((int64_t)u * nrows + row) * ntile + tile] = make_float2(m, S);
}

// grid (1, U), 256 threads: merge the tiles of every pushed row into its
// running statistics, then count the pushes
__global__ __launch_bounds__(256) void k_window_merge(Dims d, CachePtrs c, int n_tail,
                                                      const float2* __restrict__ part, int ntile) {
  const int u = blockIdx.y, tid = threadIdx.x;
  const int G = d.G, W = d.W, nrows = n_tail * G;
  const int pushed0 = c.lens[2 * u + 1];
  float* rs = rowstat_of(c, u);
  for (int row = tid; row < nrows; row += 256) {
    float m = -INFINITY, S = 0.f;
    for (int t = 0; t < ntile; ++t) {
      const float2 p = part[((int64_t)u * nrows + row) * ntile + t];
      if (p.y == 0.f) continue;
      const float mn = fmaxf(m, p.x);
      S = (m == -INFINITY ? 0.f : S * exp2f(m - mn)) + p.y * exp2f(p.x - mn);
      m = mn;
    }
    const int slot = (pushed0 + row / G) % W;
    rs[(slot * G + row % G) * 2 + 0] = m;
    rs[(slot * G + row % G) * 2 + 1] = S;
  }
  __syncthreads();
  if (tid == 0) c.lens[2 * u + 1] = pushed0 + n_tail;
}

int64_t window_init_tiles(const Dims& d, int64_t L) {
  const int64_t nc = L - d.s - d.nrec;
  return nc > 0 ? (nc + kWinTile - 1) / kWinTile : 1;
}

size_t window_init_ws_bytes(const Dims& d, int64_t U, int64_t L, int n_tail) {
  return (size_t)U * n_tail * d.G * window_init_tiles(d, L) * sizeof(float2);
}

hipError_t launch_window_init(const Dims& d, int U, int64_t L, int n_tail, const void* q_tail,
                              const CachePtrs& c, void* ws, hipStream_t st) {
  const float qscale = kLog2e / sqrtf((float)d.r);
  const size_t lds = (size_t)d.G * d.D * sizeof(float);
  if (d.dtype == 0)
    hipLaunchKernelGGL(k_window_push<float>, dim3(n_tail, U), dim3(256), lds, st, d, c,
                       (const float*)q_tail, n_tail, qscale);
  else
    hipLaunchKernelGGL(k_window_push<uint16_t>, dim3(n_tail, U), dim3(256), lds, st, d, c,
                       (const uint16_t*)q_tail, n_tail, qscale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nrows = n_tail * d.G;
  const int ntile = (int)window_init_tiles(d, L);
  float2* part = (float2*)ws;
  const dim3 grid(ntile, (nrows + kWinRows - 1) / kWinRows, U);
  const size_t lq = (size_t)kWinRows * d.r * sizeof(float);
  if (d.dtype == 0)
    hipLaunchKernelGGL(k_window_stats<float>, grid, dim3(256), lq, st, d, c, n_tail, qscale, part, ntile);
  else
    hipLaunchKernelGGL(k_window_stats<uint16_t>, grid, dim3(256), lq, st, d, c, n_tail, qscale, part, ntile);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_window_merge, dim3(1, U), dim3(256), 0, st, d, c, n_tail, part, ntile);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// 8. bases shared over a window of neighbouring layers: the Gram matrices of
//    the layers of a window (same sequence) are summed into the window's
//    first layer, whose eigensolve then serves the whole window; the other
//    layers' matrices are frozen so the sweeps skip them, and the basis
//    extraction copies the first layer's result to them.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gram_window_sum(double* __restrict__ A, int* __restrict__ frozen,
                                                         int n, int n_layers, int batch, int depth) {
  // grid (ceil(n * n / 256), 2 * batch * ceil(n_layers / depth)): one
  // (window, sequence, K | V) per blockIdx.y
  const int nwin = (n_layers + depth - 1) / depth;
  const int y = blockIdx.y, kind = y & 1, wb = y >> 1, win = wb / batch, b = wb % batch;
  const int l0 = win * depth, l1 = min(l0 + depth, n_layers);
  if (win >= nwin) return;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int m0 = 2 * (l0 * batch + b) + kind;
  if (e < (int64_t)n * n) {
    double acc = A[(int64_t)m0 * n * n + e];
    for (int l = l0 + 1; l < l1; ++l) acc += A[(int64_t)(2 * (l * batch + b) + kind) * n * n + e];
    A[(int64_t)m0 * n * n + e] = acc;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0)
    for (int l = l0 + 1; l < l1; ++l) frozen[2 * (l * batch + b) + kind] = 1;
}

hipError_t launch_gram_window_sum(int n, int n_layers, int batch, int depth, double* A, int* frozen,
                                  hipStream_t st) {
  const int nwin = (n_layers + depth - 1) / depth;
  const int64_t n2 = (int64_t)n * n;
  hipLaunchKernelGGL(k_gram_window_sum, dim3((unsigned)((n2 + 255) / 256), 2 * batch * nwin), dim3(256), 0,
                     st, A, frozen, n, n_layers, batch, depth);
  return hipGetLastError();
}

}  // namespace kvlr
