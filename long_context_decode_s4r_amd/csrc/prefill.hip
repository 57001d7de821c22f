// Prefill kernels: sample + token-wise normalisation, Gram matrix S^T S,
// parallel cyclic Jacobi eigensolver, top-r basis extraction, projection of
// every non-sink token onto the bases, exact sink / recent-window copies.
//
// Method: S^4R review (pith.science/paper/2608.00528), 'What carries the
// argument' (truncated SVD over a sampled, token-wise-normalised subset,
// Eqs. 1-2; coefficients c = s.B, Eq. 3) and 'Core claim' (s sinks kept in
// full precision, 7:3 recent-to-uniform sample of T' tokens).
#include "common.h"

#include <math.h>

namespace kvlr {

// --------------------------------------------------------------------------
// 1. sample + normalise: S[m][i][:] = rnd(x_p / ||x_p||), m = 2u + (0 K | 1 V)
//    sample position p(i): the first n_u entries are evenly spaced over
//    [s, L - n_r), the last n_r are the most recent prompt positions.
// --------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_sample_normalize(const T* __restrict__ K,
                                                          const T* __restrict__ V,
                                                          T* __restrict__ S, int64_t L, int D,
                                                          int nT, int s, int rnum, int rden) {
  const int i = blockIdx.x;
  const int m = blockIdx.y;
  const int u = m >> 1;
  const T* X = (m & 1) ? V : K;
  const int64_t n_r = ((int64_t)rnum * nT) / rden;
  const int64_t n_u = nT - n_r;
  int64_t p;
  if (i < n_u) {
    const int64_t span = L - n_r - s;
    p = s + ((int64_t)i * span) / n_u;
  } else {
    p = L - n_r + (i - n_u);
  }
  const T* row = X + ((int64_t)u * L + p) * D;
  double ss = 0.0;
  for (int j = threadIdx.x; j < D; j += blockDim.x) {
    double x = (double)Elem<T>::ld(row, j);
    ss += x * x;
  }
  __shared__ double red[256];
  red[threadIdx.x] = ss;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  const double tot = red[0];
  const double inv = tot > 0.0 ? 1.0 / sqrt(tot) : 0.0;
  T* out = S + ((int64_t)m * nT + i) * D;
  for (int j = threadIdx.x; j < D; j += blockDim.x)
    Elem<T>::st(out, j, (float)((double)Elem<T>::ld(row, j) * inv));
}

hipError_t launch_sample_normalize(const Dims& d, int U, int64_t L, const void* K, const void* V,
                                   void* S, hipStream_t st) {
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

hipError_t launch_gram(const Dims& d, int nmat, const void* S, double* A, double* Vm,
                       hipStream_t st) {
  const int D = d.D;
  const int64_t n2 = (int64_t)D * D;
  if (d.dtype == 0) {
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
constexpr int kJacRowsPerBlock = 16;

__global__ __launch_bounds__(256) void k_offnorm(const double* __restrict__ A,
                                                 const int* __restrict__ frozen,
                                                 double* __restrict__ part, int n, int nchunk) {
  const int m = blockIdx.y;
  if (frozen[m]) return;
  const double* Am = A + (int64_t)m * n * n;
  const int r0 = blockIdx.x * kJacRowsPerBlock;
  double off = 0.0, tr = 0.0;
  for (int r = r0; r < min(r0 + kJacRowsPerBlock, n); ++r) {
    for (int c = threadIdx.x; c < n; c += blockDim.x) {
      const double x = Am[(int64_t)r * n + c];
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
                               int* __restrict__ final_buf, int* __restrict__ n_active, int nmat,
                               int nchunk, int cur, double tol) {
  __shared__ int cnt;
  if (threadIdx.x == 0) cnt = 0;
  __syncthreads();
  for (int m = threadIdx.x; m < nmat; m += blockDim.x) {
    if (frozen[m]) continue;
    double off = 0.0, tr = 0.0;
    for (int c = 0; c < nchunk; ++c) {
      off += part[((int64_t)m * nchunk + c) * 2 + 0];
      tr += part[((int64_t)m * nchunk + c) * 2 + 1];
    }
    if (sqrt(off) <= tol * fabs(tr) || off == 0.0) {
      frozen[m] = 1;
      final_buf[m] = cur;
    } else {
      atomicAdd(&cnt, 1);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) *n_active = cnt;
}

hipError_t launch_jacobi_check(int n, int nmat, const double* A, double* part, int* frozen,
                               int* final_buf, int cur, int* n_active, double tol,
                               hipStream_t st) {
  const int nchunk = (n + kJacRowsPerBlock - 1) / kJacRowsPerBlock;
  hipLaunchKernelGGL(k_offnorm, dim3(nchunk, nmat), dim3(256), 0, st, A, frozen, part, n, nchunk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_jacobi_check, dim3(1), dim3(256), 0, st, part, frozen, final_buf, n_active,
                     nmat, nchunk, cur, tol);
  return hipGetLastError();
}

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
__global__ __launch_bounds__(kBJEigThreads) void k_bjac_eig(const double* __restrict__ Aall,
                                                            double* __restrict__ Qall,
                                                            const int* __restrict__ frozen, int n,
                                                            int k) {
  const int m = blockIdx.y;
  if (frozen[m]) return;
  constexpr int NT = kBJEigThreads, NP = kBJ2 / 2;
  static_assert(NP * NP == NT && kBJ2 * NP == 2 * NT, "one 2x2 block and two Q pairs per thread");
  static_assert((kBJ & (kBJ - 1)) == 0, "cross-round pairs use a power-of-two block");
  const int nb = n / kBJ, p = blockIdx.x, tid = threadIdx.x;
  int I, J;
  bj_pair(p, k, nb, &I, &J);
  const double* A = Aall + (int64_t)m * n * n;
  __shared__ double S[kBJ2][kBJ2 + 1];
  __shared__ double Q[kBJ2][kBJ2 + 1];
  __shared__ double rc[NP], rs[NP], rt[NP];
  __shared__ uint8_t pi[kBJ][NP], qi[kBJ][NP];
  for (int e = tid; e < kBJ2 * kBJ2; e += NT) {
    const int i = e / kBJ2, j = e % kBJ2;
    S[i][j] = A[(int64_t)bj_index(i, I, J) * n + bj_index(j, I, J)];
    Q[i][j] = i == j ? 1.0 : 0.0;
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
  double x0 = qrow == qb ? 1.0 : 0.0, y0 = 0.0, x1 = 0.0, y1 = x0;
  const int ysrc = (tid & 32) | ((tid + 1) & 31);
  {
    for (int kr = 0; kr < nround; ++kr) {
      if (tid < NP) {
        const int ip = qreg ? tid : pi[kr][tid], iq = qreg ? kBJ + ((tid + kr) & (kBJ - 1)) : qi[kr][tid];
        const double app = S[ip][ip], aqq = S[iq][iq], apq = S[ip][iq];
        double c = 1.0, sn = 0.0, t = 0.0;
        if (apq != 0.0) {
          // the rotation above with tau = d / (2 apq) multiplied through by
          // |2 apq|: t = sgn(tau) 2|apq| / (|d| + sqrt(d^2 + 4 apq^2)), one
          // square root and one division (the entries are Gram sums of unit
          // vectors, far from overflow)
          const double d = aqq - app, a2 = 2.0 * fabs(apq);
          const bool neg = (d < 0.0) != (apq < 0.0) && d != 0.0;
          t = a2 / (fabs(d) + sqrt(d * d + a2 * a2));
          t = neg ? -t : t;
          c = rsqrt(1.0 + t * t);
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
      const double m00 = S[pa][pb], m01 = S[pa][qbb], m10 = S[qa][pb], m11 = S[qa][qbb];
      const double cq = rc[qb], sq = rs[qb];
      if (a == b) {
        const double ta = rt[a];
        S[pa][pa] = m00 - ta * m01;
        S[qa][qa] = m11 + ta * m01;
        S[pa][qa] = 0.0;
        S[qa][pa] = 0.0;
      } else {
        const double ca = rc[a], sa = rs[a], cb = rc[b], sb = rs[b];
        const double r00 = ca * m00 - sa * m10, r01 = ca * m01 - sa * m11;
        const double r10 = sa * m00 + ca * m10, r11 = sa * m01 + ca * m11;
        S[pa][pb] = cb * r00 - sb * r01;
        S[pa][qbb] = sb * r00 + cb * r01;
        S[qa][pb] = cb * r10 - sb * r11;
        S[qa][qbb] = sb * r10 + cb * r11;
      }
      if (qreg) {
        const double n0 = sq * x0 + cq * y0, n1 = sq * x1 + cq * y1;
        x0 = cq * x0 - sq * y0;
        x1 = cq * x1 - sq * y1;
        y0 = kr + 1 < nround ? __shfl(n0, ysrc) : n0;
        y1 = kr + 1 < nround ? __shfl(n1, ysrc) : n1;
      } else {
        const double v00 = Q[qrow][pq], v01 = Q[qrow][qq];
        const double v10 = Q[qrow + NP][pq], v11 = Q[qrow + NP][qq];
        Q[qrow][pq] = cq * v00 - sq * v01;
        Q[qrow][qq] = sq * v00 + cq * v01;
        Q[qrow + NP][pq] = cq * v10 - sq * v11;
        Q[qrow + NP][qq] = sq * v10 + cq * v11;
      }
      __syncthreads();
    }
  }
  double* Qo = Qall + ((int64_t)m * (nb / 2) + p) * kBJ2 * kBJ2;
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

// grid ((nb/2)^2 + (n/64)(nb/2), nmat), 256 threads: the in-place update of
// A's tiles (P, P') and V's tiles (row tile R, pair P) of outer round k.
// The 64 x 64 x 64 products run on fp64 MFMA 16x16x4 (lane l: A[l % 16][l / 16],
// B[l / 16][l % 16]; D element v at row l / 16 + 4 v, column l % 16); wave w
// computes the 32 x 32 quadrant (w / 2, w % 2), four 16 x 16 tiles; the
// tile operand is read from LDS (row stride 65 doubles: the transposed
// stores of 16 lanes land in distinct banks), the Q operands from memory.
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int kBJLd = kBJ2 + 1;

__global__ __launch_bounds__(256) void k_bjac_apply(double* __restrict__ Aall,
                                                    double* __restrict__ Vall,
                                                    const double* __restrict__ Qall,
                                                    const int* __restrict__ frozen, int n, int k) {
  const int m = blockIdx.y;
  if (frozen[m]) return;
  const int nb = n / kBJ, np = nb / 2, tid = threadIdx.x;
  const int l = tid & 63, w = tid >> 6, qi = w >> 1, qj = w & 1, c16 = l & 15, r4 = l >> 4;
  const int tile = blockIdx.x;
  constexpr int NKS = kBJ2 / 4;  // MFMA k-steps
  __shared__ __attribute__((aligned(16))) double X[kBJ2][kBJLd];  // the tile (V: transposed)
  const double* Qm = Qall + (int64_t)m * np * kBJ2 * kBJ2;
  f64x4 acc[2][2];
  // the Q factors' MFMA operands come straight from memory (L2) into
  // registers: lane (r4, c16) of k-step ks needs Q[4 ks + r4][col + c16]
  auto qfrag = [&](const double* Qp, int col, double (&f0)[NKS], double (&f1)[NKS]) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      f0[ks] = Qp[(4 * ks + r4) * kBJ2 + col + c16];
      f1[ks] = Qp[(4 * ks + r4) * kBJ2 + col + 16 + c16];
    }
  };
  auto zero = [&]() {
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int tj = 0; tj < 2; ++tj) acc[ti][tj] = f64x4{0.0, 0.0, 0.0, 0.0};
  };
  // acc[ti][tj][v] = sum_k A'[k][32 qi + 16 ti + r4 + 4 v] B'[k][32 qj + 16 tj + c16]
  // with A' from registers (a0, a1) and B' = X, or A' = X and B' from registers
  auto gemm_ra = [&](const double (&a0)[NKS], const double (&a1)[NKS]) {
    zero();
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int kr = 4 * ks + r4;
      const double b0 = X[kr][32 * qj + c16], b1 = X[kr][32 * qj + 16 + c16];
      acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0[ks], b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0[ks], b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1[ks], b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1[ks], b1, acc[1][1], 0, 0, 0);
    }
  };
  auto gemm_rb = [&](const double (&b0)[NKS], const double (&b1)[NKS]) {
    zero();
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int kr = 4 * ks + r4;
      const double a0 = X[kr][32 * qi + c16], a1 = X[kr][32 * qi + 16 + c16];
      acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0[ks], acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1[ks], acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0[ks], acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1[ks], acc[1][1], 0, 0, 0);
    }
  };
  // output element (ti, tj, v) of this lane: row orow(ti, v), column ocol(tj)
  auto orow = [&](int ti, int v) { return 32 * qi + 16 * ti + r4 + 4 * v; };
  auto ocol = [&](int tj) { return 32 * qj + 16 * tj + c16; };
  if (tile < np * np) {
    const int P = tile / np, P2 = tile % np;
    int I, J, I2, J2;
    bj_pair(P, k, nb, &I, &J);
    bj_pair(P2, k, nb, &I2, &J2);
    double* A = Aall + (int64_t)m * n * n;
    double qa0[NKS], qa1[NKS];
    qfrag(Qm + (int64_t)P * kBJ2 * kBJ2, 32 * qi, qa0, qa1);  // A' = Q_P (rows of Q_P^T)
    for (int e = tid; e < kBJ2 * kBJ2 / 2; e += 256) {  // pairs of columns, 16-byte loads
      const int i = e / (kBJ2 / 2), j = 2 * (e % (kBJ2 / 2));
      const double2 x = *reinterpret_cast<const double2*>(A + (int64_t)bj_index(i, I, J) * n + bj_index(j, I2, J2));
      X[i][j] = x.x;
      X[i][j + 1] = x.y;
    }
    __syncthreads();
    gemm_ra(qa0, qa1);  // T = Q_P^T X
    double qb0[NKS], qb1[NKS];
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
          A[(int64_t)bj_index(orow(ti, v), I, J) * n + bj_index(ocol(tj), I2, J2)] = acc[ti][tj][v];
  } else {
    const int t2 = tile - np * np, R = t2 / np, P = t2 % np;
    int I, J;
    bj_pair(P, k, nb, &I, &J);
    double* V = Vall + (int64_t)m * n * n;
    double qb0[NKS], qb1[NKS];
    qfrag(Qm + (int64_t)P * kBJ2 * kBJ2, 32 * qj, qb0, qb1);  // B' = Q_P
    for (int e = tid; e < kBJ2 * kBJ2 / 2; e += 256) {
      const int i = e / (kBJ2 / 2), j = 2 * (e % (kBJ2 / 2));
      const double2 x = *reinterpret_cast<const double2*>(V + (int64_t)(kBJ2 * R + i) * n + bj_index(j, I, J));
      X[j][i] = x.x;
      X[j + 1][i] = x.y;
    }
    __syncthreads();
    gemm_rb(qb0, qb1);  // V[R, P] Q_P
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int tj = 0; tj < 2; ++tj)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          V[(int64_t)(kBJ2 * R + orow(ti, v)) * n + bj_index(ocol(tj), I, J)] = acc[ti][tj][v];
  }
}

bool bjac_supported(int n) { return n >= 2 * kBJ2 && n % kBJ2 == 0; }

size_t bjac_q_bytes(int n, int nmat) { return (size_t)nmat * (n / kBJ2) * kBJ2 * kBJ2 * sizeof(double); }

hipError_t launch_bjac_round(int n, int nmat, double* A, double* V, double* Qbuf, const int* frozen,
                             int k, hipStream_t st) {
  const int nb = n / kBJ, np = nb / 2;
  hipLaunchKernelGGL(k_bjac_eig, dim3(np, nmat), dim3(kBJEigThreads), 0, st, A, Qbuf, frozen, n, k);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_bjac_apply, dim3(np * np + (n / kBJ2) * np, nmat), dim3(256), 0, st, A, V, Qbuf,
                     frozen, n, k);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// 4. eigenvalues descending (bitonic sort of (lambda, slot) in LDS), basis =
//    the first r eigenvector columns, rounded to storage.
// --------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(1024) void k_extract(const double* __restrict__ A0,
                                                  const double* __restrict__ A1,
                                                  const double* __restrict__ V0,
                                                  const double* __restrict__ V1,
                                                  const int* __restrict__ frozen,
                                                  const int* __restrict__ final_buf, int cur,
                                                  int n, int r, T* __restrict__ BK,
                                                  T* __restrict__ BV, float* __restrict__ eigK,
                                                  float* __restrict__ eigV) {
  extern __shared__ unsigned char smem_raw[];
  const int m = blockIdx.x, u = m >> 1, kind = m & 1;
  const int buf = frozen[m] ? final_buf[m] : cur;
  const double* A = (buf ? A1 : A0) + (int64_t)m * n * n;
  const double* Vm = (buf ? V1 : V0) + (int64_t)m * n * n;
  int np2 = 1;
  while (np2 < n) np2 <<= 1;
  double* key = reinterpret_cast<double*>(smem_raw);
  int* idx = reinterpret_cast<int*>(key + np2);
  for (int i = threadIdx.x; i < np2; i += blockDim.x) {
    key[i] = i < n ? A[(int64_t)i * n + i] : -INFINITY;
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
  T* B = (kind ? BV : BK) + (int64_t)u * n * r;
  for (int64_t e = threadIdx.x; e < (int64_t)n * r; e += blockDim.x) {
    const int i = (int)(e / r), c = (int)(e % r);
    Elem<T>::st(B, e, (float)Vm[(int64_t)i * n + idx[c]]);
  }
}

hipError_t launch_extract(const Dims& d, int nmat, const double* A0, const double* A1,
                          const double* V0, const double* V1, const int* frozen,
                          const int* final_buf, int cur, void* basis_k, void* basis_v,
                          float* eig_k, float* eig_v, hipStream_t st) {
  int np2 = 1;
  while (np2 < d.D) np2 <<= 1;
  const size_t lds = (size_t)np2 * (sizeof(double) + sizeof(int));
  if (d.dtype == 0)
    hipLaunchKernelGGL(k_extract<float>, dim3(nmat), dim3(1024), lds, st, A0, A1, V0, V1, frozen,
                       final_buf, cur, d.D, d.r, (float*)basis_k, (float*)basis_v, eig_k, eig_v);
  else
    hipLaunchKernelGGL(k_extract<uint16_t>, dim3(nmat), dim3(1024), lds, st, A0, A1, V0, V1,
                       frozen, final_buf, cur, d.D, d.r, (uint16_t*)basis_k, (uint16_t*)basis_v,
                       eig_k, eig_v);
  return hipGetLastError();
}

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
                                                      int64_t Lmax, int D, int r, int s) {
  const int u = blockIdx.y >> 1, kind = blockIdx.y & 1;
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

__global__ __launch_bounds__(256) void k_basis_t(const uint16_t* __restrict__ BK,
                                                 const uint16_t* __restrict__ BV,
                                                 uint16_t* __restrict__ BT, int D, int r) {
  // tile of 32 channels x 32 columns; BT[u][kind][n][k] = B[u][kind][k][n]
  __shared__ uint16_t t[32][33];
  const int um = blockIdx.z, u = um >> 1, kind = um & 1;
  const uint16_t* B = (kind ? BV : BK) + (int64_t)u * D * r;
  uint16_t* T = BT + (int64_t)um * r * D;
  const int k0 = blockIdx.x * 32, n0 = blockIdx.y * 32;
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

// NS = D' / 64 steps when known at compile time (the loop then unrolls), 0 =
// runtime
template <int R, int NS>
__global__ __launch_bounds__(kProjWaves * 64) void k_project_mfma(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ BT, uint16_t* __restrict__ CK, uint16_t* __restrict__ CV,
    int64_t L, int64_t Lmax, int D, int s) {
  constexpr int NT = kProjWaves * 64;
  constexpr int NCB = R / 32;
  constexpr int SB = R * kProjK * 2;         // stage bytes
  constexpr int NPB = SB / 16 / NT;          // 16-byte B^T pieces per thread per step
  constexpr int AR = kProjRing;
  static_assert(SB % (16 * NT) == 0, "rank must be a multiple of 64");
  __shared__ __attribute__((aligned(16))) uint8_t stg[2 * SB];
  const int um = blockIdx.y, u = um >> 1, kind = um & 1;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, mm = l & 31, kg = l >> 5;
  const uint16_t* X = (kind ? V : K) + (int64_t)u * L * D;
  const uint16_t* Bt = BT + (int64_t)um * R * D;
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
                                                     int64_t L, int64_t Lmax, int D, int r, int s) {
  const int u = blockIdx.y >> 1, kind = blockIdx.y & 1;
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

template <int R>
static hipError_t launch_project_mfma(const Dims& d, int U, int64_t L, int64_t Lmax, const void* K,
                                      const void* V, const void* BK, const void* BV, void* CK,
                                      void* CV, uint16_t* BT, hipStream_t st) {
  hipLaunchKernelGGL(k_basis_t, dim3((d.D + 31) / 32, R / 32, 2 * U), dim3(256), 0, st,
                     (const uint16_t*)BK, (const uint16_t*)BV, BT, d.D, R);
  const int64_t nrow = L - d.s;
  const dim3 grid((unsigned)((nrow + kProjRows - 1) / kProjRows), 2 * U);
#define KVLR_PROJ_LAUNCH(NS)                                                                     \
  hipLaunchKernelGGL((k_project_mfma<R, NS>), grid, dim3(kProjWaves * 64), 0, st,               \
                     (const uint16_t*)K,                                                        \
                     (const uint16_t*)V, (const uint16_t*)BT, (uint16_t*)CK, (uint16_t*)CV, L,  \
                     Lmax, d.D, d.s)
  switch (d.D / kProjK) {
    case 8: KVLR_PROJ_LAUNCH(8); break;
    case 16: KVLR_PROJ_LAUNCH(16); break;
    default: KVLR_PROJ_LAUNCH(0); break;
  }
#undef KVLR_PROJ_LAUNCH
  return hipGetLastError();
}

size_t project_ws_bytes(const Dims& d, int64_t U) {
  if (d.dtype == 0 || d.r % 64 != 0 || d.D % (kProjRing * kProjK) != 0) return 0;
  return (size_t)U * 2 * d.r * d.D * sizeof(uint16_t);
}

hipError_t launch_project(const Dims& d, int U, int64_t L, int64_t Lmax, const void* K,
                          const void* V, const void* BK, const void* BV, void* CK, void* CV,
                          void* ws, hipStream_t st) {
  const int64_t nrow = L - d.s;
  if (nrow <= 0) return hipSuccess;
  if (project_ws_bytes(d, U) > 0) {
    uint16_t* BT = (uint16_t*)ws;
    switch (d.r) {
      case 64: return launch_project_mfma<64>(d, U, L, Lmax, K, V, BK, BV, CK, CV, BT, st);
      case 128: return launch_project_mfma<128>(d, U, L, Lmax, K, V, BK, BV, CK, CV, BT, st);
      case 192: return launch_project_mfma<192>(d, U, L, Lmax, K, V, BK, BV, CK, CV, BT, st);
      case 256: return launch_project_mfma<256>(d, U, L, Lmax, K, V, BK, BV, CK, CV, BT, st);
      default: break;
    }
  }
  if (d.dtype == 0) {
    const int64_t tot = nrow * d.r;
    hipLaunchKernelGGL(k_project_f32, dim3((unsigned)((tot + 255) / 256), 2 * U), dim3(256), 0, st,
                       (const float*)K, (const float*)V, (const float*)BK, (const float*)BV,
                       (float*)CK, (float*)CV, L, Lmax, d.D, d.r, d.s);
  } else {
    hipLaunchKernelGGL(k_project_bf16, dim3((unsigned)((nrow + 63) / 64), 2 * U), dim3(256), 0,
                       st, (const uint16_t*)K, (const uint16_t*)V, (const uint16_t*)BK,
                       (const uint16_t*)BV, (uint16_t*)CK, (uint16_t*)CV, L, Lmax, d.D, d.r, d.s);
  }
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// 6. exact sinks + recent ring, window / statistics reset, lens = {L, 0}
// --------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_exact_reset(const T* __restrict__ K,
                                                     const T* __restrict__ V, T* __restrict__ sk,
                                                     T* __restrict__ sv, T* __restrict__ rk,
                                                     T* __restrict__ rv, float* __restrict__ qwin,
                                                     uint16_t* __restrict__ qsplit,
                                                     float* __restrict__ rowstat,
                                                     int32_t* __restrict__ lens, int64_t L, int D,
                                                     int s, int nrec, int qw_per_unit,
                                                     int rs_per_unit) {
  const int u = blockIdx.y;
  const int row = blockIdx.x;  // [0, s + nrec) exact rows, then one block for the reset
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
    for (int j = threadIdx.x; j < qw_per_unit; j += blockDim.x) qwin[(int64_t)u * qw_per_unit + j] = 0.f;
    for (int j = threadIdx.x; j < 2 * qw_per_unit; j += blockDim.x) qsplit[(int64_t)u * 2 * qw_per_unit + j] = 0;
    for (int j = threadIdx.x; j < rs_per_unit; j += blockDim.x) rowstat[(int64_t)u * rs_per_unit + j] = 0.f;
    if (threadIdx.x == 0) {
      lens[2 * u] = (int32_t)L;
      lens[2 * u + 1] = 0;
    }
  }
}

hipError_t launch_exact_and_reset(const Dims& d, int U, int64_t L, const void* K, const void* V,
                                  void* sink_k, void* sink_v, void* ring_k, void* ring_v,
                                  float* qwin, float* rowstat, int32_t* lens, uint16_t* qsplit,
                                  hipStream_t st) {
  dim3 grid(d.s + d.nrec + 1, U);
  const int qw = d.W * d.G * d.r, rs = d.W * d.G * 2;
  if (d.dtype == 0)
    hipLaunchKernelGGL(k_exact_reset<float>, grid, dim3(256), 0, st, (const float*)K,
                       (const float*)V, (float*)sink_k, (float*)sink_v, (float*)ring_k,
                       (float*)ring_v, qwin, qsplit, rowstat, lens, L, d.D, d.s, d.nrec, qw, rs);
  else
    hipLaunchKernelGGL(k_exact_reset<uint16_t>, grid, dim3(256), 0, st, (const uint16_t*)K,
                       (const uint16_t*)V, (uint16_t*)sink_k, (uint16_t*)sink_v,
                       (uint16_t*)ring_k, (uint16_t*)ring_v, qwin, qsplit, rowstat, lens, L, d.D, d.s,
                       d.nrec, qw, rs);
  return hipGetLastError();
}

}  // namespace kvlr
