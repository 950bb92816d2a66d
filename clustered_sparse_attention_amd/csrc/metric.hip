// Interaction-aware key clustering for gfx950 ("iCATS: Fast Video
// Generation via Interaction-Aware Sparse Attention and Timestep-Adaptive
// Sparsity", method section, interaction-aware clustering).
//
// The error of the query-key products when keys are replaced by their
// centre is the quadratic form (k - c) M (k - c)^T with M = Q^T Q, which the
// page approximates by M_Q = sum_r |A_r| mu_r^T mu_r over the query
// clusters.  The key assignment then minimises
//   (k - c) M (k - c)^T = k M k^T + c M c^T - 2 k . (M c),
// whose first term is the same for every centre: the existing MFMA
// assignment (argmin of norm_c - 2 x . op_c) runs unchanged with op_c = M c
// (bf16 high and low parts) and norm_c = c M c^T.
#include "common.h"
#include "internal.h"

namespace ac {

namespace {

// Sum of the raw member queries of query cluster blockIdx.x (fp64), in
// counting-sort order; D threads per member row, 256 / D rows at a time.
template <int D>
__global__ __launch_bounds__(256) void k_qsum(const uint16_t *__restrict__ Q, const int *__restrict__ perm,
                                              const int *__restrict__ seg, const int *__restrict__ ncl, int L,
                                              int nqcap, double *__restrict__ qsum, int *__restrict__ qcnt) {
  constexpr int RP = 256 / D;  // member rows in flight
  const int h = blockIdx.y, r = blockIdx.x, tid = threadIdx.x;
  const int dd = tid % D, sub = tid / D;
  __shared__ double red[RP][D];
  const int *sg = seg + (int64_t)h * (nqcap + 1);
  const bool live = r < ncl[h];
  const int b = live ? sg[r] : 0, e = live ? sg[r + 1] : 0;
  double acc = 0.0;
  for (int i = b + sub; i < e; i += RP) {
    const int64_t row = perm[(int64_t)h * L + i];
    acc += (double)bf2f(Q[((int64_t)h * L + row) * D + dd]);
  }
  red[sub][dd] = acc;
  __syncthreads();
  if (sub == 0) {
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < RP; ++k) s += red[k][dd];
    qsum[((int64_t)h * nqcap + r) * D + dd] = s;
    if (dd == 0) qcnt[(int64_t)h * nqcap + r] = e - b;
  }
}

// M_Q[h] = sum_r |A_r| mu_r^T mu_r = sum_r s_r^T s_r / |A_r| (s_r the member
// sum), accumulated in fp64 over the clusters in index order.
template <int D>
__global__ __launch_bounds__(256) void k_mq(const double *__restrict__ qsum, const int *__restrict__ qcnt, int nq,
                                            int nqcap, float *__restrict__ M) {
  const int h = blockIdx.y;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= D * D) return;
  const int i = idx / D, j = idx % D;
  const double *s = qsum + (int64_t)h * nqcap * D;
  const int *n = qcnt + (int64_t)h * nqcap;
  double acc = 0.0;
  for (int r = 0; r < nq; ++r)
    if (n[r] > 0) acc += s[(int64_t)r * D + i] * s[(int64_t)r * D + j] / (double)n[r];
  M[(int64_t)h * D * D + idx] = (float)acc;
}

// Centre operands under the metric: op = M c (bf16 high and low parts),
// norm = c M c^T, both from fp64 sums; one block per centre, one thread per
// dimension.
template <int D>
__global__ __launch_bounds__(D) void k_cent_prep_metric(KmArgs a, CentOps op, const float *__restrict__ M) {
  const int h = blockIdx.y, c = blockIdx.x, i = threadIdx.x;
  if (c >= a.m[h]) return;
  __shared__ float cs[D];
  __shared__ double red[D / 64];
  const float *cr = a.cent + (int64_t)h * a.cent_hs + (int64_t)(a.coff[h] + c) * D;
  cs[i] = cr[i];
  __syncthreads();
  const float *Mi = M + ((int64_t)h * D + i) * D;
  double v = 0.0;
  for (int j = 0; j < D; ++j) v += (double)Mi[j] * (double)cs[j];
  const float vf = (float)v;
  const uint16_t bh = f2bf(vf);
  op.hi[((int64_t)h * op.cap + c) * D + i] = bh;
  op.lo[((int64_t)h * op.cap + c) * D + i] = f2bf(vf - bf2f(bh));
  double t = wave_sum((double)cs[i] * v);
  if ((i & 63) == 0) red[i >> 6] = t;
  __syncthreads();
  if (i == 0) {
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < D / 64; ++k) s += red[k];
    op.norm[(int64_t)h * op.cap + c] = (float)s;
  }
}

}  // namespace

void launch_interaction_matrix(int D, const uint16_t *Q, const int *perm, const int *seg, const int *ncl, int L,
                               int nq, int nqcap, double *qsum, int *qcnt, float *M, int BH, hipStream_t st) {
  const dim3 g1((unsigned)nqcap, (unsigned)BH), g2((unsigned)((D * D + 255) / 256), (unsigned)BH);
  if (D == 64) {
    hipLaunchKernelGGL(k_qsum<64>, g1, dim3(256), 0, st, Q, perm, seg, ncl, L, nqcap, qsum, qcnt);
    hipLaunchKernelGGL(k_mq<64>, g2, dim3(256), 0, st, qsum, qcnt, nq, nqcap, M);
  } else {
    hipLaunchKernelGGL(k_qsum<128>, g1, dim3(256), 0, st, Q, perm, seg, ncl, L, nqcap, qsum, qcnt);
    hipLaunchKernelGGL(k_mq<128>, g2, dim3(256), 0, st, qsum, qcnt, nq, nqcap, M);
  }
}

void launch_cent_prep_metric(int D, const KmArgs &a, const CentOps &op, const float *M, int BH, int mmax,
                             hipStream_t st) {
  const dim3 g((unsigned)(mmax > 0 ? mmax : 1), (unsigned)BH);
  if (D == 64) hipLaunchKernelGGL(k_cent_prep_metric<64>, g, dim3(64), 0, st, a, op, M);
  else hipLaunchKernelGGL(k_cent_prep_metric<128>, g, dim3(128), 0, st, a, op, M);
}

}  // namespace ac
