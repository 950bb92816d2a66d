// k-means++ seeding (Arthur and Vassilvitskii 2007) for gfx950, one block
// per head.
//
// The m rounds are sequential, so a head's seeding stays inside one
// 1024-thread block: no inter-block synchronisation at all.  A round updates
// D^2 of every point of the strided subsample {floor(j*n/s)} (exact-input
// fp64 over bf16 points, 16 lanes per point so every row read is coalesced),
// then draws the next centre with probability proportional to D^2 using a
// fixed-order block scan.  The first rows of the subsample are staged in LDS
// once and stay there for all rounds; only the rest is re-read each round.
#include "common.h"
#include "internal.h"

namespace ac {

constexpr int KPP_THREADS = 1024;
constexpr int KPP_WAVES = KPP_THREADS / 64;
constexpr int KPP_GROUPS = KPP_THREADS / 16;  // points handled at once
constexpr int KPP_LDS_BYTES = 147456;         // subsample rows kept in LDS (144 KiB)

// Inclusive block scan of one double per thread in a fixed order (wave
// shuffle scan, then wave offsets summed in order).  *excl receives the
// inclusive value of the previous thread (0 for thread 0) bit-for-bit and
// *total that of the last thread.
AC_DEV double block_scan(double v, double *excl, double *total, double *sh_wt, double *sh_off) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  double inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  const double prev_local = __shfl_up(inc, 1, 64);
  if (lane == 63) sh_wt[wave] = inc;
  __syncthreads();
  if (tid == 0) {
    double off = 0.0;
    for (int w = 0; w < KPP_WAVES; ++w) {
      sh_off[w] = off;
      off = off + sh_wt[w];
    }
    sh_off[KPP_WAVES] = off;
  }
  __syncthreads();
  const double o = sh_off[wave];
  *excl = lane == 0 ? o : o + prev_local;
  *total = sh_off[KPP_WAVES];
  const double incl = o + inc;
  __syncthreads();
  return incl;
}

template <int D>
__global__ __launch_bounds__(KPP_THREADS) void k_kpp(KmArgs a, double *__restrict__ d2buf, int init_sample,
                                                    uint64_t seed, int role, int stage) {
  constexpr int PL = D / 16;  // dims per lane
  const int h = blockIdx.x;
  const int n = a.n[h], m = a.m[h];
  if (n <= 0 || m <= 0) return;
  const int s = init_sample > 0 ? min(n, init_sample * m) : n;  // host guarantees s <= KPP_SMAX
  double *D2 = d2buf + (int64_t)h * KPP_SMAX;
  const uint16_t *X = a.X + (int64_t)h * a.x_hs;
  const int *idx = a.idx ? a.idx + (int64_t)h * a.idx_hs : nullptr;
  float *cent = a.cent + (int64_t)h * a.cent_hs + (int64_t)a.coff[h] * D;
  const uint64_t sid = stream_id((uint64_t)h, role, stage);
  const int tid = threadIdx.x, grp = tid >> 4, sub = tid & 15;

  __shared__ float c_sh[D];
  __shared__ double sh_wt[KPP_WAVES], sh_off[KPP_WAVES + 1];
  __shared__ int sh_pick;

  auto row_of = [&](int j) -> int64_t {
    const int li = (int)(((int64_t)j * n) / s);
    return idx ? (int64_t)idx[li] : (int64_t)li;
  };
  // a lane's PL bf16 values of a point, packed two per 32-bit word
  typedef uint32_t pw_t __attribute__((ext_vector_type(PL / 2)));
  auto load_pt = [&](int j) -> pw_t { return *(const pw_t *)(X + row_of(j) * D + sub * PL); };
  // the first R subsample rows stay in LDS for all rounds
  constexpr int RMAX = KPP_LDS_BYTES / (D * 2);
  __shared__ uint16_t xs[RMAX * D];
  const int R = min(s, RMAX);
  for (int j0 = 0; j0 < R; j0 += KPP_GROUPS) {
    const int j = j0 + grp;
    if (j < R) *(pw_t *)&xs[j * D + sub * PL] = load_pt(j);
  }
  const int cs = (s + KPP_THREADS - 1) / KPP_THREADS;  // thread chunk of the scan
  const int cb = min(s, tid * cs), ce = min(s, cb + cs);

  for (int t = 0; t < m; ++t) {
    const double u = uniform01(seed, sid, (uint64_t)t);
    if (t == 0) {
      if (tid == 0) sh_pick = min(s - 1, (int)(u * (double)s));
    } else {
      double loc = 0.0;
      for (int j = cb; j < ce; ++j) loc += D2[j];
      double excl, total;
      const double incl = block_scan(loc, &excl, &total, sh_wt, sh_off);
      if (total > 0.0) {
        const double target = u * total;
        if (tid == 0) sh_pick = s - 1;  // kept only if rounding puts the target past the end
        __syncthreads();
        if (ce > cb && excl <= target && target < incl) {
          double run = excl;
          int pj = ce - 1;
          for (int j = cb; j < ce; ++j) {
            run += D2[j];
            if (run > target) { pj = j; break; }
          }
          sh_pick = pj;
        }
      } else if (tid == 0) {
        sh_pick = min(s - 1, (int)(u * (double)s));
      }
    }
    __syncthreads();
    const int pj = sh_pick;
    if (tid < D) {
      const float v = bf2f(X[row_of(pj) * D + tid]);
      c_sh[tid] = v;
      cent[(int64_t)t * D + tid] = v;
    }
    __syncthreads();
    double cr[PL];
#pragma unroll
    for (int q = 0; q < PL; ++q) cr[q] = (double)c_sh[sub * PL + q];
    // D^2 update: LDS-resident rows, then the streamed rest
    for (int j0 = 0; j0 < s; j0 += KPP_GROUPS) {
      const int j = j0 + grp;
      double acc = 0.0;
      if (j < s) {
        const pw_t xv = j < R ? *(const pw_t *)&xs[j * D + sub * PL] : load_pt(j);
#pragma unroll
        for (int q = 0; q < PL; ++q) {
          const uint32_t w = xv[q >> 1];
          const double df = (double)bf2f((uint16_t)((q & 1) ? (w >> 16) : (w & 0xFFFFu))) - cr[q];
          acc = fma(df, df, acc);
        }
      }
      acc += __shfl_xor(acc, 1, 64);
      acc += __shfl_xor(acc, 2, 64);
      acc += __shfl_xor(acc, 4, 64);
      acc += __shfl_xor(acc, 8, 64);
      if (j < s && sub == 0) D2[j] = t == 0 ? acc : fmin(D2[j], acc);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Small subsamples: all pairwise squared distances first, then the rounds.
// Every pick is a subsample point, so ||x_j - c_t||^2 is row p_t of the
// subsample's distance matrix G.  G is computed once across all CUs as
// (|x_j|^2 + |x_k|^2) - 2 x_j.x_k with every dot product (squared norms
// included) accumulated by the same sequential fp64 fma chain over d, so
// identical rows give exactly 0; the sequential part then reads one G row per
// round instead of the whole subsample.
template <int D>
__global__ __launch_bounds__(256) void k_kpp_norms(KmArgs a, int init_sample, double *__restrict__ nx, int smax) {
  const int h = blockIdx.y;
  const int n = a.n[h], m = a.m[h];
  if (n <= 0 || m <= 0) return;
  const int s = init_sample > 0 ? min(n, init_sample * m) : n;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= s) return;
  const int li = (int)(((int64_t)j * n) / s);
  const int64_t row = a.idx ? (int64_t)a.idx[(int64_t)h * a.idx_hs + li] : (int64_t)li;
  const uint16_t *xr = a.X + (int64_t)h * a.x_hs + row * D;
  double acc = 0.0;
  for (int d = 0; d < D; ++d) {
    const double x = (double)bf2f(xr[d]);
    acc = fma(x, x, acc);
  }
  nx[(int64_t)h * smax + j] = acc;
}

template <int D>
__global__ __launch_bounds__(256) void k_kpp_gram(KmArgs a, int init_sample, const double *__restrict__ nx,
                                                  double *__restrict__ G, int smax) {
  const int h = blockIdx.y;
  const int n = a.n[h], m = a.m[h];
  if (n <= 0 || m <= 0) return;
  const int s = init_sample > 0 ? min(n, init_sample * m) : n;
  const int nt = (s + 63) / 64;
  const int tj = blockIdx.x / ((smax + 63) / 64), tk = blockIdx.x % ((smax + 63) / 64);
  if (tj >= nt || tk >= nt || tk < tj) return;
  // tiles transposed in LDS: xs[d][row] so 4 consecutive rows are one 8-byte read
  __shared__ uint16_t xj[D][64 + 4], xk[D][64 + 4];
  const int *idx = a.idx ? a.idx + (int64_t)h * a.idx_hs : nullptr;
  const uint16_t *X = a.X + (int64_t)h * a.x_hs;
  for (int q = threadIdx.x; q < 64 * (D / 8); q += 256) {
    const int r = q / (D / 8), c8 = (q % (D / 8)) * 8;
    u32x4_t vj = {0, 0, 0, 0}, vk = {0, 0, 0, 0};
    const int j = tj * 64 + r, k = tk * 64 + r;
    if (j < s) {
      const int li = (int)(((int64_t)j * n) / s);
      vj = *(const u32x4_t *)&X[(idx ? (int64_t)idx[li] : (int64_t)li) * D + c8];
    }
    if (k < s) {
      const int li = (int)(((int64_t)k * n) / s);
      vk = *(const u32x4_t *)&X[(idx ? (int64_t)idx[li] : (int64_t)li) * D + c8];
    }
    const uint16_t *ej = (const uint16_t *)&vj, *ek = (const uint16_t *)&vk;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      xj[c8 + i][r] = ej[i];
      xk[c8 + i][r] = ek[i];
    }
  }
  __syncthreads();
  const int rj = (threadIdx.x >> 4) * 4, rk = (threadIdx.x & 15) * 4;
  double acc[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[u][v] = 0.0;
  for (int d = 0; d < D; ++d) {
    const u32x2_t wj = *(const u32x2_t *)&xj[d][rj];
    const u32x2_t wk = *(const u32x2_t *)&xk[d][rk];
    double aj[4], ak[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      aj[u] = (double)bf2f((uint16_t)(u & 1 ? wj[u >> 1] >> 16 : wj[u >> 1] & 0xFFFFu));
      ak[u] = (double)bf2f((uint16_t)(u & 1 ? wk[u >> 1] >> 16 : wk[u >> 1] & 0xFFFFu));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[u][v] = fma(aj[u], ak[v], acc[u][v]);
  }
  double *Gh = G + (int64_t)h * smax * smax;
  const double *nxh = nx + (int64_t)h * smax;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = tj * 64 + rj + u, k = tk * 64 + rk + v;
      if (j < s && k < s) {
        const double g = fmax((nxh[j] + nxh[k]) - 2.0 * acc[u][v], 0.0);
        Gh[(int64_t)j * smax + k] = g;
        Gh[(int64_t)k * smax + j] = g;
      }
    }
}

template <int D>
__global__ __launch_bounds__(KPP_THREADS) void k_kpp_seq(KmArgs a, const double *__restrict__ G, int smax,
                                                        int init_sample, uint64_t seed, int role, int stage) {
  const int h = blockIdx.x;
  const int n = a.n[h], m = a.m[h];
  if (n <= 0 || m <= 0) return;
  const int s = init_sample > 0 ? min(n, init_sample * m) : n;  // <= smax <= KPP_GRAM_MAX
  const double *Gh = G + (int64_t)h * smax * smax;
  const uint16_t *X = a.X + (int64_t)h * a.x_hs;
  const int *idx = a.idx ? a.idx + (int64_t)h * a.idx_hs : nullptr;
  float *cent = a.cent + (int64_t)h * a.cent_hs + (int64_t)a.coff[h] * D;
  const uint64_t sid = stream_id((uint64_t)h, role, stage);
  const int tid = threadIdx.x;
  __shared__ double D2[KPP_GRAM_MAX];
  __shared__ double sh_wt[KPP_WAVES], sh_off[KPP_WAVES + 1];
  __shared__ int sh_pick;
  const int cs = (s + KPP_THREADS - 1) / KPP_THREADS;
  const int cb = min(s, tid * cs), ce = min(s, cb + cs);
  for (int t = 0; t < m; ++t) {
    const double u = uniform01(seed, sid, (uint64_t)t);
    if (t == 0) {
      if (tid == 0) sh_pick = min(s - 1, (int)(u * (double)s));
    } else {
      double loc = 0.0;
      for (int j = cb; j < ce; ++j) loc += D2[j];
      double excl, total;
      const double incl = block_scan(loc, &excl, &total, sh_wt, sh_off);
      if (total > 0.0) {
        const double target = u * total;
        if (tid == 0) sh_pick = s - 1;
        __syncthreads();
        if (ce > cb && excl <= target && target < incl) {
          double run = excl;
          int pj = ce - 1;
          for (int j = cb; j < ce; ++j) {
            run += D2[j];
            if (run > target) { pj = j; break; }
          }
          sh_pick = pj;
        }
      } else if (tid == 0) {
        sh_pick = min(s - 1, (int)(u * (double)s));
      }
    }
    __syncthreads();
    const int pj = sh_pick;
    if (tid < D) {
      const int li = (int)(((int64_t)pj * n) / s);
      const int64_t row = idx ? (int64_t)idx[li] : (int64_t)li;
      cent[(int64_t)t * D + tid] = bf2f(X[row * D + tid]);
    }
    const double *gr = Gh + (int64_t)pj * smax;
    for (int j = tid; j < s; j += KPP_THREADS) D2[j] = t == 0 ? gr[j] : fmin(D2[j], gr[j]);
    __syncthreads();
  }
}

void launch_kpp(int D, const KmArgs &a, int BH, double *d2buf, int init_sample, uint64_t seed, int role, int stage,
                hipStream_t st) {
  if (D == 64)
    hipLaunchKernelGGL(k_kpp<64>, dim3(BH), dim3(KPP_THREADS), 0, st, a, d2buf, init_sample, seed, role, stage);
  else
    hipLaunchKernelGGL(k_kpp<128>, dim3(BH), dim3(KPP_THREADS), 0, st, a, d2buf, init_sample, seed, role, stage);
}

void launch_kpp_gram(int D, const KmArgs &a, int BH, int smax, double *nx, double *G, int init_sample, uint64_t seed,
                     int role, int stage, hipStream_t st) {
  const int nt = (smax + 63) / 64;
  if (D == 64) {
    hipLaunchKernelGGL(k_kpp_norms<64>, dim3((smax + 255) / 256, BH), dim3(256), 0, st, a, init_sample, nx, smax);
    hipLaunchKernelGGL(k_kpp_gram<64>, dim3(nt * nt, BH), dim3(256), 0, st, a, init_sample, nx, G, smax);
    hipLaunchKernelGGL(k_kpp_seq<64>, dim3(BH), dim3(KPP_THREADS), 0, st, a, G, smax, init_sample, seed, role, stage);
  } else {
    hipLaunchKernelGGL(k_kpp_norms<128>, dim3((smax + 255) / 256, BH), dim3(256), 0, st, a, init_sample, nx, smax);
    hipLaunchKernelGGL(k_kpp_gram<128>, dim3(nt * nt, BH), dim3(256), 0, st, a, init_sample, nx, G, smax);
    hipLaunchKernelGGL(k_kpp_seq<128>, dim3(BH), dim3(KPP_THREADS), 0, st, a, G, smax, init_sample, seed, role, stage);
  }
}

}  // namespace ac
