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
// Distance matrix of the seeding subsample on fp64 matrix cores
// (v_mfma_f64_16x16x4_f64).  In k-step ks, lane group g = lane / 16 holds
// dimension g * D/4 + ks of its row, so each lane reads one contiguous run of
// D/4 values of its row once.  A dot product is the same sequence of MFMA
// accumulations wherever its pair sits, and the squared norms are the
// diagonal of the same product, so G = (|x_j|^2 + |x_k|^2) - 2 x_j.x_k is
// exactly 0 for identical rows.
typedef double f64x4_t __attribute__((ext_vector_type(4)));

template <int D>
AC_DEV void kpp_rows(const KmArgs &a, int h, int n, int s, int r0, u32x4_t (&v)[D / 32]) {
  // lane's run: row r0 + lane % 16 of the subsample, dims [g * D/4, (g + 1) * D/4)
  const int lane = threadIdx.x & 63, j = r0 + (lane & 15), g = lane >> 4;
  if (j < s) {
    const int li = (int)(((int64_t)j * n) / s);
    const int64_t row = a.idx ? (int64_t)a.idx[(int64_t)h * a.idx_hs + li] : (int64_t)li;
    const u32x4_t *src = (const u32x4_t *)(a.X + (int64_t)h * a.x_hs + row * D + g * (D / 4));
#pragma unroll
    for (int q = 0; q < D / 32; ++q) v[q] = src[q];
  } else {
#pragma unroll
    for (int q = 0; q < D / 32; ++q) v[q] = (u32x4_t){0, 0, 0, 0};
  }
}
template <int D> AC_DEV double kpp_elem(const u32x4_t (&v)[D / 32], int ks) {
  const uint32_t w = v[ks >> 3][(ks >> 1) & 3];
  return (double)bf2f((uint16_t)((ks & 1) ? (w >> 16) : (w & 0xFFFFu)));
}

// |x_j|^2 as the diagonal of a 16 x 16 block product of the rows with themselves
template <int D>
__global__ __launch_bounds__(64) void k_kpp_norms(KmArgs a, int init_sample, double *__restrict__ nx, int smax) {
  const int h = blockIdx.y;
  const int n = a.n[h], m = a.m[h];
  if (n <= 0 || m <= 0) return;
  const int s = init_sample > 0 ? min(n, init_sample * m) : n;
  const int r0 = blockIdx.x * 16;
  if (r0 >= s) return;
  u32x4_t v[D / 32];
  kpp_rows<D>(a, h, n, s, r0, v);
  f64x4_t acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int ks = 0; ks < D / 4; ++ks) {
    const double x = kpp_elem<D>(v, ks);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(x, x, acc, 0, 0, 0);
  }
  // lane holds column lane % 16 and rows lane / 16 + 4 p: the diagonal entry of
  // column c sits in lane c + 16 (c % 4), p = c / 4
  const int lane = threadIdx.x, col = lane & 15, g = lane >> 4;
  if ((col & 3) == g && r0 + col < s) nx[(int64_t)h * smax + r0 + col] = acc[col >> 2];
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
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // wave: 32 x 32 block (rows j0 + [0, 32), columns k0 + [0, 32)) as 2 x 2 MFMA tiles
  const int j0 = tj * 64 + (wave >> 1) * 32, k0 = tk * 64 + (wave & 1) * 32;
  u32x4_t vj[2][D / 32], vk[2][D / 32];
  kpp_rows<D>(a, h, n, s, j0, vj[0]);
  kpp_rows<D>(a, h, n, s, j0 + 16, vj[1]);
  kpp_rows<D>(a, h, n, s, k0, vk[0]);
  kpp_rows<D>(a, h, n, s, k0 + 16, vk[1]);
  f64x4_t acc[2][2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int w = 0; w < 2; ++w) acc[u][w] = (f64x4_t){0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int ks = 0; ks < D / 4; ++ks) {
    const double x0 = kpp_elem<D>(vj[0], ks), x1 = kpp_elem<D>(vj[1], ks);
    const double y0 = kpp_elem<D>(vk[0], ks), y1 = kpp_elem<D>(vk[1], ks);
    acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(x0, y0, acc[0][0], 0, 0, 0);
    acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(x0, y1, acc[0][1], 0, 0, 0);
    acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(x1, y0, acc[1][0], 0, 0, 0);
    acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(x1, y1, acc[1][1], 0, 0, 0);
  }
  // lane holds column k = k0 + 16 w + lane % 16 and rows j = j0 + 16 u + lane / 16 + 4 p
  double *Gh = G + (int64_t)h * smax * smax;
  const double *nxh = nx + (int64_t)h * smax;
  __shared__ double tr[4][32][33];  // this wave's block, for the transposed (symmetric) write
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int kl = 16 * w + (lane & 15);
      const int k = k0 + kl;
      const double nk = k < s ? nxh[k] : 0.0;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int jl = 16 * u + (lane >> 4) + 4 * p;
        const int j = j0 + jl;
        const double nj = j < s ? nxh[j] : 0.0;
        const double g = fmax((nj + nk) - 2.0 * acc[u][w][p], 0.0);
        tr[wave][jl][kl] = g;
        if (j < s && k < s) Gh[(int64_t)j * smax + k] = g;
      }
    }
  if (tk == tj) return;  // diagonal tiles hold both halves already
  __syncthreads();
  // G[k][j] = G[j][k]: lanes run along j, so the writes are coalesced
  for (int q = lane; q < 32 * 32; q += 64) {
    const int kl = q >> 5, jl = q & 31;
    const int j = j0 + jl, k = k0 + kl;
    if (j < s && k < s) Gh[(int64_t)k * smax + j] = tr[wave][jl][kl];
  }
}

// The m sequential rounds from the subsample's distance matrix G, one block
// per head.  Thread t holds D^2 of the subsample points [t cs, t cs + cs) in
// registers (cs <= KPP_SEQ_CS), so the draw walks the points in index order:
// wave scans of the per-thread sums, the wave totals in order through LDS,
// and the one lane whose range holds u * total finds the point.  Two barriers
// a round; the row of G of the new centre is then read straight into the
// registers (each thread its cs contiguous entries).  A round depends only on
// the previous pick's row of G, so the picks wait in LDS and their centre
// rows are copied out by the whole block every KPP_PICK_BUF rounds: the
// dependent index and point loads of a copy stay off the chain of rounds.
// 512 threads: fewer waves meet at each barrier than with 1024, while the
// per-thread runs stay short (16 points at most); 256 and 1024 measured slower.
constexpr int KPP_SEQ_THREADS = 512;
constexpr int KPP_SEQ_WAVES = KPP_SEQ_THREADS / 64;
constexpr int KPP_SEQ_CS = KPP_GRAM_MAX / KPP_SEQ_THREADS;
constexpr int KPP_PICK_BUF = 1024;

template <int D>
__global__ __launch_bounds__(KPP_SEQ_THREADS) void k_kpp_seq(KmArgs a, const double *__restrict__ G, int smax,
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
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ double sh_wt[KPP_SEQ_WAVES];
  __shared__ int sh_pick[2];
  __shared__ int sh_row[KPP_PICK_BUF];  // picks t0 + [0, KPP_PICK_BUF) not yet copied out
  const int cs = (s + KPP_SEQ_THREADS - 1) / KPP_SEQ_THREADS;
  const int cb = min(s, tid * cs), ne = min(s, cb + cs) - cb;  // this thread's points
  double d2[KPP_SEQ_CS];
  auto take_row = [&](int pj, bool first) {
    const double *gr = Gh + (int64_t)pj * smax + cb;
#pragma unroll
    for (int e = 0; e < KPP_SEQ_CS; ++e)
      if (e < ne) d2[e] = first ? gr[e] : fmin(d2[e], gr[e]);
  };
  // centres t0 + [0, cnt) from their subsample picks; called by the whole block
  auto put_centres = [&](int t0, int cnt) {
    __syncthreads();
    for (int q = tid; q < cnt; q += KPP_SEQ_THREADS) {
      const int li = (int)(((int64_t)sh_row[q] * n) / s);
      sh_row[q] = idx ? idx[li] : li;
    }
    __syncthreads();
    for (int q = tid; q < cnt * D; q += KPP_SEQ_THREADS) {
      const int tt = q / D, e = q % D;
      cent[(int64_t)(t0 + tt) * D + e] = bf2f(X[(int64_t)sh_row[tt] * D + e]);
    }
    __syncthreads();
  };
#pragma unroll
  for (int e = 0; e < KPP_SEQ_CS; ++e) d2[e] = 0.0;
  {
    const double u = uniform01(seed, sid, 0);
    const int pj = min(s - 1, (int)(u * (double)s));
    if (tid == 0) sh_row[0] = pj;
    take_row(pj, true);
  }
  for (int t = 1; t < m; ++t) {
    const double u = uniform01(seed, sid, (uint64_t)t);
    double loc = 0.0;
#pragma unroll
    for (int e = 0; e < KPP_SEQ_CS; ++e)
      if (e < ne) loc += d2[e];
    // wave scan on DPP moves: a shuffle scan costs two LDS permutes per fp64
    // step, each waited for, about a sixth of a round
    const double inc = wave_incl_scan(loc);
    const double prev = wave_prev(inc);  // the previous lane's inclusive sum, bit for bit
    if (lane == 63) sh_wt[wave] = inc;
    if (tid == 0) sh_pick[t & 1] = -1;
    __syncthreads();
    double off = 0.0, total = 0.0;
#pragma unroll
    for (int w = 0; w < KPP_SEQ_WAVES; ++w) {
      const double v = sh_wt[w];
      if (w < wave) off += v;
      total += v;
    }
    if (total > 0.0) {
      const double target = u * total;
      // the ranges [excl, incl) of consecutive lanes and waves tile [0, total)
      // exactly: both ends come from the same sums in the same order
      const double incl = off + inc, excl = lane == 0 ? off : off + prev;
      if (ne > 0 && excl <= target && target < incl) {
        double run = excl;
        int pj = cb + ne - 1;
#pragma unroll
        for (int e = 0; e < KPP_SEQ_CS; ++e) {
          if (e < ne) {
            run += d2[e];
            if (run > target) { pj = cb + e; break; }
          }
        }
        sh_pick[t & 1] = pj;
      }
    }
    __syncthreads();
    int pj = sh_pick[t & 1];
    if (total <= 0.0) pj = min(s - 1, (int)(u * (double)s));
    else if (pj < 0) pj = s - 1;  // u * total at the very top (rounding)
    if (tid == 0) sh_row[t % KPP_PICK_BUF] = pj;
    take_row(pj, false);
    if ((t + 1) % KPP_PICK_BUF == 0) put_centres(t + 1 - KPP_PICK_BUF, KPP_PICK_BUF);
  }
  if (m % KPP_PICK_BUF != 0) put_centres(m - m % KPP_PICK_BUF, m % KPP_PICK_BUF);
}

void launch_kpp(int D, const KmArgs &a, int BH, double *d2buf, int init_sample, uint64_t seed, int role, int stage,
                hipStream_t st) {
  if (D == 64)
    hipLaunchKernelGGL(k_kpp<64>, dim3(BH), dim3(KPP_THREADS), 0, st, a, d2buf, init_sample, seed, role, stage);
  else
    hipLaunchKernelGGL(k_kpp<128>, dim3(BH), dim3(KPP_THREADS), 0, st, a, d2buf, init_sample, seed, role, stage);
}

hipError_t launch_kpp_gram(int D, const KmArgs &a, int BH, int smax, double *nx, double *G, int init_sample,
                           uint64_t seed, int role, int stage, hipStream_t st, hipEvent_t after_gram) {
  const int nt = (smax + 63) / 64;
  if (D == 64) {
    hipLaunchKernelGGL(k_kpp_norms<64>, dim3((smax + 15) / 16, BH), dim3(64), 0, st, a, init_sample, nx, smax);
    hipLaunchKernelGGL(k_kpp_gram<64>, dim3(nt * nt, BH), dim3(256), 0, st, a, init_sample, nx, G, smax);
  } else {
    hipLaunchKernelGGL(k_kpp_norms<128>, dim3((smax + 15) / 16, BH), dim3(64), 0, st, a, init_sample, nx, smax);
    hipLaunchKernelGGL(k_kpp_gram<128>, dim3(nt * nt, BH), dim3(256), 0, st, a, init_sample, nx, G, smax);
  }
  const hipError_t ev = after_gram ? hipEventRecord(after_gram, st) : hipSuccess;
  if (D == 64)
    hipLaunchKernelGGL(k_kpp_seq<64>, dim3(BH), dim3(KPP_SEQ_THREADS), 0, st, a, G, smax, init_sample, seed, role, stage);
  else
    hipLaunchKernelGGL(k_kpp_seq<128>, dim3(BH), dim3(KPP_SEQ_THREADS), 0, st, a, G, smax, init_sample, seed, role, stage);
  return ev;
}

}  // namespace ac
