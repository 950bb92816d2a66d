// Clustering kernels for gfx950: query normalisation, batched k-means
// (k-means++ seeding, MFMA distance GEMM with a fused argmin, counting-sort
// based centre update), the per-stage distance / threshold / compaction steps
// of AdaCluster Algorithm 1, and the per-cluster key statistics.
//
// A "job" runs one k-means per head over that head's point list: point i of
// head h is row idx[h][i] (or row i when idx is NULL) of X[h], there are n[h]
// points and m[h] centres, stored at cent[h][coff[h] + c].  Heads with n = 0
// or m = 0 are idle.  Every launch covers all heads (grid.y = head).
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace ac {

// ---------------------------------------------------------------------------
// Query normalisation (AdaCluster §3.1): q_hat = bf16(q / ||q||), ||q|| fp32.
// Eight lanes per row; the norm and quotient are fp64, rounded once to bf16.
template <int D>
__global__ __launch_bounds__(256) void k_qnorm(const uint16_t *__restrict__ Q, uint16_t *__restrict__ Qh,
                                               float *__restrict__ qn, int64_t rows) {
  constexpr int PER = D / 8;  // dims per lane
  int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / 8;
  int sub = threadIdx.x & 7;
  if (row >= rows) return;  // whole 8-lane groups exit together
  const uint16_t *src = Q + row * D + sub * PER;
  uint16_t v[PER];
#pragma unroll
  for (int i = 0; i < PER; i += 8) *(u32x4_t *)&v[i] = *(const u32x4_t *)&src[i];
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    double x = (double)bf2f(v[i]);
    ss += x * x;
  }
  ss += __shfl_xor(ss, 1, 64);
  ss += __shfl_xor(ss, 2, 64);
  ss += __shfl_xor(ss, 4, 64);
  double nrm = sqrt(ss);
  uint16_t o[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = nrm > 0.0 ? d2bf((double)bf2f(v[i]) / nrm) : (uint16_t)0;
  uint16_t *dst = Qh + row * D + sub * PER;
#pragma unroll
  for (int i = 0; i < PER; i += 8) *(u32x4_t *)&dst[i] = *(const u32x4_t *)&o[i];
  if (sub == 0) qn[row] = (float)nrm;
}

// ---------------------------------------------------------------------------
// Centre operands for the distance GEMM: hi = bf16(c), lo = bf16(c - hi),
// and ||c||^2 (fp64 sum, stored fp32).  One wave per centre.
// at_coff: operand rows at the centres' global index coff[h] + c instead of c.
template <int D>
__global__ __launch_bounds__(256) void k_cent_prep(KmArgs a, CentOps op, int at_coff) {
  const int h = blockIdx.y;
  const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (c >= a.m[h]) return;
  const float *cr = a.cent + (int64_t)h * a.cent_hs + (int64_t)(a.coff[h] + c) * D;
  const int row = at_coff ? a.coff[h] + c : c;
  uint16_t *hi = op.hi + ((int64_t)h * op.cap + row) * D;
  uint16_t *lo = op.lo + ((int64_t)h * op.cap + row) * D;
  double ss = 0.0;
  for (int dd = lane; dd < D; dd += 64) {
    float v = cr[dd];
    uint16_t bh = f2bf(v);
    hi[dd] = bh;
    lo[dd] = f2bf(v - bf2f(bh));
    ss += (double)v * (double)v;
  }
  ss = wave_sum(ss);
  if (lane == 0) op.norm[(int64_t)h * op.cap + row] = (float)ss;
}

// ---------------------------------------------------------------------------
// Nearest centre of every point: argmin_c ||c||^2 - 2 x.c, taken as
// argmax_c x.c - ||c||^2 / 2 on bf16 MFMA (16x16x32, fp32 accumulation that
// starts at -||c||^2 / 2; x.c = x.hi + x.lo), so the products need no
// separate epilogue arithmetic.  A block holds 256 points (4 waves x 64);
// centre operands stream through LDS in chunks of 64.  Ties go to the lower
// centre index; padding centres carry -inf and never win.
template <int D>
__global__ __launch_bounds__(256) void k_assign(KmArgs a, CentOps op, int *__restrict__ labels,
                                                int64_t lab_hs, int *__restrict__ chg) {
  constexpr int KS = D / 32;   // k-steps of 32 dims
  constexpr int CH = 64;       // centres per LDS chunk
  constexpr int LDSROW = D + 8;  // padded row (bf16 elements)
  const int h = blockIdx.y;
  const int n = a.n[h], m = a.m[h];
  const int base = blockIdx.x * 256;
  if (n <= 0 || m <= 0 || base >= n) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, g = lane >> 4;

  __shared__ uint16_t s_hi[CH * LDSROW];
  __shared__ uint16_t s_lo[CH * LDSROW];
  __shared__ float s_norm[CH];

  const uint16_t *X = a.X + (int64_t)h * a.x_hs;
  const int *idx = a.idx ? a.idx + (int64_t)h * a.idx_hs : nullptr;

  // A fragments: 4 row tiles of 16 points, KS k-steps, 8 bf16 each.
  bf16x8_t af[4][KS];
  const int wbase = base + wave * 64;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    int i = wbase + rt * 16 + l16;
    if (i < n) {
      int64_t row = idx ? (int64_t)idx[i] : (int64_t)i;
      const uint16_t *xr = X + row * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) af[rt][ks] = *(const bf16x8_t *)&xr[ks * 32 + g * 8];
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) af[rt][ks] = (bf16x8_t){};
    }
  }

  float best[4][4];
  int bidx[4][4];
  int old[4][4];  // labels already in place for the points this lane writes (when counting changes)
  bool any_change = false;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      best[rt][j] = -__builtin_inff();
      bidx[rt][j] = 0x7fffffff;
      const int i = wbase + rt * 16 + g * 4 + j;
      old[rt][j] = (chg != nullptr && l16 == 0 && i < n) ? labels[(int64_t)h * lab_hs + i] : 0;
    }

  const uint16_t *ghi = op.hi + (int64_t)h * op.cap * D;
  const uint16_t *glo = op.lo + (int64_t)h * op.cap * D;
  const float *gnorm = op.norm + (int64_t)h * op.cap;

  for (int c0 = 0; c0 < m; c0 += CH) {
    const int cn = min(CH, m - c0);
    __syncthreads();
    // stage the chunk: cn rows of D bf16 (hi and lo), 16-byte pieces
    for (int q = threadIdx.x; q < CH * (D / 8); q += 256) {
      int r = q / (D / 8), cc = (q % (D / 8)) * 8;
      u32x4_t vh = {0, 0, 0, 0}, vl = {0, 0, 0, 0};
      if (r < cn) {
        vh = *(const u32x4_t *)&ghi[(int64_t)(c0 + r) * D + cc];
        vl = *(const u32x4_t *)&glo[(int64_t)(c0 + r) * D + cc];
      }
      *(u32x4_t *)&s_hi[r * LDSROW + cc] = vh;
      *(u32x4_t *)&s_lo[r * LDSROW + cc] = vl;
    }
    if (threadIdx.x < CH) s_norm[threadIdx.x] = threadIdx.x < cn ? -0.5f * gnorm[c0 + threadIdx.x] : -__builtin_inff();
    __syncthreads();
#pragma unroll 1
    for (int ct = 0; ct < CH / 16; ++ct) {
      if (ct * 16 >= cn) break;
      // lane holds centre column l16: its accumulators start at -||c||^2 / 2
      const float nh = s_norm[ct * 16 + l16];
      const f32x4_t n4 = {nh, nh, nh, nh};
      f32x4_t acc[4];
      const int crow = ct * 16 + l16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8_t bh = *(const bf16x8_t *)&s_hi[crow * LDSROW + ks * 32 + g * 8];
        bf16x8_t bl = *(const bf16x8_t *)&s_lo[crow * LDSROW + ks * 32 + g * 8];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[rt][ks], bh, ks == 0 ? n4 : acc[rt], 0, 0, 0);
          acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[rt][ks], bl, acc[rt], 0, 0, 0);
        }
      }
      // D layout: lane holds column (centre) l16, rows 4*g + j.
      const int cidx = c0 + ct * 16 + l16;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (acc[rt][j] > best[rt][j]) { best[rt][j] = acc[rt][j]; bidx[rt][j] = cidx; }
    }
  }
  // reduce over the 16 lanes that share g (same rows, different centres)
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float bv = best[rt][j];
      int bi = bidx[rt][j];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        float ov = __shfl_xor(bv, o, 64);
        int oi = __shfl_xor(bi, o, 64);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      int i = wbase + rt * 16 + g * 4 + j;
      const bool wr = l16 == 0 && i < n;
      const int nl = bi == 0x7fffffff ? 0 : bi;
      const bool changed = wr && chg != nullptr && old[rt][j] != nl;
      if (wr) labels[(int64_t)h * lab_hs + i] = nl;
      any_change |= __ballot(changed) != 0;
    }
  if (chg != nullptr && any_change && lane == 0) chg[h] = 1;  // some label of head h changed
}

// Same result as k_assign for m <= ASSIGN_RES_MAX, organised for HBM rate:
// every head's centres stay resident in LDS while a block walks a contiguous
// range of the flattened (head, 64-point sub-tile) list, one sub-tile per
// wave at a time.  Blocks are sized to one per compute unit, so there is no
// per-tile barrier and each wave's point loads overlap the other waves'
// MFMA work.
//
// Merge mode (best != NULL): the launch scores one stage's centres (global
// indices coff[h] + c, operands at op row coff[h] + c) against a running
// nearest centre per point kept in labels / best from earlier launches, and
// replaces it only for a strictly larger value, so that a sequence of such
// launches over the stages in order gives the nearest centre over all of
// them with ties to the lowest global index.  best[h][i] = -inf starts a
// point afresh.

template <int D, int NT>
__global__ __launch_bounds__(NT) void k_assign_res(KmArgs a, CentOps op, int *__restrict__ labels, int64_t lab_hs,
                                                   int BH, int mpmax, int *__restrict__ chg,
                                                   float *__restrict__ best_io) {
  constexpr int KS = D / 32;
  constexpr int LDSROW = D + 8;
  constexpr int NW = NT / 64;
  // LDS sized for the largest centre count of the launch: hi and lo rows, norms
  extern __shared__ __align__(16) uint16_t lds_res[];
  uint16_t *s_hi = lds_res;
  uint16_t *s_lo = lds_res + mpmax * LDSROW;
  float *s_norm = (float *)(lds_res + 2 * mpmax * LDSROW);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, g = lane >> 4;
  // this block's share of the flattened sub-tile list
  int64_t total = 0;
  for (int h = 0; h < BH; ++h) total += (a.n[h] > 0 && a.m[h] > 0) ? (a.n[h] + 63) / 64 : 0;
  const int64_t per = (total + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * per, hi = min(total, lo + per);
  if (lo >= hi) return;
  int64_t hb = 0;  // first flattened sub-tile of head h
  for (int h = 0; h < BH && hb < hi; ++h) {
    const int n = a.n[h], m = a.m[h];
    const int nsub = (n > 0 && m > 0) ? (n + 63) / 64 : 0;
    const int64_t he = hb + nsub;
    const int64_t r0 = max(lo, hb), r1 = min(hi, he);
    if (r0 < r1) {
      const int mp = (m + 15) & ~15;
      const int cbase = best_io ? a.coff[h] : 0;  // merge mode: the stage's first global centre
      const uint16_t *ghi = op.hi + ((int64_t)h * op.cap + cbase) * D;
      const uint16_t *glo = op.lo + ((int64_t)h * op.cap + cbase) * D;
      const float *gnorm = op.norm + (int64_t)h * op.cap + cbase;
      __syncthreads();  // previous head's centres no longer read
      for (int q = threadIdx.x; q < mp * (D / 8); q += NT) {
        const int r = q / (D / 8), cc = (q % (D / 8)) * 8;
        u32x4_t vh = {0, 0, 0, 0}, vl = {0, 0, 0, 0};
        if (r < m) {
          vh = *(const u32x4_t *)&ghi[(int64_t)r * D + cc];
          vl = *(const u32x4_t *)&glo[(int64_t)r * D + cc];
        }
        *(u32x4_t *)&s_hi[r * LDSROW + cc] = vh;
        *(u32x4_t *)&s_lo[r * LDSROW + cc] = vl;
      }
      for (int c = threadIdx.x; c < mp; c += NT) s_norm[c] = c < m ? -0.5f * gnorm[c] : -__builtin_inff();
      __syncthreads();
      const uint16_t *X = a.X + (int64_t)h * a.x_hs;
      const int *idx = a.idx ? a.idx + (int64_t)h * a.idx_hs : nullptr;
      bool any_change = false;
      for (int64_t t = r0 + wave; t < r1; t += NW) {
        const int wbase = (int)(t - hb) * 64;
        bf16x8_t af[4][KS];
        int old[4];  // labels already in place (compared when counting changes)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const int i = wbase + rt * 16 + l16;
          old[rt] = (chg != nullptr && g == 0 && i < n) ? labels[(int64_t)h * lab_hs + i] : 0;
          if (i < n) {
            const int64_t row = idx ? (int64_t)idx[i] : (int64_t)i;
            const uint16_t *xr = X + row * D;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) af[rt][ks] = *(const bf16x8_t *)&xr[ks * 32 + g * 8];
          } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) af[rt][ks] = (bf16x8_t){};
          }
        }
        // centres in the A slot, points in B: lane holds point l16 of each
        // row tile and centres 4g..4g+3 of the centre tile, so the running
        // argmax of x.c - ||c||^2 / 2 is one value per row tile and lane; the
        // accumulators start at the centres' -||c||^2 / 2 (-inf for padding).
        float best[4];
        int bidx[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) { best[rt] = -__builtin_inff(); bidx[rt] = 0x7fffffff; }
        if (best_io) {
          // the running nearest centre of earlier stages (lane group 0 holds it;
          // the other groups start empty, so the reduction below keeps it on ties)
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            const int i = wbase + rt * 16 + l16;
            if (g == 0 && i < n) {
              best[rt] = best_io[(int64_t)h * lab_hs + i];
              bidx[rt] = best[rt] == -__builtin_inff() ? 0x7fffffff : labels[(int64_t)h * lab_hs + i] - cbase;
            }
          }
        }
#pragma unroll 1
        for (int ct = 0; ct < mp / 16; ++ct) {
          const int c0 = ct * 16 + 4 * g;
          const f32x4_t nh = *(const f32x4_t *)&s_norm[c0];
          f32x4_t acc[4];
          const int crow = ct * 16 + l16;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const bf16x8_t bh = *(const bf16x8_t *)&s_hi[crow * LDSROW + ks * 32 + g * 8];
            const bf16x8_t bl = *(const bf16x8_t *)&s_lo[crow * LDSROW + ks * 32 + g * 8];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
              acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bh, af[rt][ks], ks == 0 ? nh : acc[rt], 0, 0, 0);
              acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bl, af[rt][ks], acc[rt], 0, 0, 0);
            }
          }
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (acc[rt][j] > best[rt]) { best[rt] = acc[rt][j]; bidx[rt] = c0 + j; }
        }
        // reduce over the four lane groups that hold the same point
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          float bv = best[rt];
          int bi = bidx[rt];
#pragma unroll
          for (int o = 16; o < 64; o <<= 1) {
            const float ov = __shfl_xor(bv, o, 64);
            const int oi = __shfl_xor(bi, o, 64);
            if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
          }
          const int i = wbase + rt * 16 + l16;
          const bool wr = g == 0 && i < n;
          const int nl = bi == 0x7fffffff ? 0 : bi + cbase;
          const bool changed = wr && chg != nullptr && old[rt] != nl;
          if (wr) labels[(int64_t)h * lab_hs + i] = nl;
          if (wr && best_io) best_io[(int64_t)h * lab_hs + i] = bv;
          any_change |= __ballot(changed) != 0;
        }
      }
      if (chg != nullptr && any_change && lane == 0) chg[h] = 1;  // some label of head h changed
    }
    hb = he;
  }
}

// ---------------------------------------------------------------------------
// Stable counting sort of per-head labels in [0, m): tile histograms, a
// two-level scan (tiles within groups of SORT_GROUP, then groups and labels),
// and an in-order scatter of each tile by one wave.  perm[h][p] = local index
// of the p-th point in label order; seg[h][c] the first position of label c,
// seg[h][c] = n for m <= c <= segcap.
__global__ __launch_bounds__(64) void k_sort_hist(SortArgs s) {
  const int h = blockIdx.y, tile = blockIdx.x;
  const int n = s.n[h], m = s.m[h];
  if (tile == 0 && threadIdx.x == 0 && s.chg_zero != nullptr) {
    // Lloyd loop: no label of head h changed in this assignment, so this
    // update and every later step reproduce the current centres exactly;
    // the head drops out of the loop (later kernels read neff[h] = 0)
    if (s.chg_cur != nullptr && s.chg_cur[h] == 0) s.neff[h] = 0;
    s.chg_zero[h] = 0;
  }
  const int beg = tile * SORT_TILE;
  if (beg >= n || m <= 0) return;
  extern __shared__ int sh_hist[];
  for (int c = threadIdx.x; c < m; c += 64) sh_hist[c] = 0;
  __syncthreads();
  const int *lab = s.labels + (int64_t)h * s.lab_hs;
  const int end = min(n, beg + SORT_TILE);
  for (int i = beg + threadIdx.x; i < end; i += 64) atomicAdd(&sh_hist[lab[i]], 1);
  __syncthreads();
  int *th = s.tile_hist + ((int64_t)h * s.max_tiles + tile) * s.mcap;
  for (int c = threadIdx.x; c < m; c += 64) th[c] = sh_hist[c];
}

// Exclusive scan of each label's counts over the tiles of one group (in
// place); the group's total goes to grp.  One thread per (group, label).
__global__ __launch_bounds__(256) void k_sort_gscan(SortArgs s) {
  const int g = blockIdx.x, h = blockIdx.y;
  const int c = blockIdx.z * 256 + threadIdx.x;
  const int n = s.n[h], m = s.m[h];
  const int nt = (n + SORT_TILE - 1) / SORT_TILE;
  const int t0 = g * SORT_GROUP;
  if (c >= m || t0 >= nt) return;
  const int t1 = min(nt, t0 + SORT_GROUP);
  int *p = s.tile_hist + ((int64_t)h * s.max_tiles + t0) * s.mcap + c;
  int v[SORT_GROUP];
#pragma unroll
  for (int t = 0; t < SORT_GROUP; ++t) v[t] = (t0 + t < t1) ? p[(int64_t)t * s.mcap] : 0;
  int run = 0;
#pragma unroll
  for (int t = 0; t < SORT_GROUP; ++t) {
    if (t0 + t < t1) p[(int64_t)t * s.mcap] = run;
    run += v[t];
  }
  s.grp[((int64_t)h * s.max_groups + g) * s.mcap + c] = run;
}

// Per head: each label's total over the groups, a scan of the label totals,
// then grp is rewritten to the first output position of (group, label).  With
// chunk_off set, the chunk counts of the centre update are scanned beside the
// label totals.
__global__ __launch_bounds__(1024) void k_sort_scan(SortArgs s) {
  const int h = blockIdx.x;
  const int n = s.n[h], m = s.m[h];
  int *seg = s.seg + (int64_t)h * s.seg_hs;
  const int nt = (n + SORT_TILE - 1) / SORT_TILE;
  const int ng = (nt + SORT_GROUP - 1) / SORT_GROUP;
  int *grp = s.grp + (int64_t)h * s.max_groups * s.mcap;
  __shared__ int2 part[16];  // wave totals
  const int per = (m + 1023) / 1024;
  const int cb = min(m, (int)threadIdx.x * per), ce = min(m, cb + per);
  // a label's group counts are read SCAN_BATCH at a time, so the loads of a
  // batch are in flight together
  constexpr int SCAN_BATCH = 8;
  int tot_local = 0, chunks_local = 0;
  for (int c = cb; c < ce; ++c) {
    int run = 0;
    for (int g0 = 0; g0 < ng; g0 += SCAN_BATCH) {
      int v[SCAN_BATCH];
#pragma unroll
      for (int j = 0; j < SCAN_BATCH; ++j) v[j] = g0 + j < ng ? grp[(int64_t)(g0 + j) * s.mcap + c] : 0;
#pragma unroll
      for (int j = 0; j < SCAN_BATCH; ++j) run += v[j];
    }
    seg[c] = run;  // count for now
    tot_local += run;
    chunks_local += (run + UPD_CHUNK - 1) / UPD_CHUNK;
  }
  // exclusive scan of both counts over the threads: wave scans, then the
  // wave totals through LDS (integer sums, so the order is immaterial)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int ix = tot_local, iy = chunks_local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int x = __shfl_up(ix, o, 64), y = __shfl_up(iy, o, 64);
    if (lane >= o) { ix += x; iy += y; }
  }
  if (lane == 63) part[wave] = make_int2(ix, iy);
  __syncthreads();
  int ox = 0, oy = 0, ty = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const int2 t = part[w];
    if (w < wave) { ox += t.x; oy += t.y; }
    ty += t.y;
  }
  int run = ox + ix - tot_local;
  int crun = oy + iy - chunks_local;
  int *co = s.chunk_off ? s.chunk_off + (int64_t)h * s.co_hs : nullptr;
  for (int c = cb; c < ce; ++c) {
    const int v = seg[c];
    seg[c] = run;
    int pos = run;  // first output position of (group, label c)
    for (int g0 = 0; g0 < ng; g0 += SCAN_BATCH) {
      int w[SCAN_BATCH];
#pragma unroll
      for (int j = 0; j < SCAN_BATCH; ++j) w[j] = g0 + j < ng ? grp[(int64_t)(g0 + j) * s.mcap + c] : 0;
#pragma unroll
      for (int j = 0; j < SCAN_BATCH; ++j)
        if (g0 + j < ng) {
          grp[(int64_t)(g0 + j) * s.mcap + c] = pos;
          pos += w[j];
        }
    }
    run += v;
    if (co) {
      co[c] = crun;
      crun += (v + UPD_CHUNK - 1) / UPD_CHUNK;
    }
  }
  if (co && threadIdx.x == 1023) co[max(m, 0)] = ty;
  for (int c = m + threadIdx.x; c <= s.segcap; c += 1024) seg[c] = max(n, 0);
  if (n <= 0)
    for (int c = threadIdx.x; c <= s.segcap; c += 1024) seg[c] = 0;
}

// One wave per tile.  Lanes holding the same label are found with one
// ballot per label bit; each lane's rank among them is a popcount, and the
// lowest such lane advances the label's cursor.  A wave's LDS operations
// complete in program order, so no barrier is needed between batches.
__global__ __launch_bounds__(64) void k_sort_scatter(SortArgs s) {
  const int h = blockIdx.y, tile = blockIdx.x;
  const int n = s.n[h], m = s.m[h];
  const int beg = tile * SORT_TILE;
  if (beg >= n || m <= 0) return;
  extern __shared__ int sh_base[];
  const int *gb = s.grp + ((int64_t)h * s.max_groups + tile / SORT_GROUP) * s.mcap;
  const int *th = s.tile_hist + ((int64_t)h * s.max_tiles + tile) * s.mcap;
  for (int c = threadIdx.x; c < m; c += 64) sh_base[c] = gb[c] + th[c];
  __syncthreads();
  const int *lab = s.labels + (int64_t)h * s.lab_hs;
  int *perm = s.perm + (int64_t)h * s.perm_hs;
  const int end = min(n, beg + SORT_TILE);
  const int lane = threadIdx.x;
  const int nb = m > 1 ? 32 - __builtin_clz((unsigned)(m - 1)) : 0;
  for (int i0 = beg; i0 < end; i0 += 64) {
    const int i = i0 + lane;
    const bool valid = i < end;
    const int lb = valid ? lab[i] : 0;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < nb; ++b) {
      const bool bit = (lb >> b) & 1;
      const uint64_t bb = __ballot(bit);
      same &= bit ? bb : ~bb;
    }
    const uint64_t below = same & ((1ull << lane) - 1ull);
    if (valid) {
      const int basev = sh_base[lb];
      perm[basev + __popcll(below)] = i;
      if (below == 0) sh_base[lb] = basev + __popcll(same);
    }
  }
}

// ---------------------------------------------------------------------------
// The same stable counting sort for heads of at most SORT_SMALL_MAX points and
// SORT_SMALL_M labels in one launch: one 1024-thread block per head builds the
// label histogram in LDS, scans it, and scatters the points in chunks of 1024
// (ranks among equal labels from one ballot per label bit within each wave,
// then the earlier waves' counts of the chunk).  Same outputs as launch_sort,
// including the Lloyd loop's fixed-point bookkeeping and the update's chunk
// offsets.
__global__ __launch_bounds__(1024) void k_sort_small(SortArgs s) {
  constexpr int NT = 1024, NWV = NT / 64;
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = s.n[h], m = s.m[h];
  __shared__ int hist[SORT_SMALL_M + 1];
  __shared__ int wcnt[NWV][SORT_SMALL_M];
  __shared__ int cur[SORT_SMALL_M];
  __shared__ int conv;
  if (tid == 0) {
    conv = 0;
    if (s.chg_zero != nullptr) {
      // Lloyd loop: a head whose assignment changed no label leaves the loop
      if (s.chg_cur != nullptr && s.chg_cur[h] == 0) { s.neff[h] = 0; conv = 1; }
      s.chg_zero[h] = 0;
    }
  }
  __syncthreads();
  if (conv || n <= 0 || m <= 0) {
    if (!conv) {
      int *seg = s.seg + (int64_t)h * s.seg_hs;
      for (int c = tid; c <= s.segcap; c += NT) seg[c] = 0;
    }
    return;
  }
  const int *lab = s.labels + (int64_t)h * s.lab_hs;
  int *perm = s.perm + (int64_t)h * s.perm_hs;
  int *seg = s.seg + (int64_t)h * s.seg_hs;
  for (int c = tid; c < m; c += NT) hist[c] = 0;
  for (int q = tid; q < NWV * SORT_SMALL_M; q += NT) (&wcnt[0][0])[q] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += NT) atomicAdd(&hist[lab[i]], 1);
  __syncthreads();
  if (wave == 0) {
    // exclusive scan of the m counts (and of the update's chunk counts)
    int run = 0, crun = 0;
    int *co = s.chunk_off ? s.chunk_off + (int64_t)h * s.co_hs : nullptr;
    for (int c0 = 0; c0 < m; c0 += 64) {
      const int c = c0 + lane;
      const int v = c < m ? hist[c] : 0;
      const int ck = (v + UPD_CHUNK - 1) / UPD_CHUNK;
      int iv = v, ic = ck;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int a = __shfl_up(iv, o, 64), b = __shfl_up(ic, o, 64);
        if (lane >= o) { iv += a; ic += b; }
      }
      if (c < m) {
        cur[c] = run + iv - v;
        seg[c] = run + iv - v;
        if (co) co[c] = crun + ic - ck;
      }
      run += __shfl(iv, 63, 64);
      crun += __shfl(ic, 63, 64);
    }
    for (int c = m + lane; c <= s.segcap; c += 64) seg[c] = n;
    if (co && lane == 0) co[m] = crun;
  }
  __syncthreads();
  const int nb = m > 1 ? 32 - __builtin_clz((unsigned)(m - 1)) : 0;
  for (int c0 = 0; c0 < n; c0 += NT) {
    const int i = c0 + tid;
    const bool valid = i < n;
    const int lb = valid ? lab[i] : 0;
    uint64_t same = __ballot(valid);
    for (int bt = 0; bt < nb; ++bt) {
      const bool bit = (lb >> bt) & 1;
      const uint64_t bb = __ballot(bit);
      same &= bit ? bb : ~bb;
    }
    const uint64_t below = same & ((1ull << lane) - 1ull);
    if (valid && below == 0) wcnt[wave][lb] = __popcll(same);
    __syncthreads();
    if (valid) {
      int base = cur[lb];
      for (int w = 0; w < wave; ++w) base += wcnt[w][lb];
      perm[base + __popcll(below)] = i;
    }
    __syncthreads();
    for (int c = tid; c < m; c += NT) {
      int t = 0;
#pragma unroll
      for (int w = 0; w < NWV; ++w) {
        t += wcnt[w][c];
        wcnt[w][c] = 0;
      }
      cur[c] += t;
    }
    __syncthreads();
  }
}

// Lloyd update of heads sorted by k_sort_small: one block per (cluster,
// head) sums its members in counting-sort order (fp64, 16 lanes per row,
// fixed order), divides, and writes the centre's GEMM operands.  An empty
// cluster keeps its centre.
template <int D>
__global__ __launch_bounds__(256) void k_update_small(KmArgs a, SortArgs s, CentOps op) {
  constexpr int PL = D / 16;
  typedef uint32_t pw_t __attribute__((ext_vector_type(PL / 2)));
  const int h = blockIdx.y, c = blockIdx.x;
  if (c >= a.m[h] || a.n[h] <= 0) return;
  const int *seg = s.seg + (int64_t)h * s.seg_hs;
  const int *perm = s.perm + (int64_t)h * s.perm_hs;
  const int beg = seg[c], end = seg[c + 1];
  const uint16_t *X = a.X + (int64_t)h * a.x_hs;
  const int *idx = a.idx ? a.idx + (int64_t)h * a.idx_hs : nullptr;
  const int grp = threadIdx.x >> 4, sub = threadIdx.x & 15;
  double acc[PL];
#pragma unroll
  for (int k = 0; k < PL; ++k) acc[k] = 0.0;
  for (int p0 = beg + grp; p0 < end; p0 += 64) {
    int li[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) li[j] = (p0 + 16 * j < end) ? perm[p0 + 16 * j] : -1;
    pw_t xv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (li[j] >= 0) {
        const int64_t row = idx ? (int64_t)idx[li[j]] : (int64_t)li[j];
        xv[j] = *(const pw_t *)(X + row * D + sub * PL);
      } else {
        xv[j] = (pw_t){};
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (li[j] < 0) break;
#pragma unroll
      for (int k = 0; k < PL; ++k) {
        const uint32_t w = xv[j][k >> 1];
        acc[k] += (double)bf2f((uint16_t)((k & 1) ? (w >> 16) : (w & 0xFFFFu)));
      }
    }
  }
  __shared__ double sh[16][D];
  __shared__ double red[4];
#pragma unroll
  for (int k = 0; k < PL; ++k) sh[grp][sub * PL + k] = acc[k];
  __syncthreads();
  const int cnt = end - beg;
  float *cr = a.cent + (int64_t)h * a.cent_hs + (int64_t)(a.coff[h] + c) * D;
  double ss = 0.0;
  for (int dd = threadIdx.x; dd < D; dd += 256) {
    float v;
    if (cnt > 0) {
      double t = 0.0;
#pragma unroll
      for (int g = 0; g < 16; ++g) t += sh[g][dd];
      v = (float)(t / (double)cnt);
      cr[dd] = v;
    } else {
      v = cr[dd];
    }
    const uint16_t bh = f2bf(v);
    op.hi[((int64_t)h * op.cap + c) * D + dd] = bh;
    op.lo[((int64_t)h * op.cap + c) * D + dd] = f2bf(v - bf2f(bh));
    ss += (double)v * (double)v;
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) op.norm[(int64_t)h * op.cap + c] = (float)(red[0] + red[1] + red[2] + red[3]);
}

// ---------------------------------------------------------------------------
// Lloyd update as a chunked segmented reduction over the counting-sort order:
// every cluster is cut into chunks of UPD_CHUNK members (their offsets come
// from the sort's label scan); one block sums one
// chunk in fp64 (16 lanes per row, fixed order), a second kernel adds a
// cluster's chunk sums in order and divides.  An empty cluster keeps its
// centre.  The new centre's GEMM operands are written in the same pass.
template <int D>
__global__ __launch_bounds__(256) void k_update_partial(KmArgs a, SortArgs s, const int *__restrict__ chunk_off,
                                                        int64_t co_hs, double *__restrict__ partial, int64_t part_hs) {
  constexpr int PL = D / 16;
  const int h = blockIdx.y, item = blockIdx.x;
  const int m = a.m[h];
  if (m <= 0 || a.n[h] <= 0) return;
  const int *co = chunk_off + (int64_t)h * co_hs;
  if (item >= co[m]) return;
  int lo = 0, hi = m;  // co[lo] <= item < co[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (co[mid] <= item) lo = mid; else hi = mid;
  }
  const int c = lo;
  const int *seg = s.seg + (int64_t)h * s.seg_hs;
  const int *perm = s.perm + (int64_t)h * s.perm_hs;
  const int beg = seg[c] + (item - co[c]) * UPD_CHUNK;
  const int end = min(seg[c + 1], beg + UPD_CHUNK);
  const uint16_t *X = a.X + (int64_t)h * a.x_hs;
  const int *idx = a.idx ? a.idx + (int64_t)h * a.idx_hs : nullptr;
  const int grp = threadIdx.x >> 4, sub = threadIdx.x & 15;
  double acc[PL];
#pragma unroll
  for (int k = 0; k < PL; ++k) acc[k] = 0.0;
  typedef uint32_t pw_t __attribute__((ext_vector_type(PL / 2)));
  // four rows per lane in flight; rows are still added in member order
  for (int p0 = beg + grp; p0 < end; p0 += 64) {
    int li[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) li[j] = (p0 + 16 * j < end) ? perm[p0 + 16 * j] : -1;
    pw_t xv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (li[j] >= 0) {
        const int64_t row = idx ? (int64_t)idx[li[j]] : (int64_t)li[j];
        xv[j] = *(const pw_t *)(X + row * D + sub * PL);
      } else {
        xv[j] = (pw_t){};
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (li[j] < 0) break;
#pragma unroll
      for (int k = 0; k < PL; ++k) {
        const uint32_t w = xv[j][k >> 1];
        acc[k] += (double)bf2f((uint16_t)((k & 1) ? (w >> 16) : (w & 0xFFFFu)));
      }
    }
  }
  __shared__ double sh[16][D];
#pragma unroll
  for (int k = 0; k < PL; ++k) sh[grp][sub * PL + k] = acc[k];
  __syncthreads();
  if (threadIdx.x < D) {
    double t = 0.0;
#pragma unroll
    for (int gg = 0; gg < 16; ++gg) t += sh[gg][threadIdx.x];
    partial[(int64_t)h * part_hs + (int64_t)item * D + threadIdx.x] = t;
  }
}

template <int D>
__global__ __launch_bounds__(128) void k_update_final(KmArgs a, SortArgs s, const int *__restrict__ chunk_off,
                                                      int64_t co_hs, const double *__restrict__ partial,
                                                      int64_t part_hs, CentOps op) {
  const int h = blockIdx.y, c = blockIdx.x;
  if (c >= a.m[h] || a.n[h] <= 0) return;
  const int *seg = s.seg + (int64_t)h * s.seg_hs;
  const int *co = chunk_off + (int64_t)h * co_hs;
  const int cnt = seg[c + 1] - seg[c];
  float *cr = a.cent + (int64_t)h * a.cent_hs + (int64_t)(a.coff[h] + c) * D;
  __shared__ double red[2];
  double ss = 0.0;
  for (int dd = threadIdx.x; dd < D; dd += 128) {
    float v;
    if (cnt > 0) {
      double t = 0.0;
      for (int it = co[c]; it < co[c + 1]; ++it) t += partial[(int64_t)h * part_hs + (int64_t)it * D + dd];
      v = (float)(t / (double)cnt);
      cr[dd] = v;
    } else {
      v = cr[dd];
    }
    const uint16_t bh = f2bf(v);
    op.hi[((int64_t)h * op.cap + c) * D + dd] = bh;
    op.lo[((int64_t)h * op.cap + c) * D + dd] = f2bf(v - bf2f(bh));
    ss += (double)v * (double)v;
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) op.norm[(int64_t)h * op.cap + c] = (float)(red[0] + red[1]);
}

// ---------------------------------------------------------------------------
// Distance of each point of a stage to its own centre, ||x - c(x)|| (fp64
// accumulation, stored fp32).  16 lanes per point; a block takes 16 * SD_PTS
// points and issues the index, label, row and centre loads of all of them
// before the arithmetic, so the two levels of dependent loads overlap.
constexpr int SD_PTS = 4;

template <int D>
__global__ __launch_bounds__(256) void k_stage_dist(KmArgs a, const int *__restrict__ labels, int64_t lab_hs,
                                                    float *__restrict__ dist, int64_t dist_hs) {
  constexpr int PL = D / 16;
  typedef uint32_t pw_t __attribute__((ext_vector_type(PL / 2)));
  typedef float pf_t __attribute__((ext_vector_type(PL)));
  const int h = blockIdx.y;
  const int n = a.n[h];
  const int i0 = blockIdx.x * (16 * SD_PTS) + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  if (blockIdx.x * (16 * SD_PTS) >= n || a.m[h] <= 0) return;
  const uint16_t *X = a.X + (int64_t)h * a.x_hs;
  const float *C = a.cent + (int64_t)h * a.cent_hs + (int64_t)a.coff[h] * D + sub * PL;
  int64_t row[SD_PTS];
  int c[SD_PTS];
#pragma unroll
  for (int j = 0; j < SD_PTS; ++j) {
    const int i = i0 + 16 * j;
    row[j] = i < n ? (a.idx ? (int64_t)a.idx[(int64_t)h * a.idx_hs + i] : (int64_t)i) : 0;
    c[j] = i < n ? labels[(int64_t)h * lab_hs + i] : 0;
  }
  pw_t xv[SD_PTS];
  pf_t cv[SD_PTS];
#pragma unroll
  for (int j = 0; j < SD_PTS; ++j) {
    if (i0 + 16 * j < n) {
      xv[j] = *(const pw_t *)(X + row[j] * D + sub * PL);
      cv[j] = *(const pf_t *)(C + (int64_t)c[j] * D);
    }
  }
#pragma unroll
  for (int j = 0; j < SD_PTS; ++j) {
    const int i = i0 + 16 * j;
    double acc = 0.0;
    if (i < n) {
#pragma unroll
      for (int q = 0; q < PL; ++q) {
        const uint32_t w = xv[j][q >> 1];
        const double df = (double)bf2f((uint16_t)((q & 1) ? (w >> 16) : (w & 0xFFFFu))) - (double)cv[j][q];
        acc = fma(df, df, acc);
      }
    }
    acc += __shfl_xor(acc, 1, 64);
    acc += __shfl_xor(acc, 2, 64);
    acc += __shfl_xor(acc, 4, 64);
    acc += __shfl_xor(acc, 8, 64);
    if (i < n && sub == 0) dist[(int64_t)h * dist_hs + i] = (float)sqrt(acc);
  }
}

// ---------------------------------------------------------------------------
// tau of the first stage.  MEAN_X / ABS / INF directly; PCTL by a radix
// select over the fp32 bit patterns (non-negative values order as integers).
__global__ __launch_bounds__(1024) void k_tau_direct(const float *__restrict__ dist, int64_t dist_hs,
                                                     const int *__restrict__ n_arr, int rule, float param,
                                                     float *__restrict__ tau) {
  const int h = blockIdx.x;
  const int n = n_arr[h];
  if (rule == TAU_RULE_ABS) { if (threadIdx.x == 0) tau[h] = param; return; }
  if (rule == TAU_RULE_INF) { if (threadIdx.x == 0) tau[h] = __builtin_inff(); return; }
  // MEAN_X: fixed-order fp64 sum
  __shared__ double part[1024];
  double loc = 0.0;
  const float *d = dist + (int64_t)h * dist_hs;
  for (int i = threadIdx.x; i < n; i += 1024) loc += (double)d[i];
  part[threadIdx.x] = loc;
  __syncthreads();
  for (int off = 512; off > 0; off >>= 1) {
    if (threadIdx.x < off) part[threadIdx.x] += part[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) tau[h] = n > 0 ? (float)((double)param * (part[0] / (double)n)) : 0.f;
}

// radix-select state per head: {prefix bits, remaining rank (1-based)}
__global__ __launch_bounds__(256) void k_radix_init(const int *__restrict__ n_arr, float param,
                                                    uint32_t *__restrict__ state, uint32_t *__restrict__ ghist) {
  const int h = blockIdx.x;
  for (int b = threadIdx.x; b < 256; b += 256) ghist[h * 256 + b] = 0;
  if (threadIdx.x == 0) {
    int n = n_arr[h];
    double r = ceil((double)param * (double)n);
    int rk = (int)r;
    rk = rk < 1 ? 1 : (rk > n ? n : rk);
    state[h * 2 + 0] = 0;
    state[h * 2 + 1] = (uint32_t)rk;
  }
}

__global__ __launch_bounds__(256) void k_radix_hist(const float *__restrict__ dist, int64_t dist_hs,
                                                    const int *__restrict__ n_arr, const uint32_t *__restrict__ state,
                                                    uint32_t *__restrict__ ghist, int shift) {
  const int h = blockIdx.y;
  const int n = n_arr[h];
  __shared__ uint32_t hs[256];
  hs[threadIdx.x] = 0;
  __syncthreads();
  const uint32_t prefix = state[h * 2];
  const uint32_t hmask = shift == 24 ? 0u : (0xFFFFFFFFu << (shift + 8));
  const float *d = dist + (int64_t)h * dist_hs;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) {
    uint32_t b = __float_as_uint(d[i]);
    if ((b & hmask) == prefix) atomicAdd(&hs[(b >> shift) & 255u], 1u);
  }
  __syncthreads();
  if (hs[threadIdx.x]) atomicAdd(&ghist[h * 256 + threadIdx.x], hs[threadIdx.x]);
}

__global__ __launch_bounds__(64) void k_radix_pick(uint32_t *__restrict__ state, uint32_t *__restrict__ ghist,
                                                   int shift, float *__restrict__ tau) {
  const int h = blockIdx.x;
  if (threadIdx.x == 0) {
    uint32_t rk = state[h * 2 + 1];
    uint32_t run = 0;
    int bin = 255;
    for (int b = 0; b < 256; ++b) {
      uint32_t v = ghist[h * 256 + b];
      if (run + v >= rk) { bin = b; break; }
      run += v;
    }
    state[h * 2 + 0] |= ((uint32_t)bin << shift);
    state[h * 2 + 1] = rk - run;
    if (shift == 0) tau[h] = __uint_as_float(state[h * 2 + 0]);
  }
  __syncthreads();
  for (int b = threadIdx.x; b < 256; b += 64) ghist[h * 256 + b] = 0;
}

// keep flag for compaction: label 0 = stays in U (d >= tau), 1 = removed.
__global__ __launch_bounds__(256) void k_flag_removed(const float *__restrict__ dist, int64_t dist_hs,
                                                      const int *__restrict__ n_arr, const float *__restrict__ tau,
                                                      int *__restrict__ flag, int64_t flag_hs) {
  const int h = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n_arr[h]) return;
  flag[(int64_t)h * flag_hs + i] = dist[(int64_t)h * dist_hs + i] < tau[h] ? 1 : 0;
}

// new U list = old U entries that stayed, in order: out[p] = idx[perm[p]]
// for p < seg[1]; also the new size.
__global__ __launch_bounds__(256) void k_compact_gather(const int *__restrict__ idx_old, int64_t idx_hs,
                                                        const int *__restrict__ perm, int64_t perm_hs,
                                                        const int *__restrict__ seg, int64_t seg_hs,
                                                        int *__restrict__ idx_new, int *__restrict__ n_new) {
  const int h = blockIdx.y;
  const int keep = seg[(int64_t)h * seg_hs + 1];
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (blockIdx.x == 0 && threadIdx.x == 0) n_new[h] = keep;
  if (p >= keep) return;
  int li = perm[(int64_t)h * perm_hs + p];
  idx_new[(int64_t)h * idx_hs + p] = idx_old ? idx_old[(int64_t)h * idx_hs + li] : li;
}

// ---------------------------------------------------------------------------
// Statistics of the final key clusters: count, fp64 means of K and V,
// per-dimension max / min of K (exact bf16), and each cluster's share of
// sum ||k - c(k)||^2 (fp64).  Clusters are cut into chunks of KST_CHUNK
// members so that a large cluster spreads over many blocks: a cluster of one
// chunk is finished by its block, a larger one leaves per-chunk partials that
// a second kernel combines in chunk order (deterministic).
//
// Per head, from the segments: co[c] = chunks of clusters < c, and
// po[c] = chunks of the multi-chunk clusters < c (their partial slots).  A
// cluster of k >= 2 chunks holds more than (k - 1) KST_CHUNK >= k KST_CHUNK / 2
// members, so the slots number fewer than 2 L / KST_CHUNK per head.
__global__ __launch_bounds__(1024) void k_kst_chunks(KStatsArgs s) {
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ncl = s.ncl[h];
  const int *seg = s.seg + (int64_t)h * (s.ncap + 1);
  int *co = s.co + (int64_t)h * (s.ncap + 1);
  int *po = s.po + (int64_t)h * (s.ncap + 1);
  const int per = (ncl + 1023) / 1024;
  const int c0 = min(ncl, tid * per), c1 = min(ncl, c0 + per);
  int a = 0, b = 0;
  for (int c = c0; c < c1; ++c) {
    const int k = (seg[c + 1] - seg[c] + KST_CHUNK - 1) / KST_CHUNK;
    a += k;
    b += k >= 2 ? k : 0;
  }
  // exclusive block scan of (a, b)
  int ia = a, ib = b;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int ya = __shfl_up(ia, o, 64), yb = __shfl_up(ib, o, 64);
    if (lane >= o) { ia += ya; ib += yb; }
  }
  __shared__ int wa[16], wb[16];
  if (lane == 63) { wa[wave] = ia; wb[wave] = ib; }
  __syncthreads();
  int oa = 0, ob = 0;
  for (int w = 0; w < wave; ++w) { oa += wa[w]; ob += wb[w]; }
  int ra = oa + ia - a, rb = ob + ib - b;
  for (int c = c0; c < c1; ++c) {
    const int k = (seg[c + 1] - seg[c] + KST_CHUNK - 1) / KST_CHUNK;
    co[c] = ra;
    po[c] = rb;
    ra += k;
    rb += k >= 2 ? k : 0;
  }
  if (tid == 1023) { co[ncl] = ra; po[ncl] = rb; }
}

template <int D>
__global__ __launch_bounds__(64) void k_kstats_part(KStatsArgs s) {
  // one wave per chunk: 4 row groups of 16 lanes (PL dims each), four member
  // rows per group in flight, the groups combined with shuffles
  constexpr int PL = D / 16;  // dims per lane, 16 lanes per row
  typedef uint32_t pw_t __attribute__((ext_vector_type(PL / 2)));
  const int h = blockIdx.y, item = blockIdx.x;
  const int ncl = s.ncl[h];
  const int *co = s.co + (int64_t)h * (s.ncap + 1);
  if (ncl <= 0 || item >= co[ncl]) return;
  int lo = 0, hi = ncl;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (co[mid] <= item) lo = mid; else hi = mid;
  }
  const int c = lo, j = item - co[c], nch = co[c + 1] - co[c];
  const int64_t cb = ((int64_t)h * s.ncap + c);
  const int grp = threadIdx.x >> 4, sub = threadIdx.x & 15;
  const int *seg = s.seg + (int64_t)h * (s.ncap + 1);
  const int *perm = s.perm + (int64_t)h * s.L;
  const int beg = seg[c] + j * KST_CHUNK, end = min(seg[c + 1], beg + KST_CHUNK);
  const uint16_t *K = s.K + (int64_t)h * s.L * D;
  const bool wv = s.V != nullptr;  // value means wanted
  const uint16_t *V = wv ? s.V + (int64_t)h * s.L * D : nullptr;
  const float *cent = s.cent + cb * D;
  double sk[PL], sv[PL], se = 0.0;
  float mx[PL], mn[PL], cc[PL];
#pragma unroll
  for (int k = 0; k < PL; ++k) {
    sk[k] = 0.0; sv[k] = 0.0; mx[k] = -__builtin_inff(); mn[k] = __builtin_inff();
    cc[k] = cent[sub * PL + k];
  }
  for (int p0 = beg + grp; p0 < end; p0 += 16) {
    int64_t row[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) row[jj] = (p0 + 4 * jj < end) ? (int64_t)perm[p0 + 4 * jj] : -1;
    pw_t kw[4], vw[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int64_t rr = row[jj] >= 0 ? row[jj] : row[0];
      kw[jj] = *(const pw_t *)(K + rr * D + sub * PL);
      if (wv) vw[jj] = *(const pw_t *)(V + rr * D + sub * PL);
      else vw[jj] = (pw_t){};
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      if (row[jj] < 0) break;
#pragma unroll
      for (int k = 0; k < PL; ++k) {
        const uint32_t a1 = kw[jj][k >> 1], b1 = vw[jj][k >> 1];
        const float kv = bf2f((uint16_t)((k & 1) ? (a1 >> 16) : (a1 & 0xFFFFu)));
        const float vv = bf2f((uint16_t)((k & 1) ? (b1 >> 16) : (b1 & 0xFFFFu)));
        sk[k] += (double)kv;
        sv[k] += (double)vv;
        mx[k] = fmaxf(mx[k], kv);
        mn[k] = fminf(mn[k], kv);
        const double df = (double)kv - (double)cc[k];
        se = fma(df, df, se);
      }
    }
  }
  // the four row groups (lanes sub, sub + 16, sub + 32, sub + 48)
#pragma unroll
  for (int o = 16; o < 64; o <<= 1) {
#pragma unroll
    for (int k = 0; k < PL; ++k) {
      sk[k] += __shfl_xor(sk[k], o, 64);
      sv[k] += __shfl_xor(sv[k], o, 64);
      mx[k] = fmaxf(mx[k], __shfl_xor(mx[k], o, 64));
      mn[k] = fminf(mn[k], __shfl_xor(mn[k], o, 64));
    }
  }
  se = wave_sum(se);
  // one chunk: the cluster's statistics; more: this chunk's partial slot
  const int64_t slot = (int64_t)h * s.pslots + s.po[(int64_t)h * (s.ncap + 1) + c] + j;
  const int cnt = seg[c + 1] - seg[c];
  if (grp == 0) {
#pragma unroll
    for (int k = 0; k < PL; ++k) {
      const int dd = sub * PL + k;
      if (nch == 1) {
        s.kmean[cb * D + dd] = (float)(sk[k] / cnt);
        if (wv) s.vmean[cb * D + dd] = (float)(sv[k] / cnt);
        s.kmax[cb * D + dd] = (uint16_t)(__float_as_uint(mx[k]) >> 16);
        s.kmin[cb * D + dd] = (uint16_t)(__float_as_uint(mn[k]) >> 16);
      } else {
        s.psk[slot * D + dd] = sk[k];
        if (wv) s.psv[slot * D + dd] = sv[k];
        s.pmx[slot * D + dd] = mx[k];
        s.pmn[slot * D + dd] = mn[k];
      }
    }
  }
  if (threadIdx.x == 0) {
    if (nch == 1) s.msepart[cb] = se;
    else s.pse[slot] = se;
  }
}

// Clusters of several chunks, empty clusters and unused slots up to ncap.
template <int D>
__global__ __launch_bounds__(128) void k_kstats_fin(KStatsArgs s) {
  const int h = blockIdx.y, c = blockIdx.x;
  const int ncl = s.ncl[h];
  const int64_t cb = ((int64_t)h * s.ncap + c);
  const int *seg = s.seg + (int64_t)h * (s.ncap + 1);
  const int cnt = c < ncl ? seg[c + 1] - seg[c] : 0;
  const int *co = s.co + (int64_t)h * (s.ncap + 1);
  const int nch = c < ncl ? co[c + 1] - co[c] : 0;
  if (nch == 1) return;  // finished by its chunk
  if (nch == 0) {
    for (int dd = threadIdx.x; dd < D; dd += 128) {
      s.kmax[cb * D + dd] = 0; s.kmin[cb * D + dd] = 0;
      s.kmean[cb * D + dd] = 0.f;
      if (s.V) s.vmean[cb * D + dd] = 0.f;
    }
    if (threadIdx.x == 0) s.msepart[cb] = 0.0;
    return;
  }
  const int64_t s0 = (int64_t)h * s.pslots + s.po[(int64_t)h * (s.ncap + 1) + c];
  for (int dd = threadIdx.x; dd < D; dd += 128) {
    double a = 0.0, b = 0.0;
    float x = -__builtin_inff(), y = __builtin_inff();
    for (int q = 0; q < nch; ++q) {
      a += s.psk[(s0 + q) * D + dd];
      if (s.V) b += s.psv[(s0 + q) * D + dd];
      x = fmaxf(x, s.pmx[(s0 + q) * D + dd]);
      y = fminf(y, s.pmn[(s0 + q) * D + dd]);
    }
    s.kmean[cb * D + dd] = (float)(a / cnt);
    if (s.V) s.vmean[cb * D + dd] = (float)(b / cnt);
    s.kmax[cb * D + dd] = (uint16_t)(__float_as_uint(x) >> 16);
    s.kmin[cb * D + dd] = (uint16_t)(__float_as_uint(y) >> 16);
  }
  if (threadIdx.x == 0) {
    double e = 0.0;
    for (int q = 0; q < nch; ++q) e += s.pse[s0 + q];
    s.msepart[cb] = e;
  }
}

__global__ __launch_bounds__(256) void k_mse_reduce(const double *__restrict__ msepart, int ncap,
                                                    const int *__restrict__ ncl, int L, float *__restrict__ mse) {
  const int h = blockIdx.x;
  __shared__ double part[256];
  double loc = 0.0;
  for (int c = threadIdx.x; c < ncl[h]; c += 256) loc += msepart[(int64_t)h * ncap + c];
  part[threadIdx.x] = loc;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) part[threadIdx.x] += part[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) mse[h] = (float)(part[0] / (double)L);
}

// mean of a per-token scalar over each cluster's members (rho of the query
// clusters: mean ||q||), fp64 sum in counting-sort order.
__global__ __launch_bounds__(256) void k_seg_mean(const float *__restrict__ val, const int *__restrict__ perm,
                                                  const int *__restrict__ seg, int L, int ncap,
                                                  const int *__restrict__ ncl, float *__restrict__ out) {
  const int h = blockIdx.y, c = blockIdx.x;
  if (c >= ncap) return;
  const int *sg = seg + (int64_t)h * (ncap + 1);
  const int beg = c < ncl[h] ? sg[c] : 0, end = c < ncl[h] ? sg[c + 1] : 0;
  __shared__ double part[256];
  double loc = 0.0;
  for (int p = beg + threadIdx.x; p < end; p += 256) loc += (double)val[(int64_t)h * L + perm[(int64_t)h * L + p]];
  part[threadIdx.x] = loc;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) part[threadIdx.x] += part[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[(int64_t)h * ncap + c] = end > beg ? (float)(part[0] / (double)(end - beg)) : 0.f;
}

// ---------------------------------------------------------------------------
// small per-head bookkeeping kernels
__global__ void k_fill_i32(int *__restrict__ p, int64_t n, int v) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}
// one cluster per head holding every token in order: perm = 0..L-1,
// seg = [0, L, L, ...], ncl = 1 (the layout of dense attention)
__global__ void k_identity_clusters(int *__restrict__ perm, int *__restrict__ seg, int *__restrict__ ncl, int L,
                                    int segcap) {
  const int h = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < L) perm[(int64_t)h * L + i] = (int)i;
  if (i <= segcap) seg[(int64_t)h * (segcap + 1) + i] = i == 0 ? 0 : L;
  if (i == 0) ncl[h] = 1;
}
// Labels of the heads that left the Lloyd loop (neff = 0 < n): the loop's last
// assignment, which the final one would repeat.
__global__ void k_copy_converged(const int *__restrict__ n, const int *__restrict__ neff, const int *__restrict__ src,
                                 int *__restrict__ dst, int64_t hs) {
  const int h = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (neff[h] != 0 || i >= n[h]) return;
  dst[(int64_t)h * hs + i] = src[(int64_t)h * hs + i];
}
__global__ void k_copy_i32(const int *__restrict__ src, int *__restrict__ dst, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src[i];
}
__global__ void k_copy_f32(const float *__restrict__ src, float *__restrict__ dst, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src[i];
}
__global__ void k_copy_u8(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src[i];
}
__global__ void k_fill_u8(uint8_t *__restrict__ p, int64_t n, uint8_t v) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

// ---------------------------------------------------------------------------
// Stage records of the traced entry points: copies only.
// Centres of the job, m[h] rows from cent[h][coff[h]], into dst[h] (stride dst_hs).
template <int D>
__global__ __launch_bounds__(256) void k_trace_cent(KmArgs a, float *__restrict__ dst, int64_t dst_hs) {
  const int h = blockIdx.y, c = blockIdx.x;
  if (c >= a.m[h] || a.n[h] <= 0) return;
  const float *src = a.cent + (int64_t)h * a.cent_hs + (int64_t)(a.coff[h] + c) * D;
  for (int dd = threadIdx.x; dd < D; dd += 256) dst[(int64_t)h * dst_hs + (int64_t)c * D + dd] = src[dd];
}
// Point lists of a stage: key index, stage label and distance of the first n[h] points.
__global__ void k_trace_stage(const int *__restrict__ n, const int *__restrict__ idx, int64_t idx_hs,
                              const int *__restrict__ lab, const float *__restrict__ dist, int64_t hs,
                              int *__restrict__ u_out, int *__restrict__ lab_out, float *__restrict__ dist_out,
                              int64_t out_hs) {
  const int h = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n[h]) return;
  const int64_t o = (int64_t)h * out_hs + i;
  if (u_out) u_out[o] = idx ? idx[(int64_t)h * idx_hs + i] : (int)i;
  if (lab_out) lab_out[o] = lab[(int64_t)h * hs + i];
  if (dist_out) dist_out[o] = dist[(int64_t)h * hs + i];
}
// n[h] and m[h] into column t of [BH, ld] tables.
__global__ void k_trace_nm(const int *__restrict__ n, const int *__restrict__ m, int *__restrict__ n_out,
                           int *__restrict__ m_out, int ld, int t, int BH) {
  const int h = blockIdx.x * 256 + threadIdx.x;
  if (h >= BH) return;
  if (n_out) n_out[(int64_t)h * ld + t] = n[h];
  if (m_out) m_out[(int64_t)h * ld + t] = m[h];
}

// ---------------------------------------------------------------------------
// Algorithm 1's per-head bookkeeping between stages (one thread per head).
// st[h] = {|U|, centres so far, done, fallback, stages run, m and n of the
// current stage}.  Stage 0 starts with U = all L keys.  Closing stage t - 1
// (t > 0): the head adds that stage's m centres and keeps the nnew[h] keys
// that stayed in U; a head whose U is empty is done.  Opening stage t: a head
// that would start with nmax centres or more and keys left falls back and is
// done.  Writes n, m (0 for heads that are done) and the first centre of
// stage t.
__global__ void k_stage_next(int *__restrict__ st, const int *__restrict__ nnew, int *__restrict__ n,
                             int *__restrict__ m, int *__restrict__ coff, int t, int nmax, int m0, int L, int BH) {
  const int h = blockIdx.x * 256 + threadIdx.x;
  if (h >= BH) return;
  int *x = st + (int64_t)h * KST_FIELDS;
  int nU, nC, done, F, stg;
  if (t == 0) {
    nU = L; nC = 0; done = 0; F = 0; stg = 0;
  } else {
    nU = x[0]; nC = x[1]; done = x[2]; F = x[3]; stg = x[4];
    if (!done) {
      nC += x[5];
      stg = t;
      nU = x[6] > 0 ? nnew[h] : 0;
      if (nU == 0) done = 1;
    }
  }
  if (!done && nC >= nmax) { F = 1; done = 1; }
  const int nn = done ? 0 : nU, mm = done ? 0 : min(nU, m0);
  x[0] = nU; x[1] = nC; x[2] = done; x[3] = F; x[4] = stg; x[5] = mm; x[6] = nn;
  n[h] = nn;
  m[h] = mm;
  coff[h] = nC;
}
// Outputs of Algorithm 1 from the state: centre count, fallback, stages.
__global__ void k_stage_final(const int *__restrict__ st, int *__restrict__ ncl, uint8_t *__restrict__ fallback,
                              int *__restrict__ stages, int BH) {
  const int h = blockIdx.x * 256 + threadIdx.x;
  if (h >= BH) return;
  const int *x = st + (int64_t)h * KST_FIELDS;
  ncl[h] = x[1];
  fallback[h] = (uint8_t)x[3];
  stages[h] = x[4];
}

// ---------------------------------------------------------------------------
// host launchers
static inline dim3 g2(int64_t x, int y) { return dim3((unsigned)(x > 0 ? x : 1), (unsigned)y); }

#define AC_D_DISPATCH(D, ...)            \
  do {                                   \
    if ((D) == 64) { constexpr int DD = 64; __VA_ARGS__; } \
    else { constexpr int DD = 128; __VA_ARGS__; }           \
  } while (0)

void launch_qnorm(int D, const uint16_t *Q, uint16_t *Qh, float *qn, int64_t rows, hipStream_t st) {
  int64_t blocks = (rows * 8 + 255) / 256;
  AC_D_DISPATCH(D, hipLaunchKernelGGL(k_qnorm<DD>, dim3((unsigned)blocks), dim3(256), 0, st, Q, Qh, qn, rows));
}

void launch_cent_prep(int D, const KmArgs &a, const CentOps &op, int BH, int mmax, hipStream_t st, bool at_coff) {
  AC_D_DISPATCH(D, hipLaunchKernelGGL(k_cent_prep<DD>, g2((mmax + 3) / 4, BH), dim3(256), 0, st, a, op,
                                      at_coff ? 1 : 0));
}

static int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cache[dev] = v;
  }
  return cache[dev];
}

void launch_assign(int D, const KmArgs &a, const CentOps &op, int BH, int mmax, int nmax_pts, int *labels,
                   int64_t lab_hs, hipStream_t st, int *chg, float *best_io, int spare_cus) {
  if (mmax <= ASSIGN_RES_MAX || best_io) {
    // 768 threads and LDS for this launch's centres only, one block per CU:
    // three waves a SIMD, so one wave's point loads hide behind two others'
    // MFMA work (two a SIMD measured 8% slower; four would spill registers)
    constexpr int NT = 768;
    const int mpmax = (mmax + 15) & ~15;
    const size_t lds = (size_t)mpmax * (D + 8) * 2 * 2 + (size_t)mpmax * 4;
    const int64_t subs = (int64_t)BH * ((nmax_pts + 63) / 64);
    const int all = device_cus();
    const int cus = spare_cus > 0 && spare_cus <= all / 4 ? all - spare_cus : all;
    const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>(cus, (subs + NT / 64 - 1) / (NT / 64)));
    AC_D_DISPATCH(D, {
      static bool lds_ok = hipFuncSetAttribute((const void *)k_assign_res<DD, NT>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)((size_t)ASSIGN_RES_MAX * (DD + 8) * 4 + ASSIGN_RES_MAX * 4)) ==
                           hipSuccess;
      (void)lds_ok;  // a refusal shows up as a launch error
      hipLaunchKernelGGL((k_assign_res<DD, NT>), dim3(blocks), dim3(NT), lds, st, a, op, labels, lab_hs, BH, mpmax,
                         chg, best_io);
    });
    return;
  }
  AC_D_DISPATCH(D, hipLaunchKernelGGL(k_assign<DD>, g2((nmax_pts + 255) / 256, BH), dim3(256), 0, st, a, op, labels,
                                      lab_hs, chg));
}

void launch_sort(const SortArgs &s, int BH, int nmax_pts, hipStream_t st) {
  int tiles = (nmax_pts + SORT_TILE - 1) / SORT_TILE;
  size_t sh = (size_t)s.mcap * sizeof(int);
  const int groups = (tiles + SORT_GROUP - 1) / SORT_GROUP;
  hipLaunchKernelGGL(k_sort_hist, g2(tiles, BH), dim3(64), sh, st, s);
  hipLaunchKernelGGL(k_sort_gscan, dim3((unsigned)groups, (unsigned)BH, (unsigned)((s.mcap + 255) / 256)), dim3(256), 0,
                     st, s);
  hipLaunchKernelGGL(k_sort_scan, dim3(BH), dim3(1024), 0, st, s);
  hipLaunchKernelGGL(k_sort_scatter, g2(tiles, BH), dim3(64), sh, st, s);
}

void launch_sort_small(const SortArgs &s, int BH, hipStream_t st) {
  hipLaunchKernelGGL(k_sort_small, dim3(BH), dim3(1024), 0, st, s);
}

void launch_update_small(int D, const KmArgs &a, const SortArgs &s, const CentOps &op, int BH, int mmax,
                         hipStream_t st) {
  AC_D_DISPATCH(D, hipLaunchKernelGGL(k_update_small<DD>, g2(mmax, BH), dim3(256), 0, st, a, s, op));
}

void launch_update(int D, const KmArgs &a, const SortArgs &s, const CentOps &op, int BH, int mmax, int npts,
                   double *partial, int64_t part_hs, hipStream_t st) {
  const int *chunk_off = s.chunk_off;  // written by the label scan of the sort
  const int64_t co_hs = s.co_hs;
  const int items = (npts + UPD_CHUNK - 1) / UPD_CHUNK + mmax;
  AC_D_DISPATCH(D, hipLaunchKernelGGL(k_update_partial<DD>, g2(items, BH), dim3(256), 0, st, a, s, chunk_off, co_hs,
                                      partial, part_hs));
  AC_D_DISPATCH(D, hipLaunchKernelGGL(k_update_final<DD>, g2(mmax, BH), dim3(128), 0, st, a, s, chunk_off, co_hs,
                                      partial, part_hs, op));
}

void launch_stage_dist(int D, const KmArgs &a, int BH, int nmax_pts, const int *labels, int64_t lab_hs, float *dist,
                       int64_t dist_hs, hipStream_t st) {
  AC_D_DISPATCH(D, hipLaunchKernelGGL(k_stage_dist<DD>, g2((nmax_pts + 16 * SD_PTS - 1) / (16 * SD_PTS), BH), dim3(256),
                                      0, st, a, labels, lab_hs, dist, dist_hs));
}

void launch_tau(const float *dist, int64_t dist_hs, const int *n_arr, int BH, int nmax_pts, int rule, float param,
                float *tau, uint32_t *radix_state, uint32_t *radix_hist, hipStream_t st) {
  if (rule != TAU_RULE_PCTL) {
    hipLaunchKernelGGL(k_tau_direct, dim3(BH), dim3(1024), 0, st, dist, dist_hs, n_arr, rule, param, tau);
    return;
  }
  hipLaunchKernelGGL(k_radix_init, dim3(BH), dim3(256), 0, st, n_arr, param, radix_state, radix_hist);
  int blocks = (nmax_pts + 4095) / 4096;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hipLaunchKernelGGL(k_radix_hist, g2(blocks, BH), dim3(256), 0, st, dist, dist_hs, n_arr, radix_state, radix_hist,
                       shift);
    hipLaunchKernelGGL(k_radix_pick, dim3(BH), dim3(64), 0, st, radix_state, radix_hist, shift, tau);
  }
}

void launch_flag_removed(const float *dist, int64_t dist_hs, const int *n_arr, const float *tau, int *flag,
                         int64_t flag_hs, int BH, int nmax_pts, hipStream_t st) {
  hipLaunchKernelGGL(k_flag_removed, g2((nmax_pts + 255) / 256, BH), dim3(256), 0, st, dist, dist_hs, n_arr, tau,
                     flag, flag_hs);
}

void launch_compact_gather(const int *idx_old, int64_t idx_hs, const int *perm, int64_t perm_hs, const int *seg,
                           int64_t seg_hs, int *idx_new, int *n_new, int BH, int nmax_pts, hipStream_t st) {
  hipLaunchKernelGGL(k_compact_gather, g2((nmax_pts + 255) / 256, BH), dim3(256), 0, st, idx_old, idx_hs, perm,
                     perm_hs, seg, seg_hs, idx_new, n_new);
}

void launch_trace_cent(int D, const KmArgs &a, int BH, int mmax, float *dst, int64_t dst_hs, hipStream_t st) {
  AC_D_DISPATCH(D, hipLaunchKernelGGL(k_trace_cent<DD>, g2(mmax, BH), dim3(256), 0, st, a, dst, dst_hs));
}

void launch_trace_stage(const int *n, const int *idx, int64_t idx_hs, const int *lab, const float *dist, int64_t hs,
                        int *u_out, int *lab_out, float *dist_out, int64_t out_hs, int BH, int npts, hipStream_t st) {
  hipLaunchKernelGGL(k_trace_stage, g2((npts + 255) / 256, BH), dim3(256), 0, st, n, idx, idx_hs, lab, dist, hs,
                     u_out, lab_out, dist_out, out_hs);
}

void launch_trace_nm(const int *n, const int *m, int *n_out, int *m_out, int ld, int t, int BH, hipStream_t st) {
  hipLaunchKernelGGL(k_trace_nm, dim3((BH + 255) / 256), dim3(256), 0, st, n, m, n_out, m_out, ld, t, BH);
}

void launch_stage_next(int *state, const int *nnew, int *n, int *m, int *coff, int t, int nmax, int m0, int L,
                       int BH, hipStream_t st) {
  hipLaunchKernelGGL(k_stage_next, dim3((BH + 255) / 256), dim3(256), 0, st, state, nnew, n, m, coff, t, nmax, m0, L,
                     BH);
}
void launch_stage_final(const int *state, int *ncl, uint8_t *fallback, int *stages, int BH, hipStream_t st) {
  hipLaunchKernelGGL(k_stage_final, dim3((BH + 255) / 256), dim3(256), 0, st, state, ncl, fallback, stages, BH);
}

void launch_kstats(int D, const KStatsArgs &s, int BH, hipStream_t st) {
  hipLaunchKernelGGL(k_kst_chunks, dim3(BH), dim3(1024), 0, st, s);
  const int items = (s.L + KST_CHUNK - 1) / KST_CHUNK + s.ncap;
  AC_D_DISPATCH(D, hipLaunchKernelGGL(k_kstats_part<DD>, g2(items, BH), dim3(64), 0, st, s));
  AC_D_DISPATCH(D, hipLaunchKernelGGL(k_kstats_fin<DD>, g2(s.ncap, BH), dim3(128), 0, st, s));
  hipLaunchKernelGGL(k_mse_reduce, dim3(BH), dim3(256), 0, st, s.msepart, s.ncap, s.ncl, s.L, s.mse);
}

void launch_seg_mean(const float *val, const int *perm, const int *seg, int L, int ncap, const int *ncl, float *out,
                     int BH, hipStream_t st) {
  hipLaunchKernelGGL(k_seg_mean, g2(ncap, BH), dim3(256), 0, st, val, perm, seg, L, ncap, ncl, out);
}

void launch_fill_i32(int *p, int64_t n, int v, hipStream_t st) {
  if (n > 0) hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n, v);
}
void launch_identity_clusters(int *perm, int *seg, int *ncl, int L, int segcap, int BH, hipStream_t st) {
  const int64_t n = std::max<int64_t>(L, (int64_t)segcap + 1);
  hipLaunchKernelGGL(k_identity_clusters, dim3((unsigned)((n + 255) / 256), (unsigned)BH), dim3(256), 0, st, perm, seg,
                     ncl, L, segcap);
}
void launch_fill_u8(uint8_t *p, int64_t n, uint8_t v, hipStream_t st) {
  if (n > 0) hipLaunchKernelGGL(k_fill_u8, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n, v);
}
void launch_copy_converged(const int *n, const int *neff, const int *src, int *dst, int64_t hs, int npts, int BH,
                           hipStream_t st) {
  if (npts > 0 && BH > 0)
    hipLaunchKernelGGL(k_copy_converged, g2((npts + 255) / 256, BH), dim3(256), 0, st, n, neff, src, dst, hs);
}
void launch_copy_i32(const int *s, int *d, int64_t n, hipStream_t st) {
  if (n > 0) hipLaunchKernelGGL(k_copy_i32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, s, d, n);
}
void launch_copy_f32(const float *s, float *d, int64_t n, hipStream_t st) {
  if (n > 0) hipLaunchKernelGGL(k_copy_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, s, d, n);
}
void launch_copy_u8(const uint8_t *s, uint8_t *d, int64_t n, hipStream_t st) {
  if (n > 0) hipLaunchKernelGGL(k_copy_u8, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, s, d, n);
}

}  // namespace ac
