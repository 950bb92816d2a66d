// ClusterAttention's clustering for gfx950: recursive splits along the
// leading principal direction into clusters of a preset power-of-two size b.
//
// A node of n > b points (a contiguous range of the head's token order) is
// cut in two: the n_left = b * ceil(ceil(n / b) / 2) points with the
// smallest projections onto the node's direction go left, the rest right,
// each side keeping its token order.  The tree's shape depends only on n and
// b, so every level is one launch over the internal nodes of that level
// (one workgroup per node and head; a level of large nodes is three
// launches, so that many workgroups share its projections).  A workgroup:
//   1. takes a strided subsample of s = min(n, PCA_SMAX) points and its mean;
//   2. forms the d x d covariance of the centred subsample (bf16 of x - mean)
//      with 32x32x16 bf16 MFMA (fp32 sums), gathering PCA_CHUNK points into
//      LDS at a time, and finds the point farthest from the mean;
//   3. squares it PCA_SQUARINGS times on MFMA (split bf16, trace-normalised);
//   4. runs the matching PCA_ITERS / 2^PCA_SQUARINGS power iterations from
//      the subsample row farthest from the mean (the same direction as
//      PCA_ITERS iterations with the covariance) and orients the result
//      (largest component positive);
//   5. projects every point of the node (fp32), radix-selects the n_left-th
//      smallest (projection, position) key in four 8-bit passes, and writes
//      the stable partition of the node's tokens.
#include <algorithm>
#include <utility>
#include <vector>

#include "common.h"
#include "internal.h"

namespace ac {

constexpr int PCA_CHUNK = 256;         // subsample points in LDS at a time
// dynamic LDS of a level: the larger of a chunk of the subsample (D x (chunk
// width + 8) bf16) and the split squares (2 x D x (D + 8) bf16)
constexpr int pca_lds_max(int D) {
  return D * (PCA_CHUNK + 8) * 2 > D * (D + 8) * 4 ? D * (PCA_CHUNK + 8) * 2 : D * (D + 8) * 4;
}
constexpr int PCA_SQUARINGS = 3;      // the power iteration runs with C^8
constexpr int PCA_PJ = 8;             // projection loads in flight per 16 lanes

// Internal nodes of the split tree of n points, level by level, left to
// right: nodes[k] = (first position, count); lvl[l] = first node of level l,
// lvl[levels] = node count.  One thread: the tree has about n / b nodes.
__global__ void k_pca_tree(int n, int b, int2 *__restrict__ nodes, int *__restrict__ lvl) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int head = 0, tail = 0, level = 0;
  if (n > b) nodes[tail++] = make_int2(0, n);
  while (head < tail) {
    const int end = tail;
    lvl[level++] = head;
    for (; head < end; ++head) {
      const int2 nd = nodes[head];
      const int nb = (nd.y + b - 1) / b, nl = b * ((nb + 1) / 2), nr = nd.y - nl;
      if (nl > b) nodes[tail++] = make_int2(nd.x, nl);
      if (nr > b) nodes[tail++] = make_int2(nd.x + nl, nr);
    }
  }
  lvl[level] = tail;
}

// The same list built by one 1024-thread block, level by level: each level's
// nodes sit in LDS (at most PCA_TREE_CAP), every thread takes a parent, and a
// block scan of the internal-children counts places the children (left, then
// right, parents in order), so the order is the one above.
constexpr int PCA_TREE_CAP = 4096;
__global__ __launch_bounds__(1024) void k_pca_tree_wide(int n, int b, int2 *__restrict__ nodes, int *__restrict__ lvl) {
  __shared__ int2 buf[2][PCA_TREE_CAP];
  __shared__ int wtot[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int cnt = n > b ? 1 : 0, base = 0, level = 0, cur = 0;
  if (tid == 0 && cnt) {
    buf[0][0] = make_int2(0, n);
    nodes[0] = make_int2(0, n);
  }
  __syncthreads();
  while (cnt > 0) {
    if (tid == 0) lvl[level] = base;
    int next = 0;
    for (int c0 = 0; c0 < cnt; c0 += 1024) {
      const int i = c0 + tid;
      int2 nd = make_int2(0, 0);
      int nl = 0, nr = 0, kids = 0;
      if (i < cnt) {
        nd = buf[cur][i];
        const int nb = (nd.y + b - 1) / b;
        nl = b * ((nb + 1) / 2);
        nr = nd.y - nl;
        kids = (nl > b) + (nr > b);
      }
      int inc = kids;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(inc, o, 64);
        if (lane >= o) inc += t;
      }
      if (lane == 63) wtot[wave] = inc;
      __syncthreads();
      int off = 0, tot = 0;
#pragma unroll
      for (int w = 0; w < 16; ++w) {
        const int t = wtot[w];
        if (w < wave) off += t;
        tot += t;
      }
      int o = next + off + inc - kids;
      if (nl > b) {
        const int2 c = make_int2(nd.x, nl);
        buf[cur ^ 1][o] = c;
        nodes[base + cnt + o] = c;
        ++o;
      }
      if (nr > b) {
        const int2 c = make_int2(nd.x + nl, nr);
        buf[cur ^ 1][o] = c;
        nodes[base + cnt + o] = c;
      }
      next += tot;
      __syncthreads();
    }
    base += cnt;
    cnt = next;
    cur ^= 1;
    ++level;
  }
  if (tid == 0) lvl[level] = base;
}

// Block-wide exclusive scan of two counters (512 threads = 8 waves); returns
// the thread's exclusive prefix and writes the block totals.
AC_DEV int2 block_scan2(int x, int y, int2 *sh, int2 &tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int ix = x, iy = y;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int a = __shfl_up(ix, o, 64), b = __shfl_up(iy, o, 64);
    if (lane >= o) { ix += a; iy += b; }
  }
  if (lane == 63) sh[wave] = make_int2(ix, iy);
  __syncthreads();
  int ox = 0, oy = 0, tx = 0, ty = 0;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const int2 t = sh[w];
    if (w < wave) { ox += t.x; oy += t.y; }
    tx += t.x;
    ty += t.y;
  }
  __syncthreads();
  tot = make_int2(tx, ty);
  return make_int2(ox + ix - x, oy + iy - y);
}

// Projections of the node's points [beg, end) onto the direction whose
// entries sub*PL .. sub*PL + PL - 1 the lane holds in vv: 16 lanes a point
// (lane sub takes those PL dimensions; the sum over the 16 lanes by DPP),
// groups of 16 lanes stepping by `groups`, PCA_PJ points in flight each.
// key[p] gets the order-preserving bits of the fp32 projection, tmp[p] the
// token.  k_pca_level and k_pca_project share it, so both give the same keys.
template <int D>
AC_DEV void pca_project(const uint16_t *X, const int *perm, int *tmp, uint32_t *key, const float *vv, int beg,
                        int end, int grp, int groups, int sub) {
  constexpr int PL = D / 16;
  constexpr int PJ = PCA_PJ;
  typedef uint32_t pw_t __attribute__((ext_vector_type(PL / 2)));
  for (int p0 = beg + grp; p0 < end; p0 += PJ * groups) {
    int t[PJ];
    pw_t xw[PJ];
#pragma unroll
    for (int j = 0; j < PJ; ++j) {
      const int p = p0 + j * groups;
      t[j] = p < end ? perm[p] : 0;
    }
#pragma unroll
    for (int j = 0; j < PJ; ++j) xw[j] = *(const pw_t *)(X + (int64_t)t[j] * D + sub * PL);
#pragma unroll
    for (int j = 0; j < PJ; ++j) {
      float acc2 = 0.f;
#pragma unroll
      for (int k = 0; k < PL; ++k) {
        const uint32_t w = xw[j][k >> 1];
        acc2 = fmaf(bf2f((uint16_t)((k & 1) ? (w >> 16) : (w & 0xFFFFu))), vv[k], acc2);
      }
      acc2 = row16_sum(acc2);  // the 16 lanes of the point
      const int p = p0 + j * groups;
      if (sub == 0 && p < end) {
        key[p] = f2ord(acc2 + 0.f);  // -0 and +0 order alike
        tmp[p] = t[j];
      }
    }
  }
}

// mode 0: the whole node; 1: its direction only, to a.dbuf; 2: the cut only,
// from the projection keys k_pca_project wrote (a level of large nodes runs
// modes 1, k_pca_project and 2, so that many blocks share its projections).
// sp: row stride (bf16) of a subsample chunk in LDS, its width + 8, set by
// the launch from the level's largest node; the dynamic LDS holds the larger
// of a chunk, D sp bf16, and the split squares, 2 D (D + 8) bf16 (the fp32
// D x D matrix fits in the latter); mode 2 uses none of it.
template <int D>
__global__ __launch_bounds__(512) void k_pca_level(PcaArgs a, int first, int count, int sp, int mode) {
  constexpr int NT = 512;
  const int h = blockIdx.y, node = first + (int)blockIdx.x;
  if ((int)blockIdx.x >= count) return;
  const int2 nd = a.nodes[node];
  const int start = nd.x, n = nd.y, b = a.block;
  const int nb = (n + b - 1) / b, nl = b * ((nb + 1) / 2);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint16_t *X = a.X + (int64_t)h * a.L * D;
  int *perm = a.perm + (int64_t)h * a.L + start;
  int *tmp = a.tmp + (int64_t)h * a.L + start;
  uint32_t *key = a.key + (int64_t)h * a.L + start;

  extern __shared__ __align__(16) unsigned char pca_lds[];
  uint16_t *Y = reinterpret_cast<uint16_t *>(pca_lds);  // [D][sp] bf16, later C [D][D] fp32
  float *C = reinterpret_cast<float *>(pca_lds);
  __shared__ __align__(16) float mu[D];
  __shared__ __align__(16) float wbuf[2][D];
  __shared__ __align__(16) float nrm_part[2][8];
  __shared__ __align__(16) uint32_t hist[256];
  __shared__ int sidx[PCA_SMAX];
  __shared__ float far_n[8];
  __shared__ int far_j[8];
  __shared__ int2 scan_sh[8];
  __shared__ uint32_t sh_prefix, sh_rank;
  __shared__ float sh_best;  // squared distance of the start row from the mean
  __shared__ int sh_zero;  // 0, read where a value must not be hoisted out of a loop
  if (tid == 0) sh_zero = 0;

  if (mode != 2) {
    // 1. the strided subsample's tokens (one 64-bit division each)
    const int s = min(n, PCA_SMAX);
    for (int j = tid; j < s; j += NT) sidx[j] = perm[(int)(((int64_t)j * n) / s)];
    if (tid == 0) sh_best = -1.f;
    __syncthreads();
    // mean of each dimension over the subsample, from the rows in memory:
    // thread (chunk c, point group pg) sums the 8 dimensions of chunk c over
    // points pg, pg + PG, ... (8 loads in flight); the lanes of a wave with the
    // same c, then the waves, are added in a fixed order
    {
      constexpr int CPR = D / 8;    // 16-byte chunks per row
      constexpr int PG = NT / CPR;  // point groups
      const int c = tid % CPR, pg = tid / CPR;
      float sum8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int j0 = pg; j0 < s; j0 += 8 * PG) {
        u32x4_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int j = j0 + u * PG;
          v[u] = (u32x4_t){0u, 0u, 0u, 0u};
          if (j < s) v[u] = *(const u32x4_t *)(X + (int64_t)sidx[j] * D + c * 8);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) sum8[e] += bf2f((uint16_t)((e & 1) ? (v[u][e >> 1] >> 16) : (v[u][e >> 1] & 0xFFFFu)));
      }
#pragma unroll
      for (int o = CPR; o < 64; o <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) sum8[e] += __shfl_xor(sum8[e], o, 64);
      float *part = reinterpret_cast<float *>(pca_lds);  // [NT / 64][D], in the subsample's space
      if (lane < CPR)
#pragma unroll
        for (int e = 0; e < 8; ++e) part[wave * D + c * 8 + e] = sum8[e];
      __syncthreads();
      if (tid < D) {
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) t += part[w * D + tid];
        mu[tid] = t / (float)s;
      }
      __syncthreads();
    }

    // 2. covariance C = Y Y^T of the centred subsample Y (bf16 of x - mean;
    // unnormalised, only its direction matters), over chunks of up to sp - 8
    // points: a chunk is gathered centred into LDS, dimension-major (a lane
    // takes one 16-byte chunk of 4 consecutive points and writes it as 8 rows
    // of 4 columns; the 32 lanes of a store pass cover two chunks of 16 point
    // groups, every bank once); its farthest point from the mean updates the
    // start of the power iteration; then one 32x32 tile of C per wave and pass
    // accumulates it on MFMA.
    constexpr int NTILE = (D / 32) * (D / 32);
    constexpr int TPW = (NTILE + 7) / 8;
    f32x16_t acc[TPW];
#pragma unroll
    for (int k = 0; k < TPW; ++k) acc[k] = (f32x16_t){};
    const int l32 = lane & 31, g = lane >> 5;
    const int chw = sp - 8;  // chunk width, a multiple of 16
    for (int ch0 = 0; ch0 < s; ch0 += chw) {
      const int cs = min(chw, s - ch0), cpad = (cs + 15) & ~15;
      {
        constexpr int CQ = D / 32;  // chunk quads per point (16-byte chunks: D / 8)
        const int ngrp = cpad / 4;  // groups of 4 points
        const int nitem = ((ngrp + 15) / 16) * CQ;
        for (int it = wave; it < nitem; it += NT / 64) {
          const int c = (it % CQ) * 4 + (lane >> 4), jq = (it / CQ) * 16 + (lane & 15);
          if (jq < ngrp) {
            u32x4_t v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const int j = 4 * jq + k;
              v[k] = (u32x4_t){0u, 0u, 0u, 0u};
              if (j < cs) v[k] = *(const u32x4_t *)(X + (int64_t)sidx[ch0 + j] * D + c * 8);
            }
            const float4 m0 = *(const float4 *)&mu[c * 8], m1 = *(const float4 *)&mu[c * 8 + 4];
            const float m8[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int sh = 16 * (e & 1);
              uint32_t y[4];
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                const uint16_t xb = (uint16_t)((v[k][e >> 1] >> sh) & 0xFFFFu);
                y[k] = 4 * jq + k < cs ? f2bf(bf2f(xb) - m8[e]) : 0u;  // the padding columns stay zero
              }
              *(uint2 *)&Y[(c * 8 + e) * sp + 4 * jq] = make_uint2(y[0] | (y[1] << 16), y[2] | (y[3] << 16));
            }
          }
        }
      }
      __syncthreads();
      // the chunk's point farthest from the mean (two threads a point, lowest
      // position on ties); a strictly farther one than the earlier chunks'
      // becomes the start (unnormalised; the first iteration normalises)
      {
        const int j = tid >> 1, half = tid & 1;
        float nn = -1.f;
        if (j < cs) {
          nn = 0.f;
#pragma unroll 8
          for (int i = half * (D / 2); i < (half + 1) * (D / 2); ++i) {
            const float y = bf2f(Y[i * sp + j]);
            nn = fmaf(y, y, nn);
          }
        }
        nn += dpp_f32<0xB1>(nn);  // the point's other half
        int bj = ch0 + j;
#pragma unroll
        for (int o = 32; o > 1; o >>= 1) {
          const float on = __shfl_xor(nn, o, 64);
          const int oj = __shfl_xor(bj, o, 64);
          if (on > nn || (on == nn && oj < bj)) { nn = on; bj = oj; }
        }
        if (lane == 0) { far_n[wave] = nn; far_j[wave] = bj; }
        __syncthreads();
        if (wave == 0) {
          float bn = lane < 8 ? far_n[lane] : -2.f;
          int bjj = lane < 8 ? far_j[lane] : 0x7fffffff;
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) {
            const float on = __shfl_xor(bn, o, 64);
            const int oj = __shfl_xor(bjj, o, 64);
            if (on > bn || (on == bn && oj < bjj)) { bn = on; bjj = oj; }
          }
          if (bn > sh_best) {
            float sq = 0.f;
            for (int i = lane; i < D; i += 64) {
              const float y = bf2f(Y[i * sp + (bjj - ch0)]);
              wbuf[0][i] = y;
              sq = fmaf(y, y, sq);
            }
            sq = wave_sum(sq);
            if (lane < 8) nrm_part[0][lane] = lane == 0 ? sq : 0.f;
            if (lane == 0) sh_best = bn;
          }
        }
      }
      for (int k0 = 0; k0 < cpad; k0 += 16) {
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
          const int tile = wave + 8 * k;
          if (tile < NTILE) {
            const int I = tile / (D / 32), J = tile % (D / 32);
            const bf16x8_t av = *(const bf16x8_t *)&Y[(I * 32 + l32) * sp + k0 + 8 * g];
            const bf16x8_t bv = *(const bf16x8_t *)&Y[(J * 32 + l32) * sp + k0 + 8 * g];
            acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[k], 0, 0, 0);
          }
        }
      }
      __syncthreads();  // every read of the chunk is done before the next one (or A) overwrites it
    }

    // 3. A = C / tr(C), then PCA_SQUARINGS times A <- A A^T / tr(A A^T), so that
    // A ends as C^(2^PCA_SQUARINGS) up to a positive factor; the power
    // iteration then takes PCA_ITERS / 2^PCA_SQUARINGS steps with it, which in
    // exact arithmetic is the same as PCA_ITERS steps with C.  The trace keeps
    // the leading eigenvalue in [1/D, 1].  The products run on bf16 MFMA with A
    // split into bf16 hi + lo (fp32 sums; the lo x lo term, below 2^-16 of an
    // entry, is dropped).  LDS holds A_hi and A_lo row-major with rows of
    // D + 8 bf16, so that the 16 rows of a 16-lane pass of the operand reads
    // fall on distinct banks; the last A is written fp32 in the plain layout
    // the power iteration reads.
    constexpr int AP = D + 8;
    uint16_t *Ahi = reinterpret_cast<uint16_t *>(pca_lds), *Alo = Ahi + D * AP;
    auto aidx = [](int r, int c) { return r * AP + c; };
#pragma unroll 1
    for (int sq = 0; sq <= PCA_SQUARINGS; ++sq) {
      if (sq > 0) {
#pragma unroll
        for (int k = 0; k < TPW; ++k) acc[k] = (f32x16_t){};
#pragma unroll 1
        for (int k0 = 0; k0 < D; k0 += 16) {
#pragma unroll
          for (int k = 0; k < TPW; ++k) {
            const int tile = wave + 8 * k;
            if (tile < NTILE) {
              const int I = tile / (D / 32), J = tile % (D / 32);
              const int ia = aidx(I * 32 + l32, k0 + 8 * g), ib = aidx(J * 32 + l32, k0 + 8 * g);
              const bf16x8_t ah = *(const bf16x8_t *)&Ahi[ia], al = *(const bf16x8_t *)&Alo[ia];
              const bf16x8_t bh = *(const bf16x8_t *)&Ahi[ib], bl = *(const bf16x8_t *)&Alo[ib];
              acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc[k], 0, 0, 0);
              acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc[k], 0, 0, 0);
              acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, acc[k], 0, 0, 0);
            }
          }
        }
      }
      // the diagonal: in a tile with I == J, lane (l32, g) with g = bit 2 of
      // l32 holds entry l32 in register 4 (l32 / 8) + l32 % 4
#pragma unroll
      for (int k = 0; k < TPW; ++k) {
        const int tile = wave + 8 * k;
        if (tile < NTILE && tile / (D / 32) == tile % (D / 32) && g == ((l32 >> 2) & 1)) {
          const int rr = 4 * (l32 >> 3) + (l32 & 3);
          float dv = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (r == rr) dv = acc[k][r];
          mu[(tile / (D / 32)) * 32 + l32] = dv;
        }
      }
      __syncthreads();  // the diagonal is complete; every read of Y or of A is done
      float tr = 0.f;
#pragma unroll
      for (int i = 0; i < D; i += 4) {
        const float4 t4 = *(const float4 *)&mu[i];
        tr += (t4.x + t4.y) + (t4.z + t4.w);
      }
      const float inv = tr > 0.f ? 1.f / tr : 0.f;
      // entry r of a tile sits at a lane base plus a constant; the base goes
      // through an LDS zero so that the 16 addresses are not kept in registers
      // across the stages but folded into the stores' offsets
      const int z = sh_zero;
#pragma unroll
      for (int k = 0; k < TPW; ++k) {
        const int tile = wave + 8 * k;
        if (tile < NTILE) {
          const int I = tile / (D / 32), J = tile % (D / 32);
          const int rb = I * 32 + 4 * g + z, cl = J * 32 + l32;
          if (sq < PCA_SQUARINGS) {
            uint16_t *ph = Ahi + aidx(rb, cl), *pl = Alo + aidx(rb, cl);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float v = acc[k][r] * inv;
              const uint16_t hi = f2bf(v);
              ph[(8 * (r / 4) + (r % 4)) * AP] = hi;
              pl[(8 * (r / 4) + (r % 4)) * AP] = f2bf(v - bf2f(hi));
            }
          } else {
            float *pc = C + rb * D + cl;
#pragma unroll
            for (int r = 0; r < 16; ++r) pc[(8 * (r / 4) + (r % 4)) * D] = acc[k][r] * inv;
          }
        }
      }
      __syncthreads();
    }

    // 4. power iteration (the start vector and its norm are in wbuf[0], nrm_part[0]).
    // w = C v with C the last A, normalised by the previous iterate's norm.  Wave w owns outputs
    // [D/8 w, D/8 (w + 1)); row r (16 lanes) of the wave owns NA = D/32 of
    // them, and lane l of the row the inputs 64 m + 4 l + t (m < D/64, t < 4),
    // with those C entries in registers.  A step reads the iterate in D/64
    // 16-byte loads a lane (one contiguous 256-byte span a row, the same for
    // the four rows), sums over the row with DPP moves and over the rows with
    // lane reads, and writes NA outputs and the wave's squared norm.
    constexpr int NA = D / 32, NM = D / 64;
    const int row = lane >> 4, l16 = lane & 15;
    const int o0 = wave * (D / 8) + row * NA;
    float cv[NM][4][NA];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int a2 = 0; a2 < NA; ++a2) cv[m][t][a2] = C[(64 * m + 4 * l16 + t) * D + o0 + a2];
    constexpr int NIT = PCA_ITERS >> PCA_SQUARINGS;
    static_assert(NIT << PCA_SQUARINGS == PCA_ITERS, "the squarings must divide the power iterations");
    for (int it = 0; it < NIT; ++it) {
      const int cur = it & 1, nxt = cur ^ 1;
      const float4 n0 = *(const float4 *)&nrm_part[cur][0], n1 = *(const float4 *)&nrm_part[cur][4];
      const float nrm2 = ((n0.x + n0.y) + (n0.z + n0.w)) + ((n1.x + n1.y) + (n1.z + n1.w));
      const float inv = nrm2 > 0.f ? rsqrtf(nrm2) : 0.f;  // only the direction matters
      float acc[NA];
#pragma unroll
      for (int a2 = 0; a2 < NA; ++a2) acc[a2] = 0.f;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const float4 x = *(const float4 *)&wbuf[cur][64 * m + 4 * l16];
#pragma unroll
        for (int a2 = 0; a2 < NA; ++a2) {
          acc[a2] = fmaf(cv[m][0][a2], x.x, acc[a2]);
          acc[a2] = fmaf(cv[m][1][a2], x.y, acc[a2]);
          acc[a2] = fmaf(cv[m][2][a2], x.z, acc[a2]);
          acc[a2] = fmaf(cv[m][3][a2], x.w, acc[a2]);
        }
      }
      float sq = 0.f;
#pragma unroll
      for (int a2 = 0; a2 < NA; ++a2) {
        acc[a2] = row16_sum(acc[a2]) * inv;
        sq = fmaf(acc[a2], acc[a2], sq);
      }
      const float tot = (lane_f32(sq, 0) + lane_f32(sq, 16)) + (lane_f32(sq, 32) + lane_f32(sq, 48));
      if (l16 == 0)
#pragma unroll
        for (int a2 = 0; a2 < NA; ++a2) wbuf[nxt][o0 + a2] = acc[a2];
      if (lane == 0) nrm_part[nxt][wave] = tot;
      __syncthreads();
    }
    // normalise and orient: the component of largest magnitude is positive
    if (wave == 0) {
      float nrm2 = 0.f;
#pragma unroll
      for (int w = 0; w < 8; ++w) nrm2 += nrm_part[NIT & 1][w];
      float best = -1.f, sgn = 1.f;
      int bi = 0;
      for (int i = lane; i < D; i += 64) {
        const float v = wbuf[NIT & 1][i];
        if (fabsf(v) > best) { best = fabsf(v); bi = i; sgn = v < 0.f ? -1.f : 1.f; }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(best, o, 64);
        const int oi2 = __shfl_xor(bi, o, 64);
        const float os = __shfl_xor(sgn, o, 64);
        if (ov > best || (ov == best && oi2 < bi)) { best = ov; bi = oi2; sgn = os; }
      }
      const bool zero = !(nrm2 > 0.f);
      const float scale = zero ? 0.f : sgn / sqrtf(nrm2);
      for (int i = lane; i < D; i += 64) {
        const float v = zero ? (i == 0 ? 1.f : 0.f) : wbuf[NIT & 1][i] * scale;
        mu[i] = v;  // the direction (the mean is no longer needed)
        if (a.dir) a.dir[((int64_t)h * a.ndir + node) * D + i] = v;
      }
    }
    __syncthreads();
    if (mode == 1) {
      for (int i = tid; i < D; i += NT) a.dbuf[((int64_t)h * pca_dir_cap(a.L) + blockIdx.x) * D + i] = mu[i];
      return;
    }
  }

  // 5. projections of every point (mode 0; mode 2 reads them)
  if (mode == 0) {
    constexpr int PL = D / 16;
    const int grp = tid >> 4, sub = tid & 15;
    float vv[PL];
#pragma unroll
    for (int k = 0; k < PL; ++k) vv[k] = mu[sub * PL + k];
    pca_project<D>(X, perm, tmp, key, vv, 0, n, grp, NT / 16, sub);
  }
  __syncthreads();

  // radix select of the nl-th smallest key (1-based rank nl)
  if (tid == 0) { sh_prefix = 0u; sh_rank = (uint32_t)nl; }
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int q = tid; q < 256; q += NT) hist[q] = 0u;
    __syncthreads();
    const uint32_t prefix = sh_prefix;
    const uint32_t hmask = shift == 24 ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (int p0 = tid; p0 < n; p0 += 8 * NT) {  // 8 loads in flight
      uint32_t kv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) kv[u] = p0 + u * NT < n ? key[p0 + u * NT] : 0u;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (p0 + u * NT < n && (kv[u] & hmask) == prefix) atomicAdd(&hist[(kv[u] >> shift) & 255u], 1u);
    }
    __syncthreads();
    // the first bin whose running count reaches the rank: lane l holds bins
    // 4l .. 4l+3, an inclusive scan over lanes finds the lane, the lane its bin
    if (wave == 0) {
      const uint4 hv = *(const uint4 *)&hist[4 * lane];
      const uint32_t cnt = (hv.x + hv.y) + (hv.z + hv.w);
      uint32_t inc = cnt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(inc, o, 64);
        if (lane >= o) inc += t;
      }
      const uint32_t rk = sh_rank;
      const uint64_t hit = __ballot(inc >= rk);
      // the prefix's keys number at least rk, so some lane hits; were none to,
      // the last bin is taken with every key counted, as a serial scan would
      const int f = hit ? __ffsll((long long)hit) - 1 : 63;
      if (lane == f) {
        const uint32_t hh[4] = {hv.x, hv.y, hv.z, hv.w};
        uint32_t run = inc - cnt;
        int bin = 255;
        if (hit) {
          for (int bb = 0; bb < 4; ++bb) {
            if (run + hh[bb] >= rk) { bin = 4 * lane + bb; break; }
            run += hh[bb];
          }
        } else {
          run = inc;
        }
        sh_prefix = prefix | ((uint32_t)bin << shift);
        sh_rank = rk - run;
      }
    }
    __syncthreads();
  }
  const uint32_t thr = sh_prefix;       // the nl-th smallest key
  const int eq_left = (int)sh_rank;     // keys equal to thr that still go left, in position order

  // stable partition: left = key < thr, or key == thr among the first eq_left
  // such positions.  A round takes 4 NT positions, 4 consecutive a thread.
  int base_left = 0, base_eq = 0;
  for (int c0 = 0; c0 < n; c0 += 4 * NT) {
    const int p0 = c0 + 4 * tid;
    uint32_t kv[4];
    int tv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      kv[u] = p0 + u < n ? key[p0 + u] : 0u;
      tv[u] = p0 + u < n ? tmp[p0 + u] : 0;
    }
    int nlt = 0, neq = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (p0 + u < n) {
        nlt += kv[u] < thr;
        neq += kv[u] == thr;
      }
    int2 tot;
    const int2 pre = block_scan2(nlt, neq, scan_sh, tot);
    const int room = max(eq_left - base_eq, 0);  // equal keys still admitted left
    int lt_run = pre.x, eq_run = pre.y;          // of this round, before the position
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = p0 + u;
      if (p < n) {
        const bool lt = kv[u] < thr, eq = kv[u] == thr;
        const bool left = lt || (eq && eq_run < room);
        const int left_before = base_left + lt_run + min(room, eq_run);
        perm[left ? left_before : nl + (p - left_before)] = tv[u];
        lt_run += lt;
        eq_run += eq;
      }
    }
    base_left += tot.x + min(room, tot.y);
    base_eq += tot.y;
  }
}

// The projections of a level run in three launches: block (node, chunk)
// projects PCA_PROJ_CHUNK of the node's points with the node's direction
// from a.dbuf.
template <int D>
__global__ __launch_bounds__(256) void k_pca_project(PcaArgs a, int first, int nchunk) {
  constexpr int PL = D / 16;
  const int h = blockIdx.y, nb = (int)blockIdx.x / nchunk, chunk = (int)blockIdx.x % nchunk;
  const int2 nd = a.nodes[first + nb];
  const int beg = chunk * PCA_PROJ_CHUNK, end = min(nd.y, beg + PCA_PROJ_CHUNK);
  if (beg >= end) return;
  const int64_t o = (int64_t)h * a.L + nd.x;
  const float *dir = a.dbuf + ((int64_t)h * pca_dir_cap(a.L) + nb) * D;
  const int grp = threadIdx.x >> 4, sub = threadIdx.x & 15;
  float vv[PL];
#pragma unroll
  for (int k = 0; k < PL; ++k) vv[k] = dir[sub * PL + k];
  pca_project<D>(a.X + (int64_t)h * a.L * D, a.perm + o, a.tmp + o, a.key + o, vv, beg, end, grp, 256 / 16, sub);
}

// Labels, segments and cluster count after the last level: the clusters are
// the consecutive runs of b positions (the last one ragged).
__global__ void k_pca_finish(const int *__restrict__ perm, int *__restrict__ labels, int *__restrict__ seg,
                             int *__restrict__ ncl, int L, int b, int segcap) {
  const int h = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int nc = (L + b - 1) / b;
  if (i < L) labels[(int64_t)h * L + perm[(int64_t)h * L + i]] = (int)(i / b);
  if (i <= segcap) seg[(int64_t)h * (segcap + 1) + i] = (int)min((int64_t)L, i * b);
  if (i == 0) ncl[h] = nc;
}

// Mean row of each cluster (fp64 sums in cluster order), stored fp32.
template <int D>
__global__ __launch_bounds__(256) void k_seg_rowmean(const uint16_t *__restrict__ X, const int *__restrict__ perm,
                                                     const int *__restrict__ seg, const int *__restrict__ ncl, int L,
                                                     int ncap, float *__restrict__ cent) {
  constexpr int PL = D / 16;
  typedef uint32_t pw_t __attribute__((ext_vector_type(PL / 2)));
  const int h = blockIdx.y, c = blockIdx.x;
  if (c >= ncap) return;
  float *out = cent + ((int64_t)h * ncap + c) * D;
  const int grp = threadIdx.x >> 4, sub = threadIdx.x & 15;
  __shared__ double sh[16][D];
  double acc[PL];
#pragma unroll
  for (int k = 0; k < PL; ++k) acc[k] = 0.0;
  int beg = 0, end = 0;
  if (c < ncl[h]) {
    const int *sg = seg + (int64_t)h * (ncap + 1);
    beg = sg[c];
    end = sg[c + 1];
  }
  const uint16_t *Xh = X + (int64_t)h * L * D;
  const int *ph = perm + (int64_t)h * L;
  for (int p = beg + grp; p < end; p += 16) {
    const pw_t xw = *(const pw_t *)(Xh + (int64_t)ph[p] * D + sub * PL);
#pragma unroll
    for (int k = 0; k < PL; ++k) acc[k] += (double)bf2f((uint16_t)((k & 1) ? (xw[k >> 1] >> 16) : (xw[k >> 1] & 0xFFFFu)));
  }
#pragma unroll
  for (int k = 0; k < PL; ++k) sh[grp][sub * PL + k] = acc[k];
  __syncthreads();
  for (int dd = threadIdx.x; dd < D; dd += 256) {
    double t = 0.0;
#pragma unroll
    for (int g = 0; g < 16; ++g) t += sh[g][dd];
    out[dd] = end > beg ? (float)(t / (double)(end - beg)) : 0.f;
  }
}

// perm[h] = 0 .. L-1
__global__ void k_iota_perm(int *__restrict__ perm, int L) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < L) perm[(int64_t)blockIdx.y * L + i] = (int)i;
}
// dst[h * dst_hs + i] = src[h * L + i]
__global__ void k_copy_rows_i32(const int *__restrict__ src, int *__restrict__ dst, int L, int64_t dst_hs) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < L) dst[(int64_t)blockIdx.y * dst_hs + i] = src[(int64_t)blockIdx.y * L + i];
}

// host
std::vector<int> pca_level_counts(int n, int b) {
  std::vector<int> counts;
  std::vector<std::pair<int, int>> cur, nxt;
  if (n > b) cur.push_back({0, n});
  while (!cur.empty()) {
    counts.push_back((int)cur.size());
    nxt.clear();
    for (auto &nd : cur) {
      const int nb = (nd.second + b - 1) / b, nl = b * ((nb + 1) / 2), nr = nd.second - nl;
      if (nl > b) nxt.push_back({nd.first, nl});
      if (nr > b) nxt.push_back({nd.first + nl, nr});
    }
    cur.swap(nxt);
  }
  return counts;
}

void launch_pca_split(int D, const PcaArgs &a, const std::vector<int> &counts, int BH, int *perm_trace,
                      hipStream_t st) {
  const int widest = counts.empty() ? 0 : *std::max_element(counts.begin(), counts.end());
  if (widest <= PCA_TREE_CAP)
    hipLaunchKernelGGL(k_pca_tree_wide, dim3(1), dim3(1024), 0, st, a.L, a.block, a.nodes, a.lvl);
  else
    hipLaunchKernelGGL(k_pca_tree, dim3(1), dim3(1), 0, st, a.L, a.block, a.nodes, a.lvl);
  hipLaunchKernelGGL(k_iota_perm, dim3((unsigned)((a.L + 255) / 256), (unsigned)BH), dim3(256), 0, st, a.perm, a.L);
  // dynamic LDS above the default limit (a refusal shows up as a launch error)
  static bool lds_set = hipFuncSetAttribute((const void *)k_pca_level<64>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                            pca_lds_max(64)) == hipSuccess &&
                        hipFuncSetAttribute((const void *)k_pca_level<128>,
                                            hipFuncAttributeMaxDynamicSharedMemorySize, pca_lds_max(128)) == hipSuccess;
  (void)lds_set;
  int first = 0;
  int nmax = a.L;  // largest node of the level: the left child is never the smaller one
  for (size_t l = 0; l < counts.size(); ++l) {
    // a chunk of the subsample (at most PCA_CHUNK points) sets the LDS row
    // stride; with the split squares the largest need is 69.6 KB at d = 128,
    // so every level fits two blocks a compute unit
    const int spad = (std::min(std::min(nmax, PCA_SMAX), PCA_CHUNK) + 15) & ~15;
    const int sp = spad + 8;
    const size_t lds = std::max((size_t)D * sp * 2, (size_t)D * (D + 8) * 4);
    const dim3 grid((unsigned)counts[l], (unsigned)BH);
    auto level = [&](int mode, size_t shm) {
      if (D == 64)
        hipLaunchKernelGGL(k_pca_level<64>, grid, dim3(512), shm, st, a, first, counts[l], sp, mode);
      else
        hipLaunchKernelGGL(k_pca_level<128>, grid, dim3(512), shm, st, a, first, counts[l], sp, mode);
    };
    if (nmax >= PCA_BIG_NODE && counts[l] <= pca_dir_cap(a.L)) {
      const int nchunk = (nmax + PCA_PROJ_CHUNK - 1) / PCA_PROJ_CHUNK;
      const dim3 pgrid((unsigned)(counts[l] * nchunk), (unsigned)BH);
      level(1, lds);
      if (D == 64)
        hipLaunchKernelGGL(k_pca_project<64>, pgrid, dim3(256), 0, st, a, first, nchunk);
      else
        hipLaunchKernelGGL(k_pca_project<128>, pgrid, dim3(256), 0, st, a, first, nchunk);
      level(2, 0);
    } else {
      level(0, lds);
    }
    const int nb = (nmax + a.block - 1) / a.block;
    nmax = a.block * ((nb + 1) / 2);
    if (perm_trace)
      hipLaunchKernelGGL(k_copy_rows_i32, dim3((unsigned)((a.L + 255) / 256), (unsigned)BH), dim3(256), 0, st, a.perm,
                         perm_trace + l * (int64_t)a.L, a.L, (int64_t)counts.size() * a.L);
    first += counts[l];
  }
}

void launch_pca_finish(const int *perm, int *labels, int *seg, int *ncl, int L, int b, int segcap, int BH,
                       hipStream_t st) {
  const int64_t n = std::max<int64_t>(L, (int64_t)segcap + 1);
  hipLaunchKernelGGL(k_pca_finish, dim3((unsigned)((n + 255) / 256), (unsigned)BH), dim3(256), 0, st, perm, labels,
                     seg, ncl, L, b, segcap);
}

void launch_seg_rowmean(int D, const uint16_t *X, const int *perm, const int *seg, const int *ncl, int L, int ncap,
                        float *cent, int BH, hipStream_t st) {
  if (D == 64)
    hipLaunchKernelGGL(k_seg_rowmean<64>, dim3((unsigned)ncap, (unsigned)BH), dim3(256), 0, st, X, perm, seg, ncl, L,
                       ncap, cent);
  else
    hipLaunchKernelGGL(k_seg_rowmean<128>, dim3((unsigned)ncap, (unsigned)BH), dim3(256), 0, st, X, perm, seg, ncl,
                       L, ncap, cent);
}

}  // namespace ac
