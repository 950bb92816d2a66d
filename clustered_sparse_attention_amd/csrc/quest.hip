// Per-token Quest scores for gfx950: every query token against every key
// cluster, the literal shape of AdaCluster Algorithm 2 (one score per query
// row and key column, the key side reduced to clusters), each entry the
// Quest bound of eq. (1):
//   S[i, c] = sum_d max(q_i[d] * kmax_c[d], q_i[d] * kmin_c[d]).
//
// Two engines compute the same numbers:
//  * TensorQuest (eq. (2) with the per-cluster max / min vectors as the key
//    operands): S = [q+, q-] . [kmax; kmin]^T, one bf16 MFMA product with
//    contraction 2d.  q is bf16, so q+ and q- are exact bf16 values and every
//    product is exact in fp32; only the fp32 accumulation rounds.
//  * Quest on the vector ALUs, eq. (1) per dimension as written: two
//    products, a max and an add per (token, cluster, dimension).  It is the
//    baseline the pages compare TensorQuest against.
#include "common.h"
#include "internal.h"

namespace ac {

namespace {

constexpr int TQ_THREADS = 512;  // 8 waves x 32 tokens
constexpr int TQ_TOK = 256;      // tokens per block
constexpr int TQ_CT = 64;        // key clusters per LDS tile

template <int D>
struct TqTile {
  static constexpr int ROWB = 4 * D + 16;         // bytes per cluster row: kmax | kmin (bf16), 16 B pad
  static constexpr int CHUNKS = TQ_CT * (D / 4);  // 16-byte chunks per tile
  static constexpr int PER_THREAD = (CHUNKS + TQ_THREADS - 1) / TQ_THREADS;
};

// 16-byte chunk j of a tile: cluster j / (D/4), within it the kmax half for
// the first D/8 chunks, then the kmin half.
template <int D>
AC_DEV u32x4_t tq_load_chunk(const TokQuestArgs &a, int h, int ct, int j, int nk) {
  const int cl = j / (D / 4), cc = j % (D / 4);
  const int c = ct * TQ_CT + cl;
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (c < nk) {
    const uint16_t *src = cc < D / 8 ? a.kmax : a.kmin;
    const int e = (cc % (D / 8)) * 8;
    v = *(const u32x4_t *)(src + ((int64_t)h * a.ncap + c) * D + e);
  }
  return v;
}

// S^T = [kmax; kmin] . [q+, q-]^T with v_mfma_f32_32x32x16_bf16: the A
// operand is 32 key clusters (lane -> cluster l % 32, read from the LDS
// tile), the B operand 32 tokens (lane -> token l % 32, held in registers).
// Accumulator register j of lane l then holds token l % 32 and cluster
// 8 (j / 4) + 4 (l / 32) + j % 4.  Each wave stages its 32 x 64 block of a
// tile in LDS and writes it back row by row, 16 lanes per token row, so
// every store instruction writes 256 contiguous bytes of 4 rows.
template <int D>
__global__ __launch_bounds__(TQ_THREADS, 1) void k_tq_mfma(TokQuestArgs a) {
  using T = TqTile<D>;
  constexpr int NS = D / 16;  // k-steps of 16 per half of the contraction
  constexpr int NSUB = TQ_CT / 32;
  constexpr int SROW = TQ_CT + 4;  // staging row (floats), padded against bank conflicts
  __shared__ __attribute__((aligned(16))) unsigned char tile[2][TQ_CT * T::ROWB];
  __shared__ __attribute__((aligned(16))) float stage[TQ_THREADS / 64][32 * SROW];
  __shared__ int live_s[2][TQ_CT];  // cluster of the tile is non-empty and below ncl
  const int h = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g = lane >> 5;
  const int tok0 = blockIdx.x * TQ_TOK + wave * 32;
  const int ncl = a.ncl[h];
  const int nk = min(min(ncl, a.ld), a.ncap);  // clusters that get a score
  const int ntiles = (nk + TQ_CT - 1) / TQ_CT;
  const int *seg = a.seg + (int64_t)h * (a.ncap + 1);
  float *Sh = a.S + (int64_t)h * a.L * a.ld;
  const bool vec = (a.ld & 3) == 0;
  float *st = stage[wave];

  // B operand: token l32 of the wave's 32, k-chunk g; q+ keeps the
  // non-negative halves, q- the negative ones (bf16 sign bit).
  bf16x8_t qp[NS], qm[NS];
  {
    const int row = min(tok0 + l32, a.L - 1);
    const uint16_t *qr = a.Q + ((int64_t)h * a.L + row) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const u32x4_t x = *(const u32x4_t *)(qr + 16 * s + 8 * g);
      u32x4_t p, m;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t sgn = (x[e] >> 15) & 0x00010001u;
        const uint32_t neg = sgn * 0xFFFFu;  // 0xFFFF in each negative half
        m[e] = x[e] & neg;
        p[e] = x[e] & ~neg;
      }
      qp[s] = __builtin_bit_cast(bf16x8_t, p);
      qm[s] = __builtin_bit_cast(bf16x8_t, m);
    }
  }

  u32x4_t pre[T::PER_THREAD];
  int pre_live = 0;
  auto fetch = [&](int ct) {
#pragma unroll
    for (int i = 0; i < T::PER_THREAD; ++i) {
      const int j = tid + i * TQ_THREADS;
      if (j < T::CHUNKS) pre[i] = tq_load_chunk<D>(a, h, ct, j, nk);
    }
    if (tid < TQ_CT) {
      const int c = ct * TQ_CT + tid;
      pre_live = c < nk && seg[c + 1] > seg[c];
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < T::PER_THREAD; ++i) {
      const int j = tid + i * TQ_THREADS;
      if (j < T::CHUNKS) *(u32x4_t *)(tile[buf] + (j / (D / 4)) * T::ROWB + (j % (D / 4)) * 16) = pre[i];
    }
    if (tid < TQ_CT) live_s[buf][tid] = pre_live;
  };

  if (ntiles > 0) {
    fetch(0);
    stash(0);
  }
  __syncthreads();
  for (int ct = 0; ct < ntiles; ++ct) {
    const int buf = ct & 1;
    if (ct + 1 < ntiles) fetch(ct + 1);
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      const unsigned char *arow = tile[buf] + (sub * 32 + l32) * T::ROWB + 16 * g;
      f32x16_t acc = {};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8_t k = *(const bf16x8_t *)(arow + 32 * s);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k, qp[s], acc, 0, 0, 0);
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8_t k = *(const bf16x8_t *)(arow + 2 * D + 32 * s);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k, qm[s], acc, 0, 0, 0);
      }
      // token l32, clusters sub*32 + 8q + 4g + e
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cl = sub * 32 + 8 * q + 4 * g;
        f32x4_t v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = live_s[buf][cl + e] ? acc[4 * q + e] : -__builtin_inff();
        *(f32x4_t *)(st + l32 * SROW + cl) = v;
      }
    }
    // the next tile goes to the other buffer; one barrier publishes it and
    // the staged scores (this wave reads only its own staging rows)
    if (ct + 1 < ntiles) stash(buf ^ 1);
    __syncthreads();
    // rows of the staged block: token 4i + lane / 16, clusters 4 (lane % 16) ..
    const int c = ct * TQ_CT + 4 * (lane & 15);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tr = 4 * i + (lane >> 4), t = tok0 + tr;
      const f32x4_t v = *(const f32x4_t *)(st + tr * SROW + 4 * (lane & 15));
      if (t < a.L) {
        float *dst = Sh + (int64_t)t * a.ld + c;
        if (vec && c + 3 < a.ld) {
          *(f32x4_t *)dst = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (c + e < a.ld) dst[e] = v[e];
        }
      }
    }
  }
  // columns past the last scored tile
  const int t = tok0 + l32;
  if (t < a.L)
    for (int c = ntiles * TQ_CT + g; c < a.ld; c += 2) Sh[(int64_t)t * a.ld + c] = -__builtin_inff();
}

constexpr int TQV_THREADS = 256;  // one token per lane
constexpr int TQV_CT = 16;        // key clusters per LDS tile

template <int D>
__global__ __launch_bounds__(TQV_THREADS) void k_tq_valu(TokQuestArgs a) {
  __shared__ __attribute__((aligned(16))) float kt[TQV_CT][2][D];
  const int h = blockIdx.y, tid = threadIdx.x;
  const int tok = blockIdx.x * TQV_THREADS + tid;
  const int ncl = a.ncl[h];
  const int nk = min(min(ncl, a.ld), a.ncap);
  const int ntiles = (nk + TQV_CT - 1) / TQV_CT;
  const int *seg = a.seg + (int64_t)h * (a.ncap + 1);
  float *Srow = a.S + ((int64_t)h * a.L + min(tok, a.L - 1)) * a.ld;
  float q[D];
  {
    const uint16_t *qr = a.Q + ((int64_t)h * a.L + min(tok, a.L - 1)) * D;
#pragma unroll
    for (int e = 0; e < D; e += 8) {
      const u32x4_t x = *(const u32x4_t *)(qr + e);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        q[e + 2 * u] = __uint_as_float(x[u] << 16);
        q[e + 2 * u + 1] = __uint_as_float(x[u] & 0xFFFF0000u);
      }
    }
  }
  for (int ct = 0; ct < ntiles; ++ct) {
    __syncthreads();
    for (int i = tid; i < TQV_CT * 2 * D; i += TQV_THREADS) {
      const int cl = i / (2 * D), half = (i / D) & 1, e = i % D;
      const int c = ct * TQV_CT + cl;
      const uint16_t *src = half ? a.kmin : a.kmax;
      kt[cl][half][e] = c < nk ? bf2f(src[((int64_t)h * a.ncap + c) * D + e]) : 0.f;
    }
    __syncthreads();
#pragma unroll 1
    for (int cl = 0; cl < TQV_CT; ++cl) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < D; e += 4) {
        const f32x4_t mx = *(const f32x4_t *)&kt[cl][0][e];
        const f32x4_t mn = *(const f32x4_t *)&kt[cl][1][e];
#pragma unroll
        for (int u = 0; u < 4; ++u) acc += fmaxf(q[e + u] * mx[u], q[e + u] * mn[u]);
      }
      const int c = ct * TQV_CT + cl;
      if (tok < a.L && c < a.ld) Srow[c] = (c < ncl && seg[c + 1] > seg[c]) ? acc : -__builtin_inff();
    }
  }
  if (tok < a.L)
    for (int c = ntiles * TQV_CT; c < a.ld; ++c) Srow[c] = -__builtin_inff();
}

}  // namespace

void launch_token_quest(int D, const TokQuestArgs &a, int engine, int BH, hipStream_t st) {
  if (engine == 0) {
    const dim3 grid((unsigned)((a.L + TQ_TOK - 1) / TQ_TOK), (unsigned)BH);
    if (D == 64) hipLaunchKernelGGL(k_tq_mfma<64>, grid, dim3(TQ_THREADS), 0, st, a);
    else hipLaunchKernelGGL(k_tq_mfma<128>, grid, dim3(TQ_THREADS), 0, st, a);
  } else {
    const dim3 grid((unsigned)((a.L + TQV_THREADS - 1) / TQV_THREADS), (unsigned)BH);
    if (D == 64) hipLaunchKernelGGL(k_tq_valu<64>, grid, dim3(TQV_THREADS), 0, st, a);
    else hipLaunchKernelGGL(k_tq_valu<128>, grid, dim3(TQV_THREADS), 0, st, a);
  }
}

}  // namespace ac
