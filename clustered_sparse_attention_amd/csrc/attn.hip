// Cluster-routed block-sparse flash attention for gfx950.
//
// A block takes ATT_QT = 128 queries of one query cluster (4 waves x 32) and
// walks the concatenation of the key clusters selected for that cluster in
// tiles of 64 keys.  Tiles may span cluster boundaries, so each (query tile,
// selection) has a single ragged tail however small the clusters are.  Rows
// are gathered through the counting-sort permutations inside the kernel; the
// output is scattered back to original token order.  With compensation the
// non-empty excluded clusters follow as pseudo-keys (key mean, value mean,
// logit bias log2 n_c in base-2 units); fallback heads attend to all keys.
//
// MFMA layout (v_mfma_f32_32x32x16_bf16, 64 lanes, g = lane / 32):
//   S^T = K . Q^T: A = K rows (lane -> key slot), B = Q (lane -> query),
//   accumulator lane l holds query l % 32 and 16 keys of each 32-key block,
//   register j <-> key 16*(j/8) + 8*g + (j%8) (the K rows are loaded in that
//   order).  Those 8-register halves are exactly the B operand of
//   O^T = V^T . P^T for 16 contiguous keys, and V^T comes from a transposed
//   LDS tile with one 16-byte read per lane and k-step.
#include "common.h"
#include "internal.h"

namespace ac {

template <int D>
__global__ __launch_bounds__(256) void k_attn_prep(AttnArgs a, const float *__restrict__ kmean,
                                                   const float *__restrict__ vmean, uint16_t *__restrict__ kc,
                                                   uint16_t *__restrict__ vc, float *__restrict__ lb,
                                                   int *__restrict__ tile_off, const int *__restrict__ seltok,
                                                   long long *__restrict__ pairs) {
  const int h = blockIdx.y, c = blockIdx.x;
  if (c < a.ncap && a.compensate) {
    const int64_t o = ((int64_t)h * a.ncap + c) * D;
    for (int dd = threadIdx.x; dd < D; dd += 256) {
      kc[o + dd] = f2bf(kmean[o + dd]);
      vc[o + dd] = f2bf(vmean[o + dd]);
    }
    if (threadIdx.x == 0) {
      const int *seg = a.seg_k + (int64_t)h * (a.ncap + 1);
      const int cnt = c < a.ncl_k[h] ? seg[c + 1] - seg[c] : 0;
      lb[(int64_t)h * a.ncap + c] = cnt > 0 ? log2f((float)cnt) : -__builtin_inff();
    }
  }
  if (c == 0 && threadIdx.x == 0) {
    const int *sq = a.seg_q + (int64_t)h * (a.nqcap + 1);
    int *to = tile_off + (int64_t)h * (a.nqcap + 1);
    const int nq = a.ncl_q[h];
    const bool dense = a.all_dense || (a.fallback != nullptr && a.fallback[h] != 0);
    int run = 0;
    long long pr = 0;
    for (int r = 0; r <= a.nqcap; ++r) {
      to[r] = run;
      if (r < nq) {
        const int cnt = sq[r + 1] - sq[r];
        run += (cnt + ATT_QT - 1) / ATT_QT;
        pr += (long long)cnt * (dense ? (long long)a.L : (long long)seltok[(int64_t)h * a.nqcap + r]);
      }
    }
    pairs[h] = pr;
  }
}

template <int D>
__global__ __launch_bounds__(256, 2) void k_attn(AttnArgs a) {
  constexpr int KSQ = D / 16;        // k-steps of the QK product
  constexpr int DB = D / 32;         // 32-dim blocks of O
  constexpr int KROW = D + 8;        // padded K row (bf16)
  constexpr int VROW = ATT_KT + 8;   // padded V^T row (keys)
  // XCD-aware order: the hardware deals consecutive block ids round-robin to
  // the 8 XCDs, so id -> work item w = (id % 8) * (N / 8) + id / 8 hands each
  // XCD a contiguous run of work items; the query tiles of one query cluster
  // (which stream the same key list) then share that XCD's L2.
  const int nper = gridDim.x / 8;
  const int w = (int)(blockIdx.x % 8) * nper + (int)(blockIdx.x / 8);
  const int h = w / a.blocks_per_head;
  const int blk = w % a.blocks_per_head;
  if (h >= a.BH) return;
  const int nq = a.ncl_q[h];
  const int *toff = a.tile_off + (int64_t)h * (a.nqcap + 1);
  if (nq <= 0 || blk >= toff[nq]) return;
  int lo = 0, hi = nq;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (toff[mid] <= blk) lo = mid; else hi = mid;
  }
  const int r = lo;
  const int *segq = a.seg_q + (int64_t)h * (a.nqcap + 1);
  const int qbeg = segq[r] + (blk - toff[r]) * ATT_QT;
  const int qend = segq[r + 1];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g = lane >> 5;

  __shared__ uint16_t Ks[ATT_KT * KROW];
  __shared__ uint16_t Vt[D * VROW];
  __shared__ __align__(16) float sbias[4][3][ATT_KT];
  extern __shared__ int dyn[];
  int *s_cum = dyn;                       // [ncap + 1]
  int *s_start = dyn + (a.ncap + 1);      // [ncap]
  uint32_t *s_mask = (uint32_t *)(dyn + 2 * a.ncap + 1);  // [mwords]

  const bool dense = a.all_dense || (a.fallback != nullptr && a.fallback[h] != 0);
  const int64_t rowi = (int64_t)h * a.nqcap + r;
  int nsel = 0;
  int T;
  if (!dense) {
    nsel = a.nsel[rowi];
    const int *lst = a.list + rowi * a.ncap;
    const int *segk = a.seg_k + (int64_t)h * (a.ncap + 1);
    const int per = (nsel + 255) / 256;
    const int ib = min(nsel, tid * per), ie = min(nsel, ib + per);
    int loc = 0;
    for (int i = ib; i < ie; ++i) {
      int c = lst[i];
      int s0 = segk[c];
      s_start[i] = s0;
      s_cum[i] = segk[c + 1] - s0;  // length for now
      loc += s_cum[i];
    }
    __shared__ int scan[256];
    scan[tid] = loc;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      int v = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    int run = scan[tid] - loc;
    for (int i = ib; i < ie; ++i) {
      int len = s_cum[i];
      s_cum[i] = run;
      run += len;
    }
    if (tid == 255) s_cum[nsel] = scan[255];
    if (a.compensate)
      for (int w = tid; w < a.mwords; w += 256) s_mask[w] = a.mask[rowi * a.mwords + w];
    __syncthreads();
    T = s_cum[nsel];
  } else {
    T = a.L;
  }

  // Q fragments of this wave's 32 queries (B operand of S^T = K Q^T)
  const int qi = qbeg + wave * 32 + l32;
  const bool qvalid = qi < qend;
  const int64_t qrow = qvalid ? (int64_t)a.perm_q[(int64_t)h * a.L + qi] : 0;
  bf16x8_t qf[KSQ];
  {
    const uint16_t *qr = a.Q + ((int64_t)h * a.L + qrow) * D;
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks)
      qf[ks] = qvalid ? *(const bf16x8_t *)&qr[ks * 16 + g * 8] : (bf16x8_t){};
  }

  f32x16_t acc_o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc_o[db] = (f32x16_t){};
  float m_i = -__builtin_inff();
  float l_i = 0.f;
  const float sl2 = a.scale_log2;

  const uint16_t *Kh = a.K + (int64_t)h * a.L * D;
  const uint16_t *Vh = a.V + (int64_t)h * a.L * D;
  const uint16_t *Kc = a.kc + (int64_t)h * a.ncap * D;
  const uint16_t *Vc = a.vc + (int64_t)h * a.ncap * D;
  const int *permk = a.perm_k + (int64_t)h * a.L;
  const int ncl_k = a.ncl_k[h];
  const bool comp = !dense && a.compensate;
  // tiles 0..nt0-1 walk the selected keys, nt0..ntiles-1 the pseudo-keys
  const int nt0 = (T + ATT_KT - 1) / ATT_KT;
  const int ntiles = nt0 + (comp ? (ncl_k + ATT_KT - 1) / ATT_KT : 0);

  // Key index pipeline, run by every wave for itself: lane l finds the row
  // of key l of a tile (and its logit bias) two tiles ahead.  The loads it
  // needs are unconditional and their results are first used at the end of
  // the iteration, so their latency hides behind the tile's MFMAs.  Tiles
  // advance monotonically through the selection, so a cursor replaces a
  // search: the cluster holding a key is found by stepping forward from the
  // cluster that held the previous tile's last key.
  int cur = 0;
  auto index_issue = [&](int tt, int &raw, float &braw) {
    const bool ph1 = tt >= nt0;
    const int o = (ph1 ? tt - nt0 : tt) * ATT_KT + lane;
    int pos = min(o, a.L - 1);
    if (!ph1 && !dense) {
      const int oc = min(o, T - 1);
      int c = cur;
      while (c + 1 < nsel && s_cum[c + 1] <= oc) ++c;
      pos = s_start[c] + (oc - s_cum[c]);
      cur = __shfl(c, 63, 64);
    }
    raw = permk[pos];
    braw = comp ? a.lb[(int64_t)h * a.ncap + min(o, a.ncap - 1)] : 0.f;
  };
  // final row (-1: masked) and bias of key `lane` of tile tt
  auto index_commit = [&](int tt, int raw, float braw, float *bias_dst) -> int {
    const bool ph1 = tt >= nt0;
    const int o = (ph1 ? tt - nt0 : tt) * ATT_KT + lane;
    const int total = ph1 ? ncl_k : T;
    int rw = ph1 ? o : (dense ? o : raw);
    float bias = 0.f;
    if (ph1) {
      const bool selected = (s_mask[min(o, a.ncap - 1) >> 5] >> (o & 31)) & 1u;
      bias = selected ? -__builtin_inff() : braw;
    }
    if (o >= total) { rw = -1; bias = -__builtin_inff(); }
    bias_dst[lane] = bias;
    return rw;
  };

  constexpr int KCH = (ATT_KT * D / 8) / 256;      // 16-byte K pieces per thread
  constexpr int VCH = (ATT_KT / 2 * D / 8) / 256;  // V key pairs x 8 dims per thread
  u32x4_t kreg[KCH], vreg[VCH][2];
  // rows come from lane (key) of this wave's index registers
  auto load_tile = [&](int tt, int rwv) {
    const bool ph1 = tt >= nt0;
    const uint16_t *Kp = ph1 ? Kc : Kh;
    const uint16_t *Vp = ph1 ? Vc : Vh;
#pragma unroll
    for (int it = 0; it < KCH; ++it) {
      const int q = tid + it * 256;
      const int rr = q / (D / 8), cc = (q % (D / 8)) * 8;
      const int rw = max(__shfl(rwv, rr, 64), 0);  // masked keys (-1) read row 0: their bias is -inf
      kreg[it] = *(const u32x4_t *)&Kp[(int64_t)rw * D + cc];
    }
#pragma unroll
    for (int it = 0; it < VCH; ++it) {
      const int q = tid + it * 256;
      const int kp = q % (ATT_KT / 2), dc = q / (ATT_KT / 2);
      const int r0 = max(__shfl(rwv, 2 * kp, 64), 0), r1 = max(__shfl(rwv, 2 * kp + 1, 64), 0);
      vreg[it][0] = *(const u32x4_t *)&Vp[(int64_t)r0 * D + dc * 8];
      vreg[it][1] = *(const u32x4_t *)&Vp[(int64_t)r1 * D + dc * 8];
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int it = 0; it < KCH; ++it) {
      const int q = tid + it * 256;
      const int rr = q / (D / 8), cc = (q % (D / 8)) * 8;
      *(u32x4_t *)&Ks[rr * KROW + cc] = kreg[it];
    }
#pragma unroll
    for (int it = 0; it < VCH; ++it) {
      const int q = tid + it * 256;
      const int kp = q % (ATT_KT / 2), dc = q / (ATT_KT / 2);
      const uint16_t *e0 = (const uint16_t *)&vreg[it][0];
      const uint16_t *e1 = (const uint16_t *)&vreg[it][1];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *(uint32_t *)&Vt[(dc * 8 + i) * VROW + 2 * kp] = (uint32_t)e0[i] | ((uint32_t)e1[i] << 16);
    }
  };

  float *sbw = &sbias[wave][0][0];  // this wave's bias rows, one per tile mod 3
  int rw_next = -1;                 // row of key `lane` of tile tt + 1
  if (ntiles > 0) {
    int raw;
    float braw;
    index_issue(0, raw, braw);
    const int rw0 = index_commit(0, raw, braw, sbw);
    if (ntiles > 1) {
      index_issue(1, raw, braw);
      rw_next = index_commit(1, raw, braw, sbw + ATT_KT);
    }
    load_tile(0, rw0);
  }

  // key slot l32 of each 32-key block holds tile key 16*(a/2) + 8*gg + 4*(a%2) + b, l32 = 8a + 4gg + b
  const int kslot = 16 * ((l32 >> 3) >> 1) + 8 * ((l32 >> 2) & 1) + 4 * ((l32 >> 3) & 1) + (l32 & 3);

  for (int tt = 0; tt < ntiles; ++tt) {
    __syncthreads();  // the previous tile is consumed
    store_tile();
    __syncthreads();
    if (tt + 1 < ntiles) load_tile(tt + 1, rw_next);  // in flight during this tile's MFMAs
    const bool idx_next = tt + 2 < ntiles;
    int pend_raw = 0;
    float pend_b = 0.f;
    if (idx_next) index_issue(tt + 2, pend_raw, pend_b);

    // S^T for two 32-key blocks (the two accumulation chains interleaved)
    f32x16_t acc_s[2];
    acc_s[0] = (f32x16_t){};
    acc_s[1] = (f32x16_t){};
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8_t kf = *(const bf16x8_t *)&Ks[(32 * kb + kslot) * KROW + ks * 16 + g * 8];
        acc_s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], acc_s[kb], 0, 0, 0);
      }
    }
    // scores in base-2 units: s * scale * log2(e) + bias.  Full tiles of
    // selected keys carry no bias: the row max is taken on the raw products
    // and the scale and max subtraction fold into one FMA per score.
    // Tail and pseudo-key tiles add the bias (-inf masked, log2 n_c).
    const bool biased = tt >= nt0 - 1;
    float mt = -__builtin_inff();
    if (biased) {
      const float *bz = sbw + (tt % 3) * ATT_KT;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const f32x4_t b0 = *(const f32x4_t *)&bz[32 * kb + 16 * half + 8 * g];
          const f32x4_t b1 = *(const f32x4_t *)&bz[32 * kb + 16 * half + 8 * g + 4];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float sv = fmaf(acc_s[kb][half * 8 + i], sl2, i < 4 ? b0[i] : b1[i - 4]);
            acc_s[kb][half * 8 + i] = sv;
            mt = fmaxf(mt, sv);
          }
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mt = fmaxf(mt, acc_s[kb][j]);
      mt *= sl2;
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    // lazy rescale: the reference max m_i may trail the running max by up to
    // 2^8, so p <= 256; O and l are rescaled only when a row outgrows that
    if (__ballot(mt > m_i + 8.f)) {
      const float m_new = fmaxf(m_i, mt);
      const float alpha = m_i == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m_i - m_new);
      l_i *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc_o[db][j] *= alpha;
      m_i = m_new;
    }
    const float m_use = m_i == -__builtin_inff() ? 0.f : m_i;
    // biased: exp2(s - m); unbiased: exp2(acc * sl2 - m) as one FMA
    const float mul = biased ? 1.f : sl2;
    float psum = 0.f;
    bf16x8_t pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        bf16x8_t t;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(acc_s[kb][half * 8 + i], mul, -m_use));
          psum += pv;
          t[i] = (__bf16)pv;
        }
        pb[kb * 2 + half] = t;
      }
    l_i += psum;
    // O^T += V^T P^T over 4 k-steps of 16 keys
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int kbase = 16 * s + 8 * g;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8_t vf = *(const bf16x8_t *)&Vt[(32 * db + l32) * VROW + kbase];
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[s], acc_o[db], 0, 0, 0);
      }
    }
    if (idx_next) rw_next = index_commit(tt + 2, pend_raw, pend_b, sbw + ((tt + 2) % 3) * ATT_KT);
  }

  const float lsum = l_i + __shfl_xor(l_i, 32, 64);
  if (!qvalid) return;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  uint16_t *orow = a.O + ((int64_t)h * a.L + qrow) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      const int d0 = 32 * db + 8 * jq + 4 * g;
      uint32_t w0 = (uint32_t)f2bf(acc_o[db][jq * 4 + 0] * inv) | ((uint32_t)f2bf(acc_o[db][jq * 4 + 1] * inv) << 16);
      uint32_t w1 = (uint32_t)f2bf(acc_o[db][jq * 4 + 2] * inv) | ((uint32_t)f2bf(acc_o[db][jq * 4 + 3] * inv) << 16);
      *(u32x2_t *)&orow[d0] = (u32x2_t){w0, w1};
    }
  if (a.lse != nullptr && g == 0)
    a.lse[(int64_t)h * a.L + qrow] = lsum > 0.f ? (m_i + log2f(lsum)) * 0.69314718055994530942f : -__builtin_inff();
}

void launch_attn_prep(int D, const AttnArgs &a, const float *kmean, const float *vmean, uint16_t *kc, uint16_t *vc,
                      float *lb, int *tile_off, const int *seltok, long long *pairs, int BH, hipStream_t st) {
  dim3 grid(a.compensate ? a.ncap : 1, BH);
  if (D == 64)
    hipLaunchKernelGGL(k_attn_prep<64>, grid, dim3(256), 0, st, a, kmean, vmean, kc, vc, lb, tile_off, seltok, pairs);
  else
    hipLaunchKernelGGL(k_attn_prep<128>, grid, dim3(256), 0, st, a, kmean, vmean, kc, vc, lb, tile_off, seltok, pairs);
}

void launch_attn(int D, const AttnArgs &a, int BH, int max_blocks, hipStream_t st) {
  size_t dyn = (size_t)(2 * a.ncap + 1 + a.mwords) * sizeof(int);
  AttnArgs aa = a;
  aa.blocks_per_head = max_blocks;
  aa.BH = BH;
  const long long total = ((long long)max_blocks * BH + 7) / 8 * 8;  // a multiple of the 8 XCDs
  if (D == 64)
    hipLaunchKernelGGL(k_attn<64>, dim3((unsigned)total), dim3(256), dyn, st, aa);
  else
    hipLaunchKernelGGL(k_attn<128>, dim3((unsigned)total), dim3(256), dyn, st, aa);
}

}  // namespace ac
