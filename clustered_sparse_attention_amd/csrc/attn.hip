// Cluster-routed block-sparse flash attention for gfx950.
//
// A block takes the query rows of one query cluster, 32 per wave (256 rows
// in 8 waves at d = 128; 384 in 12 waves at d = 64, whose registers allow
// three waves per SIMD), and walks the concatenation of the key clusters selected for that cluster in
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
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace ac {

// Per (head, query cluster): the key rows of its selection, concatenated in
// selection order (each cluster's members in counting-sort order), their
// count, and with compensation the logit bias of every key cluster's
// pseudo-key (log2 n_c for an excluded non-empty cluster, -inf otherwise).
// Fallback heads attend to every key and need no list.
__global__ __launch_bounds__(256) void k_attn_rows(AttnArgs a) {
  const int h = blockIdx.y, r = blockIdx.x;
  if (r >= a.ncl_q[h]) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool dense = a.all_dense || (a.fallback != nullptr && a.fallback[h] != 0);
  const int64_t rowi = (int64_t)h * a.nqcap + r;
  const int *segk = a.seg_k + (int64_t)h * (a.ncap + 1);
  if (dense) {
    if (tid == 0) a.rows_T[rowi] = a.L;
    return;
  }
  if (a.compensate) {
    const int ncl_k = a.ncl_k[h];
    for (int c = tid; c < ncl_k; c += 256) {
      const bool sel = (a.mask[rowi * a.mwords + (c >> 5)] >> (c & 31)) & 1u;
      const int cnt = segk[c + 1] - segk[c];
      a.pbias[rowi * a.pb_ld + c] = (sel || cnt <= 0) ? -__builtin_inff() : log2f((float)cnt);
    }
  }
  extern __shared__ int s_off[];  // [ncap + 1] first output position of each selected cluster
  __shared__ int scan[256];
  const int nsel = a.nsel[rowi];
  const int *lst = a.list + rowi * a.ncap;
  const int per = (nsel + 255) / 256;
  const int ib = min(nsel, tid * per), ie = min(nsel, ib + per);
  int loc = 0;
  for (int i = ib; i < ie; ++i) {
    const int c = lst[i];
    const int len = segk[c + 1] - segk[c];
    s_off[i] = len;
    loc += len;
  }
  scan[tid] = loc;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  int run = scan[tid] - loc;
  for (int i = ib; i < ie; ++i) {
    const int len = s_off[i];
    s_off[i] = run;
    run += len;
  }
  if (tid == 255) {
    s_off[nsel] = scan[255];
    a.rows_T[rowi] = scan[255];
  }
  __syncthreads();
  int *dst = a.rows + rowi * a.rows_ld;
  const int *permk = a.perm_k + (int64_t)h * a.L;
  for (int i = wave; i < nsel; i += 4) {
    const int c = lst[i];
    const int s0 = segk[c], len = segk[c + 1] - s0, o0 = s_off[i];
    for (int j = lane; j < len; j += 64) dst[o0 + j] = permk[s0 + j];
  }
}

// bf16 pseudo-keys / values, the first block of every query cluster, and the
// number of (query, key) pairs each head evaluates.
template <int D>
__global__ __launch_bounds__(256) void k_attn_prep(AttnArgs a, const float *__restrict__ kmean,
                                                   const float *__restrict__ vmean, uint16_t *__restrict__ kc,
                                                   uint16_t *__restrict__ vc, int *__restrict__ tile_off,
                                                   long long *__restrict__ pairs) {
  const int h = blockIdx.y, c = blockIdx.x;
  if (c < a.ncap && a.compensate) {
    const int64_t o = ((int64_t)h * a.ncap + c) * D;
    for (int dd = threadIdx.x; dd < D; dd += 256) {
      kc[o + dd] = f2bf(kmean[o + dd]);
      vc[o + dd] = f2bf(vmean[o + dd]);
    }
  }
  if (c == 0 && threadIdx.x == 0) {
    const int *sq = a.seg_q + (int64_t)h * (a.nqcap + 1);
    int *to = tile_off + (int64_t)h * (a.nqcap + 1);
    const int nq = a.ncl_q[h];
    int run = 0;
    long long pr = 0;
    for (int r = 0; r <= a.nqcap; ++r) {
      to[r] = run;
      if (r < nq) {
        const int cnt = sq[r + 1] - sq[r];
        run += (cnt + att_qt<D>() - 1) / att_qt<D>();
        pr += (long long)cnt * (long long)a.rows_T[(int64_t)h * a.nqcap + r];
      }
    }
    pairs[h] = pr;
  }
}

// LDS tile layouts.  K and V tiles are written by direct global->LDS loads
// (16 bytes per lane, lane i at base + 16 i), so rows are unpadded; the
// 16-byte chunks of each row are XOR-permuted instead, chunk c of row R at
// slot c ^ swz(R), which makes the MFMA operand reads conflict-free:
//  K (row-major, read 16 bytes per lane, 16 rows x one chunk per quarter
//    wave): swz = R mod 16 (D = 128) or (R / 2) mod 8 (D = 64);
//  V (row-major, read transposed with ds_read_b64_tr_b16, 4 rows x 4 chunks
//    per half wave): swz = 4 (R mod 4) (D = 128) or 4 ((R / 2) mod 2) (D = 64).
template <int D> AC_DEV int kswz(int R) { return D == 128 ? (R & 15) : ((R >> 1) & 7); }
template <int D> AC_DEV int vswz(int R) { return D == 128 ? 4 * (R & 3) : 4 * ((R >> 1) & 1); }

// One 16-byte-per-lane global->LDS load (lane i lands at lds + 16 i).  It is
// issued from inline assembly so that the compiler does not tie every later
// LDS read to its completion: the kernel waits for these loads itself, at
// the end of each tile, before the barrier that publishes the buffer.
AC_DEV void dma16(const uint16_t *src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(lds), "v"(src) : "memory", "m0");
}
// s_waitcnt vmcnt(N) alone: the N most recent vector memory operations may
// still be in flight (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt and
// lgkmcnt at their maxima).
template <int N> AC_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
AC_DEV uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void *)p);
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
#define AC_LDS(T, p) ((__attribute__((address_space(3))) T *)(p))

// One block: QT queries of one query cluster, NW waves of QG groups of 32
// queries.  Every K or V fragment a wave reads from LDS feeds QG products,
// so LDS traffic per product falls with QG.  The K and V tiles are loaded by
// the first LW waves (all of them at d = 128, 8 of 12 at d = 64).
template <int D, int QG>
__global__ __launch_bounds__(64 * att_qt<D>() / (32 * QG), 1) void k_attn(AttnArgs a) {
  constexpr int QT = att_qt<D>();             // query rows per block
  constexpr int KSQ = D / 16;                 // k-steps of the QK product
  constexpr int DB = D / 32;                  // 32-dim blocks of O
  constexpr int NC = D / 8;                   // 16-byte chunks per row
  constexpr int RPI = 64 / NC;                // rows per 64-lane global->LDS load
  constexpr int NW = QT / (32 * QG);          // waves
  constexpr int LW = ATT_KT / RPI < NW ? ATT_KT / RPI : NW;  // waves that load tiles
  constexpr int IPW = ATT_KT / RPI / LW;      // such loads per loading wave, per tensor and tile
  constexpr int TILE = ATT_KT * D;            // elements per tile
  constexpr int NST = 4;                      // K / V tile buffers
  constexpr int VPM = 8 / DB;                 // weights computed after each PV product
  static_assert(IPW >= 1 && IPW * RPI * LW == ATT_KT, "tile load split");
  // XCD-aware order: the hardware deals consecutive block ids round-robin to
  // the 8 XCDs.  Work items (head-major query tiles) are cut into chunks of
  // ATT_XCD_CHUNK and chunk k goes to XCD k % 8, so the few query tiles of a
  // query cluster (which stream the same key list) mostly share one XCD's
  // L2, while every XCD gets an even share of every head (heads can differ
  // in cost by the density factor when some fall back to dense).
  const int x = (int)(blockIdx.x % 8), j = (int)(blockIdx.x / 8);
  const int w = ((j / ATT_XCD_CHUNK) * 8 + x) * ATT_XCD_CHUNK + j % ATT_XCD_CHUNK;
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
  const int qbeg = segq[r] + (blk - toff[r]) * QT;
  const int qend = segq[r + 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;

  __shared__ __align__(1024) uint16_t Kb[NST * TILE], Vb[NST * TILE];
  __shared__ __align__(16) int ring[8][2 * ATT_KT];      // raw rows and pseudo-key biases of a tile, by tile mod 8
  __shared__ __align__(16) float sbias[NW][4][ATT_KT];   // per wave: key biases / scale, by tile mod 4

  const bool dense = a.all_dense || (a.fallback != nullptr && a.fallback[h] != 0);
  const int64_t rowi = (int64_t)h * a.nqcap + r;
  const int T = dense ? a.L : a.rows_T[rowi];
  const bool comp = !dense && a.compensate;
  const int ncl_k = a.ncl_k[h];
  // tiles 0..nt0-1 walk the selected keys, nt0..ntiles-1 the pseudo-keys
  const int nt0 = (T + ATT_KT - 1) / ATT_KT;
  const int ntiles = nt0 + (comp ? (ncl_k + ATT_KT - 1) / ATT_KT : 0);
  const int *rl = a.rows + rowi * a.rows_ld;
  const float *pbr = a.pbias + rowi * a.pb_ld;
  const int last_row_tile = max(nt0 - 1, 0);
  const int last_pb_tile = max((a.ncap + ATT_KT - 1) / ATT_KT - 1, 0);

  // Q fragments of this wave's QG x 32 queries (B operands of S^T = K Q^T)
  const bool wave_active = qbeg + wave * 32 * QG < qend;
  bool qvalid[QG];
  int64_t qrow[QG];
  bf16x8_t qf[QG][KSQ];
#pragma unroll
  for (int gq = 0; gq < QG; ++gq) {
    const int qi = qbeg + (wave * QG + gq) * 32 + l32;
    qvalid[gq] = qi < qend;
    qrow[gq] = qvalid[gq] ? (int64_t)a.perm_q[(int64_t)h * a.L + qi] : 0;
    const uint16_t *qr = a.Q + ((int64_t)h * a.L + qrow[gq]) * D;
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks)
      qf[gq][ks] = qvalid[gq] ? *(const bf16x8_t *)&qr[ks * 16 + g * 8] : (bf16x8_t){};
  }

  f32x16_t acc_o[QG][DB];
  float m_i[QG], l_i[QG], alpha[QG];
#pragma unroll
  for (int gq = 0; gq < QG; ++gq) {
#pragma unroll
    for (int db = 0; db < DB; ++db) acc_o[gq][db] = (f32x16_t){};
    m_i[gq] = -__builtin_inff();
    l_i[gq] = 0.f;
    alpha[gq] = 1.f;  // rescale of O still to apply before the next PV product
  }
  const float sl2 = a.scale_log2;
  const float inv_sl2 = 1.f / sl2;

  const char *Kh = (const char *)(a.K + (int64_t)h * a.L * D);
  const char *Vh = (const char *)(a.V + (int64_t)h * a.L * D);
  const char *Kc = (const char *)(a.kc + (int64_t)h * a.ncap * D);
  const char *Vc = (const char *)(a.vc + (int64_t)h * a.ncap * D);

  // Every global->LDS load of the loop is issued from inline assembly and the
  // loop holds no other global memory access, so the kernel alone decides
  // when to wait for them.  The row list and pseudo-key biases of a tile go
  // to a small LDS ring (wave 0, 32 lanes x 16 bytes) five tiles ahead.
  auto ring_load = [&](int tt) {
    if (wave == 0 && lane < 32) {
      const int tr = min(tt, last_row_tile);
      const int tp = min(max(tt - nt0, 0), last_pb_tile);
      const int *src = lane < 16 ? rl + tr * ATT_KT + 4 * lane : (const int *)pbr + tp * ATT_KT + 4 * (lane - 16);
      dma16((const uint16_t *)src, lds_addr(&ring[tt & 7][0]));
    }
  };
  // final row (-1: masked) of key `lane` of tile tt from the ring; its logit
  // bias, divided by the base-2 score scale so that it adds to the raw
  // product, goes to this wave's bias rows
  float *sbw = &sbias[wave][0][0];
  auto commit = [&](int tt) -> int {
    const bool ph1 = tt >= nt0;
    const int o = (ph1 ? tt - nt0 : tt) * ATT_KT + lane;
    const int total = ph1 ? ncl_k : T;
    const int raw = ring[tt & 7][lane];
    const float braw = __int_as_float(ring[tt & 7][ATT_KT + lane]);
    int rw = (ph1 || dense) ? o : raw;
    float bias = ph1 ? braw * inv_sl2 : 0.f;
    if (o >= total) { rw = -1; bias = -__builtin_inff(); }
    sbw[(tt & 3) * ATT_KT + lane] = bias;
    return rw;
  };
  // The swizzles depend on the row only modulo 16, and a lane's row moves by
  // NW * RPI (a multiple of 16) from one load to the next, so its source
  // chunk byte offset is fixed.
  static_assert((LW * RPI) % 16 == 0, "swizzle period");
  const uint32_t koff = 16u * (uint32_t)((lane % NC) ^ kswz<D>(wave * RPI + lane / NC));
  const uint32_t voff = 16u * (uint32_t)((lane % NC) ^ vswz<D>(wave * RPI + lane / NC));
  // one tensor of tile tt into buffer `buf`: loading wave w < LW writes rows
  // [RPI*(LW*ii+w), +RPI); rows come from the wave's index registers by shuffle
  auto dma = [&](bool vpart, int tt, int rwv, int buf) {
    const bool ph1 = tt >= nt0;
    const char *src = vpart ? (ph1 ? Vc : Vh) : (ph1 ? Kc : Kh);
    const uint32_t off = vpart ? voff : koff;
    const uint16_t *dst = (vpart ? Vb : Kb) + buf * TILE;
    if (wave >= LW) return;
#pragma unroll
    for (int ii = 0; ii < IPW; ++ii) {
      const int I = ii * LW + wave;
      const int R = I * RPI + lane / NC;
      const uint32_t rw = (uint32_t)max(__shfl(rwv, R, 64), 0);  // masked keys read row 0; their bias is -inf
      dma16((const uint16_t *)(src + (rw * (uint32_t)(2 * D) + off)), lds_addr(dst + I * 512));
    }
  };

  // key slot l32 of each 32-key block holds tile key 16*(a/2) + 8*gg + 4*(a%2) + b, l32 = 8a + 4gg + b
  const int kslot = 16 * ((l32 >> 3) >> 1) + 8 * ((l32 >> 2) & 1) + 4 * ((l32 >> 3) & 1) + (l32 & 3);
  const int kx = kswz<D>(kslot);  // the same for kslot + 32
  // transposed V reads: lane (i = lane % 16, half hd of the 32 dims, key half g)
  const int vi = lane & 15, vhd = (lane >> 4) & 1;
  const int vrow = 8 * g + (vi >> 2);                   // + 16 s + 4 u
  const int vxq = vswz<D>(vrow) >> 2;                   // row-dependent chunk flip (bits 2-3)
  const int vc2 = 2 * vhd + ((vi & 3) >> 1);            // chunk within the 4-chunk (32-dim) group
  const int vhalf = 4 * (vi & 1);

  // S^T = K Q^T for one tile: two 32-key blocks per query group; each K
  // fragment feeds the QG groups.  The accumulators start at the keys' logit
  // biases divided by the base-2 score scale (0 for selected keys, -inf for
  // masked ones, ln n_c / scale for pseudo-keys), so every tile takes the
  // same path and the scores need no separate add.
  auto qk = [&](const uint16_t *Ks, const float *bz, f32x16_t (*acc)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const f32x4_t b0 = *(const f32x4_t *)&bz[32 * kb + 16 * half + 8 * g];
        const f32x4_t b1 = *(const f32x4_t *)&bz[32 * kb + 16 * half + 8 * g + 4];
#pragma unroll
        for (int gq = 0; gq < QG; ++gq)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[gq][kb][half * 8 + i] = b0[i];
            acc[gq][kb][half * 8 + 4 + i] = b1[i];
          }
      }
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8_t kf = *(const bf16x8_t *)&Ks[(32 * kb + kslot) * D + (((2 * ks + g) ^ kx) << 3)];
#pragma unroll
        for (int gq = 0; gq < QG; ++gq)
          acc[gq][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[gq][ks], acc[gq][kb], 0, 0, 0);
      }
    // order: the bias reads and the K reads of two k-steps, then each
    // k-step's two products followed by the K reads of the step two ahead
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
#pragma unroll
    for (int ks = 0; ks < KSQ - 2; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * QG, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * QG, 0);
  };
  // row max of a tile in base-2 units: a tree of three-way maxima, then the
  // two key halves of the column exchanged between lane halves
  auto tile_max = [&](const f32x16_t *acc) -> float {
    float part[2] = {-__builtin_inff(), -__builtin_inff()};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      part[0] = fmaxf(part[0], acc[0][i]);
      part[1] = fmaxf(part[1], acc[1][i]);
    }
    const float mt = fmaxf(part[0], part[1]) * sl2;
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  };
  // the V^T operands of k-step s of a tile, one per 32-dim block
  auto v_frags = [&](const uint16_t *Vs, int s, bf16x8_t *vf) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int ch = (4 * (db ^ vxq) + vc2) << 3;
      const uint16_t *v0 = &Vs[(16 * s + vrow) * D + ch + vhalf];
      const i16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(AC_LDS(i16x4_t, v0));
      const i16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(AC_LDS(i16x4_t, v0 + 4 * D));
      const i16x4_t cat[2] = {lo4, hi4};
      vf[db] = *(const bf16x8_t *)cat;
    }
  };
  const bf16x2_t ones = {(__bf16)1.f, (__bf16)1.f};
  // O^T += V^T P^T for every query group over the 4 k-steps of a tile
  auto pv_all = [&](const uint16_t *Vs, const bf16x8_t (*pw)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bf16x8_t vf[DB];
      v_frags(Vs, q, vf);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int gq = 0; gq < QG; ++gq)
          acc_o[gq][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db], pw[gq][q], acc_o[gq][db], 0, 0, 0);
    }
  };

  // Pipeline.  K of tile t + 3 and V of tile t + 2 are loaded while tile t
  // is computed, into four buffers each (buffer t mod 4): K_t is read in
  // iteration t and V_t in iteration t + 1, so every load has two to three
  // iterations to land.  The row ring runs five tiles ahead.  Tiles past the
  // end are loaded from clamped, in-bounds rows and never used, which keeps
  // the number of loads per iteration fixed.  Each wave runs the PV product
  // one tile behind the scores: iteration t computes S_t = K_t Q^T and its
  // row max, then alternates the PV steps of tile t - 1 with the weights of
  // S_t, so the softmax's vector work issues while the products run.
#pragma unroll
  for (int i = 0; i < 5; ++i) ring_load(i);
  // V buffer 3 stands for "tile -1" in the first iteration: zeros (times
  // zero weights), never uninitialised LDS
  for (int e = tid; e < TILE / 8; e += 64 * NW) *(u32x4_t *)&Vb[3 * TILE + 8 * e] = (u32x4_t){0u, 0u, 0u, 0u};
  __builtin_amdgcn_s_waitcnt(0);  // the ring, the Q fragments and the scalars above have landed
  __syncthreads();
  int rw_next;  // rows of tile tt + 2, committed one iteration earlier (its K load went then)
  {
    const int rw0 = commit(0);
    const int rw1 = commit(1);
    rw_next = commit(2);
    dma(false, 0, rw0, 0);
    dma(true, 0, rw0, 0);
    dma(false, 1, rw1, 1);
    dma(true, 1, rw1, 1);
    dma(false, 2, rw_next, 2);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  bf16x8_t pb[QG][4];  // weights of the previous tile, the B operands of its PV steps
#pragma unroll
  for (int gq = 0; gq < QG; ++gq)
#pragma unroll
    for (int q = 0; q < 4; ++q) pb[gq][q] = (bf16x8_t){};
  for (int tt = 0; tt < ntiles; ++tt) {
    const int b0 = tt & 3;
    const int rw = commit(tt + 3);  // its ring slot landed by the last barrier
    ring_load(tt + 5);
    dma(false, tt + 3, rw, (tt + 3) & 3);      // K buffer of tile tt - 1, read last iteration
    dma(true, tt + 2, rw_next, (tt + 2) & 3);  // V buffer of tile tt - 2, read last iteration
    rw_next = rw;
    if (wave_active) {
      bool any = false;
#pragma unroll
      for (int gq = 0; gq < QG; ++gq) any = any || alpha[gq] != 1.f;
      if (__ballot(any)) {  // O follows the reference max set last iteration (rare)
#pragma unroll
        for (int gq = 0; gq < QG; ++gq)
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) acc_o[gq][db][jj] *= alpha[gq];
      }
      f32x16_t sc[QG][2];
      qk(Kb + b0 * TILE, sbw + (tt & 3) * ATT_KT, sc);
      // lazy rescale: the reference max m_i may trail the running max by up
      // to 2^8, so p <= 256; it moves only when a row outgrows it.
      float m_new[QG], m_use[QG];
#pragma unroll
      for (int gq = 0; gq < QG; ++gq) {
        const float mt = tile_max(sc[gq]);
        m_new[gq] = mt > m_i[gq] + 8.f ? mt : m_i[gq];
        m_use[gq] = m_new[gq] == -__builtin_inff() ? 0.f : m_new[gq];
      }
      // the PV steps of the previous tile (zero weights before the first)
      // alternate with the weights of this one: after each product, VPM
      // weights of the same step, so the vector work issues while the
      // products run.  The V^T operands of a step are read one step ahead.
      // At d = 128 the wave takes issue priority over its SIMD partner for
      // this phase (measured: about 2 % shorter; no gain at d = 64, where the
      // vector work dominates).
      if constexpr (D == 128) __builtin_amdgcn_s_setprio(1);
      const uint16_t *Vp = Vb + ((tt - 1) & 3) * TILE;
      float lt[QG];
#pragma unroll
      for (int gq = 0; gq < QG; ++gq) lt[gq] = 0.f;
      bf16x8_t vcur[DB], vnext[DB];
      v_frags(Vp, 0, vcur);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q + 1 < 4) v_frags(Vp, q + 1, vnext);
        bf16x8_t t[QG];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int gq = 0; gq < QG; ++gq) {
            acc_o[gq][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vcur[db], pb[gq][q], acc_o[gq][db], 0, 0, 0);
#pragma unroll
            for (int u = 0; u < VPM; ++u) {
              const int i = db * VPM + u;
              t[gq][i] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sc[gq][q >> 1][(q & 1) * 8 + i], sl2, -m_use[gq]));
            }
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
        for (int gq = 0; gq < QG; ++gq) {
          lt[gq] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(t[gq], t[gq], 0, 1), ones, lt[gq], false);
          lt[gq] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(t[gq], t[gq], 2, 3), ones, lt[gq], false);
          lt[gq] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(t[gq], t[gq], 4, 5), ones, lt[gq], false);
          lt[gq] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(t[gq], t[gq], 6, 7), ones, lt[gq], false);
          pb[gq][q] = t[gq];
        }
        if (q + 1 < 4)
#pragma unroll
          for (int db = 0; db < DB; ++db) vcur[db] = vnext[db];
      }
      if constexpr (D == 128) __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int gq = 0; gq < QG; ++gq) {
        alpha[gq] = m_i[gq] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m_i[gq] - m_new[gq]);
        l_i[gq] = fmaf(l_i[gq], alpha[gq], lt[gq]);
        m_i[gq] = m_new[gq];
      }
    }
    // K of tile tt + 1 and V of tile tt (issued two iterations ago) and the
    // ring slot of tile tt + 4 (wave 0, last iteration) have landed; the loads
    // issued after that ring load may still be in flight.  The barrier makes
    // them visible and frees the K buffer of tile tt and the V buffer of
    // tile tt - 1.
    if (wave == 0) wait_vmcnt<4 * IPW + 1>();
    else wait_vmcnt<4 * IPW>();
    __syncthreads();
  }
  // the last tile's PV product; no load targets its buffer
  if (wave_active && ntiles > 0) {
#pragma unroll
    for (int gq = 0; gq < QG; ++gq)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) acc_o[gq][db][jj] *= alpha[gq];
    pv_all(Vb + ((ntiles - 1) & 3) * TILE, pb);
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load may still write LDS when the block ends

#pragma unroll
  for (int gq = 0; gq < QG; ++gq) {
    const float lsum = l_i[gq] + __shfl_xor(l_i[gq], 32, 64);
    if (!qvalid[gq]) continue;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    uint16_t *orow = a.O + ((int64_t)h * a.L + qrow[gq]) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const int d0 = 32 * db + 8 * jq + 4 * g;
        uint32_t w0 = (uint32_t)f2bf(acc_o[gq][db][jq * 4 + 0] * inv) |
                      ((uint32_t)f2bf(acc_o[gq][db][jq * 4 + 1] * inv) << 16);
        uint32_t w1 = (uint32_t)f2bf(acc_o[gq][db][jq * 4 + 2] * inv) |
                      ((uint32_t)f2bf(acc_o[gq][db][jq * 4 + 3] * inv) << 16);
        *(u32x2_t *)&orow[d0] = (u32x2_t){w0, w1};
      }
    if (a.lse != nullptr && g == 0)
      a.lse[(int64_t)h * a.L + qrow[gq]] =
          lsum > 0.f ? (m_i[gq] + log2f(lsum)) * 0.69314718055994530942f : -__builtin_inff();
  }
}

void launch_attn_prep(int D, const AttnArgs &a, const float *kmean, const float *vmean, uint16_t *kc, uint16_t *vc,
                      int *tile_off, long long *pairs, int BH, hipStream_t st) {
  hipLaunchKernelGGL(k_attn_rows, dim3((unsigned)a.nqcap, (unsigned)BH), dim3(256), (size_t)(a.ncap + 1) * sizeof(int),
                     st, a);
  dim3 grid(a.compensate ? a.ncap : 1, BH);
  if (D == 64)
    hipLaunchKernelGGL(k_attn_prep<64>, grid, dim3(256), 0, st, a, kmean, vmean, kc, vc, tile_off, pairs);
  else
    hipLaunchKernelGGL(k_attn_prep<128>, grid, dim3(256), 0, st, a, kmean, vmean, kc, vc, tile_off, pairs);
}

void launch_attn(int D, const AttnArgs &a, int BH, int max_blocks, hipStream_t st) {
  AttnArgs aa = a;
  aa.blocks_per_head = max_blocks;
  aa.BH = BH;
  const long long total = ((long long)max_blocks * BH + 8 * ATT_XCD_CHUNK - 1) / (8 * ATT_XCD_CHUNK) *
                          (8 * ATT_XCD_CHUNK);  // whole chunks on all 8 XCDs
  if (D == 64)
    hipLaunchKernelGGL((k_attn<64, ATT_QG>), dim3((unsigned)total), dim3(64 * att_qt<64>() / (32 * ATT_QG)), 0, st, aa);
  else
    hipLaunchKernelGGL((k_attn<128, ATT_QG>), dim3((unsigned)total), dim3(64 * att_qt<128>() / (32 * ATT_QG)), 0, st, aa);
}

}  // namespace ac
