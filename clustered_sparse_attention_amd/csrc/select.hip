// Cluster scoring and key-cluster selection for gfx950.
//
// Scores: AdaCluster eq. (1) (Quest bound of a key cluster for a query-
// cluster centre) evaluated as one bf16 MFMA product with contraction length
// 6*D: the query side [c+, c-] is split into three bf16 terms each (hi, mid,
// lo; their sum reproduces the fp32 centre), the key side repeats the exact
// bf16 max / min vectors.  Mean scoring uses the same product with both
// sides split.  Selection: a bitonic sort of each row in LDS by (score desc,
// index asc), then the TOPK / DENSITY / TOPP prefix.
#include "common.h"
#include "internal.h"

namespace ac {

template <int D>
__global__ __launch_bounds__(256) void k_score_prep_a(ScoreArgs a) {
  const int h = blockIdx.y, r = blockIdx.x;
  uint16_t *A = a.A + ((int64_t)h * a.nq_pad + r) * (6 * D);
  for (int dd = threadIdx.x; dd < D; dd += 256) {
    uint16_t t[6] = {0, 0, 0, 0, 0, 0};
    if (r < a.nq) {
      float v = a.cq[((int64_t)h * a.nqcap + r) * D + dd];
      if (a.mode == 0) {
        float vp = v > 0.f ? v : 0.f, vm = v < 0.f ? v : 0.f;
        split3(vp, t[0], t[1], t[2]);
        split3(vm, t[3], t[4], t[5]);
      } else {
        uint16_t hh, mm, ll;
        split3(v, hh, mm, ll);
        t[0] = hh; t[1] = hh; t[2] = hh; t[3] = mm; t[4] = mm; t[5] = ll;
      }
    }
#pragma unroll
    for (int k = 0; k < 6; ++k) A[k * D + dd] = t[k];
  }
}

template <int D>
__global__ __launch_bounds__(256) void k_score_prep_b(ScoreArgs a) {
  const int h = blockIdx.y, c = blockIdx.x;
  uint16_t *B = a.Bm + ((int64_t)h * a.ncap_pad + c) * (6 * D);
  const bool live = c < a.ncl_k[h] && c < a.ncap;
  for (int dd = threadIdx.x; dd < D; dd += 256) {
    uint16_t t[6] = {0, 0, 0, 0, 0, 0};
    if (live) {
      const int64_t o = ((int64_t)h * a.ncap + c) * D + dd;
      if (a.mode == 0) {
        uint16_t mx = a.kmax[o], mn = a.kmin[o];
        t[0] = mx; t[1] = mx; t[2] = mx; t[3] = mn; t[4] = mn; t[5] = mn;
      } else {
        uint16_t hh, mm, ll;
        split3(a.kmean[o], hh, mm, ll);
        t[0] = hh; t[1] = mm; t[2] = ll; t[3] = hh; t[4] = mm; t[5] = hh;
      }
    }
#pragma unroll
    for (int k = 0; k < 6; ++k) B[k * D + dd] = t[k];
  }
}

// S[r, c] = A[r] . B[c] with 16x16x32 MFMA.  A wave computes a 32 x 32 block
// (2 x 2 tiles of 16 x 16: each A and B fragment it loads feeds two
// products), four waves a 32 x 128 block.
template <int D>
__global__ __launch_bounds__(256) void k_score_gemm(ScoreArgs a) {
  constexpr int KD = 6 * D;
  const int h = blockIdx.z;
  const int r0 = blockIdx.y * 32;
  const int c0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 32;
  const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
  if (c0 >= a.ncap_pad || r0 >= a.nq_pad) return;
  // a row or column tile beyond the padded extent reads row 0 and is not stored
  const bool rv1 = r0 + 16 < a.nq_pad, cv1 = c0 + 16 < a.ncap_pad;
  const uint16_t *A0 = a.A + ((int64_t)h * a.nq_pad + r0 + l16) * KD;
  const uint16_t *A1 = a.A + ((int64_t)h * a.nq_pad + (rv1 ? r0 + 16 : 0) + l16) * KD;
  const uint16_t *B0 = a.Bm + ((int64_t)h * a.ncap_pad + c0 + l16) * KD;
  const uint16_t *B1 = a.Bm + ((int64_t)h * a.ncap_pad + (cv1 ? c0 + 16 : 0) + l16) * KD;
  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int ks = 0; ks < KD / 32; ++ks) {
    const bf16x8_t a0 = *(const bf16x8_t *)&A0[ks * 32 + g * 8], a1 = *(const bf16x8_t *)&A1[ks * 32 + g * 8];
    const bf16x8_t b0 = *(const bf16x8_t *)&B0[ks * 32 + g * 8], b1 = *(const bf16x8_t *)&B1[ks * 32 + g * 8];
    acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0, acc[0][0], 0, 0, 0);
    acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b1, acc[0][1], 0, 0, 0);
    acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b0, acc[1][0], 0, 0, 0);
    acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, acc[1][1], 0, 0, 0);
  }
  const int *seg = a.seg_k + (int64_t)h * (a.ncap + 1);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = c0 + 16 * j + l16;
    if (c >= a.ncap) continue;
    const bool live = c < a.ncl_k[h] && seg[c + 1] > seg[c];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = r0 + 16 * i + g * 4 + q;
        if (r < a.nq) a.S[((int64_t)h * a.nqcap + r) * a.ncap + c] = live ? acc[i][j][q] : -__builtin_inff();
      }
  }
}

// ---------------------------------------------------------------------------
// Selection, one block per (query cluster, head).
__global__ __launch_bounds__(256) void k_select(SelectArgs a) {
  const int h = blockIdx.y, r = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t rowi = (int64_t)h * a.nqcap + r;
  int *list = a.list + rowi * a.ncap;
  uint32_t *mask = a.mask + rowi * a.mwords;
  __shared__ unsigned long long keys[SEL_MAXN];
  __shared__ uint32_t smask[SEL_MAXN / 32];
  __shared__ double part[256];
  __shared__ int sh_n;
  __shared__ int sh_valid;

  const int ncl = a.ncl_k[h];
  const int *seg = a.seg_k + (int64_t)h * (a.ncap + 1);
  for (int w = tid; w < a.mwords; w += 256) smask[w] = 0;
  if (r >= a.ncl_q[h]) {
    __syncthreads();
    for (int w = tid; w < a.mwords; w += 256) mask[w] = 0;
    if (tid == 0) { a.nsel[rowi] = 0; a.seltok[rowi] = 0; }
    return;
  }
  int P = 64;
  while (P < ncl) P <<= 1;
  const float *S = a.S + rowi * a.ncap;
  int nv_local = 0;
  for (int c = tid; c < P; c += 256) {
    unsigned long long k = ~0ull;
    if (c < ncl && seg[c + 1] > seg[c]) {
      k = ((unsigned long long)(~f2ord(S[c])) << 32) | (unsigned)c;
      nv_local++;
    }
    keys[c] = k;
  }
  // count of valid entries
  part[tid] = (double)nv_local;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) part[tid] += part[tid + off];
    __syncthreads();
  }
  if (tid == 0) sh_valid = (int)part[0];
  __syncthreads();
  const int nvalid = sh_valid;
  // bitonic sort, ascending
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      // compare-exchange pair q: i has bit j clear, partner i + j
      for (int q = tid; q < P / 2; q += 256) {
        const int i = 2 * q - (q & (j - 1)), ixj = i + j;
        unsigned long long x = keys[i], y = keys[ixj];
        bool up = (i & k) == 0;
        if ((x > y) == up) { keys[i] = y; keys[ixj] = x; }
      }
      __syncthreads();
    }
  }
  // cutoff
  int nsel = 0;
  if (a.mode == 0) {
    nsel = min(max(a.topk, 1), nvalid);
  } else if (a.mode == 3) {
    nsel = nvalid;
  } else {
    // chunked prefix over the sorted valid entries
    const int per = (nvalid + 255) / 256;
    const int ib = min(nvalid, tid * per), ie = min(nvalid, ib + per);
    double mx = 0.0;
    double zs[16];  // per <= SEL_MAXN / 256 = 16
    if (a.mode == 2) {
      // TOPP: logits rho * S * scale + ln n_c, max-subtracted, fp64
      double lmax = -INFINITY;
      for (int i = ib; i < ie; ++i) {
        int c = (int)(keys[i] & 0xffffffffu);
        double z = (double)a.rho[rowi] * (double)S[c] * (double)a.scale + log((double)(seg[c + 1] - seg[c]));
        zs[i - ib] = z;
        lmax = fmax(lmax, z);
      }
      part[tid] = lmax;
      __syncthreads();
      for (int off = 128; off > 0; off >>= 1) {
        if (tid < off) part[tid] = fmax(part[tid], part[tid + off]);
        __syncthreads();
      }
      mx = part[0];
      __syncthreads();
    }
    double loc = 0.0;
    for (int i = ib; i < ie; ++i) {
      int c = (int)(keys[i] & 0xffffffffu);
      double v = a.mode == 1 ? (double)(seg[c + 1] - seg[c]) : exp(zs[i - ib] - mx);
      if (a.mode == 2) zs[i - ib] = v;
      loc += v;
    }
    part[tid] = loc;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      double v = tid >= off ? part[tid - off] : 0.0;
      __syncthreads();
      part[tid] += v;
      __syncthreads();
    }
    const double total = part[255];
    const double target = a.mode == 1 ? ceil((double)a.param * (double)a.L) : (double)a.param * total;
    if (tid == 0) sh_n = nvalid;
    __syncthreads();
    const double excl = tid > 0 ? part[tid - 1] : 0.0;
    if (ie > ib && part[tid] >= target && excl < target) {
      double run = excl;
      int found = ie - 1;
      for (int i = ib; i < ie; ++i) {
        int c = (int)(keys[i] & 0xffffffffu);
        run += a.mode == 1 ? (double)(seg[c + 1] - seg[c]) : zs[i - ib];
        if (run >= target) { found = i; break; }
      }
      sh_n = found + 1;
    }
    __syncthreads();
    nsel = min(max(sh_n, 1), nvalid);
  }
  // outputs
  int tok_local = 0;
  for (int i = tid; i < nsel; i += 256) {
    int c = (int)(keys[i] & 0xffffffffu);
    list[i] = c;
    atomicOr(&smask[c >> 5], 1u << (c & 31));
    tok_local += seg[c + 1] - seg[c];
  }
  part[tid] = (double)tok_local;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) part[tid] += part[tid + off];
    __syncthreads();
  }
  for (int w = tid; w < a.mwords; w += 256) mask[w] = smask[w];
  if (tid == 0) {
    a.nsel[rowi] = nsel;
    a.seltok[rowi] = (int)part[0];
  }
}

void launch_score(int D, const ScoreArgs &a, int BH, hipStream_t st) {
  if (D == 64) {
    hipLaunchKernelGGL(k_score_prep_a<64>, dim3(a.nq_pad, BH), dim3(256), 0, st, a);
    hipLaunchKernelGGL(k_score_prep_b<64>, dim3(a.ncap_pad, BH), dim3(256), 0, st, a);
    hipLaunchKernelGGL(k_score_gemm<64>, dim3((a.ncap_pad / 32 + 4) / 4, (a.nq_pad + 31) / 32, BH), dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL(k_score_prep_a<128>, dim3(a.nq_pad, BH), dim3(256), 0, st, a);
    hipLaunchKernelGGL(k_score_prep_b<128>, dim3(a.ncap_pad, BH), dim3(256), 0, st, a);
    hipLaunchKernelGGL(k_score_gemm<128>, dim3((a.ncap_pad / 32 + 4) / 4, (a.nq_pad + 31) / 32, BH), dim3(256), 0, st, a);
  }
}

void launch_select(const SelectArgs &a, int BH, hipStream_t st) {
  hipLaunchKernelGGL(k_select, dim3(a.nqcap, BH), dim3(256), 0, st, a);
}

}  // namespace ac
