// Tail merging of query clusters ("iCATS: Fast Video Generation via
// Interaction-Aware Sparse Attention and Timestep-Adaptive Sparsity",
// method section, tail-merging design, and its worked example).
//
// Per head, one block plans both passes over the query clusters' key
// masks (exact merge of identical masks, then mutual Hamming-nearest pairs
// whose tails fit one query block); a second kernel moves every token to
// its place in the new cluster order, and a third writes the new masks and
// selection lists.  Plan, per head, as 8 arrays of nq + 1 ints:
//   rep  cluster whose token list absorbs this one in pass 1 (itself if none)
//   pre  tokens of earlier members of the same pass-1 group
//   gsz  size of a pass-1 group (at its representative)
//   cut  tail moved away by a donor (0 otherwise)
//   rcv  receiver of a donor (-1 otherwise)
//   gets donor whose tail a receiver takes (-1 otherwise)
//   nseg first position of every new cluster (nq + 1 entries)
//   nn   nearest tail cluster of pass 2 (-1 if none)
#include <climits>

#include "common.h"
#include "internal.h"

namespace ac {

enum { TM_REP, TM_PRE, TM_GSZ, TM_CUT, TM_RCV, TM_GETS, TM_NSEG, TM_NN, TM_ARRAYS };

AC_DEV bool same_mask(const uint32_t *a, const uint32_t *b, int words) {
  for (int w = 0; w < words; ++w)
    if (a[w] != b[w]) return false;
  return true;
}
AC_DEV int hamming(const uint32_t *a, const uint32_t *b, int words) {
  int d = 0;
  for (int w = 0; w < words; ++w) d += __popc(a[w] ^ b[w]);
  return d;
}

__global__ __launch_bounds__(256) void k_tm_plan(TailArgs t) {
  const int h = blockIdx.x, tid = threadIdx.x;
  const int nq = t.ncl[h];
  const int S = t.nq + 1;
  extern __shared__ int sm[];
  int *sz = sm, *rep = sm + S, *pre = sm + 2 * S, *gsz = sm + 3 * S, *cut = sm + 4 * S, *rcv = sm + 5 * S,
      *gets = sm + 6 * S, *nseg = sm + 7 * S, *nn = sm + 8 * S;
  const int *seg = t.seg_in + (int64_t)h * S;
  const uint32_t *mk = t.mask_in + (int64_t)h * t.nq * t.mwords;
  const int mw = t.mwords, B = t.block;
  for (int r = tid; r < S; r += 256) {
    sz[r] = r < nq ? seg[r + 1] - seg[r] : 0;
    cut[r] = 0;
    rcv[r] = -1;
    gets[r] = -1;
    gsz[r] = 0;
    nn[r] = -1;
  }
  __syncthreads();
  // pass 1: the lowest non-empty cluster with the same mask absorbs this one
  for (int r = tid; r < nq; r += 256) {
    int g = r;
    if (sz[r] > 0)
      for (int q = 0; q < r; ++q)
        if (sz[q] > 0 && same_mask(mk + (int64_t)q * mw, mk + (int64_t)r * mw, mw)) { g = q; break; }
    rep[r] = g;
  }
  __syncthreads();
  for (int r = tid; r < nq; r += 256) {
    const int g = rep[r];
    int p = 0, s = 0;
    for (int q = 0; q < nq; ++q)
      if (rep[q] == g && sz[q] > 0) {
        if (q < r) p += sz[q];
        s += sz[q];
      }
    pre[r] = p;
    if (g == r && sz[r] > 0) gsz[r] = s;
  }
  __syncthreads();
  // pass 2: nearest neighbour among the clusters that still have a tail
  for (int r = tid; r < nq; r += 256) {
    if (rep[r] != r || gsz[r] <= 0 || gsz[r] % B == 0) continue;
    int best = -1, bd = INT_MAX;
    for (int q = 0; q < nq; ++q) {
      if (q == r || rep[q] != q || gsz[q] <= 0 || gsz[q] % B == 0) continue;
      const int d = hamming(mk + (int64_t)r * mw, mk + (int64_t)q * mw, mw);
      if (d < bd) { bd = d; best = q; }
    }
    nn[r] = best;
  }
  __syncthreads();
  for (int r = tid; r < nq; r += 256) {
    const int q = nn[r];
    if (q <= r || nn[q] != r) continue;  // not mutual, or handled from the lower index
    const int tr = gsz[r] % B, tq = gsz[q] % B;
    if (tr + tq > B) continue;
    const bool r_gives = tr < tq || (tr == tq && r > q);
    const int donor = r_gives ? r : q, recv = r_gives ? q : r;
    cut[donor] = gsz[donor] % B;
    rcv[donor] = recv;
    gets[recv] = donor;
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int c = 0; c < nq; ++c) {
      nseg[c] = run;
      if (rep[c] == c && gsz[c] > 0) run += gsz[c] - cut[c] + (gets[c] >= 0 ? cut[gets[c]] : 0);
    }
    for (int c = nq; c < S; ++c) nseg[c] = run;
  }
  __syncthreads();
  int *plan = t.plan + (int64_t)h * TM_ARRAYS * S;
  for (int r = tid; r < S; r += 256) {
    plan[TM_REP * S + r] = r < nq ? rep[r] : r;
    plan[TM_PRE * S + r] = r < nq ? pre[r] : 0;
    plan[TM_GSZ * S + r] = gsz[r];
    plan[TM_CUT * S + r] = cut[r];
    plan[TM_RCV * S + r] = rcv[r];
    plan[TM_GETS * S + r] = gets[r];
    plan[TM_NSEG * S + r] = nseg[r];
    plan[TM_NN * S + r] = nn[r];
    t.seg_out[(int64_t)h * S + r] = nseg[r];
  }
}

// every token position of the old cluster order to its new place
__global__ __launch_bounds__(256) void k_tm_scatter(TailArgs t) {
  const int h = blockIdx.y;
  const int S = t.nq + 1;
  const int nq = t.ncl[h];
  const int *seg = t.seg_in + (int64_t)h * S;
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (nq <= 0 || p >= seg[nq]) return;
  int lo = 0, hi = nq;  // seg[lo] <= p < seg[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (seg[mid] <= p) lo = mid; else hi = mid;
  }
  const int r = lo;
  const int *plan = t.plan + (int64_t)h * TM_ARRAYS * S;
  const int g = plan[TM_REP * S + r];
  const int pos = plan[TM_PRE * S + r] + (p - seg[r]);
  const int keep = plan[TM_GSZ * S + g] - plan[TM_CUT * S + g];
  int c = g, dest;
  if (pos >= keep) {  // part of the tail a donor gives away
    c = plan[TM_RCV * S + g];
    dest = plan[TM_NSEG * S + c] + plan[TM_GSZ * S + c] + (pos - keep);
  } else {
    dest = plan[TM_NSEG * S + g] + pos;
  }
  const int tok = t.perm_in[(int64_t)h * t.L + p];
  t.perm_out[(int64_t)h * t.L + dest] = tok;
  t.labels_out[(int64_t)h * t.L + tok] = c;
}

// new masks and selection lists: a receiver ORs its donor's mask and appends
// the donor's extra clusters in the donor's order (one wave per cluster)
__global__ __launch_bounds__(64) void k_tm_sel(TailArgs t) {
  const int c = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int S = t.nq + 1;
  if (c >= t.nq) return;
  const int64_t rc = (int64_t)h * t.nq + c;
  const int *plan = t.plan + (int64_t)h * TM_ARRAYS * S;
  const int d = c < t.ncl[h] ? plan[TM_GETS * S + c] : -1;
  const uint32_t *mc = t.mask_in + rc * t.mwords;
  const uint32_t *md = d >= 0 ? t.mask_in + ((int64_t)h * t.nq + d) * t.mwords : nullptr;
  for (int w = lane; w < t.mwords; w += 64) t.mask_out[rc * t.mwords + w] = mc[w] | (md ? md[w] : 0u);
  const int n = t.n_in[rc];
  const int *li = t.list_in + rc * t.ncapk;
  int *lo = t.list_out + rc * t.ncapk;
  for (int i = lane; i < n; i += 64) lo[i] = li[i];
  int extra = 0;
  if (d >= 0) {
    const int nd = t.n_in[(int64_t)h * t.nq + d];
    const int *ld = t.list_in + ((int64_t)h * t.nq + d) * t.ncapk;
    for (int i0 = 0; i0 < nd; i0 += 64) {
      const int i = i0 + lane;
      const int e = i < nd ? ld[i] : 0;
      const bool add = i < nd && !((mc[e >> 5] >> (e & 31)) & 1u);
      const uint64_t bal = __ballot(add);
      if (add) lo[n + extra + __popcll(bal & ((1ull << lane) - 1ull))] = e;
      extra += __popcll(bal);
    }
  }
  if (lane == 0) t.n_out[rc] = n + extra;
}

void launch_tail_merge(const TailArgs &t, int BH, hipStream_t st) {
  const size_t lds = (size_t)9 * (t.nq + 1) * sizeof(int);
  hipLaunchKernelGGL(k_tm_plan, dim3(BH), dim3(256), lds, st, t);
  hipLaunchKernelGGL(k_tm_scatter, dim3((unsigned)((t.L + 255) / 256), (unsigned)BH), dim3(256), 0, st, t);
  hipLaunchKernelGGL(k_tm_sel, dim3((unsigned)t.nq, (unsigned)BH), dim3(64), 0, st, t);
}

}  // namespace ac
