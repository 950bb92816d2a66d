// Host side of the C ABI declared in include/ac.h: argument validation,
// workspace planning and the launch order of each entry point, including
// the host-driven stage loop of AdaCluster Algorithm 1.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <functional>
#include <mutex>
#include <vector>

#include "../../include/ac.h"
#include "internal.h"

#define AC_API extern "C" __attribute__((visibility("default")))

namespace ac {
namespace {

thread_local char g_err[512] = "";

ac_status fail(ac_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

#define AC_HIP(call)                                                                       \
  do {                                                                                     \
    hipError_t e_ = (call);                                                                \
    if (e_ != hipSuccess) return fail(AC_E_DEVICE, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

#define AC_CHECK_LAUNCH()                                                                       \
  do {                                                                                          \
    hipError_t e_ = hipGetLastError();                                                          \
    if (e_ != hipSuccess) return fail(AC_E_DEVICE, "kernel launch: %s", hipGetErrorString(e_)); \
  } while (0)

#define AC_TRY(expr)                 \
  do {                               \
    ac_status s_ = (expr);           \
    if (s_ != AC_OK) return s_;      \
  } while (0)

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---------------------------------------------------------------------------
// validation
ac_status check_shape(const ac_shape *s) {
  if (!s) return fail(AC_E_ARG, "shape is NULL");
  if (s->B <= 0 || s->H <= 0 || s->L <= 0 || s->d <= 0)
    return fail(AC_E_SHAPE, "B, H, L, d must be positive (got %d %d %d %d)", s->B, s->H, s->L, s->d);
  if (s->d != 64 && s->d != 128) return fail(AC_E_UNSUPPORTED, "d = %d: only 64 and 128 are supported", s->d);
  // kernels launch a row of workgroups per head: the grid's y extent is B*H
  if ((int64_t)s->B * s->H > 65535) return fail(AC_E_SHAPE, "B*H = %lld: at most 65,535 heads", (long long)s->B * s->H);
  if ((int64_t)s->L > (1 << 26)) return fail(AC_E_SHAPE, "L too large");
  // the attention's row gathers address one head's K and V with 32-bit byte offsets
  if ((int64_t)s->L * s->d * 2 >= (int64_t)1 << 32)
    return fail(AC_E_UNSUPPORTED, "L = %d: one head's rows (L * d * 2 bytes) must stay below 4 GiB", s->L);
  return AC_OK;
}

ac_status check_params(const ac_shape *s, const ac_params *p) {
  if (!p) return fail(AC_E_ARG, "params is NULL");
  if (p->nq <= 0) return fail(AC_E_ARG, "nq must be positive");
  if (p->iters < 0 || p->iters_warm < 0) return fail(AC_E_ARG, "iteration counts must be >= 0");
  if (p->m0 <= 0 || p->nmax <= 0) return fail(AC_E_ARG, "m0 and nmax must be positive");
  if (p->tau_rule < AC_TAU_MEAN_X || p->tau_rule > AC_TAU_INF) return fail(AC_E_ARG, "tau_rule out of range");
  if (p->tau_rule == AC_TAU_PCTL && !(p->tau_param > 0.f && p->tau_param <= 1.f))
    return fail(AC_E_ARG, "percentile tau_param must be in (0, 1]");
  if ((p->tau_rule == AC_TAU_MEAN_X || p->tau_rule == AC_TAU_ABS) && !(p->tau_param >= 0.f && std::isfinite(p->tau_param)))
    return fail(AC_E_ARG, "tau_param must be finite and >= 0");
  if (p->score_mode != AC_SCORE_QUEST && p->score_mode != AC_SCORE_MEAN) return fail(AC_E_ARG, "score_mode out of range");
  if (p->sel_mode < AC_SEL_TOPK || p->sel_mode > AC_SEL_DENSE) return fail(AC_E_ARG, "sel_mode out of range");
  if (p->sel_mode == AC_SEL_TOPK && p->topk <= 0) return fail(AC_E_ARG, "topk must be positive");
  if (p->sel_mode == AC_SEL_DENSITY && !(p->sel_param > 0.f && p->sel_param <= 1.f))
    return fail(AC_E_ARG, "density must be in (0, 1]");
  if (p->sel_mode == AC_SEL_TOPP && !(p->sel_param > 0.f && p->sel_param <= 1.f))
    return fail(AC_E_ARG, "top-p must be in (0, 1]");
  if (p->compensate != 0 && p->compensate != 1) return fail(AC_E_ARG, "compensate must be 0 or 1");
  if (!(p->scale >= 0.f) || !std::isfinite(p->scale)) return fail(AC_E_ARG, "scale must be finite and >= 0");
  if (p->init_sample < 0) return fail(AC_E_ARG, "init_sample must be >= 0");
  if (p->tail_block < 0) return fail(AC_E_ARG, "tail_block must be >= 0");
  if (p->min_sparse_gflop < 0) return fail(AC_E_ARG, "min_sparse_gflop must be >= 0");
  const int64_t ncap = (int64_t)p->nmax - 1 + p->m0;
  if (ncap > SEL_MAXN) return fail(AC_E_UNSUPPORTED, "nmax - 1 + m0 = %lld exceeds %d key clusters", (long long)ncap, SEL_MAXN);
  const int64_t mmax = std::max<int64_t>(std::min<int64_t>(p->nq, s->L), std::min<int64_t>(p->m0, s->L));
  const int64_t smax = p->init_sample > 0 ? std::min<int64_t>(s->L, (int64_t)p->init_sample * mmax) : s->L;
  if (smax > KPP_SMAX)
    return fail(AC_E_UNSUPPORTED, "k-means++ subsample of %lld points exceeds %d (lower init_sample)", (long long)smax, KPP_SMAX);
  return AC_OK;
}

// ---------------------------------------------------------------------------
// workspace plan: every region any entry point uses, at fixed offsets
// Scratch of one k-means engine.  Query and key clustering each have their
// own, so the two may run at the same time on different streams.
struct Scratch {
  size_t lab, lperm, lseg, thist, tgrp, ops_hi, ops_lo, ops_norm, d2buf, hn, hm, hcoff, chunk_off, upd_part;
  size_t chg, neff;  // Lloyd fixed-point detection: two change counters and the loop's n, per head
  size_t kpp_nx, kpp_G;
  int mcap, kpp_smax, upd_items;
};

struct Plan {
  int BH, L, D, nq, ncapk, max_tiles, max_groups, nq_pad, ncap_pad, mwords;
  size_t total = 0;
  Scratch sq, sk;  // query / key clustering
  size_t qhat, qn, hnew;
  size_t uidx0, uidx1, dist, flag, rstate, rhist, msepart;
  size_t scoreA, scoreB, S, seltok, kc, vc, rows, rows_T, pbias, tile_off, pairs;
  // ac_layer persistent
  size_t q_labels, q_perm, q_seg, q_cent, q_ncl, q_rho;
  size_t k_labels, k_perm, k_seg, k_cent, k_ncl;
  size_t kmax, kmin, kmean, vmean, fb, tau, mse, stages;
  size_t sel_list, sel_n, sel_mask, sel_score;
  // tail merging: its plan, and ac_layer's merged clusters and selection
  size_t tm_plan, m_labels, m_perm, m_seg, m_list, m_n, m_mask;
  // interaction matrix: raw query sums and counts per query cluster
  size_t qsum, qcnt;
  // principal-component split: token scratch, projection keys, node table
  size_t pca_tmp, pca_key, pca_nodes, pca_lvl, pca_dbuf;            // key side
  size_t pca_tmp_q, pca_key_q, pca_nodes_q, pca_lvl_q, pca_dbuf_q;  // query side (the two sides may overlap)
  // cold key clustering: operands of every stage's centres at their global
  // rows, the running nearest-centre score, per-stage centre counts and
  // offsets for the merge launches, Algorithm 1's per-head state, all-L counts
  size_t fops_hi, fops_lo, fops_norm, best, mtab, ctab, kst, nall;
  // chunked key statistics: chunk and slot offsets, per-slot partials
  size_t ks_co, ks_po, ks_psk, ks_psv, ks_pmx, ks_pmn, ks_pse;
  int ks_slots;
  int stage_slots;
};

// stride of the per-selection key row lists: whole key tiles
static inline int64_t rows_ld(int64_t n) { return (n + ATT_KT - 1) / ATT_KT * ATT_KT; }

Plan make_plan(const ac_shape *s, const ac_params *p) {
  Plan P;
  P.BH = s->B * s->H;
  P.L = s->L;
  P.D = s->d;
  P.nq = std::min(p->nq, s->L);
  P.ncapk = p->nmax - 1 + p->m0;
  P.max_tiles = (int)cdiv(P.L, SORT_TILE);
  P.max_groups = (int)cdiv(P.max_tiles, SORT_GROUP);
  P.nq_pad = (int)cdiv(P.nq, 16) * 16;
  P.ncap_pad = (int)cdiv(P.ncapk, 16) * 16;
  P.mwords = (int)cdiv(P.ncapk, 32);
  const size_t BH = P.BH, L = P.L, D = P.D;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + std::max<size_t>(bytes, 1));
    return o;
  };
  // mcap: most labels a sort of this engine sees; mm: most centres it seeds
  auto scratch = [&](Scratch &S, int mcap, int mm) {
    S.mcap = std::max(mcap, 2);
    S.lab = take(BH * L * 4);
    S.lperm = take(BH * L * 4);
    S.lseg = take(BH * (S.mcap + 1) * 4);
    S.thist = take(BH * P.max_tiles * (size_t)S.mcap * 4);
    S.tgrp = take(BH * P.max_groups * (size_t)S.mcap * 4);
    S.ops_hi = take(BH * S.mcap * D * 2);
    S.ops_lo = take(BH * S.mcap * D * 2);
    S.ops_norm = take(BH * S.mcap * 4);
    S.hn = take(3 * (size_t)BH * 4);  // n, m and centre offsets back to back: one copy per stage
    S.hm = S.hn + BH * 4;
    S.hcoff = S.hn + 2 * (size_t)BH * 4;
    S.chunk_off = take(BH * (S.mcap + 1) * 4);
    S.chg = take(2 * BH * 4);
    S.neff = take(BH * 4);
    S.upd_items = (int)cdiv(P.L, UPD_CHUNK) + S.mcap;
    S.upd_part = take(BH * (size_t)S.upd_items * D * 8);
    S.kpp_smax = p->init_sample > 0 ? (int)std::min<int64_t>(P.L, (int64_t)p->init_sample * mm) : P.L;
    const bool gram = S.kpp_smax <= KPP_GRAM_MAX;
    S.kpp_nx = take(gram ? BH * (size_t)S.kpp_smax * 8 : 0);
    S.kpp_G = take(gram ? BH * (size_t)S.kpp_smax * S.kpp_smax * 8 : 0);
    S.d2buf = take(gram ? 0 : BH * (size_t)KPP_SMAX * 8);
  };
  scratch(P.sq, P.nq, P.nq);
  scratch(P.sk, P.ncapk, std::min(p->m0, P.L));
  P.qhat = take(BH * L * D * 2);
  P.qn = take(BH * L * 4);
  P.hnew = take(BH * 4);
  P.uidx0 = take(BH * L * 4);
  P.uidx1 = take(BH * L * 4);
  P.dist = take(BH * L * 4);
  P.flag = take(BH * L * 4);
  P.rstate = take(BH * 2 * 4);
  P.rhist = take(BH * 256 * 4);
  P.msepart = take(BH * P.ncapk * 8);
  P.ks_slots = kst_slots(P.L);
  P.ks_co = take(BH * (P.ncapk + 1) * 4);
  P.ks_po = take(BH * (P.ncapk + 1) * 4);
  P.ks_psk = take(BH * (size_t)P.ks_slots * D * 8);
  P.ks_psv = take(BH * (size_t)P.ks_slots * D * 8);
  P.ks_pmx = take(BH * (size_t)P.ks_slots * D * 4);
  P.ks_pmn = take(BH * (size_t)P.ks_slots * D * 4);
  P.ks_pse = take(BH * (size_t)P.ks_slots * 8);
  P.scoreA = take(BH * P.nq_pad * 6 * D * 2);
  P.scoreB = take(BH * P.ncap_pad * 6 * D * 2);
  P.S = take(BH * P.nq * (size_t)P.ncapk * 4);
  P.seltok = take(BH * P.nq * 4);
  P.kc = take(BH * P.ncapk * D * 2);
  P.vc = take(BH * P.ncapk * D * 2);
  P.rows = take(BH * (size_t)P.nq * rows_ld(L) * 4);
  P.rows_T = take(BH * (size_t)P.nq * 4);
  P.pbias = take(BH * (size_t)P.nq * rows_ld(P.ncapk) * 4);
  P.tile_off = take(BH * (P.nq + 1) * 4);
  P.pairs = take(BH * 8);
  P.q_labels = take(BH * L * 4);
  P.q_perm = take(BH * L * 4);
  P.q_seg = take(BH * (P.nq + 1) * 4);
  P.q_cent = take(BH * P.nq * D * 4);
  P.q_ncl = take(BH * 4);
  P.q_rho = take(BH * P.nq * 4);
  P.k_labels = take(BH * L * 4);
  P.k_perm = take(BH * L * 4);
  P.k_seg = take(BH * (P.ncapk + 1) * 4);
  P.k_cent = take(BH * P.ncapk * D * 4);
  P.k_ncl = take(BH * 4);
  P.kmax = take(BH * P.ncapk * D * 2);
  P.kmin = take(BH * P.ncapk * D * 2);
  P.kmean = take(BH * P.ncapk * D * 4);
  P.vmean = take(BH * P.ncapk * D * 4);
  P.fb = take(BH);
  P.tau = take(BH * 4);
  P.mse = take(BH * 4);
  P.stages = take(BH * 4);
  P.sel_list = take(BH * P.nq * (size_t)P.ncapk * 4);
  P.sel_n = take(BH * P.nq * 4);
  P.sel_mask = take(BH * P.nq * (size_t)P.mwords * 4);
  P.sel_score = take(BH * P.nq * (size_t)P.ncapk * 4);
  P.tm_plan = take(BH * 8 * (size_t)(P.nq + 1) * 4);
  P.m_labels = take(BH * L * 4);
  P.m_perm = take(BH * L * 4);
  P.m_seg = take(BH * (P.nq + 1) * 4);
  P.m_list = take(BH * P.nq * (size_t)P.ncapk * 4);
  P.m_n = take(BH * P.nq * 4);
  P.m_mask = take(BH * P.nq * (size_t)P.mwords * 4);
  P.qsum = take(BH * P.nq * D * 8);
  P.qcnt = take(BH * P.nq * 4);
  P.pca_tmp = take(BH * L * 4);
  P.pca_key = take(BH * L * 4);
  P.pca_nodes = take((L / PCA_BLOCK_MIN + 2) * 8);  // at most ceil(L / b) - 1 internal nodes
  P.pca_lvl = take(64 * 4);
  P.pca_dbuf = take(BH * (size_t)pca_dir_cap(L) * D * 4);
  P.pca_tmp_q = take(BH * L * 4);
  P.pca_key_q = take(BH * L * 4);
  P.pca_nodes_q = take((L / PCA_BLOCK_MIN + 2) * 8);
  P.pca_lvl_q = take(64 * 4);
  P.pca_dbuf_q = take(BH * (size_t)pca_dir_cap(L) * D * 4);
  P.fops_hi = take(BH * P.ncapk * D * 2);
  P.fops_lo = take(BH * P.ncapk * D * 2);
  P.fops_norm = take(BH * P.ncapk * 4);
  P.best = take(BH * L * 4);
  // every stage but the last adds min(L, m0) centres, and none starts at nmax or beyond
  // Stages of Algorithm 1: every stage but the last adds min(m0, L) centres.
  // A stage on |U| <= m0 keys makes each its own centre (duplicates at
  // distance 0 too), so with tau > 0 it removes them all and is the last;
  // with tau = 0 nothing is ever removed and |U| stays L.  So at most
  // ceil(nmax / min(m0, L)) stages start below the cap, plus the last one.
  P.stage_slots = (int)cdiv(p->nmax, std::max(1, std::min(p->m0, P.L))) + 2;
  P.mtab = take((size_t)P.stage_slots * BH * 4);
  P.ctab = take((size_t)P.stage_slots * BH * 4);
  P.kst = take(BH * KST_FIELDS * 4);
  P.nall = take(BH * 4);
  P.total = off + 256;  // slack for aligning the base pointer
  return P;
}

template <typename T>
T *at(void *base, size_t off) {
  return reinterpret_cast<T *>(reinterpret_cast<char *>(base) + off);
}

ac_status check_ws(const Plan &P, void *ws, size_t ws_bytes) {
  if (!ws) return fail(AC_E_ARG, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return fail(AC_E_ARG, "workspace must be 256-byte aligned");
  if (ws_bytes < P.total)
    return fail(AC_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes required", ws_bytes, P.total);
  return AC_OK;
}

ac_status check_device() {
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess || n <= 0)
    return fail(AC_E_DEVICE, "no HIP device available (%s)", e == hipSuccess ? "count 0" : hipGetErrorString(e));
  return AC_OK;
}

float attn_scale(const ac_params *p, int D) { return p->scale > 0.f ? p->scale : 1.0f / std::sqrt((float)D); }

// Record of a k-means job's centres (see Engine::run): head stride hs, slot stride it.
struct TraceCent {
  float *p = nullptr;
  int64_t hs = 0, it = 0;
};

// ---------------------------------------------------------------------------
// the k-means engine: optional k-means++ seeding, iters Lloyd iterations,
// and a final assignment into labels_out.
struct Engine {
  const Plan &P;
  const Scratch &S;
  void *ws;
  hipStream_t st;
  // compute units the resident assignment leaves to work beside it (the key
  // clustering's one-block-per-head launches when the queries run beside it)
  int spare = 0;
  int *n() { return at<int>(ws, S.hn); }
  int *m() { return at<int>(ws, S.hm); }
  int *coff() { return at<int>(ws, S.hcoff); }
  CentOps ops() { return CentOps{at<uint16_t>(ws, S.ops_hi), at<uint16_t>(ws, S.ops_lo), at<float>(ws, S.ops_norm), S.mcap}; }
  SortArgs sort_args(const int *labels, int *perm, int *seg, int segcap, int mcap_used) {
    SortArgs s;
    s.labels = labels;
    s.lab_hs = P.L;
    s.n = n();
    s.m = m();
    s.tile_hist = at<int>(ws, S.thist);
    s.max_tiles = P.max_tiles;
    s.grp = at<int>(ws, S.tgrp);
    s.max_groups = P.max_groups;
    s.mcap = std::max(mcap_used, 2);
    s.perm = perm;
    s.perm_hs = P.L;
    s.seg = seg;
    s.seg_hs = segcap + 1;
    s.segcap = segcap;
    s.neff = nullptr;
    s.chg_cur = nullptr;
    s.chg_zero = nullptr;
    s.chunk_off = nullptr;
    s.co_hs = 0;
    return s;
  }
  // mmax: bound on m over heads (grid size); npts: bound on n.
  // metric: NULL for Euclidean distances, else [BH, D, D] fp32: the assignment
  // minimises (x - c) M (x - c)^T (centre operands M c and c M c^T)
  // tc (optional): record of the centres after seeding (slot 0) and after each
  // Lloyd update (slot j), head stride tc.hs, slot stride tc.it
  // k-means++ seeding of the job's centres.  Its grids depend only on the
  // engine's subsample cap, so it can be enqueued before the host knows the
  // job's point counts (heads with n = 0 or m = 0 are idle).
  // rounds (nullable): recorded on st where the wide launches end and only
  // the sequential rounds, one block per head, remain
  ac_status seed(const KmArgs &a, const ac_params *p, int role, int stage, hipEvent_t rounds = nullptr) {
    if (S.kpp_smax <= KPP_GRAM_MAX) {
      AC_HIP(launch_kpp_gram(P.D, a, P.BH, S.kpp_smax, at<double>(ws, S.kpp_nx), at<double>(ws, S.kpp_G),
                             p->init_sample, p->seed, role, stage, st, rounds));
    } else {
      if (rounds) AC_HIP(hipEventRecord(rounds, st));
      launch_kpp(P.D, a, P.BH, at<double>(ws, S.d2buf), p->init_sample, p->seed, role, stage, st);
    }
    AC_CHECK_LAUNCH();
    return AC_OK;
  }
  ac_status run(const KmArgs &a, int mmax, int npts, bool seed_init, int iters, const ac_params *p, int role,
                int stage, int *labels_out, const float *metric = nullptr, TraceCent tc = TraceCent()) {
    if (seed_init) AC_TRY(seed(a, p, role, stage));
    return lloyd(a, mmax, npts, iters, labels_out, metric, tc);
  }
  // iters Lloyd iterations from the job's current centres, then the final
  // assignment into labels_out
  ac_status lloyd(const KmArgs &a, int mmax, int npts, int iters, int *labels_out, const float *metric = nullptr,
                  TraceCent tc = TraceCent()) {
    const int D = P.D;
    auto trace = [&](int slot) {
      if (tc.p) launch_trace_cent(D, a, P.BH, mmax, tc.p + slot * tc.it, tc.hs, st);
    };
    trace(0);
    CentOps op = ops();
    launch_cent_prep(D, a, op, P.BH, mmax, st);
    if (metric) launch_cent_prep_metric(D, a, op, metric, P.BH, mmax, st);
    AC_CHECK_LAUNCH();
    int *lab = at<int>(ws, S.lab);
    // Lloyd iterations.  Once an assignment leaves every label of a head as
    // it was, the update reproduces that head's centres bit for bit (the
    // same members, summed in the same order; empty clusters keep theirs),
    // so every later iteration is a fixed point: the head leaves the loop
    // (its n in the loop's copy `neff` drops to 0) with exactly the centres
    // and labels the remaining iterations would give.  Iteration 0 has no
    // previous labels to compare with.  The final assignment covers the heads
    // still in the loop; the others keep the loop's last labels, which it
    // would repeat.
    int *chg = at<int>(ws, S.chg), *neff = at<int>(ws, S.neff);
    // heads of few points: the counting sort and the update are one launch each
    const bool small = npts <= SORT_SMALL_MAX && mmax <= SORT_SMALL_M;
    KmArgs al = a;
    if (iters > 0) {
      launch_copy_i32(a.n, neff, P.BH, st);
      al.n = neff;
    }
    for (int it = 0; it < iters; ++it) {
      int *cur = chg + (it & 1) * P.BH, *nxt = chg + ((it + 1) & 1) * P.BH;
      launch_assign(D, al, op, P.BH, mmax, npts, lab, P.L, st, it > 0 ? cur : nullptr, nullptr, spare);
      SortArgs s = sort_args(lab, at<int>(ws, S.lperm), at<int>(ws, S.lseg), S.mcap, mmax);
      s.n = neff;
      s.neff = neff;
      s.chg_cur = it > 0 ? cur : nullptr;
      s.chg_zero = nxt;
      s.chunk_off = at<int>(ws, S.chunk_off);
      s.co_hs = S.mcap + 1;
      if (small) {
        launch_sort_small(s, P.BH, st);
        launch_update_small(D, al, s, op, P.BH, mmax, st);
      } else {
        launch_sort(s, P.BH, npts, st);
        launch_update(D, al, s, op, P.BH, mmax, npts, at<double>(ws, S.upd_part), (int64_t)S.upd_items * D, st);
      }
      if (metric) launch_cent_prep_metric(D, a, op, metric, P.BH, mmax, st);
      trace(it + 1);
      AC_CHECK_LAUNCH();
    }
    if (iters > 0) {
      launch_assign(D, al, op, P.BH, mmax, npts, labels_out, P.L, st, nullptr, nullptr, spare);
      launch_copy_converged(a.n, neff, lab, labels_out, P.L, npts, P.BH, st);
    } else {
      launch_assign(D, a, op, P.BH, mmax, npts, labels_out, P.L, st, nullptr, nullptr, spare);
    }
    AC_CHECK_LAUNCH();
    return AC_OK;
  }
};

// ---------------------------------------------------------------------------
// beside_keys: the key clustering runs at the same time on another stream;
// the query assignment's resident grid then leaves one compute unit per head
// to the key side's one-block-per-head launches (seeding rounds, label scans),
// which otherwise wait until the assignment ends.
ac_status do_cluster_q(const Plan &P, const ac_params *p, const uint16_t *Q, const float *warm_cent,
                       ac_clusters *q, void *ws, hipStream_t st, float *cent_trace = nullptr,
                       bool beside_keys = false) {
  const int BH = P.BH, L = P.L, D = P.D;
  Engine E{P, P.sq, ws, st};
  E.spare = beside_keys ? BH : 0;
  uint16_t *qhat = at<uint16_t>(ws, P.qhat);
  float *qn = at<float>(ws, P.qn);
  launch_qnorm(D, Q, qhat, qn, (int64_t)BH * L, st);
  launch_fill_i32(E.n(), BH, L, st);
  launch_fill_i32(E.m(), BH, P.nq, st);
  launch_fill_i32(E.coff(), BH, 0, st);
  launch_fill_i32(q->ncl, BH, P.nq, st);
  AC_CHECK_LAUNCH();
  if (warm_cent) {
    // centres beyond nq (if ncap > nq) are left as they are
    for (int h = 0; h < BH; ++h)
      AC_HIP(hipMemcpyAsync(q->cent + (size_t)h * q->ncap * D, warm_cent + (size_t)h * q->ncap * D,
                            (size_t)P.nq * D * 4, hipMemcpyDeviceToDevice, st));
  }
  KmArgs a{qhat, (int64_t)L * D, nullptr, 0, E.n(), E.m(), E.coff(), q->cent, (int64_t)q->ncap * D};
  TraceCent tc;
  if (cent_trace) {
    tc.p = cent_trace;
    tc.it = (int64_t)q->ncap * D;
    tc.hs = (int64_t)(p->iters + 1) * tc.it;
  }
  AC_TRY(E.run(a, P.nq, L, warm_cent == nullptr, warm_cent ? p->iters_warm : p->iters, p, 0, 0, q->labels, nullptr,
               tc));
  SortArgs s = E.sort_args(q->labels, q->perm, q->seg, q->ncap, P.nq);
  launch_sort(s, BH, L, st);
  launch_seg_mean(qn, q->perm, q->seg, L, q->ncap, q->ncl, q->rho, BH, st);
  AC_CHECK_LAUNCH();
  return AC_OK;
}

// Arguments of the key statistics of clusters k into stats, with their
// workspace scratch.
KStatsArgs kstats_args(const Plan &P, const uint16_t *K, const uint16_t *V, const ac_clusters *k, ac_kstats *stats,
                       void *ws) {
  KStatsArgs a{K, V, k->perm, k->seg, k->ncl, k->cent, stats->kmax, stats->kmin, stats->kmean, stats->vmean,
               at<double>(ws, P.msepart), stats->mse, P.L, k->ncap};
  a.co = at<int>(ws, P.ks_co);
  a.po = at<int>(ws, P.ks_po);
  a.psk = at<double>(ws, P.ks_psk);
  a.psv = at<double>(ws, P.ks_psv);
  a.pmx = at<float>(ws, P.ks_pmx);
  a.pmn = at<float>(ws, P.ks_pmn);
  a.pse = at<double>(ws, P.ks_pse);
  a.pslots = P.ks_slots;
  return a;
}

// assign: with it, the final assignment of every key over all centres first
// (without, k->labels already hold it)
ac_status finish_keys(const Plan &P, const uint16_t *K, const uint16_t *V, ac_clusters *k, ac_kstats *stats,
                      void *ws, hipStream_t st, int mmax, bool assign = true) {
  // final assignment of every key over all centres, counting sort, statistics
  const int BH = P.BH, L = P.L, D = P.D;
  Engine E{P, P.sk, ws, st};
  launch_fill_i32(E.n(), BH, L, st);
  launch_copy_i32(k->ncl, E.m(), BH, st);
  launch_fill_i32(E.coff(), BH, 0, st);
  if (assign) {
    KmArgs a{K, (int64_t)L * D, nullptr, 0, E.n(), E.m(), E.coff(), k->cent, (int64_t)k->ncap * D};
    CentOps op = E.ops();
    launch_cent_prep(D, a, op, BH, mmax, st);
    launch_assign(D, a, op, BH, mmax, L, k->labels, L, st);
  }
  SortArgs s = E.sort_args(k->labels, k->perm, k->seg, k->ncap, mmax);
  launch_sort(s, BH, L, st);
  const KStatsArgs ks = kstats_args(P, K, V, k, stats, ws);
  launch_kstats(D, ks, BH, st);
  AC_CHECK_LAUNCH();
  return AC_OK;
}

// Algorithm 1 with the stage loop on the host (centre counts above the
// resident assignment's limit).
ac_status do_cluster_k_cold_plain(const Plan &P, const ac_params *p, const uint16_t *K, const uint16_t *V,
                                  ac_clusters *k, ac_kstats *stats, void *ws, hipStream_t st,
                                  const ac_ktrace *tr) {
  const int BH = P.BH, L = P.L, D = P.D;
  Engine E{P, P.sk, ws, st};
  std::vector<int> nU(BH, L), nC(BH, 0), done(BH, 0), F(BH, 0), stg(BH, 0), nmc(3 * (size_t)BH);
  int *hn = nmc.data(), *hm = hn + BH, *hc = hn + 2 * BH;
  int *uidx[2] = {at<int>(ws, P.uidx0), at<int>(ws, P.uidx1)};
  int cur = 0;
  float *dist = at<float>(ws, P.dist);
  int *flag = at<int>(ws, P.flag);
  for (int t = 0;; ++t) {
    int active = 0, mmax = 0, nmaxpts = 0;
    for (int h = 0; h < BH; ++h) {
      if (!done[h] && nC[h] >= p->nmax) { F[h] = 1; done[h] = 1; }
      if (done[h]) { hn[h] = 0; hm[h] = 0; hc[h] = nC[h]; continue; }
      hn[h] = nU[h];
      hm[h] = std::min(nU[h], p->m0);
      hc[h] = nC[h];
      active++;
      mmax = std::max(mmax, hm[h]);
      nmaxpts = std::max(nmaxpts, hn[h]);
    }
    if (!active) break;
    AC_HIP(hipMemcpyAsync(E.n(), nmc.data(), 3 * (size_t)BH * 4, hipMemcpyHostToDevice, st));
    KmArgs a{K, (int64_t)L * D, t == 0 ? nullptr : uidx[cur], L, E.n(), E.m(), E.coff(), k->cent,
             (int64_t)k->ncap * D};
    int *lab = at<int>(ws, E.S.lab);
    const bool rec = tr && t < tr->max_stages;
    TraceCent tc;
    if (rec && tr->cent) {
      tc.it = (int64_t)p->m0 * D;
      const int64_t stage_stride = (int64_t)(p->iters + 1) * tc.it;
      tc.hs = (int64_t)tr->max_stages * stage_stride;
      tc.p = tr->cent + t * stage_stride;
    }
    if (rec) launch_trace_nm(E.n(), E.m(), tr->n, tr->m, tr->max_stages, t, BH, st);
    AC_TRY(E.run(a, mmax, nmaxpts, true, p->iters, p, 1, t, lab, nullptr, tc));
    launch_stage_dist(D, a, BH, nmaxpts, lab, L, dist, L, st);
    if (rec && (tr->u || tr->labels || tr->dist)) {
      const int64_t ohs = (int64_t)tr->max_stages * L, oo = (int64_t)t * L;
      launch_trace_stage(E.n(), t == 0 ? nullptr : uidx[cur], L, lab, dist, L, tr->u ? tr->u + oo : nullptr,
                         tr->labels ? tr->labels + oo : nullptr, tr->dist ? tr->dist + oo : nullptr, ohs, BH,
                         nmaxpts, st);
    }
    if (t == 0)
      launch_tau(dist, L, E.n(), BH, nmaxpts, p->tau_rule, p->tau_param, stats->tau, at<uint32_t>(ws, P.rstate),
                 at<uint32_t>(ws, P.rhist), st);
    launch_flag_removed(dist, L, E.n(), stats->tau, flag, L, BH, nmaxpts, st);
    // stable compaction: label 0 (kept) first
    launch_fill_i32(E.m(), BH, 2, st);
    SortArgs s = E.sort_args(flag, at<int>(ws, E.S.lperm), at<int>(ws, E.S.lseg), 1, 2);
    launch_sort(s, BH, nmaxpts, st);
    launch_compact_gather(t == 0 ? nullptr : uidx[cur], L, at<int>(ws, E.S.lperm), L, at<int>(ws, E.S.lseg), 2,
                          uidx[cur ^ 1], at<int>(ws, P.hnew), BH, nmaxpts, st);
    AC_CHECK_LAUNCH();
    std::vector<int> nnew(BH);
    AC_HIP(hipMemcpyAsync(nnew.data(), at<int>(ws, P.hnew), BH * 4, hipMemcpyDeviceToHost, st));
    AC_HIP(hipStreamSynchronize(st));
    for (int h = 0; h < BH; ++h) {
      if (done[h]) continue;
      nC[h] += hm[h];
      stg[h] = t + 1;
      nU[h] = hn[h] > 0 ? nnew[h] : 0;
      if (nU[h] == 0) done[h] = 1;
    }
    cur ^= 1;
  }
  std::vector<uint8_t> fb(BH);
  int mmax = 1;
  for (int h = 0; h < BH; ++h) {
    fb[h] = (uint8_t)F[h];
    mmax = std::max(mmax, nC[h]);
  }
  AC_HIP(hipMemcpyAsync(k->ncl, nC.data(), BH * 4, hipMemcpyHostToDevice, st));
  AC_HIP(hipMemcpyAsync(stats->fallback, fb.data(), BH, hipMemcpyHostToDevice, st));
  AC_HIP(hipMemcpyAsync(stats->stages, stg.data(), BH * 4, hipMemcpyHostToDevice, st));
  AC_TRY(finish_keys(P, K, V, k, stats, ws, st, mmax));
  // the host vectors above must outlive the copies
  AC_HIP(hipStreamSynchronize(st));
  return AC_OK;
}

ac_status aux_stream(int which, hipStream_t *out, hipEvent_t *fork, hipEvent_t *join);
ac_status pinned_i32(int n, int **out);

// Algorithm 1 (AdaCluster §3.2.2) with the per-head bookkeeping on the device.
// Each stage: the Lloyd loop of its k-means (grids sized by the host from
// the counts read one stage earlier), the distances, tau (first stage), the
// removal flags and the stable compaction of U; then k_stage_next closes the
// stage and opens the next one (centre count, fallback flag, n, m, offset).
// The next stage's k-means++ seeding is enqueued at once (its grids do not
// depend on the counts), and the host reads the new counts from pinned
// memory behind it, so the GPU does not wait for the host at stage
// boundaries.  The final nearest centre of every key over all stages is
// computed stage by stage on an auxiliary stream as each stage's centres
// are final (merge-mode assignment: strictly better only, so ties keep the
// lowest centre index), each merge beside the next stage's sequential
// seeding rounds.
// after_first (optional) is called once the first stage is enqueued, before
// the host first waits: ac_layer enqueues the query clustering there, so
// that the key stream starts at once and the host's launch work for the
// queries overlaps the first stage.
ac_status do_cluster_k_cold(const Plan &P, const ac_params *p, const uint16_t *K, const uint16_t *V,
                            ac_clusters *k, ac_kstats *stats, void *ws, hipStream_t st,
                            const ac_ktrace *tr = nullptr,
                            const std::function<ac_status()> &after_first = nullptr) {
  const int BH = P.BH, L = P.L, D = P.D;
  if (std::min(p->m0, L) > ASSIGN_RES_MAX) {
    if (after_first) AC_TRY(after_first());
    return do_cluster_k_cold_plain(P, p, K, V, k, stats, ws, st, tr);
  }
  Engine E{P, P.sk, ws, st};
  int *uidx[2] = {at<int>(ws, P.uidx0), at<int>(ws, P.uidx1)};
  int cur = 0;
  float *dist = at<float>(ws, P.dist);
  int *flag = at<int>(ws, P.flag);
  int *kst = at<int>(ws, P.kst);
  int *mtab = at<int>(ws, P.mtab), *ctab = at<int>(ws, P.ctab);
  float *best = at<float>(ws, P.best);
  CentOps fops{at<uint16_t>(ws, P.fops_hi), at<uint16_t>(ws, P.fops_lo), at<float>(ws, P.fops_norm), P.ncapk};
  hipStream_t ax;
  hipEvent_t ev_fork, ev_join;
  AC_TRY(aux_stream(1, &ax, &ev_fork, &ev_join));
  int *hnm = nullptr;  // pinned: n then m of the next stage
  AC_TRY(pinned_i32(2 * BH, &hnm));
  // the merge launches start from "no centre yet"
  launch_fill_i32(at<int>(ws, P.nall), BH, L, st);
  launch_fill_i32(reinterpret_cast<int *>(best), (int64_t)BH * L, (int)0xff800000u, st);  // -inf
  launch_stage_next(kst, nullptr, E.n(), E.m(), E.coff(), 0, p->nmax, p->m0, L, BH, st);
  AC_CHECK_LAUNCH();
  int nmaxpts = L, mmax = std::min(p->m0, L);
  auto args = [&](int t, int c) {
    return KmArgs{K, (int64_t)L * D, t == 0 ? nullptr : uidx[c], L, E.n(), E.m(), E.coff(), k->cent,
                  (int64_t)k->ncap * D};
  };
  AC_TRY(E.seed(args(0, cur), p, 1, 0));
  for (int t = 0;; ++t) {
    if (t >= P.stage_slots) return fail(AC_E_DEVICE, "Algorithm 1 ran more stages (%d) than it can", t);
    KmArgs a = args(t, cur);
    int *lab = at<int>(ws, E.S.lab);
    const bool rec = tr && t < tr->max_stages;
    TraceCent tc;
    if (rec && tr->cent) {
      tc.it = (int64_t)p->m0 * D;
      const int64_t stage_stride = (int64_t)(p->iters + 1) * tc.it;
      tc.hs = (int64_t)tr->max_stages * stage_stride;
      tc.p = tr->cent + t * stage_stride;
    }
    if (rec) launch_trace_nm(E.n(), E.m(), tr->n, tr->m, tr->max_stages, t, BH, st);
    AC_TRY(E.lloyd(a, mmax, nmaxpts, p->iters, lab, nullptr, tc));
    // this stage's centres are final: their operands at global rows, and the
    // merge into every key's nearest centre on the auxiliary stream
    launch_copy_i32(E.m(), mtab + (int64_t)t * BH, BH, st);
    launch_copy_i32(E.coff(), ctab + (int64_t)t * BH, BH, st);
    launch_cent_prep(D, a, fops, BH, mmax, st, true);
    AC_CHECK_LAUNCH();
    const int mmax_t = mmax;
    launch_stage_dist(D, a, BH, nmaxpts, lab, L, dist, L, st);
    if (rec && (tr->u || tr->labels || tr->dist)) {
      const int64_t ohs = (int64_t)tr->max_stages * L, oo = (int64_t)t * L;
      launch_trace_stage(E.n(), t == 0 ? nullptr : uidx[cur], L, lab, dist, L, tr->u ? tr->u + oo : nullptr,
                         tr->labels ? tr->labels + oo : nullptr, tr->dist ? tr->dist + oo : nullptr, ohs, BH,
                         nmaxpts, st);
    }
    if (t == 0)
      launch_tau(dist, L, E.n(), BH, nmaxpts, p->tau_rule, p->tau_param, stats->tau, at<uint32_t>(ws, P.rstate),
                 at<uint32_t>(ws, P.rhist), st);
    launch_flag_removed(dist, L, E.n(), stats->tau, flag, L, BH, nmaxpts, st);
    // stable compaction: label 0 (kept) first
    launch_fill_i32(E.m(), BH, 2, st);
    SortArgs s = E.sort_args(flag, at<int>(ws, E.S.lperm), at<int>(ws, E.S.lseg), 1, 2);
    if (nmaxpts <= SORT_SMALL_MAX) launch_sort_small(s, BH, st);
    else launch_sort(s, BH, nmaxpts, st);
    launch_compact_gather(t == 0 ? nullptr : uidx[cur], L, at<int>(ws, E.S.lperm), L, at<int>(ws, E.S.lseg), 2,
                          uidx[cur ^ 1], at<int>(ws, P.hnew), BH, nmaxpts, st);
    // close this stage, open the next; read its counts behind its seeding
    launch_stage_next(kst, at<int>(ws, P.hnew), E.n(), E.m(), E.coff(), t + 1, p->nmax, p->m0, L, BH, st);
    AC_CHECK_LAUNCH();
    AC_HIP(hipMemcpyAsync(hnm, E.n(), (size_t)BH * 4, hipMemcpyDeviceToHost, st));
    AC_HIP(hipMemcpyAsync(hnm + BH, E.m(), (size_t)BH * 4, hipMemcpyDeviceToHost, st));
    AC_HIP(hipEventRecord(ev_join, st));
    cur ^= 1;
    AC_TRY(E.seed(args(t + 1, cur), p, 1, t + 1, ev_fork));
    // The merge of this stage's centres runs beside the next stage's
    // sequential seeding rounds, which keep one compute unit per head busy
    // and leave the rest idle.  It starts after the seeding's distance matrix
    // (a grid over every compute unit that it would otherwise hold up), and
    // its resident grid leaves those compute units to the rounds, so none of
    // its blocks waits behind them.
    AC_HIP(hipStreamWaitEvent(ax, ev_fork, 0));
    {
      KmArgs am{K, (int64_t)L * D, nullptr, 0, at<int>(ws, P.nall), mtab + (int64_t)t * BH,
                ctab + (int64_t)t * BH, k->cent, (int64_t)k->ncap * D};
      launch_assign(D, am, fops, BH, mmax_t, L, k->labels, L, ax, nullptr, best, BH);
      AC_CHECK_LAUNCH();
    }
    if (t == 0 && after_first) AC_TRY(after_first());
    AC_HIP(hipEventSynchronize(ev_join));
    int active = 0;
    nmaxpts = 0;
    mmax = 0;
    for (int h = 0; h < BH; ++h) {
      if (hnm[h] > 0 && hnm[BH + h] > 0) ++active;
      nmaxpts = std::max(nmaxpts, hnm[h]);
      mmax = std::max(mmax, hnm[BH + h]);
    }
    if (!active) break;
  }
  launch_stage_final(kst, k->ncl, stats->fallback, stats->stages, BH, st);
  // the last merge launch before the labels are sorted
  AC_HIP(hipEventRecord(ev_join, ax));
  AC_HIP(hipStreamWaitEvent(st, ev_join, 0));
  SortArgs s = E.sort_args(k->labels, k->perm, k->seg, k->ncap, k->ncap);
  launch_fill_i32(E.n(), BH, L, st);
  launch_copy_i32(k->ncl, E.m(), BH, st);
  launch_sort(s, BH, L, st);
  const KStatsArgs ks = kstats_args(P, K, V, k, stats, ws);
  launch_kstats(D, ks, BH, st);
  AC_CHECK_LAUNCH();
  return AC_OK;
}

ac_status do_cluster_k_warm(const Plan &P, const ac_params *p, const uint16_t *K, const uint16_t *V,
                            const ac_state *w, ac_clusters *k, ac_kstats *stats, void *ws, hipStream_t st) {
  const int BH = P.BH, L = P.L, D = P.D;
  Engine E{P, P.sk, ws, st};
  AC_HIP(hipMemcpyAsync(k->cent, w->cent_k, (size_t)BH * k->ncap * D * 4, hipMemcpyDeviceToDevice, st));
  launch_copy_i32(w->ncl_k, k->ncl, BH, st);
  launch_copy_u8(w->fallback, stats->fallback, BH, st);
  launch_copy_f32(w->tau, stats->tau, BH, st);
  launch_fill_i32(stats->stages, BH, 0, st);
  launch_fill_i32(E.n(), BH, L, st);
  launch_copy_i32(w->ncl_k, E.m(), BH, st);
  launch_fill_i32(E.coff(), BH, 0, st);
  AC_CHECK_LAUNCH();
  KmArgs a{K, (int64_t)L * D, nullptr, 0, E.n(), E.m(), E.coff(), k->cent, (int64_t)k->ncap * D};
  AC_TRY(E.run(a, k->ncap, L, false, p->iters_warm, p, 1, 0, k->labels));
  // the loop ends with the final assignment: only the order and statistics remain
  return finish_keys(P, K, V, k, stats, ws, st, k->ncap, false);
}

// ClusterAttention's clustering of the rows X of every head by recursive
// splits along principal directions into clusters of `block` rows; the
// order, labels, segments, count and member-mean centres of `out`.  The
// query and the key side have scratch of their own, so the two may overlap.
ac_status do_pca_split(const Plan &P, const uint16_t *X, int block, ac_clusters *out, const ac_pca_trace *tr,
                       void *ws, hipStream_t st, bool query_side) {
  const int BH = P.BH, L = P.L, D = P.D;
  const std::vector<int> counts = pca_level_counts(L, block);
  int ninternal = 0;
  for (int c : counts) ninternal += c;
  PcaArgs a;
  a.X = X;
  a.perm = out->perm;
  a.tmp = at<int>(ws, query_side ? P.pca_tmp_q : P.pca_tmp);
  a.key = at<uint32_t>(ws, query_side ? P.pca_key_q : P.pca_key);
  a.nodes = at<int2>(ws, query_side ? P.pca_nodes_q : P.pca_nodes);
  a.lvl = at<int>(ws, query_side ? P.pca_lvl_q : P.pca_lvl);
  a.dbuf = at<float>(ws, query_side ? P.pca_dbuf_q : P.pca_dbuf);
  a.dir = tr ? tr->dir : nullptr;
  a.ndir = ninternal;
  a.L = L;
  a.block = block;
  launch_pca_split(D, a, counts, BH, tr ? tr->perm : nullptr, st);
  launch_pca_finish(out->perm, out->labels, out->seg, out->ncl, L, block, out->ncap, BH, st);
  launch_seg_rowmean(D, X, out->perm, out->seg, out->ncl, L, out->ncap, out->cent, BH, st);
  AC_CHECK_LAUNCH();
  return AC_OK;
}

ac_status check_pca_block(const Plan &P, int block, int ncap) {
  if (block < PCA_BLOCK_MIN || block > PCA_BLOCK_MAX || (block & (block - 1)) != 0)
    return fail(AC_E_ARG, "block %d must be a power of two in [%d, %d]", block, PCA_BLOCK_MIN, PCA_BLOCK_MAX);
  const int64_t nc = cdiv(P.L, block);
  if (nc > ncap)
    return fail(AC_E_ARG, "L / block = %lld clusters exceed the cluster capacity %d", (long long)nc, ncap);
  return AC_OK;
}

// Interaction-aware keys: a fixed count m = min(m0, L) of k-means clusters,
// Euclidean k-means++ seeding, Lloyd iterations and the final assignment
// under the metric M, then the order and statistics as for the other keys.
ac_status do_cluster_k_metric(const Plan &P, const ac_params *p, const uint16_t *K, const uint16_t *V, const float *M,
                              ac_clusters *k, ac_kstats *stats, void *ws, hipStream_t st) {
  const int BH = P.BH, L = P.L, D = P.D;
  const int m = std::min(p->m0, L);
  Engine E{P, P.sk, ws, st};
  launch_fill_i32(E.n(), BH, L, st);
  launch_fill_i32(E.m(), BH, m, st);
  launch_fill_i32(E.coff(), BH, 0, st);
  launch_fill_i32(k->ncl, BH, m, st);
  launch_fill_u8(stats->fallback, BH, 0, st);
  launch_fill_i32(stats->stages, BH, 1, st);
  launch_fill_i32((int *)stats->tau, BH, 0, st);  // +0.0f: no distance threshold
  AC_CHECK_LAUNCH();
  KmArgs a{K, (int64_t)L * D, nullptr, 0, E.n(), E.m(), E.coff(), k->cent, (int64_t)k->ncap * D};
  AC_TRY(E.run(a, m, L, true, p->iters, p, 1, 0, k->labels, M));
  SortArgs s = E.sort_args(k->labels, k->perm, k->seg, k->ncap, m);
  launch_sort(s, BH, L, st);
  const KStatsArgs ks = kstats_args(P, K, V, k, stats, ws);
  launch_kstats(D, ks, BH, st);
  AC_CHECK_LAUNCH();
  return AC_OK;
}

// Scratch of the scoring and selection: the GEMM operands, the score matrix
// (when the caller passes none) and the selected token count of each row.
struct SelScratch {
  uint16_t *A, *Bm;
  float *S;
  int *seltok;
};

SelScratch sel_scratch_ws(const Plan &P, void *ws) {
  return SelScratch{at<uint16_t>(ws, P.scoreA), at<uint16_t>(ws, P.scoreB), at<float>(ws, P.S), at<int>(ws, P.seltok)};
}

ac_status do_score_select(const Plan &P, const ac_params *p, const ac_clusters *q, const ac_clusters *k,
                          const ac_kstats *stats, ac_selection *sel, const SelScratch &sc, hipStream_t st) {
  const int BH = P.BH, D = P.D;
  float *S = sel->score ? sel->score : sc.S;
  ScoreArgs sa;
  sa.cq = q->cent;
  sa.nqcap = q->ncap;
  sa.nq = P.nq;
  sa.kmax = stats->kmax;
  sa.kmin = stats->kmin;
  sa.kmean = stats->kmean;
  sa.seg_k = k->seg;
  sa.ncl_k = k->ncl;
  sa.ncap = k->ncap;
  sa.mode = p->score_mode;
  sa.A = sc.A;
  sa.Bm = sc.Bm;
  sa.nq_pad = P.nq_pad;
  sa.ncap_pad = P.ncap_pad;
  sa.S = S;
  // S rows are q->ncap wide in clusters but the kernels index [nqcap][ncap]
  launch_score(D, sa, BH, st);
  AC_CHECK_LAUNCH();
  SelectArgs se;
  se.S = S;
  se.seg_k = k->seg;
  se.ncl_k = k->ncl;
  se.rho = q->rho;
  se.ncl_q = q->ncl;
  se.nqcap = q->ncap;
  se.ncap = k->ncap;
  se.L = P.L;
  se.D = D;
  se.mode = p->sel_mode;
  se.topk = p->topk;
  se.param = p->sel_param;
  se.scale = attn_scale(p, D);
  se.list = sel->list;
  se.nsel = sel->n;
  se.mask = sel->mask;
  se.mwords = P.mwords;
  se.seltok = sc.seltok;
  launch_select(se, BH, st);
  AC_CHECK_LAUNCH();
  return AC_OK;
}

ac_status do_tail_merge(const Plan &P, int block, const ac_clusters *qi, const ac_selection *si, ac_clusters *qo,
                        ac_selection *so, void *ws, hipStream_t st) {
  TailArgs t;
  t.seg_in = qi->seg;
  t.perm_in = qi->perm;
  t.ncl = qi->ncl;
  t.list_in = si->list;
  t.n_in = si->n;
  t.mask_in = si->mask;
  t.seg_out = qo->seg;
  t.perm_out = qo->perm;
  t.labels_out = qo->labels;
  t.list_out = so->list;
  t.n_out = so->n;
  t.mask_out = so->mask;
  t.plan = at<int>(ws, P.tm_plan);
  t.nq = P.nq;
  t.ncapk = P.ncapk;
  t.mwords = P.mwords;
  t.L = P.L;
  t.block = block > 0 ? block : att_query_tile(P.D);
  launch_tail_merge(t, P.BH, st);
  launch_copy_i32(qi->ncl, qo->ncl, P.BH, st);
  AC_CHECK_LAUNCH();
  return AC_OK;
}

ac_status do_attn(const Plan &P, const ac_params *p, const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                  const ac_clusters *q, const ac_clusters *k, const ac_kstats *stats, const ac_selection *sel,
                  uint16_t *O, float *lse, void *ws, hipStream_t st) {
  const int BH = P.BH, D = P.D;
  AttnArgs a;
  a.Q = Q; a.K = K; a.V = V;
  a.perm_q = q->perm; a.seg_q = q->seg; a.ncl_q = q->ncl; a.nqcap = q->ncap;
  a.perm_k = k->perm; a.seg_k = k->seg; a.ncl_k = k->ncl; a.ncap = k->ncap;
  a.list = sel->list; a.nsel = sel->n; a.mask = sel->mask; a.mwords = P.mwords;
  a.fallback = stats->fallback;
  a.all_dense = p->sel_mode == AC_SEL_DENSE;
  a.compensate = p->compensate;
  a.kc = at<uint16_t>(ws, P.kc);
  a.vc = at<uint16_t>(ws, P.vc);
  a.rows = at<int>(ws, P.rows);
  a.rows_ld = rows_ld(P.L);
  a.pb_ld = rows_ld(P.ncapk);
  a.rows_T = at<int>(ws, P.rows_T);
  a.pbias = at<float>(ws, P.pbias);
  a.tile_off = at<int>(ws, P.tile_off);
  a.O = O;
  a.lse = lse;
  a.L = P.L;
  a.scale_log2 = attn_scale(p, D) * 1.44269504088896340736f;
  launch_attn_prep(D, a, stats->kmean, stats->vmean, at<uint16_t>(ws, P.kc), at<uint16_t>(ws, P.vc),
                   at<int>(ws, P.tile_off), at<long long>(ws, P.pairs), BH, st);
  AC_CHECK_LAUNCH();
  const int max_blocks = (int)cdiv(P.L, att_query_tile(D)) + q->ncap;
  launch_attn(D, a, BH, max_blocks, st);
  AC_CHECK_LAUNCH();
  return AC_OK;
}

// pointer checks for the public structs
ac_status check_clusters(const ac_clusters *c, const char *what, int need_cap, bool need_rho) {
  if (!c) return fail(AC_E_ARG, "%s clusters is NULL", what);
  if (!c->labels || !c->perm || !c->seg || !c->cent || !c->ncl) return fail(AC_E_ARG, "%s clusters has a NULL array", what);
  if (need_rho && !c->rho) return fail(AC_E_ARG, "%s clusters needs rho", what);
  if (c->ncap < need_cap) return fail(AC_E_ARG, "%s clusters capacity %d is below %d", what, c->ncap, need_cap);
  return AC_OK;
}
ac_status check_kstats(const ac_kstats *s) {
  if (!s) return fail(AC_E_ARG, "kstats is NULL");
  if (!s->kmax || !s->kmin || !s->kmean || !s->vmean || !s->fallback || !s->tau || !s->mse || !s->stages)
    return fail(AC_E_ARG, "kstats has a NULL array");
  return AC_OK;
}
ac_status check_sel(const ac_selection *s, int ncapk) {
  if (!s) return fail(AC_E_ARG, "selection is NULL");
  if (!s->list || !s->n || !s->mask) return fail(AC_E_ARG, "selection has a NULL array");
  if (s->ncap_k != ncapk) return fail(AC_E_ARG, "selection ncap_k %d differs from the key capacity %d", s->ncap_k, ncapk);
  return AC_OK;
}

}  // namespace
}  // namespace ac

using namespace ac;

AC_API ac_status ac_params_default(ac_params *p) {
  if (!p) return fail(AC_E_ARG, "params is NULL");
  std::memset(p, 0, sizeof(*p));
  p->nq = 65;
  p->iters = 10;
  p->iters_warm = 3;
  p->m0 = 200;
  p->nmax = 1500;
  p->tau_rule = AC_TAU_MEAN_X;
  p->tau_param = 1.5f;
  p->score_mode = AC_SCORE_QUEST;
  p->sel_mode = AC_SEL_DENSITY;
  p->topk = 8;
  p->sel_param = 0.15f;
  p->compensate = 0;
  p->scale = 0.f;
  p->init_sample = 8;
  p->seed = 0;
  return AC_OK;
}

AC_API ac_status ac_sizes(const ac_shape *s, const ac_params *p, int32_t *ncap_k, size_t *ws_bytes) {
  AC_TRY(check_shape(s));
  AC_TRY(check_params(s, p));
  if (!ncap_k || !ws_bytes) return fail(AC_E_ARG, "output pointer is NULL");
  Plan P = make_plan(s, p);
  *ncap_k = P.ncapk;
  *ws_bytes = P.total;
  return AC_OK;
}

AC_API ac_status ac_cluster_q(const ac_shape *s, const ac_params *p, const uint16_t *Q, const float *warm_cent,
                              ac_clusters *q_out, void *ws, size_t ws_bytes, ac_stream_t stream) {
  AC_TRY(check_shape(s));
  AC_TRY(check_params(s, p));
  if (!Q) return fail(AC_E_ARG, "Q is NULL");
  Plan P = make_plan(s, p);
  AC_TRY(check_clusters(q_out, "query", P.nq, true));
  if (q_out->ncap != P.nq) return fail(AC_E_ARG, "query clusters ncap must be min(nq, L) = %d", P.nq);
  AC_TRY(check_ws(P, ws, ws_bytes));
  AC_TRY(check_device());
  return do_cluster_q(P, p, Q, warm_cent, q_out, ws, (hipStream_t)stream);
}

AC_API ac_status ac_cluster_k(const ac_shape *s, const ac_params *p, const uint16_t *K, const uint16_t *V,
                              const ac_state *warm, ac_clusters *k_out, ac_kstats *stats, void *ws, size_t ws_bytes,
                              ac_stream_t stream) {
  AC_TRY(check_shape(s));
  AC_TRY(check_params(s, p));
  if (!K || !V) return fail(AC_E_ARG, "K or V is NULL");
  Plan P = make_plan(s, p);
  AC_TRY(check_clusters(k_out, "key", P.ncapk, false));
  if (k_out->ncap != P.ncapk) return fail(AC_E_ARG, "key clusters ncap must be %d", P.ncapk);
  AC_TRY(check_kstats(stats));
  const bool is_warm = warm && warm->valid;
  if (is_warm && (!warm->cent_k || !warm->ncl_k || !warm->fallback || !warm->tau))
    return fail(AC_E_ARG, "warm state has a NULL array");
  AC_TRY(check_ws(P, ws, ws_bytes));
  AC_TRY(check_device());
  if (is_warm) return do_cluster_k_warm(P, p, K, V, warm, k_out, stats, ws, (hipStream_t)stream);
  return do_cluster_k_cold(P, p, K, V, k_out, stats, ws, (hipStream_t)stream);
}

AC_API ac_status ac_cluster_k_trace(const ac_shape *s, const ac_params *p, const uint16_t *K, const uint16_t *V,
                                    ac_clusters *k_out, ac_kstats *stats, const ac_ktrace *trace, void *ws,
                                    size_t ws_bytes, ac_stream_t stream) {
  AC_TRY(check_shape(s));
  AC_TRY(check_params(s, p));
  if (!K || !V) return fail(AC_E_ARG, "K or V is NULL");
  if (!trace || trace->max_stages < 1) return fail(AC_E_ARG, "trace is NULL or max_stages < 1");
  Plan P = make_plan(s, p);
  AC_TRY(check_clusters(k_out, "key", P.ncapk, false));
  if (k_out->ncap != P.ncapk) return fail(AC_E_ARG, "key clusters ncap must be %d", P.ncapk);
  AC_TRY(check_kstats(stats));
  AC_TRY(check_ws(P, ws, ws_bytes));
  AC_TRY(check_device());
  return do_cluster_k_cold(P, p, K, V, k_out, stats, ws, (hipStream_t)stream, trace);
}

AC_API ac_status ac_cluster_q_trace(const ac_shape *s, const ac_params *p, const uint16_t *Q, ac_clusters *q_out,
                                    float *cent_trace, void *ws, size_t ws_bytes, ac_stream_t stream) {
  AC_TRY(check_shape(s));
  AC_TRY(check_params(s, p));
  if (!Q || !cent_trace) return fail(AC_E_ARG, "Q or cent_trace is NULL");
  Plan P = make_plan(s, p);
  AC_TRY(check_clusters(q_out, "query", P.nq, true));
  if (q_out->ncap != P.nq) return fail(AC_E_ARG, "query clusters ncap must be min(nq, L) = %d", P.nq);
  AC_TRY(check_ws(P, ws, ws_bytes));
  AC_TRY(check_device());
  return do_cluster_q(P, p, Q, nullptr, q_out, ws, (hipStream_t)stream, cent_trace);
}

AC_API ac_status ac_cluster_q_pca(const ac_shape *s, const ac_params *p, const uint16_t *Q, int32_t block,
                                  ac_clusters *q_out, const ac_pca_trace *trace, void *ws, size_t ws_bytes,
                                  ac_stream_t stream) {
  AC_TRY(check_shape(s));
  AC_TRY(check_params(s, p));
  if (!Q) return fail(AC_E_ARG, "Q is NULL");
  Plan P = make_plan(s, p);
  AC_TRY(check_clusters(q_out, "query", P.nq, true));
  if (q_out->ncap != P.nq) return fail(AC_E_ARG, "query clusters ncap must be min(nq, L) = %d", P.nq);
  AC_TRY(check_pca_block(P, block, q_out->ncap));
  AC_TRY(check_ws(P, ws, ws_bytes));
  AC_TRY(check_device());
  hipStream_t st = (hipStream_t)stream;
  uint16_t *qhat = at<uint16_t>(ws, P.qhat);
  float *qn = at<float>(ws, P.qn);
  launch_qnorm(P.D, Q, qhat, qn, (int64_t)P.BH * P.L, st);
  AC_TRY(do_pca_split(P, qhat, block, q_out, trace, ws, st, true));
  launch_seg_mean(qn, q_out->perm, q_out->seg, P.L, q_out->ncap, q_out->ncl, q_out->rho, P.BH, st);
  AC_CHECK_LAUNCH();
  return AC_OK;
}

AC_API ac_status ac_cluster_k_pca(const ac_shape *s, const ac_params *p, const uint16_t *K, const uint16_t *V,
                                  int32_t block, ac_clusters *k_out, ac_kstats *stats, const ac_pca_trace *trace,
                                  void *ws, size_t ws_bytes, ac_stream_t stream) {
  AC_TRY(check_shape(s));
  AC_TRY(check_params(s, p));
  if (!K || !V) return fail(AC_E_ARG, "K or V is NULL");
  Plan P = make_plan(s, p);
  AC_TRY(check_clusters(k_out, "key", P.ncapk, false));
  if (k_out->ncap != P.ncapk) return fail(AC_E_ARG, "key clusters ncap must be %d", P.ncapk);
  AC_TRY(check_kstats(stats));
  AC_TRY(check_pca_block(P, block, k_out->ncap));
  AC_TRY(check_ws(P, ws, ws_bytes));
  AC_TRY(check_device());
  hipStream_t st = (hipStream_t)stream;
  const int BH = P.BH;
  AC_TRY(do_pca_split(P, K, block, k_out, trace, ws, st, false));
  const KStatsArgs ks = kstats_args(P, K, V, k_out, stats, ws);
  launch_kstats(P.D, ks, BH, st);
  launch_fill_u8(stats->fallback, BH, 0, st);
  launch_fill_i32((int *)stats->tau, BH, 0, st);  // +0.0f: no distance threshold
  launch_fill_i32(stats->stages, BH, (int)pca_level_counts(P.L, block).size(), st);
  AC_CHECK_LAUNCH();
  return AC_OK;
}

AC_API ac_status ac_score_select(const ac_shape *s, const ac_params *p, const ac_clusters *q, const ac_clusters *k,
                                 const ac_kstats *stats, ac_selection *sel, void *ws, size_t ws_bytes,
                                 ac_stream_t stream) {
  AC_TRY(check_shape(s));
  AC_TRY(check_params(s, p));
  Plan P = make_plan(s, p);
  AC_TRY(check_clusters(q, "query", P.nq, true));
  if (q->ncap != P.nq) return fail(AC_E_ARG, "query clusters ncap must be min(nq, L) = %d", P.nq);
  AC_TRY(check_clusters(k, "key", P.ncapk, false));
  if (k->ncap != P.ncapk) return fail(AC_E_ARG, "key clusters ncap must be %d", P.ncapk);
  AC_TRY(check_kstats(stats));
  AC_TRY(check_sel(sel, P.ncapk));
  AC_TRY(check_ws(P, ws, ws_bytes));
  AC_TRY(check_device());
  return do_score_select(P, p, q, k, stats, sel, sel_scratch_ws(P, ws), (hipStream_t)stream);
}

namespace ac {
namespace {
// Scratch of ac_score_select_noalloc: a fixed array in device memory, one copy
// per GPU the library runs on, held until the process ends.  Host code never
// uses the array's name as an address: hipGetSymbolAddress gives each device's
// copy, looked up once per device with that device current.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

ac_status scratch_address(unsigned char **out) {
  static std::mutex mu;
  static void *addr[64] = {};
  int dev = 0;
  AC_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return fail(AC_E_DEVICE, "device ordinal %d out of range", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *ptr = nullptr;
    AC_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (!ptr) return fail(AC_E_DEVICE, "hipGetSymbolAddress returned no address for the scratch array");
    addr[dev] = ptr;
  }
  *out = static_cast<unsigned char *>(addr[dev]);
  return AC_OK;
}

// Carve the scoring scratch from `base`; returns the bytes it needs.
size_t sel_scratch_fixed(const Plan &P, bool need_S, unsigned char *base, SelScratch *sc) {
  const size_t BH = P.BH, D = P.D;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + std::max<size_t>(bytes, 1));
    return o;
  };
  const size_t a = take(BH * P.nq_pad * 6 * D * 2);
  const size_t b = take(BH * P.ncap_pad * 6 * D * 2);
  const size_t s = need_S ? take(BH * P.nq * (size_t)P.ncapk * 4) : 0;
  const size_t t = take(BH * P.nq * 4);
  if (sc && base)
    *sc = SelScratch{reinterpret_cast<uint16_t *>(base + a), reinterpret_cast<uint16_t *>(base + b),
                     need_S ? reinterpret_cast<float *>(base + s) : nullptr, reinterpret_cast<int *>(base + t)};
  return off;
}
}  // namespace
}  // namespace ac

AC_API ac_status ac_score_select_noalloc(const ac_shape *s, const ac_params *p, const ac_clusters *q,
                                         const ac_clusters *k, const ac_kstats *stats, ac_selection *sel,
                                         ac_stream_t stream) {
  AC_TRY(check_shape(s));
  AC_TRY(check_params(s, p));
  Plan P = make_plan(s, p);
  AC_TRY(check_clusters(q, "query", P.nq, true));
  if (q->ncap != P.nq) return fail(AC_E_ARG, "query clusters ncap must be min(nq, L) = %d", P.nq);
  AC_TRY(check_clusters(k, "key", P.ncapk, false));
  if (k->ncap != P.ncapk) return fail(AC_E_ARG, "key clusters ncap must be %d", P.ncapk);
  AC_TRY(check_kstats(stats));
  AC_TRY(check_sel(sel, P.ncapk));
  const size_t need = sel_scratch_fixed(P, sel->score == nullptr, nullptr, nullptr);
  if (need > NOALLOC_SCRATCH_BYTES)
    return fail(AC_E_UNSUPPORTED,
                "ac_score_select_noalloc needs %zu bytes of scratch for this shape; its fixed array holds %zu "
                "(use ac_score_select with a workspace, fewer heads per call, or pass sel->score)",
                need, NOALLOC_SCRATCH_BYTES);
  AC_TRY(check_device());
  unsigned char *base = nullptr;
  AC_TRY(scratch_address(&base));
  SelScratch sc;
  sel_scratch_fixed(P, sel->score == nullptr, base, &sc);
  return do_score_select(P, p, q, k, stats, sel, sc, (hipStream_t)stream);
}

AC_API ac_status ac_sparse_attn(const ac_shape *s, const ac_params *p, const uint16_t *Q, const uint16_t *K,
                                const uint16_t *V, const ac_clusters *q, const ac_clusters *k, const ac_kstats *stats,
                                const ac_selection *sel, uint16_t *O, float *lse, void *ws, size_t ws_bytes,
                                ac_stream_t stream) {
  AC_TRY(check_shape(s));
  AC_TRY(check_params(s, p));
  if (!Q || !K || !V || !O) return fail(AC_E_ARG, "Q, K, V or O is NULL");
  Plan P = make_plan(s, p);
  AC_TRY(check_clusters(q, "query", P.nq, false));
  if (q->ncap != P.nq) return fail(AC_E_ARG, "query clusters ncap must be min(nq, L) = %d", P.nq);
  AC_TRY(check_clusters(k, "key", P.ncapk, false));
  if (k->ncap != P.ncapk) return fail(AC_E_ARG, "key clusters ncap must be %d", P.ncapk);
  AC_TRY(check_kstats(stats));
  AC_TRY(check_sel(sel, P.ncapk));
  AC_TRY(check_ws(P, ws, ws_bytes));
  AC_TRY(check_device());
  return do_attn(P, p, Q, K, V, q, k, stats, sel, O, lse, ws, (hipStream_t)stream);
}

AC_API ac_status ac_tail_merge(const ac_shape *s, const ac_params *p, int32_t block, const ac_clusters *q_in,
                               const ac_selection *sel_in, ac_clusters *q_out, ac_selection *sel_out, void *ws,
                               size_t ws_bytes, ac_stream_t stream) {
  AC_TRY(check_shape(s));
  AC_TRY(check_params(s, p));
  if (block < 0) return fail(AC_E_ARG, "block must be >= 0");
  Plan P = make_plan(s, p);
  AC_TRY(check_clusters(q_in, "query", P.nq, false));
  if (q_in->ncap != P.nq) return fail(AC_E_ARG, "query clusters ncap must be min(nq, L) = %d", P.nq);
  if (!q_out || !q_out->labels || !q_out->perm || !q_out->seg || !q_out->ncl)
    return fail(AC_E_ARG, "output query clusters is NULL or has a NULL array");
  if (q_out->ncap != P.nq) return fail(AC_E_ARG, "output query clusters ncap must be min(nq, L) = %d", P.nq);
  if (q_out->perm == q_in->perm || q_out->seg == q_in->seg || q_out->labels == q_in->labels)
    return fail(AC_E_ARG, "output query clusters alias the input");
  AC_TRY(check_sel(sel_in, P.ncapk));
  AC_TRY(check_sel(sel_out, P.ncapk));
  if (sel_out->list == sel_in->list || sel_out->n == sel_in->n || sel_out->mask == sel_in->mask)
    return fail(AC_E_ARG, "output selection aliases the input");
  AC_TRY(check_ws(P, ws, ws_bytes));
  AC_TRY(check_device());
  return do_tail_merge(P, block, q_in, sel_in, q_out, sel_out, ws, (hipStream_t)stream);
}

AC_API ac_status ac_score_tokens(const ac_shape *s, const ac_params *p, const uint16_t *Q, const ac_clusters *k,
                                 const ac_kstats *stats, int32_t engine, float *S, int32_t ld, ac_stream_t stream) {
  AC_TRY(check_shape(s));
  AC_TRY(check_params(s, p));
  if (!Q || !S) return fail(AC_E_ARG, "Q or S is NULL");
  if (engine != AC_QUEST_MFMA && engine != AC_QUEST_VALU) return fail(AC_E_ARG, "engine %d is not AC_QUEST_*", engine);
  if (ld < 1) return fail(AC_E_ARG, "ld must be >= 1 (got %d)", ld);
  Plan P = make_plan(s, p);
  if (!k || !k->seg || !k->ncl) return fail(AC_E_ARG, "key clusters is NULL or has a NULL seg / ncl");
  if (k->ncap != P.ncapk) return fail(AC_E_ARG, "key clusters ncap must be %d", P.ncapk);
  if (!stats || !stats->kmax || !stats->kmin) return fail(AC_E_ARG, "kstats is NULL or has a NULL kmax / kmin");
  AC_TRY(check_device());
  TokQuestArgs a;
  a.Q = Q;
  a.kmax = stats->kmax;
  a.kmin = stats->kmin;
  a.seg = k->seg;
  a.ncl = k->ncl;
  a.ncap = P.ncapk;
  a.S = S;
  a.ld = ld;
  a.L = P.L;
  launch_token_quest(P.D, a, engine, P.BH, (hipStream_t)stream);
  AC_CHECK_LAUNCH();
  return AC_OK;
}

AC_API ac_status ac_interaction_matrix(const ac_shape *s, const ac_params *p, const uint16_t *Q, const ac_clusters *q,
                                       float *M, void *ws, size_t ws_bytes, ac_stream_t stream) {
  AC_TRY(check_shape(s));
  AC_TRY(check_params(s, p));
  if (!Q || !M) return fail(AC_E_ARG, "Q or M is NULL");
  Plan P = make_plan(s, p);
  AC_TRY(check_clusters(q, "query", P.nq, false));
  if (q->ncap != P.nq) return fail(AC_E_ARG, "query clusters ncap must be min(nq, L) = %d", P.nq);
  AC_TRY(check_ws(P, ws, ws_bytes));
  AC_TRY(check_device());
  hipStream_t st = (hipStream_t)stream;
  launch_interaction_matrix(P.D, Q, q->perm, q->seg, q->ncl, P.L, P.nq, P.nq, at<double>(ws, P.qsum),
                            at<int>(ws, P.qcnt), M, P.BH, st);
  AC_CHECK_LAUNCH();
  return AC_OK;
}

AC_API ac_status ac_cluster_k_metric(const ac_shape *s, const ac_params *p, const uint16_t *K, const uint16_t *V,
                                     const float *M, ac_clusters *k_out, ac_kstats *stats, void *ws, size_t ws_bytes,
                                     ac_stream_t stream) {
  AC_TRY(check_shape(s));
  AC_TRY(check_params(s, p));
  if (!K || !V || !M) return fail(AC_E_ARG, "K, V or M is NULL");
  Plan P = make_plan(s, p);
  AC_TRY(check_clusters(k_out, "key", P.ncapk, false));
  if (k_out->ncap != P.ncapk) return fail(AC_E_ARG, "key clusters ncap must be %d", P.ncapk);
  AC_TRY(check_kstats(stats));
  AC_TRY(check_ws(P, ws, ws_bytes));
  AC_TRY(check_device());
  return do_cluster_k_metric(P, p, K, V, M, k_out, stats, ws, (hipStream_t)stream);
}

namespace ac {
namespace {
// A second stream (default priority) per device and host thread, created on
// first use and kept until the process ends: ac_layer runs the query
// clustering on it, beside the key clustering, which shares no scratch with
// it and reads nothing it writes.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
// Auxiliary streams of the library (default priority), per device and host
// thread, created on first use and kept until the process ends: 0 runs the
// query clustering beside the key clustering (ac_layer), 1 the per-stage
// merges of the final key assignment.
ac_status aux_stream(int which, hipStream_t *out, hipEvent_t *fork, hipEvent_t *join) {
  static thread_local SideStream tab[2][64];
  int dev = 0;
  AC_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64 || which < 0 || which > 1) return fail(AC_E_DEVICE, "device ordinal %d out of range", dev);
  SideStream &x = tab[which][dev];
  if (!x.s) {
    AC_HIP(hipStreamCreateWithFlags(&x.s, hipStreamNonBlocking));
    AC_HIP(hipEventCreateWithFlags(&x.fork, hipEventDisableTiming));
    AC_HIP(hipEventCreateWithFlags(&x.join, hipEventDisableTiming));
  }
  *out = x.s;
  if (fork) *fork = x.fork;
  if (join) *join = x.join;
  return AC_OK;
}

// Pinned host staging for the stage counts, per device and host thread, grown
// on demand and kept until the process ends.
ac_status pinned_i32(int n, int **out) {
  static thread_local int *buf[64] = {};
  static thread_local int cap[64] = {};
  int dev = 0;
  AC_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return fail(AC_E_DEVICE, "device ordinal %d out of range", dev);
  if (cap[dev] < n) {
    if (buf[dev]) AC_HIP(hipHostFree(buf[dev]));
    buf[dev] = nullptr;
    cap[dev] = 0;
    void *p = nullptr;
    AC_HIP(hipHostMalloc(&p, (size_t)n * 4, hipHostMallocDefault));
    buf[dev] = static_cast<int *>(p);
    cap[dev] = n;
  }
  *out = buf[dev];
  return AC_OK;
}

ac_status side_stream(SideStream **out) {
  static thread_local SideStream tab[64];
  int dev = 0;
  AC_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return fail(AC_E_DEVICE, "device ordinal %d out of range", dev);
  SideStream &x = tab[dev];
  if (!x.s) {
    AC_HIP(hipStreamCreateWithFlags(&x.s, hipStreamNonBlocking));
    AC_HIP(hipEventCreateWithFlags(&x.fork, hipEventDisableTiming));
    AC_HIP(hipEventCreateWithFlags(&x.join, hipEventDisableTiming));
  }
  *out = &x;
  return AC_OK;
}
}  // namespace
}  // namespace ac

AC_API ac_status ac_layer(const ac_shape *s, const ac_params *p, const uint16_t *Q, const uint16_t *K,
                          const uint16_t *V, ac_state *state, uint16_t *O, ac_layer_stats *host_stats, void *ws,
                          size_t ws_bytes, ac_stream_t stream) {
  AC_TRY(check_shape(s));
  AC_TRY(check_params(s, p));
  if (!Q || !K || !V || !O) return fail(AC_E_ARG, "Q, K, V or O is NULL");
  if (!state || !state->cent_q || !state->cent_k || !state->ncl_k || !state->fallback || !state->tau)
    return fail(AC_E_ARG, "state is NULL or has a NULL array");
  Plan P = make_plan(s, p);
  AC_TRY(check_ws(P, ws, ws_bytes));
  AC_TRY(check_device());
  hipStream_t st = (hipStream_t)stream;
  const int BH = P.BH, D = P.D;
  ac_clusters q{P.nq, at<int>(ws, P.q_labels), at<int>(ws, P.q_perm), at<int>(ws, P.q_seg), at<float>(ws, P.q_cent),
                at<int>(ws, P.q_ncl), at<float>(ws, P.q_rho)};
  ac_clusters k{P.ncapk, at<int>(ws, P.k_labels), at<int>(ws, P.k_perm), at<int>(ws, P.k_seg), at<float>(ws, P.k_cent),
                at<int>(ws, P.k_ncl), nullptr};
  ac_kstats ks{at<uint16_t>(ws, P.kmax), at<uint16_t>(ws, P.kmin), at<float>(ws, P.kmean), at<float>(ws, P.vmean),
               at<uint8_t>(ws, P.fb), at<float>(ws, P.tau), at<float>(ws, P.mse), at<int>(ws, P.stages)};
  ac_selection sel{P.ncapk, at<int>(ws, P.sel_list), at<int>(ws, P.sel_n), at<uint32_t>(ws, P.sel_mask),
                   at<float>(ws, P.sel_score)};
  const double dense_gflop = 4e-9 * (double)BH * (double)P.L * (double)P.L * (double)D;
  const bool small = p->min_sparse_gflop > 0 && dense_gflop < (double)p->min_sparse_gflop;
  if (p->sel_mode == AC_SEL_DENSE || small) {
    // dense attention only: no clustering, one query "cluster" of all tokens
    // per head, the state untouched (the next sparse call starts cold if it
    // is not valid)
    launch_identity_clusters(q.perm, q.seg, q.ncl, P.L, P.nq, BH, st);
    launch_fill_i32(k.ncl, BH, 0, st);
    launch_fill_u8(ks.fallback, BH, 0, st);
    AC_CHECK_LAUNCH();
    ac_params pd = *p;
    pd.sel_mode = AC_SEL_DENSE;
    pd.compensate = 0;
    AC_TRY(do_attn(P, &pd, Q, K, V, &q, &k, &ks, &sel, O, nullptr, ws, st));
    if (host_stats) {
      AC_HIP(hipStreamSynchronize(st));
      for (int h = 0; h < BH; ++h) {
        if (host_stats->ncl_k) host_stats->ncl_k[h] = 0;
        if (host_stats->fallback) host_stats->fallback[h] = 0;
        if (host_stats->tau) host_stats->tau[h] = 0.f;
        if (host_stats->mse) host_stats->mse[h] = 0.f;
        if (host_stats->stages) host_stats->stages[h] = 0;
        if (host_stats->pairs) host_stats->pairs[h] = (int64_t)P.L * P.L;
      }
    }
    return AC_OK;
  }
  const bool warm = state->valid != 0;
  // query clustering on the side stream, key clustering on the caller's
  SideStream *ss = nullptr;
  AC_TRY(side_stream(&ss));
  AC_HIP(hipEventRecord(ss->fork, st));
  AC_HIP(hipStreamWaitEvent(ss->s, ss->fork, 0));
  auto queries = [&]() -> ac_status {
    AC_TRY(do_cluster_q(P, p, Q, warm ? state->cent_q : nullptr, &q, ws, ss->s, nullptr, true));
    AC_HIP(hipEventRecord(ss->join, ss->s));
    return AC_OK;
  };
  // the value means feed only the compensation's pseudo-keys: without it the
  // key statistics do not read V
  const uint16_t *Vs = p->compensate ? V : nullptr;
  if (warm) {
    AC_TRY(queries());
    AC_TRY(do_cluster_k_warm(P, p, K, Vs, state, &k, &ks, ws, st));
  } else {
    // the query clustering is enqueued once the first key stage is
    AC_TRY(do_cluster_k_cold(P, p, K, Vs, &k, &ks, ws, st, nullptr, queries));
  }
  AC_HIP(hipStreamWaitEvent(st, ss->join, 0));
  AC_TRY(do_score_select(P, p, &q, &k, &ks, &sel, sel_scratch_ws(P, ws), st));
  if (p->tail_block > 0) {
    ac_clusters qm{P.nq, at<int>(ws, P.m_labels), at<int>(ws, P.m_perm), at<int>(ws, P.m_seg), q.cent, q.ncl, q.rho};
    ac_selection sm{P.ncapk, at<int>(ws, P.m_list), at<int>(ws, P.m_n), at<uint32_t>(ws, P.m_mask), nullptr};
    AC_TRY(do_tail_merge(P, p->tail_block, &q, &sel, &qm, &sm, ws, st));
    AC_TRY(do_attn(P, p, Q, K, V, &qm, &k, &ks, &sm, O, nullptr, ws, st));
  } else {
    AC_TRY(do_attn(P, p, Q, K, V, &q, &k, &ks, &sel, O, nullptr, ws, st));
  }
  // carry the centres (and, after a cold step, counts, flags and tau) to the next step
  AC_HIP(hipMemcpyAsync(state->cent_q, q.cent, (size_t)BH * P.nq * D * 4, hipMemcpyDeviceToDevice, st));
  AC_HIP(hipMemcpyAsync(state->cent_k, k.cent, (size_t)BH * P.ncapk * D * 4, hipMemcpyDeviceToDevice, st));
  if (!warm) {
    launch_copy_i32(k.ncl, state->ncl_k, BH, st);
    launch_copy_u8(ks.fallback, state->fallback, BH, st);
    launch_copy_f32(ks.tau, state->tau, BH, st);
    AC_CHECK_LAUNCH();
    state->valid = 1;
  }
  if (host_stats) {
    AC_HIP(hipStreamSynchronize(st));
    if (host_stats->ncl_k) AC_HIP(hipMemcpy(host_stats->ncl_k, k.ncl, BH * 4, hipMemcpyDeviceToHost));
    if (host_stats->fallback) AC_HIP(hipMemcpy(host_stats->fallback, ks.fallback, BH, hipMemcpyDeviceToHost));
    if (host_stats->tau) AC_HIP(hipMemcpy(host_stats->tau, ks.tau, BH * 4, hipMemcpyDeviceToHost));
    if (host_stats->mse) AC_HIP(hipMemcpy(host_stats->mse, ks.mse, BH * 4, hipMemcpyDeviceToHost));
    if (host_stats->stages) AC_HIP(hipMemcpy(host_stats->stages, ks.stages, BH * 4, hipMemcpyDeviceToHost));
    if (host_stats->pairs) AC_HIP(hipMemcpy(host_stats->pairs, at<long long>(ws, P.pairs), BH * 8, hipMemcpyDeviceToHost));
  }
  return AC_OK;
}

// ---------------------------------------------------------------------------
// Multi-step policy (host only).

AC_API ac_status ac_topp_schedule(const double *log_snr, int32_t steps, int32_t warmup_steps, double p_min, double tau,
                                  int32_t t_pivot, float *topp) {
  if (!log_snr || !topp) return fail(AC_E_ARG, "log_snr or topp is NULL");
  if (steps < 2 || warmup_steps < 0 || warmup_steps >= steps - 1)
    return fail(AC_E_ARG, "need steps >= 2 and 0 <= warmup_steps < steps - 1 (got %d, %d)", steps, warmup_steps);
  if (!(p_min > 0.0 && p_min <= 1.0) || !(tau > 0.5 && tau < 1.0))
    return fail(AC_E_ARG, "need 0 < p_min <= 1 and 0.5 < tau < 1");
  for (int t = 0; t < steps; ++t)
    if (!std::isfinite(log_snr[t])) return fail(AC_E_ARG, "log_snr[%d] is not finite", t);
  if (t_pivot < 0) {
    // the sparse step where log SNR changes least
    double best = INFINITY;
    for (int t = warmup_steps; t < steps; ++t) {
      const double d = t + 1 < steps ? std::fabs(log_snr[t + 1] - log_snr[t]) : std::fabs(log_snr[t] - log_snr[t - 1]);
      if (d < best) { best = d; t_pivot = t; }
    }
  } else if (t_pivot < warmup_steps || t_pivot >= steps) {
    return fail(AC_E_ARG, "t_pivot %d outside the sparse steps", t_pivot);
  }
  const double span = log_snr[steps - 1] - log_snr[t_pivot];
  if (!(span > 0.0)) return fail(AC_E_ARG, "log SNR must grow from the pivot step to the last step");
  // sigmoid(k x_last) = tau
  const double k = std::log(tau / (1.0 - tau)) / span;
  for (int t = 0; t < steps; ++t) {
    if (t < warmup_steps) {
      topp[t] = 1.f;
      continue;
    }
    const double x = log_snr[t] - log_snr[t_pivot];
    topp[t] = (float)(p_min + (1.0 - p_min) * (1.0 - 1.0 / (1.0 + std::exp(-k * x))));
  }
  return AC_OK;
}

AC_API ac_status ac_kmax_calibrate(const int32_t *ncl, int32_t units, double frac, int32_t *kmax) {
  if (!ncl || !kmax) return fail(AC_E_ARG, "ncl or kmax is NULL");
  if (units < 1 || !(frac >= 0.0 && frac <= 1.0)) return fail(AC_E_ARG, "need units >= 1 and 0 <= frac <= 1");
  const int nd = (int)std::ceil(frac * units - 1e-9);
  if (nd <= 0) {
    *kmax = 0;
    return AC_OK;
  }
  std::vector<int32_t> v(ncl, ncl + units);
  std::sort(v.begin(), v.end(), [](int32_t a, int32_t b) { return a > b; });
  *kmax = v[std::min(nd, units) - 1];
  return AC_OK;
}

AC_API ac_status ac_step_params(const ac_params *base, const ac_schedule *sch, int32_t step, int32_t layer,
                                ac_params *out) {
  if (!base || !sch || !out) return fail(AC_E_ARG, "base, schedule or out is NULL");
  if (step < 0 || layer < 0) return fail(AC_E_ARG, "step and layer must be >= 0");
  if (sch->warmup_steps < 0 || sch->warmup_layers < 0 || sch->nmax < 0)
    return fail(AC_E_ARG, "schedule counts must be >= 0");
  if (sch->topp && step >= sch->steps) return fail(AC_E_ARG, "step %d beyond the %d scheduled steps", step, sch->steps);
  ac_params p = *base;
  if (step < sch->warmup_steps || layer < sch->warmup_layers) {
    p.sel_mode = AC_SEL_DENSE;
  } else {
    if (sch->nmax > 0) p.nmax = sch->nmax;
    if (sch->topp) {
      p.sel_mode = AC_SEL_TOPP;
      p.sel_param = sch->topp[step];
    }
  }
  *out = p;
  return AC_OK;
}

AC_API const char *ac_status_str(ac_status st) {
  switch (st) {
    case AC_OK: return "ok";
    case AC_E_ARG: return "invalid argument";
    case AC_E_SHAPE: return "invalid shape";
    case AC_E_WORKSPACE: return "workspace too small";
    case AC_E_UNSUPPORTED: return "unsupported configuration";
    case AC_E_DEVICE: return "device error";
  }
  return "unknown status";
}

AC_API const char *ac_last_error(void) { return g_err; }
