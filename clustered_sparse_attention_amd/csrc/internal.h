// Internal interfaces between the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

namespace ac {

constexpr int KPP_SMAX = 16384;  // most points a k-means++ subsample may hold
constexpr int KPP_GRAM_MAX = 8192;  // subsamples up to this size seed from a distance matrix
constexpr int SORT_TILE = 256;   // points per counting-sort tile (one wave)
constexpr int SORT_GROUP = 32;   // tiles per group in the two-level scan over tiles
constexpr int ATT_QT = 256;      // query rows per attention block at d = 128 (8 waves)
constexpr int ATT_QT64 = 384;    // at d = 64: 12 waves, three per SIMD fit its registers
constexpr int ATT_QG = 1;        // groups of 32 queries per attention wave
template <int D> constexpr int att_qt() { return D == 64 ? ATT_QT64 : ATT_QT; }
inline int att_query_tile(int D) { return D == 64 ? ATT_QT64 : ATT_QT; }
constexpr int ATT_XCD_CHUNK = 4;  // consecutive query tiles kept on one XCD
constexpr int ATT_KT = 64;       // keys per attention tile
constexpr int SEL_MAXN = 4096;   // most key clusters the select kernel sorts
constexpr int ASSIGN_RES_MAX = 224;  // most centres the LDS-resident assignment holds
constexpr int UPD_CHUNK = 256;   // members per block in the centre update
constexpr int KST_FIELDS = 8;    // ints of Algorithm 1's per-head state on the device
constexpr int SORT_SMALL_MAX = 2048;   // points per head up to which one block per head sorts (and updates)
constexpr int SORT_SMALL_M = 256;      // labels that path handles

enum { TAU_RULE_MEAN_X = 0, TAU_RULE_PCTL = 1, TAU_RULE_ABS = 2, TAU_RULE_INF = 3 };

// One batched k-means job (see kmeans.hip).
struct KmArgs {
  const uint16_t *X;  // [BH] heads of rows, head stride x_hs elements, rows of D bf16
  int64_t x_hs;
  const int *idx;     // [BH, idx_hs] point -> row, or NULL (point i is row i)
  int64_t idx_hs;
  const int *n;       // [BH] points per head
  const int *m;       // [BH] centres per head
  const int *coff;    // [BH] first centre of the job in cent
  float *cent;        // [BH, cent_hs] fp32 centres (rows of D)
  int64_t cent_hs;
};

// GEMM operands of the job's centres, indexed by local centre id.
struct CentOps {
  uint16_t *hi;  // [BH, cap, D]
  uint16_t *lo;  // [BH, cap, D]
  float *norm;   // [BH, cap]
  int cap;
};

struct SortArgs {
  const int *labels;  // [BH, lab_hs]
  int64_t lab_hs;
  const int *n;       // [BH]
  const int *m;       // [BH]
  int *tile_hist;     // [BH, max_tiles, mcap]
  int max_tiles;
  int mcap;
  int *grp;           // [BH, max_groups, mcap] per-group label offsets
  int max_groups;
  int *perm;          // [BH, perm_hs]
  int64_t perm_hs;
  int *seg;           // [BH, seg_hs], entries 0..segcap written
  int64_t seg_hs;
  int segcap;
  // Lloyd fixed-point detection (NULL outside the Lloyd loop): a head whose
  // assignment did not change (chg_cur[h] == 0) gets neff[h] = 0 (neff is the
  // n array of the loop), and chg_zero[h] is cleared for the next count
  int *neff;
  const int *chg_cur;
  int *chg_zero;
  // chunk offsets of the centre update (NULL unless the sort feeds one):
  // chunk_off[h][c] = number of UPD_CHUNK-member chunks of labels < c, c <= m
  int *chunk_off;
  int64_t co_hs;
};

struct KStatsArgs {
  const uint16_t *K, *V;  // [BH, L, D]; V NULL: no value means (vmean left as it is)
  const int *perm, *seg;  // [BH, L], [BH, ncap + 1]
  const int *ncl;         // [BH]
  const float *cent;      // [BH, ncap, D]
  uint16_t *kmax, *kmin;  // [BH, ncap, D]
  float *kmean, *vmean;   // [BH, ncap, D]
  double *msepart;        // [BH, ncap]
  float *mse;             // [BH]
  int L, ncap;
  // scratch of the chunked statistics (kst_scratch): chunk and partial-slot
  // offsets [BH, ncap + 1], per-slot partials [BH, pslots, D] and [BH, pslots]
  int *co, *po;
  double *psk, *psv;
  float *pmx, *pmn;
  double *pse;
  int pslots;
};
constexpr int KST_CHUNK = 256;  // members per block of the key statistics
// partial slots per head of the key statistics (fewer than 2 L / KST_CHUNK)
inline int kst_slots(int L) { return 2 * ((L + KST_CHUNK - 1) / KST_CHUNK); }

struct ScoreArgs {
  const float *cq;        // [BH, nqcap, D] query-cluster centres
  int nqcap;              // rows per head of cq / S
  int nq;                 // rows used
  const uint16_t *kmax, *kmin;
  const float *kmean;
  const int *seg_k;       // [BH, ncap + 1]
  const int *ncl_k;       // [BH]
  int ncap;               // key-cluster capacity
  int mode;               // 0 QUEST, 1 MEAN
  uint16_t *A;            // [BH, nq_pad, 6D]
  uint16_t *Bm;           // [BH, ncap_pad, 6D]
  int nq_pad, ncap_pad;
  float *S;               // [BH, nqcap, ncap]
};

struct SelectArgs {
  const float *S;         // [BH, nqcap, ncap]
  const int *seg_k;       // [BH, ncap + 1]
  const int *ncl_k;       // [BH]
  const float *rho;       // [BH, nqcap]
  const int *ncl_q;       // [BH]
  int nqcap, ncap, L, D;
  int mode, topk;
  float param, scale;
  int *list;              // [BH, nqcap, ncap]
  int *nsel;              // [BH, nqcap]
  uint32_t *mask;         // [BH, nqcap, mwords]
  int mwords;
  int *seltok;            // [BH, nqcap] selected key tokens
};

struct AttnArgs {
  const uint16_t *Q, *K, *V;  // [BH, L, D]
  const int *perm_q, *seg_q;  // [BH, L], [BH, nqcap + 1]
  const int *ncl_q;           // [BH]
  int nqcap;
  const int *perm_k, *seg_k;  // [BH, L], [BH, ncap + 1]
  const int *ncl_k;
  int ncap;
  const int *list, *nsel;     // [BH, nqcap, ncap], [BH, nqcap]
  const uint32_t *mask;       // [BH, nqcap, mwords]
  int mwords;
  const uint8_t *fallback;    // [BH] or NULL
  int all_dense;
  int compensate;
  const uint16_t *kc, *vc;    // [BH, ncap, D] bf16 pseudo-keys / values
  int *rows;                  // [BH, nqcap, rows_ld] key rows of each selection, concatenated
  int *rows_T;                // [BH, nqcap] their count (L on fallback heads)
  float *pbias;               // [BH, nqcap, pb_ld] pseudo-key logit bias (base 2)
  int64_t rows_ld, pb_ld;     // row strides, multiples of the key tile
  const int *tile_off;        // [BH, nqcap + 1] first block of each query cluster
  uint16_t *O;                // [BH, L, D]
  float *lse;                 // [BH, L] or NULL
  int L;
  float scale_log2;           // scale * log2(e)
  int blocks_per_head;        // grid layout (set by the launcher)
  int BH;
};

// Tail merging of query clusters (see merge.hip).
struct TailArgs {
  const int *seg_in, *perm_in, *ncl;  // [BH, nq + 1], [BH, L], [BH]
  const int *list_in, *n_in;          // [BH, nq, ncapk], [BH, nq]
  const uint32_t *mask_in;            // [BH, nq, mwords]
  int *seg_out, *perm_out, *labels_out;
  int *list_out, *n_out;
  uint32_t *mask_out;
  int *plan;                          // [BH, 8, nq + 1]
  int nq, ncapk, mwords, L, block;
};

// Recursive principal-component split (see pca.hip).
constexpr int PCA_SMAX = 512;   // subsample points that set a node's direction
constexpr int PCA_BLOCK_MIN = 16, PCA_BLOCK_MAX = 4096;  // cluster sizes (powers of two)
constexpr int PCA_ITERS = 64;   // power iterations per node
// Levels whose largest node has PCA_BIG_NODE points or more run in three
// launches: the directions (a block per node), the projections (a block per
// PCA_PROJ_CHUNK points) and the cuts (a block per node).
constexpr int PCA_BIG_NODE = 16384, PCA_PROJ_CHUNK = 4096;
__host__ __device__ inline int pca_dir_cap(int L) { return L / 4096 + 2; }  // node slots a head for such a level
struct PcaArgs {
  const uint16_t *X;  // [BH, L, D] rows to cluster
  int *perm;          // [BH, L] token order, refined level by level
  int *tmp;           // [BH, L] scratch: the node's tokens before its split
  uint32_t *key;      // [BH, L] scratch: order-preserving projection keys
  int2 *nodes;        // internal nodes (first position, count), levels in order
  int *lvl;           // [levels + 1] first node of each level
  float *dir;         // [BH, ndir, D] direction of each internal node, or NULL
  int ndir;
  float *dbuf;        // [BH, pca_dir_cap(L), D] directions of a level split in three launches
  int L, block;
};

// Per-token Quest scores (see quest.hip).
struct TokQuestArgs {
  const uint16_t *Q;            // [BH, L, D] bf16 query rows
  const uint16_t *kmax, *kmin;  // [BH, ncap, D] bf16
  const int *seg, *ncl;         // [BH, ncap + 1], [BH]
  int ncap;
  float *S;                     // [BH, L, ld]
  int ld;
  int L;
};

// kmeans.hip
void launch_qnorm(int D, const uint16_t *Q, uint16_t *Qh, float *qn, int64_t rows, hipStream_t st);
void launch_kpp(int D, const KmArgs &a, int BH, double *d2buf, int init_sample, uint64_t seed, int role, int stage,
                hipStream_t st);
// after_gram (nullable): recorded on st once the distance matrix is enqueued,
// before the m sequential rounds (one block per head) that read it; returns
// that record's status
hipError_t launch_kpp_gram(int D, const KmArgs &a, int BH, int smax, double *nx, double *G, int init_sample,
                           uint64_t seed, int role, int stage, hipStream_t st, hipEvent_t after_gram = nullptr);
// at_coff: operand rows at the centres' global index coff[h] + c (merge-mode assignment)
void launch_cent_prep(int D, const KmArgs &a, const CentOps &op, int BH, int mmax, hipStream_t st,
                      bool at_coff = false);
// chg (nullable): per-head flag set to 1 when some point's label differs from
// the one already in `labels` (the caller clears it)
// best_io (nullable): merge mode of the resident kernel (mmax <= ASSIGN_RES_MAX):
// the job's centres are one stage's, global index coff[h] + c with operands
// at op row coff[h] + c, merged into the running nearest centre kept in
// labels / best_io (scores x.c - |c|^2/2; -inf = none yet)
// spare_cus: compute units to leave to work running beside this launch, if at
// most a quarter of the device (the resident kernel's grid is one block per
// remaining compute unit)
void launch_assign(int D, const KmArgs &a, const CentOps &op, int BH, int mmax, int nmax_pts, int *labels, int64_t lab_hs,
                   hipStream_t st, int *chg = nullptr, float *best_io = nullptr, int spare_cus = 0);
void launch_sort(const SortArgs &s, int BH, int nmax_pts, hipStream_t st);
void launch_update(int D, const KmArgs &a, const SortArgs &s, const CentOps &op, int BH, int mmax, int npts,
                   double *partial, int64_t part_hs, hipStream_t st);
// one launch each for heads of at most SORT_SMALL_MAX points and SORT_SMALL_M labels
void launch_sort_small(const SortArgs &s, int BH, hipStream_t st);
void launch_update_small(int D, const KmArgs &a, const SortArgs &s, const CentOps &op, int BH, int mmax,
                         hipStream_t st);
void launch_stage_dist(int D, const KmArgs &a, int BH, int nmax_pts, const int *labels, int64_t lab_hs, float *dist,
                       int64_t dist_hs, hipStream_t st);
void launch_tau(const float *dist, int64_t dist_hs, const int *n_arr, int BH, int nmax_pts, int rule, float param,
                float *tau, uint32_t *radix_state, uint32_t *radix_hist, hipStream_t st);
void launch_flag_removed(const float *dist, int64_t dist_hs, const int *n_arr, const float *tau, int *flag,
                         int64_t flag_hs, int BH, int nmax_pts, hipStream_t st);
void launch_compact_gather(const int *idx_old, int64_t idx_hs, const int *perm, int64_t perm_hs, const int *seg,
                           int64_t seg_hs, int *idx_new, int *n_new, int BH, int nmax_pts, hipStream_t st);
void launch_kstats(int D, const KStatsArgs &s, int BH, hipStream_t st);
// Algorithm 1's bookkeeping between stages on the device (state [BH, KST_FIELDS])
void launch_stage_next(int *state, const int *nnew, int *n, int *m, int *coff, int t, int nmax, int m0, int L,
                       int BH, hipStream_t st);
void launch_stage_final(const int *state, int *ncl, uint8_t *fallback, int *stages, int BH, hipStream_t st);
// stage records of the traced entry points
void launch_trace_cent(int D, const KmArgs &a, int BH, int mmax, float *dst, int64_t dst_hs, hipStream_t st);
void launch_trace_stage(const int *n, const int *idx, int64_t idx_hs, const int *lab, const float *dist, int64_t hs,
                        int *u_out, int *lab_out, float *dist_out, int64_t out_hs, int BH, int npts, hipStream_t st);
void launch_trace_nm(const int *n, const int *m, int *n_out, int *m_out, int ld, int t, int BH, hipStream_t st);
void launch_seg_mean(const float *val, const int *perm, const int *seg, int L, int ncap, const int *ncl, float *out,
                     int BH, hipStream_t st);
void launch_fill_i32(int *p, int64_t n, int v, hipStream_t st);
void launch_fill_u8(uint8_t *p, int64_t n, uint8_t v, hipStream_t st);
void launch_identity_clusters(int *perm, int *seg, int *ncl, int L, int segcap, int BH, hipStream_t st);
void launch_copy_i32(const int *s, int *d, int64_t n, hipStream_t st);
void launch_copy_converged(const int *n, const int *neff, const int *src, int *dst, int64_t hs, int npts, int BH,
                           hipStream_t st);
void launch_copy_f32(const float *s, float *d, int64_t n, hipStream_t st);
void launch_copy_u8(const uint8_t *s, uint8_t *d, int64_t n, hipStream_t st);

// select.hip
void launch_score(int D, const ScoreArgs &a, int BH, hipStream_t st);
void launch_select(const SelectArgs &a, int BH, hipStream_t st);

// attn.hip
void launch_attn_prep(int D, const AttnArgs &a, const float *kmean, const float *vmean, uint16_t *kc, uint16_t *vc,
                      int *tile_off, long long *pairs, int BH, hipStream_t st);
void launch_attn(int D, const AttnArgs &a, int BH, int max_blocks, hipStream_t st);

// merge.hip
void launch_tail_merge(const TailArgs &t, int BH, hipStream_t st);

// metric.hip
void launch_interaction_matrix(int D, const uint16_t *Q, const int *perm, const int *seg, const int *ncl, int L,
                               int nq, int nqcap, double *qsum, int *qcnt, float *M, int BH, hipStream_t st);
void launch_cent_prep_metric(int D, const KmArgs &a, const CentOps &op, const float *M, int BH, int mmax,
                             hipStream_t st);

// pca.hip
std::vector<int> pca_level_counts(int n, int b);
void launch_pca_split(int D, const PcaArgs &a, const std::vector<int> &counts, int BH, int *perm_trace,
                      hipStream_t st);
void launch_pca_finish(const int *perm, int *labels, int *seg, int *ncl, int L, int b, int segcap, int BH,
                       hipStream_t st);
void launch_seg_rowmean(int D, const uint16_t *X, const int *perm, const int *seg, const int *ncl, int L, int ncap,
                        float *cent, int BH, hipStream_t st);

// quest.hip (engine 0: MFMA, 1: vector ALU)
void launch_token_quest(int D, const TokQuestArgs &a, int engine, int BH, hipStream_t st);

}  // namespace ac
