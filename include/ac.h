/*
 * ac.h - C ABI of the cluster-routed sparse attention layer for MI355X (gfx950).
 *
 * One attention layer of a video diffusion transformer, made sparse the way
 * AdaCluster (arXiv 2604.18348, "AdaCluster: Adaptive Query-Key Clustering for
 * Sparse Attention in Video Generation") describes it, with the optional
 * stripe-mean compensation of ClusterAttention (arXiv 2608.26965, §1.2):
 *
 *   ac_cluster_q     angular k-means on L2-normalised queries   (AdaCluster §3.1, Algorithm 3 "KMeans(Normalize(Q))")
 *   ac_cluster_k     multi-stage key k-means with dense fallback (AdaCluster §3.2.2, Algorithm 1) + per-cluster statistics
 *   ac_score_select  Quest bound per (query cluster, key cluster) and top-K / density / top-p selection
 *                    (AdaCluster §3.2.3 eq. (1), Algorithm 2, Algorithm 3 "argtopk")
 *   ac_sparse_attn   attention of each query over the keys of its cluster's selected key clusters, with
 *                    optional centroid compensation, or dense attention for fallback heads
 *                    (AdaCluster Algorithm 3; ClusterAttention §1.2 eqs. (2), (5))
 *   ac_score_tokens  Quest bound of every query token against every key cluster (Algorithm 2's literal shape),
 *                    on MFMA (TensorQuest) or on the vector ALUs (eq. (1) as written)
 *   ac_tail_merge    iCATS tail merging of the query clusters before the attention
 *   ac_interaction_matrix, ac_cluster_k_metric
 *                    iCATS interaction-aware key clustering under M_Q from the query clusters
 *   ac_layer         the whole layer, cold (first denoising step) or warm (later steps reuse the cluster
 *                    counts and centres: AdaCluster §3.2.2 "Efficient initialization"), or dense
 *   ac_topp_schedule, ac_kmax_calibrate, ac_step_params
 *                    the multi-step policy: dense warm-up, calibrated k_max, SNR-guided top-p (host only)
 *
 * Conventions (all entry points)
 * ------------------------------
 * Layout    Q, K, V, O are contiguous row-major [B, H, L, d] bfloat16, passed as uint16_t bit patterns.
 *           "BH" below is B*H; every per-head array is indexed by the flattened head b*H + h.
 *           d must be 64 or 128 (AC_E_UNSUPPORTED otherwise).  Self-attention: queries and keys share L.
 *           One head's rows must stay below 4 GiB (L * d * 2 < 2^32: L <= 16,777,215 at d = 128),
 *           else AC_E_UNSUPPORTED.  B*H <= 65,535 (kernels run a row of workgroups per head), else
 *           AC_E_SHAPE.
 * Pointers  Every array pointer is a DEVICE pointer owned by the caller, except the arrays inside
 *           ac_layer_stats, which are HOST pointers.  The library never allocates caller-visible
 *           memory, never frees, and keeps no pointer after a call returns.  Scratch memory is the
 *           caller's workspace `ws` of `ws_bytes` bytes (device memory, 256-byte aligned), sized by
 *           ac_sizes(); its contents are undefined between calls.
 * Streams   Every call enqueues its work on `stream` (a hipStream_t) and returns without waiting,
 *           except: a cold ac_cluster_k / cold ac_layer waits on the stream once per stage of
 *           Algorithm 1 (it reads the size of the unassigned set), and ac_layer waits at its end when
 *           host_stats is not NULL.  Calls on different streams with different buffers are independent.
 *           The query clusterings (ac_cluster_q, ac_cluster_q_pca) and the key clusterings
 *           (ac_cluster_k, ac_cluster_k_pca) use disjoint parts of the workspace, so a query and a key
 *           clustering may run at the same time on two streams that share one workspace (every other
 *           pair of calls that share a workspace must be ordered).  ac_layer does so itself: it runs the query
 *           clustering on a second stream of its own (created on first use, one per device and host
 *           thread, default priority, kept until the process ends) and joins it before returning
 *           control of `stream` to the caller's later work.
 * Errors    Every entry point returns an ac_status.  Argument errors (NULL pointers, bad shapes or
 *           parameters, a workspace that is too small) are detected before any device work is
 *           enqueued, so outputs are untouched.  AC_E_DEVICE reports a HIP runtime error; the text of
 *           the last error on the calling thread is returned by ac_last_error().  The dense fallback of
 *           a head (Algorithm 1's flag F) is a result, not an error.  No C++ exception crosses the ABI.
 * Precision Inputs bf16; k-means distances on bf16 MFMA with fp32 accumulation (centres split into a
 *           bf16 high and low part); statistics accumulate in fp64; attention on bf16 MFMA with fp32
 *           accumulation and an fp32 online softmax; O is rounded to bf16.
 */
#ifndef AC_H_
#define AC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *ac_stream_t; /* a hipStream_t; NULL = the default stream */

typedef enum ac_status {
  AC_OK = 0,
  AC_E_ARG = 1,         /* NULL pointer or invalid parameter value */
  AC_E_SHAPE = 2,       /* invalid B, H, L or d */
  AC_E_WORKSPACE = 3,   /* ws_bytes smaller than ac_sizes() asks for */
  AC_E_UNSUPPORTED = 4, /* valid but not supported by these kernels (e.g. d not in {64, 128}) */
  AC_E_DEVICE = 5       /* HIP runtime error (no device, launch failure, ...) */
} ac_status;

/* Rule for the distance threshold tau of Algorithm 1, taken per head from the stage-0 distances
 * ||k_i - c(k_i)|| (AdaCluster §4.1: 1.5x the mean token-to-centre distance of the first step). */
enum { AC_TAU_MEAN_X = 0, /* tau = tau_param * mean distance */
       AC_TAU_PCTL = 1,   /* tau = nearest-rank percentile: the ceil(tau_param * n)-th smallest distance */
       AC_TAU_ABS = 2,    /* tau = tau_param */
       AC_TAU_INF = 3 };  /* tau = +inf: a single stage */

/* Cluster score (AdaCluster §3.2.3 eq. (1); MEAN is the "w/o Quest" ablation of §4.4). */
enum { AC_SCORE_QUEST = 0, AC_SCORE_MEAN = 1 };

/* Engine of ac_score_tokens. */
enum { AC_QUEST_MFMA = 0, /* TensorQuest: [q+, q-] . [kmax; kmin] as one bf16 MFMA product (eq. (2)) */
       AC_QUEST_VALU = 1  /* eq. (1) per dimension on the vector ALUs (two products, a max, an add) */ };

/* Key-cluster selection per query cluster, in order of score (desc), ties by cluster index (asc).
 * Empty clusters are never selected; at least one cluster always is. */
enum { AC_SEL_TOPK = 0,    /* the first min(topk, non-empty) clusters (Algorithm 3 argtopk) */
       AC_SEL_DENSITY = 1, /* clusters until their summed sizes reach ceil(sel_param * L) keys */
       AC_SEL_TOPP = 2,    /* shortest prefix whose softmax mass reaches sel_param, with
                              pi_c = softmax_c(rho_r * S_rc * scale + ln n_c) */
       AC_SEL_DENSE = 3 }; /* every head dense (the dense baseline) */

typedef struct ac_shape {
  int32_t B, H, L, d;
} ac_shape;

typedef struct ac_params {
  int32_t nq;          /* query clusters (65); min(nq, L) are used */
  int32_t iters;       /* Lloyd iterations of a cold k-means (10) */
  int32_t iters_warm;  /* Lloyd iterations of a warm step (3) */
  int32_t m0;          /* key clusters per stage of Algorithm 1 (200); each stage uses min(|U|, m0) */
  int32_t nmax;        /* N_max: a head falls back to dense attention when a stage would start with
                          at least nmax centres and keys are left (1500) */
  int32_t tau_rule;    /* AC_TAU_* (AC_TAU_MEAN_X) */
  float tau_param;     /* 1.5 */
  int32_t score_mode;  /* AC_SCORE_* (AC_SCORE_QUEST) */
  int32_t sel_mode;    /* AC_SEL_* (AC_SEL_DENSITY) */
  int32_t topk;        /* K of AC_SEL_TOPK (8) */
  float sel_param;     /* density of AC_SEL_DENSITY or p of AC_SEL_TOPP (0.15) */
  int32_t compensate;  /* 1: add every non-empty excluded key cluster as one pseudo-key (key mean,
                          value mean, logit bias ln n_c): ClusterAttention §1.2 eq. (5) (0) */
  float scale;         /* softmax scale; 0 means 1/sqrt(d) (0) */
  int32_t init_sample; /* k-means++ runs on a strided subsample of min(n, init_sample * m) points;
                          0 = every point (8).  The subsample may hold at most 16384 points. */
  int32_t tail_block;  /* ac_layer only: > 0 applies ac_tail_merge with this query block before the
                          attention (iCATS tail merging); 0 = off (0) */
  int32_t min_sparse_gflop; /* ac_layer only: a layer whose dense attention work 4*B*H*L^2*d is below this
                          many GFLOP runs dense (no clustering, the state untouched), since the sparse
                          path has a fixed latency of ~1-2 ms on MI355X (Algorithm 1's stages, k-means++
                          rounds, launches) that such a layer's dense attention does not reach;
                          0 = always sparse (0) */
  uint64_t seed;       /* seed of the counter-based SplitMix64 stream of k-means++ (0) */
} ac_params;

/* Clusters of one side (queries or keys), per head.  All pointers are device pointers. */
typedef struct ac_clusters {
  int32_t ncap;    /* capacity of the per-cluster arrays per head: nq for queries,
                      nmax - 1 + m0 for keys (ac_sizes returns it) */
  int32_t *labels; /* [BH, L]      cluster of each token (original token order) */
  int32_t *perm;   /* [BH, L]      perm[p] = original index of the p-th token in cluster order (stable) */
  int32_t *seg;    /* [BH, ncap+1] first position of each cluster in perm; seg[ncl] = L, and
                      seg[c] = L for ncl <= c <= ncap */
  float *cent;     /* [BH, ncap, d] centres (fp32) after the last Lloyd update */
  int32_t *ncl;    /* [BH]         clusters in use */
  float *rho;      /* [BH, ncap]   queries: mean ||q|| of each cluster's members (0 if empty);
                      may be NULL for keys */
} ac_clusters;

/* Statistics of the final key clusters (device pointers). */
typedef struct ac_kstats {
  uint16_t *kmax;    /* [BH, ncap, d] bf16 per-dimension max of member keys (Quest's max(K^d)) */
  uint16_t *kmin;    /* [BH, ncap, d] bf16 per-dimension min */
  float *kmean;      /* [BH, ncap, d] mean member key   (ClusterAttention's key centroid) */
  float *vmean;      /* [BH, ncap, d] mean member value (its value centroid) */
  uint8_t *fallback; /* [BH] Algorithm 1's F: 1 = the head runs dense attention */
  float *tau;        /* [BH] distance threshold of the head */
  float *mse;        /* [BH] (1/L) sum_i ||k_i - c(k_i)||^2 (AdaCluster §3.2.1); compactness = 1/mse */
  int32_t *stages;   /* [BH] stages Algorithm 1 ran (0 on a warm step) */
} ac_kstats;

/* Selected key clusters per (head, query cluster) (device pointers). */
typedef struct ac_selection {
  int32_t ncap_k;  /* capacity of the key-cluster axis (= the key ac_clusters.ncap) */
  int32_t *list;   /* [BH, nq, ncap_k] selected cluster ids in selection order; the rest undefined */
  int32_t *n;      /* [BH, nq] number selected */
  uint32_t *mask;  /* [BH, nq, ceil(ncap_k/32)] bit c set iff cluster c is selected */
  float *score;    /* [BH, nq, ncap_k] scores (-inf for empty / unused clusters); may be NULL */
} ac_selection;

/* State carried from one denoising step to the next (device pointers, caller-owned).
 * A cold ac_layer fills it and sets valid = 1; a call with valid = 1 runs warm. */
typedef struct ac_state {
  float *cent_q;     /* [BH, nq, d] */
  float *cent_k;     /* [BH, ncap_k, d] */
  int32_t *ncl_k;    /* [BH] */
  uint8_t *fallback; /* [BH] */
  float *tau;        /* [BH] */
  int32_t valid;
} ac_state;

/* Optional per-head summary of ac_layer (HOST pointers, each [BH]; any may be NULL). */
typedef struct ac_layer_stats {
  int32_t *ncl_k;
  uint8_t *fallback;
  float *tau;
  float *mse;
  int32_t *stages;
  int64_t *pairs; /* query-key pairs attended (dense heads: L*L), compensation pseudo-keys excluded */
} ac_layer_stats;

/* Fill *p with the defaults listed in ac_params.  Returns AC_E_ARG if p is NULL. */
ac_status ac_params_default(ac_params *p);

/* Validate shape and parameters and size the workspace.  *ncap_k receives the key-cluster
 * capacity (nmax - 1 + m0) and *ws_bytes the workspace that every entry point accepts
 * for this shape and these parameters.  Host-only: touches no device. */
ac_status ac_sizes(const ac_shape *s, const ac_params *p, int32_t *ncap_k, size_t *ws_bytes);

/* AdaCluster Algorithm 3, "A_q, C_q <- KMeans(Normalize(Q))" (§3.1): each query is divided by its
 * L2 norm and rounded to bf16, then clustered by Euclidean k-means into min(nq, L) clusters
 * (k-means++ seeding and p->iters Lloyd iterations, or p->iters_warm iterations from warm_cent when
 * warm_cent is not NULL), then finally assigned.  Fills q_out (ncap must be >= min(nq, L); rho is
 * required).  Q: [B,H,L,d] bf16; warm_cent: NULL or [BH, q_out->ncap, d] fp32. */
ac_status ac_cluster_q(const ac_shape *s, const ac_params *p, const uint16_t *Q, const float *warm_cent,
                       ac_clusters *q_out, void *ws, size_t ws_bytes, ac_stream_t stream);

/* AdaCluster Algorithm 1 (MultiStageClustering, §3.2.2) on each head's keys, then the statistics
 * of the final clusters.  Cold (warm == NULL): stages of k-means with min(|U|, m0) clusters; keys
 * closer than tau to their stage centre leave U; a head whose centre count reaches nmax with keys
 * left falls back (F = 1); finally every key goes to its nearest centre over all stages.  Warm
 * (warm != NULL and warm->valid): p->iters_warm Lloyd iterations over all keys from warm->cent_k with
 * warm->ncl_k centres; F and tau are copied from warm.  V only feeds vmean.  k_out->ncap must be
 * ac_sizes' ncap_k; k_out->rho may be NULL. */
ac_status ac_cluster_k(const ac_shape *s, const ac_params *p, const uint16_t *K, const uint16_t *V,
                       const ac_state *warm, ac_clusters *k_out, ac_kstats *stats, void *ws,
                       size_t ws_bytes, ac_stream_t stream);

/* Stage-by-stage record of a cold key clustering, so that every step of Algorithm 1 (AdaCluster
 * §3.2.2) and of its k-means (k-means++ seeding, each Lloyd update, the stage's final assignment,
 * the distances that set tau and the removal) can be recomputed from the previous step at any size.
 * Device pointers owned by the caller; any array may be NULL to skip that record.  Stages
 * t >= max_stages run as usual but are not recorded; entries of stages that do not run, and slots
 * beyond n or m, are left as they were. */
typedef struct ac_ktrace {
  int32_t max_stages;
  int32_t *n;      /* [BH, max_stages] |U_t|, the keys still unassigned when stage t starts */
  int32_t *m;      /* [BH, max_stages] m_t, the centres of stage t */
  int32_t *u;      /* [BH, max_stages, L] key index (0..L-1) of the i-th point of U_t, i < n */
  float *cent;     /* [BH, max_stages, iters + 1, m0, d] stage centres (fp32): slot 0 after k-means++
                      seeding, slot j after the j-th Lloyd update, rows c < m */
  int32_t *labels; /* [BH, max_stages, L] stage centre (0..m-1) of the i-th point of U_t after the
                      stage's final assignment */
  float *dist;     /* [BH, max_stages, L] ||k - c|| of the i-th point of U_t to that centre */
} ac_ktrace;

/* ac_cluster_k (cold) with the stage record filled.  Same arguments, outputs and errors as a cold
 * ac_cluster_k; trace must not be NULL and trace->max_stages must be >= 1.  For tests and
 * diagnostics: the copies cost time. */
ac_status ac_cluster_k_trace(const ac_shape *s, const ac_params *p, const uint16_t *K, const uint16_t *V,
                             ac_clusters *k_out, ac_kstats *stats, const ac_ktrace *trace, void *ws,
                             size_t ws_bytes, ac_stream_t stream);

/* ac_cluster_q (cold) with the query centres recorded after k-means++ seeding (slot 0) and after each
 * Lloyd update (slot j): cent_trace [BH, p->iters + 1, q_out->ncap, d] fp32, device memory. */
ac_status ac_cluster_q_trace(const ac_shape *s, const ac_params *p, const uint16_t *Q, ac_clusters *q_out,
                             float *cent_trace, void *ws, size_t ws_bytes, ac_stream_t stream);

/* ClusterAttention's clustering ("ClusterAttention: training-free acceleration of bidirectional
 * attention": abstract, cluster sizes fixed to powers of two; end of section 2, recursive splits along
 * principal components into clusters of a preset size; section 3.1, per head, keys and queries
 * separately).  Per head, a node of n > block rows (initially all L) is cut in two by its leading
 * principal direction: the block * ceil(ceil(n / block) / 2) rows with the smallest projections
 * (ties: lower token index) go left, the rest right, each side keeping its token order; nodes of
 * at most block rows are clusters.  So every cluster holds exactly `block` tokens except the last
 * (L mod block when nonzero), clusters are numbered left to right, and each lists its tokens in
 * ascending order.  The direction of a node is the leading eigenvector of the covariance of a strided
 * subsample {floor(j n / s)} of s = min(n, 512) of its rows, centred and rounded to bf16 (the
 * approximation the page mentions), found as the direction of 64 power iterations from the subsample row
 * farthest from the mean (computed as 8 iterations with the covariance's eighth power) and oriented so
 * that its component of largest magnitude is positive.  block: a power of two in
 * [16, 4096] with ceil(L / block) <= the cluster capacity (AC_E_ARG otherwise).
 *
 * ac_cluster_q_pca clusters the normalised queries (bf16(q / ||q||), as ac_cluster_q): q_out gets
 * labels, perm, seg, ncl = ceil(L / block), cent = member mean of the normalised queries, rho = member
 * mean of ||q||; q_out->ncap = min(p->nq, L) must hold ceil(L / block) clusters.  ac_cluster_k_pca
 * clusters the raw keys: k_out as ac_cluster_k's (cent = member mean) and the statistics of
 * ac_cluster_k, with fallback 0, tau 0 and stages = the number of split levels.  The results feed
 * ac_score_select and ac_sparse_attn; with block equal to the attention's query tile (256 rows at
 * d = 128, 384 is not a power of two so 256 at d = 64 too) no query block is partial.
 * trace (may be NULL): dir [BH, ceil(L / block) - 1, d] fp32, each internal node's direction, levels in
 * order and left to right within a level; perm [BH, levels, L], the token order after each level. */
typedef struct ac_pca_trace {
  float *dir;
  int32_t *perm;
} ac_pca_trace;
ac_status ac_cluster_q_pca(const ac_shape *s, const ac_params *p, const uint16_t *Q, int32_t block,
                           ac_clusters *q_out, const ac_pca_trace *trace, void *ws, size_t ws_bytes,
                           ac_stream_t stream);
ac_status ac_cluster_k_pca(const ac_shape *s, const ac_params *p, const uint16_t *K, const uint16_t *V,
                           int32_t block, ac_clusters *k_out, ac_kstats *stats, const ac_pca_trace *trace,
                           void *ws, size_t ws_bytes, ac_stream_t stream);

/* Scores of every (query cluster r, key cluster c) pair and the selection of key clusters for
 * each query cluster.  QUEST: S_rc = sum_d max(cq_r[d] kmax_c[d], cq_r[d] kmin_c[d]) (AdaCluster
 * eq. (1)), evaluated as the single product [cq+, cq-] . [kmax; kmin] on MFMA (the exact form of
 * eq. (2) with per-cluster max/min vectors); MEAN: S_rc = cq_r . kmean_c.  cq_r is the query
 * cluster centre.  Empty clusters score -inf.  Selection per p->sel_mode (see AC_SEL_*). */
ac_status ac_score_select(const ac_shape *s, const ac_params *p, const ac_clusters *q,
                          const ac_clusters *k, const ac_kstats *stats, ac_selection *sel, void *ws,
                          size_t ws_bytes, ac_stream_t stream);

/* ac_score_select for callers that cannot allocate or pass a workspace (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same kernels and results,
 * with the scratch (the GEMM operands of the scores, the score matrix when sel->score is NULL, and
 * the token count of each selection) in a fixed 64 MiB array of device memory inside the library,
 * one copy per GPU it runs on, kept until the process ends.  Allocates nothing.  Returns
 * AC_E_UNSUPPORTED, before any device work, when the shape needs more scratch than the array holds
 * (about 12 * d * BH * (ncap_k + nq + 32) bytes, plus BH * nq * ncap_k * 4 when sel->score is NULL:
 * e.g. up to 20 heads with the default parameters at d = 128).  Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (several streams or host threads) race, so order them. */
ac_status ac_score_select_noalloc(const ac_shape *s, const ac_params *p, const ac_clusters *q,
                                  const ac_clusters *k, const ac_kstats *stats, ac_selection *sel,
                                  ac_stream_t stream);

/* AdaCluster Algorithm 3 lines "K* <- K[Index], V* <- V[Index], Attention(Q, K*, V*)": every query
 * of query cluster r attends, with scale p->scale (0: 1/sqrt(d)), to the keys of the key clusters
 * selected for r, softmax-normalised over that set (ClusterAttention §1.2 eq. (2)).  With
 * p->compensate every non-empty excluded cluster enters as one pseudo-key (kmean_c, vmean_c, logit
 * bias ln n_c; ClusterAttention eq. (5)).  Heads with fallback = 1, or every head when p->sel_mode is
 * AC_SEL_DENSE, attend densely to all L keys.  Rows are gathered through q->perm and k->perm inside
 * the kernel; O [B,H,L,d] bf16 is written in original token order; lse [BH, L] (natural log of the
 * softmax denominator of the scaled logits) may be NULL. */
ac_status ac_sparse_attn(const ac_shape *s, const ac_params *p, const uint16_t *Q, const uint16_t *K,
                         const uint16_t *V, const ac_clusters *q, const ac_clusters *k,
                         const ac_kstats *stats, const ac_selection *sel, uint16_t *O, float *lse,
                         void *ws, size_t ws_bytes, ac_stream_t stream);

/* Tail merging of the query clusters before the attention ("iCATS: Fast Video Generation via
 * Interaction-Aware Sparse Attention and Timestep-Adaptive Sparsity", method section, tail-merging
 * design, and its worked example).  The attention processes each query cluster in blocks of `block`
 * rows (0: the attention kernel's own query block, 256 rows at d = 128 and 384 at d = 64), so the
 * last, partial block of every cluster costs a whole block for every key it attends to.  Per head: (1) query clusters with identical key-cluster
 * masks merge into the lowest-numbered one (token lists appended in cluster order; no token's key
 * set changes); (2) among the clusters that still have a tail t = size mod block > 0, each pair that
 * are each other's nearest neighbour in Hamming distance between masks (ties to the lower index) and
 * whose tails sum to at most `block` moves the smaller tail (ties: the higher-numbered cluster's) to
 * the other cluster, whose mask becomes the OR of both and whose selection list gains the donor's
 * extra clusters in the donor's order.  Empty clusters take part in neither pass.  Every token
 * attends afterwards to a superset of its original key clusters; the block count never grows.
 * Writes q_out->labels, perm, seg and ncl (cent and rho are not touched and may alias q_in's), and
 * sel_out->list, n and mask (score is not touched).  q_out and sel_out must not alias the inputs.
 * q_in/q_out ncap must be min(nq, L); sel capacities as for ac_score_select. */
ac_status ac_tail_merge(const ac_shape *s, const ac_params *p, int32_t block, const ac_clusters *q_in,
                        const ac_selection *sel_in, ac_clusters *q_out, ac_selection *sel_out, void *ws,
                        size_t ws_bytes, ac_stream_t stream);

/* Quest bound of every query token against every key cluster: AdaCluster Algorithm 2 in its literal
 * shape (one score per query row and key column, the keys reduced to their clusters), each entry
 * eq. (1): S[bh, i, c] = sum_d max(Q[bh, i, d] kmax_c[d], Q[bh, i, d] kmin_c[d]) for the query rows as
 * given (not normalised).  engine AC_QUEST_MFMA evaluates it as TensorQuest, the product
 * [q+, q-] . [kmax; kmin] on bf16 MFMA (q+ = max(q, 0), q- = min(q, 0); every product is exact, the sum
 * accumulates in fp32); AC_QUEST_VALU evaluates eq. (1) per dimension on the vector ALUs, the form
 * §3.2.3 calls too slow (fp32, summed over d in order).  Q: [B,H,L,d] bf16; k and stats as filled by
 * ac_cluster_k (only k->seg, k->ncl, stats->kmax and stats->kmin are read; k->ncap must be ac_sizes'
 * ncap_k).  S: [BH, L, ld] fp32, row-major with leading dimension ld >= 1; columns c < ld are written:
 * the score for a non-empty cluster c < ncl_k[bh], -inf otherwise.  Clusters c >= ld get no score, so
 * pass ld >= the largest ncl_k to score them all.  Needs no workspace. */
ac_status ac_score_tokens(const ac_shape *s, const ac_params *p, const uint16_t *Q, const ac_clusters *k,
                          const ac_kstats *stats, int32_t engine, float *S, int32_t ld, ac_stream_t stream);

/* Interaction-aware key clustering ("iCATS: Fast Video Generation via Interaction-Aware Sparse
 * Attention and Timestep-Adaptive Sparsity", method section, interaction-aware clustering).  The error
 * of the query-key products when a key is replaced by its centre is (k - c) Q^T Q (k - c)^T; the page
 * approximates Q^T Q by M_Q = sum_r |A_r| mu_r^T mu_r over the query clusters A_r.
 *
 * ac_interaction_matrix: M[bh] = M_Q of head bh, with mu_r the mean of the raw member queries of query
 * cluster r of q (as filled by ac_cluster_q: perm, seg and ncl are read).  Q: [B,H,L,d] bf16;
 * M: [BH, d, d] fp32 row-major, accumulated in fp64.
 *
 * ac_cluster_k_metric: k-means of each head's keys into m = min(p->m0, L) clusters whose assignment
 * minimises (k - c) M[bh] (k - c)^T: k-means++ seeding as ac_cluster_k's first stage (Euclidean, the
 * same random stream), p->iters Lloyd iterations (member means, which minimise the form for a positive
 * semi-definite M) and a final assignment; then perm, seg and the statistics as ac_cluster_k.  No
 * stages and no fallback: ncl = m, fallback = 0, tau = 0, stages = 1.  k_out->ncap must be ac_sizes'
 * ncap_k.  The result feeds ac_score_select and ac_sparse_attn like ac_cluster_k's. */
ac_status ac_interaction_matrix(const ac_shape *s, const ac_params *p, const uint16_t *Q, const ac_clusters *q,
                                float *M, void *ws, size_t ws_bytes, ac_stream_t stream);
ac_status ac_cluster_k_metric(const ac_shape *s, const ac_params *p, const uint16_t *K, const uint16_t *V,
                              const float *M, ac_clusters *k_out, ac_kstats *stats, void *ws, size_t ws_bytes,
                              ac_stream_t stream);

/* The whole layer (AdaCluster Algorithm 3 with the optional compensation): ac_cluster_q,
 * ac_cluster_k, ac_score_select, ac_tail_merge when p->tail_block > 0, and ac_sparse_attn on
 * buffers carved from the workspace.  Cold when
 * !state->valid (fills the state and sets valid = 1), warm otherwise.  With p->sel_mode AC_SEL_DENSE
 * it runs dense attention only (no clustering; the state is left as it is; host_stats reports 0
 * clusters and L*L pairs per head).  host_stats may be NULL. */
ac_status ac_layer(const ac_shape *s, const ac_params *p, const uint16_t *Q, const uint16_t *K,
                   const uint16_t *V, ac_state *state, uint16_t *O, ac_layer_stats *host_stats,
                   void *ws, size_t ws_bytes, ac_stream_t stream);

/* ---------------------------------------------------------------------------
 * Multi-step, multi-layer policy (host only: no device work, no workspace).
 * AdaCluster §3.2.2 "Efficient initialization": the multi-stage clustering runs at a layer's first
 * sparse denoising step (ac_layer with a state that is not valid), later steps start from the
 * previous centres with the cluster counts kept (ac_layer warm).  AdaCluster §4.1: k_max (N_max)
 * is set so that the least compact ~15% of attention units use full attention.  iCATS (method
 * section, SNR-guided sparsity, and its warm-up setting): the first steps and layers stay dense; a
 * per-step top-p follows an inverse sigmoid of log SNR.  An attention unit is one (layer, head). */

typedef struct ac_schedule {
  int32_t warmup_steps;  /* steps 0 .. warmup_steps-1 run dense attention */
  int32_t warmup_layers; /* layers 0 .. warmup_layers-1 run dense attention at every step */
  int32_t nmax;          /* calibrated k_max (ac_kmax_calibrate) for the sparse units; 0 keeps base->nmax */
  int32_t steps;         /* entries of topp */
  const float *topp;     /* [steps] HOST per-step p (ac_topp_schedule): sparse units select with
                            AC_SEL_TOPP at that p; NULL keeps base->sel_mode and sel_param */
} ac_schedule;

/* SNR-guided top-p per denoising step: topp[t] = p_min + (1 - p_min) (1 - sigmoid(k x_t)) with
 * x_t = log_snr[t] - log_snr[t_pivot] and k = logit(tau) / (log_snr[steps-1] - log_snr[t_pivot]),
 * so the sigmoid is 1/2 at the pivot and tau at the last step; topp[t] = 1 for t < warmup_steps.
 * t_pivot < 0 picks the sparse step where log SNR changes least (forward difference).  log_snr:
 * [steps] HOST, log((a_t / b_t)^2) of the sampler (x_t = a_t x_0 + b_t eps), growing from the pivot to
 * the last step.  Needs steps >= 2, 0 <= warmup_steps < steps - 1, 0 < p_min <= 1, 0.5 < tau < 1. */
ac_status ac_topp_schedule(const double *log_snr, int32_t steps, int32_t warmup_steps, double p_min, double tau,
                           int32_t t_pivot, float *topp);

/* k_max from the key-cluster counts ncl[units] of an uncapped first step (ac_layer_stats.ncl_k over
 * layers and heads, run with the largest nmax): the count of the unit ranked ceil(frac * units)
 * from the top, 0 when frac * units rounds to no unit.  Run with nmax = k_max, Algorithm 1 decides
 * the fallback: a unit falls back when a stage would start with k_max centres or more and keys are
 * left, so at most that many units fall back. */
ac_status ac_kmax_calibrate(const int32_t *ncl, int32_t units, double frac, int32_t *kmax);

/* The parameters of (step, layer) for ac_layer: base with sel_mode AC_SEL_DENSE during warm-up
 * (steps < warmup_steps or layers < warmup_layers), otherwise with nmax = sch->nmax (if > 0) and,
 * when sch->topp is set, sel_mode AC_SEL_TOPP with sel_param = sch->topp[step]. */
ac_status ac_step_params(const ac_params *base, const ac_schedule *sch, int32_t step, int32_t layer,
                         ac_params *out);

/* Static description of a status code. */
const char *ac_status_str(ac_status st);
/* Text of the last error reported on the calling thread ("" if none). */
const char *ac_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* AC_H_ */
