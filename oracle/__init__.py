"""fp64 CPU oracle for one layer of cluster-routed sparse attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP
library and its Python binding never import it, and it imports nothing from
them: the two share no code.  The only thing both sides consume is the
seeded input generator (``csa_inputs``), which holds none of the method's
arithmetic.

What it computes, step by step, in the order of the pages:

* AdaCluster (arXiv 2604.18348) §3.1 and Algorithm 3 step "KMeans(Normalize(Q))":
  angular k-means on L2-normalised queries  -> ``kmeans.cluster_queries``
* AdaCluster §3.2.2, Algorithm 1 (MultiStageClustering) with dense fallback
  -> ``multistage.cluster_keys``
* AdaCluster §3.2.1 (per-head reconstruction MSE) and eq. (1) (per-dim max/min
  of a key group), ClusterAttention §1.2 eq. (5) (key/value means)
  -> ``stats.key_stats``
* AdaCluster §3.2.3 eq. (1) (Quest upper bound), computed in its literal
  max form -> ``score.quest_scores``; Algorithm 3 argtopk -> ``score.select``
* AdaCluster Algorithm 3 (Attention(Q, K*, V*), full attention when F),
  ClusterAttention §1.2 eqs. (2)-(6) (sparse attention, stripe-mean
  compensation) -> ``attention``
* The whole layer, cold and warm (AdaCluster §3.2.2 "Efficient
  initialization") -> ``layer.run_layer``
* ClusterAttention's recursive split along principal components into
  clusters of a preset power-of-two size (abstract; end of section 2)
  -> ``pcasplit.pca_split``

Where the pages leave a step open, the reading taken is stated in the
docstring of the function that implements it.

Parity status: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_*.py`` except the readings that no page fixes (the m_t
rule for stages after the first, the k-means++ subsample and the order of
its random stream, the choice of the top-p temperature, the empty-cluster
policy and the number of warm iterations).  Those are "parity unpinned":
they are checked only GPU-against-oracle.  (The percentile definition is
pinned to NumPy's inverted-CDF percentile, and the top-p mass to the
attention mass of the kept clusters.)
"""
from .numerics import Params, bf16_round, bf16_to_f64, uniform01, splitmix64_next  # noqa: F401
from . import kmeans, multistage, stats, score, attention, layer, pcasplit  # noqa: F401
