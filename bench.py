"""Benchmark of one cluster-routed sparse attention layer on one MI355X.

A step is one pass of the whole layer over one batch of synthetic input:
query clustering, multi-stage key clustering with statistics and the
cluster-order permutations, Quest scoring with selection, and the
block-sparse attention (the four C entry points, in the order ac_layer runs
them).  Inputs are resident in HBM before the timed region.

Prints ONE JSON line.  ``value`` is the dense-equivalent throughput
4*B*H*L^2*d / layer time in TFLOP/s.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def workload_params(name: str, variant: str, compensate: int):
    """Layer hyperparameters of each workload (see csa_inputs for the data)."""
    import clustered_sparse_attention_amd as nm  # enum values (AC_*)
    base = dict(nq=65, iters=10, iters_warm=3, init_sample=8, seed=0, compensate=compensate)
    if name == "tiny":
        base.update(nq=16, m0=32, nmax=64, tau_rule=nm.AC_TAU_INF, tau_param=0.0, sel_mode=nm.AC_SEL_TOPK, topk=8,
                    sel_param=0.0, init_sample=0)
    elif name == "cogvideox":
        base.update(m0=200, nmax=1000, tau_rule=nm.AC_TAU_PCTL, tau_param=0.95, sel_mode=nm.AC_SEL_DENSITY, sel_param=0.10)
    elif name == "hunyuan":
        # AdaCluster's HunyuanVideo setting (Table 7): initial K 100, an absolute key
        # threshold of 5.5, top-K 64.  A fixed threshold singles out the dispersed heads,
        # whose keys stay farther than 5.5 from any centre until N_max stops the stages.
        base.update(m0=100, nmax=1500, tau_rule=nm.AC_TAU_ABS, tau_param=5.5, sel_mode=nm.AC_SEL_TOPK, topk=64,
                    sel_param=0.0)
    elif name == "wan":
        base.update(m0=200, nmax=1500, tau_rule=nm.AC_TAU_MEAN_X, tau_param=1.5, sel_mode=nm.AC_SEL_DENSITY, sel_param=0.15)
        if variant == "topp":
            base.update(sel_mode=nm.AC_SEL_TOPP, sel_param=0.9)
    elif name == "long":
        base.update(m0=200, nmax=1500, tau_rule=nm.AC_TAU_MEAN_X, tau_param=1.5, sel_mode=nm.AC_SEL_DENSITY, sel_param=0.08)
    else:
        raise ValueError(name)
    if variant == "dense":
        base.update(sel_mode=nm.AC_SEL_DENSE)
    return base


def selection_name(kw) -> str:
    """The selection rule of a parameter set, as the pages name it."""
    import clustered_sparse_attention_amd as nm
    mode = kw["sel_mode"]
    if mode == nm.AC_SEL_TOPK:
        return f"top-K {kw['topk']}"
    if mode == nm.AC_SEL_DENSITY:
        return f"top-K at {kw['sel_param']:.0%} density"
    if mode == nm.AC_SEL_TOPP:
        return f"top-p {kw['sel_param']}"
    return "dense"


def _abi(kw):
    import clustered_sparse_attention_amd as ac
    kw = dict(kw)
    kw.setdefault("topk", 8)
    kw.setdefault("score_mode", 0)
    kw.setdefault("scale", 0.0)
    return ac.params_default(**{k: v for k, v in kw.items()})


class Layer:
    """Device buffers of one layer and the four entry points."""

    def __init__(self, Qd, Kd, Vd, shape, params, tail_block=0, key_metric=False, pca=None):
        import torch
        import clustered_sparse_attention_amd as ac
        self.ac = ac
        B, H, L, d = shape
        self.shape = ac.Shape(B, H, L, d)
        self.p = params
        self.ncap, self.ws_bytes = ac.ac_sizes(self.shape, params)
        BH = B * H
        dev = torch.device("cuda")
        nq = min(params.nq, L)
        self.Q, self.K, self.V = Qd, Kd, Vd
        self.ws = ac.workspace(self.ws_bytes, dev)
        self.q = ac.Clusters(BH, L, nq, d, dev, rho=True)
        self.k = ac.Clusters(BH, L, self.ncap, d, dev, rho=False)
        self.st = ac.KStats(BH, self.ncap, d, dev)
        self.sel = ac.Selection(BH, nq, self.ncap, dev, score=False)
        self.O = torch.empty_like(Qd)
        self.tail_block = tail_block
        params.tail_block = tail_block  # ac_layer applies the merge itself
        if tail_block:
            self.qm = ac.Clusters(BH, L, nq, d, dev, rho=False)
            self.selm = ac.Selection(BH, nq, self.ncap, dev, score=False)
        self.torch = torch
        self.side = torch.cuda.Stream()  # default priority
        self.key_metric = key_metric
        self.pca = pca  # (query block, key block) of ClusterAttention's principal-component split, or None
        if key_metric:
            self.M = torch.empty((BH, d, d), dtype=torch.float32, device=dev)

    def step(self, ev=None, warm=False):
        """One layer: the query clustering on a side stream beside the key
        clustering (the two use disjoint workspace scratch), then scoring,
        selection and attention.  ev: 7 timing events (start, key clustering
        done, query clustering start / done on the side stream, both joined,
        selection done, attention done).  warm: both clusterings start from
        the state of the last ac_layer call (the warm entry points)."""
        ac, torch = self.ac, self.torch
        main = torch.cuda.current_stream()
        if self.key_metric:
            # interaction-aware keys need the query clusters first: one stream
            if ev: ev[0].record(main)
            if ev: ev[2].record(main)
            ac.ac_cluster_q(self.shape, self.p, self.Q, None, self.q, self.ws)
            if ev: ev[3].record(main)
            ac.ac_interaction_matrix(self.shape, self.p, self.Q, self.q, self.M, self.ws)
            ac.ac_cluster_k_metric(self.shape, self.p, self.K, self.V, self.M, self.k, self.st, self.ws)
            if ev: ev[1].record(main)
            if ev: ev[4].record(main)
        elif self.pca:
            # the query split on the side stream beside the key split (disjoint scratch)
            if ev: ev[0].record(main)
            self.side.wait_stream(main)
            if ev: ev[2].record(self.side)
            ac.ac_cluster_q_pca(self.shape, self.p, self.Q, self.pca[0], self.q, self.ws,
                                stream=self.side.cuda_stream)
            if ev: ev[3].record(self.side)
            ac.ac_cluster_k_pca(self.shape, self.p, self.K, self.V, self.pca[1], self.k, self.st, self.ws)
            if ev: ev[1].record(main)
            main.wait_stream(self.side)
            if ev: ev[4].record(main)
        else:
            if ev: ev[0].record(main)
            self.side.wait_stream(main)
            if ev: ev[2].record(self.side)
            ac.ac_cluster_q(self.shape, self.p, self.Q, self.state.cent_q if warm else None, self.q, self.ws,
                            stream=self.side.cuda_stream)
            if ev: ev[3].record(self.side)
            ac.ac_cluster_k(self.shape, self.p, self.K, self.V, self.state if warm else None, self.k, self.st,
                            self.ws)
            if ev: ev[1].record(main)
            main.wait_stream(self.side)
            if ev: ev[4].record(main)
        ac.ac_score_select(self.shape, self.p, self.q, self.k, self.st, self.sel, self.ws)
        if self.tail_block:
            ac.ac_tail_merge(self.shape, self.p, self.tail_block, self.q, self.sel, self.qm, self.selm, self.ws)
        if ev: ev[5].record(main)
        self.attn_only()
        if ev: ev[6].record(main)

    def layer_step(self, warm=False):
        """One ac_layer call: the product's own orchestration (the query
        clustering starts on a second stream after the first stage of the
        key clustering).  Cold: the state is reset so every step is cold.
        Warm: the step starts from the state the previous call left (a later
        denoising step)."""
        if not hasattr(self, "state"):
            B, H, L, d = self.shape.B, self.shape.H, self.shape.L, self.shape.d
            self.state = self.ac.State(B * H, min(self.p.nq, L), self.ncap, d, self.Q.device)
            self.O_layer = self.torch.empty_like(self.Q)
        if not warm:
            self.state.valid = 0
        self.ac.ac_layer(self.shape, self.p, self.Q, self.K, self.V, self.state, self.O_layer, self.ws)

    def attn_only(self):
        q, sel = (self.qm, self.selm) if self.tail_block else (self.q, self.sel)
        self.ac.ac_sparse_attn(self.shape, self.p, self.Q, self.K, self.V, q, self.k, self.st, sel, self.O,
                               None, self.ws)

    def query_blocks(self, block):
        """Query blocks of `block` rows the attention runs, before and after the
        tail merge (equal when it is off)."""
        b0 = np.diff(self.q.seg.cpu().numpy(), axis=1)
        b1 = np.diff(self.qm.seg.cpu().numpy(), axis=1) if self.tail_block else b0
        return int(((b0 + block - 1) // block).sum()), int(((b1 + block - 1) // block).sum())


def pairs_of(layer):
    """Query-key pairs the attention computed (dense heads: L*L)."""
    L = layer.shape.L
    q, sel = (layer.qm, layer.selm) if layer.tail_block else (layer.q, layer.sel)
    seg_q = q.seg.cpu().numpy()
    cnt_q = np.diff(seg_q, axis=1)
    seg_k = layer.k.seg.cpu().numpy()
    cnt_k = np.diff(seg_k, axis=1)
    lst = sel.list.cpu().numpy()
    n = sel.n.cpu().numpy()
    fb = layer.st.fallback.cpu().numpy()
    dense_all = layer.p.sel_mode == 3
    tot = 0
    per_head = []
    for h in range(cnt_q.shape[0]):
        if dense_all or fb[h]:
            ph = L * L
        else:
            ph = 0
            for r in range(cnt_q.shape[1]):
                if cnt_q[h, r]:
                    ph += int(cnt_q[h, r]) * int(cnt_k[h][lst[h, r, :n[h, r]]].sum())
        per_head.append(ph)
        tot += ph
    return tot, per_head


def cpu_baseline(w, Q, K, V, kw, budget_s=30.0):
    """The oracle, timed on this host on head 0: clustering, scoring and
    selection, then the attention of every query row in seeded chunks of
    4096 while the time budget lasts.  When the budget ends first, the
    attention time is extrapolated from the rows done (and said so)."""
    from oracle import numerics as nm, kmeans as okm, multistage as oms, stats as ost, score as osc
    from oracle import attention as oat
    p = nm.Params(**{k: v for k, v in kw.items() if k in nm.Params.__dataclass_fields__})
    p.tau_param = float(np.float32(p.tau_param))
    p.sel_param = float(np.float32(p.sel_param))
    Qb, Kb, Vb = Q[0, 0], K[0, 0], V[0, 0]
    L, d = Qb.shape
    t0 = time.perf_counter()
    qc = okm.cluster_queries(Qb, p, 0)
    kc = oms.cluster_keys(Kb, p, 0)
    kst = ost.key_stats(Kb, Vb, kc["labels"], kc["cent"])
    S = osc.scores(p, qc["cent"], kst)
    sel = osc.select(S, kst["count"], qc["rho"], L, d, p)
    t1 = time.perf_counter()
    order = np.random.default_rng(9004).permutation(L)
    Qx, Kx, Vx = (nm.bf16_to_f64(x) for x in (Qb, Kb, Vb))
    done = 0
    while done < L and (done == 0 or time.perf_counter() - t0 < budget_s):
        rows = np.sort(order[done:done + 4096])
        if kc["fallback"] or p.sel_mode == nm.SEL_DENSE:
            oat.dense_rows(Qx, Kx, Vx, rows, p.attn_scale(d))
        else:
            oat.sparse_rows(Qx, Kx, Vx, rows, qc["labels"], kc["labels"], sel, p.attn_scale(d),
                            bool(p.compensate), kst["count"], kst["kmean"], kst["vmean"])
        done += rows.size
    t2 = time.perf_counter()
    per_head = (t1 - t0) + (t2 - t1) * (L / done)
    layer_s = per_head * w.BH
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    part = (f"all {L} query rows" if done == L else
            f"{done} of {L} query rows in the {budget_s:.0f} s budget, extrapolated x{L / done:.1f} rows")
    return dict(value=w.dense_flops / layer_s / 1e12, unit="TFLOP/s (dense-equivalent)", cores=cores, kind="oracle",
                sample=f"head 0 of {w.BH}: clustering/scoring/selection ({t1 - t0:.1f} s) + attention for "
                       f"{part} ({t2 - t1:.1f} s); the layer is x{w.BH} heads, {layer_s:.0f} s",
                complete_head=done == L, measured_s=round(t2 - t0, 2), layer_s_extrapolated=round(layer_s, 1))


def peak_probe():
    """Achievable peaks on this GPU, measured: a large bf16 GEMM through
    torch (hipBLASLt) and a device-to-device copy of 4 GiB."""
    import torch
    out = {}
    n = 8192
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    out["gemm_bf16"] = {"shape": [n, n, n], "ms": round(ms, 4), "tflops": round(2.0 * n ** 3 / ms / 1e9, 1),
                        "frac_of_2500": round(2.0 * n ** 3 / ms / 1e9 / PEAK_BF16_TFLOPS, 3)}
    del a, b
    nbytes = 4 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    reps = 10
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbs = 2.0 * nbytes / ms / 1e6
    out["copy"] = {"bytes": nbytes, "ms": round(ms, 3), "gbs_read_plus_write": round(gbs, 1),
                   "frac_of_8000": round(gbs / PEAK_HBM_GBS, 3)}
    print(json.dumps(out), flush=True)


def sdpa_ms(Qd, Kd, Vd, reps=3):
    """torch scaled_dot_product_attention restricted to the flash backend."""
    import torch
    try:
        from torch.nn.attention import sdpa_kernel, SDPBackend
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            torch.nn.functional.scaled_dot_product_attention(Qd, Kd, Vd)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                torch.nn.functional.scaled_dot_product_attention(Qd, Kd, Vd)
            e1.record()
            torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps
    except Exception as e:  # backend not available in this torch
        print(f"[bench] sdpa flash backend unavailable: {e}", file=sys.stderr)
        return None


ATTN_SRCS = [os.path.join(ROOT, "clustered_sparse_attention_amd", "csrc", f)
             for f in ("attn.hip", "common.h", "internal.h")]
TRAFFIC = os.path.join(ROOT, "profiles", "k_attn_wan_traffic.json")


def attn_source_hash() -> str:
    """SHA-256 of the sources the attention kernels compile from (attn.hip and
    the two headers it includes)."""
    import hashlib
    h = hashlib.sha256()
    for path in ATTN_SRCS:
        h.update(open(path, "rb").read())
    return h.hexdigest()


def measured_traffic(workload: str, variant: str, compensate: int):
    """HBM bytes per k_attn launch from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter's
    reading for a plain copy of known size), or None when the summary is for
    another workload or the kernel source changed since it was taken."""
    try:
        t = json.load(open(TRAFFIC))
    except (OSError, ValueError):
        return None
    if t.get("attn_source_sha256") != attn_source_hash():
        return None
    if (t.get("workload"), t.get("variant"), t.get("compensate")) != (workload, variant, compensate):
        return None
    return t.get("bytes_per_launch")


def _counter_kib(csv_path: str, kernel_regex: str):
    """Per-dispatch sums of one rocprofv3 counter (KiB) for kernels whose
    name matches kernel_regex, grouped by dispatch id."""
    import csv
    import re
    per = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if re.search(kernel_regex, r["Kernel_Name"]):
                d = int(r["Dispatch_Id"])
                per[d] = per.get(d, 0.0) + float(r["Counter_Value"])
    return per


def summarize(args):
    """Write the committed profile summaries from rocprofv3 output.

    --summarize stats <kernel_stats.csv> <out.md> <command...>
    --summarize traffic <fetch.csv> <write.csv> <copy_fetch.csv> <copy_write.csv> <copy_bytes>
                        <dispatches_per_call> <out.json> <command...>
    --summarize pca <kernel_trace.csv> <out.md> <title> <command...>
    """
    import csv
    kind, rest = args[0], args[1:]
    if kind == "stats":
        src, out, cmd = rest[0], rest[1], " ".join(rest[2:])
        rows = list(csv.DictReader(open(src)))
        rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
        lines = [f"# rocprofv3 kernel statistics", "", f"Command: `{cmd}`", "",
                 "| kernel | calls | total ms | avg us | % |", "|---|---:|---:|---:|---:|"]
        for r in rows[:30]:
            name = r["Name"].replace("void ", "").split("(")[0]
            lines.append(f"| {name} | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
                         f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
        open(out, "w").write("\n".join(lines) + "\n")
        return
    if kind == "traffic":
        f_csv, w_csv, cf_csv, cw_csv = rest[:4]
        copy_bytes, per_call, out = int(rest[4]), int(rest[5]), rest[6]
        cmd = " ".join(rest[7:])
        rx = r"k_attn"
        fetch = _counter_kib(f_csv, rx)
        write = _counter_kib(w_csv, rx)
        cf = max(_counter_kib(cf_csv, r"copy|elementwise|Copy").values())
        cw = max(_counter_kib(cw_csv, r"copy|elementwise|Copy").values())
        f_scale = copy_bytes / (cf * 1024.0)
        w_scale = copy_bytes / (cw * 1024.0)
        tot_f = sum(fetch.values()) * 1024.0 * f_scale
        tot_w = sum(write.values()) * 1024.0 * w_scale
        launches = len(fetch) / per_call
        res = {"workload": "wan", "variant": "density", "compensate": 0,
               "kernels": "k_attn_rows + k_attn_prep + k_attn (one ac_sparse_attn call)",
               "fetch_kib_raw": sum(fetch.values()), "write_kib_raw": sum(write.values()),
               "dispatches": len(fetch), "entry_point_calls": launches,
               "copy_probe_bytes": copy_bytes, "copy_fetch_kib": cf, "copy_write_kib": cw,
               "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
               "bytes_per_launch": (tot_f + tot_w) / launches,
               "attn_source_sha256": attn_source_hash(), "command": cmd}
        json.dump(res, open(out, "w"), indent=1)
        print(json.dumps(res))
        return
    if kind == "roofline":
        # per-kernel roofline of one layer step's full-size launches, from a kernel
        # trace of `bench.py --serial` (the entry points one after another) and
        # that run's bench line (the attention's algorithmic flops)
        src, bench_log, out, wl, cmd = rest[0], rest[1], rest[2], rest[3], " ".join(rest[4:])
        import csa_inputs as gen
        w = gen.get_workload(wl)
        kw = workload_params(wl, "density", 0)
        BH, L, d = w.BH, w.L, w.d
        nq, m0 = min(kw["nq"], L), min(kw["m0"], L)
        line = [json.loads(x) for x in open(bench_log) if x.startswith("{")][-1]
        attn_flops = line["roofline"]["algorithmic_flops_per_launch"]
        rows = list(csv.DictReader(open(src)))
        rows.sort(key=lambda r: int(r["Start_Timestamp"]))
        starts = [i for i, r in enumerate(rows) if "k_qnorm" in r["Kernel_Name"]]
        steps = [rows[a:b] for a, b in zip(starts, starts[1:] + [len(rows)])][1:]  # drop the warm-up step

        def dur(r):
            return (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9

        def after_seed(step, name, which, count):
            """The first `count` launches of `name` after the `which`-th seeding
            of the step (0: the queries, 1: the keys' first stage): the Lloyd
            iterations in which every head still takes part."""
            seeds = [i for i, r in enumerate(step) if "k_kpp_seq" in r["Kernel_Name"]]
            if len(seeds) <= which:
                return []
            hits = [r for r in step[seeds[which]:] if name in r["Kernel_Name"]]
            return hits[:count]

        def once(step, name):
            return [r for r in step if name in r["Kernel_Name"]][:1]

        def sum_of(step, names):
            """The first launch of each kernel in names, as one launch of their summed duration."""
            rs = [once(step, n)[0] for n in names if once(step, n)]
            t = sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rs)
            return {"Start_Timestamp": "0", "End_Timestamp": str(t), "Kernel_Name": "+".join(names)}

        x_bytes = BH * L * d * 2.0
        pad = lambda m: (m + 15) // 16 * 16
        hbm = lambda b: ("hbm", b, None)
        # (label, launches picked per step, work, what)
        specs = [
            ("k_qnorm", lambda st: once(st, "k_qnorm"), hbm(2 * x_bytes + BH * L * 4),
             "read Q, write q-hat (bf16) and norms"),
            (f"k_assign_res, queries, iterations 0-1 (n = L, m = {nq})", lambda st: after_seed(st, "k_assign_res", 0, 2),
             ("hbm+flop", x_bytes, 2.0 * BH * L * nq * d), "read X once; argmin GEMM"),
            (f"k_assign_res, keys, stage 0, iterations 0-1 (n = L, m = {m0})",
             lambda st: after_seed(st, "k_assign_res", 1, 2), ("hbm+flop", x_bytes, 2.0 * BH * L * m0 * d),
             "read X once; argmin GEMM"),
            ("k_update_partial, queries and key stage 0, iteration 0",
             lambda st: after_seed(st, "k_update_partial", 0, 1) + after_seed(st, "k_update_partial", 1, 1),
             hbm(x_bytes + BH * L * 4), "gather X in cluster order (bf16) + perm"),
            ("k_sort_scatter, queries and key stage 0, iteration 0",
             lambda st: after_seed(st, "k_sort_scatter", 0, 1) + after_seed(st, "k_sort_scatter", 1, 1),
             hbm(BH * L * 8.0), "read labels, write perm"),
            ("k_kst_chunks + k_kstats_part + k_kstats_fin (one launch each)",
             lambda st: [sum_of(st, ("k_kst_chunks", "k_kstats_part", "k_kstats_fin"))],
             hbm(2 * x_bytes + BH * L * 4), "read K, V and labels in cluster order"),
            ("k_attn", lambda st: once(st, "k_attn<"), ("flop", None, attn_flops),
             "4 d x the algorithmic query-key pairs (padding and masked keys not counted)"),
        ]
        lines = [f"# Per-kernel roofline, {w.description}", "", f"Command: `{cmd}`", "",
                 "Full-size launches of the timed layer steps (the entry points one after another; of the Lloyd "
                 "loops the iterations in which every head still takes part). Work is algorithmic: the bytes "
                 "the step must move, or its flops without padding and without the low halves of the "
                 "split centres; time is the kernel's own. Peaks: HBM 8000 GB/s, bf16 MFMA 2500 TFLOP/s "
                 f"(dense). Attention: {line['layer']['density_pairs']:.4f} of the pairs, "
                 f"{attn_flops / 1e12:.2f} TFLOP per call.", "",
                 "| kernel | launches/step | avg time | algorithmic work | achieved | fraction of peak |",
                 "|---|---:|---:|---|---|---:|"]
        for label, pick, (bound, nbytes, flops), what in specs:
            ds = [dur(r) for st in steps for r in pick(st)]
            if not ds:
                continue
            t = float(np.mean(ds))
            per = len(ds) / max(len(steps), 1)
            parts, fracs = [], []
            if nbytes is not None:
                gbs = nbytes / t / 1e9
                parts.append(f"{gbs:.0f} GB/s")
                fracs.append(("HBM", gbs / PEAK_HBM_GBS))
            if flops is not None:
                tf = flops / t / 1e12
                parts.append(f"{tf:.0f} TFLOP/s")
                fracs.append(("MFMA", tf / PEAK_BF16_TFLOPS))
            work = ", ".join(x for x in (f"{nbytes / 1e9:.3f} GB" if nbytes else "",
                                         f"{flops / 1e12:.3f} TFLOP" if flops else "") if x)
            frac = max(fracs, key=lambda f: f[1])
            lines.append(f"| {label} | {per:g} | {t * 1e3:.3f} ms | {work}: {what} | {', '.join(parts)} | "
                         f"{frac[1]:.2f} ({frac[0]}) |")
        open(out, "w").write("\n".join(lines) + "\n")
        print("\n".join(lines))
        return
    if kind == "configs":
        # one table of bench lines: --summarize configs <out.md> [title=<title>] <command> :: <log>...
        out = rest[0]
        k = rest.index("::")
        title = "Bench lines, all workloads (one MI355X)"
        if rest[1].startswith("title="):
            title, rest = rest[1][len("title="):], rest[:1] + rest[2:]
            k -= 1
        cmd, logs = " ".join(rest[1:k]), rest[k + 1:]
        lines = [f"# {title}", "", f"Command: `{cmd}`", "",
                 "A step is one `ac_layer` call on resident inputs (cold unless marked warm); the phase columns "
                 "come from a separate untimed pass through the entry points, the query clustering on a second "
                 "stream beside the key clustering (`both` is their wall time). Rows marked with the "
                 "principal-component split time the entry points in `ac_layer`'s order instead (the query "
                 "split beside the key split), with ClusterAttention's clustering in place of Algorithm 1's. "
                 "Dense baselines: the library's own dense mode and torch SDPA (flash backend) on the same "
                 "tensors.", "",
                 "| workload | step | selection | layer ms | dense-equiv TFLOP/s | cluster_q / cluster_k / both (ms) | "
                 "select ms | attention ms | attention / bf16 peak | pairs kept | fallback heads | key clusters | "
                 "own dense ms | SDPA flash ms | vs best dense | CPU oracle |",
                 "|---|---|---|---:|---:|---|---:|---:|---:|---:|---:|---|---:|---:|---:|---|"]
        raw = []
        for lg in logs:
            ls = [x for x in open(lg) if x.startswith("{")]
            if not ls:
                continue
            d = json.loads(ls[-1])
            raw.append(ls[-1].strip())
            ph, db, cb = d["phase_ms"], d.get("dense_baseline") or {}, d.get("cpu_baseline")
            sel = d["config"]["selection"] + (" + compensation" if d["config"]["compensate"] else "")
            warm = "warm" if "warm" in d["timed_step"] else "cold"
            if d.get("key_clustering", "").startswith("principal-component"):
                warm += ", principal-component split " + "/".join(re.findall(r" of (\d+)", d["key_clustering"]))
            cpu = (f"{cb['value']:.3f} TFLOP/s, {cb['cores']} cores, "
                   f"{'complete head' if cb.get('complete_head') else 'extrapolated'}") if cb else "—"
            lines.append(
                f"| {d['config']['workload']} | {warm} | {sel} | {d['ms_per_step']:.2f} | {d['value']:.0f} | "
                f"{ph['cluster_q']:.2f} / {ph['cluster_k']:.2f} / {ph['clustering_q_beside_k']:.2f} | "
                f"{ph['score_select']:.2f} | {ph['sparse_attn']:.2f} | {d['roofline']['frac']:.3f} | "
                f"{d['layer']['density_pairs']:.3f} | {d['layer']['fallback_heads']} | "
                f"{d['layer']['key_clusters_min_max'][0]}–{d['layer']['key_clusters_min_max'][1]} | "
                f"{db.get('own_dense_attn_ms', float('nan')):.2f} | {db.get('sdpa_flash_ms') or float('nan'):.2f} | "
                f"{db.get('speedup_layer_vs_best_dense', float('nan')):.2f}x | {cpu} |")
        lines += ["", "Raw JSON lines:", "", "```"] + raw + ["```"]
        open(out, "w").write("\n".join(lines) + "\n")
        return
    if kind == "denoise":
        # --summarize denoise <out.md> <command> :: <log>...  (bench.py --denoise lines)
        out = rest[0]
        k = rest.index("::")
        cmd, logs = " ".join(rest[1:k]), rest[k + 1:]
        runs = []
        for lg in logs:
            ls = [x for x in open(lg) if x.startswith("{")]
            if ls:
                runs.append(json.loads(ls[-1]))
        w = runs[0]["workload"] if runs else ""
        lines = [f"# Denoising runs under the multi-step policy, {w}", "", f"Commands: `{cmd}`", "",
                 "Each step's Q and K are a 2% perturbation of the previous step's. k_max is calibrated on an "
                 "uncapped first sparse step (untimed, target 15% of the heads); with N_max = k_max, Algorithm 1 "
                 "lets a head fall back only when a stage would start with k_max centres and keys are left. "
                 "Dense warm-up steps run the library's dense mode; the cold step runs Algorithm 1, the warm "
                 "steps Lloyd iterations from the previous step's centres.", "",
                 "| run | dense warm-up steps (ms) | cold step (ms) | warm steps, mean (ms) | total (ms) | "
                 "own dense x steps (ms) | SDPA flash x steps (ms) | vs own dense | vs SDPA flash | k_max | "
                 "heads dense |", "|---|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
        for r in runs:
            T = r["steps"]
            dense = ", ".join(str(x["ms"]) for x in r["per_step"] if x["mode"] == "dense")
            od, sd = r.get("own_dense_ms"), r.get("sdpa_flash_ms")
            name = "SNR top-p" if r.get("topp_schedule") else "density 0.15"
            lines.append(f"| {name} | {dense} | {r['cold_ms']} | {r['warm_ms_mean']} | {r['value']} | "
                         f"{od * T:.1f} | {sd * T:.1f} | {od * T / r['value']:.2f}x | {sd * T / r['value']:.2f}x | "
                         f"{r['kmax']} | {r['fallback_heads']} |")
        for r in runs:
            if r.get("topp_schedule"):
                lines += ["", "Per step (top-p run): " + ", ".join(
                    f"{x['step']}: {x['mode']} {x['ms']} ms" + (f" (p {x['sel_param']})" if "sel_param" in x else "")
                    for x in r["per_step"])]
        lines += ["", "Raw JSON lines:", "", "```"] + [json.dumps(r) for r in runs] + ["```"]
        open(out, "w").write("\n".join(lines) + "\n")
        return
    if kind == "quest":
        # per-token Quest engines: bench --quest-compare lines + kernel-trace durations
        src, lines_json, out, cmd = rest[0], rest[1], rest[2], " ".join(rest[3:])
        res = [json.loads(l) for l in open(lines_json) if l.startswith("{")]
        tr = list(csv.DictReader(open(src)))
        dur = {}
        for r in tr:
            name = r["Kernel_Name"]
            if "k_tq_" not in name:
                continue
            eng = "mfma" if "k_tq_mfma" in name else "valu"
            per_block = 512 if eng == "mfma" else 256
            toks = 256
            blocks_x = int(r["Grid_Size_X"]) // per_block
            dur.setdefault((eng, blocks_x * toks), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-6)
        lines = ["# Per-token Quest scores: TensorQuest (MFMA) against eq. (1) on the vector ALUs", "",
                 f"Command: `{cmd}`", "",
                 "Every query token of every head against every key cluster of the head (the keys clustered by "
                 "the workload's Algorithm 1 at each length); S is [H, L, ld] fp32 with ld the largest cluster "
                 "count rounded up to 32. MFMA work: write S + read Q (HBM-bound, peak 8000 GB/s); VALU work: "
                 "4 fp32 operations per (token, cluster, dimension) against 39.3 T lane-ops/s (256 CUs x 4 SIMDs "
                 "x 16 lanes x 2.4 GHz). Event time per call; kernel-trace average of the same launches beside it.",
                 "",
                 "| L | key clusters (mean, ld) | TensorQuest ms (trace) | GB/s | HBM frac | Quest VALU ms (trace) | "
                 "Tops/s | ALU frac | speedup | torch fill of S, GB/s |",
                 "|---:|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
        for r in res:
            Lp = (r["L"] + 255) // 256 * 256
            tm = np.mean(dur.get(("mfma", Lp), [float("nan")]))
            tv = np.mean(dur.get(("valu", Lp), [float("nan")]))
            lines.append(f"| {r['L']} | {r['key_clusters_mean']}, {r['ld']} | {r['tensorquest_mfma_ms']} ({tm:.4f}) | "
                         f"{r['mfma_hbm_gbs']} | {r['mfma_hbm_frac']} | {r['quest_valu_ms']} ({tv:.3f}) | "
                         f"{r['valu_tops']} | {r['valu_alu_frac']} | {r['speedup']}x | {r['fill_gbs']} |")
        open(out, "w").write("\n".join(lines) + "\n")
        print("\n".join(lines))
        return
    if kind == "pca":
        # the principal-component split of the last layer step in a kernel trace of
        # `bench.py --pca-split qb,kb`: per side (its own queue) the split tree,
        # every level's launch and the finishing kernels, and the span of both
        src, out, title, cmd = rest[0], rest[1], rest[2], " ".join(rest[3:])
        rows = list(csv.DictReader(open(src)))
        rows.sort(key=lambda r: int(r["Start_Timestamp"]))
        sides = []
        for q in sorted({r["Queue_Id"] for r in rows}):
            qr = [r for r in rows if r["Queue_Id"] == q]
            trees = [i for i, r in enumerate(qr) if "k_pca_tree" in r["Kernel_Name"]]
            if not trees:
                continue
            t = trees[-1]
            b = t - 1 if t > 0 and "k_qnorm" in qr[t - 1]["Kernel_Name"] else t
            e = t
            while e + 1 < len(qr) and not re.search(r"k_score_prep|k_pca_tree|k_qnorm", qr[e + 1]["Kernel_Name"]):
                e += 1
            seq = qr[b:e + 1]
            key = any("k_kstats" in r["Kernel_Name"] for r in seq)
            sides.append(("keys" if key else "queries", seq))
        if not sides:
            raise SystemExit("no principal-component split in the trace")
        t0 = min(int(seq[0]["Start_Timestamp"]) for _, seq in sides)
        t1 = max(int(seq[-1]["End_Timestamp"]) for _, seq in sides)
        lines = [f"# Principal-component split, {title}", "", f"Command: `{cmd}`", "",
                 "The last layer step of the trace; each side runs on its own queue (the two overlap). "
                 f"Both sides together: {(t1 - t0) / 1e6:.3f} ms from the first launch to the last end.", ""]
        for name, seq in sorted(sides):
            span = (int(seq[-1]["End_Timestamp"]) - int(seq[0]["Start_Timestamp"])) / 1e6
            lines += [f"## {name}: {span:.3f} ms", "", "| kernel | level | time | start |", "|---|---:|---:|---:|"]
            # a level of large nodes is three launches: its directions
            # (k_pca_level), the projections (k_pca_project), its cuts (k_pca_level)
            lvl, prev = -1, ""
            for r in seq:
                kn = r["Kernel_Name"].replace("void ", "").split("(")[0]
                d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                st = (int(r["Start_Timestamp"]) - t0) / 1e3
                lv = ""
                if "k_pca_level" in kn and "k_pca_project" not in prev:
                    lvl += 1
                if "k_pca_level" in kn or "k_pca_project" in kn:
                    lv = str(lvl)
                lines.append(f"| {kn} | {lv} | {d:.1f} us | {st:.1f} us |")
                prev = kn
            lines.append("")
        open(out, "w").write("\n".join(lines))
        print("\n".join(lines))
        return
    raise SystemExit(f"unknown summary kind {kind}")


PEAK_VALU_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12  # fp32 VALU lane-ops/s, unpacked: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz


def quest_compare(args):
    """Per-token Quest scores (every query token against every key cluster)
    on MFMA (TensorQuest) and on the vector ALUs (eq. (1) as written), on
    the workload's head count and clustering at several sequence lengths.
    One JSON line per length, then a markdown table on stderr."""
    import torch
    import csa_inputs as gen
    import clustered_sparse_attention_amd as ac
    base = gen.get_workload(args.workload)
    kw = workload_params(args.workload, "density", 0)
    rows = []
    for frac in (0.125, 0.25, 0.5, 1.0):
        L = int(round(base.L * frac))
        w = gen.get_workload(args.workload, L=L, H=args.heads or base.H)
        Q, K, V = gen.generate(w)
        dev = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        Qd, Kd, Vd = dev(Q), dev(K), dev(V)
        shape = ac.Shape(w.B, w.H, w.L, w.d)
        params = _abi(kw)
        ncap, wsb = ac.ac_sizes(shape, params)
        ws = ac.workspace(wsb, Qd.device)
        kcl = ac.Clusters(w.BH, w.L, ncap, w.d, Qd.device, rho=False)
        st = ac.KStats(w.BH, ncap, w.d, Qd.device)
        ac.ac_cluster_k(shape, params, Kd, Vd, None, kcl, st, ws)
        ncl = kcl.ncl.cpu().numpy()
        ld = (int(ncl.max()) + 31) // 32 * 32  # rows of whole 128-byte lines
        S = torch.empty((w.BH, w.L, ld), dtype=torch.float32, device=Qd.device)
        res = {"L": w.L, "H": w.H, "d": w.d, "ld": ld, "key_clusters_mean": round(float(ncl.mean()), 1)}
        # what a plain write of the same bytes reaches (torch fill), for scale
        S.fill_(0.0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            S.fill_(0.0)
        e1.record()
        torch.cuda.synchronize()
        res["fill_gbs"] = round(S.numel() * 4.0 * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
        for eng, name, reps in ((ac.AC_QUEST_MFMA, "tensorquest_mfma", 10), (ac.AC_QUEST_VALU, "quest_valu", 3)):
            ac.ac_score_tokens(shape, params, Qd, kcl, st, eng, S, ld)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                ac.ac_score_tokens(shape, params, Qd, kcl, st, eng, S, ld)
            e1.record()
            torch.cuda.synchronize()
            res[name + "_ms"] = round(e0.elapsed_time(e1) / reps, 4)
        t_m, t_v = res["tensorquest_mfma_ms"] * 1e-3, res["quest_valu_ms"] * 1e-3
        pairs = float(w.L) * float(ncl.sum())
        hbm = w.BH * w.L * (ld * 4.0 + w.d * 2.0) + float(ncl.sum()) * 4.0 * w.d
        res["speedup"] = round(t_v / t_m, 2)
        res["mfma_hbm_gbs"] = round(hbm / t_m / 1e9, 1)
        res["mfma_hbm_frac"] = round(hbm / t_m / 1e9 / PEAK_HBM_GBS, 3)
        res["mfma_tflops"] = round(pairs * 4.0 * w.d / t_m / 1e12, 1)
        res["valu_tops"] = round(pairs * 4.0 * w.d / t_v / 1e12, 2)
        res["valu_alu_frac"] = round(pairs * 4.0 * w.d / t_v / 1e12 / PEAK_VALU_TOPS, 3)
        print(json.dumps(res), flush=True)
        rows.append(res)
        del S, ws, kcl, st, Qd, Kd, Vd
        torch.cuda.empty_cache()
    print("| L | key clusters (mean, ld) | TensorQuest MFMA ms | HBM GB/s (frac) | torch fill of S, GB/s | "
          "Quest VALU ms | VALU Tops/s (frac) | speedup |", file=sys.stderr)
    print("|---:|---|---:|---:|---:|---:|---:|---:|", file=sys.stderr)
    for r in rows:
        print(f"| {r['L']} | {r['key_clusters_mean']}, {r['ld']} | {r['tensorquest_mfma_ms']} | {r['mfma_hbm_gbs']} "
              f"({r['mfma_hbm_frac']}) | {r['fill_gbs']} | {r['quest_valu_ms']} | {r['valu_tops']} "
              f"({r['valu_alu_frac']}) | {r['speedup']}x |", file=sys.stderr)


def flow_log_snr(T: int, shift: float = 5.0):
    """log SNR of a shifted flow-matching sampler (x_t = (1 - s) x_0 + s eps)
    over T steps: a synthetic stand-in for a video DiT's sampling schedule."""
    t = np.linspace(1.0, 0.0, T + 1)[:-1]
    s = np.clip(shift * t / (1.0 + (shift - 1.0) * t), 1e-4, 1 - 1e-4)
    return np.log(((1.0 - s) / s) ** 2)


def denoise(args):
    """T denoising steps of the workload's layer under the multi-step policy:
    dense warm-up steps, k_max calibrated on an uncapped first sparse step
    (untimed) so that a fraction of the heads falls back, the first sparse
    step cold, the rest warm; optionally the SNR-guided top-p per step.
    Each step's Q and K are a 2% perturbation of the previous step's (drawn
    on the device).  One JSON line with per-step times."""
    import torch
    import csa_inputs as gen
    import clustered_sparse_attention_amd as ac
    w = gen.get_workload(args.workload, **({"H": args.heads} if args.heads else {}))
    Q, K, V = gen.generate(w)
    dev = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    Qd, Kd, Vd = dev(Q), dev(K), dev(V)
    del Q, K, V
    kw = workload_params(args.workload, args.variant, args.compensate)
    base = _abi(kw)
    shape = ac.Shape(w.B, w.H, w.L, w.d)
    T, warm_steps = args.denoise, args.warmup_steps
    # calibration: the first sparse step with a cap no head reaches
    cal = ac.params_default(**{f: getattr(base, f) for f, _ in ac.Params._fields_})
    cal.nmax = 3000
    _, wsb = ac.ac_sizes(shape, cal)
    ws = ac.workspace(wsb, Qd.device)
    nq = min(base.nq, w.L)
    st = ac.State(w.BH, nq, cal.nmax - 1 + cal.m0, w.d, Qd.device)
    O = torch.empty_like(Qd)
    hs = ac.ac_layer(shape, cal, Qd, Kd, Vd, st, O, ws, host_stats=True)
    kmax = ac.ac_kmax_calibrate(hs["ncl_k"], args.dense_frac)
    del st, ws
    topp = ac.ac_topp_schedule(flow_log_snr(T), warm_steps, args.p_min, args.tau_sat) if args.topp_schedule else None
    sch = ac.Schedule(warmup_steps=warm_steps, warmup_layers=0, nmax=kmax, topp=topp)
    sparse_p = ac.ac_step_params(base, sch, T - 1, 0)
    ncap, wsb = ac.ac_sizes(shape, sparse_p)
    _, wsb_d = ac.ac_sizes(shape, ac.ac_step_params(base, sch, 0, 0))
    ws = ac.workspace(max(wsb, wsb_d), Qd.device)
    st = ac.State(w.BH, nq, ncap, w.d, Qd.device)
    gen_t = torch.Generator(device="cuda")
    gen_t.manual_seed(1103)

    def perturb(x):
        xf = x.float()
        rms = xf.pow(2).mean(dim=(2, 3), keepdim=True).sqrt()
        eps = torch.randn(xf.shape, generator=gen_t, device=xf.device, dtype=torch.float32)
        return (xf + 0.02 * rms * eps).to(torch.bfloat16)

    steps = []
    for step in range(T):
        if step > 0:
            Qd, Kd = perturb(Qd), perturb(Kd)
        p = ac.ac_step_params(base, sch, step, 0)
        mode = "dense" if p.sel_mode == ac.AC_SEL_DENSE else ("cold" if not st.valid else "warm")
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        ac.ac_layer(shape, p, Qd, Kd, Vd, st, O, ws)
        e1.record()
        torch.cuda.synchronize()
        rec = {"step": step, "mode": mode, "ms": round(e0.elapsed_time(e1), 3)}
        if mode != "dense":
            rec["sel_param"] = round(float(p.sel_param), 4)
        steps.append(rec)
        print(f"[bench] step {step} {mode}: {rec['ms']} ms", file=sys.stderr, flush=True)
    fb = int(st.fallback.cpu().numpy().sum())
    sd = sdpa_ms(Qd, Kd, Vd)
    dense_ms = float(np.mean([r["ms"] for r in steps if r["mode"] == "dense"])) if warm_steps else None
    total = sum(r["ms"] for r in steps)
    warm = [r["ms"] for r in steps if r["mode"] == "warm"]
    cold = [r["ms"] for r in steps if r["mode"] == "cold"]
    out = {"metric": f"{T}-step denoising run of one layer: total ms", "value": round(total, 2), "unit": "ms",
           "higher_is_better": False, "workload": w.description, "steps": T, "warmup_steps": warm_steps,
           "kmax": kmax, "dense_frac_target": args.dense_frac, "fallback_heads": fb, "heads": w.BH,
           "topp_schedule": None if topp is None else [round(float(x), 4) for x in topp],
           "per_step": steps, "cold_ms": cold[0] if cold else None,
           "warm_ms_mean": round(float(np.mean(warm)), 3) if warm else None,
           "own_dense_ms": None if dense_ms is None else round(dense_ms, 3),
           "sdpa_flash_ms": None if sd is None else round(sd, 3),
           "speedup_vs_sdpa_flash_all_steps": None if sd is None else round(sd * T / total, 3)}
    print(json.dumps(out), flush=True)


def copy_probe(nbytes: int):
    """A plain device copy of nbytes (torch), for calibrating the HBM byte
    counters: its FETCH_SIZE / WRITE_SIZE should read nbytes each."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="wan", choices=["tiny", "cogvideox", "hunyuan", "wan", "long"])
    ap.add_argument("--variant", default="density", choices=["density", "topp", "dense"])
    ap.add_argument("--compensate", type=int, default=0)
    ap.add_argument("--heads", type=int, default=0, help="run only this many heads (0 = all)")
    ap.add_argument("--seq-len", type=int, default=0,
                    help="tokens per head instead of the workload's own (0 = the workload's; same data recipe)")
    ap.add_argument("--serial", action="store_true",
                    help="run the query clustering on the main stream too (for per-kernel profiles)")
    ap.add_argument("--tail-block", type=int, default=0,
                    help="merge query-cluster tails for attention blocks of this many rows before the attention "
                         "(iCATS tail merging; 0 = off)")
    ap.add_argument("--key-metric", type=int, default=0,
                    help="cluster the keys interaction-aware (iCATS, metric M_Q from the query clusters) into this "
                         "many clusters instead of Algorithm 1 (0 = off)")
    ap.add_argument("--pca-split", default="",
                    help="QB,KB: cluster queries and keys by ClusterAttention's principal-component split into "
                         "clusters of QB and KB tokens (powers of two) instead of k-means / Algorithm 1")
    ap.add_argument("--warm", action="store_true",
                    help="time the warm step instead: a cold ac_layer call fills the state, Q and K are perturbed "
                         "by 2%%, and the timed ac_layer calls start from the state (a later denoising step)")
    ap.add_argument("--no-baselines", action="store_true", help="skip dense baselines and the CPU oracle")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, help="only run a plain copy of this many bytes")
    ap.add_argument("--peak-probe", action="store_true",
                    help="only measure achievable peaks: a bf16 GEMM (torch) and a 4 GiB device copy")
    ap.add_argument("--summarize", nargs="+", help="write a profile summary from rocprofv3 output (no GPU)")
    ap.add_argument("--denoise", type=int, default=0,
                    help="only run this many denoising steps under the multi-step policy (dense warm-up, calibrated "
                         "k_max, cold then warm steps)")
    ap.add_argument("--warmup-steps", type=int, default=2, help="dense warm-up steps of --denoise")
    ap.add_argument("--dense-frac", type=float, default=0.15, help="heads targeted for dense attention by k_max")
    ap.add_argument("--topp-schedule", action="store_true", help="--denoise: SNR-guided top-p per step")
    ap.add_argument("--p-min", type=float, default=0.7)
    ap.add_argument("--tau-sat", type=float, default=0.999)
    ap.add_argument("--quest-compare", action="store_true",
                    help="only time per-token Quest scores, TensorQuest (MFMA) against eq. (1) on the vector ALUs")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.peak_probe:
        peak_probe()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (heads shard across GPUs by design "
              "only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import csa_inputs as gen
    import clustered_sparse_attention_amd as ac
    ac.load()
    if args.quest_compare:
        quest_compare(args)
        return
    if args.denoise:
        denoise(args)
        return


    over = {}
    if args.heads:
        over["H"] = args.heads
    if args.seq_len:
        over["L"] = args.seq_len
    w = gen.get_workload(args.workload, **over)
    t0 = time.perf_counter()
    Q, K, V = gen.generate(w)
    print(f"[bench] generated {w.name} B={w.B} H={w.H} L={w.L} d={w.d} in {time.perf_counter() - t0:.1f} s",
          file=sys.stderr, flush=True)

    def dev(x):
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()

    Qd, Kd, Vd = dev(Q), dev(K), dev(V)
    kw = workload_params(args.workload, args.variant, args.compensate)
    if args.key_metric:
        kw["m0"] = args.key_metric
    pca = None
    if args.pca_split:
        pca = tuple(int(x) for x in args.pca_split.split(","))
        # one query cluster per query block and a key capacity for every key cluster
        kw["nq"] = -(-w.L // pca[0])
        kw["nmax"] = max(kw["nmax"], -(-w.L // pca[1]) - kw["m0"] + 1)
    params = _abi(kw)
    layer = Layer(Qd, Kd, Vd, (w.B, w.H, w.L, w.d), params, tail_block=args.tail_block,
                  key_metric=bool(args.key_metric), pca=pca)
    if args.serial:
        layer.side = torch.cuda.current_stream()

    # the timed step is one ac_layer call (cold), except for the variants that
    # ac_layer does not run (interaction-aware keys) or a serial profile
    use_layer = not args.key_metric and not args.serial and not pca
    if args.warm and not use_layer:
        raise SystemExit("--warm times ac_layer's warm step: not with --key-metric, --serial or --pca-split")
    for _ in range(args.warmup):
        layer.layer_step() if use_layer else layer.step()
    torch.cuda.synchronize()
    if args.warm:
        # the first step's state, then the next step's inputs: Q and K moved by 2 %
        layer.layer_step()
        Qd.copy_(dev(gen.perturb(Q, 1103)))
        Kd.copy_(dev(gen.perturb(K, 1104)))
        layer.layer_step(warm=True)
        torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(args.steps):
        layer.layer_step(warm=args.warm) if use_layer else layer.step(evs[s])
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    ms_step = (t_end - t_start) * 1e3 / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_step:.2f} ms/step", file=sys.stderr, flush=True)
    # phases: the entry points one by one with events (untimed pass when the
    # timed step was ac_layer); cluster_q (side stream), cluster_k, both,
    # score_select, sparse_attn
    nph = min(args.steps, 3) if use_layer else args.steps
    if use_layer:
        for s in range(nph):
            layer.step(evs[s], warm=args.warm)
        torch.cuda.synchronize()
    pairs_ev = [(2, 3), (0, 1), (0, 4), (4, 5), (5, 6)]
    phase = np.array([[evs[s][a].elapsed_time(evs[s][b]) for a, b in pairs_ev] for s in range(nph)])
    phase_ms = phase.mean(axis=0)

    pairs, _ = pairs_of(layer)
    attn_flops = 4.0 * w.d * pairs
    attn_ms = float(phase_ms[4])
    achieved = attn_flops / (attn_ms * 1e-3) / 1e12
    fb = layer.st.fallback.cpu().numpy()
    ncl = layer.k.ncl.cpu().numpy()
    stages = layer.st.stages.cpu().numpy()

    out = {
        "metric": "sparse-attn layer ms + dense-equiv TFLOP/s at L=75.6K,d=128; MFMA util %",
        "value": round(w.dense_flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s (dense-equivalent)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.description, "B": w.B, "H": w.H, "L": w.L, "d": w.d,
                   "selection": selection_name(kw), "compensate": args.compensate,
                   "params": {k: (round(v, 6) if isinstance(v, float) else v) for k, v in kw.items()}},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": (measured_traffic(args.workload, args.variant, args.compensate)
                                 if not args.key_metric and not args.tail_block and not pca else None),
                     "kernel": "ac_sparse_attn: k_attn_rows + k_attn_prep + k_attn (block-sparse attention)",
                     "algorithmic_flops_per_launch": attn_flops, "avg_launch_ms": round(attn_ms, 4)},
        "phase_ms": {"cluster_q": round(float(phase_ms[0]), 3), "cluster_k": round(float(phase_ms[1]), 3),
                     "clustering_q_beside_k": round(float(phase_ms[2]), 3),
                     "score_select": round(float(phase_ms[3]), 3), "sparse_attn": round(attn_ms, 3)},
        "timed_step": ("ac_layer (warm: a later denoising step after a 2% perturbation of Q and K)" if args.warm
                       else "ac_layer (cold)") if use_layer else "entry points in ac_layer order",
        "_phase_note": ("phases from a separate pass of the entry points, the query clustering beside the key "
                        "clustering from the start; " if use_layer else "") +
                       "score_select includes ac_tail_merge when tail merging is on",
        "key_clustering": ("interaction-aware, %d clusters (iCATS)" % args.key_metric if args.key_metric
                           else "principal-component split, queries in clusters of %d, keys of %d "
                                "(ClusterAttention)" % pca if pca else "Algorithm 1 (multi-stage)"),
        "tail_merge": None if not args.tail_block else dict(
            zip(("block", "query_blocks_before", "query_blocks_after"),
                (args.tail_block,) + layer.query_blocks(args.tail_block))),
        "layer": {"density_pairs": round(pairs / (w.BH * float(w.L) ** 2), 4), "fallback_heads": int(fb.sum()),
                  "key_clusters_min_max": [int(ncl.min()), int(ncl.max())],
                  "stages_max": int(stages.max())},
    }
    if not args.no_baselines:
        dense_kw = workload_params(args.workload, "dense", 0)
        dl = Layer(Qd, Kd, Vd, (w.B, w.H, w.L, w.d), _abi(dense_kw))
        dl.step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            dl.attn_only()
        e1.record()
        torch.cuda.synchronize()
        own_dense = e0.elapsed_time(e1) / 3
        del dl
        sd = sdpa_ms(Qd, Kd, Vd)
        best = min(x for x in (own_dense, sd) if x is not None)
        out["dense_baseline"] = {"own_dense_attn_ms": round(own_dense, 3), "sdpa_flash_ms": None if sd is None else round(sd, 3),
                                 "speedup_layer_vs_best_dense": round(best / ms_step, 3),
                                 "own_dense_tflops": round(w.dense_flops / (own_dense * 1e-3) / 1e12, 2)}
    if not args.no_cpu and not args.no_baselines:
        out["cpu_baseline"] = cpu_baseline(w, Q, K, V, kw)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
