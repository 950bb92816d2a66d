"""bench.py's contract and its profile summaries, on the CPU: the multi-GPU
refusal, the selection names, and the tables that `--summarize` builds from
bench lines and rocprofv3 kernel traces (synthetic inputs with known
answers)."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr


def test_selection_names():
    assert bench.selection_name(bench.workload_params("hunyuan", "density", 0)) == "top-K 64"
    assert bench.selection_name(bench.workload_params("wan", "density", 0)) == "top-K at 15% density"
    assert bench.selection_name(bench.workload_params("wan", "topp", 0)) == "top-p 0.9"
    assert bench.selection_name(bench.workload_params("wan", "dense", 0)) == "dense"


def test_hunyuan_uses_the_absolute_threshold_of_table7():
    import clustered_sparse_attention_amd as ac
    kw = bench.workload_params("hunyuan", "density", 0)
    assert kw["tau_rule"] == ac.AC_TAU_ABS and kw["tau_param"] == 5.5 and kw["m0"] == 100 and kw["topk"] == 64


def _bench_line(ms, workload="Wan2.1-14B-like H=40 L=75600 d=128", warm=False, cpu=True):
    line = {"metric": "m", "value": 117.05 / (ms * 1e-3) / 1e3, "ms_per_step": ms,
            "config": {"workload": workload, "selection": "top-K at 15% density", "compensate": 0},
            "timed_step": "ac_layer (warm: later step)" if warm else "ac_layer (cold)",
            "phase_ms": {"cluster_q": 7.0, "cluster_k": 16.0, "clustering_q_beside_k": 16.1, "score_select": 0.3,
                         "sparse_attn": 20.0},
            "roofline": {"frac": 0.36, "algorithmic_flops_per_launch": 1.8e13},
            "layer": {"density_pairs": 0.158, "fallback_heads": 0, "key_clusters_min_max": [800, 802]},
            "dense_baseline": {"own_dense_attn_ms": 120.0, "sdpa_flash_ms": 165.0,
                               "speedup_layer_vs_best_dense": round(120.0 / ms, 3)}}
    if cpu:
        line["cpu_baseline"] = {"value": 0.29, "cores": 16, "complete_head": True}
    return json.dumps(line)


def test_overridden_shapes_are_named_in_the_description():
    """A bench line run with --heads or --seq-len names the shape it ran."""
    import csa_inputs as gen
    w = gen.get_workload("wan", H=5, L=18900)
    assert (w.H, w.L) == (5, 18900) and "H=5 L=18900 d=128" in w.description
    assert gen.get_workload("wan").description.endswith("H=40 L=75600 d=128")
    assert "H=2 L=180000" in gen.get_workload("long", H=2).description


def test_summarize_configs_table(tmp_path):
    a, b = tmp_path / "a.log", tmp_path / "b.log"
    a.write_text("[bench] noise\n" + _bench_line(36.0) + "\n")
    b.write_text(_bench_line(26.5, warm=True, cpu=False) + "\n")
    out = tmp_path / "t.md"
    bench.summarize(["configs", str(out), "the", "command", "::", str(a), str(b)])
    text = out.read_text()
    rows = [l for l in text.splitlines() if l.startswith("| Wan2.1")]
    assert len(rows) == 2
    assert "| cold |" in rows[0] and "| 36.00 |" in rows[0] and "3.33x" in rows[0] and "complete head" in rows[0]
    assert "| warm |" in rows[1] and "4.53x" in rows[1] and rows[1].endswith("| — |")
    assert "Command: `the command`" in text
    assert text.startswith("# Bench lines, all workloads")
    bench.summarize(["configs", str(out), "title=Sequence sweep", "cmd", "::", str(a)])
    text = out.read_text()
    assert text.startswith("# Sequence sweep\n") and "Command: `cmd`" in text
    assert len([l for l in text.splitlines() if l.startswith("| Wan2.1")]) == 1


def test_summarize_configs_marks_the_principal_component_rows(tmp_path):
    d = json.loads(_bench_line(29.4, cpu=False))
    d["timed_step"] = "entry points in ac_layer order"
    d["key_clustering"] = "principal-component split, queries in clusters of 256, keys of 64 (ClusterAttention)"
    lg = tmp_path / "p.log"
    lg.write_text(json.dumps(d) + "\n")
    out = tmp_path / "t.md"
    bench.summarize(["configs", str(out), "cmd", "::", str(lg)])
    row = [l for l in out.read_text().splitlines() if l.startswith("| Wan2.1")][0]
    assert "| cold, principal-component split 256/64 |" in row and "| 29.40 |" in row


def test_summarize_denoise_table(tmp_path):
    steps = [{"step": 0, "mode": "dense", "ms": 116.0}, {"step": 1, "mode": "cold", "ms": 38.0, "sel_param": 0.15},
             {"step": 2, "mode": "warm", "ms": 30.0, "sel_param": 0.15}]
    run = {"value": 184.0, "workload": "W", "steps": 3, "warmup_steps": 1, "kmax": 800, "fallback_heads": 1,
           "topp_schedule": None, "per_step": steps, "cold_ms": 38.0, "warm_ms_mean": 30.0, "own_dense_ms": 116.0,
           "sdpa_flash_ms": 165.0}
    lg = tmp_path / "d.log"
    lg.write_text(json.dumps(run) + "\n")
    out = tmp_path / "d.md"
    bench.summarize(["denoise", str(out), "cmd", "::", str(lg)])
    row = [l for l in out.read_text().splitlines() if l.startswith("| density")][0]
    # 3 steps of own dense 348 ms against 184 ms; of SDPA 495 ms
    assert "| 348.0 | 495.0 | 1.89x | 2.69x |" in row


def _trace(path, launches):
    """A rocprofv3 kernel-trace CSV with the given (name, duration ns) launches in order."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 1000
        for name, dur in launches:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur})
            t += dur + 10


def test_summarize_roofline_takes_the_right_launches(tmp_path):
    step = [("k_qnorm", 300_000), ("k_kpp_seq", 1), ("k_assign_res", 200_000), ("k_update_partial", 150_000),
            ("k_sort_scatter", 30_000), ("k_assign_res", 200_000), ("k_assign_res", 999_999),
            ("k_kpp_seq", 1), ("k_assign_res", 250_000), ("k_update_partial", 150_000), ("k_sort_scatter", 30_000),
            ("k_assign_res", 250_000), ("k_kst_chunks", 10_000), ("k_kstats_part", 400_000),
            ("k_kstats_fin", 40_000), ("ac::k_attn<128, 1>", 20_000_000)]
    tr = tmp_path / "tr.csv"
    _trace(tr, step * 3)  # a warm-up step and two timed ones
    lg = tmp_path / "b.log"
    lg.write_text(_bench_line(36.0) + "\n")
    out = tmp_path / "r.md"
    bench.summarize(["roofline", str(tr), str(lg), str(out), "wan", "cmd"])
    rows = {l.split("|")[1].strip(): l for l in out.read_text().splitlines() if l.startswith("| k_")}
    wan_x = 40 * 75600 * 128 * 2.0
    # queries: iterations 0-1 after the first seeding at 200 us each; never the 999 us launch
    q = rows["k_assign_res, queries, iterations 0-1 (n = L, m = 65)"]
    assert "| 0.200 ms |" in q and f"{wan_x / 200e-6 / 1e9:.0f} GB/s" in q
    k = rows["k_assign_res, keys, stage 0, iterations 0-1 (n = L, m = 200)"]
    assert "| 0.250 ms |" in k
    ks = rows["k_kst_chunks + k_kstats_part + k_kstats_fin (one launch each)"]
    assert "| 0.450 ms |" in ks
    at = rows["k_attn"]
    assert "| 20.000 ms |" in at and "900 TFLOP/s" in at and "0.36 (MFMA)" in at


def test_summarize_pca_takes_the_last_step_of_each_side(tmp_path):
    """Two queues, two layer steps: the table lists the last step's split tree,
    levels and finishing kernels per side, and the span covers both sides."""
    def step(t0):
        key = [("ac::k_pca_tree_wide", 10_000), ("ac::k_iota_perm", 5_000), ("void ac::k_pca_level<128>", 40_000),
               ("void ac::k_pca_project<128>", 30_000), ("void ac::k_pca_level<128>", 30_000)] + \
              [("void ac::k_pca_level<128>", 100_000 * (i + 1)) for i in range(3)] + \
              [("ac::k_pca_finish", 20_000), ("void ac::k_kstats_part<128>", 300_000)]
        qry = [("void ac::k_qnorm<128>", 300_000), ("ac::k_pca_tree_wide", 9_000)] + \
              [("void ac::k_pca_level<128>", 50_000) for _ in range(2)] + [("ac::k_seg_mean", 40_000)]
        out = []
        for q, seq, t in (("1", key, t0), ("2", qry, t0 + 7_000)):
            for name, dur in seq:
                out.append({"Kernel_Name": name, "Queue_Id": q, "Start_Timestamp": t, "End_Timestamp": t + dur})
                t += dur + 1_000
        out.append({"Kernel_Name": "void ac::k_score_prep_a<128>", "Queue_Id": "1", "Start_Timestamp": t0 + 5_000_000,
                    "End_Timestamp": t0 + 5_001_000})
        return out
    tr = tmp_path / "tr.csv"
    with open(tr, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Queue_Id", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for r in step(1_000) + step(10_000_000):
            w.writerow(r)
    out = tmp_path / "p.md"
    bench.summarize(["pca", str(tr), str(out), "W", "the", "cmd"])
    text = out.read_text()
    assert "Command: `the cmd`" in text
    keys = text.split("## keys")[1].split("## queries")[0]
    qrys = text.split("## queries")[1]
    # level 0 in three launches (direction, projections, cut), then levels 1-3
    lv = [(l.split("|")[1].strip(), l.split("|")[2].strip()) for l in keys.splitlines()
          if "k_pca_level" in l or "k_pca_project" in l]
    assert [x[1] for x in lv] == ["0", "0", "0", "1", "2", "3"] and lv[1][0] == "ac::k_pca_project<128>"
    assert "| 300.0 us |" in [l for l in keys.splitlines() if "k_pca_level" in l][-1]
    assert "k_kstats_part" in keys and "k_score_prep" not in keys
    assert "k_qnorm" in qrys and "k_seg_mean" in qrys and qrys.count("k_pca_level") == 2
    # keys: 10 + 5 + 40 + 30 + 30 + 100 + 200 + 300 + 20 + 300 us and 9 gaps of 1 us
    assert keys.startswith(": 1.044 ms")
    # the last step only: every start within the second step's span
    starts = [float(l.split("|")[4].split()[0]) for l in text.splitlines() if l.startswith("| ac::") or l.startswith("| void")]
    assert min(starts) == 0.0 and max(starts) < 1000.0
