"""Host logic of bench.py (no GPU): the one-GPU contract, the algorithmic work
that the roofline figures divide by, and the source check that keeps measured
traffic tied to the code it was taken on."""

import importlib.util
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_attention_work_counts_the_visible_pairs():
    """work_attn's flops are 4 * d * heads_q per visible (query, key) pair;
    the pairs are counted here from the mask itself: every memory row, and
    local row r for query t when r <= L - T + t."""
    import msa_inputs as mi
    b = _bench()
    for t_len, loc, mem in [(1, 1, 0), (5, 9, 3), (16, 16, 8), (7, 30, 0)]:
        cfg = mi.scaled(mi.PREFILL, q_len=t_len, loc_len=loc, topk=mem // 8 if mem else 0, batch=2)
        mem_rows = cfg.mem_len
        t = np.arange(t_len)[:, None]
        r = np.arange(loc)[None, :]
        visible = int((r <= loc - t_len + t).sum()) + t_len * mem_rows
        w = b.work_attn(cfg)
        assert w["flops"] == 4 * cfg.dim * cfg.heads_q * cfg.batch * visible


def test_route_work_is_one_product_per_query_chunk_head_and_dim():
    import msa_inputs as mi
    b = _bench()
    cfg = mi.PREFILL
    w = b.work_route(cfg)
    assert w["flops"] == 2 * cfg.batch * cfg.q_len * cfg.n_doc * cfg.chunks_per_doc * cfg.heads_kv * cfg.dim
    assert w["bound"] == "mfma"                       # 2048 query tokens: well past the ridge
    dec = b.work_route(mi.DECODE)
    assert dec["bound"] == "hbm"                      # 32 single tokens: a scan of the bank


def test_roofline_entry_fractions():
    b = _bench()
    e = b.roofline_entry({"bound": "hbm", "bytes": 8e9, "flops": 0}, 1000.0)    # 8 GB in 1 s
    assert abs(e["achieved"] - 8.0) < 1e-9 and abs(e["frac"] - 8.0 / b.HBM_PEAK_GBS) < 1e-12
    e = b.roofline_entry({"bound": "mfma", "bytes": 0, "flops": 2.5e15}, 1000.0)
    assert abs(e["frac"] - 1.0) < 1e-12 and e["unit"] == "TFLOP/s"


def test_every_workload_stage_names_existing_sources():
    b = _bench()
    csrc = os.path.join(ROOT, "routed_sparse_attention_msa_amd", "csrc")
    for wl, stages in b.STAGE_KERNELS.items():
        for stage, entry in stages.items():
            for name in entry[1].split("|"):
                assert os.path.exists(os.path.join(csrc, name)), (wl, stage, name)


def test_source_hash_follows_included_headers(tmp_path, monkeypatch):
    """The recorded traffic of a stage is dropped when any file its kernels
    include changes, not only the named source."""
    b = _bench()
    src = tmp_path / "routed_sparse_attention_msa_amd" / "csrc"
    src.mkdir(parents=True)
    (src / "k.hip").write_text('#include "common.h"\nint k;\n')
    (src / "common.h").write_text("int c = 1;\n")
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    h1 = b.kernel_source_sha("k.hip")
    (src / "common.h").write_text("int c = 2;\n")
    h2 = b.kernel_source_sha("k.hip")
    assert h1 != h2


def test_traffic_summary_counts_each_kernels_launches(tmp_path, monkeypatch):
    """A stage's bytes per call sum its kernels' per-launch counters times their launches per call: the
    interleave rounds run one routing launch (all rounds' queries) and one top-k launch per round."""
    import csv
    import json
    b = _bench()
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    d = tmp_path / "traffic"

    def write(name, rows):
        p = d / name / "run"
        p.mkdir(parents=True)
        with open(p / "run_counter_collection.csv", "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Value"])
            w.writeheader()
            for k, v in rows:
                w.writerow({"Kernel_Name": k, "Counter_Value": v})

    gib_kib = (1 << 30) / 1024
    for kind in ("fetch", "write"):
        write(f"copy_{kind}", [("void at::native::neg_kernel", gib_kib)])
        write(f"interleave_{kind}", [("msa::(anonymous namespace)::route_tiled_kernel(int)", 1000.0),
                                     ("msa::(anonymous namespace)::topk_small_kernel<8>(int)", 10.0)])
    b.summarize_traffic(str(d))
    rec = json.load(open(tmp_path / "profiles" / "traffic.json"))["interleave"]["rounds"]
    assert abs(rec["read_bytes"] - (1000.0 + 3 * 10.0) * 1024) < 1e-6
    assert abs(rec["bytes_per_launch"] - 2 * (1000.0 + 3 * 10.0) * 1024) < 1e-6
