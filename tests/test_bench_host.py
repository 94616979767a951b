"""Host logic of bench.py (CPU, no GPU): the one-GPU contract, the rocprofv3 summaries and the
algorithmic work per pass that the roofline fractions divide by.

The counter summary is checked on synthetic rocprofv3 CSV files: the scale factors come from the
calibration copy's known bytes, and every pass's traffic is its FETCH and WRITE medians times those
factors.  The work accounting is checked against values written out from the definitions (a
critical block pair is QK^T and PV of 64 x 64 x d; the linear epilogue is one 64 x d x d product
per query block; pooling reads every valid row of Q once).
"""
import csv
import os
import subprocess
import sys
import types

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from workloads import WORKLOADS  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, env={**os.environ, "WORLD_SIZE": "1"})
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and '"error"' in r.stdout


def test_headline_metric_names_its_workload():
    w = WORKLOADS["wan13b_sla"]
    assert bench.metric_for(w) == "SLA fwd ms/layer + effective TFLOP/s, B1 H12 N32768 d128 bf16, 5% crit"
    assert "SALAD" in bench.metric_for(WORKLOADS["salad"])
    assert "16 selected + 512-token window" in bench.metric_for(WORKLOADS["nsa_prefill"])


def _write_csv(path, rows, fields):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=fields)
        wr.writeheader()
        wr.writerows(rows)


def test_counter_summary_calibrates_and_stamps(tmp_path):
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    copy = "void at::native::vectorized_elementwise_kernel<4, at::native::MulFunctor<float>>"
    attn = "void sla::attn_fwd_kernel<sla::bf16raw, 128, false, 1, 2, false>(sla::AttnParams)"
    pool = "void sla::pool_kernel<sla::bf16raw, 128>(...)"
    mib = 1
    # the copy moves 1 MiB each way; FETCH_SIZE counts half of it, WRITE_SIZE all (KiB per dispatch)
    fetch = [dict(Dispatch_Id=1, Kernel_Name=copy, Counter_Name="FETCH_SIZE", Counter_Value=512.0)]
    write = [dict(Dispatch_Id=1, Kernel_Name=copy, Counter_Name="WRITE_SIZE", Counter_Value=1024.0)]
    for n, (fa, wa) in enumerate([(100.0, 10.0), (300.0, 30.0), (200.0, 20.0)]):   # medians 200 and 20
        fetch.append(dict(Dispatch_Id=10 + n, Kernel_Name=attn, Counter_Name="FETCH_SIZE", Counter_Value=fa))
        write.append(dict(Dispatch_Id=10 + n, Kernel_Name=attn, Counter_Name="WRITE_SIZE", Counter_Value=wa))
    fetch.append(dict(Dispatch_Id=20, Kernel_Name=pool, Counter_Name="FETCH_SIZE", Counter_Value=64.0))
    write.append(dict(Dispatch_Id=20, Kernel_Name=pool, Counter_Name="WRITE_SIZE", Counter_Value=4.0))
    _write_csv(str(tmp_path / "f" / "run_counter_collection.csv"), fetch, fields)
    _write_csv(str(tmp_path / "w" / "run_counter_collection.csv"), write, fields)
    text = bench.summarize_counters(str(tmp_path / "f"), str(tmp_path / "w"), "wan13b_sla", mib, ["cf", "cw"])
    assert "factor 2.0000" in text and "factor 1.0000" in text
    lines = {l.split()[1]: l for l in text.splitlines() if l.startswith("TRAFFIC")}
    # attention: 200 KiB fetched x 2 + 20 KiB written x 1
    assert f"bytes_per_launch={200 * 1024 * 2 + 20 * 1024}" in lines["pass=attention"]
    assert f"kernel_source_sha={bench.kernel_source_digest('attention')}" in lines["pass=attention"]
    assert f"bytes_per_launch={64 * 1024 * 2 + 4 * 1024}" in lines["pass=pool"]
    assert "pass=marginal_states" not in lines          # no kernel of that pass in the runs


def test_counter_summary_needs_the_calibration_copy(tmp_path):
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    row = dict(Dispatch_Id=1, Kernel_Name="void sla::pool_kernel<float, 64>", Counter_Name="FETCH_SIZE",
               Counter_Value=1.0)
    _write_csv(str(tmp_path / "f" / "run_counter_collection.csv"), [row], fields)
    _write_csv(str(tmp_path / "w" / "run_counter_collection.csv"), [dict(row, Counter_Name="WRITE_SIZE")], fields)
    with pytest.raises(SystemExit):
        bench.summarize_counters(str(tmp_path / "f"), str(tmp_path / "w"), "tiny_sla", 1, ["a", "b"])


def test_trace_summary(tmp_path):
    fields = ["Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    rows = [dict(Kernel_Name="k_long", Start_Timestamp=0, End_Timestamp=3000),
            dict(Kernel_Name="k_long", Start_Timestamp=10000, End_Timestamp=15000),
            dict(Kernel_Name="k_short", Start_Timestamp=0, End_Timestamp=1000)]
    _write_csv(str(tmp_path / "t" / "run_kernel_trace.csv"), rows, fields)
    text = bench.summarize_trace(str(tmp_path / "t"), "cmd", "note").splitlines()
    assert text[0].endswith("note") and text[1].endswith("cmd")
    body = [l.split() for l in text[4:]]
    assert body[0][0] == "k_long" and body[1][0] == "k_short"      # longest total first
    assert body[0][1:] == ["2", "8.0", "4.00", "3.00", "5.00"]     # calls, total, avg, min, max (us)


def test_traffic_is_used_only_for_the_source_it_was_taken_on(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    sha = bench.kernel_source_digest("attention")
    (prof / "hbm_counters_wan13b_sla.txt").write_text(
        f"TRAFFIC pass=attention bytes_per_launch=1234 kernel_source_sha={sha}\n"
        "TRAFFIC pass=pool bytes_per_launch=99 kernel_source_sha=0000000000000000\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # kernel_source_digest reads the sources under ROOT: point it back at the real tree
    monkeypatch.setattr(bench, "kernel_source_digest",
                        lambda name: sha if name == "attention" else "ffffffffffffffff")
    assert bench.measured_traffic("attention", "wan13b_sla") == 1234
    assert bench.measured_traffic("pool", "wan13b_sla") is None       # stale digest
    assert bench.measured_traffic("attention", "salad") is None       # no summary for that workload


def _fake_layer(w, n_crit_entries, n_marg_entries, lin, fuse):
    rows = w.B * w.Hq * w.nb
    maps = {"crit_rowptr": torch.tensor([0, n_crit_entries]), "marg_rowptr": torch.tensor([0, n_marg_entries])}
    return types.SimpleNamespace(group=False, maps=maps, lin=lin, fuse_key_pooling=fuse), rows


def test_algorithmic_work_of_the_headline_layer():
    w = WORKLOADS["wan13b_sla"]
    B, H, d, Nv, nb = w.B, w.Hq, w.d, w.Nv, w.nb
    n_crit = 26 * B * H * nb                     # 26 critical blocks per row (5% of 512, rounded up)
    n_marg = 51 * B * H * nb
    layer, rows = _fake_layer(w, n_crit, n_marg, lin=1, fuse=True)
    work, pairs = bench.pass_work(w, layer)
    assert pairs == n_crit == 159744
    # attention: QK^T + PV per critical pair, plus phi(Q) S per query block of every head
    assert work["attention"] == ("mfma", n_crit * 4.0 * 64 * 64 * d + B * H * nb * 2.0 * 64 * d * d)
    assert work["attention"][1] == 347892350976.0
    # pooling of Q alone (the key block means come from the key-state pass): bf16 rows in, fp32 means out
    assert work["pool"] == ("hbm", B * H * (Nv * d * 2 + nb * d * 4)) and work["pool"][1] == 103784448
    # key states: K and V in; a bf16 d x d state, fp32 z and the fp32 key block mean out per key block
    assert work["kv_reduce"][1] == 2 * B * H * Nv * d * 2 + B * H * nb * (d * d * 2 + d * 4 + d * 4)
    # marginal sums: every state and z read once, a bf16 sum and fp32 u written per row
    assert work["marginal_states"][1] == B * H * nb * (d * d * 2 + d * 4) + rows * (d * d * 2 + d * 4)
    # scores: a d-long dot per (row, key block)
    assert work["scores"] == ("fp64", 2.0 * rows * nb * d)
    # without fusing the key means, pooling reads K as well
    layer2, _ = _fake_layer(w, n_crit, n_marg, lin=1, fuse=False)
    assert bench.pass_work(w, layer2)[0]["pool"][1] == B * 2 * H * (Nv * d * 2 + nb * d * 4)


def test_algorithmic_work_with_proj():
    """The Proj epilogue adds one 64 x d x d product per query block of every head."""
    w = WORKLOADS["wan13b_sla"]
    n_crit = 26 * w.B * w.Hq * w.nb
    layer, _ = _fake_layer(w, n_crit, 51 * w.B * w.Hq * w.nb, lin=1, fuse=True)
    plain = bench.pass_work(w, layer)[0]["attention"][1]
    layer.proj_w = object()
    assert bench.pass_work(w, layer)[0]["attention"][1] - plain == w.B * w.Hq * w.nb * 2.0 * 64 * w.d * w.d
