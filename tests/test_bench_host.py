"""Host-side logic of bench.py (no GPU): the multi-GPU refusal, the flop
accounting, and the two rocprofv3 summarizers with their staleness check."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_flops():
    d, V, N, Na = 1536, 151936, 32768, 27732
    assert bench.alg_flops("lse_partials", d, V, N, Na) == 2 * 2.0 * d * V * N
    for k in ("dz", "dh_gemm", "dw_gemm"):
        assert bench.alg_flops(k, d, V, N, Na) == 2.0 * d * V * Na
    assert bench.alg_flops("lse_merge", d, V, N, Na) is None


def _counter_csv(path, counter, rows):
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for disp, name, value in rows:
            f.write(f'{disp},"{name}",{counter},{value}\n')


def test_summarize_traffic_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    gib_kib = bench.COPY_BYTES / 1024
    kname = "void grpo::(anonymous namespace)::k_lse_partials<__bf16, false>(...)"
    # the copy reads 1 GiB and FETCH_SIZE reports half of it; the kernel reports 1000
    # and 3000 KiB (two dispatches, one of them split over two counter rows)
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE",
                 [(1, "__amd_rocclr_copyBuffer", gib_kib / 2), (2, kname, 600), (2, kname, 400),
                  (3, kname, 3000), (4, "k_lse_merge", 77)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE",
                 [(1, "__amd_rocclr_copyBuffer", gib_kib), (2, kname, 10), (3, kname, 30)])
    bench.summarize_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "wl")
    text = open(tmp_path / "traffic_lse_partials_wl.md").read()
    rec = json.loads(text.split("traffic_record: ")[1])
    assert rec["launches"] == 2
    assert rec["copy_fetch_scale"] == 0.5 and rec["copy_write_scale"] == 1.0
    assert rec["fetch_bytes_per_launch"] == round(2000 * 1024 / 0.5)    # mean 2000 KiB, x2
    assert rec["write_bytes_per_launch"] == round(20 * 1024)
    assert rec["source_hash"] == bench.kernel_source_hash()
    assert bench.read_traffic("lse_partials", "wl") == rec["hbm_bytes_per_launch"]


def test_traffic_record_goes_stale_when_the_kernels_change(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    rec = {"source_hash": "0" * 16, "hbm_bytes_per_launch": 123}
    (tmp_path / "traffic_lse_partials_wl.md").write_text("traffic_record: " + json.dumps(rec) + "\n")
    assert bench.read_traffic("lse_partials", "wl") is None
    assert bench.read_traffic("lse_partials", "other") is None


def test_summarize_stats_table(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    csv_path = tmp_path / "stats.csv"
    csv_path.write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        '"_ZN4grpo12_GLOBAL__N_14k_dzIDF16bLb0EEEvPKT_",8,8000000,1000000.0,20.0,1,2,0\n'
        '"_ZN4grpo12_GLOBAL__N_114k_lse_partialsIDF16bLb0EEEvPKT_",16,32000000,2000000.0,78.0,1,2,0\n'
        '"void at::native::vectorized_elementwise_kernel<4>",3,800000,266666.7,2.0,1,2,0\n')
    bench.summarize_stats(str(csv_path), "qwen2.5-1.5b-bf16", 3, 1)
    text = open(tmp_path / "kernel_stats_qwen2.5-1.5b-bf16.md").read()
    lines = [l for l in text.splitlines() if l.startswith("| `")]
    assert lines[0].startswith("| `k_lse_partials` | 16 | 2000.0 | 32.00 | 78.00% |")
    assert lines[1].startswith("| `k_dz` | 8 | 1000.0 | 8.00 | 20.00% |")
    assert "| (torch input generation, copies, fills) | | | 0.80 | 2.00% |" in text
    assert "--steps 3 --warmup 1" in text


@pytest.mark.parametrize("name", ["qwen2.5-1.5b-bf16", "llama3.1-8b-20k-bf16"])
def test_committed_profiles_name_their_command(name):
    text = open(os.path.join(ROOT, "profiles", f"kernel_stats_{name}.md")).read()
    assert "rocprofv3 --kernel-trace --stats" in text and f"--workload {name}" in text


def test_summarize_traffic_all_kernels_skips_idle_backward_launches(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    gib_kib = bench.COPY_BYTES / 1024
    names = {k: f"_ZN4grpo12_GLOBAL__N_19k_{k}IDF16bEEvPKT_" for k in bench.GEMM_KERNELS}
    rows_f = [(1, "__amd_rocclr_copyBuffer", gib_kib)]
    rows_w = [(1, "__amd_rocclr_copyBuffer", gib_kib)]
    disp = 2
    for k, n in names.items():
        # two working launches and one idle one (a backward chunk past the active tokens)
        for val in (5000, 7000, 3):
            rows_f.append((disp, n, val))
            rows_w.append((disp, n, val / 10))
            disp += 1
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", rows_f)
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", rows_w)
    bench.summarize_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "wl", "all")
    for k in bench.GEMM_KERNELS:
        rec = json.loads(open(tmp_path / f"traffic_{k}_wl.md").read().split("traffic_record: ")[1])
        assert rec["launches"] == 2
        assert rec["fetch_bytes_per_launch"] == 6000 * 1024
        assert rec["write_bytes_per_launch"] == 600 * 1024


def test_summarize_counters_derives_mfma_busy_and_clock(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    n = "_ZN4grpo12_GLOBAL__N_114k_lse_partialsIDF16bLb0EEEvPKT_"
    path = tmp_path / "pmc.csv"
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp\n")
        # one dispatch of 1 ms: 8 XCDs x 1.8e6 GUI cycles summed (1.8 GHz), matrix cores
        # busy 1.2e6 cycles on each of the 1024 SIMDs, 1e9 MFMA flops
        for c, v in (("GRBM_GUI_ACTIVE", 8 * 1.8e6), ("SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 1.2e6),
                     ("SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e9 / 512), ("SQ_LDS_IDX_ACTIVE", 100),
                     ("SQ_LDS_BANK_CONFLICT", 25)):
            f.write(f'7,"{n}",{c},{v},1000000,2000000\n')
    bench.summarize_counters([str(path)], "tiny-f32", 1, 1, "wl")
    text = open(tmp_path / "counters_wl.md").read()
    row = [l for l in text.splitlines() if l.startswith("| `k_lse_partials` | 0.0010")][0]
    assert "66.7%" in row and "1.80" in row and "0.250" in row


def test_sampled_parity_rescales_the_batch_gradient():
    """The bench's parity record compares the GPU's whole-batch outputs with the
    oracle's run on the first tokens alone.  Fed the oracle's own whole-batch
    outputs in place of the GPU's, it must report agreement to rounding: a
    missing or wrong 1/sum(mask) rescale of dH would not."""
    import numpy as np
    import torch

    import oracle
    import workloads

    w = workloads.BY_NAME["tiny-f32"]
    inp = workloads.generate(w, seed=3)
    H = inp["H"].double().numpy()
    Wt = inp["W"].double().numpy()
    y = inp["y"].numpy().astype(np.int64)
    mask = inp["mask"].numpy()
    adv = oracle.group_advantages(inp["rewards"].numpy(), w.G)
    ref, _ = oracle.token_logprobs(inp["H_ref"].double().numpy(), Wt, y)
    fwd = oracle.loss_forward(H, Wt, y, mask, adv, ref, w.L, workloads.BETA)
    dH, _ = oracle.loss_backward(H, Wt, y, mask, adv, ref, w.L, workloads.BETA, want_dW=False)
    full = {k: torch.from_numpy(np.asarray(v)) for k, v in
            dict(ref=ref, lp=fwd["lp"], lse=fwd["lse"], kl=fwd["kl"], dH=dH).items()}
    parity, cpu = bench.cpu_baseline(w, inp, seconds=0.2, gpu=full)
    assert cpu["kind"] == "oracle" and parity["tokens"] >= 16
    for k in ("max_abs_ref_lp", "max_abs_lp", "max_abs_lse", "max_abs_kl"):
        assert parity[k] < 1e-9, (k, parity[k])
    assert parity["dH_cosine"] > 1 - 1e-12
    assert parity["dH_max_abs_rel"] < 1e-9
    # a dH off by a factor of two is reported as such
    full["dH"] = full["dH"] * 2.0
    bad, _ = bench.cpu_baseline(w, inp, seconds=0.2, gpu=full)
    assert bad["dH_max_abs_rel"] > 0.5


def test_slab_columns_of_the_default_workspace():
    import workloads
    import grpo_policy_loss_amd as gp
    w = workloads.BY_NAME["llama3.1-8b-20k-bf16"]
    assert bench.slab_columns(w, gp.GRPO_BF16) == 81920       # the 1.25 GiB budget
    w = workloads.BY_NAME["qwen2.5-1.5b-bf16"]
    assert bench.slab_columns(w, gp.GRPO_BF16) == 152064      # the whole padded vocabulary
    w = workloads.BY_NAME["tiny-f32"]
    assert bench.slab_columns(w, gp.GRPO_F32) == 1024
