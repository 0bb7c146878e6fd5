"""Benchmark: one step = one pass of the whole fused GRPO loss hot path over
one batch of synthetic inputs on one GPU:

    advantages -> reference log-probs (no grad) -> loss forward -> loss backward

Prints ONE JSON line.  `value` is flattened tokens per second of the loss
forward + backward (the metric's rate; inputs resident in HBM before the timed
region), measured with HIP events around those two calls inside the timed
steps; the rate of the whole step (advantages and reference log-probs
included) is `step_tokens_per_s`.  Also reported: the forward + backward
fraction of dense bf16 MFMA peak, peak HBM (torch allocator peak and the
device's free memory before and after, from hipMemGetInfo), a roofline entry
for the dominant kernel, and the float64 oracle timed on the host cores on a
bounded sample of the same workload.

The roofline's per-kernel times come from a second pass of the same number of
steps, run right after the timed one with the library's per-kernel HIP events
on (each launch bracketed by two events on its own stream), so that the timed
steps carry no instrumentation.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "flattened tokens/s GRPO loss fwd+bwd (1 GPU) + % bf16 MFMA peak + peak HBM"
PEAK_FLOPS = {"bf16": 2.5e15, "f32": 157.3e12, "fp8": 5.0e15}   # MI355X dense MFMA peaks
# the largest single-GPU workload: the pages' long-context setting (Llama-3.1-8B
# LM head, 20K-token completions, 8 generations per prompt)
DEFAULT_WORKLOAD = "llama3.1-8b-20k-bf16"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


CSRC = os.path.join(ROOT, "grpo_policy_loss_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 1 << 30      # calibration copy for the HBM byte counters


def kernel_source_hash():
    """sha256 of the HIP sources: a traffic measurement is valid only for these."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def traffic_file(kernel, workload):
    return os.path.join(PROFILES, f"traffic_{kernel}_{workload}.md")


def read_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None
    when there is none or the kernels changed since the counters were taken."""
    path = traffic_file(kernel, workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        m = re.search(r"^traffic_record: (\{.*\})$", f.read(), flags=re.M)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec["hbm_bytes_per_launch"]


def summarize_traffic(fetch_csv, write_csv, workload, kernel="lse_partials"):
    """Turn two rocprofv3 --pmc runs of `bench.py --traffic-probe` (FETCH_SIZE,
    then WRITE_SIZE, in KiB per dispatch) into profiles/traffic_<kernel>_<workload>.md.
    Each counter is scaled by what it reads for the 1 GiB calibration copy.
    kernel "all": one file for each of the four GEMM kernels.  Launches of the
    backward past the last active chunk do no work (and fetch almost nothing);
    launches fetching under 1 % of the kernel's largest are left out."""
    if kernel == "all":
        for k in GEMM_KERNELS:
            summarize_traffic(fetch_csv, write_csv, workload, k)
        return
    def per_dispatch(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        return vals
    f = per_dispatch(fetch_csv, "FETCH_SIZE")
    w = per_dispatch(write_csv, "WRITE_SIZE")
    def pick(vals, pat):
        return [v for (d, n), v in sorted(vals.items(), key=lambda kv: int(kv[0][0])) if pat in n]
    kpat = "k_" + kernel + "<"
    kmangled = "k_" + kernel + "I"
    copy_f, copy_w = pick(f, "copyBuffer"), pick(w, "copyBuffer")
    kf = pick(f, kpat) or pick(f, kmangled)
    kw = pick(w, kpat) or pick(w, kmangled)
    if not (copy_f and copy_w and kf and kw):
        raise SystemExit("counter CSVs lack the calibration copy or the kernel")
    if len(kf) == len(kw):
        keep = [i for i, v in enumerate(kf) if v >= 0.01 * max(kf)]
        kf, kw = [kf[i] for i in keep], [kw[i] for i in keep]
    scale_f = copy_f[-1] * 1024 / COPY_BYTES          # KiB counted per true byte read
    scale_w = copy_w[-1] * 1024 / COPY_BYTES
    fetch = sum(kf) / len(kf) * 1024 / scale_f
    write = sum(kw) / len(kw) * 1024 / scale_w
    rec = {"kernel": kernel, "workload": workload, "source_hash": kernel_source_hash(),
           "launches": len(kf), "fetch_bytes_per_launch": round(fetch),
           "write_bytes_per_launch": round(write), "hbm_bytes_per_launch": round(fetch + write),
           "copy_fetch_scale": round(scale_f, 4), "copy_write_scale": round(scale_w, 4)}
    lines = [f"# HBM traffic of `k_{kernel}` on the {workload} workload", "",
             "Two counter runs of `bench.py --traffic-probe` (a 1 GiB device copy for calibration,",
             "then one step: reference log-probs, loss forward, loss backward), then this summary:", "",
             "```",
             "cd /tmp && export TMPDIR=/tmp",
             f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d $R/gpurun_out/tf -o run -- python3 $R/bench.py --traffic-probe --workload {workload}",
             f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d $R/gpurun_out/tw -o run -- python3 $R/bench.py --traffic-probe --workload {workload}",
             f"python3 $R/bench.py --summarize-traffic $R/gpurun_out/tf/run_counter_collection.csv $R/gpurun_out/tw/run_counter_collection.csv --workload {workload} --traffic-kernel all",
             "```", "",
             "| quantity | value |", "|---|---|",
             f"| calibration copy: FETCH_SIZE KiB counted per true KiB read | {scale_f:.4f} |",
             f"| calibration copy: WRITE_SIZE KiB counted per true KiB written | {scale_w:.4f} |",
             f"| launches measured (that did work) | {len(kf)} |",
             f"| FETCH_SIZE per launch (scaled) | {fetch / 1e6:.1f} MB |",
             f"| WRITE_SIZE per launch (scaled) | {write / 1e6:.1f} MB |",
             f"| HBM bytes per launch | {(fetch + write) / 1e6:.1f} MB |", "",
             "The benchmark reports this figure as `roofline.traffic` only while the HIP sources",
             "hash to `source_hash` below; after any kernel change it reports null.", "",
             "traffic_record: " + json.dumps(rec)]
    path = traffic_file(kernel, workload)
    with open(path, "w") as fo:
        fo.write("\n".join(lines) + "\n")
    print(path)


def summarize_stats(stats_csv, workload, steps, warmup, fp8=False):
    """Turn a `rocprofv3 --kernel-trace --stats` run of this benchmark into
    profiles/kernel_stats_<workload>[_fp8].md (per-kernel calls, average and
    total time, share of GPU time), with the command that made it."""
    import workloads

    w = workloads.BY_NAME[workload]
    rows = []
    for r in csv.DictReader(open(stats_csv)):
        name = r["Name"]
        m = re.search(r"(k_[a-z0-9_]+)", name)
        short = m.group(1) if m else None
        rows.append((short, name, int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                     float(r["TotalDurationNs"]) / 1e6, float(r["Percentage"])))
    ours = [r for r in rows if r[0] is not None]
    other_ms = sum(r[4] for r in rows if r[0] is None)
    other_pct = sum(r[5] for r in rows if r[0] is None)
    ours.sort(key=lambda r: -r[4])
    flag = " --fp8" if fp8 else ""
    kind = "fp8 e4m3 forward, bf16 backward" if fp8 else w.dtype
    lines = [f"# Kernel trace statistics: full step on the {workload} workload ({kind})", "",
             f"Workload: {w.N:,} flattened tokens ({w.prompts} prompts x {w.G} generations x {w.L}), "
             f"d = {w.d}, V = {w.V:,}, chunk {w.chunk}; one step = advantages + reference "
             f"log-probs + loss forward + loss backward. {steps} timed steps plus {warmup} "
             f"warm-up (each library kernel's launches appear {steps + warmup} times).", "",
             "Command (repo root on the GPU box, `R` = repo root):", "", "```",
             "cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv \\",
             f"    -d $R/gpurun_out/prof -o bench -- python3 $R/bench.py --workload {workload} "
             f"--steps {steps} --warmup {warmup} --no-cpu-baseline{flag}",
             f"python3 $R/bench.py --summarize-stats $R/gpurun_out/prof/bench_kernel_stats.csv "
             f"--workload {workload} --steps {steps} --warmup {warmup}{flag}",
             "```", "",
             "| kernel | calls | average (us) | total (ms) | share of GPU time |",
             "|---|---|---|---|---|"]
    for short, _, calls, avg, tot, pct in ours:
        lines.append(f"| `{short}` | {calls} | {avg:.1f} | {tot:.2f} | {pct:.2f}% |")
    lines.append(f"| (torch input generation, copies, fills) | | | {other_ms:.2f} | {other_pct:.2f}% |")
    lines.append("")
    lines.append("source_hash: " + kernel_source_hash())
    path = os.path.join(PROFILES, f"kernel_stats_{workload}{'_fp8' if fp8 else ''}.md")
    with open(path, "w") as fo:
        fo.write("\n".join(lines) + "\n")
    print(path)


def cpu_model():
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


GEMM_KERNELS = ("lse_partials", "dz", "dh_gemm", "dw_gemm")
NUM_SIMDS = 1024          # MI355X: 256 CUs x 4 SIMDs


def summarize_counters(csv_paths, workload, steps, warmup, out_name):
    """Per-kernel averages of the counters in one or more rocprofv3 --pmc runs of
    this benchmark (each counter summed over its hardware instances per
    dispatch, then averaged over the kernel's dispatches), with the derived
    MFMA figures: executed MFMA flops (SQ_INSTS_VALU_MFMA_MOPS_BF16 counts 512
    flops) against the algorithmic flops of a dispatch, the fraction of SIMD
    cycles the matrix core is busy (SQ_VALU_MFMA_BUSY_CYCLES over NUM_SIMDS x
    GRBM_GUI_ACTIVE of one XCD: rocprofv3 reports the sum over the 8), and the LDS
    bank-conflict cycles per active LDS cycle."""
    import workloads

    w = workloads.BY_NAME[workload]
    per = {}          # (kernel, dispatch) -> {counter: value}
    for path in csv_paths:
        for r in csv.DictReader(open(path)):
            # demangled ("ns::k_name(...)") or mangled ("..._114k_nameIDF16b...") names
            m = re.search(r"(?<![a-z])k_([a-z0-9_]+)", r["Kernel_Name"])
            if not m:
                continue
            key = (m.group(1), int(r["Dispatch_Id"]), path)
            d = per.setdefault(key, {})
            if "Start_Timestamp" in r and r["Start_Timestamp"]:
                d["_ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
            c = r["Counter_Name"]
            d[c] = d.get(c, 0.0) + float(r["Counter_Value"])
            if c == "GRBM_GUI_ACTIVE":
                d["_gui_n"] = d.get("_gui_n", 0) + 1
                d["_xcd"] = 8          # one value summed over the 8 XCDs
    kern = {}
    for (k, _, _), d in per.items():
        agg = kern.setdefault(k, {})
        for c, v in d.items():
            if c in ("_gui_n", "_xcd") or (c == "_ns" and "GRBM_GUI_ACTIVE" not in d):
                continue
            if c == "GRBM_GUI_ACTIVE":
                v = v / d["_xcd"]       # cycles of one XCD
            agg.setdefault(c, []).append(v)
    N_act = None
    lines = [f"# Hardware counters per kernel on the {workload} workload", "",
             f"Workload: {w.N:,} flattened tokens, d = {w.d}, V = {w.V:,}, chunk {w.chunk}; "
             f"{steps} step(s) after {warmup} warm-up, every dispatch of the library's kernels "
             "counted (launches of the backward past the last active chunk do no work and are "
             "left out of the averages).", "",
             "Commands (repo root on the GPU box, `R` = repo root), one counter set per run:", "", "```",
             "cd /tmp && export TMPDIR=/tmp"]
    for i, pth in enumerate(csv_paths):
        lines.append(f"rocprofv3 --pmc <set {i + 1}> --output-format csv -d $R/gpurun_out/pmc{i + 1} "
                     f"-o run -- python3 $R/bench.py --workload {workload} --steps {steps} "
                     f"--warmup {warmup} --no-cpu-baseline")
    lines.append(f"python3 $R/bench.py --summarize-counters <the csv files> --workload {workload} "
                 f"--steps {steps} --warmup {warmup} --counters-name {out_name}")
    lines += ["```", ""]
    counters = sorted({c for agg in kern.values() for c in agg if not c.startswith("_")})
    lines.append("Counter sets: " + ", ".join(f"`{c}`" for c in counters))
    lines += ["", "| kernel | dispatches | " + " | ".join(counters) + " |",
              "|---|---|" + "---|" * len(counters)]
    rows = {}
    for k in sorted(kern):
        agg = kern[k]
        # drop dispatches that did no MFMA work (backward launches past the last active chunk)
        mops = agg.get("SQ_INSTS_VALU_MFMA_MOPS_BF16")
        def mean(c):
            v = agg[c]
            if mops is not None and len(mops) == len(v) and k in GEMM_KERNELS:
                v = [x for x, mm in zip(v, mops) if mm > 0] or v
            return sum(v) / len(v)
        n = len(next(iter(agg.values())))
        rows[k] = {c: mean(c) for c in agg}
        lines.append(f"| `k_{k}` | {n} | " + " | ".join(
            f"{rows[k][c]:.4g}" if c in rows[k] else "" for c in counters) + " |")
    if any("SQ_INSTS_VALU_MFMA_MOPS_BF16" in r for r in rows.values()):
        lines += ["", "Derived, per dispatch that did work:", "",
                  "| kernel | executed MFMA TFLOP | matrix core busy | clock (GHz, GUI cycles / time) | LDS bank-conflict cycles per LDS cycle |",
                  "|---|---|---|---|---|"]
        for k, r in rows.items():
            if k not in GEMM_KERNELS:
                continue
            ex = r.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0) * 512 / 1e12
            busy = (r["SQ_VALU_MFMA_BUSY_CYCLES"] / (NUM_SIMDS * r["GRBM_GUI_ACTIVE"])
                    if "SQ_VALU_MFMA_BUSY_CYCLES" in r and r.get("GRBM_GUI_ACTIVE") else None)
            conf = (r["SQ_LDS_BANK_CONFLICT"] / r["SQ_LDS_IDX_ACTIVE"]
                    if r.get("SQ_LDS_IDX_ACTIVE") and "SQ_LDS_BANK_CONFLICT" in r else None)
            clk = (r["GRBM_GUI_ACTIVE"] / r["_ns"]) if r.get("_ns") and "GRBM_GUI_ACTIVE" in r else None
            lines.append(f"| `k_{k}` | {ex:.4f} | " + (f"{busy:.1%}" if busy is not None else "") +
                         " | " + (f"{clk:.2f}" if clk else "") + " | " +
                         (f"{conf:.3f}" if conf is not None else "") + " |")
    lines.append("")
    lines.append("source_hash: " + kernel_source_hash())
    path = os.path.join(PROFILES, f"counters_{out_name}.md")
    with open(path, "w") as fo:
        fo.write("\n".join(lines) + "\n")
    print(path)


def alg_flops(kind, d, V, N, N_act):
    """Algorithmic MFMA flops of one step's launches of a kernel kind."""
    if kind == "lse_partials":          # reference pass + loss forward: 2 d V per token each
        return 2 * (2.0 * d * V * N)
    if kind in ("dz", "dh_gemm", "dw_gemm"):   # backward, active tokens only
        return 2.0 * d * V * N_act
    return None


def slab_columns(w, dt):
    """Vocabulary columns of the backward's dZ slab under the default workspace:
    the two workspace sizes differ by exactly the slab beyond 256 columns."""
    import grpo_policy_loss_amd as gp
    full = gp.grpo_workspace_bytes(gp.GRPO_OP_BWD, w.N, w.d, w.V, dt, w.chunk)
    least = gp.grpo_workspace_bytes(gp.GRPO_OP_BWD_MIN, w.N, w.d, w.V, dt, w.chunk)
    cpad = -(-min(w.chunk, w.N) // 256) * 256
    es = 4 if dt == gp.GRPO_F32 else 2        # the slab is bf16 for bf16 and fp8 inputs
    return 256 + (full - least) // (cpad * es)


def cpu_baseline(w, inp, seconds=15.0, opts=None, gpu=None):
    """The float64 oracle, as it stands, on a bounded sample: the first n
    flattened tokens of the batch, run through reference log-probs, loss forward
    and loss backward, on all host threads BLAS uses.

    With `gpu` (the last timed step's outputs: ref, lp, lse, kl, dH), the
    sample's outputs are also compared with the GPU's for the same tokens; see
    sample_parity."""
    import numpy as np
    import threadpoolctl

    import oracle

    H = inp["H"].detach().cpu()
    H_ref = inp["H_ref"].detach().cpu()
    W64 = inp["W"].detach().to("cpu").double().numpy()
    y = inp["y"].cpu().numpy().astype(np.int64)
    mask = inp["mask"].cpu().numpy()
    r = inp["rewards"].cpu().numpy()

    # per-token advantages, so a sample may end inside a sequence (seq_len 1 below)
    adv_tok = np.repeat(oracle.group_advantages(r, w.G), w.L)

    last = {}

    def run(n):
        Hs = H[:n].double().numpy()
        Hr = H_ref[:n].double().numpy()
        ys, ms, adv = y[:n], mask[:n], adv_tok[:n]
        t0 = time.perf_counter()
        ref, _ = oracle.token_logprobs(Hr, W64, ys, opts=opts)
        fwd = oracle.loss_forward(Hs, W64, ys, ms, adv, ref, 1, 0.04, opts=opts)
        dH, _ = oracle.loss_backward(Hs, W64, ys, ms, adv, ref, 1, 0.04, opts=opts)
        last.update(n=n, ref=ref, lp=fwd["lp"], lse=fwd["lse"], kl=fwd["kl"], dH=dH)
        return time.perf_counter() - t0

    # size the sample to about `seconds` of work: small runs carry fixed costs, so
    # rescale from each measured run until one lands within half of the target
    cap = min(w.N, 8192)
    n, t = 16, run(16)
    for _ in range(3):
        if t >= 0.5 * seconds or n >= cap:
            break
        n = int(max(16, min(cap, n * seconds / max(t, 1e-3))))
        t = run(n)
    n2, t2 = n, t
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    parity = sample_parity(last, gpu, mask, opts) if gpu is not None else None
    return parity, {"value": n2 / t2, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"first {n2} flattened tokens of the batch (ref + fwd + bwd, float64 "
                      f"NumPy, full V={w.V}, d={w.d}); {t2:.1f} s on "
                      f"{len(os.sched_getaffinity(0))} visible host CPUs"}


def sample_parity(orc, gpu, mask, opts):
    """Errors of the GPU's outputs on the oracle's sample (the first n tokens).
    ref_lp, lp, lse and kl of a token depend only on its own row, so they are
    compared directly.  The GPU's dH rows carry the batch's 1 / sum(mask) where
    the sample's carry its own; rescaled by the ratio of the two they are
    compared by cosine and max |diff| / max |oracle|.  (Under the per-sequence
    mean the sample's weights differ token by token, so dH is left out.)"""
    import numpy as np
    n = orc["n"]
    out = {"tokens": n}
    for k in ("ref", "lp", "lse", "kl"):
        g = gpu[k][:n].double().cpu().numpy()
        out[f"max_abs_{'ref_lp' if k == 'ref' else k}"] = float(np.abs(g - orc[k]).max())
    if not (opts or {}).get("aggregation"):
        m_all = max(float(mask.sum()), 1.0)
        m_smp = max(float(mask[:n].sum()), 1.0)
        g = gpu["dH"][:n].double().cpu().numpy() * (m_all / m_smp)
        o = orc["dH"]
        den = float(np.linalg.norm(g) * np.linalg.norm(o))
        out["dH_cosine"] = float((g * o).sum() / den) if den > 0 else None
        top = float(np.abs(o).max())
        out["dH_max_abs_rel"] = float(np.abs(g - o).max() / top) if top > 0 else None
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--temperature", type=float, default=0.0,
                    help="logit temperature (0: off); the logit options apply to every pass")
    ap.add_argument("--softcap", type=float, default=0.0, help="logit softcapping (0: off)")
    ap.add_argument("--scale-multiply", type=float, default=0.0, help="logit scale multiply (0: off)")
    ap.add_argument("--scale-divide", type=float, default=0.0, help="logit scale divide (0: off)")
    ap.add_argument("--chunk", type=int, default=-1,
                    help="tokens per chunk: -1 the workload's own, 0 automatic (grpo_auto_chunk "
                         "with half of the free HBM as the budget)")
    ap.add_argument("--fp8", action="store_true",
                    help="fp8 e4m3 forward (H, H_ref per-token scales, W one scale; quantised "
                         "inside the timed step) with the bf16 backward on exact copies")
    ap.add_argument("--kl-estimator", type=int, default=0, choices=(0, 1, 2),
                    help="0 reverse k3 (default), 1 forward, 2 reverse with the factor q")
    ap.add_argument("--no-detach", action="store_true",
                    help="ratio without the detach (the advantage term has no gradient)")
    ap.add_argument("--sequence-mean", action="store_true",
                    help="per-sequence mean aggregation instead of the token mean")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run a 1 GiB calibration copy and one step, then exit")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic summary from two counter runs of --traffic-probe")
    ap.add_argument("--summarize-counters", nargs="+", metavar="PMC_CSV",
                    help="write profiles/counters_<name>.md from rocprofv3 --pmc runs of this "
                         "benchmark")
    ap.add_argument("--counters-name", default=None,
                    help="file stem for --summarize-counters (default: the workload name)")
    ap.add_argument("--traffic-kernel", default="lse_partials",
                    help="kernel for --summarize-traffic (without k_), or all four GEMM kernels")
    ap.add_argument("--summarize-stats", metavar="STATS_CSV",
                    help="write the kernel statistics summary from a rocprofv3 --stats run of "
                         "this benchmark (with the --workload/--steps/--warmup it ran with)")
    args = ap.parse_args()
    xopts = {k: v for k, v in (("logit_scale_multiply", args.scale_multiply),
                               ("logit_scale_divide", args.scale_divide),
                               ("logit_softcapping", args.softcap),
                               ("temperature", args.temperature),
                               ("kl_estimator", args.kl_estimator),
                               ("no_detach", int(args.no_detach)),
                               ("aggregation", int(args.sequence_mean))) if v} or None

    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.workload, args.steps, args.warmup,
                           args.counters_name or args.workload)
        return

    if args.summarize_stats:
        summarize_stats(args.summarize_stats, args.workload, args.steps, args.warmup, args.fp8)
        return

    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic[0], args.summarize_traffic[1], args.workload,
                          args.traffic_kernel)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import grpo_policy_loss_amd as gp
    import workloads

    w = workloads.BY_NAME[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.chunk > 0:
        w = w.scaled(chunk=args.chunk)
    elif args.chunk == 0:
        w = w.scaled(chunk=gp.auto_chunk(w.B, w.L, w.d, w.V,
                                         gp.GRPO_BF16 if w.dtype == "bf16" else gp.GRPO_F32))
    log(f"[bench] workload {w.name}: N={w.N} d={w.d} V={w.V} {w.dtype} chunk={w.chunk}")
    t0 = time.time()
    inp = workloads.generate(w, seed=args.seed, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs generated in {time.time() - t0:.1f}s")
    N, d, V, B, L = w.N, w.d, w.V, w.B, w.L
    N_act = int(inp["mask"].sum().item())
    dt = gp.GRPO_BF16 if w.dtype == "bf16" else gp.GRPO_F32
    if args.fp8:
        if w.dtype != "bf16":
            raise SystemExit("--fp8 quantises a bf16 workload")
        dt = gp.GRPO_FP8_E4M3
    ws_f = torch.empty(gp.grpo_workspace_bytes(gp.GRPO_OP_FWD, N, d, V, dt, w.chunk),
                       dtype=torch.uint8, device=dev)
    ws_b = torch.empty(gp.grpo_workspace_bytes(gp.GRPO_OP_BWD, N, d, V, dt, w.chunk),
                       dtype=torch.uint8, device=dev)
    dW = torch.zeros(V, d, dtype=torch.float32, device=dev)
    dH = torch.empty_like(inp["H"])
    stream = torch.cuda.current_stream()

    def step_fp8(ev=None):
        if ev is not None:
            ev[0].record(stream)
        adv = gp.grpo_advantages(inp["rewards"], w.G, workloads.EPS)
        Wq = gp.quantize_fp8(inp["W"], per_row=False)
        Rq = gp.quantize_fp8(inp["H_ref"], per_row=True)
        ref = gp.grpo_ref_logprobs_fp8(Rq, Wq, inp["y"], w.chunk, workspace=ws_f, opts=xopts)
        if ev is not None:
            ev[1].record(stream)
        Hq = gp.quantize_fp8(inp["H"], per_row=True)
        loss, lp, kl, lse = gp.grpo_loss_fwd_fp8(Hq, Wq, inp["y"], inp["mask"], adv, ref, B, L,
                                                 workloads.BETA, w.chunk, workspace=ws_f,
                                                 opts=xopts)
        if ev is not None:
            ev[2].record(stream)
        dW.zero_()
        gp.grpo_loss_bwd_fp8(Hq, Wq, inp["y"], inp["mask"], adv, ref, lp, lse, B, L,
                             workloads.BETA, 1.0, w.chunk, dW=dW, dH=dH, workspace=ws_b,
                             opts=xopts)
        if ev is not None:
            ev[3].record(stream)
        return loss

    last_out = {}   # the last bf16/f32 step's outputs, for the sampled parity check

    def step(ev=None):
        if args.fp8:
            return step_fp8(ev)
        if ev is not None:
            ev[0].record(stream)
        adv = gp.grpo_advantages(inp["rewards"], w.G, workloads.EPS)
        ref = gp.grpo_ref_logprobs(inp["H_ref"], inp["W"], inp["y"], w.chunk, workspace=ws_f,
                                   opts=xopts)
        if ev is not None:
            ev[1].record(stream)
        loss, lp, kl, lse = gp.grpo_loss_fwd(inp["H"], inp["W"], inp["y"], inp["mask"], adv, ref,
                                             B, L, workloads.BETA, w.chunk, workspace=ws_f,
                                             opts=xopts)
        if ev is not None:
            ev[2].record(stream)
        dW.zero_()
        gp.grpo_loss_bwd(inp["H"], inp["W"], inp["y"], inp["mask"], adv, ref, lp, lse, B, L,
                         workloads.BETA, 1.0, w.chunk, dW=dW, dH=dH, workspace=ws_b,
                         opts=xopts)
        if ev is not None:
            ev[3].record(stream)
        last_out.update(ref=ref, lp=lp, lse=lse, kl=kl, dH=dH)
        return loss

    if args.traffic_probe:
        src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        step()
        torch.cuda.synchronize()
        log("[bench] traffic probe done")
        return

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup {i + 1}/{args.warmup} done")

    torch.cuda.reset_peak_memory_stats(dev)
    free_before, total_hbm = torch.cuda.mem_get_info(dev)        # hipMemGetInfo
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    free_after, _ = torch.cuda.mem_get_info(dev)
    peak_bytes = torch.cuda.max_memory_allocated(dev)
    log(f"[bench] {args.steps} timed steps in {t_total:.3f}s")
    # per-kernel times: the same steps again, each launch bracketed by HIP events
    gp.grpo_timing_begin()
    torch.cuda.synchronize()
    t_inst = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    t_inst = time.perf_counter() - t_inst
    kernels = gp.grpo_timing_end()
    log(f"[bench] {args.steps} instrumented steps in {t_inst:.3f}s")

    ms_ref = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    ms_fwd = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    ms_bwd = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps
    ms_step = t_total * 1e3 / args.steps
    fb_flops = 2.0 * d * V * N + 6.0 * d * V * N_act
    peak = PEAK_FLOPS[w.dtype]

    # roofline of the dominant kernel: algorithmic flops / its measured time
    dom = max(kernels.items(), key=lambda kv: kv[1][1])
    dom_name, (dom_launches, dom_ms) = dom
    dom_flops = alg_flops(dom_name, d, V, N, N_act)
    roof = None
    if dom_flops is not None:
        # with --fp8 the lse pass runs fp8 MFMAs; the backward stays bf16
        if args.fp8 and dom_name == "lse_partials":
            peak = PEAK_FLOPS["fp8"]
        achieved = dom_flops * args.steps / (dom_ms * 1e-3) / 1e12
        tb = None if args.fp8 else read_traffic(dom_name, w.name)
        roof = {"kernel": dom_name, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": peak / 1e12, "unit": "TFLOP/s", "frac": round(achieved * 1e12 / peak, 4),
                "traffic": tb, "traffic_unit": "bytes per launch (HBM, counters)",
                "launches": dom_launches,
                "avg_launch_ms": round(dom_ms / dom_launches, 4)}

    # every GEMM kernel's algorithmic flops over its own measured time
    kernels_frac = {}
    for name, (_, ms) in kernels.items():
        fl = alg_flops(name, d, V, N, N_act)
        if fl is not None and ms > 0:
            pk = PEAK_FLOPS["fp8"] if (args.fp8 and name == "lse_partials") else PEAK_FLOPS[w.dtype]
            kernels_frac[name] = round(fl * args.steps / (ms * 1e-3) / pk, 4)

    cpu = parity = None
    if not args.no_cpu_baseline:
        log("[bench] timing the float64 oracle on the host ...")
        parity, cpu = cpu_baseline(w, inp, args.cpu_seconds, xopts,
                                   None if args.fp8 else last_out)
        log(f"[bench] oracle {cpu['value']:.2f} tokens/s")

    out = {
        "metric": METRIC,
        "value": round(N / ((ms_fwd + ms_bwd) * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 fwd / bf16 bwd" if args.fp8 else w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": N, "active_tokens": N_act, "d": d, "V": V,
                   "chunk": w.chunk, "beta": workloads.BETA,
                   "step": "advantages + reference log-probs + loss fwd + loss bwd",
                   **({"opts": xopts} if xopts else {}), **({"fp8": True} if args.fp8 else {})},
        "value_is": "flattened tokens / (loss forward + loss backward time)",
        "step_tokens_per_s": round(N / (ms_step * 1e-3), 1),
        "fwd_bwd_mfma_frac": round(fb_flops / ((ms_fwd + ms_bwd) * 1e-3) / PEAK_FLOPS[w.dtype], 4),
        "ms": {"advantages+ref": round(ms_ref, 3), "fwd": round(ms_fwd, 3),
               "bwd": round(ms_bwd, 3)},
        "peak_hbm_gb": round(peak_bytes / 1e9, 3),
        "hip_mem_get_info_gb": {"free_before": round(free_before / 1e9, 3),
                                "free_after": round(free_after / 1e9, 3),
                                "total": round(total_hbm / 1e9, 3)},
        "full_fp32_logits_gb": round(N * V * 4 / 1e9, 2),
        "workspace_gb": {"fwd": round(ws_f.numel() / 1e9, 3), "bwd": round(ws_b.numel() / 1e9, 3),
                         "dz_slab_columns": slab_columns(w, dt)},
        "kernels_ms_per_step": {k: round(v[1] / args.steps, 3) for k, v in kernels.items()},
        "kernels_mfma_frac": kernels_frac,
        "instrumented_ms_per_step": round(t_inst * 1e3 / args.steps, 3),
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
