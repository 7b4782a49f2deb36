#!/usr/bin/env python3
"""Benchmark of the decode-time KV-cache eviction pass on one MI355X.

One step = one whole beacon eviction pass over every layer, request and KV
head of the workload (maintenance -> scoring -> top-B selection -> in-place
compaction; the last three run as one fused kernel, each workgroup taking its
head-cache through all three), at the synchronized batch point where every
request holds
N = B + 64 slots.  Between steps, outside the timed region, 64 fresh K/V rows
per head are written into slots [B, B+64) (what the next 64 decode tokens
would append), so every timed pass sees a full cache.  Inputs are seeded
synthetic data resident in HBM before timing starts.

Prints exactly one JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KV eviction passes/sec and achieved HBM GB/s (score+select+compact), % of peak"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E peak, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, vendor figure


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(*paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_source_hash(kernel):
    """Hash of a kernel's source file and the shared device headers."""
    csrc = os.path.join(ROOT, "decode_kv_cache_beacon_amd", "csrc")
    return source_hash(os.path.join(csrc, KERNEL_SOURCES[kernel]),
                       *(os.path.join(csrc, h) for h in SHARED_HEADERS))


SHARED_HEADERS = ("bkv_internal.h", "select_util.h", "compact_util.h")
KERNEL_SOURCES = {
    "beacon_update": "beacon_update.hip",
    "beacon_evict": "beacon_score.hip",
    "beacon_evict_shared": "beacon_score.hip",
    "beacon_score": "beacon_score.hip",
    "topk_select": "topk_select.hip",
    "kv_compact": "kv_compact.hip",
    "random_score": "random_score.hip",
    "random_evict": "random_score.hip",
    "page_retain": "page_retain.hip",
    "decode_attention": "decode_attention.hip",
}


def algorithmic_bytes(wl, N, P, moved_rows, hc_per_req):
    """Bytes each kernel must move at least once per pass: the roofline basis.

    For scoring and the fused pass these are the per-head-cache bytes of the
    pass's definition: every key read once (N*d*2), the fp32 beacons (K*d*4)
    and every moved row's K and V read and written (4*M*d*2); scores and keep
    lists that stay on chip, block-table reads and re-reads of keys from the
    caches are not counted (they are in extra_bytes).
    update : queries T*G*256 + beacons read+write 2*K*512 + counts 2*K*4
    score  : keys N*256 + beacons K*512
    select : scores read (N-P)*4 + keep list written B*4 (its own input and
             output: a separate kernel cannot keep them on chip)
    compact: moved rows 4*M*256
    evict  : the fused score+select+compact kernel: keys N*256 + beacons
             K*512 + moved rows 4*M*256
    """
    T, G, K, B = wl.steps, wl.group, wl.n_beacons, wl.budget
    upd = sc = sel = 0
    for n, p in zip(N, P):
        upd += hc_per_req * (T * G * 256 + 2 * K * 512 + 2 * K * 4)
        sc += hc_per_req * (n * 256 + K * 512)
        sel += hc_per_req * ((n - p) * 4 + B * 4)
    moves = 4 * moved_rows * 256
    return {"beacon_update": upd, "beacon_score": sc, "topk_select": sel, "kv_compact": moves,
            "beacon_evict": sc + moves}


def extra_bytes(wl, N, P, hc_per_req):
    """Bytes the kernels also move that the roofline basis leaves out:
    score  : counts K*4 + block table ceil(N/16)*4 + scores written (N-P)*4
    compact: keep lists read B*4
    evict  : the score extras + the keep list written B*4 (when the caller
             asks for it, as the benchmark does)."""
    K, B = wl.n_beacons, wl.budget
    sc = sum(hc_per_req * (K * 4 + -(-n // 16) * 4 + (n - p) * 4) for n, p in zip(N, P))
    keep_lists = len(N) * hc_per_req * B * 4
    return {"beacon_update": 0, "beacon_score": sc, "topk_select": 0, "kv_compact": keep_lists,
            "beacon_evict": sc + keep_lists}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, budget_s):
    """The oracle, as it stands, on one layer of the same workload (CPU-drawn
    synthetic data of the same shapes), scaled to a full pass."""
    import numpy as np

    import oracle
    from decode_kv_cache_beacon_amd import synth

    swl = wl.with_(n_layers=min(2, wl.n_layers))
    t0 = time.time()
    batch = synth.make_batch(swl, "cpu")
    kb = [synth.bits(k) for k in batch.k_pools]
    vb = [synth.bits(v) for v in batch.v_pools]
    bt = batch.block_table.numpy()
    N = batch.seq_len.numpy()
    P = batch.prompt_len.numpy()
    R, H, L = swl.n_requests, swl.n_kv_heads, swl.n_layers
    q = synth.bits(batch.queries)
    b = batch.beacons.numpy()
    c = batch.counts.numpy()
    log(f"cpu baseline: sample generated in {time.time() - t0:.1f}s")
    # the sample's head-caches are swept again (beacon state carried over)
    # until the time budget is spent
    done, elapsed, chunk, sweeps = 0, 0.0, 32, 0
    hc_total = L * R * H
    while elapsed < budget_s:
        start = done % hc_total
        sweeps = max(sweeps, done // hc_total + 1)
        sl = slice(start, min(start + chunk, hc_total))
        hcs = range(sl.start, sl.stop)     # hc = (layer * R + r) * H + h
        keys = np.stack([oracle.gather_paged(kb[hc // (R * H)], bt[(hc // H) % R], hc % H,
                                             wl.seq_len) for hc in hcs])
        vals = np.stack([oracle.gather_paged(vb[hc // (R * H)], bt[(hc // H) % R], hc % H,
                                             wl.seq_len) for hc in hcs])
        Nh = np.array([N[(hc // H) % R] for hc in hcs], np.int32)
        Ph = np.array([P[(hc // H) % R] for hc in hcs], np.int32)
        t1 = time.perf_counter()
        nb, nc, _, _, _ = oracle.evict_batch(q[sl], b[sl], c[sl], keys, vals, Nh, Ph, wl.budget,
                                             wl.window, wl.bonus)
        elapsed += time.perf_counter() - t1
        b[sl], c[sl] = nb, nc
        done += sl.stop - sl.start
    per_hc = elapsed / done
    pass_s = per_hc * wl.n_head_caches
    return {
        "value": 1.0 / pass_s,
        "unit": "passes/s",
        "cores": oracle.num_threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"{done} head-cache eviction passes: the {min(done, hc_total)} head-caches "
                   f"of layers 0-{L - 1} (CPU-drawn data of the same shapes) swept {sweeps} "
                   f"time(s), {elapsed:.1f} s of oracle time, scaled linearly to the "
                   f"{wl.n_head_caches} head-caches of a pass ({pass_s:.1f} s/pass)"),
    }


DEFAULT_WORKLOAD = "serving_r128"


def traffic_file(workload, out=None):
    """Per-kernel counter bytes of a workload: profiles/traffic.json for the
    default workload, profiles/<workload>_traffic.json for the others."""
    name = "traffic.json" if workload == DEFAULT_WORKLOAD else f"{workload}_traffic.json"
    return os.path.join(out or os.path.join(ROOT, "profiles"), name)


def stored_counters(kernel, workload):
    """Per-launch figures from committed rocprofv3 counter runs (HBM bytes,
    bf16 MFMA flop, instruction-issue shares), if they were taken on the
    current kernel source and on this workload (else {})."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        t = json.load(f)
    if t.get("_workload", t.get("_calibration", {}).get("workload")) != workload:
        return {}
    e = t.get(kernel)
    if not e or e.get("source_sha") != kernel_source_hash(kernel):
        return {}
    return e


def stored_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter runs, or None."""
    return stored_counters(kernel, workload).get("bytes_per_launch")


# kernel symbol fragment -> kernel id
KERNEL_SYMBOLS = {
    "beacon_update_kernel": "beacon_update",
    "beacon_evict_shared_kernel": "beacon_evict_shared",
    "beacon_evict_kernel": "beacon_evict",
    "beacon_score_kernel": "beacon_score",
    "topk_select_kernel": "topk_select",
    "kv_compact_kernel": "kv_compact",
    "random_score_kernel": "random_score",
    "random_evict_kernel": "random_evict",
    "page_retain_kernel": "page_retain",
    "decode_attention_kernel": "decode_attention",
}
COPY_SYMBOL = "__amd_rocclr_copyBuffer"
PROFILE_CMDS = {
    "trace": ("cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats -f csv -d <prof-dir> "
              "-o bench -- python3 <repo>/bench.py --steps 5 --warmup 1 --no-cpu-baseline "
              "--no-side --count-cap 0 > <trace-run-log>"),
    "pmc": ("cd /tmp && TMPDIR=/tmp rocprofv3 --pmc {c} -f csv -d <pmc-dir>/{c} -o {c} -- "
            "python3 <repo>/bench.py --steps 2 --warmup 0 --no-cpu-baseline "
            "--no-shared --no-pages --no-side --count-cap 0"),
    "pmc_mfma": ("cd /tmp && TMPDIR=/tmp rocprofv3 --pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16 "
                 "-f csv -d <pmc-dir>/MFMA -o MFMA -- python3 <repo>/bench.py --steps 2 "
                 "--warmup 0 --no-cpu-baseline --no-shared --no-pages --no-side "
                 "--count-cap 0"),
    "summary": "python bench.py --summarize-profiles <prof-dir> <pmc-dir> <trace-run-log>",
}
# instruction-issue counters, two runs (at most 8 SQ counters per run)
SQ_COUNTERS = {
    "SQ1": ("SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_SALU",
            "SQ_INSTS_LDS", "SQ_ACTIVE_INST_VALU", "SQ_WAIT_INST_ANY"),
    "SQ2": ("SQ_INSTS_VMEM", "SQ_INSTS_SMEM", "SQ_INST_CYCLES_VMEM", "SQ_ACTIVE_INST_LDS",
            "SQ_ACTIVE_INST_SCA", "SQ_WAIT_ANY", "SQ_INSTS_BRANCH", "SQ_ACTIVE_INST_ANY"),
}
for _run, _cs in SQ_COUNTERS.items():
    PROFILE_CMDS["pmc_" + _run.lower()] = (
        f"cd /tmp && TMPDIR=/tmp rocprofv3 --pmc {' '.join(_cs)} -f csv -d <pmc-dir>/{_run} "
        f"-o {_run} -- python3 <repo>/bench.py --steps 2 --warmup 0 --no-cpu-baseline "
        "--no-shared --no-pages --no-side --no-random --no-separate --count-cap 0")


def summarize_hbm(paths, workload, out, kid):
    """profiles/<workload>_hbm_counters.md and the workload's traffic file from
    the FETCH_SIZE and WRITE_SIZE runs, scaled by the 4 GiB copy's readings."""
    import csv
    import statistics

    counters = {}
    for c, found in paths.items():
        path = found[0]
        per = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != c:
                continue
            name = r["Kernel_Name"]
            k = "copy" if COPY_SYMBOL in name else kid(name)
            if k:
                per.setdefault(k, []).append(float(r["Counter_Value"]))
        counters[c] = per
    # the 4 GiB device copy: the largest copyBuffer dispatches
    copy_bytes = 1 << 32
    big = max(counters["WRITE_SIZE"]["copy"])
    n_big = sum(1 for v in counters["WRITE_SIZE"]["copy"] if v >= 0.99 * big)
    fetch_copy = sorted(counters["FETCH_SIZE"]["copy"])[-n_big:]
    write_copy = sorted(counters["WRITE_SIZE"]["copy"])[-n_big:]
    f_read = copy_bytes / (statistics.mean(fetch_copy) * 1024)
    f_write = copy_bytes / (statistics.mean(write_copy) * 1024)
    traffic = {"_workload": workload, "_calibration": {
        "copy_bytes_read": copy_bytes, "copy_bytes_written": copy_bytes,
        "copy_fetch_kib": statistics.mean(fetch_copy), "copy_write_kib": statistics.mean(write_copy),
        "read_factor": f_read, "write_factor": f_write, "workload": workload,
        "commands": [profile_cmd("pmc", workload, c="FETCH_SIZE"),
                     profile_cmd("pmc", workload, c="WRITE_SIZE"), profile_cmd("summary", workload)]}}
    lines = [f"# HBM traffic per launch, workload {workload}", "",
             "FETCH_SIZE and WRITE_SIZE (KiB per dispatch, mean over each kernel's dispatches in the "
             "profiled passes) from two rocprofv3 counter runs, each scaled by what the same counter reads "
             f"for a plain 4 GiB device copy: read factor {f_read:.4f}, write factor "
             f"{f_write:.4f}.", "", "Commands:", "",
             "    " + profile_cmd("pmc", workload, c="FETCH_SIZE"),
             "    " + profile_cmd("pmc", workload, c="WRITE_SIZE"),
             "    " + profile_cmd("summary", workload), "",
             "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | read GB | written GB | total GB | "
             "source hash |", "|---|---|---|---|---|---|---|"]
    for k in KERNEL_SOURCES:
        if k not in counters["FETCH_SIZE"] or k not in counters["WRITE_SIZE"]:
            continue
        fk = statistics.mean(counters["FETCH_SIZE"][k])
        wk = statistics.mean(counters["WRITE_SIZE"][k])
        rb, wb = fk * 1024 * f_read, wk * 1024 * f_write
        sha = kernel_source_hash(k)
        traffic[k] = {"fetch_kib": fk, "write_kib": wk, "bytes_read": rb, "bytes_written": wb,
                      "bytes_per_launch": rb + wb, "source_sha": sha}
        lines.append(f"| {k} | {fk:.0f} | {wk:.0f} | {rb / 1e9:.2f} | {wb / 1e9:.2f} | "
                     f"{(rb + wb) / 1e9:.2f} | {sha} |")
    with open(os.path.join(out, f"{workload}_hbm_counters.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    return traffic


def profile_cmd(key, workload, **fmt):
    """The command that made a profile summary, for this workload."""
    cmd = PROFILE_CMDS[key].format(**fmt) if fmt else PROFILE_CMDS[key]
    if workload != DEFAULT_WORKLOAD:
        cmd = cmd.replace("bench.py --", f"bench.py --workload {workload} --")
    return cmd


def summarize_profiles(prof_dir, pmc_dir, workload, out=None, bench_log=None):
    """Write the committed summaries from rocprofv3 output: per-kernel
    durations (kernel trace), HBM bytes per launch from FETCH_SIZE and
    WRITE_SIZE, each scaled by what the counter reads for the 4 GiB device
    copy the benchmark also runs, and the workload's traffic file for the
    roofline; the counter runs are optional."""
    import csv
    import glob
    import statistics

    def kid(name):
        return next((v for k, v in KERNEL_SYMBOLS.items() if k in name), None)

    rows = list(csv.DictReader(open(glob.glob(os.path.join(prof_dir, "*kernel_trace.csv"))[0])))
    dur = {}
    for r in rows:
        k = kid(r["Kernel_Name"])
        if k:
            dur.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6)
    out = out or os.path.join(ROOT, "profiles")
    os.makedirs(out, exist_ok=True)
    lines = [f"# Kernel durations, workload {workload}", "",
             "rocprofv3 kernel trace of one benchmark run: 5 timed + 1 warm-up beacon passes "
             "(maintenance, then the fused score-select-compact kernel), as many with scoring, "
             "selection and compaction as separate kernels, as many random-selector passes "
             "(fused draw-select-compact kernel) and as many again with separate kernels, "
             "shared-position passes (beacon fused, beacon with separate kernels, random), then "
             "as many page-retention passes of each selector (maintenance and scoring also run "
             "in the page-retention beacon passes).", "",
             "Command:", "", "    " + profile_cmd("trace", workload), "",
             "| kernel | launches | mean ms | min ms | max ms |", "|---|---|---|---|---|"]
    for k in KERNEL_SOURCES:
        if k in dur:
            d = dur[k]
            lines.append(f"| {k} | {len(d)} | {statistics.mean(d):.3f} | {min(d):.3f} | "
                         f"{max(d):.3f} |")
    # the roofline fraction of the profiled run, recomputed from the trace: the
    # dominant kernel's algorithmic bytes per launch (the run's own line, whose
    # moved-row count is that run's) over the trace's mean duration
    line = None
    if bench_log and os.path.exists(bench_log):
        for raw in open(bench_log):
            raw = raw.strip()
            if raw.startswith("{") and '"roofline"' in raw:
                line = json.loads(raw)
    if line and line["roofline"].get("kernel") in dur:
        rf = line["roofline"]
        k = rf["kernel"]
        tmean = statistics.mean(dur[k])
        tfrac = rf["bytes_per_launch"] / (tmean * 1e-3) / 1e9 / HBM_PEAK_GBPS
        what = {"beacon_update": "queries read once, beacons and counts read and written",
                "beacon_evict": (f"keys read once, beacons, {rf.get('moved_rows_per_launch', 0):,} "
                                 "moved rows read and written: the run's own moved-row count")}
        lines += ["", "Roofline of the profiled run, from this trace:", "",
                  f"- dominant kernel `{k}`: {rf['bytes_per_launch']:,} algorithmic bytes per launch "
                  f"({what.get(k, 'its own inputs and outputs, each moved once')})",
                  f"- trace mean {tmean:.4f} ms -> {rf['bytes_per_launch'] / (tmean * 1e-3) / 1e9:.1f} "
                  f"GB/s = {tfrac:.4f} of the {HBM_PEAK_GBPS:.0f} GB/s peak",
                  f"- the run's own line (HIP events around its timed passes): "
                  f"{rf['ms_per_launch']:.4f} ms, frac {rf['frac']:.4f}"]
    with open(os.path.join(out, f"{workload}_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    # HBM bytes (optional: both counter runs)
    hbm = {c: glob.glob(os.path.join(pmc_dir, c, "*counter_collection.csv"))
           for c in ("FETCH_SIZE", "WRITE_SIZE")}
    counters = {"_workload": workload}
    if all(hbm.values()):
        counters = summarize_hbm(hbm, workload, out, kid)

    def entry(k):
        return counters.setdefault(k, {"source_sha": kernel_source_hash(k)})

    # MFMA utilisation (optional third counter run)
    mfma = glob.glob(os.path.join(pmc_dir, "MFMA", "*counter_collection.csv"))
    if mfma:
        per = {}
        for r in csv.DictReader(open(mfma[0])):
            k = kid(r["Kernel_Name"])
            if not k:
                continue
            d = per.setdefault(k, {}).setdefault(r["Counter_Name"], {})
            key = r.get("Dispatch_Id") or r.get("Correlation_Id") or len(d)
            d[key] = d.get(key, 0.0) + float(r["Counter_Value"])
        lines = [f"# MFMA utilisation per launch, workload {workload}", "",
                 "rocprofv3's derived MfmaUtil (MFMA-busy cycles summed over SIMDs, over "
                 "GPU-active cycles times the SIMD count, in percent) and the bf16 MFMA "
                 "operations (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 = flop), mean over the "
                 "dispatches in the profiled passes; TFLOP/s uses the kernel-trace mean duration. "
                 f"Dense bf16 peak {MFMA_BF16_PEAK_TFLOPS:.0f} TFLOP/s.", "", "Command:", "",
                 "    " + profile_cmd("pmc_mfma", workload), "",
                 "| kernel | MfmaUtil % | bf16 MFMA flop per launch | TFLOP/s | % of peak |",
                 "|---|---|---|---|---|"]
        for k in KERNEL_SOURCES:
            if k not in per:
                continue
            util = per[k].get("MfmaUtil", {})
            mops = per[k].get("SQ_INSTS_VALU_MFMA_MOPS_BF16", {})
            u = statistics.mean(util.values()) if util else float("nan")
            flop = statistics.mean(mops.values()) * 512 if mops else float("nan")
            tf = flop / (statistics.mean(dur[k]) * 1e-3) / 1e12 if k in dur and mops else float("nan")
            lines.append(f"| {k} | {u:.1f} | {flop:.3e} | {tf:.1f} | "
                         f"{100 * tf / MFMA_BF16_PEAK_TFLOPS:.1f} |")
            if mops:
                entry(k).update({"mfma_flop_per_launch": flop, "mfma_util_pct": u})
        with open(os.path.join(out, f"{workload}_mfma_counters.md"), "w") as f:
            f.write("\n".join(lines) + "\n")
    # instruction issue (optional fourth and fifth counter runs)
    sq = {}
    for run in SQ_COUNTERS:
        for path in glob.glob(os.path.join(pmc_dir, run, "*counter_collection.csv")):
            for r in csv.DictReader(open(path)):
                k = kid(r["Kernel_Name"])
                if k:
                    d = sq.setdefault(k, {}).setdefault(r["Counter_Name"], {})
                    key = r.get("Dispatch_Id") or r.get("Correlation_Id") or len(d)
                    d[key] = d.get(key, 0.0) + float(r["Counter_Value"])
    if sq:
        def m(k, c):
            v = sq[k].get(c)
            return statistics.mean(v.values()) if v else float("nan")
        lines = [f"# Instruction issue per launch, workload {workload}", "",
                 "rocprofv3 SQ counters, mean over the dispatches in the profiled passes (the "
                 "per-head beacon pass, maintenance then the fused kernel, and the decode attention "
                 "the benchmark runs after it). Instructions "
                 "are per wave. The shares divide each wave's cycles executing any instruction, "
                 "VALU or scalar instructions, and waiting, by its lifetime (SQ_WAVE_CYCLES; the "
                 "same units). With w waves resident per SIMD, a SIMD's issue is busy about w "
                 "times the per-wave share.", "", "Commands:", "",
                 *["    " + profile_cmd("pmc_" + run.lower(), workload) for run in SQ_COUNTERS],
                 "    " + profile_cmd("summary", workload), "",
                 "| kernel | waves | VALU | SALU | LDS | VMEM | branch | any-issue share | "
                 "VALU share | scalar share | wait share |",
                 "|---|---|---|---|---|---|---|---|---|---|---|"]
        for k in KERNEL_SOURCES:
            if k not in sq:
                continue
            w = m(k, "SQ_WAVES")
            life = m(k, "SQ_WAVE_CYCLES")
            lines.append(
                f"| {k} | {w:.0f} | {m(k, 'SQ_INSTS_VALU') / w:.0f} | "
                f"{m(k, 'SQ_INSTS_SALU') / w:.0f} | {m(k, 'SQ_INSTS_LDS') / w:.0f} | "
                f"{m(k, 'SQ_INSTS_VMEM') / w:.0f} | {m(k, 'SQ_INSTS_BRANCH') / w:.0f} | "
                f"{m(k, 'SQ_ACTIVE_INST_ANY') / life:.2f} | "
                f"{m(k, 'SQ_ACTIVE_INST_VALU') / life:.2f} | "
                f"{m(k, 'SQ_ACTIVE_INST_SCA') / life:.2f} | {m(k, 'SQ_WAIT_ANY') / life:.2f} |")
            entry(k).update({"issue_share": m(k, "SQ_ACTIVE_INST_ANY") / life,
                             "valu_share": m(k, "SQ_ACTIVE_INST_VALU") / life,
                             "wait_share": m(k, "SQ_WAIT_ANY") / life,
                             "valu_insts_per_wave": m(k, "SQ_INSTS_VALU") / w})
        with open(os.path.join(out, f"{workload}_issue_counters.md"), "w") as f:
            f.write("\n".join(lines) + "\n")
    if len(counters) > 1:
        with open(traffic_file(workload, out), "w") as f:
            json.dump(counters, f, indent=1)
    print(f"wrote the {workload} summaries in {out}")


def side_pass(torch, bk, synth, wl, steps, warmup, dev, selector="beacon"):
    """Mean per-kernel milliseconds of `steps` whole passes over a freshly
    generated workload (no refill between passes: the lengths stay, so every
    pass scores and selects the same number of slots), and the mean number of
    rows the compaction moved."""
    batch = synth.make_batch(wl, dev)
    cache = bk.PagedCache(batch.k_pools, batch.v_pools, batch.block_table, batch.seq_len,
                          batch.prompt_len)
    HC, R, B = cache.n_head_caches, cache.n_requests, wl.budget
    N = batch.seq_len.cpu().tolist()
    P = batch.prompt_len.cpu().tolist()
    stride = max(n - p for n, p in zip(N, P))
    beacon = selector == "beacon"
    scores = torch.zeros((HC, stride), dtype=torch.float32 if beacon else torch.int32,
                         device=dev)
    keep = torch.zeros((HC, B), dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    rid = torch.arange(R, dtype=torch.int64, device=dev)
    pss = torch.zeros(R, dtype=torch.int32, device=dev)
    ar = torch.arange(B, device=dev, dtype=torch.int32)
    nk = torch.tensor([min(N[(hc // cache.n_kv_heads) % R], B) for hc in range(HC)],
                      device=dev)
    runs, moved = [], []
    n_ev = 5 if beacon else 4
    for s in range(warmup + steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
        if beacon:
            bk.bkv_evict_pass(cache, bk.BKV_SELECT_BEACON, B, queries=batch.queries,
                              beacons=batch.beacons, counts=batch.counts, window=wl.window,
                              bonus=wl.bonus, scores_out=scores, keep_out=keep,
                              score_stride=stride, status=status, check=False, timing_events=ev)
        else:
            pss.fill_(s)
            bk.bkv_evict_pass(cache, bk.BKV_SELECT_RANDOM, B, seed=wl.seed, request_ids=rid,
                              pass_idx=pss, scores_out=scores, keep_out=keep,
                              score_stride=stride, status=status, check=False, timing_events=ev)
        if s >= warmup:
            runs.append(ev)
            neq = keep != ar
            first = torch.where(neq.any(1), neq.int().argmax(1), torch.full_like(nk, B))
            moved.append((nk - first).clamp(min=0).sum())
    torch.cuda.synchronize()
    bk.check_status(status, f"{wl.name} side passes")

    def span(i, j):
        return sum(e[i].elapsed_time(e[j]) for e in runs) / len(runs)

    fused = stride + B <= bk.FUSED_MAX_ENTRIES
    if beacon and fused:
        kms = {"beacon_update": span(0, 1), "beacon_evict": span(1, 4)}
    elif beacon:
        kms = {n: span(i, i + 1) for i, n in
               enumerate(["beacon_update", "beacon_score", "topk_select", "kv_compact"])}
    elif fused:
        kms = {"random_evict": span(0, 3)}
    else:
        kms = {n: span(i, i + 1) for i, n in
               enumerate(["random_score", "topk_select", "kv_compact"])}
    ms = span(0, n_ev - 1)
    M = float(sum(int(m) for m in moved)) / len(moved)
    del batch, cache, scores, keep
    torch.cuda.empty_cache()
    return ms, kms, N, P, M


def side_line(wl, ms, kms, N, P, M, selector):
    """A side workload's pass rate and, for the fused kernel, its algorithmic
    GB/s against the HBM peak."""
    e = {"ms_per_pass": round(ms, 4), "passes_per_s": round(1000.0 / ms, 3),
         "kernel_ms": {k: round(v, 4) for k, v in kms.items()}, "moved_rows_per_pass": int(M)}
    hc_per_req = wl.n_layers * wl.n_kv_heads
    if selector == "beacon" and "beacon_evict" in kms:
        nbytes = algorithmic_bytes(wl, N, P, M, hc_per_req)["beacon_evict"]
        gbps = nbytes / (kms["beacon_evict"] * 1e-3) / 1e9
        e.update({"fused_algorithmic_bytes": int(nbytes), "fused_gbps": round(gbps, 1),
                  "fused_hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)})
    elif selector == "random" and "random_evict" in kms:
        # the random pass reads no key and no beacon: only the moved rows count
        nbytes = 4 * M * 256
        gbps = nbytes / (kms["random_evict"] * 1e-3) / 1e9
        e.update({"fused_algorithmic_bytes": int(nbytes), "fused_gbps": round(gbps, 1),
                  "fused_hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
                  "fused_extra_bytes": int(hc_per_req * sum((n - p) * 4 + wl.budget * 4
                                                            for n, p in zip(N, P)))})
    return e


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-random", action="store_true", help="skip the random-selector A/B")
    ap.add_argument("--no-side", action="store_true",
                    help="skip the one-shot side workloads (single head, 32k slots)")
    ap.add_argument("--no-pages", action="store_true",
                    help="skip the page-retention (whole pages, no row moves) passes")
    ap.add_argument("--no-separate", action="store_true",
                    help="skip the passes with score, select and compact as separate kernels")
    ap.add_argument("--no-shared", action="store_true",
                    help="skip the shared-position (one selection per layer and request) passes")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--count-cap", type=int, default=16,
                    help="also time the maintenance kernel with this count cap (0: skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 4 GiB device copy (for counter calibration)")
    ap.add_argument("--summarize-profiles", nargs="+", metavar="DIR",
                    help="PROF_DIR PMC_DIR [TRACE_RUN_LOG]: write profiles/ summaries from "
                         "rocprofv3 output (and the traced run's bench line) and exit")
    args = ap.parse_args()
    if args.summarize_profiles:
        sp = args.summarize_profiles
        if len(sp) not in (2, 3):
            ap.error("--summarize-profiles takes PROF_DIR PMC_DIR [TRACE_RUN_LOG]")
        summarize_profiles(sp[0], sp[1], args.workload, bench_log=sp[2] if len(sp) == 3 else None)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the eviction pass has no cross-GPU work "
              "(every head-cache is independent); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from decode_kv_cache_beacon_amd import beaconkv as bk
    from decode_kv_cache_beacon_amd import synth

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    dev = torch.device("cuda:0")
    wl = synth.WORKLOADS[args.workload]
    B, W = wl.budget, wl.window
    assert wl.seq_len == B + W and B % synth.BLOCK == 0 and W % synth.BLOCK == 0, \
        "steady-state bench needs N = B + W with block-aligned B and W"

    t0 = time.time()
    batch = synth.make_batch(wl, dev)
    torch.cuda.synchronize()
    log(f"workload {wl.name}: generated on the GPU in {time.time() - t0:.1f}s")
    cache = bk.PagedCache(batch.k_pools, batch.v_pools, batch.block_table, batch.seq_len,
                          batch.prompt_len)
    HC, R, H = cache.n_head_caches, cache.n_requests, cache.n_kv_heads
    N = batch.seq_len.cpu().tolist()
    P = batch.prompt_len.cpu().tolist()
    stride = max(n - p for n, p in zip(N, P))
    q, b, c = batch.queries, batch.beacons, batch.counts
    scores = torch.zeros((HC, stride), dtype=torch.float32, device=dev)
    keep = torch.zeros((HC, B), dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    # fresh rows for the W slots appended between passes (pool layout)
    tail_blocks = batch.block_table[:, B // synth.BLOCK:(B + W) // synth.BLOCK].long()
    nb_tail = W // synth.BLOCK
    fresh = []
    for layer in range(wl.n_layers):
        fk, fv = synth.fresh_tail(wl, layer, 0, dev)          # [R, H, W, d]
        shp = (R, H, nb_tail, synth.BLOCK, wl.head_dim)
        fresh.append((fk.reshape(shp).permute(0, 2, 1, 3, 4).contiguous(),
                      fv.reshape(shp).permute(0, 2, 1, 3, 4).contiguous()))

    def refill():
        for layer, (fk, fv) in enumerate(fresh):
            cache.k_pools[layer][tail_blocks] = fk
            cache.v_pools[layer][tail_blocks] = fv

    # Every section that compares the fused kernels with the separate ones
    # starts from this same state (pools, beacons, counts), so both sides run
    # the same sequence of passes and move the same rows (their outputs are
    # bit-identical, so the state evolves identically).
    state0 = ([k.clone() for k in cache.k_pools], [v.clone() for v in cache.v_pools],
              batch.beacons.clone(), batch.counts.clone())

    def restore_state():
        for dst, src in zip(cache.k_pools + cache.v_pools, state0[0] + state0[1]):
            dst.copy_(src)
        batch.beacons.copy_(state0[2])
        batch.counts.copy_(state0[3])

    ar = torch.arange(B, device=dev, dtype=torch.int32)

    def moved_rows(kp=None, heads=1):
        """Rows the compaction moved: from the first changed slot on, per keep row."""
        kp = keep if kp is None else kp
        neq = kp != ar
        first = torch.where(neq.any(1), neq.int().argmax(1), torch.full_like(neq[:, 0], B,
                                                                            dtype=torch.long))
        nk = min(N[0], B)
        return (nk - first).clamp(min=0).sum() * heads

    # the pass runs maintenance, then the fused score+select+compact kernel;
    # its events after score, select and compact all follow the fused kernel
    names = ["beacon_update", "beacon_evict"]
    sep_names = ["beacon_score", "topk_select", "kv_compact"]

    def run_pass(events=None, separate=False):
        bk.bkv_evict_pass(cache, bk.BKV_SELECT_BEACON, B, queries=q, beacons=b, counts=c,
                          window=W, bonus=wl.bonus, scores_out=scores, keep_out=keep,
                          score_stride=stride, status=status, check=False,
                          timing_events=events, separate_steps=separate)

    for _ in range(args.warmup):
        refill()
        run_pass()
    torch.cuda.synchronize()
    bk.check_status(status, "warmup passes")

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    moved = []
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for s in range(args.steps):
        refill()
        run_pass(evs[s])
        moved.append(moved_rows())
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    bk.check_status(status, "timed passes")

    pass_ms = [e[0].elapsed_time(e[4]) for e in evs]
    ms = sum(pass_ms) / len(pass_ms)
    kms = {"beacon_update": sum(e[0].elapsed_time(e[1]) for e in evs) / len(evs),
           "beacon_evict": sum(e[1].elapsed_time(e[4]) for e in evs) / len(evs)}
    M = float(sum(int(m) for m in moved)) / len(moved)
    hc_per_req = wl.n_layers * H
    abytes = algorithmic_bytes(wl, N, P, M, hc_per_req)
    total_bytes = abytes["beacon_update"] + abytes["beacon_evict"]
    ssc_bytes = abytes["beacon_evict"]
    ssc_ms = kms["beacon_evict"]
    # logits of every key (phase 1) and of every candidate (phase 2)
    score_flops = 2.0 * wl.n_beacons * 128 * hc_per_req * sum(n + (n - p) for n, p in zip(N, P))
    update_flops = 2.0 * wl.steps * wl.group * wl.n_beacons * 128 * HC

    xbytes = extra_bytes(wl, N, P, hc_per_req)

    def kernel_entry(n, ms_, nbytes):
        gbps = nbytes / (ms_ * 1e-3) / 1e9
        e = {"ms": round(ms_, 4), "algorithmic_bytes": int(nbytes), "gbps": round(gbps, 1),
             "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}
        if xbytes.get(n):
            e["extra_bytes"] = int(xbytes[n])
        sc_ = stored_counters(n, wl.name)
        if sc_.get("bytes_per_launch"):
            e["traffic_gbps"] = round(sc_["bytes_per_launch"] / (ms_ * 1e-3) / 1e9, 1)
        if sc_.get("mfma_flop_per_launch"):
            tf = sc_["mfma_flop_per_launch"] / (ms_ * 1e-3) / 1e12
            e["mfma_tflops"] = round(tf, 1)
            e["mfma_frac"] = round(tf / MFMA_BF16_PEAK_TFLOPS, 4)
        if sc_.get("issue_share") is not None:
            e["issue_share_per_wave"] = round(sc_["issue_share"], 3)
        return e

    kernels = {n: kernel_entry(n, kms[n], abytes[n]) for n in names}
    # the cosine dots the maintenance chain needs (its MFMA split forms each
    # product exactly, so it executes more MFMA flop than this; see mfma_tflops)
    kernels["beacon_update"]["cosine_dot_flop"] = int(update_flops)

    # the dominant (slowest) kernel against the HBM peak, on the roofline
    # basis bytes of one launch (the fused kernel: keys once, beacons, moved rows)
    dom = max(names, key=lambda n: kms[n])
    ach = abytes[dom] / (kms[dom] * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": stored_traffic(dom, wl.name),
            "kernel": dom, "bytes_per_launch": int(abytes[dom]), "ms_per_launch": round(kms[dom], 4),
            "moved_rows_per_launch": int(M)}

    # the same pass with score, select and compact as three kernels: the
    # per-step breakdown (and what the fused kernel saves)
    separate = None
    if not args.no_separate:
        restore_state()
        sruns, smoved = [], []
        for s in range(args.warmup + args.steps):
            refill()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
            run_pass(ev, separate=True)
            if s >= args.warmup:
                sruns.append(ev)
                smoved.append(moved_rows())
        torch.cuda.synchronize()
        bk.check_status(status, "separate-step passes")
        sms = sum(e[0].elapsed_time(e[4]) for e in sruns) / len(sruns)
        skms = {n: sum(e[i + 1].elapsed_time(e[i + 2]) for e in sruns) / len(sruns)
                for i, n in enumerate(sep_names)}
        sab = algorithmic_bytes(wl, N, P, float(sum(int(m) for m in smoved)) / len(smoved),
                                hc_per_req)
        sk = {n: kernel_entry(n, skms[n], sab[n]) for n in sep_names}
        stf = score_flops / (skms["beacon_score"] * 1e-3) / 1e12
        sk["beacon_score"]["mfma_tflops"] = round(stf, 1)
        sk["beacon_score"]["mfma_frac"] = round(stf / MFMA_BF16_PEAK_TFLOPS, 4)
        separate = {
            "passes_per_s": round(1000.0 / sms, 3), "ms": round(sms, 4),
            "same_moved_rows_as_fused": [int(m) for m in smoved] == [int(m) for m in moved],
            "update_ms": round(sum(e[0].elapsed_time(e[1]) for e in sruns) / len(sruns), 4),
            "score_select_compact_ms": round(sum(skms.values()), 4), "kernels": sk,
            "note": "the same pass with scoring, selection and compaction as three kernels"}

    result = {
        "metric": METRIC,
        "value": round(1000.0 / ms, 3),
        "unit": "passes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "layer_passes_per_s": round(1000.0 / ms * wl.n_layers, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian-mixture keys/queries, paged pools with permuted "
                "block tables; generated on the GPU before timing)",
        "config": {"workload": wl.name, "layers": wl.n_layers, "requests": R, "kv_heads": H,
                   "query_heads_per_kv": wl.group, "head_dim": wl.head_dim,
                   "beacons": wl.n_beacons, "budget": B, "prompt": P[0] if len(set(P)) == 1
                   else f"U{{{min(P)}..{max(P)}}}", "seq_len_at_pass": N[0],
                   "decode_steps_per_pass": wl.steps, "block_size": synth.BLOCK,
                   "paged": wl.paged, "head_caches": HC},
        "hbm_gbps": round(total_bytes / (ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(total_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "score_select_compact": {
            "passes_per_s": round(1000.0 / ssc_ms, 3), "ms": round(ssc_ms, 4),
            "gbps": round(ssc_bytes / (ssc_ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(ssc_bytes / (ssc_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
        "bytes_per_pass": int(total_bytes),
        "moved_rows_per_pass": int(M),
        "kernels": kernels,
        "wall_ms_per_step_incl_append": round(wall * 1e3 / args.steps, 3),
        "roofline": roof,
    }
    if separate:
        result["separate_steps"] = separate

    # the consumer of the pass: one decode step of attention over the compacted
    # cache (every layer, request and KV head; the length set to the kept count)
    cache.seq_len.clamp_(max=B)
    q_last = q[:, -1].contiguous()                      # [HC, G, 128] bf16
    att_out = torch.empty((HC, wl.group, wl.head_dim), dtype=torch.float32, device=dev)
    bk.bkv_decode_attention(cache, q_last, att_out, status=status, check=False)
    att_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    for e0, e1 in att_ev:
        e0.record()
        bk.bkv_decode_attention(cache, q_last, att_out, status=status, check=False)
        e1.record()
    torch.cuda.synchronize()
    bk.check_status(status, "decode attention")
    att_ms = sum(a.elapsed_time(b_) for a, b_ in att_ev) / len(att_ev)
    att_bytes = HC * (min(N[0], B) * 2 * wl.head_dim * 2 + wl.group * wl.head_dim * (2 + 4))
    result["decode_attention"] = {
        "ms": round(att_ms, 4), "algorithmic_bytes": int(att_bytes),
        "gbps": round(att_bytes / (att_ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(att_bytes / (att_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "note": f"one decode step, {wl.group} query heads per KV head over the {min(N[0], B)} "
                "kept slots of every head-cache, fp32 output"}
    cache.seq_len.copy_(torch.tensor(N, dtype=torch.int32, device=dev))

    if not args.no_random:
        rid = torch.arange(R, dtype=torch.int64, device=dev)
        pss = torch.zeros(R, dtype=torch.int32, device=dev)
        u = torch.zeros((HC, stride), dtype=torch.int32, device=dev)

        def random_passes(separate, salt):
            restore_state()
            runs, rmoved = [], []
            for s in range(args.warmup + args.steps):
                pss.fill_(s + salt)
                refill()
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
                bk.bkv_evict_pass(cache, bk.BKV_SELECT_RANDOM, B, seed=wl.seed, request_ids=rid,
                                  pass_idx=pss, scores_out=u, keep_out=keep, score_stride=stride,
                                  status=status, check=False, timing_events=ev,
                                  separate_steps=separate)
                if s >= args.warmup:
                    rmoved.append(moved_rows())
                    runs.append(ev)
            torch.cuda.synchronize()
            bk.check_status(status, "random passes")
            rpass = sum(e[0].elapsed_time(e[3]) for e in runs) / len(runs)
            rk = {n: round(sum(e[i].elapsed_time(e[i + 1]) for e in runs) / len(runs), 4)
                  for i, n in enumerate(["random_score", "topk_select", "kv_compact"])}
            rM = float(sum(int(m) for m in rmoved)) / len(rmoved)
            return rpass, rk, rM, [int(m) for m in rmoved]

        # the pass's default: draws, selection and compaction in one kernel
        rpass, _, rM, rlist = random_passes(False, 1000)
        rbytes = 4 * rM * 256            # no key or beacon reads: the moved rows only
        sp, sk, sM, slist = random_passes(True, 1000)
        result["random_selector"] = {
            "passes_per_s": round(1000.0 / rpass, 3), "ms": round(rpass, 4),
            "kernel_ms": {"random_evict": round(rpass, 4)},
            "moved_rows_per_pass": int(rM),
            "gbps": round(rbytes / (rpass * 1e-3) / 1e9, 1),
            "hbm_frac": round(rbytes / (rpass * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "separate_steps": {"passes_per_s": round(1000.0 / sp, 3), "ms": round(sp, 4),
                               "kernel_ms": sk, "moved_rows_per_pass": int(sM),
                               "same_moved_rows_as_fused": slist == rlist},
            "extra_bytes": int(HC * (stride * 4 + B * 4)),
            "note": "algorithmic bytes: the moved rows (K and V read and written); the draws "
                    "and keep lists written are the extra bytes"}

    # shared positions: one selection per (layer, request) for all its heads
    if not args.no_shared:
        LR = wl.n_layers * R
        keep_s = torch.zeros((LR, B), dtype=torch.int32, device=dev)
        rid = torch.arange(R, dtype=torch.int64, device=dev)
        pss = torch.zeros(R, dtype=torch.int32, device=dev)
        us = torch.zeros((LR, stride), dtype=torch.int32, device=dev)
        shared = {}
        for sel, sep in (("beacon", False), ("beacon", True), ("random", False)):
            n_ev = 5 if sel == "beacon" else 4
            restore_state()
            runs, smoved = [], []
            for s in range(args.warmup + args.steps):
                refill()
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
                if sel == "beacon":
                    bk.bkv_evict_pass(cache, bk.BKV_SELECT_BEACON, B, queries=q, beacons=b,
                                      counts=c, window=W, bonus=wl.bonus, scores_out=scores,
                                      keep_out=keep_s, score_stride=stride, status=status,
                                      check=False, timing_events=ev, shared_positions=True,
                                      separate_steps=sep)
                else:
                    pss.fill_(s + 2000)
                    bk.bkv_evict_pass(cache, bk.BKV_SELECT_RANDOM, B, seed=wl.seed,
                                      request_ids=rid, pass_idx=pss, scores_out=us,
                                      keep_out=keep_s, score_stride=stride, status=status,
                                      check=False, timing_events=ev, shared_positions=True)
                if s >= args.warmup:
                    smoved.append(moved_rows(keep_s, H))
                    runs.append(ev)
            torch.cuda.synchronize()
            bk.check_status(status, f"shared-position {sel} passes")

            def span(i, j):
                return round(sum(e[i].elapsed_time(e[j]) for e in runs) / len(runs), 4)

            if sel == "beacon" and not sep:  # maintenance, then the fused shared kernel
                kms_ = {"beacon_update": span(0, 1), "beacon_evict_shared": span(1, 4)}
            else:
                kn_ = (["beacon_update", "beacon_score"] if sel == "beacon" else
                       ["random_score"]) + ["topk_select", "kv_compact"]
                kms_ = {n: span(i, i + 1) for i, n in enumerate(kn_)}
            tpass = span(0, n_ev - 1)
            entry = {"passes_per_s": round(1000.0 / tpass, 3), "ms": tpass, "kernel_ms": kms_,
                     "moved_rows_per_pass": int(float(sum(int(m) for m in smoved)) / len(smoved))}
            if sep:
                entry["same_moved_rows_as_fused"] = smoved_list == [int(m) for m in smoved]
                shared["beacon"]["separate_steps"] = entry
            else:
                shared[sel] = entry
                if sel == "beacon":
                    smoved_list = [int(m) for m in smoved]
        shared["note"] = ("one keep list per (layer, request) for all KV heads: beacon scores "
                          "merged by their maximum over heads (one fused kernel: a workgroup "
                          "scores the heads of its (layer, request), selects once and compacts "
                          "every head), random draws one row")
        result["shared_positions"] = shared

    # page retention: whole pages per request, the block table rewritten in
    # place instead of moving rows; between passes (untimed) the released
    # blocks take the next 64 appended tokens, as an allocator would hand them out
    if not args.no_pages:
        Bp, npages = B // synth.BLOCK, (B + W) // synth.BLOCK
        bt0 = cache.block_table.clone()
        kp_pages = torch.zeros((R, Bp), dtype=torch.int32, device=dev)
        freed = torch.zeros((R, cache.max_blocks), dtype=torch.int32, device=dev)
        rid = torch.arange(R, dtype=torch.int64, device=dev)
        pss = torch.zeros(R, dtype=torch.int32, device=dev)
        ur = torch.zeros((R, stride), dtype=torch.int32, device=dev)
        seq0 = cache.seq_len.clone()

        def append_tail():
            tb = cache.block_table[:, Bp:npages].long()
            for layer, (fk, fv) in enumerate(fresh):
                cache.k_pools[layer][tb] = fk
                cache.v_pools[layer][tb] = fv

        pages = {}
        for sel in ("beacon", "random"):
            n_ev = 4 if sel == "beacon" else 3
            runs = []
            for s in range(args.warmup + args.steps):
                append_tail()
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
                outs = (cache.block_table, cache.seq_len, freed)
                if sel == "beacon":
                    bk.bkv_evict_pass(cache, bk.BKV_SELECT_BEACON, B, queries=q, beacons=b,
                                      counts=c, window=W, bonus=wl.bonus, scores_out=scores,
                                      keep_out=kp_pages, score_stride=stride, status=status,
                                      check=False, timing_events=ev, page_retention=outs)
                else:
                    pss.fill_(s + 3000)
                    bk.bkv_evict_pass(cache, bk.BKV_SELECT_RANDOM, B, seed=wl.seed,
                                      request_ids=rid, pass_idx=pss, scores_out=ur,
                                      keep_out=kp_pages, score_stride=stride, status=status,
                                      check=False, timing_events=ev, page_retention=outs)
                if s >= args.warmup:
                    runs.append(ev)
                # the released blocks become the tail pages again; the length returns to B + W
                cache.block_table[:, Bp:npages] = freed[:, :npages - Bp]
                cache.seq_len.copy_(seq0)
            torch.cuda.synchronize()
            bk.check_status(status, f"page-retention {sel} passes")
            kn_ = (["beacon_update", "beacon_score"] if sel == "beacon" else ["random_score"]) + \
                ["page_retain"]
            tpass = sum(e[0].elapsed_time(e[-1]) for e in runs) / len(runs)
            kms_ = {n: round(sum(e[i].elapsed_time(e[i + 1]) for e in runs) / len(runs), 4)
                    for i, n in enumerate(kn_)}
            rows_read = HC if sel == "beacon" else R
            pbytes = rows_read * stride * 4 + R * (2 * cache.max_blocks * 4 + Bp * 4 + 4)
            pages[sel] = {"passes_per_s": round(1000.0 / tpass, 3), "ms": round(tpass, 4),
                          "kernel_ms": kms_,
                          "page_retain_algorithmic_bytes": int(pbytes),
                          "page_retain_gbps": round(pbytes / (kms_["page_retain"] * 1e-3) / 1e9, 1)}
        pages["note"] = ("whole 16-slot pages kept once per request for every layer and head; "
                         "the block table is rewritten in place and no K/V row moves")
        cache.block_table.copy_(bt0)
        cache.seq_len.copy_(seq0)

        # per-head pages: every head-cache keeps its own pages in its own row of
        # a per-head page table (rewritten in place).  A head-cache's tiles of a
        # block are its own, so between passes (untimed) each one takes the
        # blocks it dropped back as its tail pages, with the keys they hold
        L_ = wl.n_layers
        hrow0 = bt0.repeat_interleave(H, 0).repeat(L_, 1).contiguous()
        hlen0 = seq0.repeat_interleave(H).repeat(L_).contiguous()
        hcache = bk.PagedCache(cache.k_pools, cache.v_pools, cache.block_table, cache.seq_len,
                               cache.prompt_len, head_block_table=hrow0.clone(),
                               head_seq_len=hlen0.clone())
        kp_h = torch.zeros((HC, Bp), dtype=torch.int32, device=dev)
        dropped = torch.zeros((HC, cache.max_blocks), dtype=torch.int32, device=dev)
        uh = torch.zeros((HC, stride), dtype=torch.int32, device=dev)
        per_head = {}
        for sel in ("beacon", "random"):
            n_ev = 4 if sel == "beacon" else 3
            runs = []
            for s in range(args.warmup + args.steps):
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
                outs = (hcache.head_block_table, hcache.head_seq_len, dropped)
                if sel == "beacon":
                    bk.bkv_evict_pass(hcache, bk.BKV_SELECT_BEACON, B, queries=q, beacons=b,
                                      counts=c, window=W, bonus=wl.bonus, scores_out=scores,
                                      keep_out=kp_h, score_stride=stride, status=status,
                                      check=False, timing_events=ev, page_retention=outs,
                                      page_heads=True)
                else:
                    pss.fill_(s + 5000)
                    bk.bkv_evict_pass(hcache, bk.BKV_SELECT_RANDOM, B, seed=wl.seed,
                                      request_ids=rid, pass_idx=pss, scores_out=uh,
                                      keep_out=kp_h, score_stride=stride, status=status,
                                      check=False, timing_events=ev, page_retention=outs,
                                      page_heads=True)
                if s >= args.warmup:
                    runs.append(ev)
                hcache.head_block_table[:, Bp:npages] = dropped[:, :npages - Bp]
                hcache.head_seq_len.copy_(hlen0)
            torch.cuda.synchronize()
            bk.check_status(status, f"per-head page-retention {sel} passes")
            kn_ = (["beacon_update", "beacon_score"] if sel == "beacon" else ["random_score"]) + \
                ["page_retain"]
            tpass = sum(e[0].elapsed_time(e[-1]) for e in runs) / len(runs)
            kms_ = {n: round(sum(e[i].elapsed_time(e[i + 1]) for e in runs) / len(runs), 4)
                    for i, n in enumerate(kn_)}
            pbytes = HC * (stride * 4 + 2 * cache.max_blocks * 4 + Bp * 4 + 4)
            per_head[sel] = {"passes_per_s": round(1000.0 / tpass, 3), "ms": round(tpass, 4),
                             "kernel_ms": kms_,
                             "page_retain_algorithmic_bytes": int(pbytes),
                             "page_retain_gbps": round(pbytes / (kms_["page_retain"] * 1e-3) / 1e9,
                                                       1)}
        per_head["note"] = ("whole 16-slot pages kept per head-cache from its own scores, each "
                            "head-cache's row of a per-head page table rewritten in place; no "
                            "K/V row moves")
        pages["per_head"] = per_head
        result["page_retention"] = pages
        del hcache, kp_h, dropped, uh

    # beacon forgetting: the maintenance kernel with a count cap (moving
    # average once a row is full), timed alone on the same queries and state
    if args.count_cap > 0:
        times = {}
        for cap in (0, args.count_cap):
            bb, cc = b.clone(), c.clone()
            bk.bkv_beacon_update(q, bb, cc, count_cap=cap)           # warm-up
            evs2 = []
            for _ in range(5):
                bb.copy_(b)
                cc.copy_(c)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                bk.bkv_beacon_update(q, bb, cc, count_cap=cap)
                e1.record()
                evs2.append((e0, e1))
            torch.cuda.synchronize()
            times[cap] = round(sum(x.elapsed_time(y) for x, y in evs2) / len(evs2), 4)
            del bb, cc
        result["beacon_forgetting"] = {
            "count_cap": args.count_cap, "update_ms": times[args.count_cap],
            "update_ms_uncapped": times[0],
            "note": "maintenance kernel alone, same queries and starting state, mean of 5"}

    # reference: a plain device-to-device copy of 4 GiB (read + write), timed the same way
    src = torch.empty(1 << 31, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 5 * 2 * src.numel() * 2 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    result["copy_reference_gbps"] = round(copy_gbps, 1)
    result["copy_ceiling_frac"] = round(result["hbm_gbps"] / copy_gbps, 4)
    for n in names:
        result["kernels"][n]["copy_frac"] = round(result["kernels"][n]["gbps"] / copy_gbps, 4)
    if separate:
        for n in sep_names:
            separate["kernels"][n]["copy_frac"] = round(separate["kernels"][n]["gbps"] / copy_gbps, 4)
    del src, dst

    # the other configurations' one-shot shapes, reported beside the line
    if not args.no_side:
        twl = synth.WORKLOADS["tiny"]
        tms, tk, _, _, _ = side_pass(torch, bk, synth, twl, 20, 3, dev)
        result["tiny_one_shot"] = {
            "us_per_pass": round(tms * 1e3, 1),
            "kernel_us": {k: round(v * 1e3, 1) for k, v in tk.items()},
            "note": "one head-cache, N = 4096 (512 prompt), K = 64, B = 1024, 256 queries: "
                    "latency-bound, one workgroup per kernel"}
        owl = synth.WORKLOADS["qwen3_32b_r32"].with_(n_layers=1, seq_len=32768)
        oms, ok, oN, oP, _ = side_pass(torch, bk, synth, owl, 5, 1, dev)
        ohc = owl.n_head_caches
        oflops = 2.0 * owl.n_beacons * owl.head_dim * ohc * (oN[0] + (oN[0] - oP[0]))
        otf = oflops / (ok["beacon_score"] * 1e-3) / 1e12
        result["one_shot_32k"] = {
            "ms_per_pass": round(oms, 4), "kernel_ms": {k: round(v, 4) for k, v in ok.items()},
            "score_mfma_tflops": round(otf, 1),
            "score_mfma_frac": round(otf / MFMA_BF16_PEAK_TFLOPS, 4),
            "note": f"one layer of the 64-layer shape: {ohc} head-caches, N = 32768 "
                    f"({oP[0]} prompt), K = {owl.n_beacons}, B = {owl.budget}, "
                    f"G = {owl.group}; scoring flops count both logit passes"}
        # the Qwen3-4B-like dense batch (36 layers, 16 requests, K = 64): one pass
        # streams every layer's keys in layer-major order (about 5 GB, far more
        # than the 256 MB memory-side cache), so each layer is read cold
        q4 = synth.WORKLOADS["qwen3_4b_r16"]
        result["qwen3_4b_r16"] = side_line(q4, *side_pass(torch, bk, synth, q4, 8, 2, dev),
                                           "beacon")
        result["qwen3_4b_r16"]["note"] = ("36 layers, 16 requests, 8 KV heads, G = 4, K = 64, "
                                          "B = 2048, P = 1024, N = 2112, dense: maintenance, "
                                          "then the fused kernel")
        # the 64-layer K = 256 batch at the three budgets, steady state N = B + 64
        c4 = {}
        for Bx in (1024, 2048, 4096):
            w4 = synth.WORKLOADS["qwen3_32b_r32"].with_(budget=Bx, seq_len=Bx + 64)
            c4[f"B{Bx}"] = side_line(w4, *side_pass(torch, bk, synth, w4, 8, 2, dev), "beacon")
        c4["note"] = ("64 layers, 32 requests, 8 KV heads, G = 8, K = 256, P = 512, "
                      "N = B + 64: maintenance, then the fused kernel")
        result["qwen3_32b_budgets"] = c4
        # the long-prompt serving variant, both selectors on the same shape
        lwl = synth.WORKLOADS["long_prompt_r128"]
        result["long_prompt"] = {
            sel: side_line(lwl, *side_pass(torch, bk, synth, lwl, 8, 2, dev, sel), sel)
            for sel in ("beacon", "random")}
        result["long_prompt"]["note"] = ("serving shape with prompts drawn from 256..1536, "
                                         "B = 3072, N = 3136")

    if args.copy_calibration:
        src = torch.empty(1 << 31, dtype=torch.int16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = {"read": src.numel() * 2, "written": dst.numel() * 2}
        del src, dst

    del batch
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
