"""Throughput of the fused gating + gated delta-rule decode update on one GPU.

A step is one call of the update over one batch: by default the bs=512
decode of Qwen3-Next-shaped heads (H_k=16, H_v=32, K=V=128, bf16
activations, fp32 state in a 4096-slot pool).  Every step uses the next of 8
disjoint 512-slot sets, so each step's 1 GiB of state is read from HBM rather
than from the 256 MB Infinity Cache.

Prints one JSON line: updates/s (one update = one (sequence, v-head, token)
step of a live sequence), the kernel's HBM roofline fraction from HIP events
on the launch stream, the counter-measured traffic when the kernel source
still matches the committed counter profile, and the CPU oracle timed on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from linear_attention_recurrent_gating_amd import workloads as W  # noqa: E402

METRIC = "state updates/sec (seq·head·token) + HBM GB/s as % of peak, bs=512 decode"
HBM_PEAK_GBS = 8000.0   # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
# MI355X fp32 vector peak: 256 CUs x 4 SIMDs x 16 lanes x 2 flops (FMA) x 2
# (packed fp32) x 2.4 GHz.  The kernels are built without packed fp32 forms,
# so their issue ceiling is half of it.
VALU_FP32_PEAK_TFLOPS = 157.3
CSRC = os.path.join(ROOT, "linear_attention_recurrent_gating_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


KERNEL_NAMES = {1: "gdn_fused_update", 2: "gdn_decode_rows", 3: "gdn_vk_decode",
                4: "gdn_chunk_fwd"}  # by kernel_family (single token for 2 and 3)
ROW_SPLIT_TOKEN_LOOP = "gdn_rows_tokens"  # family 2 over several tokens per sequence
VALUE_ROWS_TOKEN_LOOP = "gdn_vk_multi"    # family 3 over several tokens per sequence
# The sources each kernel is compiled from (the counter profiles are keyed to them).
_ROWS = ("gdn_rows.hip", "gdn_tile.h", "gdn_device.h", "gdn_internal.h")
KERNEL_SOURCES = {"gdn_chunk_fwd": ("gdn_chunk.hip", "gdn_device.h", "gdn_internal.h"),
                  "gdn_decode_rows": _ROWS, ROW_SPLIT_TOKEN_LOOP: _ROWS}
DEFAULT_SOURCES = ("gdn_kernels.hip", "gdn_tile.h", "gdn_device.h", "gdn_internal.h")


def kernel_name(info) -> str:
    if info.kernel_family == 2 and info.multi_token:
        return ROW_SPLIT_TOKEN_LOOP
    if info.kernel_family == 3 and info.multi_token:
        return VALUE_ROWS_TOKEN_LOOP
    return KERNEL_NAMES[info.kernel_family]


def kernel_source_hash(kernel: str = "gdn_decode_rows") -> str:
    """Hash of the sources a kernel is compiled from, with comments and runs of
    white space removed (so editing a comment does not orphan a profile)."""
    import re
    h = hashlib.sha256()
    for name in KERNEL_SOURCES.get(kernel, DEFAULT_SOURCES):
        with open(os.path.join(CSRC, name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def profile_path(kernel: str, workload: str, kind: str) -> str:
    return os.path.join(PROFILES, f"{kernel}__{workload}__{kind}.txt")


def counter_traffic(kernel: str, workload: str):
    """Counter-measured HBM bytes per launch from the committed profile, or
    None when there is none or the kernel source changed since."""
    path = profile_path(kernel, workload, "counters")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash(kernel):
        return None
    try:
        return int(float(vals["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_threads() -> int:
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        n = min(n, int(env))
    return max(1, n)


def cpu_baseline(inp, pool_rows: np.ndarray, budget_s: float):
    """The oracle on the same batch (its own copy of the gathered states),
    repeated until about `budget_s` seconds have passed on all host cores,
    then for a third of that on one core."""
    import oracle
    threads = cpu_threads()
    B = inp.wl.num_seqs
    idx = np.where(inp.state_idx >= 0, np.arange(B), -1).astype(np.int32)
    pool = np.ascontiguousarray(pool_rows, dtype=np.float32).copy()
    oracle.build(force=False)

    def timed(nthreads, budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.update(inp.q, inp.k, inp.v, inp.a, inp.b, inp.A_log, inp.dt_bias, pool, idx,
                          inp.cu_seqlens, tokens_per_seq=inp.wl.tokens_per_seq, threads=nthreads)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return W.active_updates(inp) * reps / el, reps, el

    value, reps, el = timed(threads, budget_s)
    one, reps1, el1 = timed(1, budget_s / 3)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": value, "unit": "updates/s", "cores": threads, "kind": "oracle",
            "cpu_model": model,
            "sample": f"the whole {inp.wl.name} batch ({B} sequences x {inp.wl.num_v_heads} "
                      f"v-heads), fp64 oracle, repeated {reps}x over {el:.1f} s",
            "single_core_value": one,
            "single_core_sample": f"the same batch on 1 thread, repeated {reps1}x over {el1:.1f} s"}


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def summarize_profiles(prof_dir: str, workload: str, kernel: str, commands: dict):
    """Writes the committed text summaries of one workload from rocprofv3 CSV
    output: the --kernel-trace --stats table, and HBM traffic per launch from
    the FETCH_SIZE and WRITE_SIZE passes, each scaled by what the same counter
    reads for a plain 1 GiB device copy (__amd_rocclr_copyBuffer)."""
    os.makedirs(PROFILES, exist_ok=True)
    stats = _csv_rows(os.path.join(prof_dir, "trace", "run_kernel_stats.csv"))
    lines = [f"# rocprofv3 kernel-trace summary: {kernel}, workload {workload}",
             f"# command: {commands['trace']}",
             f"# kernel source sha256[:16] = {kernel_source_hash(kernel)}",
             "# name | calls | average_us | min_us | max_us | percent"]
    import re
    for r in stats:
        m = re.search(r"(gdn_\w+<[^>]*>)", r["Name"])
        short = m.group(1) if m else r["Name"].replace("void ", "")[:60]
        lines.append(f"{short} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f}")
    # per-dispatch durations of the measured kernel from the trace records
    recs = _csv_rows(os.path.join(prof_dir, "trace", "run_kernel_trace.csv"))
    durs = np.array([(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                     for r in recs if kernel in r["Kernel_Name"]])
    if durs.size:
        lines.append(f"# {kernel}: {durs.size} dispatches; median {np.median(durs):.1f} us, "
                     f"p10 {np.percentile(durs, 10):.1f} us, p90 {np.percentile(durs, 90):.1f} us")
    # the dispatch resources rocprofv3 records, as printed (VGPR_Count is in
    # 4-register units of the 8-register wave64 allocation granule, and
    # LDS_Block_Size leaves out the dynamic LDS of the launch)
    res = sorted({(r["VGPR_Count"], r["Accum_VGPR_Count"], r["SGPR_Count"], r["LDS_Block_Size"],
                   r["Scratch_Size"], r["Workgroup_Size_X"], r["Grid_Size_X"])
                  for r in recs if kernel in r["Kernel_Name"]})
    for v, a, sg, lds, scr, wg, grid in res:
        lines.append(f"# {kernel} dispatch fields: VGPR_Count {v} (= {2 * int(v)} VGPRs allocated), "
                     f"Accum_VGPR_Count {a}, SGPR_Count {sg}, Scratch_Size {scr}, "
                     f"LDS_Block_Size {lds}, Workgroup_Size {wg}, Grid_Size {grid}")
    with open(profile_path(kernel, workload, "kernel_trace"), "w") as f:
        f.write("\n".join(lines) + "\n")

    def per_dispatch(counter, copy):
        sub = ("copy_" if copy else "") + counter
        rows = _csv_rows(os.path.join(prof_dir, sub, "run_counter_collection.csv"))
        want = "__amd_rocclr_copyBuffer" if copy else kernel
        vals = [float(r["Counter_Value"]) for r in rows
                if want in r["Kernel_Name"] and r["Counter_Name"] == counter]
        return sum(vals) / len(vals), len(vals)

    gib_kib = (1 << 30) / 1024
    fetch, nf = per_dispatch("FETCH_SIZE", False)
    write, nw = per_dispatch("WRITE_SIZE", False)
    cfetch, _ = per_dispatch("FETCH_SIZE", True)
    cwrite, _ = per_dispatch("WRITE_SIZE", True)
    f_fac, w_fac = gib_kib / cfetch, gib_kib / cwrite
    traffic = (fetch * f_fac + write * w_fac) * 1024
    wl = W.ALL[workload]
    alg = W.algorithmic_bytes(W.make_host_inputs(wl))
    out = [f"# rocprofv3 HBM counters: {kernel}, workload {workload}",
           f"# command (FETCH_SIZE): {commands['fetch']}",
           f"# command (WRITE_SIZE): {commands['write']}",
           f"# calibration: {commands['copy']} (1 GiB read + 1 GiB written per dispatch)",
           f"# summarised by: {commands['summary']}",
           f"kernel_source_sha256_16 = {kernel_source_hash(kernel)}",
           f"fetch_kib_per_dispatch = {fetch:.1f}   # mean over {nf} dispatches",
           f"write_kib_per_dispatch = {write:.1f}   # mean over {nw} dispatches",
           f"copy_fetch_kib_per_dispatch = {cfetch:.1f}",
           f"copy_write_kib_per_dispatch = {cwrite:.1f}",
           f"fetch_calibration_factor = {f_fac:.4f}",
           f"write_calibration_factor = {w_fac:.4f}",
           f"traffic_bytes_per_launch = {traffic:.0f}",
           f"algorithmic_bytes_per_launch = {alg}",
           f"traffic_over_algorithmic = {traffic / alg:.4f}"]
    with open(profile_path(kernel, workload, "counters"), "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(lines + out))


def summarize_utilization(prof_dir: str, workload: str, kernel: str, run: str):
    """Writes profiles/<kernel>__<workload>__utilization.txt: the mean per
    dispatch of every counter found in the rocprofv3 --pmc passes under
    prof_dir (one subdirectory per pass)."""
    os.makedirs(PROFILES, exist_ok=True)
    vals, cmds = {}, []
    for sub in sorted(os.listdir(prof_dir)):
        path = os.path.join(prof_dir, sub, "run_counter_collection.csv")
        if not os.path.exists(path):
            continue
        names = set()
        for r in _csv_rows(path):
            if kernel in r["Kernel_Name"]:
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                names.add(r["Counter_Name"])
        cmds.append(f"# command: rocprofv3 --pmc {' '.join(sorted(names))} --output-format csv "
                    f"-d {prof_dir}/{sub} -o run -- {run} --steps 5 --warmup 1 --cpu-budget 0")
    lines = [f"# rocprofv3 utilization counters: {kernel}, workload {workload}", *cmds,
             f"# kernel source sha256[:16] = {kernel_source_hash(kernel)}",
             "# counter = mean over dispatches (dispatches)"]
    lines += [f"{k} = {np.mean(v):.3f}   ({len(v)})" for k, v in sorted(vals.items())]
    with open(profile_path(kernel, workload, "utilization"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=W.DECODE_B512.name, choices=sorted(W.ALL))
    ap.add_argument("--slot-sets", type=int, default=8)
    ap.add_argument("--family", type=int, default=0,
                    help="0 auto, 1 column tiles, 2 row split, 3 value rows (VK layout), "
                         "4 chunked (64-token chunks on the matrix cores)")
    ap.add_argument("--layout", default="KV", choices=["KV", "VK"],
                    help="storage order of the state tiles")
    ap.add_argument("--state-dtype", default="f32", choices=["f32", "bf16"],
                    help="storage type of the state pool (the update runs in fp32 either way)")
    ap.add_argument("--block-v", type=int, default=0)
    ap.add_argument("--block-k", type=int, default=0)
    ap.add_argument("--waves", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle time for the CPU baseline (0 skips it)")
    ap.add_argument("--graph", action="store_true",
                    help="replay captured HIP graphs (one per slot set, each holding one step's "
                         "launches) instead of launching every step from Python")
    ap.add_argument("--unfused", action="store_true",
                    help="time the unfused pair instead: gdn_gating + gdn_recurrent_update per step")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="instead: time a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="instead: write profiles/ summaries from rocprofv3 CSV output in DIR "
                         "(subdirectories trace, FETCH_SIZE, WRITE_SIZE, copy_FETCH_SIZE, "
                         "copy_WRITE_SIZE)")
    ap.add_argument("--summarize-utilization", metavar="DIR",
                    help="instead: write the profiles/ utilization summary from rocprofv3 --pmc "
                         "passes in the subdirectories of DIR")
    ap.add_argument("--kernel", default="gdn_decode_rows", help="kernel name for --summarize-profiles")
    args = ap.parse_args()

    if args.summarize_utilization:
        run = f"python3 bench.py --workload {args.workload}" + (
            f" --family {args.family}" if args.family else "")
        summarize_utilization(args.summarize_utilization, args.workload, args.kernel, run)
        return

    if args.summarize_profiles:
        d = args.summarize_profiles
        run = f"python3 bench.py --workload {args.workload}" + (
            f" --family {args.family}" if args.family else "")
        summarize_profiles(d, args.workload, args.kernel, {
            "trace": f"rocprofv3 --kernel-trace --stats --output-format csv -d {d}/trace -o run -- "
                     f"{run} --steps 50 --warmup 5 --cpu-budget 0",
            "fetch": f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/FETCH_SIZE -o run -- "
                     f"{run} --steps 5 --warmup 1 --cpu-budget 0",
            "write": f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/WRITE_SIZE -o run -- "
                     f"{run} --steps 5 --warmup 1 --cpu-budget 0",
            "copy": f"rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -d "
                    f"{d}/copy_<counter> -o run -- python3 bench.py --copy-calibration --steps 3 "
                    f"--warmup 1",
            "summary": f"{run} --kernel {args.kernel} --summarize-profiles {d}"})
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the update "
              "shards by sequence or by k-head group with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_attention_recurrent_gating_amd as gdn
    dev = torch.device("cuda:0")

    if args.copy_calibration:
        n = 1 << 28  # 1 GiB of fp32
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        el = (time.perf_counter() - t0) / args.steps
        print(json.dumps({"copy_calibration_bytes_read": 4 * n, "copy_calibration_bytes_written": 4 * n,
                          "launches": args.warmup + args.steps, "copy_gb_s": 8 * n / el / 1e9}))
        return

    wl = W.ALL[args.workload]
    inp = W.make_host_inputs(wl)
    d = W.to_torch(inp, dev)
    sets = max(1, args.slot_sets if wl.num_slots >= args.slot_sets * wl.num_seqs else 1)
    # Disjoint slot sets: set s maps sequence i to slot s*B + i of a permuted pool.
    B = wl.num_seqs
    live = inp.state_idx >= 0
    idx_sets = []
    rng = np.random.default_rng(wl.seed + 7)
    perm = rng.permutation(wl.num_slots)
    for s in range(sets):
        idx = perm[s * B:(s + 1) * B].astype(np.int32) if sets > 1 else inp.state_idx.copy()
        idx[~live] = -1
        idx_sets.append(torch.from_numpy(idx).to(dev))
    pool = W.make_pool_torch(wl, dev)
    if args.layout == "VK":
        pool = pool.transpose(-1, -2).contiguous()
    if args.state_dtype == "bf16":
        pool = pool.to(torch.bfloat16)
    act = torch.bfloat16 if wl.act == W.ACT_BF16 else torch.float32
    out = torch.empty(inp.num_tokens, wl.num_v_heads, wl.head_v_dim, dtype=act, device=dev)
    inter = None
    if wl.intermediates:
        inter = torch.empty((inp.num_tokens, wl.num_v_heads) + tuple(pool.shape[2:]),
                            dtype=pool.dtype, device=dev)
    # the oracle's copy of the first set's initial states, taken before any update
    pool_rows0 = None
    if args.cpu_budget > 0:
        rows0 = pool[idx_sets[0].clamp(min=0).long()]
        pool_rows0 = (rows0.view(torch.int16).cpu().numpy().view(np.uint16)
                      if args.state_dtype == "bf16" else rows0.cpu().numpy())
        if args.layout == "VK":
            pool_rows0 = np.ascontiguousarray(np.swapaxes(pool_rows0, -1, -2))

    stream = torch.cuda.current_stream(dev)
    g_buf = torch.empty(inp.num_tokens, wl.num_v_heads, dtype=torch.float32, device=dev)
    beta_buf = torch.empty_like(g_buf)

    def launch(i):
        # on torch's current stream: the timing stream, or the capture stream
        if args.unfused:
            gdn.gdn_gating(d["a"], d["b"], d["A_log"], d["dt_bias"], g_buf, beta_buf,
                           num_k_heads=wl.num_k_heads)
            gdn.gdn_recurrent_update(
                d["q"], d["k"], d["v"], g_buf, beta_buf, pool, idx_sets[i % sets],
                d["cu_seqlens"], out, inter, tokens_per_seq=wl.tokens_per_seq,
                kernel_family=args.family, block_v=args.block_v, block_k=args.block_k,
                waves_per_group=args.waves, state_layout=args.layout)
            return
        gdn.gdn_gating_delta_rule_update(
            d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], pool,
            idx_sets[i % sets], d["cu_seqlens"], out, inter, tokens_per_seq=wl.tokens_per_seq,
            kernel_family=args.family, block_v=args.block_v, block_k=args.block_k,
            waves_per_group=args.waves, state_layout=args.layout)

    for i in range(args.warmup):
        launch(i)
    torch.cuda.synchronize()
    if not args.graph:
        step = launch
    else:
        # One HIP graph per slot set: a replay enqueues exactly the launches of
        # one step, without the Python and argument-marshalling overhead.  (On
        # MI355X with this ROCm the replay measured ~7 us slower per step than
        # eager launches, so it is not the default.)
        graphs = []
        for s_ in range(sets):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                launch(s_)
            graphs.append(g)
        torch.cuda.synchronize()

        def step(i):
            graphs[i % sets].replay()

    # HIP events on the launch stream bracket the K timed launches: their
    # elapsed time / K is the mean device time per launch.  (An event pair
    # around every launch would add ~7 us per step to the wall time and ~4 us
    # to each measured duration.)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    kern_ms = ev0.elapsed_time(ev1) / args.steps
    updates = W.active_updates(inp)
    alg_bytes = W.algorithmic_bytes(inp, state_bytes=2 if args.state_dtype == "bf16" else 4)
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    value = updates * args.steps / wall
    info = gdn.gdn_plan(gdn.make_config(d["q"], d["v"], pool, idx_sets[0], d["cu_seqlens"],
                                        tokens_per_seq=wl.tokens_per_seq,
                                        kernel_family=args.family, block_v=args.block_v,
                                        block_k=args.block_k, waves_per_group=args.waves,
                                        state_layout=args.layout),
                        d["cu_seqlens"] is not None, inter is not None)

    # The committed counter profiles were taken with the default options
    # (fp32 state, KV layout, library tiling, fused gates); other runs get none.
    profiled = (args.state_dtype == "f32" and args.layout == "KV" and not args.unfused
                and not (args.block_v or args.block_k or args.waves))
    traffic = counter_traffic(kernel_name(info), wl.name) if profiled else None
    res = {
        "metric": METRIC,
        "value": value,
        "unit": "updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "num_seqs": B, "tokens": inp.num_tokens,
                   "num_k_heads": wl.num_k_heads, "num_v_heads": wl.num_v_heads,
                   "head_k_dim": wl.head_k_dim, "head_v_dim": wl.head_v_dim,
                   "activations": wl.act, "state": args.state_dtype, "state_layout": args.layout,
                   "pool_slots": wl.num_slots,
                   "slot_sets": sets, "kernel": kernel_name(info),
                   "block_v": info.block_v, "block_k": info.block_k,
                   "waves_per_group": info.waves_per_group, "workgroups": info.workgroups,
                   "gates": "unfused pair (gdn_gating + gdn_recurrent_update)" if args.unfused
                            else "fused",
                   "launch": "HIP graph replay" if args.graph else "eager",
                   "parallelism": "single GPU"},
        "hbm_gb_s": achieved,
        "hbm_frac_of_peak": achieved / HBM_PEAK_GBS,
        "kernel_us": kern_ms * 1e3,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "traffic_gb_s": None if traffic is None else traffic / (kern_ms * 1e-3) / 1e9,
                     "traffic_frac": None if traffic is None
                                     else traffic / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "algorithmic_bytes": alg_bytes, "kernel": kernel_name(info)},
        "cpu_baseline": None,
    }
    if info.kernel_family == gdn.GDN_KERNEL_CHUNKED:
        # Dense products of the chunked form on the bf16 matrix cores.
        flops = W.chunked_flops(inp)
        tflops = flops / (kern_ms * 1e-3) / 1e12
        res["roofline"] = {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
                           "traffic": traffic,
                           "algorithmic_flops": flops, "algorithmic_bytes": alg_bytes,
                           "kernel": KERNEL_NAMES[4]}
    else:
        # Token-by-token kernels: whichever of HBM and the fp32 VALU takes
        # longer at its peak bounds the call (long sequences: the VALU).
        flops = W.recurrent_flops(inp)
        if flops / (VALU_FP32_PEAK_TFLOPS * 1e12) > alg_bytes / (HBM_PEAK_GBS * 1e9):
            tflops = flops / (kern_ms * 1e-3) / 1e12
            res["roofline"] = {"bound": "alu", "achieved": tflops, "peak": VALU_FP32_PEAK_TFLOPS,
                               "unit": "TFLOP/s", "frac": tflops / VALU_FP32_PEAK_TFLOPS,
                               "traffic": traffic, "algorithmic_flops": flops,
                               "algorithmic_bytes": alg_bytes, "kernel": kernel_name(info)}
    if args.cpu_budget > 0:
        res["cpu_baseline"] = cpu_baseline(inp, pool_rows0, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
