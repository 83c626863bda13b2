"""Decode throughput of the fp32 Llama-2-architecture path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C5]

One step = one decode position of the whole forward pass (embedding, every
layer's RMSNorm, Q/K/V + rotary + KV write, attention over the cache, Wo +
residual, RMSNorm, SwiGLU FFN + residual, final norm, classifier, greedy
arg-max), tokens fed back on the device.  Default workload: the 7B shape at
batch 1 (512-token random prompt prefilled, then decode positions 512..1023),
weights N(0, 0.02) from seed 4, all resident in HBM before timing starts.

Prints one JSON line with the throughput, the dominant kernel's roofline
(measured with HIP events on the library's stream inside the timed region) and
the CPU oracle timed on this host on a bounded sample.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/sec at batch 1 (15M/44M/7B-shape fp32) + achieved HBM GB/s"
HBM_PEAK_GBS = 8000.0
MFMA_F32_PEAK_TFLOPS = 157.3
W13_SOURCES = ["transformer_llama_decode_amd/csrc/k_gemv.hip", "transformer_llama_decode_amd/csrc/dev_common.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_w13_gemv_7b.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def step_bytes(cfg, pos, batch=1):
    """Algorithmic HBM bytes of one decode step at position pos: every matrix
    once, plus per sequence the embedding row, norm gains, the K/V history read
    (positions 0..pos, or the max_seq of them in the window past max_seq), the
    new K/V written and the logits written."""
    d, f, V, L, kvd = cfg.dim, cfg.hidden_dim, cfg.vocab_size, cfg.n_layers, cfg.kv_dim
    weights = cfg.weight_elem_bytes * (L * (2 * d * d + 2 * kvd * d + 3 * d * f) + V * d)
    gains = 4 * (2 * L + 1) * d
    seen = min(pos + 1, cfg.max_seq)
    per_seq = 4 * (d + 2 * L * seen * kvd + 2 * L * kvd + V)
    return weights + gains + batch * per_seq


def w13_launch_bytes(cfg):
    """Algorithmic bytes of one W1/W3 + SwiGLU launch at batch 1: both weight
    matrices once (4 or 2 bytes per element), the input row and its gain read,
    the gate row written."""
    d, f = cfg.dim, cfg.hidden_dim
    return cfg.weight_elem_bytes * 2 * f * d + 4 * (2 * d + f)


def sources_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per W13 launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != sources_hash(W13_SOURCES):
        return None
    return t.get("bytes_per_launch")


def host_cpu():
    """The host's CPU as lscpu reports it: model, logical CPUs, sockets, and the
    CPUs this process may run on."""
    import subprocess
    info = {"model": None, "logical_cpus": os.cpu_count(), "sockets": None,
            "usable_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
    except (OSError, subprocess.SubprocessError):
        return info
    for line in out.splitlines():
        k, _, v = line.partition(":")
        k, v = k.strip(), v.strip()
        if k == "Model name" and info["model"] is None:
            info["model"] = v
        elif k == "Socket(s)":
            info["sockets"] = int(v) if v.isdigit() else v
    return info


def _oracle_rate(L, w, n_steps, model=None):
    """tok/s of one oracle build over positions 0..n_steps-1 of w's model from
    token 1 (greedy), one host thread; the weights are drawn beforehand."""
    import numpy as np
    from oracle import oracle as O
    m = model or O.OracleModel(w.model, w.model_seed, nthreads=min(16, os.cpu_count() or 1), L=L)
    st = m.new_state()
    logits = np.empty(w.model.vocab_size, np.float32)
    tok = 1
    t0 = time.perf_counter()
    for p in range(n_steps):
        tok, _ = m.forward(st, tok, p, logits)
    dt = time.perf_counter() - t0
    if model is None:
        m.close()
    return n_steps / dt


def cpu_baseline(w, n_steps):
    """The oracle (plain single-threaded C) on this host: the parity build (fp64
    accumulation) on a bounded sample of the benchmarked workload, and, for
    comparison with the pages' CPU figures, a timing-only build with float
    accumulators (the pages' plain fp32 loop, gcc -O3 without fast-math) on the
    same sample and on the whole 15M-shape run (256 positions)."""
    from oracle import oracle as O
    from oracle import _build as OB
    from transformer_llama_decode_amd.configs import WORKLOADS
    if not os.path.exists(OB.ORACLE_TIMING_LIB):
        OB.build_oracle_timing()
    Ld, Lf = O.lib(), O.lib(OB.ORACLE_TIMING_LIB)
    t0 = time.time()
    m = O.OracleModel(w.model, w.model_seed, nthreads=min(16, os.cpu_count() or 1), L=Ld)
    gen_s = time.time() - t0
    rate = _oracle_rate(Ld, w, n_steps, model=m)
    m.close()
    del m
    rate_f = _oracle_rate(Lf, w, n_steps)
    c1 = WORKLOADS["C1"]
    c1_d = _oracle_rate(Ld, c1, c1.end_pos)
    c1_f = _oracle_rate(Lf, c1, c1.end_pos)
    return {
        "value": rate, "unit": "tok/s", "cores": 1, "kind": "oracle",
        "sample": "%d decode positions (p=0..%d) of the %s model, batch 1, one host thread, "
                  "gcc -O3, fp32 storage / fp64 accumulation; weights drawn beforehand in %.0fs"
                  % (n_steps, n_steps - 1, w.name, gen_s),
        "float_accumulation": {
            "value": rate_f, "unit": "tok/s", "cores": 1,
            "sample": "the same %d positions, oracle built with -DOR_ACC=float (timing only)" % n_steps},
        "c1_15m_shape": {
            "fp64_accumulation_tok_s": c1_d, "float_accumulation_tok_s": c1_f, "cores": 1,
            "sample": "C1: positions 0..%d of the 15M shape from token 1 (the pages quote ~100 tok/s "
                      "for this shape on one M1 core)" % (c1.end_pos - 1)},
        "host": host_cpu(),
    }


def counter_commands(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    """The rocprofv3 passes a traffic summary comes from (each counter in a run of its own)."""
    run = "python -u bench.py --steps 16 --warmup 2 --no-cpu-baseline --no-others"
    cal = "python -u bench.py --copy-calibration"
    return ["rocprofv3 --pmc FETCH_SIZE --output-format csv -d %s -o f -- %s" % (fetch_dir, run),
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d %s -o w -- %s" % (write_dir, run),
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d %s -o f -- %s" % (copy_fetch_dir, cal),
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d %s -o w -- %s" % (copy_write_dir, cal),
            "python bench.py --summarize-counters %s %s %s %s"
            % (fetch_dir, write_dir, copy_fetch_dir, copy_write_dir)]


def summarize_counters(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, out_json, out_txt):
    """Turn four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE of the 7B decode
    bench, and of the plain 2 GiB copy of --copy-calibration) into HBM bytes per
    W1/W3 GEMV launch, each counter scaled by what it reads for the copy."""
    import csv
    import glob
    import re
    import statistics

    def per_kernel(d):
        path = glob.glob(os.path.join(d, "*_counter_collection.csv"))[0]
        out = {}
        for r in csv.DictReader(open(path)):
            name = re.sub(r"\(.*", "", r["Kernel_Name"].replace("(anonymous namespace)::", "")
                          .replace("void ", "").replace("ld::", ""))
            out.setdefault(name, []).append(float(r["Counter_Value"]) * 1024.0)   # KiB -> bytes
        return {k: statistics.median(v) for k, v in out.items()}

    copy_bytes = 4 << 29
    f_copy = max(per_kernel(copy_fetch_dir).values())
    w_copy = max(per_kernel(copy_write_dir).values())
    k_fetch = copy_bytes / f_copy
    k_write = copy_bytes / w_copy
    fetch, write = per_kernel(fetch_dir), per_kernel(write_dir)
    from transformer_llama_decode_amd.configs import WORKLOADS
    cfg = WORKLOADS["C5"].model
    lines = ["kernel  fetch_KiB_raw  write_KiB_raw  traffic_bytes(scaled)  algorithmic_bytes"]
    w13 = None
    for name in sorted(fetch, key=lambda n: -fetch[n]):
        if name not in write:
            continue
        t = fetch[name] * k_fetch + write[name] * k_write
        # the 7B W1/W3 GEMV: the SwiGLU epilogue (2) with streamed loads, the largest of them
        is_w13 = name.startswith("k_gemv<2,") and w13 is None
        alg = w13_launch_bytes(cfg) if is_w13 else None
        if is_w13:
            w13 = t
        lines.append("%-28s %14.1f %14.1f %22.0f %18s" % (name, fetch[name] / 1024, write[name] / 1024, t,
                                                           alg if alg else "-"))
    rec = {"kernel": "k_gemv<EPI_SWIGLU> (W1/W3 + SwiGLU GEMV), 7B shape, batch 1",
           "bytes_per_launch": round(w13), "algorithmic_bytes_per_launch": w13_launch_bytes(cfg),
           "fetch_scale": round(k_fetch, 4), "write_scale": round(k_write, 4),
           "kernel_source_hash": sources_hash(W13_SOURCES)}
    with open(out_json, "w") as fh:
        json.dump(rec, fh, indent=1)
    with open(out_txt, "w") as fh:
        fh.write("HBM traffic per kernel launch from rocprofv3 counters, 7B-shape decode at batch 1.\n"
                 "commands (from the repository root, on an MI355X; each pass a run of its own):\n"
                 + "".join("  %s\n" % c for c in counter_commands(fetch_dir, write_dir, copy_fetch_dir,
                                                                   copy_write_dir)) + "\n")
        fh.write("copy calibration: a 2 GiB device copy reads FETCH_SIZE %.0f KiB, WRITE_SIZE %.0f KiB "
                 "-> scale fetch x%.4f, write x%.4f\n" % (f_copy / 1024, w_copy / 1024, k_fetch, k_write))
        fh.write("\n".join(lines) + "\n")
    print(json.dumps(rec))


def summarize_trace(trace_dir, title, command, out_txt):
    """Per-kernel durations of one rocprofv3 --kernel-trace --stats run (its
    *_kernel_stats.csv) as a text table under profiles/."""
    import csv
    import glob
    import re
    path = glob.glob(os.path.join(trace_dir, "*_kernel_stats.csv"))[0]
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = ["%-52s %7s %12s %10s %10s %10s" % ("kernel", "calls", "total_ms", "avg_us", "min_us", "max_us")]
    for r in rows:
        name = re.sub(r"^void ", "", r["Name"]).replace("ld::(anonymous namespace)::", "").replace("ld::", "")
        lines.append("%-52s %7d %12.3f %10.2f %10.2f %10.2f" % (
            name[:52], int(r["Calls"]), float(r["TotalDurationNs"]) / 1e6, float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    with open(out_txt, "w") as fh:
        fh.write("rocprofv3 kernel statistics: %s\n\ncommand (from the repository root, on an MI355X):\n  %s\n  "
                 "python bench.py --summarize-trace %s '<title>' %s\n\n" % (title, command, trace_dir, out_txt))
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


MFMA_COUNTERS = "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F32 GRBM_GUI_ACTIVE"


def summarize_mfma(pmc_dir, workload, out_txt, n_xcd=8, n_simd=1024):
    """Matrix-core use per kernel of a batched decode bench from one rocprofv3 --pmc
    run of MFMA_COUNTERS: fp32 matrix flops (SQ_INSTS_VALU_MFMA_MOPS_F32 counts units
    of 512), and the busy share of the matrix cores, SQ_VALU_MFMA_BUSY_CYCLES over
    the kernel's cycles (GRBM_GUI_ACTIVE, summed over the XCDs) times the SIMDs."""
    import collections
    import csv
    import glob
    import re
    path = glob.glob(os.path.join(pmc_dir, "*_counter_collection.csv"))[0]
    tot = collections.defaultdict(lambda: collections.defaultdict(float))
    launches = collections.defaultdict(set)
    for r in csv.DictReader(open(path)):
        name = re.sub(r"\(ld::.*", "", r["Kernel_Name"].replace("(anonymous namespace)::", "")
                      .replace("void ", "").replace("ld::", ""))
        tot[name][r["Counter_Name"]] += float(r["Counter_Value"])
        launches[name].add(r["Dispatch_Id"])
    lines = ["%-46s %7s %16s %14s %11s" % ("kernel", "calls", "MFMA flops/call", "kernel cycles",
                                           "MFMA busy")]
    all_busy = all_cyc = 0.0
    for name, c in sorted(tot.items(), key=lambda kv: -kv[1]["SQ_VALU_MFMA_BUSY_CYCLES"]):
        if c["SQ_INSTS_VALU_MFMA_MOPS_F32"] == 0:
            continue
        n = len(launches[name])
        cyc = c["GRBM_GUI_ACTIVE"] / n_xcd
        busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * n_simd)
        all_busy += c["SQ_VALU_MFMA_BUSY_CYCLES"]
        all_cyc += cyc
        lines.append("%-46s %7d %16.4g %14.0f %10.1f%%" % (name[:46], n, 512 * c["SQ_INSTS_VALU_MFMA_MOPS_F32"] / n,
                                                          cyc / n, 100 * busy))
    lines.append("all matrix-core kernels: MFMA busy %.1f%% of their cycles" % (100 * all_busy / (all_cyc * n_simd)))
    with open(out_txt, "w") as fh:
        fh.write("Matrix-core use per kernel from rocprofv3 counters, workload %s (the run includes the\n"
                 "prompt's prefill: the LDS-tiled k_gemm launches with few calls).\n"
                 "command (from the repository root, on an MI355X):\n"
                 "  rocprofv3 --pmc %s --output-format csv -d %s -o m -- python -u bench.py --workload %s "
                 "--steps 16 --warmup 2 --no-cpu-baseline --no-others\n"
                 "  python bench.py --summarize-mfma %s %s\n\n"
                 % (workload, MFMA_COUNTERS, pmc_dir, workload, pmc_dir, workload))
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def gemm_flops_per_step(cfg, batch):
    """Algorithmic flops of every projection of one decode step for `batch` rows."""
    d, f, V, L, kvd = cfg.dim, cfg.hidden_dim, cfg.vocab_size, cfg.n_layers, cfg.kv_dim
    return 2 * batch * (L * (2 * d * d + 2 * kvd * d + 3 * d * f) + V * d)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="C5",
                    help="C5 (default: 7B shape, batch 1); also C1, C2, C3 (batch 256), C4, C4b32")
    ap.add_argument("--cpu-steps", type=int, default=4)
    ap.add_argument("--graph", action="store_true",
                    help="time the on-device generation loop (ld_generate: the step replayed as a "
                         "HIP graph) instead of one ld_decode_step call per position (both feed "
                         "the greedy tokens back on the device)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true",
                    help="with the default workload, skip the other configurations' sub-records")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of known size (for counter calibration)")
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("DIR", "WORKLOAD"),
                    help="a rocprofv3 --pmc run of the MFMA counters on a batched workload: writes "
                         "the matrix-core use per kernel under profiles/")
    ap.add_argument("--summarize-trace", nargs=4, metavar=("DIR", "TITLE", "COMMAND", "OUT"),
                    help="a rocprofv3 --kernel-trace --stats output dir: writes its per-kernel table to OUT")
    ap.add_argument("--summarize-counters", nargs=4, metavar="DIR",
                    help="rocprofv3 --pmc output dirs: FETCH_SIZE and WRITE_SIZE of this bench, "
                         "then of --copy-calibration; writes the traffic summary under profiles/")
    args = ap.parse_args()
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma[0], args.summarize_mfma[1],
                       os.path.join(ROOT, "profiles", "mfma_%s.txt" % args.summarize_mfma[1].lower()))
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, TRAFFIC_FILE,
                           os.path.join(ROOT, "profiles", "counters_w13_gemv_7b.txt"))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the decode path runs on a single MI355X "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = 1 << 29   # 2 GiB of fp32
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / 5
        print(json.dumps({"copy_bytes_read_per_launch": 4 * n, "copy_bytes_written_per_launch": 4 * n,
                          "launches": 6, "copy_ms": round(dt * 1e3, 3),
                          "copy_gbps_read_plus_write": round(8 * n / dt / 1e9, 1)}))
        return

    from transformer_llama_decode_amd.configs import WORKLOADS

    w = WORKLOADS[args.workload]
    rec = measure(w, args.steps, args.warmup, args.graph)
    if args.workload == "C5" and not args.no_others:
        # the other configurations of the metric, each over (up to) its first
        # decode positions: the 15M / 44M / 110M batch-1 shapes and the two
        # batched-decode shapes (matrix-core projections)
        rec["other_workloads"] = {}
        for name, steps in [("C1", 255), ("C2", 512), ("C4", 512), ("C3", 240), ("C4b32", 512)]:
            r = measure(WORKLOADS[name], steps, 16, args.graph)
            rec["other_workloads"][name] = {
                k: r[k] for k in ("value", "unit", "ms_per_step", "hbm_gbps_step", "hbm_frac_step", "prefill_ms")}
            rec["other_workloads"][name]["positions"] = r["config"]["positions"]
            rec["other_workloads"][name]["batch"] = r["config"]["batch"]
            if r["roofline"]["bound"] == "mfma":
                rec["other_workloads"][name]["mfma"] = {
                    k: r["roofline"][k] for k in ("achieved", "peak", "unit", "frac", "whole_step_frac",
                                                  "gemm_ms_per_step", "per_class_ms")}
        rec["batched"] = dict(rec["other_workloads"]["C3"], workload="C3: 15M shape, 256 sequences in lockstep")
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("cpu baseline: drawing weights for the oracle ...")
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_steps)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


def measure(w, n_steps, warmup, graph):
    """Init, prefill (timed on its own), `warmup` untimed decode steps, then
    exactly n_steps timed decode steps at positions P .. P+n_steps-1 (P = the
    prompt length), tokens fed back on the device; then the same positions again
    with HIP event pairs around the projection kernels.  Returns the JSON record."""
    import numpy as np
    import torch
    from transformer_llama_decode_amd.model import LlamaDecoder, synth_prompt
    from transformer_llama_decode_amd import _lib
    cfg = w.model
    B = w.batch
    P = max(w.prompt_len, 1)
    steps = min(n_steps, w.end_pos - P)
    if P + max(steps, warmup) > cfg.positions:
        sys.exit("steps + prompt exceed the model's %d positions" % cfg.positions)
    dev = torch.device("cuda", 0)
    t0 = time.time()
    gm = LlamaDecoder(cfg, w.model_seed)
    torch.cuda.synchronize()
    log("init %.1fs (%s, arena %.2f GB)" % (time.time() - t0, w.name, gm.arena.numel() / 1e9))

    if w.prompt_len:
        prompt = np.stack([synth_prompt(w.prompt_seed, b, w.prompt_len) for b in range(B)])
    else:
        prompt = np.full((B, 1), w.start_token, np.int32)
    bufs = [torch.zeros(B, dtype=torch.int32, device=dev) for _ in range(2)]
    # prefill (timed on its own)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if w.prompt_len:
        gm.prefill(prompt, next_out=bufs[0])
    else:
        gm.decode_step(prompt[:, 0], next_out=bufs[0])
    torch.cuda.synchronize()
    prefill_s = time.perf_counter() - t0
    log("prefill %d x %d tokens: %.1f ms" % (B, prompt.shape[1], prefill_s * 1e3))

    def run(k, tok):
        for i in range(k):
            out = bufs[(i + 1) % 2] if tok is bufs[i % 2] else bufs[i % 2]
            gm.decode_step(tok, next_out=out)
            tok = out
        return tok

    gen_out = torch.empty((max(steps, warmup), B), dtype=torch.int32, device=dev)

    def run_timed(k, tok):
        if not graph:
            return run(k, tok)
        gm.generate(tok, k, out=gen_out)
        return gen_out[k - 1]

    tok = run_timed(warmup, bufs[0]) if warmup > 0 else bufs[0]
    torch.cuda.synchronize()
    gm.set_pos(P)                      # time exactly the workload's positions P .. P+steps-1
    start_tok = tok.clone()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    run_timed(steps, start_tok)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_s = ev0.elapsed_time(ev1) / 1e3
    # Kernels timed with HIP events recorded around each of their launches on
    # the library's stream, over the same positions again (event records stall
    # the stream for a few microseconds, so they stay out of the throughput pass).
    classes = [_lib.LD_K_W13] if B == 1 else [_lib.LD_K_QKV, _lib.LD_K_WO, _lib.LD_K_W13,
                                              _lib.LD_K_W2, _lib.LD_K_CLS]
    if gm.set_pos_rc(P) != 0:
        # past max_seq the ring no longer holds position P's window: time the next
        # positions instead (the step's work does not depend on the position there)
        if gm.pos + steps > cfg.positions:
            sys.exit("no positions left for the kernel timing pass")
        log("kernel timing pass at positions %d..%d" % (gm.pos, gm.pos + steps - 1))
    for k in classes:
        gm.profile(k, True)
    run(steps, start_tok)
    kt = {k: gm.profile_read(k) for k in classes}
    for k in classes:
        gm.profile(k, False)
    status = gm.status()
    if status != 0:
        sys.exit("device reported error %d during the run" % status)

    elapsed = wall
    tok_s = B * steps / elapsed
    avg_bytes = sum(step_bytes(cfg, p, B) for p in range(P, P + steps)) / steps
    if B == 1:
        w13_ms, w13_n = kt[_lib.LD_K_W13]
        w13_bytes = w13_launch_bytes(cfg)
        achieved = w13_bytes / (w13_ms * 1e-3) / 1e9 if w13_ms > 0 else None
        roof = {
            "bound": "hbm",
            "kernel": "W1/W3 + SwiGLU GEMV (k_gemv<EPI_SWIGLU>), batch 1%s"
                      % (", bfloat16 weights" if cfg.weight_bf16 else ""),
            "achieved": round(achieved, 1) if achieved else None,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4) if achieved else None,
            "traffic": measured_traffic() if w.name == "C5" else None,
            "bytes_per_launch": w13_bytes,
            "avg_launch_ms": round(w13_ms, 5),
            "launches": w13_n,
        }
        log("decode: %.3f ms/step, %.1f tok/s, %.0f GB/s over the step; W13 %.4f ms x %d -> %.0f GB/s"
            % (elapsed / steps * 1e3, tok_s, avg_bytes * tok_s / 1e9, w13_ms, w13_n, achieved or 0))
    else:
        gemm_s = sum(ms * n for ms, n in kt.values()) / 1e3 / steps   # GEMM seconds per step
        flops = gemm_flops_per_step(cfg, B)
        achieved = flops / gemm_s / 1e12
        roof = {
            "bound": "mfma",
            "kernel": "fp32 MFMA projections (k_gemm, v_mfma_f32_32x32x2_f32), batch %d" % B,
            "achieved": round(achieved, 2),
            "peak": MFMA_F32_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_F32_PEAK_TFLOPS, 4),
            "traffic": None,
            "flops_per_step": flops,
            "gemm_ms_per_step": round(gemm_s * 1e3, 4),
            "per_class_ms": {name: round(kt[k][0], 5) for name, k in
                             [("qkv", _lib.LD_K_QKV), ("wo", _lib.LD_K_WO), ("w13", _lib.LD_K_W13),
                              ("w2", _lib.LD_K_W2), ("cls", _lib.LD_K_CLS)]},
            "whole_step_frac": round(flops * tok_s / B / 1e12 / MFMA_F32_PEAK_TFLOPS, 4),
        }
        log("decode: %.3f ms/step, %.0f tok/s; GEMMs %.3f ms/step -> %.1f TFLOP/s (%.1f%% of fp32 MFMA peak)"
            % (elapsed / steps * 1e3, tok_s, gemm_s * 1e3, achieved, 100 * achieved / MFMA_F32_PEAK_TFLOPS))
    roof["timing"] = ("HIP event pairs on the library's stream around every launch, in a second "
                      "pass over the timed positions")

    rec = {
        "metric": METRIC,
        "value": round(tok_s, 3),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(elapsed / steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",   # arithmetic; bfloat16 weights (when configured) are widened exactly
        "data": "synthetic",
        "config": {
            "workload": "%s: %s" % (w.name, w.description),
            "batch": B,
            "positions": "%d..%d" % (P, P + steps - 1),
            "prompt_tokens": int(prompt.shape[1]) if w.prompt_len else 0,
            "seed": w.model_seed,
            "weights": "bf16" if cfg.weight_bf16 else "f32",
            "loop": ("ld_generate: HIP graphs of 8 decode steps replayed" if graph else
                     "ld_decode_step per position, tokens fed back on the device"),
        },
        "hbm_gbps_step": round(avg_bytes * tok_s / B / 1e9, 1),
        "hbm_frac_step": round(avg_bytes * tok_s / B / 1e9 / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": int(avg_bytes),
        "gpu_event_ms_per_step": round(gpu_s / steps * 1e3, 4),
        "prefill_ms": round(prefill_s * 1e3, 2),
        "prefill_tok_s": round(B * prompt.shape[1] / prefill_s, 1),
        "roofline": roof,
    }
    gm.close()
    del gm
    torch.cuda.empty_cache()
    return rec




if __name__ == "__main__":
    main()
