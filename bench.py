"""Benchmark of the KV-cache compression hot path on one MI355X.

One step = the whole path over one synthetic prefill cache resident in HBM: nq_score_evict
(window sums, proxy scores, eviction), nq_encode (RoPE removal, Hadamard, E8, delta) and
nq_decode (running sum, dequantisation, inverse Hadamard, RoPE, fp16 store). The default
workload is the Mistral-7B-shaped balanced preset: 32 layers x 8 kv heads x 32768 tokens x 128,
fp16, K3V2, 60% eviction, BOS + 256-token window.

Prints ONE JSON line on stdout (diagnostics go to stderr):
  value      fp16-KV GB/s of the step = (fp16 K+V bytes encoded + fp16 K+V bytes decoded) /
             (time of the step); encode and decode rates are reported separately too
  roofline   for the dominant kernel (the one with the largest share of the step): algorithmic
             HBM bytes per launch / its average launch time (HIP events on the launch stream),
             against MI355X's 8 TB/s
  cpu_baseline  the CPU oracle timed on a bounded sample (a few layers) of the same workload
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HBM_PEAK_GBPS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", type=int, default=1, choices=[0, 1, 2, 3])
    ap.add_argument("--cpu-layers", type=int, default=4,
                    help="layers of the workload the CPU oracle baseline processes on one thread")
    ap.add_argument("--cpu-threads", type=int, default=min(16, os.cpu_count() or 1),
                    help="threads (one layer each) of the all-cores CPU oracle baseline "
                         "(default: the host's CPUs, at most 16, the CPU share of one GPU)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run one plain device copy of this many MiB (a known-size "
                         "kernel that calibrates rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    ap.add_argument("--traffic", default=None, metavar="MD",
                    help="HBM-traffic summary to read (default: profiles/hbm_traffic_<workload>.md)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the HBM-traffic summary from two rocprofv3 --pmc runs of this "
                         "script (FETCH_SIZE, then WRITE_SIZE, both with --copy-calibration) "
                         "and exit")
    ap.add_argument("--pmc-command", default="",
                    help="the profiling command, recorded in the summary")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("STATS_CSV", "NAME"),
                    help="write profiles/kernel_trace_<NAME>.md from a rocprofv3 --kernel-trace "
                         "--stats run's kernel_stats.csv (the command given by --pmc-command) "
                         "and exit")
    ap.add_argument("--title", default="", help="title line of a --summarize-trace summary")
    ap.add_argument("--timed-steps", type=int, default=0,
                    help="with --summarize-trace: also average each kernel over its last N "
                         "dispatches (the profiled run's timed steps), from the kernel_trace.csv "
                         "beside the stats CSV")
    ap.add_argument("--bench-log", default="",
                    help="with --summarize-trace: the profiled run's output; its JSON line's "
                         "roofline kernel and event-timed launch average are quoted")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("PMC_DIR", "NAME"),
                    help="write profiles/counters_<NAME>.md from a rocprofv3 --pmc run of SQ "
                         "instruction counters (the command given by --pmc-command) and exit")
    ap.add_argument("--attn-score", action="store_true",
                    help="time the attention-weight scorer (nq_score_evict_attn, 32 query heads, "
                         "W-query observation window) against the key-key proxy scorer on the "
                         "headline workload instead")
    ap.add_argument("--scalar", action="store_true",
                    help="time and compare the equal-bit Lloyd-Max scalar baseline against the E8 "
                         "codec on the same keep-set instead (throughput, SNR, cosine)")
    ap.add_argument("--entropy", action="store_true",
                    help="compress the workload on the GPU, then measure the host zstd stage's "
                         "post-entropy ratio (off the timed path) instead")
    ap.add_argument("--decode-step", action="store_true",
                    help="time the one-token GQA decode step over the long-context compressed "
                         "cache instead: fused nq_decode_attend against nq_decode + "
                         "nq_attend_decode")
    return ap.parse_args()


ROOT = os.path.dirname(os.path.abspath(__file__))
PHASE_KERNELS = {"score_evict": ("k_window_sum", "k_scores", "k_select", "k_select_reg"),
                 "encode": ("k_encode",),
                 "decode": ("k_decode_reset", "k_decode")}
# the fused decode step's kernels (bench.py --decode-step)
DECODE_STEP_KERNELS = {"decode_attend": ("k_decode_reset", "k_decode_attend",
                                         "k_decode_attend_merge")}
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def kernel_source_hash() -> str:
    """Hash of the HIP sources and the header: a traffic figure is valid only for the kernels
    it was measured on."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kv_cache_compression_proxy_amd", "csrc")
    for f in sorted(os.listdir(csrc)) + ["../../include/nq.h"]:
        if f.endswith((".hpp", ".hip", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_path(w, decode_step: bool = False) -> str:
    name = f"decode-step_{w.name}" if decode_step else w.name
    return os.path.join(ROOT, "profiles", f"hbm_traffic_{name}.md")


def summarize_pmc(args, w, decode_step: bool = False):
    """rocprofv3 counter CSVs -> profiles/hbm_traffic_<workload>.md (the headline step's phases)
    or profiles/hbm_traffic_decode-step_<cache>.md (the fused decode step, --decode-step).
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what they read for a device copy
    of known size."""
    import csv
    from collections import defaultdict

    def per_kernel(d, counter):
        vals = defaultdict(list)
        for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
            if r["Counter_Name"] == counter and ("nq::" in r["Kernel_Name"] or
                                                 COPY_KERNEL in r["Kernel_Name"]):
                name = r["Kernel_Name"].split("(")[0].split("<")[0]
                name = name.replace("void ", "").replace("nq::", "").strip()
                vals[name].append(float(r["Counter_Value"]))
        out = {k: (sum(v) / len(v), len(v)) for k, v in vals.items()}
        # the runtime's copy kernel also stages the host-to-device input uploads (smaller
        # copies): the calibration copy is its largest dispatch
        if COPY_KERNEL in vals:
            out[COPY_KERNEL] = (max(vals[COPY_KERNEL]), len(vals[COPY_KERNEL]))
        return out

    fetch = per_kernel(args.summarize_pmc[0], "FETCH_SIZE")
    write = per_kernel(args.summarize_pmc[1], "WRITE_SIZE")
    copy_bytes = args.copy_calibration << 20
    if not copy_bytes or COPY_KERNEL not in fetch or COPY_KERNEL not in write:
        sys.exit("--summarize-pmc needs the runs' --copy-calibration size and its copy kernel")
    fk = copy_bytes / (fetch[COPY_KERNEL][0] * 1024)
    wk = copy_bytes / (write[COPY_KERNEL][0] * 1024)
    title = f"fused decode step over {w.name}" if decode_step else w.name
    lines = [f"# HBM traffic per launch: {title}", "",
             "rocprofv3 counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch, averaged over the "
             "run's dispatches), each in a run of its own, scaled by what the same counter reads "
             f"for a plain device copy of {args.copy_calibration} MiB ({COPY_KERNEL}: reads and "
             "writes exactly that many bytes).", "",
             "Commands (from /tmp with TMPDIR=/tmp; `$REPO` is the repository root):", "", "```",
             args.pmc_command or "(not recorded)", "```", "",
             f"Calibration: FETCH_SIZE x {fk:.4f}, WRITE_SIZE x {wk:.4f} "
             f"(copy read {fetch[COPY_KERNEL][0]:.0f} KiB, wrote {write[COPY_KERNEL][0]:.0f} KiB "
             f"for {copy_bytes >> 10} KiB)", "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read GB | written GB |",
             "|---|---|---|---|---|---|"]
    for k in sorted(set(fetch) | set(write)):
        if k == COPY_KERNEL:
            continue
        f, n = fetch.get(k, (0.0, 0))
        wr = write.get(k, (0.0, 0))[0]
        lines.append(f"| {k} | {n} | {f:.0f} | {wr:.0f} | {f * 1024 * fk / 1e9:.4f} | "
                     f"{wr * 1024 * wk / 1e9:.4f} |")
    lines += ["", "Per launch of each phase (bytes; the figures bench.py reports as `traffic`):",
              "", "```"]
    for ph, ks in (DECODE_STEP_KERNELS if decode_step else PHASE_KERNELS).items():
        tot = sum(fetch.get(k, (0.0, 0))[0] * 1024 * fk + write.get(k, (0.0, 0))[0] * 1024 * wk
                  for k in ks)
        lines.append(f"traffic {ph} {int(round(tot))}")
    lines += [f"kernel-sources {kernel_source_hash()}", "```", ""]
    out = traffic_path(w, decode_step)
    open(out, "w").write("\n".join(lines))
    log(f"[bench] wrote {out}")


def summarize_trace(args):
    """rocprofv3 kernel stats CSV -> profiles/kernel_trace_<name>.md (per-kernel calls and
    durations; with --timed-steps N also each kernel's average over its last N dispatches, the
    steps the profiled run timed, next to the run's own event-timed figure from --bench-log)."""
    import csv
    from collections import defaultdict
    rows = list(csv.DictReader(open(args.summarize_trace[0])))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    name = args.summarize_trace[1]
    timed = {}
    if args.timed_steps > 0:
        durs = defaultdict(list)
        trace = os.path.join(os.path.dirname(args.summarize_trace[0]), "run_kernel_trace.csv")
        for r in sorted(csv.DictReader(open(trace)), key=lambda r: int(r["Start_Timestamp"])):
            durs[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        for k, v in durs.items():
            if len(v) >= args.timed_steps:
                last = v[-args.timed_steps:]
                timed[k] = (sum(last) / len(last), min(last), max(last))
    head = "| kernel | calls | avg us | min us | max us | share % |"
    rule = "|---|---|---|---|---|---|"
    if timed:
        head += f" avg us, last {args.timed_steps} |"
        rule += "---|"
    lines = [f"# rocprofv3 kernel stats: {args.title or name}", "",
             "Command (from /tmp, with TMPDIR=/tmp; `$REPO` is the repository root):", "", "```",
             args.pmc_command or "(not recorded)", "```", "", head, rule]
    for r in rows:
        line = (f"| {r['Name'][:120]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                f"{float(r['Percentage']):.2f} |")
        if timed:
            t = timed.get(r["Name"])
            line += f" {t[0]:.2f} |" if t else " |"
        lines.append(line)
    lines += ["", "Kernels outside `nq::` belong to bench.py itself (torch's fills and copies of "
              "inputs; in a headline run also the 1 GiB device copy timed as the achievable "
              "line); the shares include them."]
    if timed:
        lines += ["", f"`avg us, last {args.timed_steps}`: each kernel's average over its last "
                  f"{args.timed_steps} dispatches in the per-dispatch trace -- the run's timed "
                  "steps, after its warm-up steps (the first dispatches run while the board's "
                  "clock settles)."]
    if args.bench_log:
        res = [json.loads(ln) for ln in open(args.bench_log) if ln.startswith("{")]
        if res and "roofline" in res[-1]:
            rf = res[-1]["roofline"]
            lines += ["", f"The profiled run's own line: roofline kernel `{rf.get('kernel')}`, "
                      f"event-timed average {rf.get('avg_launch_ms')} ms per launch over its "
                      f"{res[-1].get('steps')} timed steps."]
    lines += ["", f"Kernel sources: {kernel_source_hash()}", ""]
    out = os.path.join(ROOT, "profiles", f"kernel_trace_{name}.md")
    open(out, "w").write("\n".join(lines))
    log(f"[bench] wrote {out}")


def summarize_counters(args):
    """rocprofv3 SQ counter CSV -> profiles/counters_<name>.md: per-dispatch averages of the
    instruction counters of the library's kernels."""
    import csv
    from collections import defaultdict
    vals = defaultdict(lambda: defaultdict(list))
    clock = defaultdict(list)   # GHz: GRBM busy cycles of one XCD over the dispatch's duration
    d = args.summarize_counters[0]
    for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
        if "nq::" not in r["Kernel_Name"]:
            continue
        name = r["Kernel_Name"].split("(")[0].replace("void ", "").replace("nq::", "").strip()
        vals[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
        dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        if r["Counter_Name"] == "GRBM_GUI_ACTIVE" and dur > 0:
            clock[name].append(float(r["Counter_Value"]) / 8 / dur)
    cols = [("SQ_WAVES", "waves", 1.0, "{:.0f}"), ("SQ_INSTS_VALU", "VALU instr (M)", 1e-6, "{:.1f}"),
            ("SQ_INSTS_VMEM_RD", "VMEM rd instr (M)", 1e-6, "{:.2f}"),
            ("SQ_INSTS_VMEM_WR", "VMEM wr instr (M)", 1e-6, "{:.2f}"),
            ("SQ_WAVE_CYCLES", "wave cycles (M)", 1e-6, "{:.0f}"),
            ("SQ_WAIT_INST_ANY", "waiting wave cycles (M)", 1e-6, "{:.0f}"),
            ("GRBM_GUI_ACTIVE", "GPU busy cycles (M, all XCDs)", 1e-6, "{:.2f}")]
    name = args.summarize_counters[1]
    lines = [f"# Instruction counters: {args.title or name}", "",
             "Per-dispatch averages of rocprofv3 SQ counters over the run's dispatches of each "
             "kernel. `VALU ms (4 cyc)` = SQ_INSTS_VALU x 4 cycles / (1024 SIMDs x 2.4 GHz): "
             "the time if every VALU instruction took the 4 issue cycles of a wave64 instruction "
             "on a 16-lane SIMD (plain fp32 add/mul, integer and bitwise ops issue in about half "
             "that on this chip, so this bounds the VALU time from above). `clock GHz` = "
             "GRBM_GUI_ACTIVE / 8 XCDs / the dispatch's duration: the average shader clock "
             "while the kernel ran (2.4 GHz nominal; meaningful for dispatches longer than "
             "~50 us).", "",
             "Command (from /tmp with TMPDIR=/tmp; `$REPO` is the repository root):", "", "```",
             args.pmc_command or "(not recorded)", "```", "",
             "| kernel | " + " | ".join(c[1] for c in cols) + " | VALU ms (4 cyc) | clock GHz |",
             "|---|" + "---|" * (len(cols) + 2)]
    for k in sorted(vals):
        m = {c: sum(v) / len(v) for c, v in vals[k].items()}
        cells = [fmt.format(m[c] * sc) if c in m else "" for c, _, sc, fmt in cols]
        valu_ms = m.get("SQ_INSTS_VALU", 0.0) * 4 / (1024 * 2.4e9) * 1e3
        ghz = f"{sum(clock[k]) / len(clock[k]):.2f}" if clock[k] else ""
        lines.append(f"| {k} | " + " | ".join(cells) + f" | {valu_ms:.3f} | {ghz} |")
    lines += ["", f"Kernel sources: {kernel_source_hash()}", ""]
    out = os.path.join(ROOT, "profiles", f"counters_{name}.md")
    open(out, "w").write("\n".join(lines))
    log(f"[bench] wrote {out}")


def read_traffic(path, phase):
    """Bytes per launch of a phase from a traffic summary, or None when absent or when the
    kernels have changed since the counters were taken."""
    try:
        txt = open(path).read().split("\n")
    except OSError:
        return None
    kv = {}
    for ln in txt:
        parts = ln.split()
        if len(parts) == 3 and parts[0] == "traffic":
            kv[parts[1]] = int(parts[2])
        elif len(parts) == 2 and parts[0] == "kernel-sources":
            kv["_hash"] = parts[1]
    if kv.get("_hash") != kernel_source_hash():
        return None
    return kv.get(phase)


def algorithmic_bytes(w, n_keep):
    """Bytes the method must move per launch of each kernel group (no cache reuse assumed)."""
    Lc, H, T = w.compressed_layers, w.kv_heads, w.tokens
    row = 256                                            # one fp16 head row
    kept_th = Lc * H * n_keep                            # kept token-heads
    enc = kept_th * (2 * row + 2 * 128 + 2 * 32)         # K+V rows in, codes + scales out
    enc += Lc * n_keep * 4 + T * 64 * 4 * 2              # positions; rotary table once
    dec = kept_th * (2 * 128 + 2 * 32 + 2 * row)         # codes + scales in, fp16 K+V out
    dec += Lc * n_keep * 4 + T * 64 * 4 * 2
    n_cand = max(T - w.window - 1, 0)
    score = Lc * H * T * row                             # one pass over all keys
    score += Lc * T * 8 * 2 + Lc * n_keep * 4            # scores written + read, positions
    return {"score_evict": score, "encode": enc, "decode": dec}


def cpu_baseline(w, layers: int, threads: int):
    """The oracle as it stands (plain sequential C, untuned), timed on the host's cores on a
    bounded sample of the workload: `layers` layers one after another on one thread, then
    `threads` layers at once on `threads` threads (one layer per thread; the oracle holds no
    shared state and ctypes releases the GIL during each call). Inputs are generated into host
    RAM before each timed region."""
    import kvsynth
    import oracle
    T = w.tokens
    Ct, St = oracle.rope_table(T, w.rope_base)
    n_keep = oracle.keep_count(T, w.window, w.evict_permille)
    kv_enc_layer = w.kv_heads * T * 256 * 2
    kv_dec_layer = w.kv_heads * n_keep * 256 * 2

    def work(KV):
        K, V = KV
        t0 = time.perf_counter()
        enc = oracle.compress_layer(K, V, w.window, w.evict_permille, w.bits_k, w.bits_v, Ct, St)
        t1 = time.perf_counter()
        oracle.decode_layer(enc["codes_k"], enc["codes_v"], enc["scales_k"], enc["scales_v"],
                            enc["positions"], Ct, St)
        return t1 - t0, time.perf_counter() - t1

    # one thread
    t_enc = t_dec = 0.0
    for l in range(layers):
        te, td = work(kvsynth.layer_kv(w, w.layer_begin + l))
        t_enc += te
        t_dec += td
        log(f"[cpu] 1 thread, layer {l}: encode {te:.2f}s decode {td:.2f}s")
    one = (kv_enc_layer + kv_dec_layer) * layers / (t_enc + t_dec) / 1e9
    # all threads: one layer each, all started together
    n = max(1, min(threads, w.compressed_layers))
    with ThreadPoolExecutor(min(n, 8)) as ex:
        inputs = list(ex.map(lambda l: kvsynth.layer_kv(w, w.layer_begin + l), range(n)))
    t0 = time.perf_counter()
    with ThreadPoolExecutor(n) as ex:
        parts = list(ex.map(work, inputs))
    wall = time.perf_counter() - t0
    del inputs
    many = (kv_enc_layer + kv_dec_layer) * n / wall / 1e9
    log(f"[cpu] {n} threads, {n} layers: {wall:.2f}s wall "
        f"(per-layer encode {np.mean([p[0] for p in parts]):.2f}s decode "
        f"{np.mean([p[1] for p in parts]):.2f}s)")
    return {
        "value": round(many, 4),
        "unit": "GB/s",
        "cores": n,
        "kind": "oracle",
        "sample": f"{n} of {w.compressed_layers} layers of the same workload, one layer per "
                  f"thread on {n} threads (score, evict, encode, decode per layer; the plain C "
                  f"oracle, inputs in host RAM, generation excluded); the 1-thread figure from "
                  f"{layers} layers one after another",
        "one_thread": {"value": round(one, 4), "cores": 1, "layers": layers,
                       "encode_GBps": round(kv_enc_layer * layers / t_enc / 1e9, 4),
                       "decode_GBps": round(kv_dec_layer * layers / t_dec / 1e9, 4)},
        "host_cpus": os.cpu_count(),
    }


def upload_workload(w, dev):
    """K, V [L, H, T, 128] fp16 on the device, generated on the host a few layers at a time."""
    import torch
    import kvsynth
    H, T = w.kv_heads, w.tokens
    K = torch.empty((w.layers, H, T, 128), dtype=torch.float16, device=dev)
    V = torch.empty_like(K)
    chunk = 4
    for l0 in range(0, w.layers, chunk):
        ls = list(range(l0, min(w.layers, l0 + chunk)))
        hk = np.empty((len(ls), H, T, 128), np.float16)
        hv = np.empty_like(hk)

        def one(i):
            hk[i], hv[i] = kvsynth.layer_kv(w, ls[i])
        with ThreadPoolExecutor(8) as ex:
            list(ex.map(one, range(len(ls))))
        K[l0:l0 + len(ls)].copy_(torch.from_numpy(hk))
        V[l0:l0 + len(ls)].copy_(torch.from_numpy(hv))
    torch.cuda.synchronize()
    return K, V


def attn_score(args):
    """The attention-weight scorer on the headline workload: 32 query heads (GQA 4) with a
    W-query observation window per head, two matrix-core passes over all keys, then the
    selection -- timed against the key-key proxy scorer on the same keys."""
    import torch
    import kv_cache_compression_proxy_amd as nq
    import kvsynth
    w = kvsynth.workload(args.workload)
    p = nq.make_params(w.layers, w.kv_heads, w.tokens, w.window, w.evict_permille, w.bits_k,
                       w.bits_v, w.rope_base, w.layer_begin, w.layer_end)
    Lc, H, T, W = w.compressed_layers, w.kv_heads, w.tokens, w.window
    Hq = 4 * H
    n = nq.nq_keep_count(p)
    dev = torch.device("cuda:0")
    log(f"[attn-score] workload {w.name}: Lc={Lc} H={H} Hq={Hq} T={T} W={W} n_keep={n}")
    K, V = upload_workload(w, dev)
    del V
    Qs = np.stack([kvsynth.window_queries(w, w.layer_begin + lc, q_heads=Hq) for lc in range(Lc)])
    Q = torch.from_numpy(Qs).to(dev)
    pos_a = torch.empty((Lc, n), dtype=torch.int32, device=dev)
    pos_k = torch.empty_like(pos_a)
    ws_a = nq.workspace(nq.nq_score_evict_attn_workspace_bytes(p, Hq), dev)
    ws_k = nq.workspace(nq.nq_score_evict_workspace_bytes(p), dev)
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    ms_a = timed(lambda: nq.nq_score_evict_attn(p, K, Q, Hq, pos_a, ws_a, stream=stream))
    ms_k = timed(lambda: nq.nq_score_evict(p, K, pos_k, ws_k, stream=stream))
    same = int((pos_a == pos_k).all(dim=1).sum().item())
    overlap = float(np.mean([len(set(pos_a[l].tolist()) & set(pos_k[l].tolist())) / n
                             for l in range(Lc)]))
    # two matrix-core passes over every (query row, key) pair of each (layer, kv head):
    # pass 1 over keys up to each row block's last position, pass 2 over the candidates
    R, c_end = 4 * W, T - W
    flop = 2.0 * Lc * H * R * 128 * (T + c_end)
    exps = 1.0 * Lc * H * R * (T + c_end)
    tflops = flop / (ms_a * 1e-3) / 1e12
    log(f"[attn-score] {ms_a:.3f} ms (key-key proxy {ms_k:.3f} ms); {tflops:.1f} TFLOP/s; "
        f"keep-set overlap with the proxy {overlap:.3f}")
    res = {
        "metric": "attention-weight scorer: candidate scores + eviction per step",
        "value": round(Lc * H * T * 256 / (ms_a * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_a, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 products, f32 sums",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": Lc, "kv_heads": H, "q_heads": Hq,
                   "tokens": T, "window": W, "n_keep": n, "parallelism": "none (1 GPU)"},
        "key_key_proxy_ms": round(ms_k, 4),
        "keep_overlap_with_proxy": round(overlap, 4),
        "layers_with_identical_keep_sets": same,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": 2500.0,
                     "unit": "TFLOP/s", "frac": round(tflops / 2500.0, 4), "traffic": None,
                     "kernel": "k_attn_rowbias+k_attn_colsum+k_attn_finish+k_select",
                     "algorithmic_flop_per_launch": flop, "exp2_per_launch": exps,
                     "avg_launch_ms": round(ms_a, 4)},
    }
    print(json.dumps(res), flush=True)


def scalar_baseline(args):
    """E8 codec vs the equal-bit Lloyd-Max scalar baseline on the same keep-set: encode and
    decode (fp16 out) times, and reconstruction quality (SNR, mean cosine against the original
    kept rows, fp32 reconstructions) on two sampled layers."""
    import torch
    import kv_cache_compression_proxy_amd as nq
    import kvsynth
    w = kvsynth.workload(args.workload)
    p = nq.make_params(w.layers, w.kv_heads, w.tokens, w.window, w.evict_permille, w.bits_k,
                       w.bits_v, w.rope_base, w.layer_begin, w.layer_end)
    Lc, H, T = w.compressed_layers, w.kv_heads, w.tokens
    n = nq.nq_keep_count(p)
    dev = torch.device("cuda:0")
    K, V = upload_workload(w, dev)
    cos, sin = nq.rope_table(p, dev)
    pos = torch.empty((Lc, n), dtype=torch.int32, device=dev)
    nq.nq_score_evict(p, K, pos, nq.workspace(nq.nq_score_evict_workspace_bytes(p), dev))
    ck = torch.empty((Lc, H, n, 128), dtype=torch.int8, device=dev)
    cv = torch.empty_like(ck)
    ik = torch.empty((Lc, H, n, 128), dtype=torch.uint8, device=dev)
    iv = torch.empty_like(ik)
    sk = torch.empty((Lc, H, n, 16), dtype=torch.float16, device=dev)
    sv, sk2, sv2 = torch.empty_like(sk), torch.empty_like(sk), torch.empty_like(sk)
    Ko = torch.empty((Lc, H, n, 128), dtype=torch.float16, device=dev)
    Vo = torch.empty_like(Ko)
    ws_d = nq.workspace(nq.nq_decode_workspace_bytes(p), dev)
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    t_e8_enc = timed(lambda: nq.nq_encode(p, K, V, pos, cos, sin, ck, cv, sk, sv, stream))
    t_e8_dec = timed(lambda: nq.nq_decode(p, ck, cv, sk, sv, pos, cos, sin, Ko, Vo,
                                          nq.NQ_OUT_F16, ws_d, stream))
    t_sc_enc = timed(lambda: nq.nq_encode_scalar(p, K, V, pos, cos, sin, ik, iv, sk2, sv2,
                                                 stream))
    t_sc_dec = timed(lambda: nq.nq_decode_scalar(p, ik, iv, sk2, sv2, pos, cos, sin, Ko, Vo,
                                                 nq.NQ_OUT_F16, stream))
    # quality on two sampled layers, fp32 reconstructions of every kept row
    q = {"E8": [0.0, 0.0, 0.0, 0.0, 0.0, 0.0], "LloydMax": [0.0, 0.0, 0.0, 0.0, 0.0, 0.0]}
    cosines = {"E8": [[], []], "LloydMax": [[], []]}
    for lc in (0, Lc - 1):
        pl = nq.make_params(1, H, T, w.window, w.evict_permille, w.bits_k, w.bits_v, w.rope_base)
        layer = w.layer_begin + lc
        Kl, Vl, Pl = K[layer:layer + 1], V[layer:layer + 1], pos[lc:lc + 1]
        orig = [Kl[0][:, Pl[0].long()].float(), Vl[0][:, Pl[0].long()].float()]
        Kf = torch.empty((1, H, n, 128), dtype=torch.float32, device=dev)
        Vf = torch.empty_like(Kf)
        nq.nq_decode(pl, ck[lc:lc + 1], cv[lc:lc + 1], sk[lc:lc + 1], sv[lc:lc + 1], Pl, cos,
                     sin, Kf, Vf, nq.NQ_OUT_F32, nq.workspace(nq.nq_decode_workspace_bytes(pl),
                                                              dev))
        Ks, Vs = torch.empty_like(Kf), torch.empty_like(Vf)
        nq.nq_decode_scalar(pl, ik[lc:lc + 1], iv[lc:lc + 1], sk2[lc:lc + 1], sv2[lc:lc + 1], Pl,
                            cos, sin, Ks, Vs, nq.NQ_OUT_F32)
        for name, rec in (("E8", [Kf[0], Vf[0]]), ("LloydMax", [Ks[0], Vs[0]])):
            for t_ in range(2):
                x, y = orig[t_].double(), rec[t_].double()
                q[name][2 * t_] += float((x * x).sum())
                q[name][2 * t_ + 1] += float(((x - y) ** 2).sum())
                cosines[name][t_].append(float(torch.nn.functional.cosine_similarity(
                    x, y, dim=-1).mean()))
    quality = {}
    for name in q:
        quality[name] = {
            "snr_db_k": round(10 * np.log10(q[name][0] / q[name][1]), 3),
            "snr_db_v": round(10 * np.log10(q[name][2] / q[name][3]), 3),
            "cos_k": round(float(np.mean(cosines[name][0])), 5),
            "cos_v": round(float(np.mean(cosines[name][1])), 5)}
    kv = Lc * H * n * 2 * 256
    log(f"[scalar] E8 encode {t_e8_enc:.3f} decode {t_e8_dec:.3f} ms; Lloyd-Max encode "
        f"{t_sc_enc:.3f} decode {t_sc_dec:.3f} ms; quality {quality}")
    res = {
        "metric": "equal-bit comparison: E8 codec vs Lloyd-Max scalar codec (same keep-set, "
                  "front end and fp16 group scales)",
        "value": round(quality["E8"]["snr_db_k"] - quality["LloydMax"]["snr_db_k"], 3),
        "unit": "dB (key SNR, E8 minus Lloyd-Max)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
        "vs_baseline": None, "data": "synthetic",
        "config": {"workload": w.name, "bits_k": w.bits_k, "bits_v": w.bits_v, "n_keep": n},
        "ms": {"e8_encode": round(t_e8_enc, 4), "e8_decode": round(t_e8_dec, 4),
               "lloydmax_encode": round(t_sc_enc, 4), "lloydmax_decode": round(t_sc_dec, 4)},
        "fp16_kv_GBps": {"e8_encode": round(kv / (t_e8_enc * 1e-3) / 1e9, 1),
                         "e8_decode": round(kv / (t_e8_dec * 1e-3) / 1e9, 1),
                         "lloydmax_encode": round(kv / (t_sc_enc * 1e-3) / 1e9, 1),
                         "lloydmax_decode": round(kv / (t_sc_dec * 1e-3) / 1e9, 1)},
        "quality_two_sampled_layers": quality,
    }
    print(json.dumps(res), flush=True)


def entropy_stage(args):
    """Measured post-entropy ratio of a full workload: the GPU compresses it (score, evict,
    encode), then the host zstd stage sizes the delta streams, scales and keep-set bitmaps of
    every compressed layer. Also reported: zstd of the absolute codes (no delta), the raw int8
    storage ratio, the closed-form nominal ratio, and the host stage's throughput."""
    import torch
    import kv_cache_compression_proxy_amd as nq
    from kv_cache_compression_proxy_amd import entropy
    import kvsynth
    w = kvsynth.workload(args.workload)
    dev = torch.device("cuda:0")
    K, V = upload_workload(w, dev)
    preset = {1: "balanced", 2: "max", 3: "high"}.get(args.workload, "balanced")
    c = nq.compress(K, V, preset, window=w.window, evict_permille=w.evict_permille,
                    bits_k=w.bits_k, bits_v=w.bits_v, rope_base=w.rope_base,
                    protect_boundary=w.protect_boundary)
    torch.cuda.synchronize()
    del K, V
    Lc, H, T, n = w.compressed_layers, w.kv_heads, w.tokens, c.n_keep
    t0 = time.perf_counter()
    tot = entropy.cache_ratio(c)
    dt = time.perf_counter() - t0
    # absolute codes (running sum of the deltas) of a few layers, for comparison
    abs_z = abs_raw = 0
    for lc in range(min(4, Lc)):
        for cc in (c.codes_k[lc], c.codes_v[lc]):
            a = torch.cumsum(cc.to(torch.int32), dim=1).to(torch.int8).cpu().numpy()
            abs_z += entropy.zstd_size(a)
            abs_raw += a.nbytes
    dz = 0
    for lc in range(min(4, Lc)):
        dz += entropy.zstd_size(c.codes_k[lc].cpu().numpy()) + \
            entropy.zstd_size(c.codes_v[lc].cpu().numpy())
    nominal = 4096.0 * H * T / (n * (H * (128 * (w.bits_k + w.bits_v) + 2 * 16 * 16) + 32))
    raw = tot["fp16_kv"] / (tot["codes_raw"] + tot["scales_raw"] + tot["keep_bitmap"])
    log(f"[entropy] {w.name}: zstd ratio {tot['ratio']:.2f} (raw {raw:.2f}, nominal "
        f"{nominal:.2f}); codes {tot['codes_ratio_zstd']:.2f}x; host stage {dt:.1f} s")
    res = {
        "metric": "post-entropy compression ratio of the compressed cache (host zstd level 3)",
        "value": round(tot["ratio"], 3),
        "unit": "x",
        "n_gpus": 1,
        "higher_is_better": True,
        "vs_baseline": None,
        "data": "synthetic",
        "config": {"workload": w.name, "preset": preset, "compressed_layers": Lc, "n_keep": n},
        "nominal_ratio": round(nominal, 3),
        "raw_int8_storage_ratio": round(raw, 3),
        "codes_zstd_ratio_delta": round(tot["codes_ratio_zstd"], 3),
        "codes_zstd_ratio_absolute_first4layers": round(abs_raw / abs_z, 3),
        "codes_zstd_ratio_delta_first4layers": round(abs_raw / dz, 3),
        "scales_zstd_ratio": round(tot["scales_raw"] / tot["scales_zstd"], 3),
        "bytes": {k: int(v) for k, v in tot.items() if k not in ("ratio", "codes_ratio_zstd")},
        "host_stage_s": round(dt, 2),
        "host_stage_MBps_of_codes_and_scales": round((tot["codes_raw"] + tot["scales_raw"]) /
                                                     dt / 1e6, 1),
        "zstd_version": entropy.zstd_version(),
    }
    print(json.dumps(res), flush=True)


def decode_step(args):
    """One-token GQA decode step over the long-context compressed cache (32 query heads over 8
    kv heads, one fp16 query per layer): the fused nq_decode_attend against the two-call path
    nq_decode (fp16 K_hat/V_hat written to HBM) + nq_attend_decode (read back)."""
    import torch
    import kv_cache_compression_proxy_amd as nq
    import kvsynth
    w4 = kvsynth.workload(4)
    w = kvsynth.workload(2)   # the cache the decode step attends over
    p = nq.make_params(w.layers, w.kv_heads, w.tokens, w.window, w.evict_permille, w.bits_k,
                       w.bits_v, w.rope_base, w.layer_begin, w.layer_end)
    Lc, H, T = w.compressed_layers, w.kv_heads, w.tokens
    n = nq.nq_keep_count(p)
    dev = torch.device("cuda:0")
    log(f"[decode-step] cache {w.name}: Lc={Lc} H={H} T={T} n_keep={n}, {w4.q_heads} query heads")
    t0 = time.time()
    K, V = upload_workload(w, dev)
    cos, sin = nq.rope_table(p, dev)
    positions = torch.empty((Lc, n), dtype=torch.int32, device=dev)
    nq.nq_score_evict(p, K, positions, nq.workspace(nq.nq_score_evict_workspace_bytes(p), dev))
    ck = torch.empty((Lc, H, n, 128), dtype=torch.int8, device=dev)
    cv = torch.empty_like(ck)
    sk = torch.empty((Lc, H, n, 16), dtype=torch.float16, device=dev)
    sv = torch.empty_like(sk)
    nq.nq_encode(p, K, V, positions, cos, sin, ck, cv, sk, sv)
    torch.cuda.synchronize()
    del K, V
    torch.cuda.empty_cache()
    log(f"[decode-step] compressed cache built in {time.time() - t0:.1f}s")
    if args.copy_calibration:   # the copy whose counters calibrate a --pmc run
        src = torch.ones(args.copy_calibration << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    Hq = w4.q_heads
    Q = torch.from_numpy(kvsynth.queries(w4)).to(dev)
    out = torch.empty((Lc, Hq, 128), dtype=torch.float32, device=dev)
    ws_f = nq.workspace(nq.nq_decode_attend_workspace_bytes(p, Hq), dev)
    Ko = torch.empty((Lc, H, n, 128), dtype=torch.float16, device=dev)
    Vo = torch.empty_like(Ko)
    ws_d = nq.workspace(nq.nq_decode_workspace_bytes(p), dev)
    ws_a = nq.workspace(nq.nq_attend_workspace_bytes(p, Hq, n), dev)
    out2 = torch.empty_like(out)
    stream = torch.cuda.current_stream()

    def fused():
        nq.nq_decode_attend(p, ck, cv, sk, sv, positions, cos, sin, Q, Hq, out, ws_f, stream)

    def two_call(ev=None):
        nq.nq_decode(p, ck, cv, sk, sv, positions, cos, sin, Ko, Vo, nq.NQ_OUT_F16, ws_d, stream)
        if ev is not None:
            ev.record(stream)
        nq.nq_attend_decode(p, Q, Hq, Ko, Vo, n, out2, ws_a, stream)

    def timed(fn, mid=False):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        mids = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        a.record(stream)
        for i in range(args.steps):
            starts[i].record(stream)
            fn(mids[i]) if mid else fn()
        b.record(stream)
        torch.cuda.synchronize()
        first = sum(s.elapsed_time(m) for s, m in zip(starts, mids)) / args.steps if mid else None
        return a.elapsed_time(b) / args.steps, first

    ms_f, _ = timed(fused)
    ms_2, ms_dec = timed(two_call, mid=True)
    diff = (out - out2).abs().max().item() / max(Vo.float().abs().max().item(), 1e-30)
    log(f"[decode-step] fused {ms_f:.3f} ms; two-call {ms_2:.3f} ms (decode {ms_dec:.3f}); "
        f"max |fused - two-call| / max|v_hat| = {diff:.2e}")
    kept = Lc * H * n
    kv16 = kept * 2 * 256                                  # fp16 K+V the step attends over
    alg_f = kept * (2 * 128 + 2 * 32) + Lc * n * 4 + T * 64 * 4 * 2 + Lc * Hq * (256 + 512)
    alg_2 = kept * (2 * 128 + 2 * 32 + 2 * 256) * 1 + kept * 2 * 256 + Lc * n * 4 + T * 512
    alg_dec = kept * (2 * 128 + 2 * 32 + 2 * 256) + Lc * n * 4 + T * 512
    achieved = alg_f / (ms_f * 1e-3) / 1e9
    res = {
        "metric": "one-token GQA decode step over the compressed cache: fp16-KV GB/s attended",
        "value": round(kv16 / (ms_f * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_f, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w4.name, "cache": w.name, "layers": Lc, "kv_heads": H,
                   "q_heads": Hq, "tokens": T, "n_keep": n, "parallelism": "none (1 GPU)"},
        "two_call_ms": round(ms_2, 4),
        "two_call_decode_ms": round(ms_dec, 4),
        "speedup_vs_two_call": round(ms_2 / ms_f, 3),
        "two_call_value": round(kv16 / (ms_2 * 1e-3) / 1e9, 2),
        "max_abs_diff_vs_two_call_rel": float(f"{diff:.3e}"),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": read_traffic(args.traffic or traffic_path(w, decode_step=True),
                                             "decode_attend"),
                     "kernel": "+".join(DECODE_STEP_KERNELS["decode_attend"]),
                     "algorithmic_bytes_per_launch": alg_f, "avg_launch_ms": round(ms_f, 4)},
        "two_call_algorithmic_frac_of_peak": round(alg_2 / (ms_2 * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                                   4),
        # nq_decode alone on this cache (the decode direction of the long-context workload):
        # codes + scales in, fp16 K/V out
        "decode_only": {
            "ms": round(ms_dec, 4),
            "fp16_KV_GBps": round(kv16 / (ms_dec * 1e-3) / 1e9, 2),
            "algorithmic_bytes": alg_dec,
            "algorithmic_frac_of_peak": round(alg_dec / (ms_dec * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        },
    }
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for "
              f"--gpus {args.gpus}). The hot path shards by layer with no communication; run "
              f"with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import kvsynth
    w = kvsynth.workload(args.workload)
    if args.summarize_trace:
        summarize_trace(args)
        return
    if args.summarize_counters:
        summarize_counters(args)
        return
    if args.summarize_pmc:
        if args.decode_step:
            summarize_pmc(args, kvsynth.workload(2), decode_step=True)
        else:
            summarize_pmc(args, w)
        return
    if args.decode_step:
        decode_step(args)
        return
    if args.attn_score:
        attn_score(args)
        return
    if args.entropy:
        entropy_stage(args)
        return
    if args.scalar:
        scalar_baseline(args)
        return
    import torch
    import kv_cache_compression_proxy_amd as nq

    p = nq.make_params(w.layers, w.kv_heads, w.tokens, w.window, w.evict_permille, w.bits_k,
                       w.bits_v, w.rope_base, w.layer_begin, w.layer_end)
    Lc, H, T = w.compressed_layers, w.kv_heads, w.tokens
    n_keep = nq.nq_keep_count(p)
    dev = torch.device("cuda:0")
    log(f"[bench] workload {w.name}: Lc={Lc} H={H} T={T} n_keep={n_keep}")

    t0 = time.time()
    K, V = upload_workload(w, dev)
    log(f"[bench] inputs generated and uploaded in {time.time() - t0:.1f}s")

    if args.copy_calibration:
        src = torch.ones(args.copy_calibration << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cos, sin = nq.rope_table(p, dev)
    positions = torch.empty((Lc, n_keep), dtype=torch.int32, device=dev)
    ws_s = nq.workspace(nq.nq_score_evict_workspace_bytes(p), dev)
    ck = torch.empty((Lc, H, n_keep, 128), dtype=torch.int8, device=dev)
    cv = torch.empty_like(ck)
    sk = torch.empty((Lc, H, n_keep, 16), dtype=torch.float16, device=dev)
    sv = torch.empty_like(sk)
    Ko = torch.empty((Lc, H, n_keep, 128), dtype=torch.float16, device=dev)
    Vo = torch.empty_like(Ko)
    ws_d = nq.workspace(nq.nq_decode_workspace_bytes(p), dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        nq.nq_score_evict(p, K, positions, ws_s, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        nq.nq_encode(p, K, V, positions, cos, sin, ck, cv, sk, sv, stream)
        if ev is not None:
            ev[2].record(stream)
        nq.nq_decode(p, ck, cv, sk, sv, positions, cos, sin, Ko, Vo, nq.NQ_OUT_F16, ws_d, stream)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = start.elapsed_time(end) / args.steps
    phase = {"score_evict": 0.0, "encode": 0.0, "decode": 0.0}
    for e in evs:
        phase["score_evict"] += e[0].elapsed_time(e[1])
        phase["encode"] += e[1].elapsed_time(e[2])
        phase["decode"] += e[2].elapsed_time(e[3])
    phase = {k: v / args.steps for k, v in phase.items()}
    log(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step (wall {wall / args.steps * 1e3:.3f}); "
        f"phases ms: " + ", ".join(f"{k} {v:.3f}" for k, v in phase.items()))

    # the achievable line: torch's device copy of 1 GiB (1 GiB read + 1 GiB written); not in
    # counter runs, whose copy dispatches calibrate the byte counters
    copy_gbps = None
    if not args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(20):
            dst.copy_(src)
        c1.record(stream)
        torch.cuda.synchronize()
        copy_gbps = round(2 * (1 << 30) / (c0.elapsed_time(c1) / 20 * 1e-3) / 1e9, 1)
        del src, dst

    kv_enc = Lc * H * T * 256 * 2
    kv_dec = Lc * H * n_keep * 256 * 2
    value = (kv_enc + kv_dec) / (ms_step * 1e-3) / 1e9
    alg = algorithmic_bytes(w, n_keep)
    dom = max(phase, key=phase.get)
    achieved = alg[dom] / (phase[dom] * 1e-3) / 1e9
    traffic = read_traffic(args.traffic or traffic_path(w), dom)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": "+".join(PHASE_KERNELS[dom]), "algorithmic_bytes_per_launch": alg[dom],
                "avg_launch_ms": round(phase[dom], 4),
                "traffic_GBps": (None if traffic is None
                                 else round(traffic / (phase[dom] * 1e-3) / 1e9, 1))}
    out = {
        "metric": "encode/decode fp16-KV GB/s on 1 MI355X; % of HBM peak",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": w.layers, "kv_heads": H, "tokens": T,
                   "head_dim": 128, "window": w.window, "evict_permille": w.evict_permille,
                   "bits_k": w.bits_k, "bits_v": w.bits_v, "rope_base": w.rope_base,
                   "compressed_layers": Lc, "n_keep": n_keep, "parallelism": "none (1 GPU)"},
        "encode_GBps": round(kv_enc / ((phase["score_evict"] + phase["encode"]) * 1e-3) / 1e9, 2),
        "decode_GBps": round(kv_dec / (phase["decode"] * 1e-3) / 1e9, 2),
        "phase_ms": {k: round(v, 4) for k, v in phase.items()},
        "algorithmic_frac_of_peak": {
            k: round(alg[k] / (phase[k] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4) for k in phase},
        "step_algorithmic_frac_of_peak": round(sum(alg.values()) / (ms_step * 1e-3) / 1e9
                                               / HBM_PEAK_GBPS, 4),
        "copy_GBps_torch": copy_gbps,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, min(args.cpu_layers, Lc), args.cpu_threads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
