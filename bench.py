"""Benchmark: accepted tokens/s of layer-parallel speculative decoding at
batch 1 on one MI355X, with draft-step and verify HBM rooflines.

Workload (default): Llama-3.2-1B-shaped draft (16 layers, d 2048, 32/8 heads,
ffn 8192) with a Llama-3-8B-shaped base (32 layers, d 4096, 32/8 heads, ffn
14336), bf16, vocab 128256, N(0, 0.02) random-init weights; 512-token seeded
uniform-random prompt; k = 5 draft tokens per round; layer-parallel set size
N = 2 (paper plan); batch 1; greedy.

A step is one speculative round: k-1 layer-parallel draft steps, the k+1-token
base verification, accept / resample, and the calibration pass.  `value` is
committed tokens per second over the K timed rounds (inputs and KV resident in
HBM).  Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFS = 2500.0   # dense bf16 matrix-core peak (MI355X published)


PROBE_COPY_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "pmc_traffic.md")


def kernel_source_hash():
    """sha256 over the HIP sources, so stored counter figures are used only
    for the kernels they were taken on."""
    import hashlib
    d = os.path.join(os.path.dirname(os.path.abspath(__file__)), "layer_speculative_decoding_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(d, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def stored_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    or None if there is none for it or the kernels changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            lines = [line.strip() for line in f]
    except OSError:
        return None
    sha = [ln.split(": ", 1)[1] for ln in lines if ln.startswith("source_sha256: ")]
    if not sha or sha[0] != kernel_source_hash():
        return None
    for i, ln in enumerate(lines[:-1]):
        if ln == f"kernel: {kernel}" and lines[i + 1].startswith("traffic_bytes_per_launch: "):
            return int(lines[i + 1].split(": ", 1)[1])
    return None


def pmc_summary(fetch_csv, write_csv, kernels, command):
    """Markdown summary of two counter runs (FETCH_SIZE, WRITE_SIZE; KiB per
    dispatch) of `bench.py --pmc-probe`: each counter is scaled by what it
    reads for the probe's device copy of PROBE_COPY_BYTES, then averaged over
    the dispatches of each kernel in `kernels`."""
    import csv

    def load(path, counter, kernel):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        copy = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]][-1]
        factor = PROBE_COPY_BYTES / 1024 / copy
        vals = [float(r["Counter_Value"]) for r in rows if kernel + "(" in r["Kernel_Name"]]
        return copy, factor, vals

    print(f"# HBM traffic of {', '.join(kernels)} (hardware counters)")
    print()
    print("Commands (from the repository root, TMPDIR=/tmp):")
    print()
    for c in command:
        print(f"    {c}")
    print()
    fc, ff, _ = load(fetch_csv, "FETCH_SIZE", kernels[0])
    wc, wf, _ = load(write_csv, "WRITE_SIZE", kernels[0])
    print(f"Calibration: the probe's device copy of {PROBE_COPY_BYTES} bytes reads FETCH_SIZE {fc:.1f} KiB and "
          f"WRITE_SIZE {wc:.1f} KiB, so the counters are scaled by {ff:.4f} (fetch) and {wf:.4f} (write).")
    print()
    print(f"| kernel | counter | dispatches | raw avg KiB | scaled avg bytes |")
    print(f"|---|---|---|---|---|")
    totals = []
    for kernel in kernels:
        _, _, fv = load(fetch_csv, "FETCH_SIZE", kernel)
        _, _, wv = load(write_csv, "WRITE_SIZE", kernel)
        fetch = sum(fv) / len(fv) * ff * 1024
        write = sum(wv) / len(wv) * wf * 1024
        print(f"| {kernel} | FETCH_SIZE | {len(fv)} | {sum(fv) / len(fv):.1f} | {fetch:.0f} |")
        print(f"| {kernel} | WRITE_SIZE | {len(wv)} | {sum(wv) / len(wv):.1f} | {write:.0f} |")
        totals.append((kernel, int(round(fetch + write))))
    print()
    for kernel, t in totals:
        print(f"kernel: {kernel}")
        print(f"traffic_bytes_per_launch: {t}")
    print(f"source_sha256: {kernel_source_hash()}")


def mfma_profile_name(cfg):
    """File name of a workload's matrix-core utilisation summary under profiles/."""
    return "mfma_util.md" if cfg.name == "llama-1b-8b" else f"mfma_util_{cfg.name}.md"


def pmc_mfma_summary(csv_path, command, cfg):
    """Markdown summary of one counter run of `bench.py --pmc-probe` with the
    matrix-core counters: per kernel family, the matrix-core flops the
    hardware counted (MOPS x 512), the dispatch durations (the run's own
    timestamps; counter runs serialise dispatches) and the MFMA-busy share of
    the SIMDs: SQ_VALU_MFMA_BUSY_CYCLES / (active cycles x 1024 SIMDs), where
    the active cycles are GRBM_GUI_ACTIVE / 8 (the CSV value sums the eight
    XCDs' GRBM instances; per XCD it tracks the dispatch's duration at the
    shader clock)."""
    import csv
    import re
    disp = {}
    for r in csv.DictReader(open(csv_path)):
        d = disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"],
                                                    "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    fam = {}
    for d in disp.values():
        m = re.search(r"(k_\w+)<([^()]*)>\(", d["name"])
        if not m:
            continue
        key = f"{m.group(1)}<{m.group(2)}>"
        f = fam.setdefault(key, {"n": 0, "ns": 0.0, "bf16": 0.0, "f32": 0.0, "busy": 0.0, "gui": 0.0})
        f["n"] += 1
        f["ns"] += d["ns"]
        f["bf16"] += d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
        f["f32"] += d.get("SQ_INSTS_VALU_MFMA_MOPS_F32", 0.0) * 512
        f["busy"] += d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        f["gui"] += d.get("GRBM_GUI_ACTIVE", 0.0)
    print("# Matrix-core utilisation per kernel (hardware counters)")
    print()
    print("Commands (from the repository root, TMPDIR=/tmp):")
    print()
    for c in command:
        print(f"    {c}")
    print()
    B, P = cfg.batch, cfg.prompt_len
    print(f"The run covers the {cfg.name} workload ({B} sequence{'s' if B > 1 else ''} of {P} prompt tokens, "
          f"k = {cfg.k}, N = {cfg.group_size}): three prompt prefills (base {P - 1} rows, draft {P} rows per "
          f"sequence, {'all sequences in one call; ' if B > 1 else ''}products on k_gemm_tile, attention on "
          "k_attn_prompt), then the warm-up and three probe rounds: draft steps, verify and calibration on "
          "k_gemv, k_gemm_mfma or k_gemm_tile by their row count, attention on k_attn (bf16 matrix "
          "instructions on the bf16 caches; q and the probabilities enter them as two bf16 pieces in both "
          "attention kernels).  Flops are what the matrix cores executed (padding rows and both pieces "
          "included); the bf16 peak is 2500 TFLOP/s, the float32 one 157.3.")
    print()
    top, ft = max(fam.items(), key=lambda kv: kv[1]["ns"])
    print(f"GRBM_GUI_ACTIVE / 8 per ns of `{top}` (the longest-running kernel): {ft['gui'] / 8 / ft['ns']:.2f} GHz.")
    print()
    print("| kernel | dispatches | avg us | MFMA bf16 TFLOP/s | of bf16 peak | MFMA f32 TFLOP/s | MFMA busy |")
    print("|---|---|---|---|---|---|---|")
    for key, f in sorted(fam.items(), key=lambda kv: -kv[1]["ns"]):
        sec = f["ns"] * 1e-9
        bf, f32 = f["bf16"] / sec / 1e12, f["f32"] / sec / 1e12
        busy = f["busy"] / (f["gui"] / 8 * 1024) if f["gui"] else 0.0
        print(f"| `{key}` | {f['n']} | {f['ns'] / f['n'] / 1e3:.1f} | {bf:.1f} | {bf / MFMA_BF16_PEAK_TFS:.1%} | "
              f"{f32:.2f} | {busy:.1%} |")


def profile_name(cfg):
    """File name of a workload's kernel-statistics summary under profiles/."""
    return f"kernel_stats_{cfg.name}_k{cfg.k}_N{cfg.group_size}" + (f"_B{cfg.batch}" if cfg.batch > 1 else "") + ".md"


def rocprof_summary(stats_csv, trace_csv, command, cfg):
    """Markdown summary of a `rocprofv3 --kernel-trace --stats` run of a
    workload: the per-kernel statistics, then the kernels of one steady-state
    round split into its phases (a round runs calibration, the draft steps,
    verify, accept; every calibration and draft step ends with
    k_sample_reduce, accept starts with k_acc_stats)."""
    import collections
    import csv

    def short(n):
        n = n.replace("spec::(anonymous namespace)::", "").replace("void ", "")
        return n.split("(spec::")[0].split("(float const")[0][:70]

    rows = list(csv.DictReader(open(stats_csv)))
    def shape(sh):
        return (f"{sh.n_layers}-layer d{sh.d_model} ({sh.n_q_heads} q / {sh.n_kv_heads} kv heads of {sh.head_dim}, "
                f"ffn {sh.d_ffn}{', QKV bias' if sh.qkv_bias else ''})")

    print(f"# rocprofv3 kernel statistics: {cfg.name} workload")
    print()
    print(f"Workload: draft {shape(cfg.draft)} -> base {shape(cfg.base)}, "
          f"{'bf16' if cfg.base.dtype == 1 else 'float32'}, vocab {cfg.base.vocab}, {cfg.prompt_len}-token prompt, "
          f"k = {cfg.k}, layer-parallel set size N = {cfg.group_size}, batch {cfg.batch}, greedy; the prompt "
          "prefills (k_gemm_tile), the warm-up, timed and instrumented rounds of the command below, and the "
          "weight generation (the at::native kernels).  Template arguments: k_gemm_mfma<row tiles, epilogue, "
          "waves per block, K in segments>, "
          "k_gemv<type, rows, epilogue, operand mode>, k_gemm_tile<epilogue, 32-row weight blocks, K split, "
          "32-row activation blocks>; "
          "epilogues 0 store, 1 QKV RoPE + KV append, 2 SiLU gate, 3 residual add, 4 logits + arg-max, "
          "5 attention-output routing.")
    print()
    print("Commands (from the repository root, TMPDIR=/tmp):")
    print()
    for c in command:
        print(f"    {c}")
    print()
    print("Source: run_kernel_stats.csv (durations in microseconds).")
    print()
    print("| kernel | calls | avg us | min us | max us | total ms | % |")
    print("|---|---|---|---|---|---|---|")
    for r in rows[:24]:
        print(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
              f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
              f"{float(r['TotalDurationNs']) / 1e6:.2f} | {float(r['Percentage']):.1f} |")
    tr = list(csv.DictReader(open(trace_csv)))
    tr.sort(key=lambda r: int(r["Start_Timestamp"]))
    def dims(r, key):
        return [int(r.get(f"{key}_{a}", 1) or 1) for a in "XYZ"]

    def grid(r):
        # workgroups per dimension x threads per workgroup, e.g. (1, 16, 5) x 256
        g, w = dims(r, "Grid_Size"), dims(r, "Workgroup_Size")
        wg = tuple(gi // max(wi, 1) for gi, wi in zip(g, w))
        blk = w[0] * w[1] * w[2]
        return (f"{wg[0]}" if wg[1:] == (1, 1) else f"({wg[0]}, {wg[1]}, {wg[2]})"), blk
    ks = [(short(r["Kernel_Name"]), int(r["Start_Timestamp"]), int(r["End_Timestamp"])) + grid(r) for r in tr]
    idx = [i for i, r in enumerate(ks) if r[0] == "k_acc_stats"]
    seg = ks[idx[-2]:idx[-1]]
    sr = [i for i, r in enumerate(seg) if r[0] == "k_sample_reduce"]
    per = f" per sequence, {cfg.batch} sequences" if cfg.batch > 1 else ""
    phases = {f"calibration (a + 1 rows{per}: 1 at acceptance 0)": seg[3:sr[0] + 1],
              f"one draft step (1 row{per})": seg[sr[0] + 1:sr[1] + 1],
              f"verify (k + 1 = {cfg.k + 1} rows{per})": seg[sr[-1] + 1:]}
    print()
    print("One steady-state round from run_kernel_trace.csv (the last instrumented round; busy = sum of kernel "
          "durations, which excludes the profiler's own dispatch gaps):")
    for name, st in phases.items():
        busy = sum(r[2] - r[1] for r in st) / 1e3
        print()
        print(f"**{name}**: {len(st)} kernels, busy {busy:.1f} us")
        print()
        print("| kernel | workgroups x threads | launches | total us | avg us |")
        print("|---|---|---|---|---|")
        agg = collections.defaultdict(lambda: [0, 0.0])
        for r in st:
            key = (r[0], f"{r[3]} x {r[4]}")
            agg[key][0] += 1
            agg[key][1] += (r[2] - r[1]) / 1e3
        for k, v in sorted(agg.items(), key=lambda x: -x[1][1])[:10]:
            print(f"| {k[0]} | {k[1]} | {v[0]} | {v[1]:.1f} | {v[1] / v[0]:.2f} |")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def draft_step_bytes(sh, ctx):
    """Algorithmic HBM bytes of one draft step (batch 1): every weight byte
    read once (layers + lm head; the embedding row is negligible) plus the KV
    read at context ctx."""
    es = 2 if sh.dtype == 1 else 4
    d, L = sh.d_model, sh.n_layers
    per_layer = sh.qkv_rows * d + d * sh.q_dim + 3 * sh.d_ffn * d
    w = (L * per_layer + sh.vocab * d) * es
    kv = 2 * L * sh.n_kv_heads * sh.head_dim * es * ctx
    return w + kv


def verify_bytes(sh, ctx):
    return draft_step_bytes(sh, ctx)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="llama-1b-8b")
    ap.add_argument("--temperature", type=float, default=0.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-vanilla", action="store_true")
    ap.add_argument("--group-size", type=int, default=0,
                    help="layer-parallel set size N of the default plan (0: the workload's own)")
    ap.add_argument("--plan", default="",
                    help="explicit layer-parallel plan as comma-separated stage offsets (0, ..., n_layers), "
                         "for ablations of the plan reading; overrides --group-size")
    ap.add_argument("--separate-calibration", action="store_true",
                    help="ablation: the other reading of the calibration (all k drafts from fuzzy steps, then a "
                         "precise pass over the committed fuzzy tokens)")
    ap.add_argument("--mlp-parallel", action="store_true",
                    help="the parallel reading of the set's MLPs (every MLP fed from the set input; the set's "
                         "gate/up and down projections as one product each)")
    ap.add_argument("--no-calibration", action="store_true",
                    help="ablation: keep the fuzzy KV of accepted drafts, run only the emitted token precisely")
    ap.add_argument("--n1-compare", action="store_true",
                    help="also run the timed rounds with the sequential draft plan (N = 1) and report its "
                         "acceptance and tokens/s")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="run a few rounds and one device copy of known size, for hardware-counter runs")
    ap.add_argument("--pmc-summary", nargs="+", metavar="FETCH_CSV WRITE_CSV KERNEL",
                    help="print the traffic summary of two counter runs of --pmc-probe for one or more kernels")
    ap.add_argument("--pmc-mfma-summary", metavar="CSV",
                    help="print the matrix-core utilisation summary of a counter run of --pmc-probe")
    ap.add_argument("--rocprof-summary", nargs=2, metavar=("STATS_CSV", "TRACE_CSV"),
                    help="print the kernel statistics and one round's phases of a kernel-trace run")
    ap.add_argument("--rocprof-timeout", type=int, default=300,
                    help="the time limit of the summarised profiler run, as quoted in the summary")
    args = ap.parse_args()
    # the profiler's output directory of a summarised run: where its CSV is
    odir = lambda path: os.path.dirname(path) or "."
    if args.rocprof_summary:
        # describes the profiled run: the same --config / --steps / --warmup
        from synth import get_config as _cfg
        st, tr = args.rocprof_summary
        cfg = _cfg(args.config)
        run = (f"--config {args.config} " if args.config != "llama-1b-8b" else "") + \
            f"--steps {args.steps} --warmup {args.warmup}"
        rocprof_summary(st, tr, [
            f"timeout -k 10 {args.rocprof_timeout} rocprofv3 --kernel-trace --stats --output-format csv "
            f"-d {odir(st)} -o run "
            f"-- python bench.py {run} --no-cpu-baseline --no-vanilla",
            f"python bench.py {run}" + (f" --rocprof-timeout {args.rocprof_timeout}" if args.rocprof_timeout != 300
                                        else "") + f" --rocprof-summary {st} {tr} > profiles/{profile_name(cfg)}"],
                        cfg)
        return
    if args.pmc_mfma_summary:
        from synth import get_config as _cfg
        cfg = _cfg(args.config)
        cf = f"--config {args.config} " if args.config != "llama-1b-8b" else ""
        pmc_mfma_summary(args.pmc_mfma_summary, [
            f"timeout -s KILL {args.rocprof_timeout if cf else 240} rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 "
            "SQ_INSTS_VALU_MFMA_MOPS_F32 "
            f"SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE --output-format csv -d {odir(args.pmc_mfma_summary)} -o run "
            f"-- python bench.py {cf}--warmup 1 --pmc-probe",
            f"python bench.py {cf}" + (f"--rocprof-timeout {args.rocprof_timeout} " if cf else "") +
            f"--pmc-mfma-summary {args.pmc_mfma_summary} > profiles/{mfma_profile_name(cfg)}"], cfg)
        return
    if args.pmc_summary:
        if len(args.pmc_summary) < 3:
            ap.error("--pmc-summary needs FETCH_CSV WRITE_CSV KERNEL [KERNEL ...]")
        f, w, knames = args.pmc_summary[0], args.pmc_summary[1], args.pmc_summary[2:]
        kname = "' '".join(knames)
        pmc_summary(f, w, knames, [
            f"timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --output-format csv -d {odir(f)} -o run "
            "-- python bench.py --warmup 1 --pmc-probe",
            f"timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE --output-format csv -d {odir(w)} -o run "
            "-- python bench.py --warmup 1 --pmc-probe",
            f"python bench.py --pmc-summary {f} {w} '{kname}' > profiles/pmc_traffic.md"])
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer-parallel path here "
              f"is a single-GPU build", file=sys.stderr)
        sys.exit(2)

    import torch
    from layer_speculative_decoding_amd import api
    from layer_speculative_decoding_amd.runtime import SpecDecoder, VanillaDecoder
    from synth import get_config, make_prompts, make_weights

    cfg = get_config(args.config)
    if cfg.batch != 1:
        log("note: this config has batch", cfg.batch)
    K, W = args.steps, args.warmup
    k = cfg.k
    dev = "cuda"
    torch.cuda.init()
    log(f"config {cfg.name}: generating weights on the GPU")
    t0 = time.time()
    dw = make_weights(cfg.draft, cfg.seed_draft, device=dev)
    bw = make_weights(cfg.base, cfg.seed_base, device=dev)
    torch.cuda.synchronize()
    log(f"  weights ready in {time.time() - t0:.1f}s")
    N = args.group_size or cfg.group_size
    offs = api.spec_default_group_plan(cfg.draft.n_layers, N)
    if args.plan:
        offs = [int(x) for x in args.plan.split(",")]
        if offs[0] != 0 or offs[-1] != cfg.draft.n_layers or any(b <= a for a, b in zip(offs, offs[1:])):
            ap.error(f"--plan must be increasing stage offsets from 0 to {cfg.draft.n_layers}")
    seq_offs = list(range(cfg.draft.n_layers + 1))      # every layer its own stage (N = 1)
    P = cfg.prompt_len
    rounds_cap = W + K + 4
    cap = P + rounds_cap * (k + 1) + k + 2
    cap = max(cap, P + 64 + 2 * k + 4)     # the fixed-context draft step and calibration at P + 64
    prompts = make_prompts(cfg.draft.vocab, P, cfg.batch, cfg.prompt_seed)
    inv_t = 0.0 if args.temperature == 0 else 1.0 / args.temperature
    mlp_mode = 1 if args.mlp_parallel else 0
    dec = SpecDecoder(cfg.draft, dw, cfg.base, bw, cfg.batch, cap, k, offs, P, inv_t, cfg.sample_seed,
                      mlp_mode=mlp_mode, calibrate=not args.no_calibration, separate=args.separate_calibration)

    ev = lambda: torch.cuda.Event(enable_timing=True)
    e0, e1 = ev(), ev()
    dec.prefill(prompts)                  # first call: code objects load
    torch.cuda.synchronize()
    e0.record()
    dec.prefill(prompts)                  # idempotent: rewrites the same KV
    e1.record()
    torch.cuda.synchronize()
    prefill_ms = e0.elapsed_time(e1)
    log(f"  prefill (base {P - 1} + draft {P} tokens): {prefill_ms:.1f} ms")
    # instrumented prefill: tiled matrix-core products' flops and launch time
    api.spec_profile_reset()
    api.spec_profile_enable(True)
    dec.prefill(prompts)
    torch.cuda.synchronize()
    api.spec_profile_enable(False)
    pprof = api.spec_profile_collect()
    tiled = {n: v for n, v in pprof.items() if n.startswith("k_gemm_tile")}
    pf_ms = sum(v[1] for v in tiled.values())
    pf_fl = sum(v[3] for v in tiled.values())
    pf_tfs = pf_fl / (pf_ms * 1e-3) / 1e12 if pf_ms > 0 else 0.0
    attn_ms = sum(v[1] for n, v in pprof.items() if n.startswith("k_attn"))
    log(f"  prefill products: {pf_fl / 1e12:.2f} TFLOP in {pf_ms:.1f} ms -> {pf_tfs:.0f} TFLOP/s "
        f"({pf_tfs / MFMA_BF16_PEAK_TFS:.1%} of bf16 peak); attention {attn_ms:.1f} ms")
    for name, (n, t, by, fl) in sorted(pprof.items(), key=lambda kv: -kv[1][1]):
        log(f"    {name:34s} {n:5d} launches {t / n * 1e3:8.1f} us avg {fl / (t * 1e-3) / 1e12:7.1f} TFLOP/s")

    big = 1 << 30
    for _ in range(W):
        dec.step(big)
    torch.cuda.synchronize()
    if args.pmc_probe:
        # rounds of the timed mix, then a plain device copy of PROBE_COPY_BYTES
        # (read once, written once) that calibrates the byte counters
        for _ in range(3):
            dec.step(big)
        src = torch.ones(PROBE_COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"  probe: 3 rounds and one {PROBE_COPY_BYTES} byte device copy")
        return

    # timed region: K whole rounds; phase events recorded on the same stream
    n_before = sum(len(o) for o in dec.out)
    ph = {"draft": [], "verify": [], "accept": [], "calib": []}
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(K):
        marks = [ev() for _ in range(5)]
        dec.step(big, marks)
        ph["draft"].append((marks[0], marks[1]))
        ph["verify"].append((marks[1], marks[2]))
        ph["accept"].append((marks[2], marks[3]))
        ph["calib"].append((marks[3], marks[4]))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    tokens = sum(len(o) for o in dec.out) - n_before
    ms = {key: float(np.mean([a.elapsed_time(b) for a, b in v])) for key, v in ph.items()}
    acc_rate = (tokens - K * cfg.batch) / (K * cfg.batch * k)
    ctx = P + (W + K // 2) * (1 + acc_rate * k)
    # draft steps per round: k-1 (the calibration yields d_1), k with the
    # separate-pass calibration
    n_dsteps = k if args.separate_calibration else max(k - 1, 1)
    d_step_ms = ms["draft"] / n_dsteps
    d_bytes = draft_step_bytes(cfg.draft, ctx)
    v_bytes = verify_bytes(cfg.base, ctx)
    d_gbs = d_bytes / (d_step_ms * 1e-3) / 1e9
    v_gbs = v_bytes / (ms["verify"] * 1e-3) / 1e9
    value = tokens / elapsed
    log(f"  {K} rounds: {tokens} tokens in {elapsed * 1e3:.1f} ms -> {value:.1f} tok/s; "
        f"acceptance {acc_rate:.3f}")
    log(f"  phases (ms/round): " + ", ".join(f"{a} {b:.3f}" for a, b in ms.items()))
    log(f"  draft step {d_step_ms * 1e3:.0f} us, {d_gbs:.0f} GB/s ({d_gbs / HBM_PEAK_GBS:.1%} of 8 TB/s); "
        f"verify {ms['verify'] * 1e3:.0f} us, {v_gbs:.0f} GB/s")

    # instrumented pass: per-kernel-instance launch durations (HIP events on
    # the launch stream) and algorithmic bytes, for the dominant kernel's
    # roofline; kept apart from the timed region above
    api.spec_profile_reset()
    api.spec_profile_enable(True)
    for _ in range(max(2, min(K, 5))):
        dec.step(big)
    torch.cuda.synchronize()
    api.spec_profile_enable(False)
    prof = api.spec_profile_collect()
    dom = max(prof.items(), key=lambda kv: kv[1][1])
    dom_name, (dom_n, dom_ms, dom_bytes, _) = dom
    dom_gbs = dom_bytes / (dom_ms * 1e-3) / 1e9
    traffic = stored_traffic(dom_name)
    log(f"  dominant kernel {dom_name}: {dom_n} launches, avg {dom_ms / dom_n * 1e3:.1f} us, "
        f"{dom_bytes / dom_n / 1e6:.1f} MB/launch, {dom_gbs:.0f} GB/s")
    for name, (n, t, by, fl) in sorted(prof.items(), key=lambda kv: -kv[1][1]):
        log(f"    {name:34s} {n:5d} launches {t / n * 1e3:8.1f} us avg {by / (t * 1e-3) / 1e9:7.0f} GB/s")
    # matrix-core utilisation of the decode-phase products (skinny: k+1 rows)
    mf = {n: v for n, v in prof.items() if n.startswith("k_gemm_mfma")}
    mf_ms, mf_fl = sum(v[1] for v in mf.values()), sum(v[3] for v in mf.values())
    mf_tfs = mf_fl / (mf_ms * 1e-3) / 1e12 if mf_ms > 0 else 0.0

    # drafting speedup of the layer-parallel plan over the sequential draft
    # (every layer its own stage): the k-1 draft steps of a round, at the
    # round's current positions, each plan timed alternately
    t_plan = {"n": [], "seq": []}
    for _ in range(5):
        for key, plan in (("seq", seq_offs), ("n", offs)):
            dec.plan = plan
            dec._upload_positions()
            a_, b_ = ev(), ev()
            a_.record()
            dec.draft_phase()
            b_.record()
            torch.cuda.synchronize()
            t_plan[key].append(a_.elapsed_time(b_) / n_dsteps)
    dec.plan = offs
    step_n, step_seq = float(np.median(t_plan["n"])), float(np.median(t_plan["seq"]))
    log(f"  draft step: plan {step_n * 1e3:.0f} us, sequential (N = 1) {step_seq * 1e3:.0f} us -> drafting "
        f"speedup {step_seq / step_n:.3f}x")

    # cosine diagnostic of the fuzzy inputs (rebuttal discussion of Table 3):
    # per layer, cos(set input h0, the state a sequential pass would feed the
    # layer), for the round's first draft step at the current positions
    Ld = cfg.draft.n_layers
    cosv = torch.zeros(cfg.batch, Ld, device=dev)
    dec._upload_positions()
    api.spec_draft_attention_cosine(dec.draft, dec.dkv, offs, cfg.batch, dec.vtok[:, 1], k + 1, dec.tab[1],
                                    max(dec.t) + 1, cosv, Ld, dec.ws)
    cos_layers = [round(float(x), 5) for x in cosv.mean(0).cpu().numpy()]
    firsts = set(offs[:-1])
    inner = [c for l, c in enumerate(cos_layers) if l not in firsts]
    log(f"  attention-input cosine (fuzzy vs sequential), layers not first in their set: "
        f"min {min(inner) if inner else 1.0:.4f}, mean {float(np.mean(inner)) if inner else 1.0:.4f}")

    # stage overlap (PEARL-style, measurement only): a round's draft steps and
    # its verify run back to back, then concurrently on two streams (the
    # verify with its own workspace; the overlapped pair ignores their data
    # dependence, so only the times mean anything)
    ws2 = torch.empty_like(dec.ws)
    s2 = torch.cuda.Stream()
    main = torch.cuda.current_stream()

    def verify_into(w):
        api.spec_verify_forward(dec.base, dec.bkv, cfg.batch, dec.vtok, dec.tab[0], k + 1, max(dec.t) + k,
                                dec.p_logits, w)
    t_ser, t_ovl = [], []
    dec._upload_positions()
    for _ in range(5):
        a_, b_ = ev(), ev()
        a_.record()
        dec.draft_phase()
        verify_into(ws2)
        b_.record()
        torch.cuda.synchronize()
        t_ser.append(a_.elapsed_time(b_))
        a_, b_ = ev(), ev()
        a_.record()
        s2.wait_stream(main)
        dec.draft_phase()
        with torch.cuda.stream(s2):
            verify_into(ws2)
        main.wait_stream(s2)
        b_.record()
        torch.cuda.synchronize()
        t_ovl.append(a_.elapsed_time(b_))
    ser_ms, ovl_ms = float(np.median(t_ser)), float(np.median(t_ovl))
    log(f"  draft steps + verify: back to back {ser_ms:.3f} ms, on two streams {ovl_ms:.3f} ms")
    del ws2

    # the draft step at a fixed context P + 64 (comparable across acceptance
    # rates): the round's k-1 steps at positions P+64 .. (their KV writes land
    # beyond the committed positions and are rewritten before they are read)
    t_keep = list(dec.t)
    dec.t = [P + 64] * cfg.batch
    dec._upload_positions()
    t_fix = []
    for _ in range(5):
        a_, b_ = ev(), ev()
        a_.record()
        dec.draft_phase()
        b_.record()
        torch.cuda.synchronize()
        t_fix.append(a_.elapsed_time(b_) / n_dsteps)
    step_fix = float(np.median(t_fix))
    fix_bytes = draft_step_bytes(cfg.draft, P + 64)
    log(f"  draft step at context {P + 64}: {step_fix * 1e3:.0f} us, "
        f"{fix_bytes / (step_fix * 1e-3) / 1e9:.0f} GB/s")
    # calibration cost per row count (a + 1 = 1 .. k + 1 emitted tokens), at
    # the same positions, for the projections below
    cal_ms = []
    ntok = torch.zeros(cfg.batch, dtype=torch.int32, device=dev)
    start = torch.full((cfg.batch,), P + 64, dtype=torch.int32, device=dev)
    for m_ in range(1, k + 2):
        ntok.fill_(m_)
        tt = []
        for _ in range(5):
            a_, b_ = ev(), ev()
            a_.record()
            api.spec_calibrate_kv(dec.draft, dec.dkv, cfg.batch, dec.commit, start, ntok, k + 1, P + 64 + m_ - 1,
                                  dec.inv_temp, dec.seed, dec.q_logits[:, 0], k * dec.V, dec.vtok[:, 1], k + 1,
                                  dec.ws, tokens_stride=k + 1)
            b_.record()
            torch.cuda.synchronize()
            tt.append(a_.elapsed_time(b_))
        cal_ms.append(float(np.median(tt)))
    dec.t = t_keep
    log("  calibration by rows: " + ", ".join(f"{i + 1}: {c * 1e3:.0f} us" for i, c in enumerate(cal_ms)))

    # tokens/s at acceptance rates alpha per draft (E[a] under a truncated
    # geometric law, Leviathan et al.): the measured phases with the
    # calibration cost of a + 1 rows, the same kernels and shapes
    base_ms = ms["draft"] + ms["verify"] + ms["accept"]

    def projected(alpha):
        pa = [alpha ** j * (1 - alpha) for j in range(k)] + [alpha ** k]
        tok = sum(p_ * (j + 1) for j, p_ in enumerate(pa))
        rnd = base_ms + sum(p_ * cal_ms[j] for j, p_ in enumerate(pa))
        return round(cfg.batch * tok / (rnd * 1e-3), 2)
    proj = {"0.5": projected(0.5), "0.8": projected(0.8)}
    log(f"  projected tokens/s at acceptance 0.5: {proj['0.5']}, at 0.8: {proj['0.8']}")

    # copy ceiling measured on this GPU: a 2 GiB device-to-device copy (bytes
    # read + bytes written over its time)
    src = torch.empty(1 << 30, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    tc = []
    for _ in range(5):
        a_, b_ = ev(), ev()
        a_.record()
        dst.copy_(src)
        b_.record()
        torch.cuda.synchronize()
        tc.append(a_.elapsed_time(b_))
    copy_gbs = 2 * src.numel() * 2 / (float(np.median(tc)) * 1e-3) / 1e9
    del src, dst
    log(f"  device copy ceiling: {copy_gbs:.0f} GB/s")

    n1 = None
    if args.n1_compare:
        d1 = SpecDecoder(cfg.draft, dw, cfg.base, bw, cfg.batch, cap, k, seq_offs, P, inv_t, cfg.sample_seed,
                         mlp_mode=mlp_mode, calibrate=not args.no_calibration, separate=args.separate_calibration)
        d1.prefill(prompts)
        for _ in range(W):
            d1.step(big)
        nb = sum(len(o) for o in d1.out)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(K):
            d1.step(big)
        torch.cuda.synchronize()
        el1 = time.perf_counter() - t1
        tok1 = sum(len(o) for o in d1.out) - nb
        acc1 = (tok1 - K * cfg.batch) / (K * cfg.batch * k)
        n1 = {"tokens_per_s": round(tok1 / el1, 3), "acceptance_rate": round(acc1, 4)}
        log(f"  sequential draft plan (N = 1): {tok1 / el1:.1f} tok/s, acceptance {acc1:.3f} "
            f"(layer-parallel plan: {value:.1f} tok/s, acceptance {acc_rate:.3f})")
        del d1

    vanilla = None
    if not args.no_vanilla:
        vd = VanillaDecoder(cfg.base, bw, cfg.batch, P + 64 + 2, P, inv_t, cfg.sample_seed)
        vd.generate(prompts, 4)
        nv = 48
        vd.generate(prompts, nv)          # decode loop timed apart from its prefill
        vanilla_tok_s = nv / vd.decode_s
        vanilla = round(vanilla_tok_s, 2)
        log(f"  vanilla decoding ~{vanilla_tok_s:.1f} tok/s")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, dw, bw, offs, k, P, inv_t)

    out = {
        "metric": "accepted tokens/s at batch 1; draft-step us and HBM GB/s vs peak (1B->8B shapes)",
        "value": round(value, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(elapsed * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.draft.dtype == 1 else "f32",
        "data": "synthetic (seeded random-init weights, uniform-random prompt)",
        "config": {"workload": f"{cfg.name}: draft {cfg.draft.n_layers}L d{cfg.draft.d_model} -> base "
                               f"{cfg.base.n_layers}L d{cfg.base.d_model}, V {cfg.draft.vocab}, P {P}, k {k}, "
                               f"N {N}, batch {cfg.batch}, T {args.temperature}"
                               + (", no KV calibration" if args.no_calibration else "")
                               + (", parallel MLPs" if args.mlp_parallel else ""),
                   "plan": offs, "global_batch": cfg.batch, "seq_len": P},
        "acceptance_rate": round(acc_rate, 4),
        "draft_step_us": round(d_step_ms * 1e3, 1),
        "verify_us": round(ms["verify"] * 1e3, 1),
        "accept_us": round(ms["accept"] * 1e3, 1),
        "calibrate_us": round(ms["calib"] * 1e3, 1),
        "prefill_ms": round(prefill_ms, 2),
        "vanilla_tokens_per_s": vanilla,
        "draft_step_us_sequential_plan": round(step_seq * 1e3, 1),
        "drafting_speedup": round(step_seq / step_n, 4),
        "sequential_plan": n1,
        "stage_overlap": {"back_to_back_ms": round(ser_ms, 3), "two_streams_ms": round(ovl_ms, 3)},
        "attention_input_cosine": {"per_layer": cos_layers,
                                   "mean_fuzzy_layers": round(float(np.mean(inner)), 5) if inner else None},
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "launches": dom_n, "avg_launch_us": round(dom_ms / dom_n * 1e3, 2),
                     "bytes_per_launch": int(dom_bytes / dom_n)},
        "roofline_draft_step": {"bound": "hbm", "achieved": round(d_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(d_gbs / HBM_PEAK_GBS, 4), "frac_of_copy_ceiling": round(d_gbs / copy_gbs, 4),
                                "bytes_per_step": int(d_bytes)},
        "draft_step_at_fixed_context": {"context": P + 64, "us": round(step_fix * 1e3, 1),
                                        "gbs": round(fix_bytes / (step_fix * 1e-3) / 1e9, 1),
                                        "frac": round(fix_bytes / (step_fix * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "roofline_verify": {"bound": "hbm", "achieved": round(v_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(v_gbs / HBM_PEAK_GBS, 4), "frac_of_copy_ceiling": round(v_gbs / copy_gbs, 4),
                            "bytes_per_step": int(v_bytes)},
        "copy_ceiling_gbs": round(copy_gbs, 1),
        "calibrate_us_by_rows": [round(c * 1e3, 1) for c in cal_ms],
        "projected_tokens_per_s": proj,
        "kernels": {name: {"launches": n, "avg_us": round(t / n * 1e3, 2),
                           "gbs": round(by / (t * 1e-3) / 1e9, 1)} for name, (n, t, by, _) in prof.items()},
        "mfma_decode": {"bound": "mfma", "achieved": round(mf_tfs, 2), "peak": MFMA_BF16_PEAK_TFS,
                        "unit": "TFLOP/s", "frac": round(mf_tfs / MFMA_BF16_PEAK_TFS, 5)},
        "prefill": {"ms": round(prefill_ms, 2), "products_ms": round(pf_ms, 2),
                    "products_tflop": round(pf_fl / 1e12, 3), "attention_ms": round(attn_ms, 2),
                    "roofline": {"bound": "mfma", "achieved": round(pf_tfs, 1), "peak": MFMA_BF16_PEAK_TFS,
                                 "unit": "TFLOP/s", "frac": round(pf_tfs / MFMA_BF16_PEAK_TFS, 4)}},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(cfg, dw, bw, offs, k, P, inv_t, budget_s=10.0, max_rounds=40):
    """The oracle, timed on the host cores on a bounded sample: consecutive
    speculative rounds of the same workload (full-depth float32 models, from
    context P, unfilled KV cache: values do not change the work) until about
    budget_s seconds of oracle time have run."""
    import torch
    from oracle import sampling
    from oracle.model import KVCache, OracleModel, forward, fuzzy_step
    from oracle.plan import offsets_to_sets
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    log(f"  cpu baseline: converting weights to float32 on the host ({cores} cores)")
    t0 = time.time()
    od = OracleModel.from_torch(cfg.draft, dw, np.float32)
    ob = OracleModel.from_torch(cfg.base, bw, np.float32)
    log(f"    converted in {time.time() - t0:.1f}s")
    sets = offsets_to_sets(offs)
    cap = P + max_rounds * (k + 1) + 4
    dkv = KVCache(cfg.draft, 1, cap, np.float32)
    bkv = KVCache(cfg.base, 1, cap, np.float32)
    rng = np.random.default_rng(0)
    t = P - 1
    emitted, rounds = 0, 0
    ts = time.perf_counter()
    while rounds < max_rounds and (rounds == 0 or time.perf_counter() - ts < budget_s):
        toks = rng.integers(0, cfg.draft.vocab, size=k + 1)
        qs = [rng.normal(size=cfg.draft.vocab).astype(np.float32)]   # q_1 comes from the previous calibration
        for j in range(1, k):
            qs.append(fuzzy_step(od, dkv, 0, int(toks[j]), t + j, sets))
        pl = forward(ob, bkv, 0, list(toks), range(t, t + k + 1), logits="all")
        a, y, _ = sampling.accept_resample(pl, np.stack(qs), list(toks[1:]), t, inv_t, cfg.sample_seed, 0)
        forward(od, dkv, 0, list(toks[1:a + 1]) + [y], range(t + 1, t + a + 2), logits="last")
        t += a + 1
        emitted += a + 1
        rounds += 1
    dt = time.perf_counter() - ts
    log(f"    {rounds} oracle rounds: {dt:.2f}s")
    del od, ob
    return {"value": round(emitted / dt, 5), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{rounds} consecutive speculative rounds of {cfg.name} from context {P} (k={k}, float32 "
                      f"NumPy, full depth; {emitted} token(s) emitted in {dt:.2f}s)"}


if __name__ == "__main__":
    main()
