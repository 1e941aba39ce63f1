"""Benchmark of the fast-weight prefill on one MI355X.

One step = reset of the fast weight to W_0 (a new sequence) + one
ipttt_prefill_layer call over the whole sequence: gate/up, conv, projection,
update scan and apply for every chunk. Inputs are seeded synthetic tensors of
the workload's shape, resident in HBM before the timed region. Prints one JSON
line. Per-kernel durations come from HIP events that the library records on
the launch stream during the timed steps.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import workloads as wl  # noqa: E402

METRIC = "fast-weight prefill tokens/s per MLP layer at L=128k,B=1024; % MFMA/HBM roofline"
KERNEL_SRCS = [os.path.join(ROOT, "chunked_weight_mlp_amd", "csrc", f)
               for f in ("kernels_mfma.hip", "mfma_common.h")]
KERNEL_TAGS = {"gateup": "k_gateup", "conv": "k_conv", "proj": "k_proj", "update": "k_update",
               "apply": "k_apply", "gram": "k_gram", "snapshot": "k_snapshot",
               "mse_fix": "k_mse_fix", "copy": "copyBuffer"}


def kernel_source_hash() -> str:
    """Hash of the sources the measured kernels are built from."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def summarize_traffic(workload: str, fetch_csv: str, write_csv: str) -> dict:
    """HBM bytes per launch of each kernel from two rocprofv3 --pmc runs of this
    benchmark (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled by
    what the same counter reads for the reset's plain device copy of W_0
    (d * d_ff * 4 bytes read and written, one per sequence) in the same run:
    the median over those copies, so a stray small copy of the runtime's does
    not skew it."""
    import csv
    w = wl.WORKLOADS[workload]
    copy_bytes = w.d * w.d_ff * 4

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            for k, tag in KERNEL_TAGS.items():
                if tag in r["Kernel_Name"]:
                    vals.setdefault(k, []).append(float(r["Counter_Value"]) * 1024.0)
        out = {k: sum(v) / len(v) for k, v in vals.items()}
        if "copy" in vals:
            c = sorted(vals["copy"])
            out["copy"] = c[len(c) // 2]
        return out

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    f_fetch, f_write = copy_bytes / fetch["copy"], copy_bytes / write["copy"]
    out = {"workload": workload, "kernel_source_sha": kernel_source_hash(),
           "calibration": {"copy_bytes": copy_bytes, "fetch_factor": round(f_fetch, 4),
                           "write_factor": round(f_write, 4)},
           "bytes_per_launch": {}}
    for k in fetch:
        if k == "copy" or k not in write:
            continue
        out["bytes_per_launch"][k] = {"fetch": round(fetch[k] * f_fetch),
                                      "write": round(write[k] * f_write),
                                      "total": round(fetch[k] * f_fetch + write[k] * f_write)}
    return out


def load_traffic(workload: str, kernel: str):
    """Traffic of `kernel` if a summary exists for this workload and the kernel
    sources (kernels_mfma.hip, mfma_common.h) have not changed since the
    counters were taken; else None."""
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    if t.get("kernel_source_sha") != kernel_source_hash():
        return None
    b = t["bytes_per_launch"].get(kernel)
    return None if b is None else b["total"]
PEAK = {"bf16": 2500.0, "f32": 157.3}  # dense TFLOP/s (MFMA bf16, fp32)
HBM_PEAK = 8000.0                       # GB/s


def achievable_peaks() -> dict:
    """The chip's achievable rates, measured here by the library's micro-benchmarks
    (ipttt_probe): bf16 MFMA issue at two waves per SIMD for each MFMA shape, with
    no memory traffic, a streaming read of 4 GiB (more than the caches hold),
    conflict-free LDS reads and direct copies from L2 into LDS. Best of a few
    launches, HIP events on the launch stream."""
    from chunked_weight_mlp_amd import probe
    dev = "cuda:0"
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    out_buf = torch.empty(1 << 20, dtype=torch.float32, device=dev)
    nbytes = 4 << 30
    src = torch.zeros(nbytes // 4, dtype=torch.float32, device=dev)

    def best(kind, n, a, reps=4):
        rates = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            work = probe.ipttt_probe(kind, n, a, nbytes if a is not None else 0,
                                     ctypes.c_void_p(out_buf.data_ptr()), out_buf.numel() * 4, sp)
            e1.record(stream)
            e1.synchronize()
            rates.append(work / (e0.elapsed_time(e1) * 1e-3))
        return max(rates)

    m16 = best(probe.IPTTT_PROBE_MFMA16, 20000, None) / 1e12
    m32 = best(probe.IPTTT_PROBE_MFMA32, 20000, None) / 1e12
    rd = best(probe.IPTTT_PROBE_READ, nbytes, ctypes.c_void_p(src.data_ptr())) / 1e9
    lds = best(probe.IPTTT_PROBE_LDS, 20000, None) / 1e12
    cp = best(probe.IPTTT_PROBE_COPY, 4000, ctypes.c_void_p(src.data_ptr())) / 1e12
    del src
    return {"mfma16_bf16_tflops": round(m16, 1), "mfma32_bf16_tflops": round(m32, 1),
            "mfma_bf16_tflops": round(max(m16, m32), 1), "hbm_read_gbps": round(rd, 1),
            "lds_read_tbps": round(lds, 2), "l2_to_lds_copy_tbps": round(cp, 2),
            "source": "ipttt_probe micro-benchmarks on this GPU"}


def achievable_fracs(ach: dict, roof: dict, n3_tflops=None) -> dict:
    """The dominant kernel (and the fast-weight step) against the measured rates."""
    if roof["unit"] == "TFLOP/s":
        dom = roof["achieved"] / ach["mfma_bf16_tflops"]
    else:
        dom = roof["achieved"] / ach["hbm_read_gbps"]
    out = dict(ach, dominant_frac=round(dom, 4))
    if n3_tflops is not None:
        out["fast_weight_step_frac"] = round(n3_tflops / ach["mfma_bf16_tflops"], 4)
    return out


def group_chunks(w: wl.Workload, requested: int, generic: bool) -> int:
    """Chunks per group, as the library picks them on the bf16 MFMA path:
    about 1024 chunk-padded rows with the linear rule, 2048 with the MSE rule;
    1 on the generic kernels."""
    if w.dtype != "bf16" or generic:
        return 1
    rows = 2048 if w.update == "mse" else 1024
    return requested or max(1, rows // (-(-w.chunk // 64) * 64))


def kernel_work(w: wl.Workload, tokens: int, G: int = 1):
    """Algorithmic FLOPs and HBM bytes of one launch of each kernel over `tokens`
    tokens (all sequences of one pass), with one W snapshot per G chunks. Bytes
    count each operand once per use the method makes of it: the linear scan
    reads and writes each sequence's fp32 W once per pass and writes one bf16
    copy per group; the MSE rule reads and writes W and its copy every group.
    The apply counts the method's product Z W only; the Gram kernel's work (and
    the apply's use of it, and the MSE rule's per-chunk corrections) is what
    the chunk-parallel form spends to skip snapshots, reported for its own
    rate."""
    d, F, Kc, n = w.d, w.d_ff, w.conv_k, w.n_seq
    el = 2 if w.dtype == "bf16" else 4
    chunks = -(-(tokens // n) // w.chunk)   # per sequence
    groups = -(-chunks // G)
    rows = G * (-(-w.chunk // 64) * 64)
    W32, Wb = 4 * F * d, el * F * d         # one sequence's fp32 W and its copy
    if w.update == "mse":
        upd = el * tokens * (F + d) + n * groups * (2 * W32 + Wb)
        app = el * tokens * (F + d) + n * groups * Wb + 4 * tokens * d
    else:
        upd = el * tokens * (F + d) + n * (2 * W32 + groups * Wb)
        app = el * tokens * F + n * groups * Wb + 4 * tokens * d
    work = {
        "gateup": (4 * d * F * tokens, el * (tokens * d + 2 * F * d + tokens * F)),
        "conv": (2 * Kc * d * tokens, el * (2 * tokens * d + Kc * d)),
        "proj": (2 * d * d * tokens, el * (2 * tokens * d + d * d)),
        "update": (2 * d * F * tokens, upd),
        "apply": (2 * d * F * tokens, app),
    }
    if G > 1:  # block-causal Z Z^T: about half of each group's rows x rows x F
        work["gram"] = (rows * F * tokens, el * tokens * F + el * tokens * rows // 2)
    if G > 1 and w.update == "mse":
        # chunk jl of a group: O += P R over the jl Bp earlier rows, all chunks but
        # the first; P and R blocks read, O read and written, V read, Rt written
        Bp = rows // G
        pairs = n * groups * G * (G - 1) // 2
        later = tokens * (G - 1) // G
        work["mse_fix"] = (2 * pairs * Bp * Bp * d,
                           el * pairs * Bp * (Bp + d) + later * d * (8 + 2 * el))
    return work


def kernel_rates(prof: dict, work: dict, steps: int, ms_total: float, passes: int, dtype: str):
    """Per-kernel launches, durations and rates, and the roofline entry of the
    kernel with the largest total time among those with a work model."""
    kernels = {}
    for k, (n, ms) in prof.items():
        if n == 0:
            continue
        avg = ms / n
        entry = {"launches_per_step": n / steps, "avg_ms": round(avg, 4),
                 "share": round(ms / max(ms_total, 1e-9), 4)}
        if k in work:
            per_pass = n / steps / passes          # launches of this kernel per pass
            fl, by = (v / per_pass for v in work[k])
            entry["tflops"] = round(fl / (avg * 1e-3) / 1e12, 2)
            entry["gbps"] = round(by / (avg * 1e-3) / 1e9, 1)
        kernels[k] = entry
    dom = max((k for k in kernels if k in work), key=lambda k: prof[k][1])
    per_pass = prof[dom][0] / steps / passes
    dom_fl, dom_by = (v / per_pass for v in work[dom])
    dom_avg_s = prof[dom][1] / prof[dom][0] * 1e-3
    intensity = dom_fl / max(dom_by, 1)
    ridge = PEAK[dtype] * 1e12 / (HBM_PEAK * 1e9)
    if intensity >= ridge:
        ach = dom_fl / dom_avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK[dtype], "unit": "TFLOP/s",
                "frac": round(ach / PEAK[dtype], 4)}
    else:
        ach = dom_by / dom_avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK, 4)}
    roof["algorithmic_bytes"] = round(dom_by)
    roof["kernel"] = dom
    return kernels, roof, dom


def backward_work(w: wl.Workload, tokens: int):
    """Algorithmic FLOPs and HBM bytes of one launch of each backward kernel kind
    over `tokens` tokens (all sequences); launches of a kind within one step
    share the step's work equally. The recompute and the reverse pass keep one
    bf16 W and one bf16 G per chunk; the MSE rule also reads and writes the fp32
    state every chunk. bw_small (dC, dProj, the conv adjoint, the dW_0 sum) and
    bw_misc (transposes, fills) are left without a model."""
    d, F, Kc, n = w.d, w.d_ff, w.conv_k, w.n_seq
    el = 2
    chunks = -(-(tokens // n) // w.chunk)
    W32, Wb = 4 * F * d, el * F * d
    snaps = n * chunks * Wb
    state = n * chunks * 2 * W32 if w.update == "mse" else n * 2 * W32
    return {
        "gateup": (4 * d * F * tokens, el * (tokens * d + 2 * F * d + 3 * tokens * F)),
        "conv": (2 * Kc * d * tokens, el * (2 * tokens * d + Kc * d)),
        "proj": (2 * d * d * tokens, el * (2 * tokens * d + d * d)),
        "update": (2 * d * F * tokens, el * tokens * (F + d) + state + snaps),
        "apply": (2 * d * F * tokens, el * tokens * (F + d) + snaps),
        "bw_scan": (2 * d * F * tokens, el * tokens * (F + d) + state + snaps),
        "bw_dz": (4 * d * F * tokens, el * (2 * tokens * d + 4 * tokens * F) + 2 * snaps),
        "bw_dv": (2 * d * F * tokens, el * (tokens * F + 2 * tokens * d) + snaps),
        "bw_dx": (4 * d * F * tokens, el * (2 * tokens * F + 2 * F * d) + 4 * tokens * d),
        "bw_dw": (4 * d * F * tokens, el * (2 * tokens * F + tokens * d) + 8 * F * d),
    }


def host_info() -> dict:
    """The host the oracle runs on: logical CPUs, CPU model, the BLAS numpy
    calls (vendor, version, threads) and the thread variables in effect."""
    from threadpoolctl import threadpool_info
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = [dict(api=p.get("internal_api"), version=p.get("version"), threads=p.get("num_threads"),
                 arch=p.get("architecture")) for p in threadpool_info() if p.get("user_api") == "blas"]
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"os_cpu_count": os.cpu_count(), "cpus_in_affinity": affinity, "cpu_model": model,
            "blas": blas, "env": {k: os.environ.get(k) for k in
                                  ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
                                  if os.environ.get(k) is not None}}


def cpu_baseline(w: wl.Workload, x, e, weights, n_chunks: int):
    from threadpoolctl import threadpool_info

    import oracle

    tokens = min(w.seq_len, n_chunks * w.chunk)
    ow = wl.to_oracle(weights)
    X = x[:1, :tokens].double().numpy()
    E = e[:1, :tokens].double().numpy()
    t0 = time.perf_counter()
    oracle.prefill(X, E, ow["W_g"], ow["W_u"], ow["conv_w"], ow["Proj"], ow["W_0"], w.eta, w.chunk,
                   update=w.update)
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {
        "value": tokens / dt,
        "unit": "tokens/s",
        "gflops": round(w.flops_per_token() * tokens / dt / 1e9, 2),  # float64, algorithmic
        "cores": threads,
        "kind": "oracle",
        "sample": f"the oracle's chunk scan (float64 numpy) over the first {tokens} tokens "
                  f"({-(-tokens // w.chunk)} chunks) of sequence 0 of this workload, {dt:.1f} s; "
                  f"value = those tokens / that time (the scan's cost per chunk does not depend "
                  f"on the chunk's position)",
        "host": host_info(),
    }


def packed_doc_starts(w: wl.Workload, n_docs: int):
    """n_docs - 1 seeded document starts in (0, L): lengths drawn uniformly
    around L / n_docs, so documents end mid-chunk."""
    import numpy as np
    r = np.random.default_rng(31)
    cuts = np.sort(r.choice(np.arange(1, w.seq_len), size=n_docs - 1, replace=False))
    return [int(c) for c in cuts]


def trace_summary(path: str) -> str:
    """Markdown table (kernel, calls, avg / min / max ms, share) of a rocprofv3
    kernel_stats.csv, template arguments and namespaces shortened."""
    import csv
    import re
    rows = sorted(csv.DictReader(open(path)), key=lambda r: -float(r["TotalDurationNs"]))
    out = ["| kernel | calls | avg ms | min ms | max ms | share % |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("(anonymous namespace)::", "")
        name = re.sub(r"ipttt::mfma::|ipttt::", "", name)
        name = re.sub(r"\(.*$", "", name).replace("void ", "")
        if name.startswith("_Z"):  # not demangled (bf16 template arguments): the kernel's identifier
            m = re.search(r"\d(k_\w+?)I", name)
            if m:
                name = m.group(1)
        if "_Accum" in name:  # bf16 template arguments the profiler could not render
            name = name.split("<")[0]
        name = name.replace("__amd_rocclr_", "")
        out.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e6:.3f} | "
                   f"{float(r['MinNs']) / 1e6:.3f} | {float(r['MaxNs']) / 1e6:.3f} | "
                   f"{float(r['Percentage']):.2f} |")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=None, choices=sorted(wl.WORKLOADS),
                    help="default: the 128k / B = 1024 prefill; 32k / B = 512 with --backward")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward through the scan (ipttt_backward_layer) instead")
    ap.add_argument("--decode", action="store_true",
                    help="time token-by-token decode (ipttt_decode_step) over whole chunks")
    ap.add_argument("--decode-batch", type=int, default=1, help="sequences decoded together")
    ap.add_argument("--packed-docs", type=int, default=0,
                    help="time ipttt_prefill_packed on one sequence cut into this many documents "
                         "at seeded random positions (the fast weight resets at each)")
    ap.add_argument("--slab-chunks", type=int, default=0, help="chunks per pass (0 = all)")
    ap.add_argument("--cpu-chunks", type=int, default=0,
                    help="chunks in the oracle sample (default 40; 4 with --backward)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the achievable-peak micro-benchmarks")
    ap.add_argument("--generic", action="store_true", help="generic FMA kernels instead of MFMA")
    ap.add_argument("--group-chunks", type=int, default=0,
                    help="chunks per W snapshot of the linear scan (0 = library choice, 1 = plain)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<workload>.json from two rocprofv3 --pmc "
                         "counter_collection.csv files (FETCH_SIZE, WRITE_SIZE) and exit")
    ap.add_argument("--trace-summary", metavar="KERNEL_STATS_CSV",
                    help="print a markdown table of a rocprofv3 --stats kernel_stats.csv and exit")
    args = ap.parse_args()
    if args.trace_summary:
        print(trace_summary(args.trace_summary))
        return
    if args.workload is None:
        args.workload = "qwen3_4b_L32k_B512" if args.backward else wl.HEADLINE
    if not args.cpu_chunks:
        args.cpu_chunks = 4 if args.backward else 40

    if args.traffic_from:
        t = summarize_traffic(args.workload, *args.traffic_from)
        with open(traffic_path(args.workload), "w") as fh:
            json.dump(t, fh, indent=1)
        print(json.dumps(t))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    from chunked_weight_mlp_amd import ipttt

    ipttt.load()
    w = wl.WORKLOADS[args.workload]
    if args.backward:
        return bench_backward(args, w)
    if args.decode:
        return bench_decode(args, w)
    dev = "cuda:0"
    t0 = time.perf_counter()
    weights = wl.make_weights(w)
    x, e = wl.make_inputs(w)
    print(f"[bench] inputs {w.name} generated in {time.perf_counter() - t0:.1f} s", file=sys.stderr,
          flush=True)
    wdev = {k: v.to(dev) for k, v in weights.items()}
    xd, ed = x.to(dev), e.to(dev)
    slab = args.slab_chunks or w.n_chunks
    layer = ipttt.Layer(**wdev, chunk=w.chunk, eta=w.eta, update=w.update, max_batch=w.n_seq,
                        slab_chunks=slab, group_chunks=args.group_chunks,
                        flags=ipttt.IPTTT_FLAG_GENERIC_KERNELS if args.generic else 0)
    o = torch.empty(xd.shape, dtype=torch.float32, device=dev)

    starts = packed_doc_starts(w, args.packed_docs) if args.packed_docs > 1 else None
    if starts is not None and w.n_seq != 1:
        sys.exit("--packed-docs needs a one-sequence workload")

    def step():
        layer.reset()
        if starts is None:
            layer.prefill(xd, ed, o)
        else:
            layer.prefill_packed(xd[0], ed[0], starts, o=o[0])

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        print(f"[bench] warmup {i + 1}/{args.warmup} done", file=sys.stderr, flush=True)

    torch.cuda.synchronize()
    # one event between consecutive steps (recording adds no synchronisation):
    # the total and each step's own time
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ipttt.ipttt_profile_begin(layer.handle)
    wall0 = time.perf_counter()
    evs[0].record()
    for i in range(args.steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    prof = ipttt.ipttt_profile_end(layer.handle)
    ms_total = evs[0].elapsed_time(evs[-1])
    ms_step = ms_total / args.steps
    step_ms = step_stats([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    tokens = w.n_seq * w.seq_len
    value = tokens / (ms_step / 1e3)
    print(f"[bench] {args.steps} steps in {ms_total:.1f} ms (wall {wall * 1e3:.1f} ms)", file=sys.stderr,
          flush=True)

    # per-kernel live durations and the dominant kernel's roofline
    G = min(group_chunks(w, args.group_chunks, args.generic), slab)
    if slab < w.n_chunks:
        slab = slab // G * G   # the library runs whole groups per pass
    passes = -(-w.n_chunks // slab)
    tok_per_pass = w.n_seq * min(w.seq_len, slab * w.chunk)
    if starts is not None:  # one scan per document; the model uses their mean length
        passes = len(starts) + 1
        tok_per_pass = w.seq_len // passes
    work = kernel_work(w, tok_per_pass, G)
    kernels, roof, dom = kernel_rates(prof, work, args.steps, ms_total, passes, w.dtype)
    # measured HBM bytes per launch (rocprofv3 counters, profiles/traffic_*.json)
    roof["traffic"] = None if args.generic else load_traffic(w.name, dom)
    # the fast-weight step on its own (apply + update, and the Gram product of
    # chunk groups): algorithmic 4 d d_ff FLOPs per token
    n3_ms = sum(prof[k][1] for k in ("update", "apply", "gram", "snapshot", "mse_fix")
                if prof[k][0]) / args.steps
    n3_fl = 4 * w.d * w.d_ff * tokens
    n3 = {"ms_per_step": round(n3_ms, 4), "tflops": round(n3_fl / (n3_ms * 1e-3) / 1e12, 2),
          "frac_of_peak": round(n3_fl / (n3_ms * 1e-3) / 1e12 / PEAK[w.dtype], 4)}

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "step_ms": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian inputs and weights of the workload's shape)",
        "config": {"workload": w.name, "d": w.d, "d_ff": w.d_ff, "seq_len": w.seq_len,
                   "chunk": w.chunk, "batch": w.n_seq, "update": w.update, "eta": w.eta,
                   "packed_docs": args.packed_docs or 1,
                   "chunks_per_pass": slab, "chunks_per_snapshot": G,
                   "kernels": "generic" if args.generic else "mfma"},
        "tflops": round(w.flops_per_token() * tokens / (ms_step * 1e-3) / 1e12, 2),
        "roofline": roof,
        "fast_weight_step": n3,
        "kernels": kernels,
    }
    if not args.no_probe:
        out["achievable"] = achievable_fracs(achievable_peaks(), roof, n3["tflops"])
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, x, e, weights, args.cpu_chunks)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def step_stats(ms: list[float]) -> dict:
    """Median, minimum and maximum of the timed steps' own durations (ms)."""
    v = sorted(ms)
    n = len(v)
    med = v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])
    return {"median": round(med, 4), "min": round(v[0], 4), "max": round(v[-1], 4)}


def cpu_baseline_backward(w: wl.Workload, x, e, weights, d_o, n_chunks: int):
    from threadpoolctl import threadpool_info

    import oracle

    tokens = min(w.seq_len, n_chunks * w.chunk)
    ow = wl.to_oracle(weights)
    t0 = time.perf_counter()
    oracle.backward(x[:1, :tokens].double().numpy(), e[:1, :tokens].double().numpy(), ow["W_g"],
                    ow["W_u"], ow["conv_w"], ow["Proj"], ow["W_0"], w.eta, w.chunk,
                    d_o[:1, :tokens].double().numpy(), update=w.update)
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the oracle's backward (float64 numpy) over the first {tokens} tokens "
                      f"({-(-tokens // w.chunk)} chunks) of sequence 0, {dt:.1f} s",
            "host": host_info()}


def bench_backward(args, w: wl.Workload):
    """One step = one ipttt_backward_layer call over the whole batch (forward
    recompute from w0, reverse scan, every gradient), inputs and upstream
    gradients resident in HBM."""
    from chunked_weight_mlp_amd import ipttt

    dev = "cuda:0"
    weights = wl.make_weights(w)
    x, e = wl.make_inputs(w)
    d_o, d_wf = wl.make_upstream(w)
    wdev = {k: v.to(dev) for k, v in weights.items()}
    xd, ed, dod, dwfd = x.to(dev), e.to(dev), d_o.to(dev), d_wf.to(dev)
    layer = ipttt.Layer(**wdev, chunk=w.chunk, eta=w.eta, update=w.update, max_batch=w.n_seq)
    need = ipttt.ipttt_backward_workspace_bytes(layer.desc, w.n_seq, w.seq_len)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    grads = layer.backward(xd, ed, dod, dwfd, workspace=ws)
    torch.cuda.synchronize()
    print(f"[bench] backward {w.name}: workspace {need / 2**30:.1f} GiB", file=sys.stderr, flush=True)

    def step():
        layer.backward(xd, ed, dod, dwfd, workspace=ws, grads=grads)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        print(f"[bench] warmup {i + 1}/{args.warmup} done", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    # timed region: the calls as a caller makes them. The library's per-launch
    # profiling events would add about 14 us of GPU time to every call here
    # (two kernels of ~16 us each), so the kernel durations come from a second
    # pass over the same steps with profiling on.
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    print(f"[bench] {args.steps} steps in {ms_total:.1f} ms; profiled pass", file=sys.stderr, flush=True)
    ipttt.ipttt_profile_begin(layer.handle)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = ipttt.ipttt_profile_end(layer.handle)
    ms_step = ms_total / args.steps
    tokens = w.n_seq * w.seq_len
    kernels, roof, _ = kernel_rates(prof, backward_work(w, tokens), args.steps, ms_total, 1, w.dtype)
    roof["traffic"] = None
    d, F = w.d, w.d_ff
    flops_tok = 22 * d * F + 6 * d * d
    out = {
        "metric": "fast-weight backward tokens/s per MLP layer (gradients through the scan)",
        "value": round(tokens / (ms_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian inputs, weights and upstream gradients)",
        "config": {"workload": w.name, "mode": "backward", "d": d, "d_ff": F, "seq_len": w.seq_len,
                   "chunk": w.chunk, "batch": w.n_seq, "update": w.update, "eta": w.eta},
        "tflops": round(flops_tok * tokens / (ms_step * 1e-3) / 1e12, 2),
        "roofline": roof,
        "kernels": kernels,
    }
    if not args.no_probe:
        out["achievable"] = achievable_fracs(achievable_peaks(), out["roofline"])
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle backward on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_backward(w, x, e, weights, d_o, args.cpu_chunks)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def bench_decode(args, w: wl.Workload):
    """One step = one whole chunk decoded token by token for `--decode-batch`
    sequences: B calls of ipttt_decode_step, the last of which also runs the
    chunk's update. Each call's apply reads every sequence's fp32 fast weight,
    so the per-token cost is bound by HBM (or the 256 MB Infinity Cache, which
    can hold one 4B-layer state)."""
    from chunked_weight_mlp_amd import ipttt

    dev = "cuda:0"
    nb, Bc = args.decode_batch, w.chunk
    weights = wl.make_weights(w)
    x, e = wl.make_inputs(w, seq_len=Bc, n_seq=nb)
    wdev = {k: v.to(dev) for k, v in weights.items()}
    xc, ec = x.to(dev).contiguous(), e.to(dev).contiguous()
    layer = ipttt.Layer(**wdev, chunk=Bc, eta=w.eta, update=w.update, max_batch=nb)
    layer.reset()
    o = torch.empty((nb, w.d), dtype=torch.float32, device=dev)

    def step():
        for pos in range(Bc):
            layer.decode_step(xc, ec, pos, o)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        print(f"[bench] warmup {i + 1}/{args.warmup} done", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    # timed region: the calls as a caller makes them. The library's per-launch
    # profiling events would add about 14 us of GPU time to every call here
    # (two kernels of ~16 us each), so the kernel durations come from a second
    # pass over the same steps with profiling on.
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    print(f"[bench] {args.steps} steps in {ms_total:.1f} ms; profiled pass", file=sys.stderr, flush=True)
    ipttt.ipttt_profile_begin(layer.handle)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = ipttt.ipttt_profile_end(layer.handle)
    tokens = nb * Bc * args.steps
    d, F = w.d, w.d_ff
    el = 2 if w.dtype == "bf16" else 4
    # decode apply: every sequence's fp32 W, its z, its output row
    n_apply, ms_apply = prof["apply"]
    apply_bytes = nb * (4 * d * F + el * F + 4 * d)
    ach = apply_bytes / (ms_apply / n_apply * 1e-3) / 1e9
    kernels = {k: {"launches_per_step": n / args.steps, "avg_ms": round(ms / n, 5),
                   "share": round(ms / max(ms_total, 1e-9), 4)} for k, (n, ms) in prof.items() if n}
    out = {
        "metric": "fast-weight decode tokens/s per MLP layer (one token per sequence per call)",
        "value": round(tokens / (ms_total * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_total / args.steps, 4),
        "ms_per_token_call": round(ms_total / (args.steps * Bc), 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian inputs and weights)",
        "config": {"workload": w.name, "mode": "decode", "d": d, "d_ff": F, "chunk": Bc,
                   "batch": nb, "update": w.update, "eta": w.eta},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK, 4), "traffic": None,
                     "algorithmic_bytes": apply_bytes, "kernel": "decode apply"},
        "kernels": kernels,
        "kernel_timing": "HIP events from a profiled pass over the same steps after the timed one",
    }
    if not args.no_probe:
        out["achievable"] = achievable_fracs(achievable_peaks(), out["roofline"])
    if not args.no_cpu_baseline:
        import oracle
        from threadpoolctl import threadpool_info
        ow = wl.to_oracle(weights)
        t0 = time.perf_counter()
        oracle.decode_steps(x[0].double().numpy(), e[0].double().numpy(), ow["W_g"], ow["W_u"],
                            ow["conv_w"], ow["Proj"], ow["W_0"], w.eta, Bc, update=w.update)
        dt = time.perf_counter() - t0
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        out["cpu_baseline"] = {"value": Bc / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                               "sample": f"decode_steps over one chunk of {Bc} tokens of one sequence, "
                                         f"float64 numpy, {dt:.1f} s", "host": host_info()}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
