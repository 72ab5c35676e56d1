"""Benchmark of the routed-MoE hot path on one MI355X.

One step is one pass over every operation of the path, each on its own
synthetic workload with its inputs resident in HBM:

  grouped GEMM C3   -- skewed MoE FC2: E=128 experts, Zipf(1.1) counts of
                       4096 tokens x top-8 (cum_m=32768, 8 empty experts),
                       k=2048, n=7168, bf16 out: cold, then warm
  grouped GEMM C2   -- uniform: E=8 x 128 rows, k=4096, n=2048, bf16 out
                       (the grouped_mm_bf16 example shape): cold, then warm
  LoRA delta C4     -- T=8192 tokens, top_k=8, E=64, I=2048, H=4096,
                       8 adapters of rank 16, 10% inactive slots: cold, warm
  fold              -- lora_b [8192, 16] for the prepared path
  NVFP4 raw         -- M=4096, N=8192, K=8192, r=16, with bias
  NVFP4 prepared    -- the same call on the folded adapter

"Cold": a 1 GiB scratch write (its own kernel, outside the op's timing)
evicts the L2s and the 256 MB MALL right before the op; "warm": the op runs
again straight after, with whatever its first run left in the caches.

Prints one JSON line.  ``value`` is the metric's grouped-GEMM half on the
largest grouped workload: C3 TFLOP/s, cold (mean over the timed steps);
``config`` carries the metric's other half (the LoRA delta's GB/s and % of
HBM peak) and ``ops`` every operation's own figures.  Op times come from HIP
events recorded on the stream the library launches on.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "grouped-GEMM TFLOP/s (% bf16 MFMA peak); LoRA-delta GB/s (% HBM peak)"
PEAK_MFMA_TFLOPS = 2516.6   # bf16 / fp16 dense MFMA, MI355X
PEAK_HBM_GBPS = 8000.0      # HBM3E
FLUSH_BYTES = 1 << 30       # scratch write that evicts L2 and MALL before a cold op
COPY_PROBE_BYTES = 512 << 20  # per direction
CSRC = os.path.join(ROOT, "moe_expert_grouped_amd", "csrc")

# Ops whose dominant kernel has a committed HBM-traffic summary (two rocprofv3
# --pmc passes, FETCH_SIZE then WRITE_SIZE, scaled on the copy probe).  The
# summary is used only while the kernel's source file is unchanged.
TRAFFIC = {
    "grouped_gemm_c3": dict(
        kernel="grouped_mm_dma_kernel", src="grouped_mm.hip",
        file="profiles/grouped_mm_dma_kernel_e128_zipf_k2048_n7168_traffic.txt",
        what="grouped_mm_dma_kernel, skewed MoE FC2 (E=128, cum_m=32768 Zipf 1.1, k=2048, "
             "n=7168, bf16 out), cold"),
    "grouped_gemm_c2": dict(
        kernel="grouped_mm_dma64_kernel", src="grouped_mm.hip",
        file="profiles/grouped_mm_dma64_kernel_e8_m128_k4096_n2048_traffic.txt",
        what="grouped_mm_dma64_kernel, uniform grouped GEMM (E=8 x 128 rows, k=4096, "
             "n=2048, bf16 out), cold"),
    "nvfp4_raw": dict(
        kernel="nvfp4_lora_kernel", src="nvfp4_lora.hip",
        file="profiles/nvfp4_lora_kernel_m4096_n8192_k8192_traffic.txt",
        what="nvfp4_lora_kernel, M=4096 N=8192 K=8192 r=16 (raw path)"),
    # the delta is four launches: its bytes per call are the sum of theirs
    "lora_delta": dict(
        kernel=["plan_kernel", "list_kernel", "shrink_le_kernel", "expand_kernel"],
        src="lora_delta.hip",
        file="profiles/fc2_lora_delta_t8192_k8_e64_h4096_r16_traffic.txt",
        what="FC2 LoRA delta (plan, list, shrink by (adapter, expert), expand), T=8192 "
             "top_k=8 E=64 H=4096 8 adapters r=16, bf16 out, cold and warm calls"),
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true", help="skip the ops timed outside the step")
    p.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay of the step")
    p.add_argument("--only", default="", help="comma list of step ops to run (profiling aid); "
                   "'copy_probe' (not part of the step) is a 512 MiB fp32 negation (read + "
                   "write) that calibrates the HBM byte counters; extra-op names ("
                   "'grouped_gemm_c3_alone', 'finalize', 'permute', 'nvfp4_grouped', "
                   "'fp4_quantize', 'fc1_lora_delta', 'fc1_swiglu') time the ops outside the step")
    p.add_argument("--pmc-summary", nargs=3, metavar=("OP", "FETCH_DIR", "WRITE_DIR"),
                   help="no GPU: turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                   "'--only OP,copy_probe' into the committed traffic summary of OP "
                   f"(one of {sorted(TRAFFIC)})")
    p.add_argument("--pmc-table", nargs=3, metavar=("OUT_MD", "FETCH_DIR", "WRITE_DIR"),
                   help="no GPU: per-kernel HBM bytes of every library kernel in two rocprofv3 "
                   "--pmc runs (FETCH_SIZE, WRITE_SIZE), calibrated on the copy probe")
    p.add_argument("--trace-summary", nargs=3, metavar=("OUT_MD", "TRACE_DIR", "COMMAND"),
                   help="no GPU: per-kernel durations from a rocprofv3 --kernel-trace run of "
                   "bench.py (COMMAND is the command line that made it, quoted)")
    return p.parse_args()


def src_hash(src: str) -> str:
    return hashlib.sha256(open(os.path.join(CSRC, src), "rb").read()).hexdigest()[:16]


def read_traffic(op: str):
    """HBM bytes per launch of the op's kernel from its committed PMC summary,
    or None when there is none or the kernel source changed since."""
    t = TRAFFIC.get(op)
    if t is None:
        return None
    path = os.path.join(ROOT, t["file"])
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.split("#")[0].strip()
    if kv.get("kernel_source_sha256_16") != src_hash(t["src"]):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# algorithmic work (flops, bytes) per call
# ---------------------------------------------------------------------------
def grouped_work(cum_m, k, n, counts, out_bytes=2):
    nonempty = int((np.asarray(counts) > 0).sum())
    flops = 2.0 * n * k * cum_m
    nbytes = 2.0 * cum_m * k + 2.0 * n * k * nonempty + out_bytes * cum_m * n + 4.0 * (len(counts) + 1)
    return flops, nbytes


def delta_work(perm, lids, eids, T, top_k, E, I, H, rank):
    perm = perm.reshape(T, top_k)
    act_mask = (perm >= 0) & (lids[:, None] >= 0)
    n_active = int(act_mask.sum())
    keys = {(int(l), int(e)) for l, e in zip(np.broadcast_to(lids[:, None], eids.shape)[act_mask],
                                             eids[act_mask])}
    nbytes = 2.0 * I * n_active + 2.0 * (rank * I + H * rank) * len(keys) + 2.0 * T * H + \
        12.0 * T * top_k + 4.0 * T + 16.0 * E
    flops = n_active * (2.0 * rank * I + 2.0 * H * rank)
    return flops, nbytes, n_active


def nvfp4_work(M, N, K, r):
    flops = 2.0 * M * N * K + 2.0 * M * N * r
    nbytes = M * K / 2 + N * K / 2 + (M + N) * K / 16 + 2.0 * M * N + 2.0 * (M + N) * r + 2.0 * N
    return flops, nbytes


# ---------------------------------------------------------------------------
# profile summaries (no GPU)
# ---------------------------------------------------------------------------
def _csv_rows(d, pattern):
    files = glob.glob(os.path.join(d, "**", pattern), recursive=True)
    if not files:
        raise SystemExit(f"no {pattern} under {d}")
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    return rows


def _pmc_avg(rows, counter, pick):
    vals = [float(r["Counter_Value"]) for r in rows
            if r["Counter_Name"] == counter and pick(r["Kernel_Name"])]
    if not vals:
        raise SystemExit(f"no {counter} rows for the requested kernel")
    return sum(vals) / len(vals), len(vals)


def _is_copy(k):
    return "at::native" in k and "neg_kernel" in k


def _short(k):
    k = k.replace("void ", "").replace("mi::(anonymous namespace)::", "")
    return k[:k.index("(")] if "(" in k else k


def pmc_summary(op, fetch_dir, write_dir):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the op's kernel, each
    scaled by what the same counter reads for the copy probe of known size."""
    t = TRAFFIC[op]
    names = t["kernel"] if isinstance(t["kernel"], list) else [t["kernel"]]
    fr = _csv_rows(fetch_dir, "*counter_collection.csv")
    wr = _csv_rows(write_dir, "*counter_collection.csv")
    k_f = k_w = 0.0
    n_kf = n_kw = 0
    for nm in names:  # one dispatch of each kernel per call: sum their averages
        if isinstance(t["kernel"], list):
            pick = lambda k, nm=nm: _short(k).startswith(nm) and "true" not in _short(k)
        else:
            pick = lambda k, nm=nm: nm in k and "true" not in _short(k)
        f, nf = _pmc_avg(fr, "FETCH_SIZE", pick)
        w, nw = _pmc_avg(wr, "WRITE_SIZE", pick)
        k_f, k_w, n_kf, n_kw = k_f + f, k_w + w, n_kf + nf, n_kw + nw
    cp_f, n_cf = _pmc_avg(fr, "FETCH_SIZE", _is_copy)
    cp_w, n_cw = _pmc_avg(wr, "WRITE_SIZE", _is_copy)
    f_fac = COPY_PROBE_BYTES / (cp_f * 1024.0)
    w_fac = COPY_PROBE_BYTES / (cp_w * 1024.0)
    fetch_b = k_f * 1024.0 * f_fac
    write_b = k_w * 1024.0 * w_fac
    out = os.path.join(ROOT, t["file"])
    with open(out, "w") as fh:
        fh.write(f"# HBM traffic of {t['what']}\n"
                 "# commands (repo root, one MI355X; each pass its own run):\n"
                 f"#   rocprofv3 --pmc FETCH_SIZE -d <FETCH_DIR> -o f --output-format csv -- "
                 f"python3 bench.py --only {op},copy_probe --steps 3 --warmup 1 "
                 "--no-cpu-baseline --no-extra --no-graph\n"
                 f"#   rocprofv3 --pmc WRITE_SIZE -d <WRITE_DIR> -o w --output-format csv -- "
                 f"python3 bench.py --only {op},copy_probe --steps 3 --warmup 1 "
                 "--no-cpu-baseline --no-extra --no-graph\n"
                 f"#   python3 bench.py --pmc-summary {op} <FETCH_DIR> <WRITE_DIR>\n"
                 "# Counters are KiB per dispatch; each is scaled by the factor that maps the\n"
                 "# same counter on the copy probe (a 512 MiB fp32 read + 512 MiB write) to its\n"
                 "# known size.\n")
        if len(names) > 1:
            fh.write(f"# per call: the sum over its kernels {', '.join(names)} (one dispatch each)\n")
        fh.write(f"kernel_source_sha256_16 = {src_hash(t['src'])}\n")
        fh.write(f"fetch_kib_per_dispatch = {k_f:.1f}   # {n_kf} dispatches\n")
        fh.write(f"write_kib_per_dispatch = {k_w:.1f}   # {n_kw} dispatches\n")
        fh.write(f"copy_probe_fetch_kib = {cp_f:.1f}   # {n_cf} dispatches\n")
        fh.write(f"copy_probe_write_kib = {cp_w:.1f}   # {n_cw} dispatches\n")
        fh.write(f"fetch_scale = {f_fac:.4f}\nwrite_scale = {w_fac:.4f}\n")
        fh.write(f"hbm_fetch_bytes_per_launch = {fetch_b:.0f}\n")
        fh.write(f"hbm_write_bytes_per_launch = {write_b:.0f}\n")
        fh.write(f"hbm_bytes_per_launch = {fetch_b + write_b:.0f}\n")
    print(f"wrote {out}: {(fetch_b + write_b) / 1e6:.1f} MB per launch "
          f"(fetch scale {f_fac:.3f}, write scale {w_fac:.3f})")


def pmc_table(out_md, fetch_dir, write_dir):
    """FETCH_SIZE / WRITE_SIZE per dispatch of every library kernel of a run,
    scaled like pmc_summary, as a Markdown table."""
    fr = _csv_rows(fetch_dir, "*counter_collection.csv")
    wr = _csv_rows(write_dir, "*counter_collection.csv")
    cp_f, _ = _pmc_avg(fr, "FETCH_SIZE", _is_copy)
    cp_w, _ = _pmc_avg(wr, "WRITE_SIZE", _is_copy)
    f_fac = COPY_PROBE_BYTES / (cp_f * 1024.0)
    w_fac = COPY_PROBE_BYTES / (cp_w * 1024.0)
    names = []
    for r in fr:
        if "mi::" in r["Kernel_Name"] and _short(r["Kernel_Name"]) not in names:
            names.append(_short(r["Kernel_Name"]))
    # keep the hand-written head of OUT_MD, replace any table a previous run wrote
    marker = "Counters are KiB per dispatch,"
    head = open(out_md).read() if os.path.exists(out_md) else ""
    if marker in head:
        head = head[:head.index(marker)].rstrip("\n") + "\n"
    with open(out_md, "w") as fh:
        fh.write(head)
        fh.write(f"\nCounters are KiB per dispatch, scaled by the factors that map the same "
                 f"counters on the copy probe (512 MiB read + 512 MiB written) to its size: "
                 f"fetch {f_fac:.4f}, write {w_fac:.4f}.  They count what the L2 fetches from "
                 "and writes to memory (the MALL included).\n\n"
                 "| kernel | dispatches | fetch MB | write MB | total MB |\n"
                 "|---|---:|---:|---:|---:|\n")
        for n in names:
            pick = lambda k, n=n: "mi::" in k and _short(k) == n
            f, nd = _pmc_avg(fr, "FETCH_SIZE", pick)
            w, _ = _pmc_avg(wr, "WRITE_SIZE", pick)
            fb, wb = f * 1024.0 * f_fac / 1e6, w * 1024.0 * w_fac / 1e6
            fh.write(f"| {n} | {nd} | {fb:.1f} | {wb:.1f} | {fb + wb:.1f} |\n")
    print(f"wrote the table into {out_md}")


def trace_summary(out_md, trace_dir, command):
    """Per-kernel dispatch count and duration (mean/min/max, us) of a
    rocprofv3 kernel trace, library kernels first, in a Markdown file.  For
    kernels that run twice per step (a cold and a warm call, or raw and
    prepared), the eager dispatches are also split by their position in the
    step."""
    import re
    m_s, m_w = re.search(r"--steps\s+(\d+)", command), re.search(r"--warmup\s+(\d+)", command)
    eager = (int(m_s.group(1)) if m_s else 20) + (int(m_w.group(1)) if m_w else 3)
    rows = _csv_rows(trace_dir, "*kernel_trace.csv")
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    per, lib = {}, set()
    for r in rows:
        k = _short(r["Kernel_Name"])
        per.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        if "mi::" in r["Kernel_Name"]:
            lib.add(k)
    with open(out_md, "w") as fh:
        fh.write("# Kernel durations of a bench run (rocprofv3 kernel trace)\n\n"
                 "Command (repo root, one MI355X):\n\n```\n"
                 f"rocprofv3 --kernel-trace --stats -d <DIR> -o trace --output-format csv -- "
                 f"{command}\npython3 bench.py --trace-summary <OUT_MD> <DIR> '<COMMAND>'\n```\n\n"
                 "Durations in microseconds (the trace's end minus start timestamps).  "
                 "`dispatches`, `mean`, `min`, `max` cover every dispatch of the kernel in the "
                 f"run (the {eager} eager steps, the graph replays and the ops timed outside "
                 "the step).  The step calls the grouped GEMMs and the delta twice (cold: after "
                 "a 1 GiB scratch write, then warm) and the NVFP4 kernel twice (raw, then "
                 f"prepared): `step 1st` / `step 2nd` are the means over the first {eager} pairs "
                 "of dispatches of such a kernel, i.e. the eager steps' first and second call.\n\n"
                 "| kernel | dispatches | mean | min | max | step 1st | step 2nd |\n"
                 "|---|---:|---:|---:|---:|---:|---:|\n")
        for k in sorted(per, key=lambda k: -sum(per[k])):
            v = np.asarray(per[k])
            if not (k in lib or v.mean() > 50):
                continue
            first = second = ""
            if len(v) >= 2 * eager:
                first, second = f"{v[:2 * eager:2].mean():.1f}", f"{v[1:2 * eager:2].mean():.1f}"
            fh.write(f"| {k[:90]} | {len(v)} | {v.mean():.1f} | {v.min():.1f} | {v.max():.1f} | "
                     f"{first} | {second} |\n")
    print(f"wrote {out_md}")


# ---------------------------------------------------------------------------
# the run
# ---------------------------------------------------------------------------
def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.pmc_table:
        pmc_table(*args.pmc_table)
        return
    if args.trace_summary:
        trace_summary(*args.trace_summary)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU; --gpus must be 1 (the path is "
                                   "data-parallel per GPU: each GPU runs these kernels on its "
                                   "own share, see the sharding notes)"}))
        sys.exit(2)
    import torch

    import synth
    import moe_expert_grouped_amd as mi

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    only = set(filter(None, args.only.split(",")))

    def want(name):
        return not only or name in only

    def log(msg):
        print(f"# {msg}", file=sys.stderr, flush=True)

    # ---------------- inputs (resident in HBM before timing) ----------------
    need_c3 = want("grouped_gemm_c3") or want("grouped_gemm_c3_warm") or \
        (not args.no_extra and want("grouped_gemm_c3_alone"))
    g3 = synth.grouped_zipf(device=dev) if need_c3 else None
    if g3 is not None:
        out3 = torch.empty((g3.a.shape[0], g3.b.shape[1]), dtype=torch.bfloat16, device=dev)
        c3_counts = np.diff(g3.m_indptr.cpu().numpy())
        c3_work = grouped_work(g3.a.shape[0], g3.a.shape[1], g3.b.shape[1], c3_counts)
    log("C3 inputs ready")
    g2 = synth.grouped_uniform(device=dev)
    out2 = torch.empty((g2.a.shape[0], g2.b.shape[1]), dtype=torch.bfloat16, device=dev)
    c2_work = grouped_work(g2.a.shape[0], g2.a.shape[1], g2.b.shape[1],
                           np.diff(g2.m_indptr.cpu().numpy()))
    dc = synth.delta_at_scale(device=dev)
    wa, wb = mi.fill_w_ptr(dc.A), mi.fill_w_ptr(dc.B)
    sa = dc.E * dc.rank * dc.I
    sb = dc.E * dc.H * dc.rank
    dout = torch.empty((dc.T, dc.H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(mi.delta_workspace_bytes(dc.T, dc.top_k, dc.E, dc.L, dc.rank),
                     dtype=torch.uint8, device=dev)
    perm_h = dc.perm.cpu().numpy()
    d_flops, d_bytes, _ = delta_work(perm_h, dc.lora_ids.cpu().numpy(), dc.topk_ids.cpu().numpy(),
                                     dc.T, dc.top_k, dc.E, dc.I, dc.H, dc.rank)
    nc = synth.nvfp4_lora_case(device=dev)
    nout_raw = torch.empty((nc.M, nc.N), dtype=torch.bfloat16, device=dev)
    nout_prep = torch.empty_like(nout_raw)
    adapter = mi.prepare_nvfp4_lora_adapter(nc.lora_b, nc.lora_scale, nc.alpha)
    nv_w = nvfp4_work(nc.M, nc.N, nc.K, nc.rank)
    fold_w = (float(nc.N * nc.rank), 2.0 * 2 * nc.N * nc.rank + 8)
    flush_buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    log("inputs ready")

    stream = torch.cuda.current_stream(dev)
    c3 = (lambda: mi.grouped_mm_bf16(g3.a, g3.b, g3.m_indptr, out=out3)) if g3 is not None else None
    c2 = lambda: mi.grouped_mm_bf16(g2.a, g2.b, g2.m_indptr, out=out2)
    delta = lambda: mi.bgmv_moe_gemm2_lora_delta(
        dc.act, dc.perm, wa, sa, wb, sb, dc.topk_ids, dc.topk_weights, dc.lora_ids, dc.rank,
        dc.H, num_adapters=dc.L, scale=dc.scale, out=dout, workspace=ws)
    # (name, fn, flush before it, (flops, bytes))
    spec = [
        ("grouped_gemm_c3", c3, True, c3_work if g3 is not None else None),
        ("grouped_gemm_c3_warm", c3, False, c3_work if g3 is not None else None),
        ("grouped_gemm_c2", c2, True, c2_work),
        ("grouped_gemm_c2_warm", c2, False, c2_work),
        ("lora_delta", delta, True, (d_flops, d_bytes)),
        ("lora_delta_warm", delta, False, (d_flops, d_bytes)),
        ("fold", lambda: mi.prepare_nvfp4_lora_adapter(nc.lora_b, nc.lora_scale, nc.alpha,
                                                        out=adapter), False, fold_w),
        ("nvfp4_raw", lambda: mi.mm_nvfp4_lora(nc.a, nc.b, nc.a_sf, nc.b_sf, nc.alpha, nc.d,
                                                nc.lora_b, nc.lora_scale, bias=nc.bias,
                                                out=nout_raw), False, nv_w),
        ("nvfp4_prepared", lambda: mi.mm_nvfp4_lora(nc.a, nc.b, nc.a_sf, nc.b_sf, nc.alpha,
                                                     nc.d, lora_adapter=adapter, bias=nc.bias,
                                                     out=nout_prep), False, nv_w),
    ]
    if "copy_probe" in only:
        cp_src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
        cp_dst = torch.empty_like(cp_src)
        spec.append(("copy_probe", lambda: torch.neg(cp_src, out=cp_dst), False,
                     (0.0, 2.0 * COPY_PROBE_BYTES)))
    spec = [s for s in spec if s[1] is not None and (not only or s[0] in only)]
    work = {name: w for name, _, _, w in spec}

    def flush():
        flush_buf.fill_(1.0)

    def step(ev=None):
        for i, (name, fn, cold, _) in enumerate(spec):
            if cold:
                flush()
            if ev is not None:
                ev[i][0].record(stream)
            fn()
            if ev is not None:
                ev[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in spec] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for s in range(args.steps):
        step(evs[s])
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(stop) / args.steps
    per_op = {name: np.array([evs[s][i][0].elapsed_time(evs[s][i][1])
                              for s in range(args.steps)]) for i, (name, *_) in enumerate(spec)}
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step (host wall {wall:.3f} s)")

    op_report = {}
    for name, ms_all in per_op.items():
        fl, by = work[name]
        ms = float(ms_all.mean())
        sec = ms * 1e-3
        op_report[name] = {
            "ms": round(ms, 5), "ms_min": round(float(ms_all.min()), 5),
            "ms_p90": round(float(np.percentile(ms_all, 90)), 5),
            "tflops": round(fl / sec / 1e12, 2), "gbps": round(by / sec / 1e9, 1),
            "frac_mfma_peak": round(fl / sec / 1e12 / PEAK_MFMA_TFLOPS, 4),
            "frac_hbm_peak": round(by / sec / 1e9 / PEAK_HBM_GBPS, 4),
            "cache": ("warm" if name.endswith("_warm") else
                      "cold (1 GiB scratch write first)" if any(s[0] == name and s[2]
                                                                for s in spec) else "in step"),
            "algorithmic_flops": fl, "algorithmic_bytes": by}

    # roofline of the dominant kernel: the op with the largest mean time; the
    # grouped GEMM on C3 sits below the ridge point (233 flop/B against 315),
    # so HBM bounds it; the NVFP4 GEMM is MFMA-bound
    bounds = {"grouped_gemm_c3": "hbm", "grouped_gemm_c3_warm": "hbm", "grouped_gemm_c2": "hbm",
              "grouped_gemm_c2_warm": "hbm", "lora_delta": "hbm", "lora_delta_warm": "hbm",
              "fold": "hbm", "nvfp4_raw": "mfma", "nvfp4_prepared": "mfma", "copy_probe": "hbm"}
    kernels = {"grouped_gemm_c3": "grouped_mm_dma_kernel", "grouped_gemm_c3_warm":
               "grouped_mm_dma_kernel", "grouped_gemm_c2": "grouped_mm_dma64_kernel",
               "grouped_gemm_c2_warm": "grouped_mm_dma64_kernel", "lora_delta":
               "plan + list + shrink_le + expand kernels", "lora_delta_warm":
               "plan + list + shrink_le + expand kernels", "fold": "fold_kernel",
               "nvfp4_raw": "nvfp4_lora_kernel", "nvfp4_prepared": "nvfp4_lora_kernel",
               "copy_probe": "torch neg"}

    def roof(name):
        r = op_report[name]
        fl, by = work[name]
        sec = r["ms"] * 1e-3
        if bounds[name] == "mfma":
            ach, peak, unit = fl / sec / 1e12, PEAK_MFMA_TFLOPS, "TFLOP/s"
        else:
            ach, peak, unit = by / sec / 1e9, PEAK_HBM_GBPS, "GB/s"
        return {"op": name, "kernel": kernels[name], "bound": bounds[name],
                "achieved": round(ach, 1), "peak": peak, "unit": unit,
                "frac": round(ach / peak, 4), "traffic": read_traffic(name),
                "algorithmic": by if bounds[name] == "hbm" else fl}

    # the kernel that takes most of the step is the C3 grouped GEMM (cold and
    # warm calls of one kernel); its cold call is the one `value` measures
    timed = [n for n in op_report if n != "copy_probe"]
    lead = "grouped_gemm_c3" if "grouped_gemm_c3" in op_report else \
        (max(timed, key=lambda n: op_report[n]["ms"]) if timed else None)
    roofline = roof(lead) if lead else None
    other_rooflines = [roof(n) for n in ("nvfp4_raw", "lora_delta", "grouped_gemm_c2")
                       if n in op_report and (roofline is None or n != roofline["op"])]

    # The same step captured once in a HIP graph and replayed: the calls do no
    # host read, allocation or memset, so the capture holds the step's kernels
    # and the launch gaps of the eager step drop out.  Informational only.
    step_graph = None
    if not only and not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        gms = g0.elapsed_time(g1) / args.steps
        step_graph = {"ms_per_step": round(gms, 4),
                      "note": "the step (flushes included) captured once in a HIP graph, "
                              "replayed back to back"}
        del graph
        log(f"graph replay: {gms:.3f} ms/step")

    extra = None if args.no_extra else extra_ops(args, only, dev, stream, mi, synth, dc, wa, wb,
                                                  sa, sb, perm_h, d_flops, d_bytes, g3,
                                                  c3 if g3 is not None else None,
                                                  c3_work if g3 is not None else None)

    cpu = accuracy = None
    if not args.no_cpu_baseline and not only:
        cpu, accuracy = cpu_baseline(g3, dc, nc, wa, wb, sa, sb, nout_raw, nout_prep, adapter)

    head = op_report.get("grouped_gemm_c3") or op_report.get("grouped_gemm_c2") or {}
    dl = op_report.get("lora_delta", {})
    line = {
        "metric": METRIC,
        "value": head.get("tflops"),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "moe-fc2-lora hot path; value: ragged grouped GEMM on the skewed MoE FC2 "
                        "(E=128, cum_m=32768 Zipf(1.1) over 4096 tokens x top-8, 8 empty "
                        "experts, k=2048, n=7168, bf16 out), cold (1 GiB scratch write before "
                        "each call); the step also runs it warm, the uniform grouped GEMM (E=8 x "
                        "128 rows, k=4096, n=2048) cold and warm, the FC2 LoRA delta (T=8192, "
                        "top_k=8, E=64, I=2048, H=4096, 8 adapters r=16) cold and warm, the fold "
                        "and NVFP4+LoRA raw and prepared (M=4096, N=8192, K=8192, r=16)",
            "value_definition": "grouped-GEMM algorithmic TFLOP/s (2*cum_m*n*k / mean event time "
                                "of the cold call)",
            "grouped_gemm_tflops": head.get("tflops"),
            "grouped_gemm_frac_bf16_mfma_peak": head.get("frac_mfma_peak"),
            "grouped_gemm_frac_hbm_peak": head.get("frac_hbm_peak"),
            "lora_delta_gbps": dl.get("gbps"),
            "lora_delta_frac_hbm_peak": dl.get("frac_hbm_peak"),
            "ms_per_step_note": "the whole step: three 1 GiB flushes plus every op",
            "parallelism": "single GPU",
        },
        "ops": op_report,
        "extra_ops": extra,
        "step_graph": step_graph,
        "roofline": roofline,
        "other_rooflines": other_rooflines,
        "accuracy_nvfp4": accuracy,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def extra_ops(args, only, dev, stream, mi, synth, dc, wa, wb, sa, sb, perm_h, d_flops, d_bytes,
              g3, c3, c3_work):
    """Ops outside the step, each timed on its own with events, back to back."""
    import torch

    def want(name):
        return not only or name in only

    def time_alone(fn):
        for _ in range(3):
            fn()
        fe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        torch.cuda.synchronize()
        for a_, b_ in fe:
            a_.record(stream)
            fn()
            b_.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a_.elapsed_time(b_) for a_, b_ in fe]))

    def entry(ms, nbytes, note, flops=None):
        e = {"ms": round(ms, 5), "gbps": round(nbytes / ms / 1e6, 1),
             "frac_hbm_peak": round(nbytes / ms / 1e6 / PEAK_HBM_GBPS, 4),
             "algorithmic_bytes": nbytes, "note": note}
        if flops is not None:
            e["tflops"] = round(flops / ms / 1e9, 2)
            e["frac_mfma_peak"] = round(flops / ms / 1e9 / PEAK_MFMA_TFLOPS, 4)
            e["algorithmic_flops"] = flops
        return e

    extra = {}
    if c3 is not None and want("grouped_gemm_c3_alone"):
        ms = time_alone(c3)
        extra["grouped_gemm_c3_back_to_back"] = entry(
            ms, c3_work[1], "the C3 grouped GEMM repeated back to back (no flush)", c3_work[0])
    if want("finalize"):
        fc2 = synth.bf16_normal((dc.act.shape[0], dc.H), 1.0, synth.gen(77, dev), dev)
        fout = torch.empty((dc.T, dc.H), dtype=torch.bfloat16, device=dev)
        fws = torch.empty(mi.finalize_workspace_bytes(dc.T, dc.top_k, dc.E, dc.L, dc.rank, dc.H),
                          dtype=torch.uint8, device=dev)
        fms = time_alone(lambda: mi.moe_finalize_lora(
            fc2, dc.act, dc.perm, wa, sa, wb, sb, dc.topk_ids, dc.topk_weights, dc.lora_ids,
            dc.rank, dc.H, num_adapters=dc.L, scale=dc.scale, out=fout, workspace=fws))
        n_routed = int((perm_h >= 0).sum())
        extra["finalize_fused"] = entry(
            fms, d_bytes + 2.0 * dc.H * n_routed,
            "MoE finalize (weighted combine of the routed FC2 rows) with the LoRA delta added, "
            "delta workload, two passes (fp32 delta in the workspace, then the combine)",
            d_flops + 2.0 * dc.H * n_routed)
        del fc2, fout, fws
    if want("permute"):
        nslot = dc.T * dc.top_k
        rws = torch.empty(mi.route_workspace_bytes(nslot, dc.E), dtype=torch.uint8, device=dev)
        rms = time_alone(lambda: mi.moe_route_permutation(dc.topk_ids, dc.E, with_inverse=True,
                                                          workspace=rws))
        extra["route_permutation"] = entry(
            rms, 12.0 * nslot + 4.0 * (dc.E + 1),
            "topk_ids [8192, 8] -> m_indptr, expanded_idx_to_permuted_idx and its inverse "
            "(E=64); three launches, latency-bound at this size")
        _, rperm = mi.moe_route_permutation(dc.topk_ids, dc.E)
        xtok = synth.bf16_normal((dc.T, dc.H), 1.0, synth.gen(78, dev), dev)
        xperm = torch.empty((nslot, dc.H), dtype=torch.bfloat16, device=dev)
        pms = time_alone(lambda: mi.moe_permute_rows(xtok, rperm, dc.top_k, out=xperm))
        extra["permute_rows"] = entry(
            pms, 2.0 * dc.H * (dc.T + nslot) + 4.0 * nslot,
            "token rows bf16 [8192, 4096] -> permuted rows [65536, 4096] (each token row read "
            "once, written top_k times)")
        del xtok, xperm
    if want("nvfp4_grouped"):
        ng = synth.nvfp4_grouped_case(device=dev)
        ngo = torch.empty((ng.a.shape[0], ng.b.shape[1]), dtype=torch.bfloat16, device=dev)
        gms = time_alone(lambda: mi.grouped_mm_nvfp4(ng.a, ng.a_sf, ng.b, ng.b_sf, ng.m_indptr,
                                                     ng.alpha, out=ngo))
        cnts = np.diff(ng.m_indptr.cpu().numpy())
        nn, kk = ng.b.shape[1], ng.k
        per_e = ng.b_sf.numel() // ng.b.shape[0]
        gbytes = ng.a.numel() + ng.a_sf.numel() + (nn * kk / 2 + per_e) * int((cnts > 0).sum()) + \
            2.0 * ng.a.shape[0] * nn + 4.0 * (len(cnts) + 1) + 4.0 * len(cnts)
        extra["nvfp4_grouped"] = entry(
            gms, gbytes, "NVFP4 grouped GEMM, E=128 Zipf(1.1) routing of 4096 tokens x top-8 "
            "(cum_m=32768), n=7168, k=2048, per-expert alpha, bf16 out; the fp16 MFMA peak is "
            "the denominator", 2.0 * ng.a.shape[0] * nn * kk)
        del ng, ngo
    if want("fp4_quantize"):
        # NVFP4 quantisation of the skewed MoE FC2 activations [32768, 2048] bf16
        xq = synth.bf16_normal((32768, 2048), 1.0, synth.gen(79, dev), dev)
        gq = torch.tensor([448.0 * 6.0 / float(xq.float().abs().max())], dtype=torch.float32,
                          device=dev)
        qc = torch.empty((32768, 1024), dtype=torch.uint8, device=dev)
        qs = torch.empty(256 * 32 * 512, dtype=torch.uint8, device=dev)
        qms = time_alone(lambda: mi.fp4_quantize(xq, gq, codes=qc, sf=qs))
        extra["fp4_quantize"] = entry(
            qms, 2.0 * xq.numel() + qc.numel() + qs.numel(),
            "NVFP4 quantisation of bf16 [32768, 2048] (the skewed MoE FC2 activations): codes "
            "and 128x4 UE4M3 scales")
        del xq, qc, qs
    if want("fc1_lora_delta"):
        # FC1 LoRA delta on the delta workload's routing (T=8192, top_k=8, E=64,
        # 8 adapters r=16): hidden 4096 in, 4096 gate/up columns out
        f1 = synth.delta_at_scale(device=dev, I=4096, H=4096)
        fwa, fwb = mi.fill_w_ptr(f1.A), mi.fill_w_ptr(f1.B)
        fsa, fsb = f1.E * f1.rank * f1.I, f1.E * f1.H * f1.rank
        f1o = torch.zeros((f1.act.shape[0], f1.H), dtype=torch.bfloat16, device=dev)
        f1w = torch.empty(mi.delta_workspace_bytes(f1.T, f1.top_k, f1.E, f1.L, f1.rank),
                          dtype=torch.uint8, device=dev)
        f1ms = time_alone(lambda: mi.moe_fc1_lora_delta(
            f1.act, f1.perm, fwa, fsa, fwb, fsb, f1.topk_ids, f1.lora_ids, f1.rank, f1.H,
            num_adapters=f1.L, scale=f1.scale, out=f1o, workspace=f1w))
        pr = f1.perm.cpu().numpy().reshape(f1.T, f1.top_k)
        lid = f1.lora_ids.cpu().numpy()
        eid = f1.topk_ids.cpu().numpy()
        act_m = (pr >= 0) & (lid[:, None] >= 0)
        keys = {(int(l), int(e)) for l, e in zip(np.broadcast_to(lid[:, None], eid.shape)[act_m],
                                                 eid[act_m])}
        n_act, n_rows = int(act_m.sum()), int((pr >= 0).sum())
        f1bytes = 2.0 * f1.I * n_act + 2.0 * (f1.rank * f1.I + f1.H * f1.rank) * len(keys) + \
            2.0 * f1.H * n_rows + 8.0 * f1.T * f1.top_k + 4.0 * f1.T
        extra["fc1_lora_delta"] = entry(
            f1ms, f1bytes, "FC1 LoRA delta, delta workload routing (T=8192, top_k=8, E=64, 8 "
            "adapters r=16), hidden 4096 -> 4096 gate/up columns, one bf16 row per routed slot",
            n_act * (2.0 * f1.rank * f1.I + 2.0 * f1.H * f1.rank))
        del f1, f1o, f1w
    if want("fc1_swiglu"):
        fc = synth.fc1_case(device=dev)
        fco = torch.empty((fc.a.shape[0], fc.b.shape[1] // 2), dtype=torch.bfloat16, device=dev)
        fms = time_alone(lambda: mi.grouped_mm_swiglu(fc.a, fc.b, fc.m_indptr, out=fco))
        cnts = np.diff(fc.m_indptr.cpu().numpy())
        cm, hid, two_i = fc.a.shape[0], fc.a.shape[1], fc.b.shape[1]
        fbytes = 2.0 * cm * hid + 2.0 * two_i * hid * int((cnts > 0).sum()) + \
            2.0 * cm * two_i / 2 + 4.0 * (len(cnts) + 1)
        extra["fc1_swiglu"] = entry(
            fms, fbytes, "FC1 gate/up grouped GEMM with the SwiGLU epilogue, E=128 Zipf(1.1) "
            "routing (cum_m=32768), hidden=7168, inter=2048, bf16; weights read once per expert "
            "(7.3 GB)", 2.0 * cm * two_i * hid)
        del fc, fco
    return extra or None


def cpu_baseline(g3, dc, nc, wa, wb, sa, sb, nout_raw, nout_prep, adapter):
    """The fp64 oracle, as it stands, on a bounded sample of the same
    workloads; and the NVFP4 accuracy figures against it."""
    import torch

    from oracle import nvfp4 as NV
    from oracle.fold import fold
    from oracle.grouped_mm import grouped_mm
    from oracle.lora_delta import Bank, moe_fc2_lora_delta

    def bits(t):
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            cores = min(cores, max(blas))
    except Exception:
        pass
    cpu = {"unit": "TFLOP/s", "cores": cores, "kind": "oracle"}
    # grouped GEMM on the skewed MoE FC2 workload: the oracle over whole
    # experts, in expert order, until 10 s of oracle time (at most 4 passes
    # over the whole workload)
    if g3 is not None:
        mi_h = g3.m_indptr.cpu().numpy().astype(np.int64)
        k, n = g3.a.shape[1], g3.b.shape[1]
        flops, t_tot, calls, rows = 0.0, 0.0, 0, 0
        nonempty = [e for e in range(len(mi_h) - 1) if mi_h[e + 1] > mi_h[e]]
        for e in nonempty * 4:
            s, t = int(mi_h[e]), int(mi_h[e + 1])
            a_e, b_e = bits(g3.a[s:t]), bits(g3.b[e:e + 1])
            t0 = time.perf_counter()
            grouped_mm(a_e, b_e, np.array([0, t - s]))
            t_tot += time.perf_counter() - t0
            flops += 2.0 * (t - s) * n * k
            calls += 1
            rows += t - s
            if t_tot >= 10.0:
                break
        cpu.update({"value": round(flops / t_tot / 1e12, 5), "seconds": round(t_tot, 2),
                    "sample": f"grouped GEMM oracle, one call per non-empty expert in expert "
                              f"order over the skewed MoE FC2 workload ({calls} calls, "
                              f"{rows} rows; 120 calls and 32768 rows make one pass); "
                              "algorithmic flops / oracle time"})
    # LoRA delta on the first tokens of its workload, until 3 s
    act = bits(dc.act)
    ba = Bank(bits(dc.A.reshape(-1)), dc.A.data_ptr())
    bb = Bank(bits(dc.B.reshape(-1)), dc.B.data_ptr())
    perm = dc.perm.cpu().numpy()
    lids = dc.lora_ids.cpu().numpy()
    wa_h, wb_h = wa.cpu().numpy(), wb.cpu().numpy()
    ids_h, w_h = dc.topk_ids.cpu().numpy(), dc.topk_weights.cpu().numpy()
    done, t_tot = 0, 0.0
    while done < dc.T and t_tot < 3.0:
        toks = list(range(done, min(dc.T, done + 256)))
        t0 = time.perf_counter()
        moe_fc2_lora_delta(act, perm, ba, wa_h, sa, bb, wb_h, sb, ids_h, w_h, lids, dc.rank, dc.H,
                           dc.scale, tokens=toks)
        t_tot += time.perf_counter() - t0
        done += len(toks)
    pr = perm.reshape(dc.T, dc.top_k)[:done]
    n_act = int(((pr >= 0) & (lids[:done, None] >= 0)).sum())
    sample_bytes = 2.0 * dc.I * n_act + 2.0 * dc.H * done
    cpu["lora_delta"] = {"value": round(sample_bytes / t_tot / 1e9, 4), "unit": "GB/s",
                         "seconds": round(t_tot, 2),
                         "sample": f"delta oracle over the first {done} of {dc.T} tokens; "
                                   "gathered activation rows + output bytes / oracle time"}
    # NVFP4 accuracy against the fp64 formula, on 32 rows x 128 columns
    rng = np.random.default_rng(1)
    rows = np.sort(np.concatenate([[0, nc.M - 1], rng.choice(nc.M, 30, replace=False)]))
    cols = np.sort(np.concatenate([[0, nc.N - 1], rng.choice(nc.N, 126, replace=False)]))
    base = NV.base_product(nc.a.cpu().numpy()[rows], nc.b.cpu().numpy()[cols],
                           nc.a_sf.cpu().numpy(), nc.b_sf.cpu().numpy(), nc.K, rows, cols)
    alpha, s = float(nc.alpha[0]), float(nc.lora_scale[0])
    d_h, lb_h, bias_h = bits(nc.d)[rows], bits(nc.lora_b)[cols], bits(nc.bias)[cols]
    ref_raw = NV.mm_nvfp4_raw(base, alpha, d_h, lb_h, s, bias_h)
    fb, zero = fold(bits(nc.lora_b), s, alpha)
    ref_prep = NV.mm_nvfp4_prepared(base, alpha, d_h, fb[cols], zero, bias_h)
    rt, ct = torch.from_numpy(rows).to(nout_raw.device), torch.from_numpy(cols).to(nout_raw.device)
    sel = lambda t: t.index_select(0, rt).index_select(1, ct).double().cpu().numpy()
    g_raw, g_prep = sel(nout_raw), sel(nout_prep)

    def sqnr(g, r):
        return round(float(10 * np.log10(np.sum(r ** 2) / max(np.sum((g - r) ** 2), 1e-300))), 2)

    accuracy = {
        "sample": "NVFP4+LoRA M=4096 N=8192 K=8192 r=16: 32 rows x 128 columns (row/column 0 and "
                  "the last included), against the fp64 oracle",
        "sqnr_db_raw": sqnr(g_raw, ref_raw),
        "max_abs_err_raw": round(float(np.abs(g_raw - ref_raw).max()), 5),
        "sqnr_db_prepared_vs_raw_formula": sqnr(g_prep, ref_raw),
        "max_abs_err_prepared_vs_raw_formula": round(float(np.abs(g_prep - ref_raw).max()), 5),
        "sqnr_db_prepared_vs_prepared_formula": sqnr(g_prep, ref_prep),
        "max_abs_err_prepared_vs_prepared_formula": round(float(np.abs(g_prep - ref_prep).max()),
                                                          5),
        "rms_output": round(float(np.sqrt(np.mean(ref_raw ** 2))), 4),
        "pages_context": "mm_nvfp4_lora (prepared-path bullet) quotes SQNR 53.8 dB prepared / "
                         "55.6 dB raw and max |err| vs fp64 of 0.038-0.042 / 0.031 on rows it "
                         "does not describe (no hardware stated); not comparable workloads",
    }
    return cpu, accuracy


if __name__ == "__main__":
    main()
