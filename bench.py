"""Benchmark of the routed-MoE hot path on one MI355X.

One step is one pass over every operation of the path, each on its own
synthetic workload, inputs resident in HBM:

  1. grouped GEMM   -- uniform MoE: E=8 experts x 128 rows, k=4096, n=2048,
                       bf16 out (the grouped_mm_bf16 example shape)
  2. LoRA delta     -- T=8192 tokens, top_k=8, E=64, I=2048, H=4096,
                       8 adapters of rank 16, 10% inactive slots
  3. fold           -- lora_b [8192, 16] for the prepared path
  4. NVFP4 raw      -- M=4096, N=8192, K=8192, r=16, with bias
  5. NVFP4 prepared -- the same call on the folded adapter

Prints one JSON line.  ``value`` is the whole step's algorithmic TFLOP/s;
``ops`` carries each operation's own figures (TFLOP/s and % of the bf16 MFMA
peak for the GEMMs, GB/s and % of HBM peak for the delta).  Op times come
from HIP events recorded on the stream the library launches on.
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

METRIC = "grouped-GEMM TFLOP/s (% bf16 MFMA peak); LoRA-delta GB/s (% HBM peak)"
PEAK_MFMA_TFLOPS = 2516.6   # bf16 / fp16 dense MFMA, MI355X
PEAK_HBM_GBPS = 8000.0      # HBM3E
KERNEL_SRC = os.path.join(ROOT, "moe_expert_grouped_amd", "csrc", "nvfp4_lora.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "nvfp4_lora_kernel_m4096_n8192_k8192_traffic.txt")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only", default="", help="comma list of ops to run (profiling aid); "
                   "'copy_probe' (not part of the step) is a 512 MiB fp32 negation (read + write) used to "
                   "calibrate the HBM byte counters; 'finalize', 'permute', 'nvfp4_grouped' and "
                   "'fc1_swiglu' time the ops outside the step")
    p.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="no GPU: turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                   "'--only nvfp4_raw,copy_probe' into the committed traffic summary")
    p.add_argument("--pmc-table", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="no GPU: per-kernel HBM bytes from two rocprofv3 --pmc runs (FETCH_SIZE, "
                   "WRITE_SIZE) of '--only grouped_gemm,lora_delta,copy_probe', calibrated on "
                   "the copy probe")
    return p.parse_args()


def src_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch of the NVFP4 kernel from the committed PMC summary,
    or None when the kernel source changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != src_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


COPY_PROBE_BYTES = 512 << 20  # per direction


def _pmc_rows(d):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
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


def pmc_summary(fetch_dir, write_dir):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the NVFP4 kernel, each
    scaled by what the same counter reads for the copy probe of known size."""
    is_nv = lambda k: "nvfp4_lora_kernel" in k
    is_copy = lambda k: "at::native" in k and "neg_kernel" in k
    fr, wr = _pmc_rows(fetch_dir), _pmc_rows(write_dir)
    nv_f, n_nf = _pmc_avg(fr, "FETCH_SIZE", is_nv)
    cp_f, n_cf = _pmc_avg(fr, "FETCH_SIZE", is_copy)
    nv_w, n_nw = _pmc_avg(wr, "WRITE_SIZE", is_nv)
    cp_w, n_cw = _pmc_avg(wr, "WRITE_SIZE", is_copy)
    f_fac = COPY_PROBE_BYTES / (cp_f * 1024.0)
    w_fac = COPY_PROBE_BYTES / (cp_w * 1024.0)
    fetch_b = nv_f * 1024.0 * f_fac
    write_b = nv_w * 1024.0 * w_fac
    out = os.path.join(ROOT, "profiles", os.path.basename(TRAFFIC_FILE))
    with open(out, "w") as fh:
        fh.write("# HBM traffic of nvfp4_lora_kernel, M=4096 N=8192 K=8192 r=16 (raw path)\n"
                 "# commands (repo root, one MI355X; each pass its own run):\n"
                 "#   rocprofv3 --pmc FETCH_SIZE -d <FETCH_DIR> -o f --output-format csv -- "
                 "python3 bench.py --only nvfp4_raw,copy_probe --steps 3 --warmup 1\n"
                 "#   rocprofv3 --pmc WRITE_SIZE -d <WRITE_DIR> -o w --output-format csv -- "
                 "python3 bench.py --only nvfp4_raw,copy_probe --steps 3 --warmup 1\n"
                 "#   python3 bench.py --pmc-summary <FETCH_DIR> <WRITE_DIR>\n"
                 "# Counters are KiB per dispatch; each is scaled by the factor that maps the\n"
                 "# same counter on the copy probe (a 512 MiB fp32 read + 512 MiB write) to its\n"
                 "# known size.  Algorithmic bytes per launch: 124141568.\n")
        fh.write(f"kernel_source_sha256_16 = {src_hash()}\n")
        fh.write(f"fetch_kib_per_dispatch = {nv_f:.1f}   # {n_nf} dispatches\n")
        fh.write(f"write_kib_per_dispatch = {nv_w:.1f}   # {n_nw} dispatches\n")
        fh.write(f"copy_probe_fetch_kib = {cp_f:.1f}   # {n_cf} dispatches\n")
        fh.write(f"copy_probe_write_kib = {cp_w:.1f}   # {n_cw} dispatches\n")
        fh.write(f"fetch_scale = {f_fac:.4f}\nwrite_scale = {w_fac:.4f}\n")
        fh.write(f"hbm_fetch_bytes_per_launch = {fetch_b:.0f}\n")
        fh.write(f"hbm_write_bytes_per_launch = {write_b:.0f}\n")
        fh.write(f"hbm_bytes_per_launch = {fetch_b + write_b:.0f}\n")
    print(f"wrote {out}: {(fetch_b + write_b) / 1e6:.1f} MB per launch "
          f"(fetch scale {f_fac:.3f}, write scale {w_fac:.3f})")


def pmc_table(fetch_dir, write_dir):
    """FETCH_SIZE / WRITE_SIZE per dispatch of every library kernel of the
    grouped-GEMM and delta run, scaled like pmc_summary, as a Markdown table."""
    is_copy = lambda k: "at::native" in k and "neg_kernel" in k
    fr, wr = _pmc_rows(fetch_dir), _pmc_rows(write_dir)
    cp_f, _ = _pmc_avg(fr, "FETCH_SIZE", is_copy)
    cp_w, _ = _pmc_avg(wr, "WRITE_SIZE", is_copy)
    f_fac = COPY_PROBE_BYTES / (cp_f * 1024.0)
    w_fac = COPY_PROBE_BYTES / (cp_w * 1024.0)

    def short(k):
        k = k.replace("void ", "").replace("mi::(anonymous namespace)::", "")
        return k[:k.index("(")] if "(" in k else k

    names = []
    for r in fr:
        if "mi::" in r["Kernel_Name"] and short(r["Kernel_Name"]) not in names:
            names.append(short(r["Kernel_Name"]))
    out = os.path.join(ROOT, "profiles", "grouped_gemm_c2_and_delta_c4_hbm_traffic.md")
    with open(out, "w") as fh:
        fh.write("# HBM traffic per kernel: grouped GEMM (E=8 x 128 rows, k=4096, n=2048) and "
                 "the FC2 LoRA delta (T=8192, top_k=8, E=64, I=2048, H=4096, 8 adapters r=16)\n\n"
                 "Commands (repo root, one MI355X; each pass its own run):\n\n```\n"
                 "rocprofv3 --pmc FETCH_SIZE -d <FETCH_DIR> -o f --output-format csv -- python3 "
                 "bench.py --only grouped_gemm,lora_delta,copy_probe --steps 3 --warmup 1 "
                 "--no-cpu-baseline\n"
                 "rocprofv3 --pmc WRITE_SIZE -d <WRITE_DIR> -o w --output-format csv -- python3 "
                 "bench.py --only grouped_gemm,lora_delta,copy_probe --steps 3 --warmup 1 "
                 "--no-cpu-baseline\n"
                 "python3 bench.py --pmc-table <FETCH_DIR> <WRITE_DIR>\n```\n\n"
                 "Counters are KiB per dispatch, scaled by the factors that map the same counters "
                 f"on the copy probe (512 MiB read + 512 MiB written) to its size: fetch "
                 f"{f_fac:.4f}, write {w_fac:.4f}.  They count what the L2 fetches from and "
                 "writes to memory (the MALL included).  Algorithmic bytes per call: grouped GEMM "
                 "146.8 MB, delta 384.7 MB (all four kernels).\n\n"
                 "| kernel | dispatches | fetch MB | write MB | total MB |\n|---|---:|---:|---:|---:|\n")
        for n in names:
            pick = lambda k, n=n: "mi::" in k and short(k) == n
            f, nd = _pmc_avg(fr, "FETCH_SIZE", pick)
            w, _ = _pmc_avg(wr, "WRITE_SIZE", pick)
            fb, wb = f * 1024.0 * f_fac / 1e6, w * 1024.0 * w_fac / 1e6
            fh.write(f"| {n} | {nd} | {fb:.1f} | {wb:.1f} | {fb + wb:.1f} |\n")
    print(f"wrote {out}")


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.pmc_table:
        pmc_table(*args.pmc_table)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU; --gpus must be 1 (the path is "
                                   "data-parallel per GPU, see the sharding notes)"}))
        sys.exit(2)
    import torch

    import synth
    import moe_expert_grouped_amd as mi

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    only = set(filter(None, args.only.split(",")))

    # ---------------- inputs (resident in HBM before timing) ----------------
    g2 = synth.grouped_uniform(device=dev)
    out2 = torch.empty((g2.a.shape[0], g2.b.shape[1]), dtype=torch.bfloat16, device=dev)
    dc = synth.delta_at_scale(device=dev)
    wa, wb = mi.fill_w_ptr(dc.A), mi.fill_w_ptr(dc.B)
    sa = dc.E * dc.rank * dc.I
    sb = dc.E * dc.H * dc.rank
    dout = torch.empty((dc.T, dc.H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(mi.delta_workspace_bytes(dc.T, dc.top_k, dc.E, dc.L, dc.rank),
                     dtype=torch.uint8, device=dev)
    nc = synth.nvfp4_lora_case(device=dev)
    nout_raw = torch.empty((nc.M, nc.N), dtype=torch.bfloat16, device=dev)
    nout_prep = torch.empty_like(nout_raw)
    adapter = mi.prepare_nvfp4_lora_adapter(nc.lora_b, nc.lora_scale, nc.alpha)

    # ---------------- algorithmic work per op ----------------
    mi2 = g2.m_indptr.cpu().numpy()
    cum_m, k2, n2, E2 = g2.a.shape[0], g2.a.shape[1], g2.b.shape[1], g2.b.shape[0]
    gemm_flops = 2.0 * n2 * k2 * cum_m
    gemm_bytes = 2.0 * cum_m * k2 + 2.0 * n2 * k2 * int((np.diff(mi2) > 0).sum()) + \
        2.0 * cum_m * n2 + 4 * (E2 + 1)
    perm = dc.perm.cpu().numpy().reshape(dc.T, dc.top_k)
    lids = dc.lora_ids.cpu().numpy()
    eids = dc.topk_ids.cpu().numpy()
    act_mask = (perm >= 0) & (lids[:, None] >= 0)
    n_active = int(act_mask.sum())
    n_keys = len({(int(l), int(e)) for l, e in zip(np.broadcast_to(lids[:, None], eids.shape)[act_mask],
                                                   eids[act_mask])})
    delta_bytes = 2.0 * dc.I * n_active + 2.0 * (dc.rank * dc.I + dc.H * dc.rank) * n_keys + \
        2.0 * dc.T * dc.H + 12.0 * dc.T * dc.top_k + 4.0 * dc.T + 16.0 * dc.E
    delta_flops = n_active * (2.0 * dc.rank * dc.I + 2.0 * dc.H * dc.rank)
    M, N, K, r = nc.M, nc.N, nc.K, nc.rank
    nv_flops = 2.0 * M * N * K + 2.0 * M * N * r
    nv_bytes = M * K / 2 + N * K / 2 + (M + N) * K / 16 + 2.0 * M * N + 2.0 * (M + N) * r + 2.0 * N
    fold_bytes = 2.0 * 2 * N * r + 8
    fold_flops = float(N * r)

    stream = torch.cuda.current_stream(dev)
    ops = {
        "grouped_gemm": lambda: mi.grouped_mm_bf16(g2.a, g2.b, g2.m_indptr, out=out2),
        "lora_delta": lambda: mi.bgmv_moe_gemm2_lora_delta(
            dc.act, dc.perm, wa, sa, wb, sb, dc.topk_ids, dc.topk_weights, dc.lora_ids, dc.rank,
            dc.H, num_adapters=dc.L, scale=dc.scale, out=dout, workspace=ws),
        "fold": lambda: mi.prepare_nvfp4_lora_adapter(nc.lora_b, nc.lora_scale, nc.alpha,
                                                      out=adapter),
        "nvfp4_raw": lambda: mi.mm_nvfp4_lora(nc.a, nc.b, nc.a_sf, nc.b_sf, nc.alpha, nc.d,
                                              nc.lora_b, nc.lora_scale, bias=nc.bias,
                                              out=nout_raw),
        "nvfp4_prepared": lambda: mi.mm_nvfp4_lora(nc.a, nc.b, nc.a_sf, nc.b_sf, nc.alpha, nc.d,
                                                   lora_adapter=adapter, bias=nc.bias,
                                                   out=nout_prep),
    }
    if "copy_probe" in only:
        cp_src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
        cp_dst = torch.empty_like(cp_src)
        ops["copy_probe"] = lambda: torch.neg(cp_src, out=cp_dst)
    if only:
        ops = {k: v for k, v in ops.items() if k in only}
    work = {"grouped_gemm": (gemm_flops, gemm_bytes), "lora_delta": (delta_flops, delta_bytes),
            "fold": (fold_flops, fold_bytes), "nvfp4_raw": (nv_flops, nv_bytes),
            "nvfp4_prepared": (nv_flops, nv_bytes), "copy_probe": (0.0, 2.0 * COPY_PROBE_BYTES)}

    def step(ev=None):
        for i, (name, fn) in enumerate(ops.items()):
            if ev is not None:
                ev[name][0].record(stream)
            fn()
            if ev is not None:
                ev[name][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"# warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    evs = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for n in ops} for _ in range(args.steps)]
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
    per_op_ms = {n: float(np.mean([e[n][0].elapsed_time(e[n][1]) for e in evs])) for n in ops}
    print(f"# timed {args.steps} steps: {ms_step:.3f} ms/step (host wall {wall:.3f} s)",
          file=sys.stderr, flush=True)

    op_report = {}
    for n, ms in per_op_ms.items():
        fl, by = work[n]
        sec = ms * 1e-3
        rep = {"ms": round(ms, 5), "tflops": round(fl / sec / 1e12, 2), "gbps": round(by / sec / 1e9, 1),
               "algorithmic_flops": fl, "algorithmic_bytes": by}
        rep["frac_mfma_peak"] = round(fl / sec / 1e12 / PEAK_MFMA_TFLOPS, 4)
        rep["frac_hbm_peak"] = round(by / sec / 1e9 / PEAK_HBM_GBPS, 4)
        op_report[n] = rep
    step_flops = sum(work[n][0] for n in ops)

    roofline = None
    if "nvfp4_raw" in ops and "nvfp4_prepared" in ops:
        avg_ms = (per_op_ms["nvfp4_raw"] + per_op_ms["nvfp4_prepared"]) / 2
        ach = nv_flops / (avg_ms * 1e-3) / 1e12
        roofline = {"kernel": "nvfp4_lora_kernel", "bound": "mfma", "achieved": round(ach, 1),
                    "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(ach / PEAK_MFMA_TFLOPS, 4), "traffic": read_traffic()}

    # The same step captured once in a HIP graph and replayed: the calls do no
    # host read, allocation or memset, so the capture holds the step's kernels
    # and the launch gaps of the eager step drop out.  Informational only;
    # `value` is the eager step.
    step_graph = None
    if not only:
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
                      "tflops": round(step_flops / (gms * 1e-3) / 1e12, 2),
                      "note": "the step captured once in a HIP graph, replayed back to back"}
        del graph
        print(f"# graph replay: {gms:.3f} ms/step", file=sys.stderr, flush=True)

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

    def hbm_entry(ms, nbytes, note, flops=None):
        e = {"ms": round(ms, 5), "gbps": round(nbytes / ms / 1e6, 1),
             "frac_hbm_peak": round(nbytes / ms / 1e6 / PEAK_HBM_GBPS, 4),
             "algorithmic_bytes": nbytes, "note": note}
        if flops is not None:
            e["algorithmic_flops"] = flops
        return e

    # Outside the step, each timed on its own: the MoE finalize with the delta
    # added (FC2 rows of the delta workload's routing, bf16 [padded_rows, H]),
    # and the routing -> permutation -> permuted FC1 input rows of the same
    # routing (T=8192, top_k=8, E=64; bf16 token rows of H=4096).
    extra = {}
    if not only or "finalize" in only:
        fc2 = synth.bf16_normal((dc.act.shape[0], dc.H), 1.0, synth.gen(77, dev), dev)
        fout = torch.empty((dc.T, dc.H), dtype=torch.bfloat16, device=dev)
        fws = torch.empty(mi.finalize_workspace_bytes(dc.T, dc.top_k, dc.E, dc.L, dc.rank, dc.H),
                          dtype=torch.uint8, device=dev)
        fms = time_alone(lambda: mi.moe_finalize_lora(
            fc2, dc.act, dc.perm, wa, sa, wb, sb, dc.topk_ids, dc.topk_weights, dc.lora_ids,
            dc.rank, dc.H, num_adapters=dc.L, scale=dc.scale, out=fout, workspace=fws))
        n_routed = int((perm >= 0).sum())
        extra["finalize_fused"] = hbm_entry(
            fms, delta_bytes + 2.0 * dc.H * n_routed,
            "MoE finalize (weighted combine of the routed FC2 rows) with the LoRA delta added, "
            "delta workload, two passes (fp32 delta in the workspace, then the combine); not "
            "part of the step", delta_flops + 2.0 * dc.H * n_routed)
    if not only or "permute" in only:
        nslot = dc.T * dc.top_k
        rws = torch.empty(mi.route_workspace_bytes(nslot, dc.E), dtype=torch.uint8, device=dev)
        rms = time_alone(lambda: mi.moe_route_permutation(dc.topk_ids, dc.E, with_inverse=True,
                                                          workspace=rws))
        extra["route_permutation"] = hbm_entry(
            rms, 12.0 * nslot + 4.0 * (dc.E + 1),
            "topk_ids [8192, 8] -> m_indptr, expanded_idx_to_permuted_idx and its inverse "
            "(E=64); three launches, latency-bound at this size")
        _, rperm = mi.moe_route_permutation(dc.topk_ids, dc.E)
        xtok = synth.bf16_normal((dc.T, dc.H), 1.0, synth.gen(78, dev), dev)
        xperm = torch.empty((nslot, dc.H), dtype=torch.bfloat16, device=dev)
        pms = time_alone(lambda: mi.moe_permute_rows(xtok, rperm, dc.top_k, out=xperm))
        extra["permute_rows"] = hbm_entry(
            pms, 2.0 * dc.H * (dc.T + nslot) + 4.0 * nslot,
            "token rows bf16 [8192, 4096] -> permuted rows [65536, 4096] (each token row read "
            "once, written top_k times)")
    if not only or "nvfp4_grouped" in only:
        # NVFP4 grouped GEMM on the skewed MoE FC2 routing (E=128, cum_m=32768,
        # Zipf 1.1 counts, 8 empty experts) with FP4 weights n=7168, k=2048
        ng = synth.nvfp4_grouped_case(device=dev)
        ngo = torch.empty((ng.a.shape[0], ng.b.shape[1]), dtype=torch.bfloat16, device=dev)
        gms = time_alone(lambda: mi.grouped_mm_nvfp4(ng.a, ng.a_sf, ng.b, ng.b_sf, ng.m_indptr,
                                                     ng.alpha, out=ngo))
        cnts = np.diff(ng.m_indptr.cpu().numpy())
        nn, kk = ng.b.shape[1], ng.k
        gflops = 2.0 * ng.a.shape[0] * nn * kk
        per_e = ng.b_sf.numel() // ng.b.shape[0]
        gbytes = ng.a.numel() + ng.a_sf.numel() + (nn * kk / 2 + per_e) * int((cnts > 0).sum()) + \
            2.0 * ng.a.shape[0] * nn + 4.0 * (len(cnts) + 1) + 4.0 * len(cnts)
        sec = gms * 1e-3
        extra["nvfp4_grouped"] = {
            "ms": round(gms, 5), "tflops": round(gflops / sec / 1e12, 2),
            "frac_mfma_peak": round(gflops / sec / 1e12 / PEAK_MFMA_TFLOPS, 4),
            "gbps": round(gbytes / sec / 1e9, 1), "algorithmic_flops": gflops,
            "algorithmic_bytes": gbytes,
            "note": "NVFP4 grouped GEMM, E=128 Zipf(1.1) routing of 4096 tokens x top-8 "
                    "(cum_m=32768), n=7168, k=2048, per-expert alpha, bf16 out; the fp16 MFMA "
                    "peak (2516.6 TFLOP/s) is the denominator"}
    if not only or "fc1_swiglu" in only:
        # FC1: gate/up grouped GEMM + SwiGLU on the same skewed routing
        # (E=128, cum_m=32768), hidden=7168, inter=2048 (b is [128, 4096, 7168])
        fc = synth.fc1_case(device=dev)
        fco = torch.empty((fc.a.shape[0], fc.b.shape[1] // 2), dtype=torch.bfloat16, device=dev)
        fms = time_alone(lambda: mi.grouped_mm_swiglu(fc.a, fc.b, fc.m_indptr, out=fco))
        cnts = np.diff(fc.m_indptr.cpu().numpy())
        cm, hid, two_i = fc.a.shape[0], fc.a.shape[1], fc.b.shape[1]
        fflops = 2.0 * cm * two_i * hid
        fbytes = 2.0 * cm * hid + 2.0 * two_i * hid * int((cnts > 0).sum()) + \
            2.0 * cm * two_i / 2 + 4.0 * (len(cnts) + 1)
        sec = fms * 1e-3
        extra["fc1_swiglu"] = {
            "ms": round(fms, 5), "tflops": round(fflops / sec / 1e12, 2),
            "frac_mfma_peak": round(fflops / sec / 1e12 / PEAK_MFMA_TFLOPS, 4),
            "gbps": round(fbytes / sec / 1e9, 1), "algorithmic_flops": fflops,
            "algorithmic_bytes": fbytes,
            "note": "FC1 gate/up grouped GEMM with the SwiGLU epilogue, E=128 Zipf(1.1) routing "
                    "(cum_m=32768), hidden=7168, inter=2048, bf16; weights read once per expert "
                    "(7.3 GB)"}
        del fc, fco
    extra = extra or None

    cpu = None
    if not args.no_cpu_baseline and not only:
        cpu = cpu_baseline(g2, dc, nc, wa, wb, sa, sb)

    line = {
        "metric": METRIC,
        "value": round(step_flops / (max(ms_step, 1e-9) * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "step_graph": step_graph,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "moe-fc2-lora hot-path step: grouped GEMM (E=8, 128 rows/expert, k=4096, "
                        "n=2048, bf16 out) + FC2 LoRA delta (T=8192, top_k=8, E=64, I=2048, "
                        "H=4096, 8 adapters r=16) + fold + NVFP4+LoRA raw and prepared "
                        "(M=4096, N=8192, K=8192, r=16)",
            "value_definition": "sum of the step's algorithmic flops / step time",
            "grouped_gemm_tflops": op_report.get("grouped_gemm", {}).get("tflops"),
            "grouped_gemm_frac_bf16_mfma_peak": op_report.get("grouped_gemm", {}).get(
                "frac_mfma_peak"),
            "lora_delta_gbps": op_report.get("lora_delta", {}).get("gbps"),
            "lora_delta_frac_hbm_peak": op_report.get("lora_delta", {}).get("frac_hbm_peak"),
            "parallelism": "single GPU",
        },
        "ops": op_report,
        "extra_ops": extra,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(g2, dc, nc, wa, wb, sa, sb):
    """The fp64 oracle, as it stands, on a bounded sample of the same step."""
    import torch

    from oracle import nvfp4 as NV
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
    # inputs as the oracle takes them (host copies, outside the timing)
    a, b, mi_ = bits(g2.a), bits(g2.b), g2.m_indptr.cpu().numpy()
    toks = list(range(dc.T))
    act = bits(dc.act)
    ba, bb = Bank(bits(dc.A.reshape(-1)), dc.A.data_ptr()), Bank(bits(dc.B.reshape(-1)),
                                                                 dc.B.data_ptr())
    perm = dc.perm.cpu().numpy()
    lids = dc.lora_ids.cpu().numpy()
    wa_h, wb_h = wa.cpu().numpy(), wb.cpu().numpy()
    ids_h, w_h = dc.topk_ids.cpu().numpy(), dc.topk_weights.cpu().numpy()
    pr = perm.reshape(dc.T, dc.top_k)
    n_act = int(((pr[toks] >= 0) & (lids[toks][:, None] >= 0)).sum())
    rows = np.arange(nc.M)
    a_c = nc.a.cpu().numpy()[rows]
    b_c, asf, bsf = nc.b.cpu().numpy(), nc.a_sf.cpu().numpy(), nc.b_sf.cpu().numpy()
    d_h, lb_h, bias_h = bits(nc.d)[rows], bits(nc.lora_b), bits(nc.bias)
    pass_flops = (2.0 * g2.a.shape[0] * g2.a.shape[1] * g2.b.shape[1] +
                  n_act * (2.0 * dc.rank * dc.I + 2.0 * dc.H * dc.rank) +
                  2.0 * len(rows) * nc.N * nc.K + 2.0 * len(rows) * nc.N * nc.rank)
    # whole passes over the three workloads until at least 10 s of oracle time
    # (at most 4 passes)
    flops, t_total, passes = 0.0, 0.0, 0
    while passes < 4 and (passes == 0 or t_total < 10.0):
        t = time.perf_counter()
        grouped_mm(a, b, mi_)
        moe_fc2_lora_delta(act, perm, ba, wa_h, sa, bb, wb_h, sb, ids_h, w_h, lids, dc.rank, dc.H,
                           dc.scale, tokens=toks)
        base = NV.base_product(a_c, b_c, asf, bsf, nc.K, rows, None)
        NV.mm_nvfp4_raw(base, float(nc.alpha[0]), d_h, lb_h, float(nc.lora_scale[0]), bias_h)
        t_total += time.perf_counter() - t
        flops += pass_flops
        passes += 1
    return {"value": round(flops / t_total / 1e12, 5), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "seconds": round(t_total, 2),
            "sample": f"{passes} pass(es) over the whole grouped GEMM, LoRA delta and NVFP4 raw "
                      "workloads; flops / oracle time"}


if __name__ == "__main__":
    main()
