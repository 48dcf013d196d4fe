"""Benchmark of causal GQA prefill attention on one MI355X.

A step is one gqa_attn_prefill_ws call (the whole hot path: Q load/quantise, K/V
tile fetch, Q·K^T, scale and causal mask, softmax, P·V, epilogue, and the merge of
KV segments when the call splits the history) over
the q_len 4096 x kv_len 32768 chunk (24 query heads, 4 KV heads, head_dim 256,
bf16, contiguous KV) unless --workload says otherwise. Inputs are seeded
synthetic tensors already resident in HBM when the timed region starts.

Prints one JSON line: TFLOP/s counted causal-effectively (4 * 24 * 256 * the
number of visible query/key pairs per head, divided by the time), the roofline
of the kernel against the MI355X dense bf16 MFMA peak (with, from the committed
rocprofv3 counter record of the same kernel build, its HBM traffic per launch, that
traffic's rate over this run's step time against 8 TB/s, and the MFMA busy share),
and the CPU oracle timed on a bounded sample of the same workload as a baseline.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GQA causal prefill attn TFLOP/s + % MFMA peak, q4096×kv32K, 24Q/4KV d256"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 flop/clk (the published 2.5 PFLOP/s dense)
PEAK_INT8_TOPS = 5033.2
HQ, HKV, D = 24, 4, 256
# The MI355X raises its clock over roughly the first 100 ms of sustained load: a 4096 x
# 4096 launch took 0.222 ms in a burst of 30 and 0.177 ms after 600 back-to-back launches.
WARMUP_SECONDS = 0.3
KERNEL_SOURCE = os.path.join(ROOT, "gqa_causal_prefill_amd", "csrc", "gqa_prefill.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: at least 20, and enough for about "
                         f"{WARMUP_SECONDS} s of GPU work, so the clock has settled)")
    ap.add_argument("--workload", type=int, default=3,
                    help="1 tiny, 2 4096x8192, 3 4096x32768 (default), 4 paged 512x32768, "
                         "5 int8-k 3072x16384, 6 4096x16384, 7 paged int8-k 512x32768, "
                         "8 decode 1x32768, 9 paged decode 1x32768, "
                         "10 paged int8-k decode 1x32768, "
                         "11 3072x16384 with bf16 keys (workload 5's inputs), "
                         "12 3072x16384 with INT8 keys and values (workload 5's inputs)")
    ap.add_argument("--query-block", type=int, default=3, choices=(3, 2),
                    help="query columns per wave in 16-column blocks: 3 (the library: a "
                         "workgroup is 32 tokens x the 6 heads of a KV head) or 2 (the second "
                         "build: 64 tokens x 2 heads), for comparing the two shapes")
    ap.add_argument("--library", default=None,
                    help="load this build of the library instead (a variant from "
                         "gqa_causal_prefill_amd.build.build_variant, for comparing a tuning "
                         "constant; such lines carry no counter record)")
    ap.add_argument("--q-len", type=int, default=None,
                    help="run the workload's kind (contiguous only) at this q_len instead")
    ap.add_argument("--kv-len", type=int, default=None,
                    help="run the workload's kind (contiguous only) at this kv_len instead")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=3072,
                    help="query rows of the workload the CPU oracle computes (all 24 heads)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="before warm-up, run a plain device copy of MIB MiB (for scaling "
                         "HBM counters by a kernel whose traffic is known)")
    return ap.parse_args()


def source_digest() -> str:
    """sha256[:16] of the kernel source followed by the hipcc flags it is built with
    (a flag change changes the kernel as much as a source change)."""
    from gqa_causal_prefill_amd.build import HIPCC_FLAGS

    h = hashlib.sha256()
    with open(KERNEL_SOURCE, "rb") as f:
        h.update(f.read())
    h.update(" ".join(HIPCC_FLAGS).encode())
    return h.hexdigest()[:16]


def load_counters(workload_name: str):
    """The committed rocprofv3 counter record of the workload's attention kernel
    (profiles/traffic_<workload>.json), if it was taken on the current kernel source and
    build flags; else None. It holds the HBM bytes per launch (FETCH_SIZE + WRITE_SIZE,
    scaled by a device copy of known size) and the MFMA busy fraction
    (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE per XCD x 1024 SIMDs)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_build_sha256_16") != source_digest():
        return None
    return rec


def load_traffic(workload_name: str):
    """HBM bytes per launch from the counter record (None when it is stale or absent)."""
    rec = load_counters(workload_name)
    return None if rec is None else rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, d, rows_n):
    """Oracle time on the last `rows_n` query rows (x 24 heads) of the workload."""
    import numpy as np
    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    rows = np.arange(w.q_len - rows_n, w.q_len)
    off = w.kv_len - w.q_len
    pairs = int(np.sum(off + rows + 1))
    flops = 4.0 * HQ * D * pairs
    t = time.perf_counter()
    if w.int8v:
        kq, ks = oracle.quantize_rows_int8(d["k"])
        vq, vs = oracle.quantize_v_int8(d["v"])
        oracle.attention_int8kv(d["q"], kq, ks, vq, vs, rows=rows)
    elif w.int8k:
        kq, ks = oracle.quantize_rows_int8(d["k"])
        oracle.attention_int8k(d["q"], kq, ks, d["v"], rows=rows)
    else:
        oracle.attention(d["q"], d["k"], d["v"], rows=rows)
    dt = time.perf_counter() - t
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), cpu)
    except OSError:  # pragma: no cover
        pass
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "cpu": cpu, "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"query rows {rows[0]}..{rows[-1]} ({rows_n} rows) x 24 heads of {w.name}"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; "
                                   f"--gpus {args.gpus} is not supported"}))
        sys.exit(2)
    import torch

    import gqa_causal_prefill_amd as gqa
    from gqa_causal_prefill_amd import binding as gqa_binding, build as gqa_build
    from gqa_synth import WORKLOADS, make_workload

    if args.query_block == 2:
        gqa_binding.LIB = gqa_build.QB2_LIB   # before the library is first loaded
    if args.library is not None:
        gqa_binding.LIB = os.path.abspath(args.library)

    w = WORKLOADS[args.workload]
    if args.q_len is not None or args.kv_len is not None:
        if w.paged:
            print(json.dumps({"error": "--q-len / --kv-len take a contiguous workload"}))
            sys.exit(2)
        import dataclasses

        q_len = w.q_len if args.q_len is None else args.q_len
        kv_len = w.kv_len if args.kv_len is None else args.kv_len
        if not 0 < q_len <= kv_len:
            print(json.dumps({"error": "need 0 < q_len <= kv_len"}))
            sys.exit(2)
        kind = "int8kv" if w.int8v else ("int8k" if w.int8k else "bf16")
        w = dataclasses.replace(w, name=f"{kind}_{q_len}x{kv_len}", q_len=q_len, kv_len=kv_len)
    dev = torch.device("cuda:0")
    print(f"bench: {w.name} generating inputs", file=sys.stderr, flush=True)
    d = make_workload(w)
    q = d["q"].to(dev)
    v = (d["v_cache"] if w.paged else d["v"]).to(dev)
    kw = {}
    if w.paged and w.int8k:
        from gqa_synth import scatter_paged_int8_splitd, scatter_paged_scales
        kq, ks = gqa.gqa_quantize_rows_int8(d["k"].to(dev))
        torch.cuda.synchronize()
        k = scatter_paged_int8_splitd(kq.cpu(), d["block_table"], w.num_blocks).to(dev)
        kw = dict(block_table=d["block_table"].to(dev), kv_len=w.kv_len,
                  k_scale=scatter_paged_scales(ks.cpu(), d["block_table"], w.num_blocks).to(dev))
    elif w.paged:
        k = d["k_cache"].to(dev)
        kw = dict(block_table=d["block_table"].to(dev), kv_len=w.kv_len)
    elif w.int8k:
        k, ks = gqa.gqa_quantize_rows_int8(d["k"].to(dev))
        kw = dict(k_scale=ks)
        if w.int8v:   # the producer's V codes, feature-major [4, 256, ld]
            v, vs = gqa.gqa_quantize_v_int8(d["v"].to(dev))
            kw["v_scale"] = vs
    else:
        k = d["k"].to(dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)
    # KV-segment workspace (empty when the call runs unsplit), allocated before timing
    int8k_arg = 2 if w.int8v else int(w.int8k)
    ws_bytes = gqa.gqa_attn_prefill_workspace_size(w.q_len, w.kv_len, w.paged, int8k_arg)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def step():
        if w.int8v:
            gqa.gqa_attn_prefill_int8kv(q, k, kw["k_scale"], v, kw["v_scale"], out=out, stream=stream)
        else:
            gqa.gqa_attn_prefill_ws(q, k, v, out=out, workspace=ws, stream=stream, **kw)

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"bench: copied {n} bytes twice for counter calibration", file=sys.stderr, flush=True)
        del src, dst
    done = 0   # warm-up steps run so far
    if args.warmup is None:
        # the first 4 warm-up steps also time the step; then warm up for WARMUP_SECONDS
        # of work in all (at least 20 steps)
        probe = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        step()
        probe[0].record(stream)
        for _ in range(3):
            step()
        probe[1].record(stream)
        torch.cuda.synchronize()
        done = 4
        per_step = probe[0].elapsed_time(probe[1]) / 3 / 1e3
        args.warmup = max(20, int(WARMUP_SECONDS / max(per_step, 1e-6)))
    print(f"bench: {w.name} warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup - done):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    print(f"bench: {w.name} {args.steps} steps, {ms:.4f} ms/step", file=sys.stderr, flush=True)

    flops = 4.0 * HQ * D * w.pairs_per_head
    tflops = flops / (ms * 1e-3) / 1e12
    # algorithmic bytes: Q and out once, each K and V row once (int8 K: 1 byte a feature
    # plus its scale; int8 V: 1 byte a feature plus a scale per feature), the block table
    kv_rows = w.kv_len * HKV
    alg_bytes = (2 * w.q_len * HQ * D * 2 + kv_rows * D * (1 if w.int8k else 2)
                 + kv_rows * D * (1 if w.int8v else 2) + (kv_rows * 4 if w.int8k else 0)
                 + (HKV * D * 4 if w.int8v else 0)
                 + (4 * ((w.kv_len + 15) // 16) if w.paged else 0))
    # the committed counter records are of the default build (query block 3)
    counters = load_counters(w.name) if args.query_block == 3 and args.library is None else None
    traffic = None if counters is None else counters.get("hbm_bytes_per_launch")
    # HBM rate of the counted traffic over this run's step time, and the MFMA pipe's busy
    # share from the counter pass (both null without a current counter record)
    hbm_gbs = None if traffic is None else round(traffic / (ms * 1e-3) / 1e9, 1)
    mfma_busy = None if counters is None else counters.get("mfma_busy")
    if flops / alg_bytes < 315.0:
        # below the ridge (2516.6 TFLOP/s / 8 TB/s): a decode-sized chunk is HBM-bound
        gbs = alg_bytes / (ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                    "frac": round(gbs / 8000.0, 4), "traffic": traffic, "hbm_gbs": hbm_gbs,
                    "mfma_busy": mfma_busy}
    if w.int8v:
        peak = PEAK_INT8_TOPS   # Q·K^T and P·V both on int8 MFMA
    elif w.int8k:
        # Q·K^T on int8 MFMA, P·V on bf16 MFMA: time at peak is the sum of both halves
        t_peak = (flops / 2) / (PEAK_INT8_TOPS * 1e12) + (flops / 2) / (PEAK_BF16_TFLOPS * 1e12)
        peak = flops / t_peak / 1e12
    else:
        peak = PEAK_BF16_TFLOPS
    if flops / alg_bytes >= 315.0:
        roofline = {"bound": "mfma", "achieved": round(tflops, 3), "peak": round(peak, 1),
                    "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                    "traffic": traffic, "hbm_gbs": hbm_gbs, "mfma_busy": mfma_busy}
    rec = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8" if w.int8v else ("int8+bf16" if w.int8k else "bf16"),
        "data": "synthetic",
        "config": {"workload": w.name, "q_len": w.q_len, "kv_len": w.kv_len, "q_heads": HQ,
                   "kv_heads": HKV, "head_dim": D,
                   "kv_layout": ("paged16_splitd" if w.int8k else "paged16") if w.paged else "contiguous",
                   "keys": "int8" if w.int8k else "bf16",
                   "values": "int8" if w.int8v else "bf16",
                   "variant": gqa.gqa_attn_prefill_plan(w.q_len, w.kv_len, w.paged, int8k_arg)},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        print(f"bench: cpu oracle on {args.cpu_rows} rows", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(w, d, min(args.cpu_rows, w.q_len))
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
