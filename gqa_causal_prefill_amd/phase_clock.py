"""Shader cycles per phase of the tile loop, and the shader clock under load, from the
library's phase-clock measurement build.

The measurement build is the library's source compiled with -DGQA_PHASE_CLOCK (build it
first, on any machine with hipcc):

    python -c 'from gqa_causal_prefill_amd import build; build.build_variant("phase", ["-DGQA_PHASE_CLOCK=1"])'

(-DGQA_PHASE_CLOCK=2, built as "phase2" and run with --library, also pins each counter read in
the instruction order, which makes the phase split exact for an order that is then no longer
the library's.)

Its kernels read the shader cycle counter (s_memtime) and the 100 MHz real-time counter
(s_memrealtime) around the tile loop of every wave: loop cycles over tiles is the cost of a
tile, and loop cycles over loop time the shader clock the loop ran at. They also add up the
cycles between reads placed at the phase boundaries of each tile (Q·K^T with the softmax of
the previous tile, P·V, the copy wait and barrier) and of the INT8-value maximum sweep. The
compiler moves instructions across those reads (they order nothing), so the phase split is
approximate: the report gives the share of the loop's cycles that falls inside the timed
phases. The arithmetic is the library's; only the counter reads are added.

    python -m gqa_causal_prefill_amd.phase_clock [--workloads 3 5 12] [--markdown PATH]

For each workload it warms the GPU up for about 0.3 s of launches, runs one more launch
timed with HIP events and reads the counters of that launch. Needs one GPU.
"""

from __future__ import annotations

import argparse
import ctypes
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SLOTS = 10
REALTIME_HZ = 100e6
NAMES = {3: "4096 x 32768, bf16 keys", 5: "3072 x 16384, INT8 keys (2 KV segments for the 32 longest token blocks)",
         12: "3072 x 16384, INT8 keys and values", 4: "paged 512 x 32768 tail, bf16 keys (4 KV segments)",
         2: "4096 x 8192, bf16 keys", 6: "4096 x 16384, bf16 keys", 11: "3072 x 16384, bf16 keys"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workloads", type=int, nargs="+", default=[3, 5, 12])
    ap.add_argument("--library", default=os.path.join(ROOT, "gqa_causal_prefill_amd", "variants",
                                                      "libgqa_prefill_phase.so"))
    ap.add_argument("--markdown", default=None, help="also write the table to this file")
    ap.add_argument("--verbose", action="store_true", help="also print per-wave details")
    ap.add_argument("--append", action="store_true", help="append the table to --markdown as a new section")
    ap.add_argument("--q-len", type=int, nargs="+", default=None,
                    help="run each workload's kind (contiguous only) at these q_len instead")
    ap.add_argument("--kv-len", type=int, default=None, help="with --q-len: the kv_len (default the workload's)")
    ap.add_argument("--unsplit", action="store_true",
                    help="call gqa_attn_prefill (never cut into KV segments) instead of gqa_attn_prefill_ws")
    args = ap.parse_args()
    sys.path.insert(0, ROOT)
    import numpy as np
    import torch

    from gqa_causal_prefill_amd import binding
    if not os.path.exists(args.library):
        raise SystemExit(f"{args.library} is missing: build the measurement build first (see the module docstring)")
    binding.LIB = args.library   # before the library is first loaded
    import gqa_causal_prefill_amd as gqa
    from gqa_synth import WORKLOADS, make_workload

    lib = gqa.library()
    lib.gqa_phase_clock_read.restype = ctypes.c_int
    lib.gqa_phase_clock_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    rows = []
    import dataclasses
    runs = []
    for wl in args.workloads:
        w = WORKLOADS[wl]
        if args.q_len:
            if w.paged:
                raise SystemExit("--q-len takes contiguous workloads")
            for ql in args.q_len:
                kv = args.kv_len or w.kv_len
                runs.append((wl, dataclasses.replace(w, name=f"{w.name.split('_')[0]}_{ql}x{kv}", q_len=ql, kv_len=kv)))
        else:
            runs.append((wl, w))
    for wl, w in runs:
        if w.paged and w.int8k:
            raise SystemExit("paged INT8 workloads are not covered by this runner")
        print(f"phase_clock: workload {wl} {w.name}", file=sys.stderr, flush=True)
        d = make_workload(w)
        q = d["q"].to(dev)
        out = torch.empty_like(q)
        if w.int8v:
            k, ks = gqa.gqa_quantize_rows_int8(d["k"].to(dev))
            vq, vs = gqa.gqa_quantize_v_int8(d["v"].to(dev))

            def step():
                gqa.gqa_attn_prefill_int8kv(q, k, ks, vq, vs, out=out, stream=stream)
        else:
            kw = {}
            if w.paged:
                k, v = d["k_cache"].to(dev), d["v_cache"].to(dev)
                kw = dict(block_table=d["block_table"].to(dev), kv_len=w.kv_len)
            elif w.int8k:
                k, ks = gqa.gqa_quantize_rows_int8(d["k"].to(dev))
                v = d["v"].to(dev)
                kw = dict(k_scale=ks)
            else:
                k, v = d["k"].to(dev), d["v"].to(dev)
            nbytes = gqa.gqa_attn_prefill_workspace_size(w.q_len, w.kv_len, w.paged, w.int8k)
            ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)

            def step():
                if args.unsplit:
                    gqa.gqa_attn_prefill(q, k, v, out=out, stream=stream, **kw)
                else:
                    gqa.gqa_attn_prefill_ws(q, k, v, out=out, workspace=ws, stream=stream, **kw)
        t = time.time()
        while time.time() - t < 0.3:
            for _ in range(4):
                step()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        plan = gqa.gqa_attn_prefill_plan(w.q_len, w.kv_len, w.paged, 2 if w.int8v else int(w.int8k))
        nwg = int(dict(x.split("=") for x in plan.split())["workgroups"])
        if args.unsplit and not w.int8v:   # one workgroup per (KV head, token block)
            nwg = 4 * ((w.q_len + 31) // 32) if w.q_len > 4 else 4 * ((w.q_len + 3) // 4)
        buf = np.zeros(nwg * 4 * SLOTS, dtype=np.uint64)
        st = lib.gqa_phase_clock_read(buf.ctypes.data_as(ctypes.c_void_p), buf.nbytes)
        if st != 0:
            raise SystemExit(f"gqa_phase_clock_read returned {st}")
        p = buf.reshape(nwg * 4, SLOTS).astype(np.float64)
        n = p[:, 3].sum()
        per = [p[:, i].sum() / n for i in range(3)]
        loop_tile = p[:, 8].sum() / (n + p[:, 5].sum())
        inside = (p[:, 0] + p[:, 1] + p[:, 2] + p[:, 4]).sum() / p[:, 8].sum()
        clock = p[:, 8].sum() / (p[:, 9].sum() / REALTIME_HZ) / 1e9
        sweep = p[:, 6].sum() / p[:, 7].sum() if p[:, 7].sum() > 0 else None
        rows.append(dict(wl=wl, name=w.name if args.q_len else NAMES.get(wl, w.name), wgs=nwg, ms=ms, qk=per[0], pv=per[1], sync=per[2], tile=sum(per),
                         loop_tile=loop_tile, inside=inside,
                         masked=p[:, 4].sum() / max(p[:, 5].sum(), 1), sweep=sweep, clock=clock,
                         span=p[:, 9].max() / REALTIME_HZ * 1e3, tiles=n / (nwg * 4)))
        r = rows[-1]
        if args.verbose:
            busy = p[:, 0] + p[:, 1] + p[:, 2] + p[:, 4]
            i = int(np.argmax(p[:, 9]))
            print(f"  loop cycles summed {p[:, 8].sum():.4g} vs tile-body cycles summed {busy.sum():.4g}; "
                  f"longest wave {i}: {p[i, 3]:.0f}+{p[i, 5]:.0f} tiles, {p[i, 8]:.4g} cycles, {p[i, 9]:.4g} ticks, "
                  f"sweep {p[i, 6]:.4g} cycles / {p[i, 7]:.0f} tiles; per-wave clock GHz min/median/max "
                  + " ".join(f"{x:.3f}" for x in np.percentile(p[:, 8] / (p[:, 9] / REALTIME_HZ) / 1e9, [0, 50, 100])),
                  flush=True)
        print(f"{w.name}: launch {ms:.4f} ms; loop {loop_tile:.0f} cycles per tile, {100 * inside:.0f}% of them in the "
              f"timed phases; per unmasked tile {r['tile']:.0f} cycles (Q·K^T + softmax "
              f"{r['qk']:.0f}, P·V {r['pv']:.0f}, wait + barrier {r['sync']:.0f}); masked tile {r['masked']:.0f}"
              + (f"; sweep {sweep:.0f} per tile" if sweep else "")
              + f"; loop clock {clock:.3f} GHz; longest wave loop {r['span']:.4f} ms", flush=True)
    if args.markdown:
        name = os.path.basename(args.library)[len("libgqa_prefill_"):-len(".so")]
        level = {"phase": 1, "phase2": 2}.get(name, 1)
        cmd = "python -m gqa_causal_prefill_amd.phase_clock --workloads " + " ".join(map(str, args.workloads))
        if args.q_len:
            cmd += " --q-len " + " ".join(map(str, args.q_len)) + (f" --kv-len {args.kv_len}" if args.kv_len else "")
        if args.unsplit:
            cmd += " --unsplit"

        if name != "phase":
            cmd += f" --library gqa_causal_prefill_amd/variants/libgqa_prefill_{name}.so"
        title = ("counter reads where the library's instruction order puts them" if level == 1 else
                 "every counter read pinned in the instruction order")
        note = []
        if args.q_len and args.unsplit:
            title += ", grids of fewer workgroups"
            note = [f"Each workload's kind at q_len {', '.join(map(str, args.q_len))} over the same keys, called without KV segments",
                    "(`gqa_attn_prefill`): 4 workgroups per 32 query tokens, at most one per CU, so grids of 256 and",
                    "more keep every CU busy and smaller ones leave CUs idle.", ""]
        md = ([] if args.append else ["# Shader cycles per loop phase and the shader clock under load", ""]) + [
              f"## -DGQA_PHASE_CLOCK={level}: {title}", ""] + note + [
              "Repository root, one MI355X; the measurement build of the library (its source with the phase clock",
              f"compiled in; the library's own machine code has none of it):", "", "```",
              f"python -c 'from gqa_causal_prefill_amd import build; build.build_variant(\"{name}\", [\"-DGQA_PHASE_CLOCK={level}\"])'",
              cmd, "```", "",
              "One launch after about 0.3 s of warm-up launches, every wave's counters summed. Cycles are shader clock",
              "cycles (`s_memtime`). Loop cycles per tile: the tile loop's cycles over its tiles (the INT8-value maximum",
              "sweep, a loop of its own before the main one, separately). The phase columns add up the cycles between",
              "counter reads at the phase boundaries of the unmasked tiles; the compiler moves instructions across such",
              "reads, so they hold only the share of the loop's cycles given in the next column. Shader clock: loop cycles",
              "over loop time from the 100 MHz `s_memrealtime` counter.", "",
              "| workload | workgroups | launch ms | loop cycles per tile | share in timed phases | Q·K^T + softmax | P·V | copy wait + barrier | max sweep per tile | shader clock GHz |",
              "|---|---|---|---|---|---|---|---|---|---|"]
        for r in rows:
            sweep = "" if r["sweep"] is None else f"{r['sweep']:.0f}"
            md.append(f"| {r['name']} | {r['wgs']} | {r['ms']:.4f} | {r['loop_tile']:.0f} | {100 * r['inside']:.0f}% | "
                      f"{r['qk']:.0f} | {r['pv']:.0f} | {r['sync']:.0f} | {sweep} | {r['clock']:.3f} |")
        with open(args.markdown, "a" if args.append else "w") as f:
            f.write(("\n" if args.append else "") + "\n".join(md) + "\n")


if __name__ == "__main__":
    main()
