"""Where one persistent decode step spends its time.

Runs the 2B-class model (seeded synthetic weights) to position 511 with the
graph executor, then traces persistent decode steps with the in-kernel
event trace of workgroup 0 (rd_debug_trace_step) and prints, per segment
between consecutive events, the time per step and per occurrence; then the
latency of each grid-barrier scheme (rd_debug_barrier_probe).

    python -m request_decode_amd.trace_step [--reps 5] [--kv fp16]
"""
from __future__ import annotations

import argparse
import collections
import os
import sys

import numpy as np

PHASES = ["qkv", "att", "o", "gu", "down", "lm"]
POINTS = ["wait", "staged", "done", "arrived", "issued"]


def event_name(c: int) -> str:
    if c == 99:
        return "start"
    if c == 98:
        return "end"
    return f"{PHASES[c // 10]}.{POINTS[c % 10]}"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--kv", default="fp16", choices=["fp16", "e5m2", "int8"])
    ap.add_argument("--prompt", type=int, default=512)
    args = ap.parse_args()
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import request_decode_amd as rd
    import synth

    shape = synth.SHAPES["2b"]
    blob = synth.make_blob(shape, seed=2)
    m = rd.Model(blob, max_context=args.prompt + args.reps + 8, kv_format=args.kv, executor="persistent")
    m.set_executor("graph")
    prompt = synth.prompt(103, args.prompt, shape.vocab)
    for t in prompt[:-1]:
        m.decode_step(int(t), want_logits=False)
    m.set_executor("persistent")
    tok = int(prompt[-1])
    seg = collections.defaultdict(list)
    totals = []
    for rep in range(args.reps):
        codes, clk = m.trace_step(tok)
        totals.append((clk[-1] - clk[0]) * 0.01)
        if rep == 0:
            continue                      # first traced step: cold
        for i in range(len(codes) - 1):
            seg[(event_name(codes[i]), event_name(codes[i + 1]))].append((clk[i + 1] - clk[i]) * 0.01)
    n = args.reps - 1
    print(f"step time (workgroup 0, start to end): " + ", ".join(f"{t:.1f}" for t in totals) + " us")
    print(f"{'segment':>30s} {'us/step':>9s} {'us/each':>8s} {'per step':>8s}")
    rows = sorted(((sum(v) / n, k, float(np.mean(v)), len(v) // n) for k, v in seg.items()), reverse=True)
    for tot, k, mean, cnt in rows:
        print(f"{k[0]:>13s} -> {k[1]:<14s} {tot:9.1f} {mean:8.2f} {cnt:8d}")
    names = {0: "counter tree + generation word", 1: "one counter", 2: "monotonic counter tree",
             3: "packed flags, all threads poll", 4: "one flag per line"}
    for mode, name in names.items():
        print(f"barrier mode {mode} ({name}): {rd.rd_debug_barrier_probe(0, 20000, mode):.3f} us")
    m.close()


if __name__ == "__main__":
    main()
