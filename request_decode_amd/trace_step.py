"""Where one persistent decode step spends its time.

Runs the 2B-class model (seeded synthetic weights) to position 511 with the
graph executor, then traces persistent decode steps with the in-kernel
event trace of workgroup 0 (rd_debug_trace_step) and prints, per segment
between consecutive events, the time per step and per occurrence; then the
latency of an all-to-all exchange of 2048 words (rd_debug_barrier_probe).

    python -m request_decode_amd.trace_step [--reps 5] [--kv fp16]
"""
from __future__ import annotations

import argparse
import collections
import os
import sys

import numpy as np

PHASES = ["qkv", "att", "merge", "o", "gu", "down", "lm"]
POINTS = ["recv", "staged", "done", "pub"]


SPHASES = ["qkv", "o", "gu", "down", "lm"]
SPOINTS = ["go", "first", "end"]


def event_name(c: int) -> str:
    if c == 99:
        return "start"
    if c == 98:
        return "end"
    if c >= 200:   # stream wave 0, first rows of a phase: before the ring wait, after it,
        c -= 200   # after reading the slots, after issuing the refills
        return f"c.{SPHASES[c // 10]}.{['pre', 'landed', 'read', 'issued'][c % 10]}"
    if c >= 100:   # stream wave 0: released, first rows landed, rows reduced
        c -= 100
        return f"s.{SPHASES[c // 10]}.{SPOINTS[c % 10]}"
    return f"{PHASES[c // 10]}.{POINTS[c % 10]}"


def wg_report(tr):
    """Per exchange of the last traced step: when the last producer published,
    and when consumers received (first / median / last), in us from the
    step start of workgroup 0."""
    per = []
    for codes, clk in tr:
        occ = collections.Counter()
        d = {}
        for c, t in zip(codes, clk):
            k = (int(c), occ[int(c)])
            occ[int(c)] += 1
            d[k] = t
        per.append(d)
    t0 = min(d[(99, 0)] for d in per if (99, 0) in d)
    keys = sorted({k for d in per for k in d}, key=lambda k: np.median([d[k] for d in per if k in d]))
    print(f"{'event':>14s} {'occ':>4s} {'n_wg':>5s} {'first':>8s} {'median':>8s} {'last':>8s}  (us)")
    for k in keys:
        v = np.array([d[k] for d in per if k in d], np.float64)
        v = (v - t0) * 0.01
        if k[1] < 2 or k[1] > 21:   # first two and last layers of the step
            print(f"{event_name(k[0]):>14s} {k[1]:4d} {len(v):5d} {v.min():8.2f} {np.median(v):8.2f} {v.max():8.2f}")
    # mean over layers 2..21 of (median - first) and (last - first) per event
    agg = collections.defaultdict(list)
    for k in keys:
        if 2 <= k[1] <= 21:
            v = np.array([d[k] for d in per if k in d], np.float64) * 0.01
            agg[k[0]].append((np.median(v), v.min(), v.max()))
    print("mean over layers 2..21, relative to the layer's first qkv.recv:")
    base = {}
    for k in keys:
        if k[0] == 0 and 2 <= k[1] <= 21:
            base[k[1]] = min(d[k] for d in per if k in d) * 0.01
    rows = []
    for code in sorted(agg):
        rel = []
        for occ in range(2, 22):
            k = (code, occ)
            vs = np.array([d[k] for d in per if k in d], np.float64) * 0.01
            if len(vs) and occ in base:
                rel.append((vs.min() - base[occ], np.median(vs) - base[occ], vs.max() - base[occ]))
        if rel:
            r = np.mean(np.array(rel), axis=0)
            rows.append((r[1], event_name(code), r))
    for _, name, r in sorted(rows):
        print(f"{name:>14s}  first {r[0]:7.2f}  median {r[1]:7.2f}  last {r[2]:7.2f}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--kv", default="fp16", choices=["fp16", "e5m2", "int8"])
    ap.add_argument("--prompt", type=int, default=512)
    ap.add_argument("--all", action="store_true", help="also trace every workgroup: exchange latency and skew")
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
    if args.all:
        for rep in range(2):
            tr = m.trace_step_all(tok)
        wg_report(tr)
    names = {0: "epoch flags, then the data read", 1: "tagged data words (the decode kernel's exchange)"}
    for mode, name in names.items():
        print(f"exchange of 2048 words, mode {mode} ({name}): {rd.rd_debug_barrier_probe(0, 20000, mode):.3f} us")
    m.close()


if __name__ == "__main__":
    main()
