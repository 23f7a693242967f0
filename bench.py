"""Decode-speed benchmark of the batch-1 decode step on one MI355X.

Workload (default): the 2B-class dense model (24 layers, d_model 2048, 16
query heads x 128, 8 KV heads, SwiGLU 5632, vocab 32000, untied LM head,
fp16 weights N(0, 0.02), gains 1), a 512-token random prompt fed by
teacher-forced decode steps (untimed), then greedy decode steps with the
token fed back on the device.  A "step" is one whole decode step (all
layers, LM head, argmax).  Timed: exactly --steps steps at positions
511 .. 511+steps-1 (the configuration's 256 steps at context 512..767),
after --warmup untimed steps over the same positions (rewound afterwards).

With the persistent executor the dominant kernel is the persistent decode
kernel itself: one launch runs all timed steps, so its algorithmic bytes
per launch are the sum over those steps of every streamed weight byte plus
the K/V bytes each step reads.  The prompt is fed with the graph executor,
so the only persistent launches are the warmup and the timed one (equal
size: the profiler's average duration for the kernel is the timed launch's).

Prints one JSON line (rank 0, N = 1).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
SEG = 128


def step_bytes(shape, L: int, kv: str = "fp16", batch: int = 1) -> float:
    """Algorithmic HBM bytes of one decode step attending to L positions:
    every streamed weight once (all layer matrices and gains, the final gain,
    the LM head, one embedding row per sequence) plus, for each of the batch
    sequences, the K and V rows read in their
    stored format: fp16 2 B per element, E5M2 1 B; INT8: 1 B per element of
    sealed 128-position segments plus their (scale, zero point) pair, 2 B per
    element of the open segment's fp16 staging rows."""
    D, H, Hk, hd, F, V, NL = (shape.d_model, shape.n_heads, shape.n_kv_heads, shape.head_dim, shape.d_ff,
                              shape.vocab, shape.n_layers)
    per_layer = ((H + 2 * Hk) * hd * D + D * H * hd + 2 * F * D + D * F + 2 * D) * 2
    weights = NL * per_layer + (batch * D + V * D + D) * 2
    if kv == "fp16":
        kvb = 2 * Hk * hd * 2 * L
    elif kv == "e5m2":
        kvb = 2 * Hk * hd * L
    else:
        sealed = (L - 1) // SEG * SEG      # the row being written is in the open segment
        kvb = 2 * Hk * (hd * (sealed + 2 * (L - sealed)) + (sealed // SEG) * 8)
    return weights + batch * NL * kvb


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "k_persist_2b_decode_fp16_traffic.json")


def measured_traffic(args, bytes_run):
    """HBM bytes (read + write) of the timed persistent launch: the
    calibrated counter runs recorded under profiles/ for this workload
    (512-token prompt, fp16 KV, batch 1) give counter bytes per algorithmic
    byte over a 256-step launch at positions 511..766; the timed launch's
    algorithmic bytes times that ratio.  None if the run is another workload
    or the kernel's sources changed since the counters were taken."""
    import json as _json
    from request_decode_amd.traffic import source_hash
    if not (args.prompt == 512 and args.kv == "fp16" and args.batch == 1) or not os.path.exists(TRAFFIC_RECORD):
        return None
    rec = _json.load(open(TRAFFIC_RECORD))
    if rec.get("source_sha256") != source_hash():
        return None
    return int(round(bytes_run * rec["traffic_bytes"] / rec["algorithmic_bytes"]))


def cpu_model_name() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(blob, shape, seconds: float, base: int, first: int):
    """Oracle tokens/s on the machine's host cores at the timed positions: the
    oracle's fp16 cache holds seeded synthetic rows at positions 0..base-1
    (the step's cost does not depend on their values), then greedy decode
    steps from position `base` until `seconds` of CPU work have run (at
    least 3, at most 64)."""
    cores = len(os.sched_getaffinity(0))
    os.environ["OMP_NUM_THREADS"] = str(cores)
    import numpy as np
    import oracle
    import synth
    om = oracle.OracleModel(blob, base + 72, kv_format="fp16")
    fill = synth.normal_f16(7, (base, shape.head_dim)).view(np.uint16)
    for l in range(shape.n_layers):
        for w in (0, 1):
            for g in range(shape.n_kv_heads):
                om.set_rows(l, w, g, 0, fill)
    om.set_pos(base)
    t = first
    n, t0 = 0, time.perf_counter()
    while True:
        _, nxt = om.step([t])
        t = int(nxt[0])
        n += 1
        el = time.perf_counter() - t0
        if (el >= seconds and n >= 3) or n >= 64:
            break
    om.close()
    return {"value": n / el, "unit": "tokens/s", "cores": cores, "cpu": cpu_model_name(), "kind": "oracle",
            "sample": f"2B model, fp16 cache filled with synthetic rows at positions 0..{base - 1}, then {n} "
                      f"greedy decode steps at positions {base}..{base + n - 1} (the timed positions' start)"}


def layer_trace(m, token: int, reps: int, rewind: bool = True):
    """Where a layer of one persistent step spends its time, from the kernel's
    in-kernel event trace of every workgroup (rd_debug_trace_step_all; the
    wall clock is shared by all CUs).  Per workgroup and layer (the middle
    layers 2..21 of the step), the control wave's events give its own work
    per phase (input received -> output published) and its waits (own
    output published -> next input received).  The six exchanges of a layer
    are the waits of the workgroups that consume them: QKV <- down, the
    attention split <- QKV (attention workgroups), the merge <- attention
    (merge workgroups), O <- merge (merge workgroups), gate/up <- O and
    down <- gate/up.  Reported: medians over workgroups and layers, in us,
    of the last of `reps` traced steps (the first is not used).  A cache
    that cannot be rewound (INT8) is traced on consecutive positions."""
    import numpy as np
    for _ in range(max(2, reps)):
        tr = m.trace_step_all(token)
        if rewind:
            m.set_position(m.position() - 1)
    per = []
    for codes, clk in tr:
        d, occ = {}, {}
        for c, t in zip(codes.tolist(), clk.tolist()):
            k = occ.get(c, 0)
            occ[c] = k + 1
            d[(c, k)] = t * 0.01        # 100 MHz clock -> us
        per.append(d)
    seg = {k: [] for k in ("layer", "qkv", "att", "merge", "o", "gu", "down", "x_qkv", "x_att", "x_merge", "x_o",
                           "x_gu", "x_down", "att.start", "att.loop", "att.tail")}
    # inside each GEMV phase (stream wave 0's events 100 + 10 * kind + point:
    # phase entered, first rows reduced, all rows reduced; kinds 0 QKV, 1 O,
    # 2 gate/up, 3 down).  The stream waves enter a phase before its input is
    # there and reduce their first rows as its chunks are posted, so: the
    # control wave's staging (QKV only), first rows reduced counted from the
    # control wave's input received (negative: before the whole input was
    # in), the rest of the rows, the control wave's epilogue
    ctrl = {"qkv": 0, "o": 30, "gu": 40, "down": 50}
    kind = {"qkv": 0, "o": 1, "gu": 2, "down": 3}
    for ph in ctrl:
        for part in ("stage", "first", "rows", "epilogue", "barrier", "publish"):
            seg[f"{ph}.{part}"] = []
    for d in per:
        for l in range(2, 22):
            g = lambda c, ll=l: d.get((c, ll))
            if None in (g(0), g(3), g(30), g(33), g(40), g(43), g(50), g(53)) or (0, l + 1) not in d:
                continue
            seg["layer"].append(d[(0, l + 1)] - g(0))
            seg["qkv"].append(g(3) - g(0))
            seg["o"].append(g(33) - g(30))
            seg["gu"].append(g(43) - g(40))
            seg["down"].append(g(53) - g(50))
            seg["x_gu"].append(g(40) - g(33))
            seg["x_down"].append(g(50) - g(43))
            seg["x_qkv"].append(d[(0, l + 1)] - g(53))
            for ph, c in ctrl.items():
                k = 100 + 10 * kind[ph]
                staged = g(c + 1) if g(c + 1) is not None else g(c)   # only QKV records its staging
                ev = (g(c), staged, g(k + 1), g(k + 2), g(c + 3), g(c + 2))
                if None not in ev:
                    seg[f"{ph}.stage"].append(ev[1] - ev[0])
                    seg[f"{ph}.first"].append(ev[2] - ev[0])
                    seg[f"{ph}.rows"].append(ev[3] - ev[2])
                    seg[f"{ph}.epilogue"].append(ev[4] - ev[3])
                    # the epilogue in two: until the row sums' barrier has
                    # passed (the other stream waves' rows), then the
                    # control wave's own work
                    seg[f"{ph}.barrier"].append(ev[5] - ev[3])
                    seg[f"{ph}.publish"].append(ev[4] - ev[5])
            if g(10) is not None and g(13) is not None:
                seg["x_att"].append(g(10) - g(3))
                seg["att"].append(g(13) - g(10))
                # stream wave 0: attention start (q staged), its batches reduced
                if g(140) is not None and g(141) is not None:
                    seg["att.start"].append(g(140) - g(10))
                    seg["att.loop"].append(g(141) - g(140))
                    seg["att.tail"].append(g(13) - g(141))
            if g(20) is not None and g(23) is not None:
                seg["x_merge"].append(g(20) - (g(13) if g(13) is not None else g(3)))
                seg["merge"].append(g(23) - g(20))
                seg["x_o"].append(g(30) - g(23))
    # The step's tail: the final RMSNorm's input wait (after layer NL-1's down
    # publish), the LM head phase (input received -> row sums complete), the
    # argmax exchange (-> next token in hand)
    nl = max((k[1] for d in per for k in d if k[0] == 53), default=-1)
    lm = {"lm.wait": [], "lm.rows": [], "lm.argmax": []}
    for d in per:
        if None not in (d.get((53, nl)), d.get((60, 0)), d.get((62, 0)), d.get((63, 0))):
            lm["lm.wait"].append(d[(60, 0)] - d[(53, nl)])
            lm["lm.rows"].append(d[(62, 0)] - d[(60, 0)])
            lm["lm.argmax"].append(d[(63, 0)] - d[(62, 0)])
    seg.update({k: v for k, v in lm.items() if v})
    # Each exchange seen across workgroups (the clock is shared): how far the
    # last producer's publish trails the median producer's ("skew"), and how
    # long after the last publish the median consumer has its input ("after
    # last"); per layer, then the median over layers.  (producer event,
    # consumer event, consumer in the next layer)
    xch = {"qkv>att": (3, 10, 0), "att>merge": (13, 20, 0), "merge>o": (23, 30, 0), "o>gu": (33, 40, 0),
           "gu>down": (43, 50, 0), "down>qkv": (53, 0, 1)}
    for name, (pe, ce, nxt) in xch.items():
        sk, al = [], []
        for l in range(2, 21):
            prod = [d[(pe, l)] for d in per if (pe, l) in d]
            cons = [d[(ce, l + nxt)] for d in per if (ce, l + nxt) in d]
            if prod and cons:
                last = max(prod)
                sk.append(last - float(np.median(prod)))
                al.append(float(np.median(cons)) - last)
        if sk:
            seg[f"skew.{name}"] = sk
            seg[f"after_last.{name}"] = al
    med = {k: round(float(np.median(v)), 3) for k, v in seg.items() if v}
    for k in ("qkv", "att", "merge", "o", "gu", "down"):   # spread of the phases' own time
        if seg[k]:
            med[f"p90.{k}"] = round(float(np.percentile(seg[k], 90)), 3)
            med[f"max.{k}"] = round(float(np.max(seg[k])), 3)
    med["exchanges"] = round(sum(med.get(k, 0.0) for k in ("x_qkv", "x_att", "x_merge", "x_o", "x_gu", "x_down")), 3)
    med["workgroups"] = len(per)
    return med


GEMV_SHAPES = [(16384, 4096), (6144, 2048), (4096, 2048), (11264, 2048), (2048, 5632)]
COLD_BYTES = 768 << 20   # > 2x the 256 MB last-level (MALL) cache


def gemv_microbench(rd, torch, stream, iters: int = 3):
    """The weight-streaming GEMV alone: y = W x (fp16 in, fp32 out) at batch
    1 and 8 on the listed shapes, and at batch 1 with the weights in INT4
    (groups of 128 columns, fp32 scales: 0.53 bytes per weight).  Cold cache: launches rotate over distinct
    copies of W totalling >= 768 MiB, so every launch streams W from HBM.
    Kernel time: the launches are captured into one graph and replayed
    back to back between one pair of events, so no per-launch host or event
    overhead is counted; reported: mean time per launch and algorithmic
    GB/s (W + x + y bytes)."""
    import synth
    out = []
    for N, K in GEMV_SHAPES:
        W, X = synth.gemv_inputs(N, K, 8, seed_w=2, seed_x=3)
        wbytes = N * K * 2
        ncopy = max(2, -(-COLD_BYTES // wbytes))
        Wd = torch.from_numpy(W).to("cuda")
        copies = [Wd] + [Wd.clone() for _ in range(ncopy - 1)]
        Xd = torch.from_numpy(X).to("cuda")
        y = torch.empty((8, N), dtype=torch.float32, device="cuda")
        row = {"N": N, "K": K, "weight_bytes": wbytes, "copies": ncopy}
        for batch in (1, 8):
            for c in copies:    # warm the code path, touch every copy once
                rd.rd_gemv_f16(c.data_ptr(), Xd.data_ptr(), y.data_ptr(), N, K, batch, stream.cuda_stream)
            torch.cuda.synchronize()
            n = ncopy * iters
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(n):
                    rd.rd_gemv_f16(copies[i % ncopy].data_ptr(), Xd.data_ptr(), y.data_ptr(), N, K, batch,
                                   stream.cuda_stream)
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / n
            del g
            nbytes = wbytes + batch * K * 2 + batch * N * 4
            gbps = nbytes / (us * 1e-6) / 1e9
            row[f"b{batch}"] = {"us": round(us, 3), "gbps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)}
            print(f"[bench] gemv [{N},{K}] batch {batch}: {us:.2f} us, {gbps:.0f} GB/s", file=sys.stderr, flush=True)
        # weight-only INT4 (groups of 128 columns, fp32 scales) at batch 1
        qbytes = N * K // 2 + N * (K // 128) * 4
        nq = max(2, -(-COLD_BYTES // qbytes))
        qc = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
        qs = torch.empty((N, K // 128), dtype=torch.float32, device="cuda")
        rd.rd_q4_quantize(Wd.data_ptr(), N, K, qc.data_ptr(), qs.data_ptr(), stream.cuda_stream)
        del copies
        qcopies = [(qc, qs)] + [(qc.clone(), qs.clone()) for _ in range(nq - 1)]
        for c, sc in qcopies:
            rd.rd_gemv_q4(c.data_ptr(), sc.data_ptr(), Xd.data_ptr(), y.data_ptr(), N, K, stream.cuda_stream)
        torch.cuda.synchronize()
        n = nq * iters
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                c, sc = qcopies[i % nq]
                rd.rd_gemv_q4(c.data_ptr(), sc.data_ptr(), Xd.data_ptr(), y.data_ptr(), N, K, stream.cuda_stream)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / n
        del g
        nbytes = qbytes + K * 2 + N * 4
        gbps = nbytes / (us * 1e-6) / 1e9
        row["q4_b1"] = {"us": round(us, 3), "gbps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4),
                        "bytes": nbytes, "copies": nq}
        print(f"[bench] gemv int4 [{N},{K}] batch 1: {us:.2f} us, {gbps:.0f} GB/s", file=sys.stderr, flush=True)
        del qcopies, qc, qs, Wd
        torch.cuda.empty_cache()
        out.append(row)
    return out


DELTA_SEGS = 24 * 2 * 8 * 64   # K and V segments of the 2B cache at 8192 keys: layers x 2 x kv heads x 64


def delta_kv_bench(rd, torch, stream, iters: int = 5):
    """Delta quantization of K/V segments (rd_delta_seal, rd_delta_restore)
    over the K and V segments of the whole 2B cache at 8192 keys: 24576
    segments of 128 rows x 128 fp16 values, seeded random walks along the
    rows drawn on the device.  Each kernel timed over `iters` launches
    between HIP events on the bench stream; algorithmic bytes: seal reads
    the rows and writes anchor, codes and (scale, zp); restore reads those
    and writes the rows in fp32."""
    n_seg, n, hd = DELTA_SEGS, 128, 128
    g = torch.Generator(device="cuda").manual_seed(17)
    with torch.cuda.stream(stream):
        x = torch.randn((n_seg, 1, hd), generator=g, device="cuda")
        x = (x + torch.cumsum(0.05 * torch.randn((n_seg, n, hd), generator=g, device="cuda"), dim=1)).half()
        anchor = torch.empty((n_seg, hd), dtype=torch.int16, device="cuda")
        codes = torch.empty((n_seg, n - 1, hd), dtype=torch.uint8, device="cuda")
        meta = torch.empty((n_seg, 2), dtype=torch.float32, device="cuda")
        out = torch.empty((n_seg, n, hd), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    s = stream.cuda_stream
    seal = lambda: rd.rd_delta_seal(x.data_ptr(), n_seg, n, hd, anchor.data_ptr(), codes.data_ptr(), meta.data_ptr(), s)
    restore = lambda: rd.rd_delta_restore(anchor.data_ptr(), codes.data_ptr(), meta.data_ptr(), n_seg, n, hd,
                                          out.data_ptr(), s)
    sealed = hd * 2 + (n - 1) * hd + 8
    res = {"segments": n_seg, "rows": n, "head_dim": hd}
    for name, f, nbytes in (("seal", seal, n_seg * (n * hd * 2 + sealed)), ("restore", restore, n_seg * (sealed + n * hd * 4))):
        f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / iters
        gbps = nbytes / (us * 1e-6) / 1e9
        res[name] = {"us": round(us, 1), "bytes": nbytes, "gbps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)}
        print(f"[bench] delta {name}: {n_seg} segments, {us:.1f} us, {gbps:.0f} GB/s", file=sys.stderr, flush=True)
    del x, anchor, codes, meta, out
    torch.cuda.empty_cache()
    return res


def delta_oracle_time(seconds: float = 2.0):
    """The oracle's delta seal of one 128 x 128 segment, timed on one host
    core over about `seconds` (random walks as in delta_kv_bench)."""
    import time
    import numpy as np
    import oracle
    rng = np.random.default_rng(17)
    segs = (np.cumsum(rng.normal(0, 0.05, (16, 128, 128)), axis=1) + rng.normal(0, 1, (16, 1, 128)))
    segs = segs.astype(np.float16).view(np.uint16)
    oracle.delta_seal(segs[0])
    t0, k = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        oracle.delta_seal(segs[k % 16])
        k += 1
    return {"us_per_segment": round((time.perf_counter() - t0) / k * 1e6, 1), "segments": k, "cores": 1}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=None, help="default: --steps (one equal-size warmup launch)")
    ap.add_argument("--kv", default="fp16", choices=["fp16", "e5m2", "int8"])
    ap.add_argument("--batch", type=int, default=1, help="sequences in lockstep (1..8; > 1: graph executor)")
    ap.add_argument("--kv-pages", type=int, default=0,
                    help="batch > 1: a paged KV cache of this many page groups (-1: just enough for the run)")
    ap.add_argument("--prompt", type=int, default=512,
                    help="prompt length (512: the 2B decode workload; 32768: long context; 8192: quantized KV)")
    ap.add_argument("--executor", default="auto", choices=["auto", "graph", "eager", "persistent"])
    ap.add_argument("--attn-splits", type=int, default=0, help="key splits per kv head (0: the library's default)")
    ap.add_argument("--phase-iters", type=int, default=96)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemv", action="store_true", help="skip the standalone GEMV and delta-quantization microbenchmarks")
    ap.add_argument("--prefill", default="batched", choices=["batched", "steps"],
                    help="how the prompt is fed: the batched prefill (matrix products per layer), or one "
                         "teacher-forced decode step per token")
    ap.add_argument("--trace", type=int, default=0,
                    help="persistent executor: trace this many steps in the middle of the timed range and "
                         "report where a layer's time goes (exchange waits and per-phase work)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the decode path runs on one GPU only (asked for {args.gpus}); "
              "multi-GPU sharding is designed but not built", file=sys.stderr)
        sys.exit(2)
    if args.warmup is None:
        args.warmup = args.steps
    PROMPT = args.prompt
    if args.steps < 1 or args.warmup < 0 or PROMPT < 1 or PROMPT + max(args.steps, args.warmup) > 65536:
        sys.exit("bench.py: --prompt/--steps/--warmup must keep the context within 65536")

    import torch

    import request_decode_amd as rd
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    shape = synth.SHAPES["2b"]
    t0 = time.time()
    blob = synth.make_blob(shape, seed=2)
    print(f"[bench] blob {blob.size / 1e9:.3f} GB generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    # prompt seeds: 103 for the 512-token workload, 104 long context, 105 the 8K quantized-KV comparison
    pseed = 104 if PROMPT >= 16384 else 105 if PROMPT == 8192 else 103
    B = args.batch
    prompt = synth.prompt(pseed, PROMPT, shape.vocab) if B == 1 else synth.prompts(pseed, PROMPT, shape.vocab, B)
    # INT8 KV can only be rewound to a segment start: there the timed steps
    # follow the warmup steps instead of repeating their positions
    rewind = args.kv != "int8" and not args.kv_pages
    # +1: the phase run; an INT8 cache is traced on further positions
    ctx = PROMPT + (max(args.steps, args.warmup) if rewind else args.steps + args.warmup + max(2, args.trace)) + 1
    kv_pages = args.kv_pages
    if kv_pages < 0:   # every sequence's rows of the run, 4 KiB pages of one (layer, K/V, kv head)
        page_rows = 4096 // (shape.head_dim * (2 if args.kv == "fp16" else 1))
        kv_pages = B * -(-ctx // page_rows)
    m = rd.Model(blob, max_context=ctx, kv_format=args.kv, executor=args.executor, stream=stream.cuda_stream,
                 batch=B, attn_splits=args.attn_splits, kv_pages=kv_pages)
    executor = m.get_info().executor
    persistent = executor == rd.RD_EXEC_PERSISTENT
    batched = args.prefill == "batched" and B == 1
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if batched:
        m.prefill_batched(prompt[:-1])
    else:
        m.prefill(prompt[:-1] if B == 1 else prompt[:, :-1].T)   # teacher-forced decode steps (graph path)
    pf_s = time.perf_counter() - t0
    n_pf = PROMPT - 1
    print(f"[bench] prompt of {PROMPT} fed in {pf_s:.2f}s ({'batched prefill' if batched else 'decode steps'}, "
          f"{n_pf / pf_s:.0f} tokens/s)", file=sys.stderr, flush=True)
    first = int(prompt[-1]) if B == 1 else prompt[:, -1].copy()
    base = PROMPT - 1
    out = torch.empty(max(args.steps, args.warmup, 1) * B, dtype=torch.int32, device="cuda")
    if args.warmup:
        warm = m.generate(first, args.warmup)
        if rewind:
            m.set_position(base)
        else:
            first, base = (int(warm[-1]) if B == 1 else warm[-1].copy()), base + args.warmup
    print(f"[bench] warmup {args.warmup} done", file=sys.stderr, flush=True)

    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    ev0.record(stream)
    m.generate_async(first, args.steps, out.data_ptr())
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    m.synchronize()
    ms = ev0.elapsed_time(ev1)
    ms_per_step = ms / args.steps
    tok_s = args.steps * B / (ms / 1e3)
    Ls = [base + 1 + i for i in range(args.steps)]
    bytes_run = sum(step_bytes(shape, L, args.kv, B) for L in Ls)
    bytes_step = bytes_run / args.steps
    gbps = bytes_run / (ms / 1e3) / 1e9
    print(f"[bench] timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step, {tok_s:.1f} tok/s, "
          f"{gbps:.0f} GB/s (host wall clock {wall * 1e6 / args.steps:.1f} us/step)", file=sys.stderr, flush=True)

    trace = None
    if args.trace and persistent and B == 1:
        if rewind:
            m.set_position(base + args.steps // 2)
            tok = int(out[args.steps // 2 - 1].item()) if args.steps >= 2 else first
        else:
            tok = int(out[args.steps - 1].item())
        trace = layer_trace(m, tok, args.trace, rewind)
        print(f"[bench] layer trace (us, medians over workgroups and layers 2..21): {trace}", file=sys.stderr,
              flush=True)

    # the gate/up GEMV phase kernel of the (batch-1) graph executor, timed
    # alone, rotating over the 24 layers so that its weights come from HBM
    k_us = k_gbps = None
    k_bytes = (2 * shape.d_ff * shape.d_model + shape.d_model) * 2
    if B == 1:
        if rewind:
            m.set_position(base + args.steps // 2)
        m.run_phase(3, 0, 24)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        m.run_phase(3, 0, args.phase_iters)
        e1.record(stream)
        torch.cuda.synchronize()
        m.synchronize()
        k_us = e0.elapsed_time(e1) * 1e3 / args.phase_iters
        k_gbps = k_bytes / (k_us * 1e-6) / 1e9
        print(f"[bench] gate/up phase kernel: {k_us:.2f} us/launch, {k_gbps:.0f} GB/s", file=sys.stderr, flush=True)
    m.close()
    del out
    gemv = None if args.no_gemv else gemv_microbench(rd, torch, stream)
    delta = None if args.no_gemv else delta_kv_bench(rd, torch, stream)

    if persistent:
        roof = {"bound": "hbm", "kernel": "k_persist (whole decode steps, one launch for all timed steps)",
                "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(args, bytes_run),
                "bytes_per_launch": int(bytes_run), "us_per_launch": round(ms * 1e3, 1)}
    elif B > 1:
        roof = {"bound": "hbm", "kernel": "batch step: graph of per-phase kernels (thin GEMMs k_gemm_b8 on MFMA)",
                "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                "bytes_per_launch": int(bytes_step), "us_per_launch": round(ms_per_step * 1e3, 1)}
    else:
        roof = {"bound": "hbm", "kernel": "k_gateup (RMSNorm + gate/up GEMV + SwiGLU)",
                "achieved": round(k_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(k_gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                "bytes_per_launch": k_bytes, "us_per_launch": round(k_us, 3)}
    workload = ("2b-dense-decode" if PROMPT == 512 and args.kv == "fp16" and B == 1 else
                "2b-long-context-decode" if PROMPT >= 16384 else f"2b-{args.kv}-kv-decode")
    if B > 1:
        workload += f"-batch{B}" + ("-paged" if kv_pages else "")
    res = {
        "metric": ("batch-1 decode tokens/s + achieved HBM GB/s (MBU %) on 2B-class fp16 model" if B == 1 else
                   f"batch-{B} decode tokens/s (all sequences) + achieved HBM GB/s on 2B-class fp16 model"),
        "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp16",
        "data": "synthetic: seeded N(0,0.02) fp16 weights, uniform random prompt ids",
        "config": {"workload": workload, "layers": 24, "d_model": 2048, "heads": 16, "kv_heads": 8,
                   "head_dim": 128, "d_ff": 5632, "vocab": 32000, "prompt": PROMPT, "batch": B, "kv_pages": kv_pages,
                   "kv_cache": args.kv, "executor": ["auto", "eager", "graph", "persistent"][executor],
                   "positions": [base, base + args.steps - 1]},
        "hbm_gbps": round(gbps, 1), "mbu": round(gbps / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": int(bytes_step),
        "roofline": roof,
    }
    if k_us is not None:
        res["gateup_phase_kernel"] = {"us_per_launch": round(k_us, 3), "gbps": round(k_gbps, 1)}
    # prefill: matrix-product FLOPs (2 per weight and token; attention: QK^T
    # and PV over positions 0..p of every prompt position)
    D, H, Hk, hd, F, NL = (shape.d_model, shape.n_heads, shape.n_kv_heads, shape.head_dim, shape.d_ff,
                           shape.n_layers)
    w_tok = NL * ((H + 2 * Hk) * hd * D + D * H * hd + 2 * F * D + D * F)
    attn = NL * H * hd * 4 * (n_pf * (n_pf + 1) // 2)
    res["prefill"] = {"mode": "batched" if batched else "decode steps", "tokens": n_pf, "seconds": round(pf_s, 4),
                      "tokens_per_s": round(n_pf / pf_s, 1),
                      "tflops": round((2 * w_tok * n_pf + attn) / pf_s / 1e12, 2)}
    if trace is not None:
        res["layer_trace_us"] = trace
    if gemv is not None:
        res["gemv_microbench"] = gemv
        big = [r for r in gemv if (r["N"], r["K"]) == (16384, 4096)]
        if big:
            res["gemv_16384x4096_b1_frac"] = big[0]["b1"]["frac"]
    if delta is not None:
        res["delta_kv"] = delta
    # device resources released before the interpreter's own teardown
    torch.cuda.synchronize()
    rd.release_scratch()
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(blob, shape, args.cpu_seconds, base,
                                           first if B == 1 else int(first[0]))
        if delta is not None:   # the oracle's delta seal beside the kernel's
            res["delta_kv"]["oracle_seal"] = delta_oracle_time()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
