"""A short run for hardware-counter collection under rocprofv3.

Builds the 2B-class model (the bench's seeded weights), feeds a prompt with
the batched prefill (no graph launches), then makes one persistent launch of --steps greedy steps;
afterwards one plain copy kernel (out = in + 0, elementwise) of --copy-mib
MiB whose input was written before the run (its HBM traffic is known: that
many bytes read and written) to calibrate FETCH_SIZE / WRITE_SIZE.  Prints the algorithmic bytes of the persistent
launch.

    rocprofv3 --pmc FETCH_SIZE -d <dir> -o <name> -- python3 -m request_decode_amd.profile_run
"""
from __future__ import annotations

import argparse
import os
import sys


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--prompt", type=int, default=512)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--kv", default="fp16", choices=["fp16", "e5m2", "int8"])
    ap.add_argument("--copy-mib", type=int, default=1024)
    args = ap.parse_args()
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import torch

    import bench
    import request_decode_amd as rd
    import synth

    # the copy's source is written first, so that by the time it is copied
    # the decode run has pushed it out of every cache: the copy reads HBM
    n = args.copy_mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    shape = synth.SHAPES["2b"]
    blob = synth.make_blob(shape, seed=2)
    prompt = synth.prompt(103, args.prompt, shape.vocab)
    m = rd.Model(blob, max_context=args.prompt + args.steps, kv_format=args.kv, executor="persistent")
    m.prefill_batched(prompt[:-1])       # (counter collection and graph launches do not mix in the profiler)
    m.generate(int(prompt[-1]), args.steps)
    Ls = range(args.prompt, args.prompt + args.steps)
    nbytes = sum(bench.step_bytes(shape, L, args.kv) for L in Ls)
    print(f"persistent launch: {args.steps} steps at positions {args.prompt - 1}..{args.prompt + args.steps - 2}, "
          f"algorithmic bytes {int(nbytes)}", flush=True)
    m.close()
    torch.cuda.synchronize()
    torch.add(src, 0.0, out=dst)         # an elementwise kernel: n bytes read, n written
    torch.cuda.synchronize()
    print(f"copy: {n} bytes read and {n} bytes written", flush=True)
    # device memory handed back before the interpreter's teardown
    del src, dst
    rd.release_scratch()
    torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
