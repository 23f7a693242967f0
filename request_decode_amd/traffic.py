"""HBM traffic of the persistent decode kernel from rocprofv3 counter runs.

Reads the counter CSVs of three `rocprofv3 --pmc` runs of
`python3 -m request_decode_amd.profile_run` (FETCH_SIZE; WRITE_SIZE;
TCC_EA0_RDREQ_32B/64B/128B/TCC_EA0_RDREQ), scales FETCH_SIZE and WRITE_SIZE by
what they read for the run's plain copy kernel (out = in + 0 over a known
number of bytes), and writes a JSON record for bench.py plus a markdown
summary.  The record carries a hash of the kernel's sources: bench.py
reports the traffic only while the sources are unchanged.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["csrc/rd_persistent.hip", "csrc/rd_phases.h", "csrc/rd_device.h", "csrc/rd_internal.h"]


def _code_only(text: str) -> str:
    """The source with its comments and layout removed, so that the hash
    follows the code the counters were taken from, not its commentary."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(HERE, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def _counters(path: str) -> dict:
    out: dict = {}
    for r in csv.DictReader(open(path)):
        name = r["Kernel_Name"]
        k = "kernel" if "k_persist" in name else "copy" if "add" in name.lower() else None
        if k:
            out.setdefault(k, {})[r["Counter_Name"]] = float(r["Counter_Value"])
            out.setdefault(k + "_name", name)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--raw", required=True)
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    ap.add_argument("--algorithmic-bytes", type=int, required=True, help="as printed by profile_run")
    ap.add_argument("--workload", default="2b-dense-decode prompt 512, 256 steps, fp16 KV")
    ap.add_argument("--out", required=True, help="JSON record; a .md summary is written beside it")
    ap.add_argument("--command", default="")
    args = ap.parse_args()
    f, w, r = _counters(args.fetch), _counters(args.write), _counters(args.raw)
    fscale = args.copy_bytes / (f["copy"]["FETCH_SIZE"] * 1024)
    wscale = args.copy_bytes / (w["copy"]["WRITE_SIZE"] * 1024)
    fetch = f["kernel"]["FETCH_SIZE"] * 1024 * fscale
    write = w["kernel"]["WRITE_SIZE"] * 1024 * wscale
    rk = r["kernel"]
    raw = 32 * rk["TCC_EA0_RDREQ_32B"] + 64 * rk["TCC_EA0_RDREQ_64B"] + 128 * rk["TCC_EA0_RDREQ_128B"]
    rec = {"kernel": f["kernel_name"], "workload": args.workload, "source_sha256": source_hash(),
           "fetch_bytes": int(fetch), "write_bytes": int(write), "traffic_bytes": int(fetch + write),
           "fetch_scale": fscale, "write_scale": wscale, "raw_read_bytes": int(raw),
           "algorithmic_bytes": args.algorithmic_bytes, "command": args.command}
    with open(args.out, "w") as fh:
        json.dump(rec, fh, indent=1)
    md = os.path.splitext(args.out)[0] + ".md"
    with open(md, "w") as fh:
        fh.write(f"# HBM traffic: `{rec['kernel'].split('(')[0]}`, {args.workload}\n\n")
        fh.write("Commands (repo root, one MI355X), one counter set per run:\n\n```\n")
        fh.write(args.command + "\n```\n\n")
        fh.write("| quantity | per launch |\n|---|---:|\n")
        fh.write(f"| FETCH_SIZE of the kernel | {f['kernel']['FETCH_SIZE']:.0f} KiB |\n")
        fh.write(f"| FETCH_SIZE of the copy ({args.copy_bytes} B read) | {f['copy']['FETCH_SIZE']:.1f} KiB "
                 f"-> scale {fscale:.5f} |\n")
        fh.write(f"| WRITE_SIZE of the kernel | {w['kernel']['WRITE_SIZE']:.0f} KiB |\n")
        fh.write(f"| WRITE_SIZE of the copy ({args.copy_bytes} B written) | {w['copy']['WRITE_SIZE']:.1f} KiB "
                 f"-> scale {wscale:.5f} |\n")
        fh.write(f"| read bytes, scaled FETCH_SIZE | {fetch:.4e} |\n")
        fh.write(f"| read bytes, 32/64/128-byte request counts | {raw:.4e} "
                 f"({rk['TCC_EA0_RDREQ_128B']:.0f} x 128 B, {rk['TCC_EA0_RDREQ_64B']:.0f} x 64 B, "
                 f"{rk['TCC_EA0_RDREQ_32B']:.0f} x 32 B) |\n")
        fh.write(f"| written bytes, scaled WRITE_SIZE | {write:.4e} |\n")
        fh.write(f"| algorithmic bytes | {args.algorithmic_bytes:.4e} |\n")
        fh.write(f"| read / algorithmic | {fetch / args.algorithmic_bytes:.4f} |\n")
        fh.write(f"| (read + write) / algorithmic | {(fetch + write) / args.algorithmic_bytes:.4f} |\n\n")
        fh.write("The copy reads with 128-byte requests and FETCH_SIZE reports half its bytes: on this "
                 "architecture the counter's formula takes 128-byte read requests for 64-byte ones. The raw "
                 "request counts agree with the scaled figure. Kernel sources hash: "
                 f"`{rec['source_sha256'][:16]}`.\n")
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()
