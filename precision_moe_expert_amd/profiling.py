"""Measurement helpers for rocprofv3 runs of the MoE expert library.

  python -m precision_moe_expert_amd.profiling copy --mib 1024
      a plain device-to-device copy of a known size (the calibration kernel
      for the FETCH_SIZE / WRITE_SIZE counters)
  python -m precision_moe_expert_amd.profiling stats <kernel_stats.csv> <out.txt> <command...>
      per-kernel duration summary from `rocprofv3 --kernel-trace --stats`
  python -m precision_moe_expert_amd.profiling traffic <read_dir> <write_dir> <copy_read_dir>
      <copy_write_dir> <kernel substring> <out.txt> <kernel source> <copy bytes> <command...>
      HBM bytes per dispatch of one kernel, scaled by the copy calibration.
      Reads come from the request-size counters TCC_EA0_RDREQ_{32B,64B,128B}
      (bytes = 32 n32 + 64 n64 + 128 n128); writes from WRITE_SIZE.  On the
      MI355X machine the FETCH_SIZE derived counter reads a 1 GiB copy as 384 MiB
      (it under-weights 128-byte requests, which this library issues almost
      exclusively), while the request counters read it as exactly 1 GiB.

The traffic summary carries the SHA-256 of the kernel's source file; the
benchmark reports the figure only while that file is unchanged.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))


def source_sha(kernel_files: str) -> str:
    """SHA-256 over comma-separated csrc/ files (kernel, scheduler, host)."""
    h = hashlib.sha256()
    for name in kernel_files.split(","):
        with open(os.path.join(PKG, "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _find(d: str, pattern: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no {pattern} under {d}")
    return hits[0]


def copy_kernel(mib: int = 1024, reps: int = 3) -> None:
    import torch
    n = mib * 1024 * 1024
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"copied {mib} MiB x {reps}")


def kernel_stats(stats_csv: str, out_txt: str, command: str) -> None:
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# rocprofv3 kernel statistics", f"command: {command}", "",
             f"{'kernel':70s} {'calls':>6s} {'avg_us':>10s} {'total_ms':>10s} {'pct':>6s}"]
    for r in rows:
        name = r.get("Name") or r.get("KernelName") or r.get("Kernel_Name")
        calls = int(float(r.get("Calls", 0)))
        avg = float(r.get("AverageNs", 0)) / 1e3
        tot = float(r.get("TotalDurationNs", 0)) / 1e6
        pct = float(r.get("Percentage", 0))
        lines.append(f"{name[:70]:70s} {calls:6d} {avg:10.2f} {tot:10.3f} {pct:6.2f}")
    open(out_txt, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter_per_dispatch(d: str, counter: str, kernel_sub: str) -> tuple[float, int]:
    path = _find(d, "*counter_collection.csv")
    vals = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter or kernel_sub not in r["Kernel_Name"]:
            continue
        key = r["Dispatch_Id"]
        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    if not vals:
        raise ValueError(f"{counter} for {kernel_sub!r} not in {path}")
    return sum(vals.values()) / len(vals), len(vals)


def _read_bytes_per_dispatch(d: str, kernel_sub: str) -> tuple[float, int]:
    path = _find(d, "*counter_collection.csv")
    per = {}
    size = {"TCC_EA0_RDREQ_32B": 32.0, "TCC_EA0_RDREQ_64B": 64.0, "TCC_EA0_RDREQ_128B": 128.0}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] not in size or kernel_sub not in r["Kernel_Name"]:
            continue
        per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + size[r["Counter_Name"]] * float(r["Counter_Value"])
    if not per:
        raise ValueError(f"read-request counters for {kernel_sub!r} not in {path}")
    return sum(per.values()) / len(per), len(per)


def traffic(read_dir, write_dir, copy_read_dir, copy_write_dir, kernel_sub, out_txt, command, kernel_file,
            copy_bytes) -> None:
    rb, nd = _read_bytes_per_dispatch(read_dir, kernel_sub)
    wk, _ = _counter_per_dispatch(write_dir, "WRITE_SIZE", kernel_sub)
    crb, _ = _read_bytes_per_dispatch(copy_read_dir, "copyBuffer")
    cwk, _ = _counter_per_dispatch(copy_write_dir, "WRITE_SIZE", "copyBuffer")
    rscale = copy_bytes / crb
    wscale = copy_bytes / (cwk * 1024.0)
    hbm = rb * rscale + wk * 1024.0 * wscale
    lines = ["# HBM traffic of one kernel from rocprofv3 --pmc (read-request sizes, then WRITE_SIZE)",
             f"command: {command}",
             f"kernel = {kernel_sub}",
             f"kernel_source = {kernel_file}",
             f"kernel_source_sha = {source_sha(kernel_file)}",
             f"dispatches = {nd}",
             f"read_bytes_per_dispatch = {rb:.0f}",
             f"write_kib_per_dispatch = {wk:.1f}",
             f"copy_bytes = {copy_bytes:.0f}",
             f"copy_read_bytes = {crb:.0f}",
             f"copy_write_kib = {cwk:.1f}",
             f"read_scale = {rscale:.4f}",
             f"write_scale = {wscale:.4f}",
             f"hbm_bytes_per_dispatch = {hbm:.0f}"]
    open(out_txt, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def read_traffic(path: str) -> dict | None:
    """Parse a traffic summary; None if missing or the kernel source changed."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if " = " in line:
            k, v = line.strip().split(" = ", 1)
            kv[k] = v
    try:
        if kv.get("kernel_source_sha") != source_sha(kv["kernel_source"]):
            return None
        return dict(kernel=kv["kernel"], hbm_bytes_per_dispatch=float(kv["hbm_bytes_per_dispatch"]))
    except (KeyError, ValueError, FileNotFoundError):
        return None


if __name__ == "__main__":
    cmd = sys.argv[1]
    if cmd == "copy":
        mib = int(sys.argv[sys.argv.index("--mib") + 1]) if "--mib" in sys.argv else 1024
        copy_kernel(mib)
    elif cmd == "stats":
        kernel_stats(sys.argv[2], sys.argv[3], " ".join(sys.argv[4:]))
    elif cmd == "traffic":
        (fd, wd, cfd, cwd, ksub, out, kfile, cbytes), rest = sys.argv[2:10], sys.argv[10:]
        traffic(fd, wd, cfd, cwd, ksub, out, " ".join(rest), kfile, float(cbytes))
    else:
        raise SystemExit(__doc__)
