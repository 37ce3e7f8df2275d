"""Summaries of rocprofv3 output for the kernels of the training step.

Two reports, both plain text:

* ``stats``: the per-kernel table of a ``rocprofv3 --kernel-trace --stats
  --output-format csv`` run (``*_kernel_stats.csv``): calls, total, average.
* ``traffic``: HBM bytes per launch of one kernel from two ``--pmc`` runs
  (``FETCH_SIZE``, then ``WRITE_SIZE``; each counter is KiB per dispatch).
  Both counters are scaled by what they read for a plain copy kernel of known
  size in the same run (``torch.neg`` over a buffer of ``copy_bytes`` bytes:
  that many bytes fetched and written), so the result is in algorithmic-byte
  units. The report carries a digest of the kernel's sources; ``bench.py``
  reports the figure only while that digest still matches.

* ``mfma``: per kernel, from one ``--pmc`` run with
  ``SQ_INSTS_VALU_MFMA_MOPS_BF16`` (bf16 MFMA operations / 512),
  ``SQ_VALU_MFMA_BUSY_CYCLES`` and ``SQ_BUSY_CYCLES``: the MFMA FLOPs each
  dispatch executed (recomputation included), its duration from the
  dispatch's own timestamps, the executed TFLOP/s, and the MFMA-busy share
  busy_cycles / (SIMDs x duration x clock) at the given engine clock.

Usage:
  python -m decoder_only_transformer_gpt_amd.profsum stats CSV --command CMD [--top N]
  python -m decoder_only_transformer_gpt_amd.profsum mfma DIR --command CMD --clock-mhz F [--simds 1024]
  python -m decoder_only_transformer_gpt_amd.profsum traffic --fetch DIR --write DIR --kernel SUBSTR
         --tag TAG --copy-bytes N --command-fetch CMD --command-write CMD
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")

# Source files whose text decides each kernel tag's code.
TAG_SOURCES = {
    "attn": ["attention.hip"], "gemm": ["gemm.hip"], "rmsnorm": ["norm.hip"], "rope": ["norm.hip"],
    "embed_rmsnorm": ["norm.hip"], "ce": ["ce.hip"], "embed_bwd": ["embed_bwd.hip"],
    "embed_sort": ["embed_bwd.hip"], "weight": ["norm.hip"], "fp8": ["fp8.hip"], "x0_mix": ["resid.hip"],
    "ve_add": ["resid.hip"], "ve_bwd": ["resid.hip", "embed_bwd.hip"], "opt_adamw": ["optim.hip"],
    "opt_muon": ["optim.hip", "gemm.hip"],
}
COMMON = ["common.h", "kernels.h"]


def sources_for_tag(tag: str) -> list[str]:
    for prefix in sorted(TAG_SOURCES, key=len, reverse=True):
        if tag.startswith(prefix):
            return TAG_SOURCES[prefix] + COMMON
    raise KeyError(tag)


def source_digest(tag: str) -> str:
    h = hashlib.sha256()
    for f in sources_for_tag(tag):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def short_name(n: str) -> str:
    """Readable kernel name: demangled text when rocprofv3 gave one, else the
    last identifier of an Itanium-mangled name plus its template arguments."""
    if n.startswith("_ZN"):
        i, ident = 3, ""
        while i < len(n) and n[i].isdigit():
            j = i
            while n[j].isdigit():
                j += 1
            ln = int(n[i:j])
            ident, i = n[j:j + ln], j + ln
        rest = n[i:]
        if rest.startswith("I"):
            body = rest[1:rest.find("EE") + 1] if "EE" in rest else rest[1:]
            body = re.sub(r"LNS_3EpiE(\d+)E", r"Epi\1,", body)
            body = re.sub(r"Lb([01])E", lambda m: ("true" if m.group(1) == "1" else "false") + ",", body)
            body = re.sub(r"Li(\d+)E", r"\1,", body)
            body = re.sub(r"^f", "float,", body.replace("DF16b", "bf16,"))
            ident += "<" + body.strip(",E") + ">"
        return ident[:100]
    n = n.replace("gk::(anonymous namespace)::", "").replace("__hip_bfloat16", "bf16")
    n = re.sub(r"\(gk::Epi\)(\d+)", r"Epi\1", n)
    n = re.sub(r"^void ", "", n)
    n = re.sub(r"\(.*", "", n)
    return n[:100]


def stats_report(csv_path: str, command: str, top: int = 30) -> str:
    rows = list(csv.DictReader(open(csv_path)))
    tot = sum(float(r["TotalDurationNs"]) for r in rows)
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = [f"command: {command}", f"source: {os.path.basename(csv_path)}", "",
           f"{'total ms':>10} {'calls':>6} {'avg ms':>9} {'min ms':>9} {'max ms':>9} {'%':>6}  kernel"]
    for r in rows[:top]:
        t = float(r["TotalDurationNs"]) / 1e6
        out.append(f"{t:10.3f} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e6:9.4f} "
                   f"{float(r['MinNs']) / 1e6:9.4f} {float(r['MaxNs']) / 1e6:9.4f} "
                   f"{100 * float(r['TotalDurationNs']) / tot:6.2f}  {short_name(r['Name'])}")
    out.append(f"all kernels: {tot / 1e6:.3f} ms over {sum(int(r['Calls']) for r in rows)} dispatches")
    return "\n".join(out) + "\n"


def _counter_avgs(d: str, counter: str) -> dict:
    agg: dict = {}
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            # one row per dispatch and counter (values already summed over instances)
            key = r["Kernel_Name"]
            agg.setdefault(key, {}).setdefault(r.get("Dispatch_Id", str(len(agg))), 0.0)
            agg[key][r.get("Dispatch_Id", str(len(agg)))] += float(r["Counter_Value"])
    return {k: (sum(v.values()) / len(v), len(v)) for k, v in agg.items()}


def _pick(avgs: dict, substr: str, what: str):
    hits = [(k, v) for k, v in avgs.items() if substr in k]
    if len(hits) != 1:
        raise ValueError(f"{what}: {len(hits)} kernels match {substr!r}: {[short_name(k) for k, _ in hits]}")
    return hits[0]


def traffic_report(fetch_dir: str, write_dir: str, kernel: str, tag: str, copy_bytes: int, cmd_fetch: str,
                   cmd_write: str, copy_kernel: str = "neg_kernel") -> str:
    fa, wa = _counter_avgs(fetch_dir, "FETCH_SIZE"), _counter_avgs(write_dir, "WRITE_SIZE")
    (kname, (kf, nf)), (_, (cf, _)) = _pick(fa, kernel, "fetch"), _pick(fa, copy_kernel, "fetch copy")
    (_, (kw, nw)), (_, (cw, _)) = _pick(wa, kernel, "write"), _pick(wa, copy_kernel, "write copy")
    f_scale = copy_bytes / (cf * 1024.0)
    w_scale = copy_bytes / (cw * 1024.0)
    fetch_b = kf * 1024.0 * f_scale
    write_b = kw * 1024.0 * w_scale
    out = [f"kernel: {short_name(kname)}", f"tag: {tag}",
           f"command (FETCH_SIZE): {cmd_fetch}", f"command (WRITE_SIZE): {cmd_write}",
           f"copy calibration: torch.neg over {copy_bytes} bytes; FETCH_SIZE read {cf:.1f} KiB "
           f"(scale {f_scale:.4f}), WRITE_SIZE read {cw:.1f} KiB (scale {w_scale:.4f})",
           f"dispatches averaged: {nf} (fetch), {nw} (write)",
           f"FETCH_SIZE per launch: {kf:.1f} KiB raw",
           f"WRITE_SIZE per launch: {kw:.1f} KiB raw",
           f"fetch_bytes_per_launch: {fetch_b:.0f}",
           f"write_bytes_per_launch: {write_b:.0f}",
           f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}",
           f"source_sha256: {source_digest(tag)}"]
    return "\n".join(out) + "\n"


def mfma_report(d: str, command: str, clock_mhz: float, simds: int = 1024, top: int = 40) -> str:
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    disp: dict = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            key = (f, r["Dispatch_Id"])
            e = disp.setdefault(key, {"name": r["Kernel_Name"],
                                      "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
            e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    per: dict = {}
    for e in disp.values():
        k = short_name(e["name"])
        a = per.setdefault(k, {"n": 0, "ns": 0.0, "mops": 0.0, "busy": 0.0})
        a["n"] += 1
        a["ns"] += e["ns"]
        a["mops"] += e.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
        a["busy"] += e.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
    rows = sorted(((k, a) for k, a in per.items() if a["mops"] > 0), key=lambda kv: -kv[1]["ns"])
    out = [f"command: {command}",
           f"MFMA-busy share = SQ_VALU_MFMA_BUSY_CYCLES / ({simds} SIMDs x duration x {clock_mhz:.0f} MHz); "
           "executed FLOPs = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (recomputation included); durations are the "
           "profiled dispatches' own timestamps", "",
           f"{'calls':>5} {'avg ms':>8} {'GFLOP/call':>11} {'TFLOP/s':>8} {'MFMA busy':>9}  kernel"]
    for k, a in rows[:top]:
        avg_ms = a["ns"] / a["n"] / 1e6
        fl = a["mops"] * 512 / a["n"]
        busy = a["busy"] / (simds * (a["ns"] * 1e-9) * clock_mhz * 1e6)
        out.append(f"{a['n']:5d} {avg_ms:8.4f} {fl / 1e9:11.1f} {fl / (avg_ms * 1e-3) / 1e12:8.1f} {busy:9.3f}  {k}")
    return "\n".join(out) + "\n"


def read_traffic(path: str, tag: str) -> float | None:
    """Traffic per launch from a report, or None if absent or its sources changed."""
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("tag") != tag or vals.get("source_sha256") != source_digest(tag):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", required=True)
    s.add_argument("--top", type=int, default=30)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--tag", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("dir")
    m.add_argument("--command", required=True)
    m.add_argument("--clock-mhz", type=float, required=True)
    m.add_argument("--simds", type=int, default=1024)
    a = ap.parse_args()
    if a.mode == "mfma":
        print(mfma_report(a.dir, a.command, a.clock_mhz, a.simds), end="")
    elif a.mode == "stats":
        print(stats_report(a.csv, a.command, a.top), end="")
    else:
        print(traffic_report(a.fetch, a.write, a.kernel, a.tag, a.copy_bytes, a.command_fetch, a.command_write),
              end="")


if __name__ == "__main__":
    main()
