"""Turn rocprofv3 CSV output into the short text summaries kept in profiles/.

    python -m fp8_block_scaled_03_amd.profiling stats  STATS_CSV --cmd "<command>"
    python -m fp8_block_scaled_03_amd.profiling traffic --fetch FETCH_CSV --write WRITE_CSV \
        --kernel gemm_tile_kernel --copy-bytes 268435456 --cmd "<command>"
    python -m fp8_block_scaled_03_amd.profiling counters P1_CSV P2_CSV --kernel KERNEL \
        --k-blocks KB --cmd "<command>"

``traffic`` scales FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by what the same
counters read for a plain device copy of known size in the same run
(``__amd_rocclr_copyBuffer``), and records the hash of the GEMM sources so that
the bench reports the figure only while the kernel is unchanged.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import os
import re
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEMM_SOURCES = ["fp8_block_scaled_03_amd/csrc/gemm.hip", "fp8_block_scaled_03_amd/csrc/common.hpp",
                "fp8_block_scaled_03_amd/csrc/launch.hpp"]


def _code_only(text: str) -> str:
    """Source text without comments, trailing blanks or empty lines, so that a
    comment edit does not retire a profile of unchanged code."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def source_sha(paths=GEMM_SOURCES) -> str:
    """Hash of the listed sources (code only) and of the compiler flags every
    HIP source is built with: a change to either retires a profile.  Include
    paths are left out: they name the checkout's location, which differs
    between the machine that writes a summary and the one that reads it."""
    from . import build
    h = hashlib.sha256()
    h.update(" ".join(f for f in build.COMMON_FLAGS if not f.startswith("-I")).encode())
    for p in paths:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    name = name.split("(")[0]
    return name.replace("void ", "")


def stats_summary(path: str, cmd: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = [f"# rocprofv3 kernel statistics", f"# command: {cmd}",
           f"{'kernel':60s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}"]
    for r in rows:
        out.append(f"{_short(r['Name'])[:60]:60s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                   f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):6.2f}")
    return "\n".join(out) + "\n"


def _counter(path: str, counter: str):
    per = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        per.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return per


def traffic_summary(fetch: str, write: str, kernel: str, copy_bytes: int, cmd: str,
                    sources=GEMM_SOURCES) -> str:
    f = _counter(fetch, "FETCH_SIZE")
    w = _counter(write, "WRITE_SIZE")
    copy_name = [k for k in f if "copyBuffer" in k][0]
    f_factor = statistics.median(f[copy_name]) * 1024 / copy_bytes
    w_factor = statistics.median(w[copy_name]) * 1024 / copy_bytes
    name = [k for k in f if k.endswith(kernel)]
    if len(name) != 1:
        raise ValueError(f"kernel {kernel!r} matches {name}")
    name = name[0]
    fk = statistics.median(f[name])
    wk = statistics.median(w[name])
    read_b = fk * 1024 / f_factor
    write_b = wk * 1024 / w_factor
    lines = [
        "# HBM traffic per launch from rocprofv3 counters (FETCH_SIZE, WRITE_SIZE in KiB per dispatch),",
        "# each divided by what the counter reads for a plain device copy of known size in the same run.",
        f"# command: {cmd}",
        f"kernel: {kernel}",
        f"source_sha: {source_sha(sources)}",
        f"sources: {' '.join(sources)}",
        f"copy_bytes: {copy_bytes}",
        f"fetch_factor: {f_factor:.4f}",
        f"write_factor: {w_factor:.4f}",
        f"fetch_kib_raw: {fk:.1f}",
        f"write_kib_raw: {wk:.1f}",
        f"hbm_read_bytes_per_launch: {read_b:.0f}",
        f"hbm_write_bytes_per_launch: {write_b:.0f}",
        f"hbm_bytes_per_launch: {read_b + write_b:.0f}",
    ]
    for k in sorted(f):
        if k in w:
            lines.append(f"# other kernel {k[:50]}: read {statistics.median(f[k]) * 1024 / f_factor / 1e6:.1f} MB, "
                         f"write {statistics.median(w[k]) * 1024 / w_factor / 1e6:.1f} MB")
    return "\n".join(lines) + "\n"


def counters_summary(paths, kernel: str, k_blocks: int, cmd: str) -> str:
    """SQ counters of one kernel (median over its dispatches) and the ratios
    derived from them.  GRBM_GUI_ACTIVE is summed over the 8 XCDs and the SQ
    cycle counters over the 1024 SIMDs, so a fraction of SIMD time is
    counter / (GRBM_GUI_ACTIVE / 8 * 1024)."""
    per = {}
    for path in paths:
        for r in csv.DictReader(open(path)):
            if not _short(r["Kernel_Name"]).endswith(kernel):
                continue
            per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    med = {k: statistics.median(v) for k, v in per.items()}
    lines = ["# rocprofv3 SQ counters (median per dispatch) and ratios derived from them",
             f"# command: {cmd}", f"kernel: {kernel}", f"source_sha: {source_sha()}"]
    for k in sorted(med):
        lines.append(f"{k}: {med[k]:.0f}")
    waves = med.get("SQ_WAVES", 0.0)
    if waves:
        for name in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU"):
            if name in med:
                lines.append(f"{name.lower()}_per_wave_per_kblock: {med[name] / waves / k_blocks:.1f}")
    if "SQ_LDS_BANK_CONFLICT" in med and med.get("SQ_LDS_IDX_ACTIVE"):
        lines.append(f"lds_bank_conflict_share_of_active: {med['SQ_LDS_BANK_CONFLICT'] / med['SQ_LDS_IDX_ACTIVE']:.3f}")
    if med.get("GRBM_GUI_ACTIVE"):
        simd_cycles = med["GRBM_GUI_ACTIVE"] / 8 * 1024
        # (SQ_ACTIVE_INST_* read the same as the instruction counts here, so
        # they give no busy fraction; only the MFMA counter does)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in med:
            lines.append(f"mfma_busy_fraction_of_simd_time: {med['SQ_VALU_MFMA_BUSY_CYCLES'] / simd_cycles:.3f}")
    return "\n".join(lines) + "\n"


def read_traffic(path: str):
    """Parse a traffic summary; returns a dict of its key: value lines."""
    d = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        d[k.strip()] = v.strip()
    return d


def main():
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--cmd", required=True)
    t.add_argument("--sources", nargs="+", default=GEMM_SOURCES,
                   help="files whose hash ties the figure to the profiled kernel")
    q = sub.add_parser("counters")
    q.add_argument("csv", nargs="+")
    q.add_argument("--kernel", required=True)
    q.add_argument("--k-blocks", type=int, required=True, help="K/32 of the profiled launch")
    q.add_argument("--cmd", required=True)
    a = p.parse_args()
    if a.what == "stats":
        print(stats_summary(a.csv, a.cmd), end="")
    elif a.what == "counters":
        print(counters_summary(a.csv, a.kernel, a.k_blocks, a.cmd), end="")
    else:
        print(traffic_summary(a.fetch, a.write, a.kernel, a.copy_bytes, a.cmd, a.sources), end="")


if __name__ == "__main__":
    main()
