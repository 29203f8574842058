"""Short text summaries of rocprofv3 output for the ISA kernels.

    python -m sparse_attention_context_amd.profile_summary trace <run_kernel_stats.csv> [bench.json] > out.txt
    python -m sparse_attention_context_amd.profile_summary counters <dir> > out.txt

`trace` formats a `rocprofv3 --kernel-trace --stats` kernel table (calls,
average duration, share of GPU time), followed by the figures of the bench
JSON line of the same run when it is given.

`counters` reads the counter CSVs of several `rocprofv3 --pmc ...
--kernel-trace --output-format csv -d <dir>/pN -o run -- python3 bench.py
--profile-pass` runs (one counter set per run, sub-directories p1, p2, ...),
labels every dispatch of the profile pass, and prints per dispatch the HBM
bytes (FETCH_SIZE and WRITE_SIZE, in KiB, each scaled by what it reads for
the pass's 1 GiB elementwise copy, the last dispatch), the MFMA busy share,
the LDS bank-conflict ratio and the wave-cycle breakdown when those
counters were collected.  The header carries a digest of the kernel sources,
which bench.py compares before it quotes a traffic figure.
"""

import csv
import glob
import hashlib
import json
import os
import sys
from collections import OrderedDict, defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
GIB = float(1 << 30)


def sources_digest():
    """sha256 over the kernel sources (csrc/*.hip, *.h, *.cpp, by name)."""
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h")) +
                       glob.glob(os.path.join(CSRC, "*.cpp"))):
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def short_name(name):
    n = name.replace("void ", "").replace("isa::", "").replace("unsigned short", "bf16")
    if "(" in n:
        n = n[:n.index("(")]
    return n.replace(", ", ",")


def trace(stats_csv, bench_json=None):
    rows = list(csv.DictReader(open(stats_csv)))
    total = sum(float(r["TotalDurationNs"]) for r in rows) or 1.0
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = ["%-72s %6s %12s %8s" % ("kernel", "calls", "avg_us", "pct")]
    for r in rows:
        name = r["Name"]
        name = name if len(name) <= 72 else name[:69] + "..."
        out.append("%-72s %6d %12.2f %8.2f" % (name, int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                                             100.0 * float(r["TotalDurationNs"]) / total))
    if bench_json:
        line = [ln for ln in open(bench_json).read().splitlines() if ln.startswith("{")][-1]
        b = json.loads(line)
        out.append("")
        out.append("# bench.py JSON line of the same run (HIP events on the launch stream):")
        out.append("#   ms_per_step %s (median of %s flushed steps), warm median %s" %
                   (b["ms_per_step"], b["timing"]["n"], b["timing"]["warm_median_ms"]))
        rf = b.get("roofline") or {}
        if rf:
            out.append("#   dominant kernel avg %s ms -> %s %s (frac %s of %s)" %
                       (rf.get("avg_launch_ms"), rf.get("achieved"), rf.get("unit"), rf.get("frac"), rf.get("peak")))
        for o in b.get("other_rooflines") or []:
            out.append("#   %s: avg %s ms -> %s %s (frac %s)" % (o["kernel"], o.get("avg_launch_ms"), o["achieved"],
                                                                o["unit"], o["frac"]))
        out.append("#   stages (ms): " + ", ".join("%s %s" % kv for kv in (b.get("stage_ms") or {}).items()))
    return "\n".join(out)


def _dispatches(run_dir):
    """{dispatch id: (kernel name, {counter: value})} of one counter run."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % run_dir)
    d = OrderedDict()
    for r in csv.DictReader(open(files[0])):
        k = int(r["Dispatch_Id"])
        if k not in d:
            d[k] = (r["Kernel_Name"], defaultdict(float))
        d[k][1][r["Counter_Name"]] += float(r["Counter_Value"])
    return d


def _labels(names):
    """Labels of the profile pass's dispatches: the layer's kernels by name,
    torch's kernels by position (input casts first; the ones fill and the
    elementwise copy probe last)."""
    labels = []
    n = len(names)
    for i, name in enumerate(names):
        if "isa::" in name:
            s = short_name(name)
            if s.startswith("isa_flash_pps_kernel"):
                s = "isa_flash_pps_kernel full route"
            elif s.startswith("isa_flash_pp_kernel<1,1,"):
                s = s[:s.index(">") + 1] + " full route"
            elif s.startswith("isa_flash_pp_kernel<0,0,"):
                s = s[:s.index(">") + 1] + " dense"
            labels.append(s)
        elif "rocclr" in name:
            labels.append("runtime copy (input upload)")
        elif i == n - 1:
            labels.append("copy probe: torch.mul(src, 1.0, out=dst), 1 GiB")
        elif i == n - 2:
            labels.append("torch.ones fill, 1 GiB out")
        else:
            labels.append("torch input cast (outside the layer)")
    seen = defaultdict(int)
    out = []
    for s in labels:
        seen[s] += 1
        out.append(s if s.startswith("isa") else "%s #%d" % (s, seen[s]))
    return out


def counters(base):
    runs = sorted(p for p in glob.glob(os.path.join(base, "p*")) if os.path.isdir(p))
    per_run = [_dispatches(r) for r in runs]
    n = min(len(d) for d in per_run)
    names = [v[0] for v in list(per_run[0].values())[:n]]
    for d in per_run[1:]:
        if [v[0] for v in list(d.values())[:n]] != names:
            raise SystemExit("the counter runs dispatched different kernels")
    vals = [defaultdict(float) for _ in range(n)]
    for d in per_run:
        for i, (_, c) in enumerate(list(d.values())[:n]):
            for k, v in c.items():
                vals[i][k] += v
    labels = _labels(names)
    probe = vals[-1]
    fetch_scale = GIB / (probe["FETCH_SIZE"] * 1024.0) if probe.get("FETCH_SIZE") else None
    write_scale = GIB / (probe["WRITE_SIZE"] * 1024.0) if probe.get("WRITE_SIZE") else None
    out = ["# calibration: the copy probe reads and writes 1 GiB; it reads FETCH_SIZE %.0f KiB, WRITE_SIZE %.0f KiB"
           % (probe.get("FETCH_SIZE", 0.0), probe.get("WRITE_SIZE", 0.0)),
           "#   fetch_scale %s   write_scale %s   (HBM bytes = (FETCH_SIZE*fetch_scale + WRITE_SIZE*write_scale) * 1024)"
           % ("%.4f" % fetch_scale if fetch_scale else "-", "%.4f" % write_scale if write_scale else "-"),
           "# MFMA_busy% = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs * 1024 SIMDs); "
           "LDS_confl = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE",
           "# kernel sources sha256: %s" % sources_digest(), "#",
           "%-48s %12s %12s %10s %10s %9s" % ("kernel", "FETCH_KiB", "WRITE_KiB", "HBM_MB", "MFMA_busy%", "LDS_confl")]
    for lab, v in zip(labels, vals):
        hbm = None
        if fetch_scale and write_scale:
            hbm = (v["FETCH_SIZE"] * fetch_scale + v["WRITE_SIZE"] * write_scale) * 1024.0 / 1e6
        mfma = None
        if v.get("GRBM_GUI_ACTIVE") and "SQ_VALU_MFMA_BUSY_CYCLES" in v:
            mfma = 100.0 * v["SQ_VALU_MFMA_BUSY_CYCLES"] / (v["GRBM_GUI_ACTIVE"] / 8.0 * 1024.0)
        confl = v["SQ_LDS_BANK_CONFLICT"] / v["SQ_LDS_IDX_ACTIVE"] if v.get("SQ_LDS_IDX_ACTIVE") else None
        out.append("%-48s %12.0f %12.0f %10s %10s %9s" % (
            lab[:48], v.get("FETCH_SIZE", 0.0), v.get("WRITE_SIZE", 0.0), "-" if hbm is None else "%.1f" % hbm,
            "-" if mfma is None else "%.1f" % mfma, "-" if confl is None else "%.3f" % confl))
    if any(v.get("SQ_WAVE_CYCLES") for v in vals):
        out += ["", "# wave-cycle shares (SQ counters summed over the chip): wait = SQ_WAIT_ANY, "
                    "issue-wait = SQ_WAIT_INST_ANY, active = SQ_ACTIVE_INST_ANY, lds-wait = SQ_WAIT_INST_LDS, "
                    "each / SQ_WAVE_CYCLES",
                "%-48s %8s %8s %8s %9s" % ("kernel", "wait%", "issue%", "active%", "ldswait%")]
        for lab, v in zip(labels, vals):
            wc = v.get("SQ_WAVE_CYCLES")
            if not wc:
                continue
            f = lambda k: "%.1f" % (100.0 * v[k] / wc) if k in v else "-"
            out.append("%-48s %8s %8s %8s %9s" % (lab[:48], f("SQ_WAIT_ANY"), f("SQ_WAIT_INST_ANY"),
                                                   f("SQ_ACTIVE_INST_ANY"), f("SQ_WAIT_INST_LDS")))
    return "\n".join(out)


def main(argv):
    if len(argv) >= 2 and argv[0] == "trace":
        print(trace(argv[1], argv[2] if len(argv) > 2 else None))
    elif len(argv) == 2 and argv[0] == "counters":
        print(counters(argv[1]))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
