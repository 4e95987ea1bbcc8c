"""Short text summaries of rocprofv3 output for this library's kernels.

  python -m long_context_decode_attn_amd.profsum kernels TRACE.csv [--match S]
      per-kernel launch count and median / mean / p10 / p90 duration from a
      --kernel-trace CSV (run_kernel_trace.csv)
  python -m long_context_decode_attn_amd.profsum counters COUNTERS.csv [--match S]
      mean value per dispatch of every counter, per kernel, from a --pmc CSV
  python -m long_context_decode_attn_amd.profsum traffic --fetch F.csv --write W.csv \\
          --copy-fetch CF.csv --copy-write CW.csv --copy-bytes N --match S --bytes ALG --out FILE
      HBM bytes per launch of the kernel matching S: FETCH_SIZE and WRITE_SIZE (KiB per
      dispatch) each scaled by what the same counter reads for a plain copy of N bytes
      (which reads N and writes N bytes), written with the digest of the kernel sources
      so that a reader can tell whether the figure still applies.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
# The sources each measured kernel is built from (the digest of a traffic summary).
_C = "long_context_decode_attn_amd/csrc/"
KERNEL_SOURCES = {
    "split_mfma": (_C + "split_mfma.hip", _C + "mfma_tile.h", _C + "common.h", _C + "internal.h"),
    "split_rows": (_C + "split_rows.hip", _C + "mfma_tile.h", _C + "common.h", _C + "internal.h"),
    "split_valu": (_C + "split_valu.hip", _C + "common.h", _C + "internal.h"),
    "topk_unit": (_C + "sig_topk_unit.hip", _C + "sparse.h", _C + "sig_proj.h", _C + "common.h", _C + "internal.h"),
    "wide": (_C + "sig_topk_wide.hip", _C + "wide.h", _C + "common.h", _C + "internal.h"),
}


def kernel_source_digest(kind: str = "split_mfma") -> str:
    """First 16 hex digits of the sha256 over the sources of kernel family `kind`."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    name = name.replace("void ", "").replace("lcda::(anonymous namespace)::", "").replace("lcda::", "")
    return name[:name.index("(")] if "(" in name else name


def _quant(v, q):
    v = sorted(v)
    return v[min(len(v) - 1, int(q * len(v)))]


def kernels(path: str, match: str = "") -> str:
    d = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        nm = r["Kernel_Name"]
        if match and match not in nm:
            continue
        wgs = 1
        for ax in "XYZ":
            wgs *= max(1, int(r.get("Grid_Size_" + ax, 1) or 1))
        wg = max(1, int(r.get("Workgroup_Size_X", 1) or 1)) * max(1, int(r.get("Workgroup_Size_Y", 1) or 1)) * \
            max(1, int(r.get("Workgroup_Size_Z", 1) or 1))
        d[(short_name(nm), wgs // wg)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["%-58s %8s %6s %10s %10s %10s %10s" % ("kernel", "WGs", "calls", "median_us", "mean_us", "p10_us",
                                                    "p90_us")]
    for (nm, wgs), v in sorted(d.items(), key=lambda kv: -sum(kv[1])):
        lines.append("%-58s %8d %6d %10.2f %10.2f %10.2f %10.2f" % (nm[:58], wgs, len(v), _quant(v, 0.5),
                                                                   sum(v) / len(v), _quant(v, 0.1), _quant(v, 0.9)))
    return "\n".join(lines)


def counter_means(path: str, match: str = "") -> dict:
    """{(kernel, counter): mean value per dispatch} from a rocprofv3 --pmc CSV."""
    per = collections.defaultdict(lambda: collections.defaultdict(float))   # (kernel, counter) -> dispatch -> sum
    for r in csv.DictReader(open(path)):
        nm = r["Kernel_Name"]
        if match and match not in nm:
            continue
        did = r.get("Dispatch_Id") or r.get("Correlation_Id")
        per[(short_name(nm), r["Counter_Name"])][did] += float(r["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in per.items()}


def counters(path: str, match: str = "") -> str:
    m = counter_means(path, match)
    lines = ["%-58s %-28s %16s" % ("kernel", "counter", "mean/dispatch")]
    for (k, c), v in sorted(m.items()):
        lines.append("%-58s %-28s %16.1f" % (k[:58], c, v))
    return "\n".join(lines)


def _one(path, counter, match):
    m = {k: v for k, v in counter_means(path, match).items() if k[1] == counter}
    if not m:
        raise SystemExit("no %s for a kernel matching %r in %s" % (counter, match, path))
    # the copy run holds one kernel of interest; the library runs hold one per name
    key = max(m, key=lambda k: m[k])
    return key[0], m[key]


def traffic(a) -> str:
    kname, f_kib = _one(a.fetch, "FETCH_SIZE", a.match)
    _, w_kib = _one(a.write, "WRITE_SIZE", a.match)
    cname, cf_kib = _one(a.copy_fetch, "FETCH_SIZE", a.copy_match)
    _, cw_kib = _one(a.copy_write, "WRITE_SIZE", a.copy_match)
    ff = a.copy_bytes / (cf_kib * 1024.0)
    fw = a.copy_bytes / (cw_kib * 1024.0)
    hbm = f_kib * 1024.0 * ff + w_kib * 1024.0 * fw
    out = [
        "# HBM traffic per launch of %s" % kname,
        "# FETCH_SIZE / WRITE_SIZE in KiB per dispatch (rocprofv3 --pmc, one counter per run), each",
        "# scaled by the same counter's reading for a plain copy of copy_bytes (%s)" % cname,
        "kernel = %s" % kname,
        "fetch_kib_per_dispatch = %.1f" % f_kib,
        "write_kib_per_dispatch = %.1f" % w_kib,
        "copy_bytes = %d" % a.copy_bytes,
        "copy_fetch_kib = %.1f" % cf_kib,
        "copy_write_kib = %.1f" % cw_kib,
        "fetch_scale = %.4f" % ff,
        "write_scale = %.4f" % fw,
        "hbm_bytes_per_launch = %.0f" % hbm,
        "algorithmic_bytes_per_launch = %d" % a.bytes,
        "hbm_over_algorithmic = %.4f" % (hbm / a.bytes),
        "source_kind = %s" % a.kind,
        "source_digest = %s" % kernel_source_digest(a.kind),
    ]
    for c in a.command or []:
        out.append("command = %s" % c)
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("csv")
    k.add_argument("--match", default="lcda")
    c = sub.add_parser("counters")
    c.add_argument("csv")
    c.add_argument("--match", default="")
    t = sub.add_parser("traffic")
    for f in ("fetch", "write", "copy_fetch", "copy_write"):
        t.add_argument("--" + f.replace("_", "-"), dest=f, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--copy-match", default="")
    t.add_argument("--match", required=True)
    t.add_argument("--bytes", type=int, required=True, help="algorithmic bytes per launch")
    t.add_argument("--kind", default="split_mfma", choices=sorted(KERNEL_SOURCES),
                   help="kernel family whose sources the digest covers")
    t.add_argument("--command", action="append", help="command that produced the inputs (repeatable)")
    t.add_argument("--out")
    a = ap.parse_args(argv)
    if a.cmd == "kernels":
        text = kernels(a.csv, a.match)
    elif a.cmd == "counters":
        text = counters(a.csv, a.match)
    else:
        text = traffic(a)
    if getattr(a, "out", None):
        with open(a.out, "w") as f:
            f.write(text)
    else:
        sys.stdout.write(text + ("" if text.endswith("\n") else "\n"))


if __name__ == "__main__":
    main()
