"""Summaries of rocprofv3 output for the decode kernels.

    python profsum.py stats RUN_kernel_stats.csv --command "..."
        Markdown table of per-kernel launch counts and durations.

    python profsum.py sq RUN_counter_collection.csv --last 32
        Per-kernel SQ instruction counts per wave and the VALU issue share:
        SQ_INSTS_VALU * 4 cycles (a wave64 VALU instruction on a 16-lane SIMD)
        / (1024 SIMDs * GRBM_GUI_ACTIVE / 8), GRBM_GUI_ACTIVE being summed over
        the 8 XCDs.

    python profsum.py traffic --fetch BENCH_FETCH.csv \
        --write BENCH_WRITE.csv --copy-fetch COPY_FETCH.csv --copy-write COPY_WRITE.csv \
        --kernel mamba2_decode_kernel --replay --last 32 --copy-bytes 1073741824 \
        [--ea-rd BENCH_EA_RD.csv --ea-wr BENCH_EA_WR.csv]
        HBM bytes per launch of one kernel from the FETCH_SIZE and WRITE_SIZE
        counters (KiB per dispatch), each scaled by the ratio between the known
        size of a plain device copy and what the same counter reads for it;
        with the --ea-* runs, the same bytes counted a second way, from the
        L2-to-fabric request counters by request size (no scaling).
        Prints JSON; ``source_sha256`` fingerprints the kernel sources the
        counters were taken on, so a reader can tell when they are stale.
"""

import argparse
import csv
import hashlib
import json
import os
import sys

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "linear_recurrence_amd", "csrc")
KERNEL_SOURCES = {
    "mamba2_decode_kernel": ("mamba2_kernel.hpp", "mamba2_decode.hip", "rssm_device.hpp",
                             "rssm_host.hpp"),
    "gdn_decode_kernel": ("gdn_common.hpp", "gdn_decode.hip", "rssm_device.hpp", "rssm_host.hpp"),
}


def source_sha256(kernel):
    """SHA-256 over the source files a kernel is compiled from."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(name.encode())
            h.update(fh.read())
    return h.hexdigest()


def _rows(path):
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def _is_replay(name):
    """The REPLAY template argument of a kernel name: the sixth of
    mamba2_decode_kernel<ST, IT, OT, P, N, REPLAY, SR, PER>, the fifth of
    gdn_decode_kernel<IT, OT, V, K, REPLAY, KDA>."""
    args = [a.strip() for a in name[name.index("<") + 1:name.rindex(">(")].split(",")]
    return (args[5] if "mamba2_decode_kernel" in name else args[4]) == "true"


def _dispatch_kib(path, kernel, replay, last):
    """Counter value (KiB) per dispatch of `kernel`, the last `last` ones."""
    per = {}
    for r in _rows(path):
        name = r["Kernel_Name"]
        if kernel not in name or _is_replay(name) != replay:
            continue
        d = int(r["Dispatch_Id"])
        per[d] = per.get(d, 0.0) + float(r["Counter_Value"])
    ids = sorted(per)[-last:] if last else sorted(per)
    if not ids:
        raise SystemExit(f"no dispatches of {kernel} (replay={replay}) in {path}")
    return [per[i] for i in ids]


def _dispatch_counters(path, kernel, replay, last):
    """{counter: value} per dispatch of `kernel` (summed over instances), the last `last`."""
    per = {}
    for r in _rows(path):
        name = r["Kernel_Name"]
        if kernel not in name or _is_replay(name) != replay:
            continue
        c = per.setdefault(int(r["Dispatch_Id"]), {})
        c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    ids = sorted(per)[-last:] if last else sorted(per)
    if not ids:
        raise SystemExit(f"no dispatches of {kernel} (replay={replay}) in {path}")
    return [per[i] for i in ids]


def ea_bytes(rd_path, wr_path, kernel, replay, last):
    """HBM-side bytes per dispatch from the L2-to-fabric request counters,
    each request counted at its size: reads 32 B x RDREQ_32B + 64 B x
    RDREQ_64B + 128 B x RDREQ_128B, writes 64 B x WRREQ_64B + 32 B x the
    other write requests.  No copy-kernel scaling is involved."""
    rd = _dispatch_counters(rd_path, kernel, replay, last)
    wr = _dispatch_counters(wr_path, kernel, replay, last)
    n = len(rd)
    g = lambda lst, k: sum(c.get(k, 0.0) for c in lst) / len(lst)
    r32, r64, r128 = (g(rd, "TCC_EA0_RDREQ_32B_sum"), g(rd, "TCC_EA0_RDREQ_64B_sum"),
                      g(rd, "TCC_EA0_RDREQ_128B_sum"))
    rall = g(rd, "TCC_EA0_RDREQ_sum")
    w64, wall = g(wr, "TCC_EA0_WRREQ_64B_sum"), g(wr, "TCC_EA0_WRREQ_sum")
    return {
        "dispatches": [n, len(wr)],
        "rdreq_per_dispatch": {"all": rall, "32B": r32, "64B": r64, "128B": r128},
        "wrreq_per_dispatch": {"all": wall, "64B": w64},
        "rdreq_dram_per_dispatch": g(wr, "TCC_EA0_RDREQ_DRAM_sum"),
        "wrreq_dram_per_dispatch": g(wr, "TCC_EA0_WRREQ_DRAM_sum"),
        "read_bytes_per_launch": 32 * r32 + 64 * r64 + 128 * r128,
        "write_bytes_per_launch": 64 * w64 + 32 * (wall - w64),
    }


def _copy_factor(path, known_bytes):
    """known bytes / counter bytes for the largest dispatches (the probe copies)."""
    per = {}
    for r in _rows(path):
        d = int(r["Dispatch_Id"])
        per[d] = per.get(d, 0.0) + float(r["Counter_Value"])
    vals = sorted(per.values())
    big = [v for v in vals if v >= 0.5 * vals[-1]]
    kib = sum(big) / len(big)
    return known_bytes / (kib * 1024.0), kib


def cmd_stats(args):
    rows = _rows(args.csv)
    out = []
    if args.command:
        out.append("Command:\n\n```\n" + args.command + "\n```\n")
    out.append("| kernel | calls | avg us | min us | max us | share |")
    out.append("|---|---:|---:|---:|---:|---:|")
    for r in rows:
        name = r["Name"] if "rssm::" in r["Name"] else r["Name"][:60] + "..."
        out.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                   f"{float(r['Percentage']):.1f}% |")
    print("\n".join(out))


def cmd_sq(args):
    per, name = {}, {}
    for r in _rows(args.csv):
        d = int(r["Dispatch_Id"])
        c = per.setdefault(d, {})
        c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        name[d] = r["Kernel_Name"]
    groups = {}
    for d in sorted(per):
        if "rssm::" in name[d]:
            groups.setdefault(name[d], []).append(per[d])
    out = []
    if args.command:
        out.append("Command:\n\n```\n" + args.command + "\n```\n")
    out.append("| kernel | dispatches | waves | VALU/wave | SALU/wave | LDS/wave | "
               "active us | VALU issue share | wait share of wave cycles |")
    out.append("|---|---:|---:|---:|---:|---:|---:|---:|---:|")
    for n, lst in groups.items():
        lst = lst[-args.last:] if args.last else lst
        avg = {k: sum(c[k] for c in lst) / len(lst) for k in lst[0]}
        w = avg["SQ_WAVES"]
        gui = avg["GRBM_GUI_ACTIVE"] / 8.0
        share = avg["SQ_INSTS_VALU"] * 4.0 / (1024.0 * gui)
        out.append(f"| `{n}` | {len(lst)} | {w:.0f} | {avg['SQ_INSTS_VALU'] / w:.0f} | "
                   f"{avg['SQ_INSTS_SALU'] / w:.0f} | {avg['SQ_INSTS_LDS'] / w:.0f} | "
                   f"{gui / 2400.0:.1f} | {share:.2f} | "
                   f"{avg['SQ_WAIT_INST_ANY'] / avg['SQ_WAVE_CYCLES']:.2f} |")
    print("\n".join(out))


def cmd_traffic(args):
    ff, fkib = _copy_factor(args.copy_fetch, args.copy_bytes)
    wf, wkib = _copy_factor(args.copy_write, args.copy_bytes)
    fetch = _dispatch_kib(args.fetch, args.kernel, args.replay, args.last)
    write = _dispatch_kib(args.write, args.kernel, args.replay, args.last)
    fb = sum(fetch) / len(fetch) * 1024.0 * ff
    wb = sum(write) / len(write) * 1024.0 * wf
    res = {
        "kernel": args.kernel + (" (replay)" if args.replay else " (standard)"),
        "dispatches": [len(fetch), len(write)],
        "fetch_kib_per_dispatch": sum(fetch) / len(fetch),
        "write_kib_per_dispatch": sum(write) / len(write),
        "copy_probe_bytes": args.copy_bytes,
        "copy_fetch_kib": fkib, "copy_write_kib": wkib,
        "fetch_factor": ff, "write_factor": wf,
        "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
        "bytes_per_launch": fb + wb,
        "source_sha256": source_sha256(args.kernel),
    }
    if args.ea_rd and args.ea_wr:
        ea = ea_bytes(args.ea_rd, args.ea_wr, args.kernel, args.replay, args.last)
        ea["bytes_per_launch"] = ea["read_bytes_per_launch"] + ea["write_bytes_per_launch"]
        res["ea_request_counters"] = ea
    if args.command:
        res["commands"] = args.command
    print(json.dumps(res, indent=1))


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", default=None)
    q = sub.add_parser("sq")
    q.add_argument("csv")
    q.add_argument("--last", type=int, default=0)
    q.add_argument("--command", default=None)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--kernel", required=True, choices=sorted(KERNEL_SOURCES))
    t.add_argument("--replay", action="store_true")
    t.add_argument("--last", type=int, default=0)
    t.add_argument("--copy-bytes", type=float, default=float(1 << 30))
    t.add_argument("--ea-rd", default=None,
                   help="counter CSV with TCC_EA0_RDREQ{,_32B,_64B,_128B}_sum")
    t.add_argument("--ea-wr", default=None,
                   help="counter CSV with TCC_EA0_WRREQ{,_64B}_sum (and the _DRAM pair)")
    t.add_argument("--command", action="append", default=None)
    args = ap.parse_args(argv)
    {"stats": cmd_stats, "sq": cmd_sq, "traffic": cmd_traffic}[args.mode](args)


if __name__ == "__main__":
    main(sys.argv[1:])
