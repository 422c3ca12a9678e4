#!/usr/bin/env python3
"""HBM traffic of the benchmark's fill kernels from rocprofv3 counters.

Runs, each as its own child process under `rocprofv3 --pmc`:
  * a calibration: a device-to-device copy of COPY_BYTES, whose FETCH_SIZE and
    WRITE_SIZE readings give the factor from counter KiB to bytes moved;
  * the benchmark step driver (this file with --drive) for 1 and for 3 steps,
    once per counter.  The difference of the two runs, halved, is one step's
    traffic: the set-up work (data upload, the first tree that fixes the row
    lists) cancels out;
  * the same pair of driver runs once more with four SQ counters of the LDS
    (instructions, active cycles, bank- and address-conflict cycles), for the
    fill's second ceiling.

Writes profiles/counters_<config>_p<bits>.json (read by bench.py, which reports
it as roofline.traffic while the kernel sources are unchanged) and a short text
summary beside it.  Run from the repository root on a machine with the GPU:

    python bench_counters.py --config c3 --precision 30
"""
from __future__ import annotations

import argparse
import collections
import glob
import hashlib
import json
import os
import re
import shutil
import sqlite3
import subprocess
import tempfile
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30
FILL_CLASS = ("k_fill_root", "k_fill_root_il", "k_fill_rows", "k_fill_cols", "k_merge")
OTHER = ("k_gather", "k_zero_slices", "k_subtract", "k_subtract_split", "k_split_feature",
         "k_split_reduce", "k_split_feature_sliced", "k_subtract_split_sliced", "k_quantize",
         "k_grad_hess_max")
# one --pmc pass of SQ counters for the LDS side of the fill (5 of the 8 SQ slots)
LDS_COUNTERS = ("SQ_INSTS_LDS", "SQ_INSTS_LDS_ATOMIC", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT",
                "SQ_LDS_ADDR_CONFLICT")
# one --pmc pass of the L2's memory read requests by size (3 of the 4 TCC
# slots): all requests, the 32-byte ones, and the 128-byte ones (BUBBLE);
# the rest are 64-byte.  FETCH_SIZE is derived from these three.
REQ_COUNTERS = ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_BUBBLE_sum")
# --stalls: what holds the fills up, one --pmc pass per set: the vector L1's
# requests to L2, their summed latency and its stalls (in-flight limit, data
# pending from L2); the address unit stalled by the L1 and the data unit by
# it; the SQ's wave cycles, waits and instruction counts
STALL_SETS = (
    ("TCP_TCC_READ_REQ_sum", "TCP_TCC_READ_REQ_LATENCY_sum", "TCP_UTCL1_STALL_INFLIGHT_MAX_sum",
     "TCP_PENDING_STALL_CYCLES_sum"),
    ("TA_ADDR_STALLED_BY_TC_CYCLES_sum", "TD_TC_STALL_sum"),
    ("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_INSTS_VALU", "SQ_INSTS_LDS",
     "SQ_INSTS_VMEM_RD", "SQ_LDS_BANK_CONFLICT"),
)
SOURCES = ("histogram_gradient_boosted_amd/csrc/*.hip", "histogram_gradient_boosted_amd/csrc/*.h",
           "include/*.h")


def _code_only(text: str) -> str:
    """The text without its comments and with whitespace collapsed, so that a
    change to comments alone keeps the hash (the counters measure the code).
    The sources hold no comment markers inside string literals."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash() -> str:
    """sha256 over the code of the HIP sources and the public header."""
    h = hashlib.sha256()
    for pat in SOURCES:
        for path in sorted(glob.glob(os.path.join(ROOT, pat))):
            h.update(os.path.relpath(path, ROOT).encode())
            with open(path, encoding="utf-8") as f:
                h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def drive(config: str, precision: int, steps: int) -> None:
    """Set up the benchmark workload and run `steps` steps (no timing)."""
    sys.path.insert(0, ROOT)
    import torch
    import bench
    from histogram_gradient_boosted_amd import binding, synth
    w = synth.make(config)
    ctx = binding.Context(0)
    ctx.set_precision(precision)
    ctx.set_async_begin(True)   # as bench.py runs it
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    g, h = bench.step_inputs(w, bench.resolve_objective(w, "auto"), torch)
    plan = bench.prepare(ctx, w, g, h, torch)
    for _ in range(steps):
        bench.step(ctx, w, plan, g, h)
    ctx.sync()
    torch.cuda.synchronize()
    ctx.close()
    print(f"drive {config} p{precision}: {steps} steps done", flush=True)


def copy_kernel() -> None:
    """Four device-to-device copies of COPY_BYTES."""
    import torch
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(4):
        b.copy_(a)
    torch.cuda.synchronize()
    print("copy done", flush=True)


REUSE = False   # --reuse: read the databases a previous run left under --out


def run_counter(counter, out_dir: str, args: list, log_path: str) -> str:
    """One rocprofv3 pass (from /tmp, the program right after --).  `counter`
    is one counter name or a tuple of names collected together."""
    if REUSE:
        dbs = glob.glob(os.path.join(out_dir, "**", "*.db"), recursive=True)
        if not dbs:
            raise SystemExit(f"--reuse: no counter database under {out_dir}")
        return dbs[0]
    if os.path.exists(out_dir):
        shutil.rmtree(out_dir)
    env = dict(os.environ, TMPDIR="/tmp")
    names = [counter] if isinstance(counter, str) else list(counter)
    cmd = ["timeout", "-s", "KILL", "600", "rocprofv3", "--pmc", *names, "-d", out_dir, "-o", "p",
           "--", sys.executable] + args
    print("[counters]", " ".join(cmd), flush=True)
    with open(log_path, "w") as log:
        r = subprocess.run(cmd, cwd="/tmp", env=env, stdout=log, stderr=subprocess.STDOUT)
    dbs = glob.glob(os.path.join(out_dir, "**", "*.db"), recursive=True)
    if r.returncode != 0 and not dbs:
        raise SystemExit(f"rocprofv3 pass failed ({r.returncode}); see {log_path}")
    if not dbs:
        raise SystemExit(f"no counter database under {out_dir}")
    return dbs[0]


def read_counter(db: str, counter: str) -> dict:
    """Sum of the counter (KiB) and dispatch count per kernel base name."""
    con = sqlite3.connect(db)
    rows = con.execute("select kernel_name, counter_name, value from counters_collection").fetchall()
    out = collections.defaultdict(lambda: [0.0, 0])
    for name, cname, value in rows:
        if cname != counter:
            continue
        base = name.split("(")[0].replace("void ", "").split("<")[0].split("::")[-1].strip()
        out[base][0] += value
        out[base][1] += 1
    return dict(out)


def stalls(args, me: str) -> None:
    """--stalls: STALL_SETS per step for the fill class and the level tail
    (3-step run - 1-step run, halved), written to
    profiles/stalls_<config>_p<bits><tag>.{json,md}.  HGB_FILL_TUNE, if set,
    is passed to the step driver and recorded with the command."""
    t0 = time.time()
    per_step = collections.defaultdict(dict)
    for i, names in enumerate(STALL_SETS):
        got = {}
        for steps in (1, 3):
            db = run_counter(names, os.path.join(args.out, f"{args.config}_p{args.precision}_stall{i}_{steps}"),
                             [me, "--drive", "--config", args.config, "--precision", str(args.precision),
                              "--steps", str(steps)],
                             os.path.join(args.out, f"{args.config}_p{args.precision}_stall{i}_{steps}.log"))
            got[steps] = {c: read_counter(db, c) for c in names}
        for c in names:
            for k in FILL_CLASS + OTHER:
                a = got[3][c].get(k, [0.0, 0])
                b = got[1][c].get(k, [0.0, 0])
                if a[1] > b[1]:
                    per_step[k][c] = (a[0] - b[0]) / 2.0
    tune = os.environ.get("HGB_FILL_TUNE", "")
    cmd = (f"HGB_FILL_TUNE={tune} " if tune else "") + \
        f"python bench_counters.py --stalls --config {args.config} --precision {args.precision}" + \
        (f" --tag {args.tag}" if args.tag else "")
    record = {"config": args.config, "precision": args.precision, "fill_tune": tune, "source_hash": source_hash(),
              "command": cmd, "per_step": per_step, "seconds": round(time.time() - t0, 1)}
    base = os.path.join(ROOT, "profiles", f"stalls_{args.config}_p{args.precision}{args.tag}")
    with open(base + ".json", "w") as f:
        json.dump(record, f, indent=1)
    lines = [f"# Stall counters per step, {args.config}, P = {args.precision}" +
             (f", HGB_FILL_TUNE={tune}" if tune else ""), "",
             f"Command: `{cmd}` (rocprofv3 --pmc, one pass per counter set; per step = (3-step run - 1-step run) / 2;",
             "summed over the chip's instances).  L2 latency is TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ; the",
             "SQ wait counters are wave-cycles (in units of 4 cycles), shown as shares of SQ_WAVE_CYCLES.", "",
             "| kernel | L1->L2 read requests | mean L2 latency (cycles) | L1 in-flight-limit stall | L1 pending-data stall "
             "| address unit stalled by L1 | data unit stalled by L1 | wait on an instruction | of it on LDS "
             "| VALU / LDS instructions | LDS bank-conflict cycles |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for k in FILL_CLASS + OTHER:
        r = per_step.get(k)
        if not r or r.get("TCP_TCC_READ_REQ_sum", 0) <= 0:
            continue
        wave = max(r.get("SQ_WAVE_CYCLES", 0.0), 1.0)
        lines.append(
            f"| {k} | {r['TCP_TCC_READ_REQ_sum']:,.0f} | "
            f"{r.get('TCP_TCC_READ_REQ_LATENCY_sum', 0) / r['TCP_TCC_READ_REQ_sum']:.0f} | "
            f"{r.get('TCP_UTCL1_STALL_INFLIGHT_MAX_sum', 0):,.0f} | {r.get('TCP_PENDING_STALL_CYCLES_sum', 0):,.0f} | "
            f"{r.get('TA_ADDR_STALLED_BY_TC_CYCLES_sum', 0):,.0f} | {r.get('TD_TC_STALL_sum', 0):,.0f} | "
            f"{r.get('SQ_WAIT_INST_ANY', 0) / wave:.2f} | {r.get('SQ_WAIT_INST_LDS', 0) / wave:.2f} | "
            f"{r.get('SQ_INSTS_VALU', 0) / max(r.get('SQ_INSTS_LDS', 0), 1):.2f} | "
            f"{r.get('SQ_LDS_BANK_CONFLICT', 0):,.0f} |")
    with open(base + ".md", "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def trace_summary(db: str, step_equiv: int, command: str) -> str:
    """Per-kernel durations from a rocprofv3 --kernel-trace database.  With
    step_equiv 0 the trees are counted from the trace: every tree starts with
    one k_max_final (the end of begin_tree's maxima)."""
    con = sqlite3.connect(db)
    rows = con.execute("select name, start, end from kernels").fetchall()
    per = collections.defaultdict(list)
    for name, start, end in rows:
        per[name.split("(")[0].replace("void ", "").strip()].append((end - start) / 1e3)
    if step_equiv <= 0:
        step_equiv = max(1, sum(len(ds) for name, ds in per.items() if name.split("::")[-1] == "k_max_final"))
    lines = [f"# Kernel trace: `{command}`", "",
             f"Summarized by `python bench_counters.py --trace-summary <dir>/kt_results.db --trace-command "
             f"'<the command above>' --trace-out <this file>`.", "",
             "rocprofv3 --kernel-trace --stats; durations in microseconds.  One process runs "
             f"{step_equiv} step-equivalents of the tree (the set-up tree, warm-up, the timed and "
             "the event-timed passes, counted by begin_tree's k_max_final); 'per step' divides "
             "the total by that.", "",
             "| kernel | dispatches | total us | avg us | min us | max us | us per step |",
             "|---|---|---|---|---|---|---|"]
    fill_total = 0.0
    for name, ds in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        tot = sum(ds)
        base = name.split("<")[0].split("::")[-1]
        if base in FILL_CLASS:
            fill_total += tot
        lines.append(f"| {name} | {len(ds)} | {tot:.1f} | {tot / len(ds):.2f} | {min(ds):.2f} | "
                     f"{max(ds):.2f} | {tot / step_equiv:.2f} |")
    lines += ["", f"Fill class ({', '.join(FILL_CLASS)}): {fill_total / step_equiv:.1f} us per step."]
    return "\n".join(lines) + "\n"


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--config", default="c3")
    ap.add_argument("--precision", type=int, default=30)
    ap.add_argument("--drive", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--copy", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--steps", type=int, default=1, help=argparse.SUPPRESS)
    ap.add_argument("--out", default=os.path.join(tempfile.gettempdir(), "hgb_counters"),
                    help="where the raw rocprofv3 databases go")
    ap.add_argument("--reuse", action="store_true",
                    help="summarize the databases already under --out instead of profiling")
    ap.add_argument("--trace-summary", metavar="DB",
                    help="summarize a rocprofv3 kernel-trace database instead")
    ap.add_argument("--step-equiv", type=int, default=0,
                    help="trees the traced process ran (0: count them from the trace)")
    ap.add_argument("--trace-command", default="")
    ap.add_argument("--trace-out")
    ap.add_argument("--stalls", action="store_true",
                    help="collect the stall counters (profiles/stalls_*) instead of the traffic counters")
    ap.add_argument("--tag", default="", help="--stalls: suffix of the output files")
    args = ap.parse_args()
    if args.trace_summary:
        text = trace_summary(args.trace_summary, args.step_equiv, args.trace_command)
        if args.trace_out:
            with open(args.trace_out, "w") as f:
                f.write(text)
        print(text, end="")
        return
    if args.drive:
        drive(args.config, args.precision, args.steps)
        return
    if args.copy:
        copy_kernel()
        return

    global REUSE
    REUSE = args.reuse
    me = os.path.abspath(__file__)
    os.makedirs(args.out, exist_ok=True)
    if args.stalls:
        stalls(args, me)
        return
    t0 = time.time()
    raw = {}
    cal = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        tag = counter.lower()
        db = run_counter(counter, os.path.join(args.out, f"copy_{tag}"), [me, "--copy"],
                         os.path.join(args.out, f"copy_{tag}.log"))
        per = read_counter(db, counter)
        copies = {k: v for k, v in per.items() if "copy" in k.lower()}
        if not copies:
            raise SystemExit(f"no copy kernel in the calibration run: {sorted(per)}")
        kib, n = max(copies.values(), key=lambda v: v[0])
        cal[counter] = {"kib_per_copy": kib / n, "factor": COPY_BYTES / (kib / n * 1024.0)}
        for steps in (1, 3):
            db = run_counter(counter, os.path.join(args.out, f"{args.config}_p{args.precision}_{tag}_{steps}"),
                             [me, "--drive", "--config", args.config, "--precision", str(args.precision),
                              "--steps", str(steps)],
                             os.path.join(args.out, f"{args.config}_p{args.precision}_{tag}_{steps}.log"))
            raw[(counter, steps)] = read_counter(db, counter)

    lds_raw = {}
    for steps in (1, 3):
        db = run_counter(LDS_COUNTERS, os.path.join(args.out, f"{args.config}_p{args.precision}_lds_{steps}"),
                         [me, "--drive", "--config", args.config, "--precision", str(args.precision),
                          "--steps", str(steps)],
                         os.path.join(args.out, f"{args.config}_p{args.precision}_lds_{steps}.log"))
        lds_raw[steps] = {c: read_counter(db, c) for c in LDS_COUNTERS}
    lds = {}
    for k in FILL_CLASS:
        rec = {}
        for c in LDS_COUNTERS:
            a = lds_raw[3][c].get(k, [0.0, 0])
            b = lds_raw[1][c].get(k, [0.0, 0])
            rec[c] = (a[0] - b[0]) / 2.0
        if rec["SQ_INSTS_LDS"] > 0:
            rec["bank_conflict_per_active"] = round(rec["SQ_LDS_BANK_CONFLICT"] / max(rec["SQ_LDS_IDX_ACTIVE"], 1.0), 4)
            lds[k] = rec

    # read requests by size: the copy (whose bytes are known), then the step
    req_raw = {}
    db = run_counter(REQ_COUNTERS, os.path.join(args.out, "copy_req"), [me, "--copy"],
                     os.path.join(args.out, "copy_req.log"))
    copy_req = {c: read_counter(db, c) for c in REQ_COUNTERS}
    for steps in (1, 3):
        db = run_counter(REQ_COUNTERS, os.path.join(args.out, f"{args.config}_p{args.precision}_req_{steps}"),
                         [me, "--drive", "--config", args.config, "--precision", str(args.precision),
                          "--steps", str(steps)],
                         os.path.join(args.out, f"{args.config}_p{args.precision}_req_{steps}.log"))
        req_raw[steps] = {c: read_counter(db, c) for c in REQ_COUNTERS}

    def req_split(vals):
        total, r32, r128 = (vals[c] for c in REQ_COUNTERS)
        return {"requests": total, "req_32B": r32, "req_128B": r128, "req_64B": total - r32 - r128,
                "bytes": 32 * r32 + 64 * (total - r32 - r128) + 128 * r128}
    copy_name = max((k for k in copy_req[REQ_COUNTERS[0]] if "copy" in k.lower()),
                    key=lambda k: copy_req[REQ_COUNTERS[0]][k][0])
    copy_n = copy_req[REQ_COUNTERS[0]][copy_name][1]
    req_copy = req_split({c: copy_req[c].get(copy_name, [0.0, 1])[0] / copy_n for c in REQ_COUNTERS})
    req_copy["copy_bytes_read"] = COPY_BYTES
    requests = {}
    for k in FILL_CLASS + OTHER:
        vals = {}
        for c in REQ_COUNTERS:
            a = req_raw[3][c].get(k, [0.0, 0])
            b = req_raw[1][c].get(k, [0.0, 0])
            vals[c] = (a[0] - b[0]) / 2.0
        if vals[REQ_COUNTERS[0]] > 0:
            requests[k] = req_split(vals)

    kernels = sorted(set(k for d in raw.values() for k in d) & set(FILL_CLASS + OTHER))
    per_step = {}
    for k in kernels:
        rec = {}
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            a = raw[(counter, 3)].get(k, [0.0, 0])
            b = raw[(counter, 1)].get(k, [0.0, 0])
            kib = (a[0] - b[0]) / 2.0
            rec[counter] = {"kib_raw": round(kib, 1),
                            "bytes": int(kib * 1024.0 * cal[counter]["factor"]),
                            "dispatches": (a[1] - b[1]) // 2}
        per_step[k] = rec
    fill_fetch = sum(per_step[k]["FETCH_SIZE"]["bytes"] for k in per_step if k in FILL_CLASS)
    fill_write = sum(per_step[k]["WRITE_SIZE"]["bytes"] for k in per_step if k in FILL_CLASS)
    record = {
        "config": args.config,
        "precision": args.precision,
        "source_hash": source_hash(),
        "command": f"python bench_counters.py --config {args.config} --precision {args.precision}",
        "calibration": {"copy_bytes": COPY_BYTES, **cal},
        "per_step": per_step,
        "fill_traffic": {"bytes_per_step": fill_fetch + fill_write, "fetch_bytes": fill_fetch,
                         "write_bytes": fill_write, "kernels": list(FILL_CLASS)},
        "lds_per_step": lds,
        "read_requests_per_step": requests,
        "read_requests_copy": req_copy,
        "seconds": round(time.time() - t0, 1),
    }
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    base = os.path.join(ROOT, "profiles", f"counters_{args.config}_p{args.precision}")
    with open(base + ".json", "w") as f:
        json.dump(record, f, indent=1)
    lines = [f"# HBM traffic per step, {args.config}, P = {args.precision}", "",
             f"Command: `{record['command']}` (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE;",
             "per step = (3-step run - 1-step run) / 2).", "",
             "Calibration, device-to-device copy of 1 GiB: "
             f"FETCH_SIZE reads {cal['FETCH_SIZE']['kib_per_copy']:.0f} KiB (factor "
             f"{cal['FETCH_SIZE']['factor']:.3f}), WRITE_SIZE reads {cal['WRITE_SIZE']['kib_per_copy']:.0f} KiB "
             f"(factor {cal['WRITE_SIZE']['factor']:.3f}).", "",
             "| kernel | dispatches/step | fetch KiB raw | fetch bytes | write KiB raw | write bytes |",
             "|---|---|---|---|---|---|"]
    for k, rec in per_step.items():
        lines.append(f"| {k} | {rec['FETCH_SIZE']['dispatches']} | {rec['FETCH_SIZE']['kib_raw']:.0f} | "
                     f"{rec['FETCH_SIZE']['bytes']:,} | {rec['WRITE_SIZE']['kib_raw']:.0f} | "
                     f"{rec['WRITE_SIZE']['bytes']:,} |")
    lines += ["", f"Fill class ({', '.join(FILL_CLASS)}): {fill_fetch + fill_write:,} bytes per step "
              f"({fill_fetch:,} fetched, {fill_write:,} written).", "",
              f"LDS counters per step (rocprofv3 --pmc {' '.join(LDS_COUNTERS)}, same differencing; "
              "summed over the chip's SQs; IDX_ACTIVE and the conflicts are cycles):", "",
              "| kernel | LDS instructions | of them atomics | LDS active cycles | bank-conflict cycles | address-conflict cycles | bank conflicts / active |",
              "|---|---|---|---|---|---|---|"]
    for k, rec in lds.items():
        lines.append(f"| {k} | {rec['SQ_INSTS_LDS']:,.0f} | {rec['SQ_INSTS_LDS_ATOMIC']:,.0f} | "
                     f"{rec['SQ_LDS_IDX_ACTIVE']:,.0f} | {rec['SQ_LDS_BANK_CONFLICT']:,.0f} | "
                     f"{rec['SQ_LDS_ADDR_CONFLICT']:,.0f} | {rec['bank_conflict_per_active']:.3f} |")
    lines += ["",
              f"L2 read requests to memory per step by size (rocprofv3 --pmc {' '.join(REQ_COUNTERS)}, "
              "same differencing; 64-byte = all - 32-byte - 128-byte).  The 1 GiB copy reads with "
              f"{req_copy['req_32B']:,.0f} 32-byte, {req_copy['req_64B']:,.0f} 64-byte and "
              f"{req_copy['req_128B']:,.0f} 128-byte requests: {req_copy['bytes']:,.0f} bytes by that count "
              f"for {COPY_BYTES:,} read.", "",
              "| kernel | requests | 32-byte | 64-byte | 128-byte | bytes by size |",
              "|---|---|---|---|---|---|"]
    for k, r in requests.items():
        lines.append(f"| {k} | {r['requests']:,.0f} | {r['req_32B']:,.0f} | {r['req_64B']:,.0f} | "
                     f"{r['req_128B']:,.0f} | {r['bytes']:,.0f} |")
    lines += ["",
              f"Kernel sources sha256: `{record['source_hash']}`."]
    with open(base + ".md", "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines), flush=True)


if __name__ == "__main__":
    main()
