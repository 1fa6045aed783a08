"""Summaries of rocprofv3 runs of ``bench.py`` for ``profiles/``.

Every bench call is matched to its GPU dispatches by position: the bench's
JSON line lists its kernels in launch order (the step's kernels, then the
ones timed outside the step, then the 1 GiB device copy), each call of the
C ABI launches one grid, or two when a GEMM runs its last wave as a second
grid of 128x256 tiles, or three when a BF16 GEMM runs its last wave with K
split in two (the split grid, the kernel adding the halves, the grid of the
other columns), and bench.py runs every step kernel (warm-up + timed
steps) before the outside-step ones (2 untimed + timed calls each, and for a
quantizer with a "warm" entry as many calls again back to back).  Each figure
is the mean over the timed calls (for the outside-step ones, the cold calls).

  python profile_summary.py trace BENCH_JSON TRACE_DIR --steps K
      kernel-trace table (rocprofv3 --kernel-trace --stats) -> stdout (markdown)
  python profile_summary.py traffic BENCH_JSON FETCH_DIR WRITE_DIR CLOCK_DIR --steps K
      calibrated HBM bytes per launch (FETCH_SIZE, WRITE_SIZE, scaled by what the
      counters read for the plain 1 GiB copy) and the GEMMs' average shader clock
      (GRBM_GUI_ACTIVE / (8 XCDs x duration)) -> profiles/hbm_traffic.json + markdown on stdout

  python profile_summary.py counters BENCH_JSON MFMA_DIR WAIT_DIR --steps K
      per-GEMM matrix-core utilisation from two SQ counter runs (MFMA_PASS, WAIT_PASS
      below) -> profiles/gemm_counters.json + markdown on stdout

BENCH_JSON is a file holding the bench's JSON line (any run of the same tree).

Counter units on gfx950, as read here: GRBM_GUI_ACTIVE adds the busy cycles of
the 8 XCDs; SQ_VALU_MFMA_BUSY_CYCLES adds, over every SIMD, the cycles its
matrix core is busy (32 per v_mfma_*_16x16x128_f8f6f4); SQ_INSTS_* count
instructions over all waves; SQ_WAVE_CYCLES, SQ_WAIT_* and SQ_ACTIVE_INST_ANY
count wave cycles in units of 4.  MFMA busy = MFMA busy cycles / (SIMDs x
GRBM_GUI_ACTIVE / 8); the VALU estimate charges each non-MFMA VALU
instruction 4 cycles (a wave64 FP32 operation on a 16-lane SIMD).
"""

import argparse
import csv
import glob
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))

# kernel family expected for each bench name (checked on every matched dispatch)
FAMILIES = [
    ("requant", "quant_128x1_kernel<unsigned char"),    # the 128x1 kernel reading FP8 codes
    ("quant 1x128+128x1", "quant_dual_kernel"),
    ("quant_128x128", ("quant_128x128_kernel", "quant_128x256_kernel")),   # one- or two-block workgroups
    ("quant_1x128", "quant_1x128_kernel"),
    ("quant_128x1", "quant_128x1_kernel"),
    ("gemm", "gemm_blockscaled_kernel"),
]
COPY = "calibration copy 1 GiB"
XCDS = 8
SIMDS = 256 * 4        # MI355X: 256 compute units of 4 SIMDs
# the two counter passes of the `counters` command (each within the per-pass
# limits: at most 8 SQ and 2 GRBM counters)
MFMA_PASS = ["GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_INSTS_VALU",
             "SQ_INSTS_MFMA", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS", "SQ_WAVE_CYCLES"]
WAIT_PASS = ["GRBM_GUI_ACTIVE", "SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY",
             "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_SALU", "SQ_BUSY_CYCLES", "SQ_INSTS_SMEM"]


def family(bench_name):
    """Kernel names (a tuple) that a bench call of this name may launch."""
    for prefix, fam in FAMILIES:
        if bench_name.startswith(prefix):
            return fam if isinstance(fam, tuple) else (fam,)
    raise ValueError(f"no kernel family for bench name {bench_name!r}")


def is_second_grid(kernel_name):
    """The 128x256 grid that a GEMM call launches after its first grid."""
    return "gemm_blockscaled_kernel<128, 256, 2, 4," in kernel_name


def continues_call(call, kernel_name):
    """Whether a dispatch belongs to the GEMM call whose dispatches so far are `call`: the 128x256 grid of a
    balanced last wave, or, for a BF16 call whose last wave ran with K split in two, the kernel that adds the two
    halves and then the grid of the remaining columns."""
    first, last = call[0]["name"], call[-1]["name"]
    if "gemm_blockscaled_kernel" not in first:
        return False
    if is_second_grid(kernel_name):
        return True
    if "ksplit_sum_bf16_kernel" in kernel_name:
        return "gemm_blockscaled_kernel" in last and len(call) == 1
    return "ksplit_sum_bf16_kernel" in last and "gemm_blockscaled_kernel" in kernel_name


def read_bench(path):
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if line.startswith("{"):
                return json.loads(line)
    raise ValueError(f"no JSON line in {path}")


def read_csv(d, suffix):
    files = glob.glob(os.path.join(d, "**", f"*_{suffix}.csv"), recursive=True)
    if len(files) != 1:
        raise ValueError(f"expected one *_{suffix}.csv under {d}, found {files}")
    with open(files[0]) as fh:
        return list(csv.DictReader(fh))


def dispatches(rows):
    """Dispatch_Id -> {name, start, end, counters} in dispatch order."""
    out = {}
    for r in rows:
        d = out.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "start": int(r["Start_Timestamp"]),
                                                   "end": int(r["End_Timestamp"]), "counters": {}})
        if "Counter_Name" in r:
            d["counters"][r["Counter_Name"]] = d["counters"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [out[k] for k in sorted(out)]


def match(bench, disp, steps):
    """bench name -> list (one entry per timed call) of lists of dispatches."""
    kern = bench["kernels"]
    step_names = [k for k, v in kern.items() if not v.get("outside_step")]
    extra_names = [k for k, v in kern.items() if v.get("outside_step") and k != COPY]
    fp8q = [d for d in disp if "fp8q::" in d["name"]]
    # the warm-up count is not needed: step calls come first, so the number of
    # step rounds is what remains after the outside-step calls
    warm = {n for n in extra_names if "warm" in kern[n]}     # these also ran `steps` calls back to back
    n_extra = sum(2 + steps + (steps if n in warm else 0) for n in extra_names)
    calls = []          # consecutive calls, each a list of dispatches
    i = 0
    while i < len(fp8q):
        c = [fp8q[i]]
        i += 1
        while i < len(fp8q) and continues_call(c, fp8q[i]["name"]):
            c.append(fp8q[i])
            i += 1
        calls.append(c)
    n_step_calls = len(calls) - n_extra
    if n_step_calls <= 0 or n_step_calls % len(step_names):
        raise ValueError(f"{len(calls)} calls do not split into step rounds of {len(step_names)} "
                         f"plus {n_extra} outside-step calls")
    rounds = n_step_calls // len(step_names)
    if rounds < steps:
        raise ValueError(f"only {rounds} step rounds for --steps {steps}")
    seq = [n for _ in range(rounds) for n in step_names]
    for n in extra_names:
        seq += [n] * (2 + steps) + [(n, "warm")] * (steps if n in warm else 0)
    timed = {}
    for pos, (n, c) in enumerate(zip(seq, calls)):
        base = n[0] if isinstance(n, tuple) else n
        if not any(f in c[0]["name"] for f in family(base)):
            raise ValueError(f"call {pos} ({base}) matched dispatch {c[0]['name'][:80]}")
        if n == base:                   # the warm calls are matched but not summarised: the cold ones are timed
            timed.setdefault(n, []).append(c)
    for n in timed:
        timed[n] = timed[n][-steps:]
    copies = [d for d in disp if "copy" in d["name"].lower()]
    if copies:
        big = max(d["end"] - d["start"] for d in copies)
        timed[COPY] = [[d] for d in copies if d["end"] - d["start"] > big / 4][-5:]
    return timed, list(kern)


def dur_us(call):
    return sum(d["end"] - d["start"] for d in call) / 1e3


def cmd_trace(a):
    bench = read_bench(a.bench)
    disp = dispatches(read_csv(a.trace_dir, "kernel_trace"))
    timed, order = match(bench, disp, a.steps)
    stats = read_csv(a.trace_dir, "kernel_stats")
    durs = {}
    for d in disp:
        durs.setdefault(d["name"], []).append((d["end"] - d["start"]) / 1e3)
    print("| kernel | calls | avg us | median us | min us | max us | share |")
    print("|---|---|---|---|---|---|---|")
    for r in stats:
        name = r["Name"] if len(r["Name"]) <= 110 else r["Name"][:107] + "..."
        med = statistics.median(durs.get(r["Name"], [0.0]))
        print(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {med:.1f} | "
              f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    print()
    print(f"Per bench call (mean over the {a.steps} timed calls; a call's grids summed), "
          "beside the bench's own HIP-event time from its JSON line:")
    print()
    print("| bench kernel | grids per call | rocprofv3 us | HIP events us (bench line) |")
    print("|---|---|---|---|")
    for n in order:
        if n not in timed:
            continue
        cs = timed[n]
        us = statistics.mean(dur_us(c) for c in cs)
        print(f"| {n} | {len(cs[0])} | {us:.1f} | {bench['kernels'][n]['us']:.1f} |")


def compute_traffic(bench, fetch_rows, write_rows, clock_rows, steps, source_hash):
    """hbm_traffic.json content from the three counter runs' counter_collection rows."""
    runs = {}
    for key, rows in (("FETCH_SIZE", fetch_rows), ("WRITE_SIZE", write_rows), ("clock", clock_rows)):
        runs[key] = match(bench, dispatches(rows), steps)
    order = runs["FETCH_SIZE"][1]
    cal = {}
    for key in ("FETCH_SIZE", "WRITE_SIZE"):
        kib = statistics.median(c[0]["counters"][key] for c in runs[key][0][COPY])
        cal[key] = {"copy_1GiB_counter_KiB": kib, "scale": (1 << 30) / (kib * 1024)}
    per = {}
    for key in ("FETCH_SIZE", "WRITE_SIZE"):
        timed = runs[key][0]
        per[key] = {n: statistics.mean(sum(d["counters"][key] for d in c) for c in timed[n]) * 1024
                    * cal[key]["scale"] for n in order if n in timed and n != COPY}
    clock = {}
    for n, cs in runs["clock"][0].items():
        if not n.startswith("gemm"):
            continue
        cyc = sum(d["counters"]["GRBM_GUI_ACTIVE"] for c in cs for d in c)
        ns = sum(d["end"] - d["start"] for c in cs for d in c)
        clock[n] = round(cyc / (XCDS * ns), 3)
    cmd = "rocprofv3 --pmc {} -d <dir> --output-format csv -- python3 -u bench.py --steps %d --warmup 1 " \
          "--no-cpu-baseline" % steps
    return {
        "source_hash": source_hash,
        "command": cmd.format("FETCH_SIZE (then WRITE_SIZE)"),
        "calibration": cal,
        "fetch_bytes": per["FETCH_SIZE"],
        "write_bytes": per["WRITE_SIZE"],
        "kernels": {n: per["FETCH_SIZE"][n] + per["WRITE_SIZE"][n] for n in per["FETCH_SIZE"]},
        "clock_command": cmd.format("GRBM_GUI_ACTIVE GRBM_COUNT"),
        "clock_ghz": clock,
    }


def cmd_traffic(a):
    sys.path.insert(0, ROOT)
    from bench import source_hash
    bench = read_bench(a.bench)
    out = compute_traffic(bench, read_csv(a.fetch_dir, "counter_collection"),
                          read_csv(a.write_dir, "counter_collection"), read_csv(a.clock_dir, "counter_collection"),
                          a.steps, source_hash())
    cal, clock = out["calibration"], out["clock_ghz"]
    per = {"FETCH_SIZE": out["fetch_bytes"], "WRITE_SIZE": out["write_bytes"]}
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    print(f"Calibration on the 1 GiB device copy (1,073,741,824 bytes read and written): FETCH_SIZE reads "
          f"{cal['FETCH_SIZE']['copy_1GiB_counter_KiB']:.1f} KiB (scale {cal['FETCH_SIZE']['scale']:.4f}), "
          f"WRITE_SIZE reads {cal['WRITE_SIZE']['copy_1GiB_counter_KiB']:.1f} KiB "
          f"(scale {cal['WRITE_SIZE']['scale']:.4f}).")
    print()
    print("| kernel (bench name) | fetched MB | written MB | total MB | algorithmic MB |")
    print("|---|---|---|---|---|")
    for n in per["FETCH_SIZE"]:
        k = bench["kernels"][n]
        alg = k.get("bytes")
        alg_s = f"{alg / 1e6:.1f}" if alg else "-"
        f, w = per["FETCH_SIZE"][n], per["WRITE_SIZE"][n]
        print(f"| {n} | {f / 1e6:.1f} | {w / 1e6:.1f} | {(f + w) / 1e6:.1f} | {alg_s} |")
    print()
    print("| GEMM | average shader clock GHz |")
    print("|---|---|")
    for n, g in clock.items():
        print(f"| {n} | {g:.2f} |")
    print()
    print(f"Kernel sources hash: `{out['source_hash']}`")


def compute_counters(bench, mfma_rows, wait_rows, steps, source_hash):
    """gemm_counters.json content: per GEMM bench call, the counters summed over its grids and averaged over
    the timed calls, and the derived utilisation figures."""
    runs = {"mfma": match(bench, dispatches(mfma_rows), steps)[0],
            "wait": match(bench, dispatches(wait_rows), steps)[0]}
    out = {}
    for n, calls in runs["mfma"].items():
        if not n.startswith("gemm"):
            continue
        c = {}
        for key, passes in (("mfma", MFMA_PASS), ("wait", WAIT_PASS)):
            for name in passes:
                vals = [sum(d["counters"].get(name, 0.0) for d in call) for call in runs[key][n]]
                c[f"{name}@{key}"] = statistics.mean(vals)
        gui_m, gui_w = c["GRBM_GUI_ACTIVE@mfma"], c["GRBM_GUI_ACTIVE@wait"]
        simd_cycles = SIMDS * gui_m / XCDS
        mfma = c["SQ_INSTS_MFMA@mfma"]
        valu_other = c["SQ_INSTS_VALU@mfma"] - mfma
        wave = c["SQ_WAVE_CYCLES@wait"]
        us = statistics.mean(dur_us(call) for call in runs["mfma"][n])
        flop = bench["kernels"][n].get("flop")
        out[n] = {
            "counters": {k: round(v, 1) for k, v in c.items()},
            "dispatch_us_under_counters": round(us, 1),
            "clock_ghz": round(gui_m / (XCDS * us * 1e3), 3),
            "mfma_busy": round(c["SQ_VALU_MFMA_BUSY_CYCLES@mfma"] / simd_cycles, 4),
            "mfma_f8_flop": c["SQ_INSTS_VALU_MFMA_MOPS_F8@mfma"] * 512,
            "algorithmic_flop": flop,
            "valu_insts_per_mfma": round(valu_other / mfma, 3) if mfma else None,
            "valu_busy_est": round(4 * valu_other / simd_cycles, 4),
            "coexec_of_mfma_busy": round(c["SQ_VALU_MFMA_COEXEC_CYCLES@mfma"] / c["SQ_VALU_MFMA_BUSY_CYCLES@mfma"], 4)
            if c["SQ_VALU_MFMA_BUSY_CYCLES@mfma"] else None,
            "lds_bank_conflict_cycles": c["SQ_LDS_BANK_CONFLICT@mfma"],
            "lds_insts_per_mfma": round(c["SQ_INSTS_LDS@mfma"] / mfma, 3) if mfma else None,
            "wave_issuing": round(c["SQ_ACTIVE_INST_ANY@wait"] / wave, 4) if wave else None,
            "wave_waiting_on_counters": round(c["SQ_WAIT_ANY@wait"] / wave, 4) if wave else None,
            "wave_waiting_to_issue": round(c["SQ_WAIT_INST_ANY@wait"] / wave, 4) if wave else None,
            "clock_ghz_wait_pass": round(gui_w / (XCDS * statistics.mean(dur_us(call) for call in runs["wait"][n])
                                                  * 1e3), 3),
        }
    cmd = "rocprofv3 --pmc {} -d <dir> --output-format csv -- python3 -u bench.py --steps %d --warmup 1 " \
          "--no-cpu-baseline" % steps
    return {"source_hash": source_hash, "mfma_command": cmd.format(" ".join(MFMA_PASS)),
            "wait_command": cmd.format(" ".join(WAIT_PASS)), "gemms": out}


def cmd_counters(a):
    sys.path.insert(0, ROOT)
    from bench import source_hash
    bench = read_bench(a.bench)
    out = compute_counters(bench, read_csv(a.mfma_dir, "counter_collection"),
                           read_csv(a.wait_dir, "counter_collection"), a.steps, source_hash())
    with open(os.path.join(ROOT, "profiles", "gemm_counters.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    print("| GEMM | us (under counters) | clock GHz | MFMA busy | VALU instr. / MFMA | VALU busy (est.) | "
          "co-issued with MFMA | LDS bank-conflict cycles | LDS instr. / MFMA | wave issuing / waiting on "
          "counters / waiting to issue |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for n, g in out["gemms"].items():
        print(f"| {n} | {g['dispatch_us_under_counters']:.1f} | {g['clock_ghz']:.2f} | {g['mfma_busy']:.3f} | "
              f"{g['valu_insts_per_mfma']:.2f} | {g['valu_busy_est']:.3f} | {g['coexec_of_mfma_busy']:.3f} | "
              f"{g['lds_bank_conflict_cycles']:.0f} | {g['lds_insts_per_mfma']:.2f} | "
              f"{g['wave_issuing']:.2f} / {g['wave_waiting_on_counters']:.2f} / {g['wave_waiting_to_issue']:.2f} |")
    print()
    print(f"Kernel sources hash: `{out['source_hash']}`")


def main():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = p.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("bench")
    t.add_argument("trace_dir")
    t.add_argument("--steps", type=int, required=True)
    f = sub.add_parser("traffic")
    f.add_argument("bench")
    f.add_argument("fetch_dir")
    f.add_argument("write_dir")
    f.add_argument("clock_dir")
    f.add_argument("--steps", type=int, required=True)
    c = sub.add_parser("counters")
    c.add_argument("bench")
    c.add_argument("mfma_dir")
    c.add_argument("wait_dir")
    c.add_argument("--steps", type=int, required=True)
    a = p.parse_args()
    {"trace": cmd_trace, "traffic": cmd_traffic, "counters": cmd_counters}[a.cmd](a)


if __name__ == "__main__":
    main()
