"""HBM traffic per kernel launch from rocprofv3 counter runs.

Two counter passes (FETCH_SIZE, then WRITE_SIZE, each in KiB per dispatch)
over the benchmark, and the same two passes over a plain copy kernel of known
size, give calibrated bytes per launch:

    traffic = FETCH_SIZE * (copy bytes read / copy FETCH_SIZE)
            + WRITE_SIZE * (copy bytes written / copy WRITE_SIZE)

FETCH_SIZE weighs memory requests by an assumed size, so the factor depends
on the request mix: the calibration copy (libbdmcal.so) reads with the same
16-byte non-temporal wave-contiguous loads as the weight-streaming kernels.
A torch elementwise copy (ordinary loads) is measured beside it and its
factor is reported for comparison only.

    python -m block_diffusion_moe_amd.traffic copy
        the two copies (1 GiB read + 1 GiB written each), run under
        `rocprofv3 --pmc FETCH_SIZE` and `--pmc WRITE_SIZE` for the factors
    python -m block_diffusion_moe_amd.traffic summarize --fetch DIR --write DIR \\
        --cal-fetch DIR --cal-write DIR --out FILE [--command TEXT]
        writes a markdown summary with a per-kernel table; its first lines are
        `<!-- key = value -->` records (source digest, traffic of the head GEMM
        kernel) that bench.py reads back.
    python -m block_diffusion_moe_amd.traffic mfma --dir DIR --out FILE [--command TEXT]
        per-kernel matrix-core activity from one counter pass of
        SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16
        and GRBM_GUI_ACTIVE: MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES (summed over
        every SIMD) / (GRBM_GUI_ACTIVE / XCDs (it is summed over the XCDs) x
        CUs x 4 SIMDs); MFMA flop per launch = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512.
    python -m block_diffusion_moe_amd.traffic timeline --trace FILE --out FILE [--command TEXT]
        from a `rocprofv3 --kernel-trace` CSV of the benchmark: where the time
        of one denoise step, and of the MoE layer launched back to back, goes
        (median duration of each kernel in launch order and median idle gap
        before it, over every matching launch sequence).
    python -m block_diffusion_moe_amd.traffic stats --csv FILE --out FILE [--command TEXT]
        [--note TEXT]
        the `rocprofv3 --stats` kernel table (calls, mean, min and max
        duration of every kernel of this library and of the calibration
        library) as markdown.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30
# the head GEMM of the unmask step over one block (either kernel; not the
# verify epilogue's instance head_coop_kernel<KSW, MT, true, false> nor the
# many-row one head_coop_kernel<KSW, MT, false, true>)
HEAD_KERNELS = ("head_coop_kernel", "head_tile_kernel")
HEAD_SOURCES = ("head.hip", "device.hpp", "internal.hpp")
MOE_SOURCES = ("router.hip", "experts.hip", "device.hpp", "internal.hpp")
# the launches of the one-block MoE layer (32 tokens, 256 experts) and their
# grids in threads: router 16 x 1 x 4 workgroups of 256, top-k 8 of 256,
# grouping 1 of 1,024, gate/up and down (one-block kernels, used below 256
# tokens only), combine 32 of 256
MOE_LAYER_GRIDS = {"bdm::router_kernel<1, false>": 16384,
                   "bdm::select_kernel<4, 4, false, false>": 2048,
                   "bdm::group_kernel<4>": 1024, "bdm::gateup_kernel<8, false>": None,
                   "bdm::down_kernel<16, false>": None, "bdm::combine_kernel": 8192}


def kernel_source_digest(files=HEAD_SOURCES) -> str:
    """sha256 over the csrc files a kernel is compiled from."""
    d = hashlib.sha256()
    for f in files:
        with open(os.path.join(HERE, "csrc", f), "rb") as fh:
            d.update(fh.read())
    return d.hexdigest()


def copy_kernel():
    """Plain copies of COPY_BYTES, each launch reading COPY_BYTES and writing
    COPY_BYTES: the non-temporal stream copy of libbdmcal.so, then a torch
    elementwise copy (float32 negation into a second buffer)."""
    import ctypes

    import torch
    lib_path = os.path.join(HERE, "libbdmcal.so")
    if not os.path.exists(lib_path):
        raise SystemExit(f"{lib_path} is not built (python -m block_diffusion_moe_amd.build)")
    lib = ctypes.CDLL(lib_path)
    lib.bdmcal_stream_copy.restype = ctypes.c_int
    lib.bdmcal_stream_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_long,
                                       ctypes.c_void_p]
    dev = torch.device("cuda:0")
    n = COPY_BYTES // 4
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream().cuda_stream
    for _ in range(3):
        if lib.bdmcal_stream_copy(a.data_ptr(), b.data_ptr(), COPY_BYTES, st) != 0:
            raise SystemExit("bdmcal_stream_copy failed")
    torch.cuda.synchronize()
    if not torch.equal(a, b):
        raise SystemExit("bdmcal_stream_copy: copy mismatch")
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    print(f"copy done: 3 + 3 launches of {COPY_BYTES} B read + {COPY_BYTES} B written",
          flush=True)


def read_counters(d: str, by_grid: bool = False):
    """{(kernel short name, counter): [value per dispatch]} from one pass; with
    `by_grid` the key is (name, grid size, counter), which tells apart calls
    of one kernel at different sizes (e.g. 256 against 2,048 tokens)."""
    agg = collections.defaultdict(list)
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"].replace("(anonymous namespace)::", "")
                name = name.split("(")[0].replace("void ", "").strip()
                key = (name, int(r.get("Grid_Size") or 0)) if by_grid else name
                agg[(key, r["Counter_Name"])].append(float(r["Counter_Value"]))
    return agg


def _copy_factor(agg, counter: str, kernel: str = "stream_copy_kernel") -> float:
    vals = [v for (n, c), vs in agg.items() if c == counter and kernel in n for v in vs]
    if not vals:
        raise SystemExit(f"no copy-kernel dispatches with {counter} found")
    mean_kib = sum(vals) / len(vals)
    return COPY_BYTES / (mean_kib * 1024.0)


def summarize(a):
    fetch, write = read_counters(a.fetch, True), read_counters(a.write, True)
    cal_f, cal_w = read_counters(a.cal_fetch), read_counters(a.cal_write)
    f_fac = _copy_factor(cal_f, "FETCH_SIZE")
    w_fac = _copy_factor(cal_w, "WRITE_SIZE")
    f_ew = _copy_factor(cal_f, "FETCH_SIZE", "neg_kernel")
    w_ew = _copy_factor(cal_w, "WRITE_SIZE", "neg_kernel")
    keys = sorted({k for k, _ in fetch} | {k for k, _ in write})
    rows = []
    head_bytes = None
    for key in keys:
        n, grid = key
        fv = fetch.get((key, "FETCH_SIZE"), [])
        wv = write.get((key, "WRITE_SIZE"), [])
        if not fv or not wv or "bdm" not in n:
            continue
        fb = f_fac * 1024.0 * sum(fv) / len(fv)
        wb = w_fac * 1024.0 * sum(wv) / len(wv)
        rows.append((n, grid, len(fv), fb, wb))
        short = n.split("::")[-1]
        other_variant = short.startswith("head_coop_kernel<") and "true" in short
        if short.startswith(HEAD_KERNELS) and not other_variant:
            head_bytes = fb + wb if head_bytes is None else max(head_bytes, fb + wb)
    # the one-block MoE layer: its kernels at their one-block grids
    layer = {}
    for n, grid, c, fb, wb in rows:
        want = MOE_LAYER_GRIDS.get(n, -1)
        if want == -1 or (want is not None and grid != want):
            continue
        layer[n] = max(layer.get(n, 0.0), fb + wb)
    out = [f"<!-- source_sha256 = {kernel_source_digest()} -->"]
    if head_bytes is not None:
        out.append(f"<!-- traffic_bytes = {head_bytes:.0f} -->")
    if len(layer) == len(MOE_LAYER_GRIDS):
        out.append(f"<!-- moe_source_sha256 = {kernel_source_digest(MOE_SOURCES)} -->")
        out.append(f"<!-- moe_layer_traffic_bytes = {sum(layer.values()):.0f} -->")
    out += ["", "# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE, calibrated)", ""]
    if a.command:
        out += ["Made by:", "", "```", a.command, "```", ""]
    out += [f"Calibration (plain copy of {COPY_BYTES} B read + written, 16 B non-temporal "
            f"loads as in the weight streams): FETCH_SIZE x {f_fac:.4f}, WRITE_SIZE x "
            f"{w_fac:.4f}.  For comparison, a torch elementwise copy (ordinary loads) reads "
            f"FETCH_SIZE x {f_ew:.4f}, WRITE_SIZE x {w_ew:.4f}.", "",
            "One row per kernel and launch grid (threads): calls of one kernel at "
            "different sizes are told apart by their grids.", "",
            "| kernel | grid | dispatches | read B / launch | written B / launch | "
            "total B / launch |",
            "|---|---:|---:|---:|---:|---:|"]
    for n, grid, c, fb, wb in rows:
        out.append(f"| `{n}` | {grid} | {c} | {fb:.4g} | {wb:.4g} | {fb + wb:.4g} |")
    out.append("")
    with open(a.out, "w") as fh:
        fh.write("\n".join(out))
    print("\n".join(out))


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                 "GRBM_GUI_ACTIVE")


def mfma(a):
    agg = read_counters(a.dir)
    names = sorted({n for n, _ in agg if "bdm" in n})
    out = ["# Matrix-core (MFMA) activity per kernel (rocprofv3 counters)", ""]
    if a.command:
        out += ["Made by:", "", "```", a.command, "```", ""]
    out += [f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {a.xcds} XCDs x {a.cus} "
            "CUs x 4 SIMDs) (both counters are sums over the chip: the busy cycles over every "
            "SIMD, GUI_ACTIVE over the XCDs); MFMA flop = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512.  "
            "Means per dispatch.", "",
            "| kernel | dispatches | GRBM_GUI_ACTIVE | SQ_BUSY_CYCLES | SQ_VALU_MFMA_BUSY_CYCLES "
            "| SQ_INSTS_VALU_MFMA_MOPS_BF16 | MFMA flop | MFMA busy |",
            "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for n in names:
        v = {c: agg.get((n, c), []) for c in MFMA_COUNTERS}
        if not all(v.values()):
            continue
        m = {c: sum(x) / len(x) for c, x in v.items()}
        cycles = m["GRBM_GUI_ACTIVE"] / a.xcds
        busy = m["SQ_VALU_MFMA_BUSY_CYCLES"] / max(1.0, cycles * a.cus * 4)
        out.append(f"| `{n}` | {len(v['GRBM_GUI_ACTIVE'])} | {m['GRBM_GUI_ACTIVE']:.4g} | "
                   f"{m['SQ_BUSY_CYCLES']:.4g} | {m['SQ_VALU_MFMA_BUSY_CYCLES']:.4g} | "
                   f"{m['SQ_INSTS_VALU_MFMA_MOPS_BF16']:.4g} | "
                   f"{512 * m['SQ_INSTS_VALU_MFMA_MOPS_BF16']:.4g} | {100 * busy:.2f}% |")
    out.append("")
    with open(a.out, "w") as fh:
        fh.write("\n".join(out))
    print("\n".join(out))


# launch sequences of the single-block path (kernel names without arguments)
MOE_SEQ = ("bdm::router_kernel<1, false>", "bdm::select_kernel<4, 4, false, false>",
           "bdm::group_kernel<4>", "bdm::gateup_kernel<8, false>", "bdm::down_kernel<16, false>",
           "bdm::combine_kernel")
STEP_SEQ = ("bdm::rmsnorm_kernel",) + MOE_SEQ + ("bdm::head_coop_kernel<8, 2, false, false>",
                                                   "bdm::head_merge_kernel")
# the layer with the block coreset selector over one 32-token block
CORESET_SEQ = ("bdm::router_kernel<1, false>", "bdm::select_kernel<4, 4, false, true>",
               "bdm::coreset_kernel<4, true>", "bdm::gateup_kernel<8, false>",
               "bdm::down_kernel<16, false>", "bdm::combine_kernel")
# many-token calls: 256 tokens (the load-skew batch; one-tile router) and
# 512 .. 2,048 tokens (multi-block batches; four-tile router)
SKEW_SEQ = ("bdm::router_kernel<1, false>", "bdm::select_kernel<4, 4, false, false>",
            "bdm::group_kernel<4>", "bdm::gateup_wide_kernel<8>", "bdm::down_wide_kernel<16>",
            "bdm::combine_kernel")
MULTI_SEQ = ("bdm::router_kernel<4, false>",) + SKEW_SEQ[1:]


def _kernel_name(n: str) -> str:
    n = n[5:] if n.startswith("void ") else n
    return n.split("(", 1)[0]


def read_trace(path: str):
    """(start ns, end ns, name, grid size) of every bdm kernel dispatch, in
    start order."""
    out = []
    with open(path, newline="") as fh:
        for r in csv.DictReader(fh):
            n = _kernel_name(r["Kernel_Name"])
            if n.startswith("bdm"):
                grid = int(r.get("Grid_Size_X") or r.get("Grid_Size") or 0)
                out.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), n, grid))
    out.sort()
    return out


def sequences(trace, seq, before=None, after=None):
    """Start indices where the dispatches are exactly `seq`; with `before` /
    `after`, also preceded / followed by a dispatch of that name."""
    names = [t[2] for t in trace]
    hits = []
    for i in range(len(names) - len(seq) + 1):
        if tuple(names[i:i + len(seq)]) != seq:
            continue
        if before is not None and (i == 0 or names[i - 1] != before):
            continue
        if after is not None and (i + len(seq) >= len(names) or names[i + len(seq)] != after):
            continue
        hits.append(i)
    return hits


def _median(v):
    v = sorted(v)
    n = len(v)
    return 0.0 if n == 0 else (v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2]))


def _table(trace, seq, hits, title):
    out = [f"## {title}", "", f"{len(hits)} launch sequences.", "",
           "| kernel | median µs | median gap before µs |", "|---|---:|---:|"]
    tot_d = tot_g = 0.0
    for j, n in enumerate(seq):
        d = _median([(trace[i + j][1] - trace[i + j][0]) / 1e3 for i in hits])
        g = _median([(trace[i + j][0] - trace[i + j - 1][1]) / 1e3 for i in hits]) if j else 0.0
        tot_d += d
        tot_g += g
        out.append(f"| `{n}` | {d:.2f} | {g:.2f} |" if j else f"| `{n}` | {d:.2f} | — |")
    span = _median([(trace[i + len(seq) - 1][1] - trace[i][0]) / 1e3 for i in hits])
    out += [f"| sum | {tot_d:.2f} | {tot_g:.2f} |", "",
            f"First start to last end: median {span:.2f} µs.", ""]
    return out


def timeline(a):
    trace = read_trace(a.trace)
    out = ["# Where the time goes: denoise step and MoE layer (rocprofv3 kernel trace)", ""]
    if a.command:
        out += ["Made by:", "", "```", a.command, "```", ""]
    out += ["Medians over every matching launch sequence in the trace; a gap is the idle "
            "time between the end of the previous dispatch and the start of this one.", ""]
    step = sequences(trace, STEP_SEQ)
    moe = sequences(trace, MOE_SEQ, before=MOE_SEQ[-1], after=MOE_SEQ[0])
    if step:
        out += _table(trace, STEP_SEQ, step, "Denoise step (eager, plain and graph replays)")
    if moe:
        out += _table(trace, MOE_SEQ, moe, "MoE layer launched back to back")
    cs = sequences(trace, CORESET_SEQ, before=CORESET_SEQ[-1], after=CORESET_SEQ[0])
    if cs:
        out += _table(trace, CORESET_SEQ, cs,
                      "MoE layer with the coreset selector (top_p 0.9), back to back")
    sk = sequences(trace, SKEW_SEQ, before=SKEW_SEQ[-1], after=SKEW_SEQ[0])
    if sk:
        out += _table(trace, SKEW_SEQ, sk,
                      "Load-skew batch (8 blocks, 256 tokens, log-Zipf offset), back to back")
    # the multi-block calls, one table per size (the combine's grid is one
    # workgroup per token)
    by_size = collections.defaultdict(list)
    for i in sequences(trace, MULTI_SEQ):
        by_size[trace[i + len(MULTI_SEQ) - 1][3] // 256].append(i)
    for T in sorted(by_size):
        hits = by_size[T]
        if len(hits) >= 4:                    # the timed loop (not the routing probes)
            out += _table(trace, MULTI_SEQ, hits,
                          f"Multi-block call, {T} tokens ({T // 32} blocks), back to back")
    with open(a.out, "w") as fh:
        fh.write("\n".join(out))
    print("\n".join(out))


def stats(a):
    rows = []
    with open(a.csv, newline="") as fh:
        for r in csv.DictReader(fh):
            n = r["Name"].replace("(anonymous namespace)::", "")
            n = (n[5:] if n.startswith("void ") else n).split("(", 1)[0]
            if not n.startswith("bdm"):
                continue
            rows.append((float(r["TotalDurationNs"]), n, int(r["Calls"]),
                         float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                         float(r["MaxNs"]) / 1e3))
    rows.sort(reverse=True)
    out = ["# rocprofv3 kernel statistics", ""]
    if a.note:
        out += [a.note, ""]
    if a.command:
        out += ["Command (run from the repository root on one MI355X):", "", "```", a.command,
                "```", ""]
    out += ["| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for _, n, calls, avg, mn, mx in rows:
        out.append(f"| {n} | {calls} | {avg:.2f} | {mn:.2f} | {mx:.2f} |")
    out.append("")
    with open(a.out, "w") as fh:
        fh.write("\n".join(out))
    print("\n".join(out))


def main(argv=None):
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="cmd", required=True)
    sub.add_parser("copy")
    s = sub.add_parser("summarize")
    for k in ("fetch", "write", "cal_fetch", "cal_write", "out"):
        s.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    s.add_argument("--command", default="")
    m = sub.add_parser("mfma")
    m.add_argument("--dir", required=True)
    m.add_argument("--out", required=True)
    m.add_argument("--cus", type=int, default=256)
    m.add_argument("--xcds", type=int, default=8)
    m.add_argument("--command", default="")
    t = sub.add_parser("timeline")
    t.add_argument("--trace", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--command", default="")
    k = sub.add_parser("stats")
    k.add_argument("--csv", required=True)
    k.add_argument("--out", required=True)
    k.add_argument("--command", default="")
    k.add_argument("--note", default="")
    a = p.parse_args(argv)
    if a.cmd == "copy":
        copy_kernel()
    elif a.cmd == "stats":
        stats(a)
    elif a.cmd == "mfma":
        mfma(a)
    elif a.cmd == "timeline":
        timeline(a)
    else:
        summarize(a)


if __name__ == "__main__":
    sys.exit(main())
