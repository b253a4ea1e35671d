"""The rocprofv3 digest tool (block_diffusion_moe_amd.traffic) on the CPU:
the kernel-trace timeline finds exactly the launch sequences of the denoise
step and of the back-to-back MoE layer in a synthetic trace, with their
durations and idle gaps."""
import csv

from block_diffusion_moe_amd import traffic as tr


def _trace(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for s, e, n in rows:
            w.writerow([n, s, e])


def test_timeline_sequences_and_gaps(tmp_path):
    rows, t = [], 0

    def add(name, dur, gap):
        nonlocal t
        t += gap
        rows.append((t, t + dur, f"void {name}(int const*, float*)"))
        t += dur

    add("at::native::fill_kernel", 100, 0)             # not ours: ignored
    for _ in range(3):                                  # three steps
        for j, n in enumerate(tr.STEP_SEQ):
            add(n, 4000 + 1000 * j, 700)
    for _ in range(5):                                  # five layers back to back
        for j, n in enumerate(tr.MOE_SEQ):
            add(n, 2000 + 500 * j, 300)
    add("bdm::rmsnorm_kernel", 3000, 300)
    trace_path = tmp_path / "run_kernel_trace.csv"
    _trace(trace_path, rows)
    trace = tr.read_trace(str(trace_path))
    assert len(trace) == 3 * len(tr.STEP_SEQ) + 5 * len(tr.MOE_SEQ) + 1
    assert tr.sequences(trace, tr.STEP_SEQ) == [0, 9, 18]
    # the first layer follows a head merge, the last is followed by RMSNorm
    moe = tr.sequences(trace, tr.MOE_SEQ, before=tr.MOE_SEQ[-1], after=tr.MOE_SEQ[0])
    assert moe == [27 + 6, 27 + 12, 27 + 18]
    out = tmp_path / "t.md"
    tr.main(["timeline", "--trace", str(trace_path), "--out", str(out)])
    text = out.read_text()
    assert "| `bdm::head_merge_kernel` | 12.00 | 0.70 |" in text
    assert "| `bdm::combine_kernel` | 4.50 | 0.30 |" in text
    # step: 9 kernels 4..12 us and 8 gaps of 0.7 us; layer: 6 kernels 2..4.5 us
    assert "median 77.60 µs" in text and "median 21.00 µs" in text
