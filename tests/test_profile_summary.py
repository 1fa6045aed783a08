"""Host logic of profile_summary.py: matching bench calls to rocprofv3 dispatches
and calibrating the HBM counters (synthetic counter rows, no GPU)."""

import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import profile_summary as ps  # noqa: E402

DUAL = "void fp8q::quant_dual_kernel<unsigned short, 0>(unsigned short const*, long)"
GEMM_A = "void fp8q::gemm_blockscaled_kernel<256, 256, 4, 2, 0, 0, false, 0>(fp8q::GemmArgs)"
GEMM_B = "void fp8q::gemm_blockscaled_kernel<128, 256, 2, 4, 0, 0, false, 0>(fp8q::GemmArgs)"
Q1 = "void fp8q::quant_1x128_kernel<unsigned short, 1>(unsigned short const*, long)"
REDUCE = "void at::native::reduce_kernel<512, 1>(...)"
COPY = "__amd_rocclr_copyBuffer"

BENCH = {"kernels": {
    "quant 1x128+128x1 X": {"us": 50.0},
    "gemm Dgrad": {"us": 900.0},
    "quant_1x128 X (pow2 scales)": {"us": 30.0, "outside_step": True, "warm": {"us": 28.0}},
    ps.COPY: {"us": 400.0, "outside_step": True},
}}
# the same with an outside-step GEMM after the warm quantizer calls
P2_NAME = "gemm Fprop (pow2 operands, hardware-scaled MFMA)"
BENCH_P2 = {"kernels": {**{k: v for k, v in BENCH["kernels"].items() if k != ps.COPY},
                        P2_NAME: {"us": 850.0, "outside_step": True}, ps.COPY: {"us": 400.0, "outside_step": True}}}
GEMM_P2 = "void fp8q::gemm_blockscaled_kernel<256, 256, 4, 2, 0, 0, false, 3>(fp8q::GemmArgs)"


def _rows(steps, warmup, counter, p2_gemm=False):
    """Dispatch rows as the bench would launch them; each call's counter value encodes
    (kind, call index) so that the expected means are known."""
    rows, t = [], 0
    did = [0]

    def add(name, value, dur=1000):
        nonlocal t
        did[0] += 1
        rows.append({"Dispatch_Id": str(did[0]), "Kernel_Name": name, "Start_Timestamp": str(t),
                     "End_Timestamp": str(t + dur), "Counter_Name": counter, "Counter_Value": str(value)})
        t += dur + 10

    add(COPY, 1.0, dur=5)                     # an early small copy (input upload)
    for s in range(warmup + steps):
        add(DUAL, 100 + s)
        add(GEMM_A, 1000 + s, dur=8000)
        add(GEMM_B, 10, dur=2000)             # second grid of the same Dgrad call
    for c in range(2 + steps):
        add(REDUCE, 0.0)                      # the cache scrub between timed calls
        add(Q1, 50 + c)
    for c in range(steps):
        add(Q1, 90 + c)                       # the same quantizer back to back (warm)
    for c in range(2 + steps if p2_gemm else 0):
        add(REDUCE, 0.0)
        add(GEMM_P2, 70 + c, dur=8000)
    for c in range(3 + 5):
        add(COPY, 524288.0 if counter == "FETCH_SIZE" else 1048576.0, dur=400000)
    return rows


def test_match_pairs_split_grids_and_keeps_the_timed_calls():
    steps, warmup = 2, 1
    timed, order = ps.match(BENCH, ps.dispatches(_rows(steps, warmup, "FETCH_SIZE")), steps)
    assert order == list(BENCH["kernels"])
    assert [len(c) for c in timed["gemm Dgrad"]] == [2, 2]
    assert [c[0]["counters"]["FETCH_SIZE"] for c in timed["gemm Dgrad"]] == [1001, 1002]
    assert [c[0]["counters"]["FETCH_SIZE"] for c in timed["quant 1x128+128x1 X"]] == [101, 102]
    assert [c[0]["counters"]["FETCH_SIZE"] for c in timed["quant_1x128 X (pow2 scales)"]] == [52, 53]   # cold
    assert len(timed[ps.COPY]) == 5 and all(len(c) == 1 for c in timed[ps.COPY])
    # an outside-step call after the warm ones is still matched to its own dispatches
    timed, _ = ps.match(BENCH_P2, ps.dispatches(_rows(steps, warmup, "FETCH_SIZE", p2_gemm=True)), steps)
    assert [c[0]["counters"]["FETCH_SIZE"] for c in timed[P2_NAME]] == [72, 73]
    assert [c[0]["counters"]["FETCH_SIZE"] for c in timed["quant_1x128 X (pow2 scales)"]] == [52, 53]
    assert len(timed[ps.COPY]) == 5 and all(len(c) == 1 for c in timed[ps.COPY])


def test_match_rejects_a_sequence_of_the_wrong_kind():
    rows = _rows(2, 1, "FETCH_SIZE")
    for r in rows:
        if r["Kernel_Name"] == Q1:
            r["Kernel_Name"] = DUAL
    with pytest.raises(ValueError):
        ps.match(BENCH, ps.dispatches(rows), 2)


def test_traffic_is_calibrated_on_the_copy_and_sums_the_grids():
    steps, warmup = 2, 1
    fetch = _rows(steps, warmup, "FETCH_SIZE")
    write = _rows(steps, warmup, "WRITE_SIZE")
    clock = _rows(steps, warmup, "GRBM_GUI_ACTIVE")
    out = ps.compute_traffic(BENCH, fetch, write, clock, steps, "hash")
    # the copy moves 1 GiB each way; FETCH_SIZE read half of it -> scale 2
    assert out["calibration"]["FETCH_SIZE"]["scale"] == pytest.approx(2.0)
    assert out["calibration"]["WRITE_SIZE"]["scale"] == pytest.approx(1.0)
    # Dgrad: mean of (1001 + 10) and (1002 + 10) KiB, times 1024 and the scale
    assert out["fetch_bytes"]["gemm Dgrad"] == pytest.approx(1011.5 * 1024 * 2.0)
    assert out["write_bytes"]["gemm Dgrad"] == pytest.approx(1011.5 * 1024 * 1.0)
    assert out["kernels"]["gemm Dgrad"] == pytest.approx(1011.5 * 1024 * 3.0)
    assert ps.COPY not in out["kernels"]
    # clock: cycles over 8 XCDs x ns, both grids of both timed calls
    assert out["clock_ghz"]["gemm Dgrad"] == pytest.approx(round((1001 + 10 + 1002 + 10) / (8 * 20000), 3))
    assert set(out["clock_ghz"]) == {"gemm Dgrad"}
    assert out["source_hash"] == "hash"


def _multi_rows(steps, warmup, values):
    """Dispatch rows carrying several counters per dispatch: values[name] for the GEMM's first grid (its second
    grid carries a tenth of each)."""
    rows = []
    for r in _rows(steps, warmup, "GRBM_GUI_ACTIVE"):
        for name, v in values.items():
            rr = dict(r, Counter_Name=name)
            if r["Kernel_Name"] == GEMM_A:
                rr["Counter_Value"] = str(v)
            elif r["Kernel_Name"] == GEMM_B:
                rr["Counter_Value"] = str(v / 10)
            else:
                rr["Counter_Value"] = "1.0"
            rows.append(rr)
    return rows


def test_counters_derive_mfma_busy_and_wait_split():
    steps, warmup = 2, 1
    # per dispatch of the first grid: 8000 ns at GUI 8*16000 cycles = 2 GHz; 1000 MFMAs busy 32 cycles each
    mfma = {"GRBM_GUI_ACTIVE": 128000.0, "SQ_VALU_MFMA_BUSY_CYCLES": 32000.0, "SQ_INSTS_VALU_MFMA_MOPS_F8": 128000.0,
            "SQ_INSTS_VALU": 6000.0, "SQ_INSTS_MFMA": 1000.0, "SQ_VALU_MFMA_COEXEC_CYCLES": 16000.0,
            "SQ_LDS_BANK_CONFLICT": 0.0, "SQ_INSTS_LDS": 750.0, "SQ_WAVE_CYCLES": 100.0}
    wait = {"GRBM_GUI_ACTIVE": 128000.0, "SQ_WAVE_CYCLES": 100.0, "SQ_WAIT_ANY": 30.0, "SQ_WAIT_INST_ANY": 40.0,
            "SQ_ACTIVE_INST_ANY": 30.0, "SQ_LDS_IDX_ACTIVE": 1.0, "SQ_INSTS_SALU": 1.0, "SQ_BUSY_CYCLES": 1.0,
            "SQ_INSTS_SMEM": 1.0}
    bench = {"kernels": dict(BENCH["kernels"])}
    bench["kernels"]["gemm Dgrad"] = {"us": 900.0, "flop": 1.0}
    out = ps.compute_counters(bench, _multi_rows(steps, warmup, mfma), _multi_rows(steps, warmup, wait), steps, "h")
    g = out["gemms"]["gemm Dgrad"]
    # the two grids of a call are summed: counters x 1.1, duration 8000 + 2000 ns
    assert g["counters"]["SQ_VALU_MFMA_BUSY_CYCLES@mfma"] == pytest.approx(35200.0)
    assert g["mfma_busy"] == pytest.approx(35200.0 / (ps.SIMDS * 140800.0 / 8), abs=1e-4)
    assert g["clock_ghz"] == pytest.approx(140800.0 / (8 * 10000.0), abs=1e-3)
    assert g["mfma_f8_flop"] == pytest.approx(140800.0 * 512)
    assert g["valu_insts_per_mfma"] == pytest.approx(5.0)
    assert g["coexec_of_mfma_busy"] == pytest.approx(0.5)
    assert g["lds_insts_per_mfma"] == pytest.approx(0.75)
    assert (g["wave_issuing"], g["wave_waiting_on_counters"], g["wave_waiting_to_issue"]) == \
        pytest.approx((0.3, 0.3, 0.4))
    assert set(out["gemms"]) == {"gemm Dgrad"}


KSPLIT = "void fp8q::gemm_blockscaled_kernel<256, 256, 4, 2, 0, 1, false, 0, 2>(fp8q::GemmArgs)"
KSUM = "fp8q::(anonymous namespace)::ksplit_sum_bf16_kernel(float const*, long, long, unsigned short*, long, long, long)"


def test_a_ksplit_gemm_call_is_one_call_of_three_dispatches():
    """A BF16 GEMM whose last wave runs with K split in two launches the split grid, the kernel that adds the
    halves and the grid of the other columns: matched as one call, its three durations summed."""
    bench = {"kernels": {"quant 1x128+128x1 X": {"us": 50.0}, "gemm Dgrad": {"us": 900.0},
                         ps.COPY: {"us": 400.0, "outside_step": True}}}
    rows, t = [], 0
    did = [0]

    def add(name, dur):
        nonlocal t
        did[0] += 1
        rows.append({"Dispatch_Id": str(did[0]), "Kernel_Name": name, "Start_Timestamp": str(t),
                     "End_Timestamp": str(t + dur)})
        t += dur + 10

    for _ in range(3):                       # warm-up 1 + 2 timed steps
        add(DUAL, 1000)
        add(KSPLIT, 100000)
        add(KSUM, 15000)
        add(GEMM_A, 700000)
    for _ in range(8):
        add(COPY, 400000)
    timed, _ = ps.match(bench, ps.dispatches(rows), 2)
    assert [len(c) for c in timed["gemm Dgrad"]] == [3, 3]
    assert ps.dur_us(timed["gemm Dgrad"][0]) == pytest.approx(815.0)
    assert [len(c) for c in timed["quant 1x128+128x1 X"]] == [1, 1]
    # the pieces only continue a GEMM call, in their order
    one = [{"name": GEMM_A}]
    assert ps.continues_call([{"name": KSPLIT}], KSUM)
    assert ps.continues_call([{"name": KSPLIT}, {"name": KSUM}], GEMM_A)
    assert not ps.continues_call(one, GEMM_A) and not ps.continues_call([{"name": DUAL}], KSUM)
    assert not ps.continues_call([{"name": KSPLIT}, {"name": KSUM}, {"name": GEMM_A}], KSUM)
