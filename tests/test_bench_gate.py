"""The benchmark's parity gate (CPU, no GPU): a correct product passes, and a
result corrupted on the host (one sign flipped, one NaN, one inf, one element
off by more than the bound) is counted, so bench.py prints the failure record,
with no value and no throughput, instead of a measurement."""
import numpy as np

import bench
import oracle
from shape_driven_tile_amd import inputs


def _case():
    A = inputs.uniform_f16((64, 96), 501)
    B = inputs.uniform_f16((40, 96), 502)
    ref = oracle.gemm(A, B)
    # what a correct kernel returns: the exact sum rounded once to fp16
    good = ref.astype(np.float16)
    return ref, good


def test_correct_result_passes():
    ref, good = _case()
    assert bench.outside_tolerance(good, ref) == 0
    assert bench.gate_failure({"gemm_64_full": 0, "rows_checked": 64}) is None


def test_corrupted_results_fail():
    ref, good = _case()
    for corrupt in ("sign", "nan", "inf", "offset"):
        bad = good.copy()
        if corrupt == "sign":
            i = np.unravel_index(np.argmax(np.abs(ref)), ref.shape)   # |ref| well above the bound
            bad[i] = -bad[i]
        elif corrupt == "nan":
            bad[3, 5] = np.nan
        elif corrupt == "inf":
            bad[7, 1] = np.inf
        else:
            bad[10, 10] = np.float16(ref[10, 10] + 2 * oracle.tolerance(ref[10, 10]))
        assert bench.outside_tolerance(bad, ref) == 1, corrupt
        record = bench.gate_failure({"gemm_64_full": 1, "gemm_64_rows_checked": 64})
        assert record["value"] is None and record["error"] == "parity gate failed"
        assert "roofline" not in record and "ms_per_step" not in record


def test_rows_checked_counts_are_not_failures():
    assert bench.gate_failure({"gemm_8192_rows": 0, "gemm_8192_rows_checked": 7000}) is None
    assert bench.gate_failure({"gemv_8_buffers": 3})["gate"]["gemv_8_buffers"] == 3


def test_bf16_bound_is_the_wider_one():
    ref = np.array([100.0, -3.0, 0.0])
    # half a bf16 ulp at 100 is 0.25: outside the fp16 bound, inside the bf16 one
    got = ref + np.array([0.25, 0.0, 0.0])
    assert bench.outside_tolerance(got, ref, "f16") == 1
    assert bench.outside_tolerance(got, ref, "bf16") == 0
