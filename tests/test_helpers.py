"""CPU checks of the GPU tests' comparison helpers."""
import numpy as np

from gpu_helpers import bf16_ulp_distance, tolerance_report


def test_ulp_helper_pins():
    """The ulp distance used above counts representable steps across zero."""
    a = np.array([0x3F80, 0x3F80, 0x0000, 0x8000, 0x8001], np.uint16)
    b = np.array([0x3F80, 0x3F81, 0x8000, 0x0001, 0x0001], np.uint16)
    assert bf16_ulp_distance(a, b).tolist() == [0, 1, 0, 1, 2]


def test_tolerance_reading():
    """bf16 passes iff |d| <= max(2e-2, 1e-2 |ref|); fp32 iff |d| <= 1e-5 max(1, |ref|)."""
    from oracle import twnorm_oracle as O
    ref = np.array([0.0, 0.5, 8.5, -100.0])
    ok = O.bf16_encode_rne(ref + np.array([0.019, -0.019, 0.08, 0.9]))
    assert tolerance_report(ok, ref, "bf16")["fails"] == 0
    bad = O.bf16_encode_rne(ref + np.array([0.03, 0.0, 0.0, 0.0]))
    assert tolerance_report(bad, ref, "bf16")["fails"] == 1
    f = np.array([1e-6, 2.0], np.float32)
    assert tolerance_report(f, np.array([0.0, 2.0 + 1.9e-5]), "f32")["fails"] == 0
    assert tolerance_report(f, np.array([2e-5, 2.0]), "f32")["fails"] == 1
