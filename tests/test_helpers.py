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


def test_cancellation_moves_tiny_results_by_several_ulps():
    """Why the one-ulp check skips results far below the array's magnitude:
    summing in float32 in index order (the kernel's specified arithmetic)
    next to a cancellation legitimately lands several bf16 ulps from the
    correctly rounded exact sum, at ~1e-8 absolute."""
    import numpy as np
    from oracle import twnorm_oracle as O
    terms = [-1.1875, 0.8828125, -1.555308699607849e-07, 0.3046875]   # bf16-exact values
    for t in terms:
        assert O.bf16_decode(O.bf16_encode_rne(np.array([t])))[0] == t
    s32 = np.float32(0.0)
    for t in terms:
        s32 = np.float32(s32 + np.float32(t))
    exact = sum(terms)
    ulps = bf16_ulp_distance(O.bf16_encode_rne(np.array([float(s32)])),
                             O.bf16_encode_rne(np.array([exact])))[0]
    assert ulps == 7
    assert abs(float(s32) - exact) < 1e-8
