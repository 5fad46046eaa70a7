"""Tolerances of the parity tests, in one place.

* integer, index and bit-copy data (plans, key/gate records, memory the call
  must not touch): bit-exact;
* FP32 values (FP32 state, corrections, decays): |gpu - ref| <= 1e-5 + 1e-4 |ref|;
* BF16 values (BF16 state, outputs o): at most 1 BF16 ulp apart in the ordered
  bit encoding, or |gpu - ref| <= 1e-5 (an absolute floor for values near zero,
  where one FP32 rounding can move the BF16 result by more than one ulp of a
  tiny number).

The gated RMSNorm output stage (assert_gated_close) is held to 1 BF16 ulp as
well, except at elements whose FP64 o (exported by the oracle before any
rounding) lies within GATED_TIE_ATOL + GATED_TIE_RTOL |o| of a BF16 rounding
boundary. That band covers the FP32 evaluation error of o with a margin: o is
a 128-term FP32 dot product plus a solve sum of at most 8 terms, with terms
below 1 in these workloads, so its FP32 error is of order 1e-7, ten times
below the band. At such elements
the stage first rounds o to BF16 (a rounding point of the method), and there
the stage's BF16 rounding of the kernel's FP32 o may go to the other
neighbour; that one-ulp difference of its input carries into the output,
whose own rounding can add a second ulp, so those elements (and only those)
are allowed 2 ulps.

The reference side is the FP64 oracle's output rounded once to the stored type.
"""
import numpy as np

F32_RTOL = 1e-4
F32_ATOL = 1e-5
BF16_ULPS = 1
BF16_ATOL = 1e-5
GATED_OUT_ULPS = 2
GATED_TIE_ATOL = 1e-6
GATED_TIE_RTOL = 1e-5


def _bf16_ordered(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def _bf16_value(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_mismatch(gpu_bits: np.ndarray, ref_bits: np.ndarray, ulps: int = BF16_ULPS) -> np.ndarray:
    """Boolean mask of BF16 elements outside the tolerance."""
    gpu_bits = np.asarray(gpu_bits, dtype=np.uint16)
    ref_bits = np.asarray(ref_bits, dtype=np.uint16)
    ulps_d = np.abs(_bf16_ordered(gpu_bits) - _bf16_ordered(ref_bits))
    absd = np.abs(_bf16_value(gpu_bits) - _bf16_value(ref_bits))
    return (ulps_d > ulps) & (absd > BF16_ATOL)


def bf16_tie_distance(o: np.ndarray) -> np.ndarray:
    """Distance of each FP64 value from the BF16 rounding boundary between the
    two BF16 values around it (their midpoint)."""
    o = np.asarray(o, dtype=np.float64)
    # The BF16 neighbours of o: its FP32 value truncated to 16 bits (toward
    # zero) and the next one away from zero. FP32's own rounding of o (2^-24
    # relative) only matters within 2^-24 of a BF16 value, half an ulp from
    # any boundary.
    bits = o.astype(np.float32).view(np.uint32)
    lo = (bits & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)
    hi = ((bits & np.uint32(0xFFFF0000)) + np.uint32(0x10000)).view(np.float32).astype(np.float64)
    return np.abs(o - 0.5 * (lo + hi))


def bf16_near_tie(o: np.ndarray, atol: float = GATED_TIE_ATOL,
                  rtol: float = GATED_TIE_RTOL) -> np.ndarray:
    """Boolean mask of FP64 values within atol + rtol |o| of a BF16 rounding
    boundary."""
    o = np.asarray(o, dtype=np.float64)
    return bf16_tie_distance(o) <= atol + rtol * np.abs(o)


def f32_mismatch(gpu: np.ndarray, ref: np.ndarray) -> np.ndarray:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return ~(np.abs(gpu - ref) <= F32_ATOL + F32_RTOL * np.abs(ref))


def _report(name, bad, gpu, ref):
    idx = np.argwhere(bad)[:5]
    ex = ", ".join(f"{tuple(i)}: gpu={gpu[tuple(i)]!r} ref={ref[tuple(i)]!r}" for i in idx)
    return f"{name}: {int(bad.sum())} of {bad.size} outside tolerance; e.g. {ex}"


def assert_bf16_close(name, gpu_bits, ref_bits, ulps: int = BF16_ULPS):
    gpu_bits = np.asarray(gpu_bits, dtype=np.uint16)
    ref_bits = np.asarray(ref_bits, dtype=np.uint16)
    assert gpu_bits.shape == ref_bits.shape, (name, gpu_bits.shape, ref_bits.shape)
    bad = bf16_mismatch(gpu_bits, ref_bits, ulps)
    assert not bad.any(), _report(name, bad, gpu_bits, ref_bits)


def assert_gated_close(name, gpu_bits, ref_bits, o_raw):
    """The gated output stage: 1 ulp (or the absolute floor) everywhere, 2 ulps
    where the oracle's unrounded o is near a BF16 rounding boundary."""
    gpu_bits = np.asarray(gpu_bits, dtype=np.uint16)
    ref_bits = np.asarray(ref_bits, dtype=np.uint16)
    o_raw = np.asarray(o_raw, dtype=np.float64)
    assert gpu_bits.shape == ref_bits.shape == o_raw.shape, (name, gpu_bits.shape,
                                                              ref_bits.shape, o_raw.shape)
    near = bf16_near_tie(o_raw)
    bad = bf16_mismatch(gpu_bits, ref_bits, BF16_ULPS) & ~(
        near & ~bf16_mismatch(gpu_bits, ref_bits, GATED_OUT_ULPS))
    assert not bad.any(), _report(name, bad, gpu_bits, ref_bits) + (
        f"; {int(near.sum())} of {near.size} elements near a tie")


def assert_f32_close(name, gpu, ref):
    gpu = np.asarray(gpu)
    ref = np.asarray(ref)
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    bad = f32_mismatch(gpu, ref)
    assert not bad.any(), _report(name, bad, gpu, ref)


def assert_exact(name, gpu, ref):
    gpu = np.asarray(gpu)
    ref = np.asarray(ref)
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    bad = gpu != ref
    assert not bad.any(), _report(name, bad, gpu, ref)
