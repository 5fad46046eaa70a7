"""Tolerances of the parity tests, in one place.

* integer, index and bit-copy data (plans, key/gate records, memory the call
  must not touch): bit-exact;
* FP32 values (FP32 state, corrections, decays): |gpu - ref| <= 1e-5 + 1e-4 |ref|;
* BF16 values (BF16 state, outputs o): at most 1 BF16 ulp apart in the ordered
  bit encoding, or |gpu - ref| <= 1e-5 (an absolute floor for values near zero,
  where one FP32 rounding can move the BF16 result by more than one ulp of a
  tiny number).

The gated RMSNorm output stage allows 2 BF16 ulps (GATED_OUT_ULPS): it first
rounds o to BF16 (a rounding point of the method), and at a near-tie the FP32
and FP64 values of o can round to neighbouring BF16 values; that one-ulp
difference of its input carries into the output, whose own rounding can add a
second ulp.

The reference side is the FP64 oracle's output rounded once to the stored type.
"""
import numpy as np

F32_RTOL = 1e-4
F32_ATOL = 1e-5
BF16_ULPS = 1
BF16_ATOL = 1e-5
GATED_OUT_ULPS = 2


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
