"""Pins of the oracle's low-rank gate projection (fused page, KdaFused.kernel:
raw_g = BF16(F_A F_B^T), the gate projection feeding the decays).

* on the exact grid of the workload generator, the projection is an integer
  matrix product times 2^-13 (numpy int64), rounded once;
* one-hot F_A rows select F_B columns bit for bit (operand order and indexing);
* F_A read as a column slice of wider packed rows equals the contiguous copy;
* on general BF16 inputs it is numpy's FP64 product rounded once.
"""
import numpy as np
import torch

import oracle
import workloads as W

K = 128


def test_exact_grid_is_an_integer_product():
    fa, fb = W.draw_gate_factors(W._gen(1), 37, 2)
    fa_b, fb_b = W.bits(fa), W.bits(fb)
    ma = np.rint(fa.float().numpy() * 64).astype(np.int64)
    mb = np.rint(fb.float().numpy() * 128).astype(np.int64)
    assert np.array_equal(ma.astype(np.float64) / 64, fa.float().numpy().astype(np.float64))
    prod = ma @ mb.T  # exact
    assert np.abs(prod).max() < 2 ** 21  # every partial sum is exact in FP32
    want = oracle.round_bf16(prod.astype(np.float64) * 2.0 ** -13)
    got = oracle.gate_projection(fa_b, fb_b)
    assert np.array_equal(got, want)
    assert 0.5 < np.std(prod * 2.0 ** -13) < 1.2


def test_one_hot_rows_select_columns():
    fb = W.bits(W.draw_gate_factors(W._gen(2), 1, 3, exact=False)[1])  # [384, 128]
    N = 20
    fa = np.zeros((N, K), np.float32)
    js = np.random.default_rng(3).integers(0, K, N)
    fa[np.arange(N), js] = 1.0
    got = oracle.gate_projection(oracle.round_bf16(fa.astype(np.float64)), fb)
    assert np.array_equal(got, fb[:, js].T)


def test_row_stride_reads_a_column_slice():
    N, H, pitch, col0 = 9, 2, 1000, 600
    fa, fb = W.draw_gate_factors(W._gen(4), N, H, exact=False)
    packed = W.bits(W.normal(W._gen(5), (N, pitch)).to(torch.bfloat16))
    packed[:, col0:col0 + K] = W.bits(fa)
    flat = packed.reshape(-1)[col0:]
    got = oracle.gate_projection(flat, W.bits(fb), f_a_row_stride=pitch, tokens=N)
    want = oracle.gate_projection(W.bits(fa), W.bits(fb))
    assert np.array_equal(got, want)


def test_general_inputs_match_fp64_product():
    fa, fb = W.draw_gate_factors(W._gen(6), 33, 2, exact=False)
    exact = fa.double().numpy() @ fb.double().numpy().T
    got = oracle.gate_projection(W.bits(fa), W.bits(fb))
    assert np.array_equal(got, oracle.round_bf16(exact))
