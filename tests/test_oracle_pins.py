"""Pins of the FP64 oracle against what the pages and mathematics fix.

Nothing here retypes the oracle's formulas: each test checks the oracle
against a special value, a closed form, an exact rational brute force of a
different algorithm (closed-form commit, chunked WY verify), an invariant the
pages state, or a library routine for a step that reduces to one.

Pages (vLLM API docs on Kimi-K3 KDA): "vllm.models.kimi_k3.nvidia.recoverssm.
cutedsl.commit" (commit page), "vllm.models.kimi_k3.nvidia.specialized_decode.
recoverssm.kernels" (kernels page), "vllm.models.kimi_k3.nvidia.
specialized_decode.cutedsl.kda.fused" (fused page).
"""
import math
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import exact


# --------------------------------------------------------------------------
# Conversions
# --------------------------------------------------------------------------

def test_bf16_round_matches_torch_on_fp32_values():
    """For FP32-representable inputs, a direct double->BF16 RNE equals torch's
    FP32->BF16 RNE (a library routine), including exact ties."""
    rng = np.random.default_rng(0)
    u = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    u &= np.uint32(0xBFFFFFFF)  # finite, moderate exponents
    u[::3] = (u[::3] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)  # exact ties
    f = u.view(np.float32)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_bf16(f.astype(np.float64))
    assert np.array_equal(got, want)


def test_bf16_round_no_double_rounding():
    """1 + 2^-8 + 2^-30 lies just above a BF16 tie: it must round up to
    1 + 2^-7 (0x3F81). Rounding through FP32 first would land on the tie and
    round to even (0x3F80)."""
    x = 1.0 + 2.0**-8 + 2.0**-30
    assert oracle.round_bf16(np.array([x]))[0] == 0x3F81
    assert oracle.round_bf16(np.array([-x]))[0] == 0xBF81
    assert oracle.round_bf16(np.array([1.0 + 2.0**-8]))[0] == 0x3F80  # tie -> even
    assert oracle.round_bf16(np.array([1.0 + 3 * 2.0**-8]))[0] == 0x3F82  # tie -> even (up)


def test_bf16_to_double_matches_torch():
    b = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    b = b[((b >> 7) & 0xFF) != 0xFF]  # finite only
    want = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_to_f64(b), want)


# --------------------------------------------------------------------------
# Decay, sigmoid, key normalisation: special values and closed forms
# --------------------------------------------------------------------------

def test_decay_special_values():
    # g + dt_bias = 0: sigmoid(0) = 1/2, so d = e^{lb/2}  (fused page, KdaFused.decay)
    assert oracle.decay(0.3, 0.7, -0.3, -5.0) == pytest.approx(math.exp(-2.5), rel=1e-15)
    # lb = 0: d = 1 exactly, whatever the gate
    for g in (-3.0, 0.0, 2.5):
        assert oracle.decay(g, 0.1, 0.2, 0.0) == 1.0
    # exp(A_log) = 2 and g + dt_bias = ln(3)/2: the logit is ln 3, sigmoid 3/4
    g = math.log(3.0) / 2 - 0.125
    assert oracle.decay(g, math.log(2.0), 0.125, -4.0) == pytest.approx(math.exp(-3.0), rel=1e-14)
    # limits: a large positive logit gives e^{lb}, a large negative one 1
    assert oracle.decay(60.0, 0.0, 0.0, -5.0) == pytest.approx(math.exp(-5.0), rel=1e-15)
    assert oracle.decay(-60.0, 0.0, 0.0, -5.0) == pytest.approx(1.0, rel=1e-15)


def test_decay_monotone_and_bounded():
    gs = np.linspace(-8, 8, 401)
    ds = [oracle.decay(g, 0.3, -0.05, -5.0) for g in gs]
    assert all(a > b for a, b in zip(ds, ds[1:]))  # lb < 0: decreasing in g
    assert all(math.exp(-5.0) < d < 1.0 for d in ds)


def test_sigmoid_values():
    assert oracle.sigmoid(0.0) == 0.5
    assert oracle.sigmoid(math.log(3.0)) == pytest.approx(0.75, rel=1e-15)
    assert oracle.sigmoid(-math.log(3.0)) == pytest.approx(0.25, rel=1e-15)


def test_knorm_closed_form():
    k = np.array([3.0, 4.0])
    out = oracle.knorm(k)
    assert out == pytest.approx(k / math.sqrt(25.0 + 1e-6), rel=1e-15)
    rng = np.random.default_rng(1)
    x = rng.standard_normal(128) * 0.01  # small norm: the 1e-6 term matters
    s = float(np.sum(x * x))
    kn = oracle.knorm(x)
    assert float(np.sum(kn * kn)) == pytest.approx(s / (s + 1e-6), rel=1e-13)
    assert np.allclose(kn / np.linalg.norm(kn), x / np.linalg.norm(x), rtol=1e-14)


# --------------------------------------------------------------------------
# Exact rational brute force (K = V = 3): the three forms agree exactly, and
# the C oracle matches them to FP64 rounding.
# --------------------------------------------------------------------------

def _rand_frac(rnd, lo, hi, den=64):
    return Fraction(rnd.randint(int(lo * den), int(hi * den)), den)


def _exact_case(seed, K=3, V=3, T=5):
    rnd = random.Random(seed)
    S0 = [[_rand_frac(rnd, -1, 1) for _ in range(K)] for _ in range(V)]
    d = [[Fraction(rnd.randint(1, 16), 16) for _ in range(K)] for _ in range(T)]  # (0, 1]
    kn = [[_rand_frac(rnd, -1, 1) for _ in range(K)] for _ in range(T)]
    q = [[_rand_frac(rnd, -1, 1) for _ in range(K)] for _ in range(T)]
    u = [[_rand_frac(rnd, -2, 2) for _ in range(V)] for _ in range(T)]
    v = [[_rand_frac(rnd, -2, 2) for _ in range(V)] for _ in range(T)]
    beta = [Fraction(rnd.randint(0, 16), 16) for _ in range(T)]
    return S0, d, kn, q, u, v, beta


def _f(M):
    return np.array([[float(x) for x in row] for row in M], dtype=np.float64)


@pytest.mark.parametrize("seed", range(6))
def test_exact_commit_forms_agree(seed):
    S0, d, kn, q, u, v, beta = _exact_case(seed, T=8)
    for n in range(0, 9):
        seq = exact.commit_seq(S0, u, kn, d, n)
        closed = exact.commit_closed(S0, u, kn, d, n)
        assert seq == closed
        # The C oracle against the exact result (inputs are exact dyadics).
        for fn in (oracle.commit_seq, oracle.commit_closed, oracle.commit_logspace):
            got = fn(_f(S0), _f(u), _f(kn), _f(d), n)
            assert np.allclose(got, _f(seq), rtol=1e-13, atol=1e-14), fn.__name__


@pytest.mark.parametrize("seed", range(6))
def test_exact_verify_forms_agree(seed):
    for T in (1, 2, 3, 5):
        S0, d, kn, q, u, v, beta = _exact_case(100 + seed, T=T)
        o_seq, u_seq, _ = exact.verify_seq(S0, q, kn, v, d, beta)
        o_wy, u_wy = exact.verify_wy(S0, q, kn, v, d, beta)
        assert o_seq == o_wy and u_seq == u_wy
        o, uu, _ = oracle.verify_seq(_f(S0), _f(q), _f(kn), _f(v), _f(d),
                                     np.array([float(b) for b in beta]))
        assert np.allclose(o, _f(o_seq), rtol=1e-12, atol=1e-13)
        assert np.allclose(uu, _f(u_seq), rtol=1e-12, atol=1e-13)
        o2, u2 = oracle.verify_wy(_f(S0), _f(q), _f(kn), _f(v), _f(d),
                                  np.array([float(b) for b in beta]))
        assert np.allclose(o2, _f(o_seq), rtol=1e-12, atol=1e-13)
        assert np.allclose(u2, _f(u_seq), rtol=1e-12, atol=1e-13)


def test_exact_recoverssm_identity():
    """The commit of the first n verify tokens with the verify's own corrections
    reproduces the recurrence's state after n tokens, exactly (fused page,
    module docstring: the verify leaves the checkpoint and the commit rebuilds
    the state from the records)."""
    S0, d, kn, q, _, v, beta = _exact_case(7, T=6)
    _, u, _ = exact.verify_seq(S0, q, kn, v, d, beta)
    for n in range(0, 7):
        _, _, Sn = exact.verify_seq(S0, q[:n], kn[:n], v[:n], d[:n], beta[:n])
        assert exact.commit_seq(S0, u, kn, d, n) == Sn


def test_hand_worked_commit_2x2():
    """A 2x2 example worked by hand from the closed form (commit page, module
    docstring): S0 = [[1,2],[3,4]], d0 = [1/2,1/4], d1 = [1,1/2], keys e0 and
    e1, u0 = [1,1], u1 = [2,0], n = 2. D_2 = [1/2, 1/8]; P_0 = d1; P_1 = 1.
    S_2 = [[1/2,1/4],[3/2,1/2]] + [[1,0],[1,0]] + [[0,2],[0,0]]."""
    S0 = np.array([[1.0, 2.0], [3.0, 4.0]])
    d = np.array([[0.5, 0.25], [1.0, 0.5]])
    kn = np.array([[1.0, 0.0], [0.0, 1.0]])
    u = np.array([[1.0, 1.0], [2.0, 0.0]])
    want = np.array([[1.5, 2.25], [2.5, 0.5]])
    assert np.array_equal(oracle.commit_seq(S0, u, kn, d, 2), want)
    # and after one token only: S0 diag(d0) + u0 e0^T
    assert np.array_equal(oracle.commit_seq(S0, u, kn, d, 1), np.array([[1.5, 0.5], [2.5, 1.0]]))


# --------------------------------------------------------------------------
# Invariants at K = V = 128 (FP64)
# --------------------------------------------------------------------------

def _rand_item(rng, T, K=128, V=128):
    S0 = rng.standard_normal((V, K)) * 0.1
    d = np.exp(-5.0 * rng.uniform(0.0, 1.0, (T, K)))
    x = rng.standard_normal((T, K))
    kn = x / np.linalg.norm(x, axis=1, keepdims=True)
    q = rng.standard_normal((T, K)) / math.sqrt(K)
    v = rng.standard_normal((T, V))
    u = rng.standard_normal((T, V)) * 0.5
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    return S0, d, kn, q, v, u, beta


def test_commit_forms_agree_fp64():
    rng = np.random.default_rng(2)
    S0, d, kn, q, v, u, beta = _rand_item(rng, 8)
    for n in range(9):
        a = oracle.commit_seq(S0, u, kn, d, n)
        b = oracle.commit_closed(S0, u, kn, d, n)
        c = oracle.commit_logspace(S0, u, kn, d, n)
        assert np.allclose(a, b, rtol=1e-12, atol=1e-14)
        assert np.allclose(a, c, rtol=1e-12, atol=1e-14)


def test_commit_invariants():
    rng = np.random.default_rng(3)
    S0, d, kn, q, v, u, beta = _rand_item(rng, 8)
    # n = 0 leaves S unchanged, bit for bit
    assert np.array_equal(oracle.commit_seq(S0, u, kn, d, 0), S0)
    # u = 0: pure decay S0 diag(prod d)
    got = oracle.commit_seq(S0, np.zeros_like(u), kn, d, 8)
    assert np.allclose(got, S0 * np.prod(d, axis=0)[None, :], rtol=1e-13)
    # d = 1 (lower bound 0): plain delta-rule accumulation S0 + sum u_t kn_t^T
    got = oracle.commit_seq(S0, u, kn, np.ones_like(d), 8)
    assert np.allclose(got, S0 + u.T @ kn, rtol=1e-12, atol=1e-14)
    # associativity: commit(n) = commit(n - m) after commit(m), records shifted
    for m in range(0, 9):
        first = oracle.commit_seq(S0, u, kn, d, m)
        second = oracle.commit_seq(first, u[m:], kn[m:], d[m:], 8 - m)
        assert np.allclose(second, oracle.commit_seq(S0, u, kn, d, 8), rtol=1e-12, atol=1e-14)


def test_verify_forms_agree_fp64():
    rng = np.random.default_rng(4)
    for T in (1, 2, 4, 7, 8):
        S0, d, kn, q, v, u, beta = _rand_item(rng, T)
        o1, u1, _ = oracle.verify_seq(S0, q, kn, v, d, beta)
        o2, u2 = oracle.verify_wy(S0, q, kn, v, d, beta)
        assert np.allclose(o1, o2, rtol=1e-10, atol=1e-12)
        assert np.allclose(u1, u2, rtol=1e-10, atol=1e-12)


def test_verify_delta_rule_retrieval():
    """beta = 1 and q_t = kn_t with unit keys: the written value is read back,
    o_t = v_t, for any decay (S_t kn_t = v_t after a full delta-rule write)."""
    rng = np.random.default_rng(5)
    S0, d, kn, q, v, u, beta = _rand_item(rng, 8)
    o, uu, _ = oracle.verify_seq(S0, kn, kn, v, d, np.ones(8))
    assert np.allclose(o, v, rtol=1e-12, atol=1e-12)


def test_verify_beta_zero():
    """beta = 0: no writes, u = 0, o_t = S0 (Gamma_t * q_t)."""
    rng = np.random.default_rng(6)
    S0, d, kn, q, v, u, beta = _rand_item(rng, 6)
    o, uu, Sf = oracle.verify_seq(S0, q, kn, v, d, np.zeros(6))
    assert np.all(uu == 0.0)
    gamma = np.cumprod(d, axis=0)
    assert np.allclose(o, (S0 @ (gamma * q).T).T, rtol=1e-12, atol=1e-14)
    assert np.allclose(Sf, S0 * gamma[-1][None, :], rtol=1e-12)


def test_verify_basis_keys_no_decay():
    """lb = 0 (d = 1), beta = 1, keys the standard basis vectors e_0..e_{T-1}:
    each token overwrites column c_t with v_t, so o_t = S_t q_t with S_t equal
    to S0 whose first t+1 columns are replaced by v_0..v_t."""
    rng = np.random.default_rng(7)
    K = V = 16
    T = 4
    S0 = rng.standard_normal((V, K))
    kn = np.eye(K)[:T]
    q = rng.standard_normal((T, K))
    v = rng.standard_normal((T, V))
    o, uu, _ = oracle.verify_seq(S0, q, kn, v, np.ones((T, K)), np.ones(T))
    for t in range(T):
        St = S0.copy()
        for s in range(t + 1):
            St[:, s] = v[s]
        assert np.allclose(o[t], St @ q[t], rtol=1e-13, atol=1e-13)
        assert np.allclose(uu[t], v[t] - S0[:, t], rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# Plan steps: properties over exhaustive small cases
# --------------------------------------------------------------------------

def _plan_cases():
    vals_rec = (-1, 0, 1)
    vals_src = (-1, 0, 2)
    vals_len = (-2, 0, 3, 9)
    for r0 in vals_rec:
        for r1 in vals_rec:
            if r0 >= 0 and r0 == r1:
                continue  # shared record rows are outside the contract
            for s0 in vals_src:
                for s1 in vals_src:
                    for l0 in vals_len:
                        for l1 in vals_len:
                            for e in (None, (0, 1), (1, 0)):
                                yield (r0, r1), (s0, s1), (l0, l1), e


def test_plan_defer_flush_properties():
    """The defer step moves a valid request's commit length into its record
    row's pending count (eager: pending 0, length kept); the flush plan reads
    it back clamped to [0, q], with final = source and no boundary; invalid
    rows (record row < 0 or slot <= null) change nothing (kernels page,
    _defer_commit_kernel and _prepare_flush_plan_kernel docstrings)."""
    q = 4
    for rows, srcs, lens, eager in _plan_cases():
        rr = np.array(rows, np.int32)
        si = np.array(srcs, np.int32)
        cl = np.array(lens, np.int32)
        pending = np.full(3, 77, np.int32)
        eg = None if eager is None else np.array(eager, np.int32)
        oracle.defer(si, cl, rr, pending, eg, null_slot=0)
        for b in range(2):
            valid = rows[b] >= 0 and srcs[b] > 0
            is_eager = eager is not None and eager[b] != 0
            if not valid:
                assert cl[b] == lens[b]
            elif is_eager:
                assert pending[rows[b]] == 0 and cl[b] == lens[b]
            else:
                assert pending[rows[b]] == lens[b] and cl[b] == 0
        untouched = [r for r in range(3) if r not in [rows[b] for b in range(2)
                                                     if rows[b] >= 0 and srcs[b] > 0]]
        assert all(pending[r] == 77 for r in untouched)
        before = pending.copy()
        fl, fin, bnd, blen = oracle.flush_plan(si, rr, pending, q, null_slot=0)
        assert np.array_equal(pending, before)  # read only
        assert np.array_equal(fin, si) and np.all(bnd == 0) and np.all(blen == 0)
        for b in range(2):
            n = pending[rows[b]] if rows[b] >= 0 else 0
            n = min(max(int(n), 0), q)
            assert fl[b] == (n if (srcs[b] > 0 and n > 0) else 0)
            valid = rows[b] >= 0 and srcs[b] > 0
            is_eager = eager is not None and eager[b] != 0
            if valid and not is_eager:  # round trip: what was deferred is flushed
                assert fl[b] == min(max(lens[b], 0), q)
            if valid and is_eager:
                assert fl[b] == 0
