"""Buffer-level pins of the oracle: the library's semantics on host arrays.

The buffer functions (commit, verify, fused replay+verify) are checked against
the item-level recurrence (itself pinned in test_oracle_pins.py) through
properties the pages state: the RecoverSSM identity (a commit of the verify's
own records rebuilds the recurrence state), fused = commit followed by verify,
the deferred protocol's end-to-end claim (fused over a prior window's records
continues the recurrence), and the no-op rules (null slot, record row < 0,
n = 0, slots nobody names).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _pinned_cases import gated_rounding_case

K = V = 128


def _np(t):
    if t.dtype == torch.bfloat16:
        return W.bits(t)
    return t.detach().cpu().contiguous().numpy().copy()


def _bf(bits):
    return oracle.bf16_to_f64(bits)


def _item_inputs(win, b, h, T, a_log, dtb, lb):
    """Double-precision per-item inputs from a window (decays, normalised keys
    and beta computed by the oracle's own pinned scalar steps)."""
    q = _bf(_np(win.q))[b * T:(b + 1) * T, h]
    kr = _bf(_np(win.k))[b * T:(b + 1) * T, h]
    v = _bf(_np(win.v))[b * T:(b + 1) * T, h]
    g = _bf(_np(win.raw_g))[b * T:(b + 1) * T, h]
    rb = _bf(_np(win.raw_beta))[b * T:(b + 1) * T, h]
    kn = np.stack([oracle.knorm(kr[t]) for t in range(T)])
    d = np.array([[oracle.decay(g[t, c], a_log[h], dtb[h, c], lb) for c in range(K)]
                  for t in range(T)])
    beta = np.array([oracle.sigmoid(x) for x in rb])
    return q, kn, v, d, beta


def _case(seed=11, H=2, B=3, T=4, RQ=4, slots=6, **kw):
    c = W.small_fused_case(seed, H, B, T, RQ, slots, **kw)
    return c


def _run_verify(c, H, B, T, RQ, fused, state=None, corr=None, kg=None, pending=None,
                win=None, rows="given"):
    state = _np(c["state"]) if state is None else state
    corr = _np(c["corr"]) if corr is None else corr
    kg = _np(c["kg"]) if kg is None else kg
    win = c["window"] if win is None else win
    out = np.full((B * T, H * V), 0x7FFF, dtype=np.uint16)  # a sentinel pattern
    args = dict(heads=H, tokens=T, batch=B, q=_np(win.q), k=_np(win.k), v=_np(win.v),
                raw_g=_np(win.raw_g), raw_beta=_np(win.raw_beta),
                a_log=_np(c["a_log"])[0], dt_bias=_np(c["dt_bias"])[0],
                lower_bound=W.LOWER_BOUND, state=state, state_slot_stride=H * V * K,
                state_indices=_np(c["state_indices"]), corr=corr, kg=kg,
                record_tokens=RQ, out=out,
                record_rows=_np(c["record_rows"]) if rows == "given" else rows)
    if fused:
        oracle.fused_replay_verify(pending=_np(c["pending"]) if pending is None else pending,
                                   **args)
    else:
        oracle.verify(**args)
    return state, corr, kg, out


def test_verify_writes_records_and_not_state():
    H, B, T, RQ = 2, 3, 4, 6
    c = _case(H=H, B=B, T=T, RQ=RQ, no_record_rows=(2,))
    s0 = _np(c["state"])
    corr0, kg0 = _np(c["corr"]), _np(c["kg"])
    state, corr, kg, out = _run_verify(c, H, B, T, RQ, fused=False)
    assert np.array_equal(state, s0)  # the checkpoint is never written
    rows = _np(c["record_rows"])
    win = c["window"]
    k_bits, g_bits = _np(win.k), _np(win.raw_g)
    for b in range(B):
        r = rows[b]
        if r < 0:
            continue
        for h in range(H):
            for t in range(T):
                tok = b * T + t
                assert np.array_equal(kg[r, h, t, :K], k_bits[tok, h])
                assert np.array_equal(kg[r, h, t, K:], g_bits[tok, h])
            # tokens past T in the record keep their old contents
            assert np.array_equal(kg[r, h, T:], kg0[r, h, T:])
            assert np.array_equal(corr[r, h, T:], corr0[r, h, T:])
    # the row with record row -1 wrote nothing, but produced outputs
    written = {int(r) for r in rows if r >= 0}
    for r in range(corr.shape[0]):
        if r not in written:
            assert np.array_equal(corr[r], corr0[r]) and np.array_equal(kg[r], kg0[r])
    assert not np.any(out == 0x7FFF)


def test_verify_matches_item_recurrence():
    H, B, T, RQ = 2, 2, 5, 5
    c = _case(seed=12, H=H, B=B, T=T, RQ=RQ, slots=4)
    state, corr, kg, out = _run_verify(c, H, B, T, RQ, fused=False)
    a_log, dtb = _np(c["a_log"])[0], _np(c["dt_bias"])[0]
    slots, rows = _np(c["state_indices"]), _np(c["record_rows"])
    for b in range(B):
        for h in range(H):
            S0 = state.reshape(-1, H, V, K)[slots[b], h].astype(np.float64)
            q, kn, v, d, beta = _item_inputs(c["window"], b, h, T, a_log, dtb, W.LOWER_BOUND)
            o, u, _ = oracle.verify_seq(S0, q, kn, v, d, beta)
            assert np.array_equal(out[b * T:(b + 1) * T, h * V:(h + 1) * V], oracle.round_bf16(o))
            assert np.array_equal(corr[rows[b], h, :T], u.astype(np.float32))


def test_null_slot_rows_output_zero_and_touch_nothing():
    H, B, T, RQ = 2, 3, 3, 4
    c = _case(seed=13, H=H, B=B, T=T, RQ=RQ, null_rows=(1,))
    s0, corr0, kg0 = _np(c["state"]), _np(c["corr"]), _np(c["kg"])
    for fused in (False, True):
        state, corr, kg, out = _run_verify(c, H, B, T, RQ, fused=fused, state=s0.copy(),
                                           corr=corr0.copy(), kg=kg0.copy())
        assert np.all(out[T:2 * T] == 0)
        r = _np(c["record_rows"])[1]
        assert np.array_equal(corr[r], corr0[r]) and np.array_equal(kg[r], kg0[r])


def test_commit_buffer_rules_and_identity():
    """Verify writes the records; the commit of n of them (FP32 state, source =
    destination) equals the recurrence after n tokens (RecoverSSM identity,
    through FP32-stored corrections); n = 0 and null rows write nothing; a slot
    nobody names is unchanged."""
    H, B, T, RQ = 2, 3, 4, 4
    c = _case(seed=14, H=H, B=B, T=T, RQ=RQ, slots=6)
    s0 = _np(c["state"])
    state, corr, kg, out = _run_verify(c, H, B, T, RQ, fused=False, state=s0.copy())
    slots, rows = _np(c["state_indices"]), _np(c["record_rows"])
    lens = np.array([3, 0, 4], np.int32)
    st = state.copy()
    oracle.commit(heads=H, window=RQ, batch=B, state_bf16=False, state_layers=[st],
                  state_slot_strides=[H * V * K], corr_layers=[corr],
                  corr_row_strides=[H * RQ * V], kg_layers=[kg],
                  kg_row_strides=[H * RQ * 2 * K], a_log=_np(c["a_log"]),
                  dt_bias=_np(c["dt_bias"]), sources=slots, commit_lens=lens,
                  destinations=slots, record_rows=rows, lower_bound=W.LOWER_BOUND)
    pages0 = s0.reshape(-1, H, V, K)
    pages = st.reshape(-1, H, V, K)
    a_log, dtb = _np(c["a_log"])[0], _np(c["dt_bias"])[0]
    for b in range(B):
        for h in range(H):
            if lens[b] == 0:
                assert np.array_equal(pages[slots[b], h], pages0[slots[b], h])
                continue
            q, kn, v, d, beta = _item_inputs(c["window"], b, h, T, a_log, dtb, W.LOWER_BOUND)
            n = int(lens[b])
            _, _, Sn = oracle.verify_seq(pages0[slots[b], h].astype(np.float64), q[:n],
                                         kn[:n], v[:n], d[:n], beta[:n])
            assert np.allclose(pages[slots[b], h], Sn, rtol=1e-5, atol=1e-6)
    others = set(range(6)) - set(int(s) for s in slots)
    for s in others:
        assert np.array_equal(pages[s], pages0[s])


def test_commit_align_boundary_and_bf16():
    """Align: the boundary slot gets the commit of min(m, n) tokens, the
    destination that of n; both BF16, rounded once from FP64 (commit page,
    module docstring and KdaCommit.kernel)."""
    H, B, Q = 2, 3, 8
    g = W._gen(21)
    corr, kgr = W.draw_records(g, B, H, Q)
    corr, kgr = _np(corr), _np(kgr)
    a_log, dtb = W.draw_gate_params(g, 1, H)
    a_log, dtb = _np(a_log), _np(dtb)
    S = 10
    stride = H * V * K + 64
    pool = W.bits(W.draw_state(5, S * stride, torch.bfloat16))
    src = np.array([1, 2, 3], np.int32)
    dst = np.array([4, 5, 6], np.int32)
    bnd = np.array([7, 0, 8], np.int32)
    lens = np.array([6, 5, 3], np.int32)
    blen = np.array([2, 3, 7], np.int32)  # row 2: m > n -> S_n
    st = pool.copy()
    oracle.commit(heads=H, window=Q, batch=B, state_bf16=True, state_layers=[st],
                  state_slot_strides=[stride], corr_layers=[corr],
                  corr_row_strides=[H * Q * V], kg_layers=[kgr],
                  kg_row_strides=[H * Q * 2 * K], a_log=a_log, dt_bias=dtb, sources=src,
                  commit_lens=lens, destinations=dst, boundaries=bnd, boundary_lens=blen,
                  lower_bound=W.LOWER_BOUND)

    def page(arr, slot, h):
        return arr[slot * stride + h * V * K: slot * stride + (h + 1) * V * K].reshape(V, K)

    for b in range(B):
        for h in range(H):
            S0 = _bf(page(pool, src[b], h))
            kn = np.stack([oracle.knorm(_bf(kgr[b, h, t, :K])) for t in range(Q)])
            d = np.array([[oracle.decay(x, a_log[0, h], dtb[0, h, c], W.LOWER_BOUND)
                           for c, x in enumerate(_bf(kgr[b, h, t, K:]))] for t in range(Q)])
            u = corr[b, h].astype(np.float64)
            n = int(lens[b])
            want = oracle.round_bf16(oracle.commit_closed(S0, u, kn, d, n))
            assert np.array_equal(page(st, dst[b], h), want)
            if bnd[b] > 0:
                m = min(int(blen[b]), n)
                want_b = oracle.round_bf16(oracle.commit_closed(S0, u, kn, d, m))
                assert np.array_equal(page(st, bnd[b], h), want_b)
            # the source page is unchanged (source != destination)
            assert np.array_equal(page(st, src[b], h), page(pool, src[b], h))
    assert np.array_equal(page(st, 9, 0), page(pool, 9, 0))  # unnamed slot


def test_fused_equals_commit_then_verify():
    """fused(S0, records, pending) = commit(pending of the records) in place,
    then verify, with the records rewritten (fused page, module docstring)."""
    H, B, T, RQ = 2, 4, 3, 5
    c = _case(seed=15, H=H, B=B, T=T, RQ=RQ, slots=8, null_rows=(3,), no_record_rows=(2,))
    s0, corr0, kg0 = _np(c["state"]), _np(c["corr"]), _np(c["kg"])
    pending = np.array([2, 0, 4, 5], np.int32)  # row with rec=-1 ignores its pending
    rows = _np(c["record_rows"])
    pend_by_row = np.zeros(B, np.int32)
    for b in range(B):
        if rows[b] >= 0:
            pend_by_row[rows[b]] = pending[b]
    st_f, corr_f, kg_f, out_f = _run_verify(c, H, B, T, RQ, True, state=s0.copy(),
                                            corr=corr0.copy(), kg=kg0.copy(),
                                            pending=pend_by_row)
    # composition: commit with lens = pending (0 for rec < 0), then verify
    slots = _np(c["state_indices"])
    lens = np.array([pend_by_row[rows[b]] if rows[b] >= 0 else 0 for b in range(B)], np.int32)
    st_c = s0.copy()
    oracle.commit(heads=H, window=RQ, batch=B, state_bf16=False, state_layers=[st_c],
                  state_slot_strides=[H * V * K], corr_layers=[corr0],
                  corr_row_strides=[H * RQ * V], kg_layers=[kg0],
                  kg_row_strides=[H * RQ * 2 * K], a_log=_np(c["a_log"]),
                  dt_bias=_np(c["dt_bias"]), sources=slots, commit_lens=lens,
                  destinations=slots, record_rows=rows, lower_bound=W.LOWER_BOUND)
    st_v, corr_v, kg_v, out_v = _run_verify(c, H, B, T, RQ, False, state=st_c.copy(),
                                            corr=corr0.copy(), kg=kg0.copy())
    assert np.array_equal(st_f, st_c)  # the same FP32 rounding of S_n
    assert np.array_equal(kg_f, kg_v)
    assert np.allclose(corr_f, corr_v, rtol=1e-6, atol=1e-7)
    diff = np.abs(out_f.view(np.int16).astype(np.int32) - out_v.view(np.int16).astype(np.int32))
    assert diff.max() <= 1
    # n = 0 items keep their page bit for bit
    pages0 = s0.reshape(-1, H, V, K)
    pages = st_f.reshape(-1, H, V, K)
    assert np.array_equal(pages[slots[1]], pages0[slots[1]])
    assert np.array_equal(pages[slots[2]], pages0[slots[2]])  # rec < 0: no replay


@pytest.mark.parametrize("n", [0, 1, 3, 4])
def test_deferred_protocol_continues_the_recurrence(n):
    """Verify a prior window (records written), defer n accepted tokens, then
    fused-verify a new window: its outputs equal the stock recurrence run over
    the first n prior tokens followed by the new window, from the original
    checkpoint (fused page, module docstring; kernels page, defer step)."""
    H, B, T, RQ = 2, 2, 4, 4
    c = _case(seed=16, H=H, B=B, T=T, RQ=RQ, slots=4)
    prior = W.draw_window(W._gen(99), B, T, H)
    s0 = _np(c["state"])
    state, corr, kg, _ = _run_verify(c, H, B, T, RQ, False, state=s0.copy(), win=prior)
    slots, rows = _np(c["state_indices"]), _np(c["record_rows"])
    pending = np.zeros(B, np.int32)
    lens = np.full(B, n, np.int32)
    oracle.defer(slots, lens, rows, pending)
    assert np.all(lens == 0)
    state, corr, kg, out = _run_verify(c, H, B, T, RQ, True, state=state, corr=corr, kg=kg,
                                       pending=pending)
    a_log, dtb = _np(c["a_log"])[0], _np(c["dt_bias"])[0]
    for b in range(B):
        for h in range(H):
            p = _item_inputs(prior, b, h, T, a_log, dtb, W.LOWER_BOUND)
            x = _item_inputs(c["window"], b, h, T, a_log, dtb, W.LOWER_BOUND)
            seq = [np.concatenate([p[i][:n], x[i]]) for i in range(5)]
            S0 = s0.reshape(-1, H, V, K)[slots[b], h].astype(np.float64)
            o, _, _ = oracle.verify_seq(S0, *seq)
            got = out[b * T:(b + 1) * T, h * V:(h + 1) * V]
            want = oracle.round_bf16(o[n:])
            diff = np.abs(got.view(np.int16).astype(np.int32) - want.view(np.int16).astype(np.int32))
            assert diff.max() <= 1  # FP32-stored corrections, then one BF16 rounding


def test_fused_pending_clamped_to_record_capacity():
    """A pending count above the records' capacity replays RQ tokens; a negative
    one replays none (fused page, KdaFused.kernel: n clamped to [0, RQ])."""
    H, B, T, RQ = 1, 2, 2, 3
    c = _case(seed=17, H=H, B=B, T=T, RQ=RQ, slots=4)
    s0, corr0, kg0 = _np(c["state"]), _np(c["corr"]), _np(c["kg"])
    rows = _np(c["record_rows"])

    def run(p0, p1):
        pend = np.zeros(B, np.int32)
        pend[rows[0]], pend[rows[1]] = p0, p1
        return _run_verify(c, H, B, T, RQ, True, state=s0.copy(), corr=corr0.copy(),
                           kg=kg0.copy(), pending=pend)

    hi = run(RQ + 5, -4)
    ref = run(RQ, 0)
    for a, b in zip(hi, ref):
        assert np.array_equal(a, b)
    mid = run(RQ - 1, 1)
    assert not np.array_equal(mid[0], ref[0])  # the clamp point matters


# --------------------------------------------------------------------------
# Gated RMSNorm output stage (fused page, KdaFused output stage)
# --------------------------------------------------------------------------

def _gated_run(c, H, B, T, RQ, state, v_scale=1.0, gate_val=None, w=None, eps=0.0, seed=3):
    win = c["window"]
    g = W._gen(seed)
    gate = W.bits(W.bf16(W.normal(g, (B * T, H * V)))) if gate_val is None else \
        np.full((B * T, H * V), W.bits(torch.tensor([gate_val]).to(torch.bfloat16))[0], np.uint16)
    wv = np.ones(V, np.float32) if w is None else w
    vbits = W.bits((win.v.float() * v_scale).to(torch.bfloat16))
    out = np.zeros((B * T, H * V), np.uint16)
    oracle.verify(heads=H, tokens=T, batch=B, q=_np(win.q), k=_np(win.k), v=vbits,
                  raw_g=_np(win.raw_g), raw_beta=_np(win.raw_beta), a_log=_np(c["a_log"])[0],
                  dt_bias=_np(c["dt_bias"])[0], lower_bound=W.LOWER_BOUND, state=state,
                  state_slot_stride=H * V * K, state_indices=_np(c["state_indices"]),
                  corr=_np(c["corr"]), kg=_np(c["kg"]), record_tokens=RQ, out=out,
                  record_rows=_np(c["record_rows"]), gate=gate, norm_weight=wv, norm_eps=eps)
    return out


def test_gated_rmsnorm_scale_invariance_exact():
    """With eps = 0 the output is invariant under scaling the state and v by 2:
    o scales by 2 exactly, BF16 rounding commutes with it, rstd halves exactly."""
    H, B, T, RQ = 2, 3, 4, 4
    c = _case(seed=31, H=H, B=B, T=T, RQ=RQ, slots=5, null_rows=(2,))
    s0 = _np(c["state"])
    a = _gated_run(c, H, B, T, RQ, s0.copy())
    b = _gated_run(c, H, B, T, RQ, (s0 * 2.0).astype(np.float32), v_scale=2.0)
    assert np.array_equal(a, b)
    assert np.all(a[2 * T:3 * T] == 0)  # the null-slot request: zeros
    assert np.count_nonzero(a[:2 * T]) > 0.9 * a[:2 * T].size


def test_gated_rmsnorm_unit_rms_and_gate_half():
    """Saturated gate (sigmoid(60) == 1 in FP64), unit weight, eps = 0: every
    (token, head) output row has mean square 1 up to BF16 rounding. Gate 0
    halves every output exactly (sigmoid(0) = 1/2 and halving is exact)."""
    H, B, T, RQ = 2, 2, 3, 3
    c = _case(seed=32, H=H, B=B, T=T, RQ=RQ, slots=4)
    s0 = _np(c["state"])
    full = _gated_run(c, H, B, T, RQ, s0.copy(), gate_val=60.0)
    half = _gated_run(c, H, B, T, RQ, s0.copy(), gate_val=0.0)
    f = oracle.bf16_to_f64(full).reshape(B * T, H, V)
    ms = (f * f).mean(axis=2)
    assert np.allclose(ms, 1.0, atol=3e-3)  # BF16 output rounding moves it by ~1e-3 at most here
    assert np.array_equal(oracle.bf16_to_f64(half), oracle.bf16_to_f64(full) * 0.5)


def test_gated_rmsnorm_weight_scales_channels():
    """A weight of 2 on one channel doubles that channel's output exactly and
    leaves the others (the mean is over o, not over the weighted output)."""
    H, B, T, RQ = 1, 2, 2, 2
    c = _case(seed=33, H=H, B=B, T=T, RQ=RQ, slots=3)
    s0 = _np(c["state"])
    w = np.ones(V, np.float32)
    base = _gated_run(c, H, B, T, RQ, s0.copy(), w=w, eps=1e-5)
    w2 = w.copy()
    w2[17] = 2.0
    two = _gated_run(c, H, B, T, RQ, s0.copy(), w=w2, eps=1e-5)
    bv, tv = oracle.bf16_to_f64(base), oracle.bf16_to_f64(two)
    assert np.array_equal(tv[:, 17], 2.0 * bv[:, 17])
    other = np.arange(V) != 17
    assert np.array_equal(tv[:, other], bv[:, other])


def test_gated_rmsnorm_eps_dominated_exact():
    """eps = 2^24, far above mean(o^2): rstd = 2^-12 (1 + O(1e-9)), so with a
    saturated gate and unit weight the output is the plain BF16 output times
    2^-12, exactly (a power-of-two scale of a BF16 value needs no rounding)."""
    H, B, T, RQ = 2, 2, 3, 3
    c = _case(seed=34, H=H, B=B, T=T, RQ=RQ, slots=4)
    s0 = _np(c["state"])
    gated = _gated_run(c, H, B, T, RQ, s0.copy(), gate_val=60.0, eps=2.0 ** 24)
    _, _, _, plain = _run_verify(c, H, B, T, RQ, False, state=s0.copy())
    assert np.array_equal(oracle.bf16_to_f64(gated), oracle.bf16_to_f64(plain) * 2.0 ** -12)


def test_gated_rmsnorm_rounds_o_before_both_uses():
    """The output stage's BF16 rounding of o, pinned at both of its uses by the
    hand-derived case above: exact expected bits, and the raw o exported for
    the GPU tests' near-tie flags equals S_0[:, 0] exactly."""
    args, want, a = gated_rounding_case()
    out = np.zeros((1, V), np.uint16)
    o_raw = np.zeros((1, V), np.float64)
    oracle.verify(out=out, o_raw=o_raw, **args)
    assert np.array_equal(out[0], want), [hex(x) for x in out[0, :4]]
    assert o_raw[0, 0] == a and o_raw[0, 1] == 2.0 ** -4 and not o_raw[0, 2:].any()
    # The fused step from the same slot with nothing pending gives the same row.
    out_f = np.zeros((1, V), np.uint16)
    oracle.fused_replay_verify(out=out_f, pending=np.zeros(1, np.int32),
                               **{k: (v.copy() if isinstance(v, np.ndarray) else v)
                                  for k, v in args.items()})
    assert np.array_equal(out_f, out)
    # The case discriminates: the values each dropped rounding would give lie on
    # the other side of a rounding boundary (closed forms from the docstring).
    bf = lambda x: int(oracle.round_bf16(np.array([x]))[0])
    rstd = np.sqrt(128.0 / (1.0 + 2.0 ** -8))
    w = args["norm_weight"].astype(np.float64)
    assert bf(2.0 ** -4 * np.sqrt(128.0 / (a * a + 2.0 ** -8)) * w[1]) == 0x3F7F
    assert bf(a * rstd * w[0]) == 0x3F81


def test_fused_bf16_state_matches_fp32_state():
    """The same BF16-representable pool as BF16 bits and as FP32: the outputs
    and records are bit-identical (both continue from the FP64 S_n), and the
    BF16 page written back is the FP32 page's value rounded to nearest even
    (they differ only by the final store rounding)."""
    H, B, T, RQ = 2, 4, 3, 5
    c = _case(seed=41, H=H, B=B, T=T, RQ=RQ, slots=7, null_rows=(3,), no_record_rows=(2,))
    s_bits = W.bits(c["state"].to(torch.bfloat16))
    s_f32 = oracle.bf16_to_f64(s_bits).astype(np.float32)
    rows = _np(c["record_rows"])
    pend = np.zeros(B, np.int32)
    for b, n in enumerate([4, 0, 3, 5]):
        if rows[b] >= 0:
            pend[rows[b]] = n
    rb = _run_verify(c, H, B, T, RQ, True, state=s_bits.copy(), pending=pend)
    rf = _run_verify(c, H, B, T, RQ, True, state=s_f32.copy(), pending=pend)
    assert np.array_equal(rb[1], rf[1]) and np.array_equal(rb[2], rf[2])  # records
    assert np.array_equal(rb[3], rf[3])  # outputs
    got = oracle.bf16_to_f64(rb[0])
    want = oracle.bf16_to_f64(oracle.round_bf16(rf[0].astype(np.float64)))
    # float -> bf16 of the FP32 page can differ from double -> bf16 only at an
    # exact FP32 tie: allow those, nothing else.
    diff = got != want
    assert diff.mean() < 1e-3
    assert np.all(np.abs(got[diff] - want[diff]) <= np.abs(want[diff]) * 2.0 ** -7)
    # slots nobody names are untouched bit for bit
    named = set(int(x) for x in _np(c["state_indices"]))
    pages = rb[0].reshape(-1, H * V * K)
    for sl in range(pages.shape[0]):
        if sl not in named:
            assert np.array_equal(pages[sl], s_bits.reshape(-1, H * V * K)[sl])
