"""Pins of the boundary (align) stores inside the fused replay: the fused step
with boundaries writes to each boundary slot exactly what the align commit
(commit page, KdaCommit with boundaries) of the same records writes there, and
the same S_n; m >= n stores S_n; a null boundary slot, m <= 0 or n = 0 store
nothing."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

K = V = 128


def _np(t):
    if t.dtype == torch.bfloat16:
        return W.bits(t)
    return t.detach().cpu().contiguous().numpy().copy()


def _fused(c, H, B, T, RQ, state, pending, bnd, blen):
    win = c["window"]
    out = np.zeros((B * T, H * V), np.uint16)
    oracle.fused_replay_verify(
        heads=H, tokens=T, batch=B, q=_np(win.q), k=_np(win.k), v=_np(win.v),
        raw_g=_np(win.raw_g), raw_beta=_np(win.raw_beta), a_log=_np(c["a_log"])[0],
        dt_bias=_np(c["dt_bias"])[0], lower_bound=W.LOWER_BOUND, state=state,
        state_slot_stride=H * V * K, state_indices=_np(c["state_indices"]),
        corr=_np(c["corr"]), kg=_np(c["kg"]), record_tokens=RQ,
        record_rows=_np(c["record_rows"]), pending=pending, out=out, boundaries=bnd,
        boundary_lens=blen)
    return state


@pytest.mark.parametrize("bf16", [False, True])
def test_fused_boundaries_equal_the_align_commit(bf16):
    H, B, T, RQ, S = 2, 6, 3, 6, 14
    c = W.small_fused_case(51, H, B, T, RQ, S, null_rows=(5,), no_record_rows=(4,))
    slots = _np(c["state_indices"])
    rows = _np(c["record_rows"])
    state0 = _np(c["state"])
    if bf16:
        state0 = W.bits(c["state"].to(torch.bfloat16))
    # pending (by record row) and boundaries (by request)
    n_req = [4, 6, 2, 0, 3, 5]
    m_req = [2, 9, 2, 3, 1, 4]           # m > n on request 1 stores S_n
    free = [sl for sl in range(1, S) if sl not in set(slots.tolist())]
    bnd = np.array(free[:B], np.int32)  # boundary slots no request owns
    bnd[2] = 0                          # request 2: null boundary
    pending = np.zeros(B, np.int32)
    for b in range(B):
        if rows[b] >= 0:
            pending[rows[b]] = n_req[b]
    blen = np.array(m_req, np.int32)
    fused = _fused(c, H, B, T, RQ, state0.copy(), pending, bnd, blen)
    # the align commit of the same records, in place (source = destination = slot)
    com = state0.copy()
    lens = np.array([pending[rows[b]] if rows[b] >= 0 else 0 for b in range(B)], np.int32)
    oracle.commit(heads=H, window=RQ, batch=B, state_bf16=bf16, state_layers=[com],
                  state_slot_strides=[H * V * K], corr_layers=[_np(c["corr"])],
                  corr_row_strides=[H * RQ * V], kg_layers=[_np(c["kg"])],
                  kg_row_strides=[H * RQ * 2 * K], a_log=_np(c["a_log"]),
                  dt_bias=_np(c["dt_bias"]), sources=slots, commit_lens=lens,
                  destinations=slots, boundaries=bnd, boundary_lens=blen, record_rows=rows,
                  lower_bound=W.LOWER_BOUND)
    page = H * V * K
    for b in range(B):
        live = lens[b] > 0 and slots[b] > 0
        for sl in (slots[b], bnd[b]):
            if sl <= 0:
                continue
            got = fused[sl * page:(sl + 1) * page]
            want = com[sl * page:(sl + 1) * page]
            assert np.array_equal(got, want), (b, sl)
        if live and bnd[b] > 0 and m_req[b] >= n_req[b]:
            # m >= n: the boundary holds S_n
            assert np.array_equal(fused[bnd[b] * page:(bnd[b] + 1) * page],
                                  fused[slots[b] * page:(slots[b] + 1) * page])
        if not live and bnd[b] > 0:
            assert np.array_equal(fused[bnd[b] * page:(bnd[b] + 1) * page],
                                  state0[bnd[b] * page:(bnd[b] + 1) * page])
    # slots nobody names are untouched
    named = set(slots.tolist()) | set(bnd.tolist())
    for sl in range(S):
        if sl not in named:
            assert np.array_equal(fused[sl * page:(sl + 1) * page],
                                  state0[sl * page:(sl + 1) * page])


def test_zero_boundary_length_stores_nothing():
    H, B, T, RQ, S = 1, 3, 2, 4, 8
    c = W.small_fused_case(53, H, B, T, RQ, S)
    rows = _np(c["record_rows"])
    pending = np.zeros(B, np.int32)
    pending[rows] = 3
    state0 = _np(c["state"])
    free = [sl for sl in range(1, S) if sl not in set(_np(c["state_indices"]).tolist())]
    bnd = np.array(free[:B], np.int32)
    fused = _fused(c, H, B, T, RQ, state0.copy(), pending, bnd, np.array([0, -1, 0], np.int32))
    plain = _fused(c, H, B, T, RQ, state0.copy(), pending, None, None)
    assert np.array_equal(fused, plain)
