"""Pins of variable-length windows (kernels page, kda_recoverssm_verify: the
query_start_loc metadata): request b's tokens are rows qsl[b] .. qsl[b+1] - 1.

* uniform offsets [0, T, 2T, ...] give exactly the fixed-window results;
* each request of a ragged batch gives exactly what a one-request call with
  tokens = its length gives (outputs, records, replayed state);
* a zero-length window reads and writes nothing; rows past qsl[B] and record
  tokens past a request's length keep their values; lengths above the window
  are clamped to it.
"""
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


def _args(c, H, B, T, RQ, rows_total, qsl=None):
    win = c["window"]
    n = B * T
    def rows(x):
        a = _np(x)
        out = np.zeros((rows_total,) + a.shape[1:], a.dtype)
        out[:min(n, rows_total)] = a[:rows_total]
        return out
    return dict(heads=H, tokens=T, batch=B, q=rows(win.q), k=rows(win.k), v=rows(win.v),
                raw_g=rows(win.raw_g), raw_beta=rows(win.raw_beta),
                a_log=_np(c["a_log"])[0], dt_bias=_np(c["dt_bias"])[0],
                lower_bound=W.LOWER_BOUND, state=_np(c["state"]), state_slot_stride=H * V * K,
                state_indices=_np(c["state_indices"]), corr=_np(c["corr"]), kg=_np(c["kg"]),
                record_tokens=RQ, record_rows=_np(c["record_rows"]),
                out=np.full((rows_total, H * V), 0x7FFF, np.uint16), query_start_loc=qsl)


def _run(fused, args, pending=None):
    if fused:
        oracle.fused_replay_verify(pending=pending, **args)
    else:
        oracle.verify(**args)
    return args


@pytest.mark.parametrize("fused", [False, True])
def test_uniform_offsets_equal_fixed_windows(fused):
    H, B, T, RQ = 2, 4, 3, 5
    c = W.small_fused_case(31, H, B, T, RQ, 7, null_rows=(2,), no_record_rows=(1,))
    pend = _np(c["pending"])
    a = _run(fused, _args(c, H, B, T, RQ, B * T), pend)
    qsl = np.arange(0, (B + 1) * T, T, dtype=np.int32)
    b = _run(fused, _args(c, H, B, T, RQ, B * T, qsl), pend)
    for key in ("out", "corr", "kg", "state"):
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("fused", [False, True])
def test_ragged_requests_equal_one_request_calls(fused):
    H, T, RQ = 2, 4, 6
    lens = [3, 0, 1, 4, 2, 9]  # 9 is clamped to T
    B = len(lens)
    c = W.small_fused_case(33, H, B, T, RQ, 9, null_rows=(4,))
    pend = _np(c["pending"])
    qsl = np.zeros(B + 1, np.int32)
    eff = [min(max(l, 0), T) for l in lens]
    qsl[1:] = np.cumsum(lens)
    total = int(qsl[-1]) + 3  # three rows nobody owns
    full = _args(c, H, B, T, RQ, total + 64, qsl)
    # the window rows of request b are rows qsl[b] ..: fill them from the drawn window
    win = {n: _np(getattr(c["window"], n)) for n in ("q", "k", "v", "raw_g", "raw_beta")}
    for n in win:
        for b in range(B):
            for t in range(eff[b]):
                full[n][qsl[b] + t] = win[n][b * T + t]
    out0, corr0, kg0, state0 = full["out"].copy(), full["corr"].copy(), full["kg"].copy(), \
        full["state"].copy()
    _run(fused, full, pend)
    rows = _np(c["record_rows"])
    slots = _np(c["state_indices"])
    owned = np.zeros(full["out"].shape[0], bool)
    for b in range(B):
        L = eff[b]
        if L == 0:
            r = rows[b]
            assert np.array_equal(full["corr"][r], corr0[r])
            assert np.array_equal(full["kg"][r], kg0[r])
            page = slice(slots[b] * H * V * K, (slots[b] + 1) * H * V * K)
            assert np.array_equal(full["state"][page], state0[page])
            continue
        owned[qsl[b]:qsl[b] + L] = True
        one = dict(full)
        one.update(tokens=L, batch=1, query_start_loc=None,
                   state_indices=slots[b:b + 1], record_rows=rows[b:b + 1],
                   state=state0.copy(), corr=corr0.copy(), kg=kg0.copy(),
                   out=np.full((L, H * V), 0x7FFF, np.uint16))
        for n in win:
            one[n] = np.ascontiguousarray(win[n][b * T:b * T + L])
        _run(fused, one, pend)
        assert np.array_equal(full["out"][qsl[b]:qsl[b] + L], one["out"]), b
        r = rows[b]
        assert np.array_equal(full["corr"][r], one["corr"][r]), b
        assert np.array_equal(full["kg"][r], one["kg"][r]), b
        page = slice(slots[b] * H * V * K, (slots[b] + 1) * H * V * K)
        assert np.array_equal(full["state"][page], one["state"][page]), b
        # record tokens past the length keep their values
        assert np.array_equal(full["corr"][r, :, L:], corr0[r, :, L:])
    assert np.all(full["out"][~owned] == 0x7FFF)
