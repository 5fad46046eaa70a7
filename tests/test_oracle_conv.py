"""Pins of the oracle's convolution prologue (fused page, KdaFused.kernel: the
convolution and SiLU of q, k, v, the q/k normalisation and the window roll).

Each pin checks the oracle against something other than itself:
* its FP32 exp against libm's exp (closed form, within a few FP32 ulps);
* its BF16 SiLU decision against the FP64 SiLU rounded once (equal except at
  near-ties, where FP32 and FP64 may round to neighbours);
* the convolution's tap order against one-hot weights (a shift, by definition);
* the window roll over several fused steps against a textbook causal
  convolution of the accepted token stream (numpy, FP64);
* the q normalisation and scale against a closed form of a one-token verify
  from a zero state;
* the window write-back against its definition.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W

K = V = 128
EPS = 1e-6


def _np(t):
    if t.dtype == torch.bfloat16:
        return W.bits(t)
    return t.detach().cpu().contiguous().numpy().copy()


def _f(bits):
    return oracle.bf16_to_f64(np.asarray(bits, np.uint16))


def _silu64(a):
    return a / (1.0 + np.exp(-a))


def _near_tie(x, rel=2.0 ** -18):
    """True where the FP64 value x lies within rel (relative) of a BF16 rounding
    midpoint, so that an FP32 evaluation may round to the other neighbour."""
    x = np.asarray(x, np.float64)
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    ulp = np.exp2(e - 7)
    frac = ax / ulp - np.floor(ax / ulp)
    return (np.abs(frac - 0.5) * ulp <= rel * ax) & (ax > 0)


def _ulps(a_bits, b_bits):
    a = np.asarray(a_bits, np.int32)
    b = np.asarray(b_bits, np.int32)
    oa = np.where(a & 0x8000, -(a & 0x7FFF), a & 0x7FFF)
    ob = np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    return np.abs(oa - ob)


# ---------------------------------------------------------------- scalar steps

def test_exp_f32_against_libm():
    xs = np.concatenate([np.linspace(-80, 80, 20001),
                         np.random.default_rng(0).normal(0, 6, 20000)]).astype(np.float32)
    xs = np.clip(xs, -80, 80)
    got = np.array([oracle.exp_f32(float(x)) for x in xs])
    want = np.exp(xs.astype(np.float64))
    rel = np.abs(got - want) / want
    assert rel.max() < 2.0 ** -21, rel.max()
    assert oracle.exp_f32(0.0) == 1.0
    # the argument is clamped to [-80, 80]
    assert oracle.exp_f32(200.0) == oracle.exp_f32(80.0)
    assert oracle.exp_f32(-200.0) == oracle.exp_f32(-80.0)


def test_silu_bf16_is_the_fp64_silu_rounded_once():
    rng = np.random.default_rng(1)
    acc = np.concatenate([rng.normal(0, 4, 30000), rng.normal(0, 0.05, 5000),
                          [0.0, 1.0, -1.0, 20.0, -20.0]]).astype(np.float32)
    got = np.array([oracle.silu_bf16(float(a)) for a in acc], np.uint16)
    exact = _silu64(acc.astype(np.float64))
    want = oracle.round_bf16(exact)
    tie = _near_tie(exact)
    assert np.all(got[~tie] == want[~tie])
    assert np.all(_ulps(got[tie], want[tie]) <= 1)
    assert tie.mean() < 4e-3  # about 2 * 2^-18 / 2^-7.5 of the values
    assert oracle.silu_bf16(0.0) == 0
    # SiLU(x) -> x for large x, and is odd-symmetric up to x: SiLU(-x) = SiLU(x) - x
    assert _f(oracle.silu_bf16(40.0)) == 40.0


def test_conv_tap_order_by_one_hot_weights():
    rng = np.random.default_rng(2)
    T = 6
    seq = _f(oracle.round_bf16(rng.normal(0, 1, 3 + T))).astype(np.float32)
    for i in range(4):
        w = np.zeros(4, np.float32)
        w[i] = 1.0
        y = oracle.conv_silu(seq, w)
        # output t sees seq[t + i]: weight 0 the oldest tap, weight 3 the input
        want = [oracle.silu_bf16(float(seq[t + i])) for t in range(T)]
        assert list(y) == want
    # zero weights: only the bias
    y = oracle.conv_silu(seq, np.zeros(4, np.float32), bias=0.75)
    assert list(y) == [oracle.silu_bf16(0.75)] * T
    # linear in the taps before the SiLU: w = (a, b, 0, 0) is a two-term sum
    w = np.array([0.5, -2.0, 0.0, 0.0], np.float32)
    y = oracle.conv_silu(seq, w)
    pre = 0.5 * seq[:T].astype(np.float64) - 2.0 * seq[1:T + 1]
    assert np.all(_ulps(y, oracle.round_bf16(_silu64(pre))) <= 1)


def test_conv_offset_is_the_history_after_n_accepted_tokens():
    assert [oracle.conv_offset(n) for n in range(9)] == [0, 0, 1, 2, 3, 4, 5, 6, 7]


# ---------------------------------------------------------------- buffer level

def _setup(seed, H, B, T, RQ, S, dim_first=True):
    c = W.small_fused_case(seed, H, B, T, RQ, S)
    cv = W.draw_conv_inputs(W._gen(seed + 1000), B, T, H, RQ, S)
    hk = H * K
    Wn = RQ + 2
    win = _np(cv.window)  # [S, 3hk, W]
    if dim_first:
        strides = (3 * hk * Wn, Wn, 1)
        pool = win.reshape(-1).copy()
    else:  # window-major: [S, W, 3hk]
        strides = (3 * hk * Wn, 1, 3 * hk)
        pool = win.transpose(0, 2, 1).reshape(-1).copy()
    return c, cv, pool, strides


def _window_of(pool, strides, slot, col, W):
    ss, cs, ts = strides
    return pool[slot * ss + col * cs + np.arange(W) * ts]


def _run(c, cv, pool, strides, H, B, T, RQ, pending, state=None, corr=None, kg=None,
         rows="given", gate=None, norm_weight=None, bias=True):
    state = _np(c["state"]) if state is None else state
    corr = _np(c["corr"]) if corr is None else corr
    kg = _np(c["kg"]) if kg is None else kg
    out = np.full((B * T, H * V), 0x7FFF, np.uint16)
    win = c["window"]
    oracle.fused_conv_replay_verify(
        heads=H, tokens=T, batch=B, x=_np(cv.x), x_row_stride=cv.pitch,
        conv_weight=_np(cv.weight), conv_bias=_np(cv.bias) if bias else None,
        conv_state=pool, conv_slot_stride=strides[0], conv_channel_stride=strides[1],
        conv_tap_stride=strides[2], q_scale=K ** -0.5, raw_g=_np(win.raw_g),
        raw_beta=_np(win.raw_beta), a_log=_np(c["a_log"])[0], dt_bias=_np(c["dt_bias"])[0],
        lower_bound=W.LOWER_BOUND, state=state, state_slot_stride=H * V * K,
        state_indices=_np(c["state_indices"]),
        corr=corr, kg=kg, record_tokens=RQ,
        record_rows=_np(c["record_rows"]) if isinstance(rows, str) else rows,
        pending=pending, out=out, gate=gate, norm_weight=norm_weight)
    return state, corr, kg, out


@pytest.mark.parametrize("dim_first", [True, False])
def test_window_roll_is_a_causal_convolution_of_the_accepted_stream(dim_first):
    """Three fused steps; after each, a request accepts n in 1..T tokens, which
    the defer step turns into the next step's pending count. The recorded keys
    of every step (the k part's SiLU outputs, bit for bit) equal a textbook
    causal convolution over the accepted stream, computed here in FP64."""
    H, B, T, RQ, S = 2, 3, 4, 5, 5
    c, cv, pool, strides = _setup(21, H, B, T, RQ, S, dim_first)
    hk = H * K
    slots = _np(c["state_indices"])
    rows = _np(c["record_rows"])
    x = _f(_np(cv.x))
    wt = _f(_np(cv.weight))  # [3, 4, hk]
    bias = _f(_np(cv.bias))
    rng = np.random.default_rng(5)
    pending = np.zeros(B, np.int32)
    pending[rows] = np.array([0, 2, RQ])[:B]  # step 0: offsets 0, 1, RQ-1
    # the history (last 3 pre-activations) each request's first step sees
    hist = {}
    for b in range(B):
        off = oracle.conv_offset(int(pending[rows[b]]))
        for part in range(3):
            for h in range(H):
                for ch in range(K):
                    col = part * hk + h * K + ch
                    w = _f(_window_of(pool, strides, slots[b], col, RQ + 2))
                    hist[(b, col)] = list(w[off:off + 3])
    state, corr, kg = _np(c["state"]), _np(c["corr"]), _np(c["kg"])
    for step in range(3):
        # the same x every step is fine: the stream differs by the roll
        state, corr, kg, out = _run(c, cv, pool, strides, H, B, T, RQ, pending.copy(),
                                    state=state, corr=corr, kg=kg)
        acc = rng.integers(1, T + 1, B)
        for b in range(B):
            r = rows[b]
            for h in range(H):
                col = hk + h * K + np.arange(K)  # the k part
                seqs = np.array([hist[(b, int(cc))] for cc in col])  # [K, 3]
                xs = x[b * T:(b + 1) * T, col].T  # [K, T]
                stream = np.concatenate([seqs, xs], axis=1)  # [K, 3 + T]
                w = wt[1][:, h * K:(h + 1) * K].T  # [K, 4]
                pre = bias[col][:, None] + sum(w[:, i:i + 1] * stream[:, i:i + T]
                                               for i in range(4))
                want = oracle.round_bf16(_silu64(pre)).T  # [T, K]
                got = kg[r, h, :T, :K]
                tie = _near_tie(_silu64(pre)).T
                assert np.all(got[~tie] == want[~tie]), (step, b, h)
                assert np.all(_ulps(got[tie], want[tie]) <= 1)
        # the next step replays the accepted tokens: history rolls by n
        for b in range(B):
            n = int(acc[b])
            for part in range(3):
                for h in range(H):
                    for ch in range(K):
                        col = part * hk + h * K + ch
                        s = hist[(b, col)] + list(x[b * T:b * T + n, col])
                        hist[(b, col)] = s[-3:]
            pending[rows[b]] = n


def test_window_write_back():
    H, B, T, RQ, S = 2, 3, 3, 6, 5
    c, cv, pool, strides = _setup(23, H, B, T, RQ, S)
    before = pool.copy()
    slots = _np(c["state_indices"])
    rows = _np(c["record_rows"])
    pending = np.zeros(B, np.int32)
    pending[rows] = np.array([0, 3, 6])
    _run(c, cv, pool, strides, H, B, T, RQ, pending)
    x = _np(cv.x)
    hk = H * K
    Wn = RQ + 2
    touched = np.zeros(pool.size, bool)
    for b in range(B):
        off = oracle.conv_offset(int(pending[rows[b]]))
        for col in range(3 * hk):
            old = _window_of(before, strides, slots[b], col, Wn)
            new = _window_of(pool, strides, slots[b], col, Wn)
            want = old.copy()
            want[0], want[1] = old[off + 1], old[off + 2]
            want[2:2 + T] = x[b * T:(b + 1) * T, col]
            assert np.array_equal(new, want), (b, col)
            ss, cs, ts = strides
            touched[slots[b] * ss + col * cs + np.arange(Wn) * ts] = True
    assert np.array_equal(pool[~touched], before[~touched])


def test_null_slot_leaves_the_window():
    H, B, T, RQ, S = 1, 3, 2, 2, 5
    c, cv, pool, strides = _setup(25, H, B, T, RQ, S)
    si = c["state_indices"].clone()
    si[1] = 0
    c["state_indices"] = si
    before = pool.copy()
    pending = np.zeros(B, np.int32)
    _, _, _, out = _run(c, cv, pool, strides, H, B, T, RQ, pending)
    Wn = RQ + 2
    for col in range(3 * H * K):
        assert np.array_equal(_window_of(pool, strides, 0, col, Wn),
                              _window_of(before, strides, 0, col, Wn))
    assert np.all(out[T:2 * T] == 0)


@pytest.mark.parametrize("tiny", [False, True])
def test_q_normalisation_and_scale_closed_form(tiny):
    """One token from a zero state with n = 0: S_1 = beta v kn^T and
    o = S_1 qn = beta v (kn . qn). With the q and k parts given the same
    pre-activations, weights and bias, kn . qn = scale * ss / (ss + 1e-6)
    with ss the squared norm of the SiLU outputs, so
    o[v] = beta * y_v[v] * scale * ss / (ss + 1e-6) (FP64, rounded once).
    tiny: q and k pre-activations of 2^-20 (bias only), so that ss is about
    3e-11 and the 1e-6 inside the root dominates the norm."""
    H, B, T, RQ, S = 2, 2, 1, 1, 4
    c, cv, pool, strides = _setup(27, H, B, T, RQ, S)
    hk = H * K
    x = _np(cv.x)
    wt = _np(cv.weight)
    bias = _np(cv.bias)
    Wn = RQ + 2
    win = pool.reshape(S, 3 * hk, Wn)
    if tiny:
        x[:, 0:hk] = 0
        win[:, 0:hk] = 0
        bias[0:hk] = oracle.round_bf16(np.full(hk, 2.0 ** -20))
    x[:, hk:2 * hk] = x[:, 0:hk]  # k pre-activations = q pre-activations
    wt[1] = wt[0]
    bias[hk:2 * hk] = bias[0:hk]
    win[:, hk:2 * hk] = win[:, 0:hk]
    cv = W.ConvInputs(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16),
                      torch.from_numpy(wt.view(np.int16)).view(torch.bfloat16),
                      torch.from_numpy(bias.view(np.int16)).view(torch.bfloat16), None)
    pool0 = pool.copy()
    state = np.zeros(S * H * V * K, np.float32)
    pending = np.zeros(B, np.int32)
    _, _, _, out = _run(c, cv, pool, strides, H, B, T, RQ, pending, state=state)
    slots = _np(c["state_indices"])
    rb = _f(_np(c["window"].raw_beta))
    scale = K ** -0.5
    for b in range(B):
        for h in range(H):
            ys = []
            for part in (0, 2):
                y = []
                for ch in range(K):
                    col = part * hk + h * K + ch
                    w0 = _f(_window_of(pool0, strides, slots[b], col, Wn)).astype(np.float32)
                    xin = float(_f(x[b:b + 1, col])[0])
                    seq = np.array([w0[0], w0[1], w0[2], xin], np.float32)
                    y.append(oracle.conv_silu(seq, _f(wt[part, :, h * K + ch]).astype(np.float32),
                                              float(_f(bias[col:col + 1])[0]))[0])
                ys.append(_f(np.array(y, np.uint16)))
            yq, yv = ys
            ss = float(np.dot(yq, yq))
            assert (ss < 1e-9) == tiny
            beta = 1.0 / (1.0 + math.exp(-rb[b, h]))
            want = oracle.round_bf16(beta * yv * scale * ss / (ss + EPS))
            got = out[b, h * V:(h + 1) * V]
            assert np.all(_ulps(got, want) <= 1), (b, h)


@pytest.mark.parametrize("dim_first", [True, False])
def test_plain_silu_key_check_on_the_oracle(dim_first):
    """The GPU tests' check of the recorded keys against the plain FP64
    convolution and SiLU (check_conv_keys_plain) passes on the oracle's own
    records for every window offset, with a small near-tie share; and it fails
    when a key is one ulp off outside the band."""
    from _kda_cases import check_conv_keys_plain
    H, B, T, RQ, S = 2, 4, 4, 6, 6
    c, cv, pool, strides = _setup(29, H, B, T, RQ, S, dim_first)
    rows = _np(c["record_rows"])
    pending = np.zeros(B, np.int32)
    pending[rows] = np.array([0, 1, 4, RQ])
    before = pool.copy()
    _, _, kg, _ = _run(c, cv, pool, strides, H, B, T, RQ, pending.copy())
    kw = dict(H=H, T=T, RQ=RQ, x=_np(cv.x), pitch=cv.pitch, conv_w=_np(cv.weight),
              conv_b=_np(cv.bias), pool=before, strides=strides,
              slots=_np(c["state_indices"]), rows=rows, pending=pending)
    share = check_conv_keys_plain("oracle", kg, **kw)
    assert share < 0.01
    # a planted one-ulp error on a key far from a tie is caught
    from _kda_cases import silu_keys_plain
    want, near = silu_keys_plain(H=H, T=T, RQ=RQ, x=kw["x"], pitch=cv.pitch, conv_w=kw["conv_w"],
                                 conv_b=kw["conv_b"], pool=before, strides=strides,
                                 slot=int(kw["slots"][0]), n=int(pending[rows[0]]), tok0=0)
    h, t, ch = np.argwhere(~near & (want != 0))[0]
    bad = kg.copy()
    bad[rows[0], h, t, ch] ^= 1
    with pytest.raises(AssertionError):
        check_conv_keys_plain("planted", bad, **kw)
