"""FP64 CPU oracle of the KDA gated delta-rule state update (TEST INFRASTRUCTURE).

Only tests/, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package. The GPU library (``spec_decode_amd``) never
imports, links or calls it, and shares no code with it.

This module is a thin ctypes/numpy wrapper over ``libkda_oracle.so`` (built
from ``kda_oracle.c`` by ``oracle/build.py``). Every function works on host
numpy arrays with the same layouts the GPU library uses:

* state pools ``[slots, H, V, K]`` (FP32 as float32, BF16 as uint16 bits),
* records: corrections ``[rows, H, RQ, V]`` float32, key/gate
  ``[rows, H, RQ, 2K]`` uint16 (raw key, then raw gate),
* activations ``[B*T, H, K]`` uint16 BF16 bits, raw beta ``[B*T, H]``,
* outputs ``[B*T, H*V]`` uint16 BF16 bits.

Buffer-level functions modify their output arrays in place, as the library does.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.environ.get("KDA_ORACLE_LIB") or os.path.join(_HERE, "libkda_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build

        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    i, d, l = ctypes.c_int, ctypes.c_double, ctypes.c_long
    sig = {
        "kda_o_decay": (d, [d, d, d, d]),
        "kda_o_sigmoid": (d, [d]),
        "kda_o_knorm": (None, [i, _dp, _dp]),
        "kda_o_double_to_bf16": (ctypes.c_uint16, [d]),
        "kda_o_bf16_to_double": (d, [ctypes.c_uint16]),
        "kda_o_round_bf16_buf": (None, [l, _dp, _u16p]),
        "kda_o_bf16_to_double_buf": (None, [l, _u16p, _dp]),
        "kda_o_commit_seq": (None, [i, i, i, _dp, _dp, _dp, _dp, _dp]),
        "kda_o_commit_closed": (None, [i, i, i, _dp, _dp, _dp, _dp, _dp]),
        "kda_o_commit_logspace": (None, [i, i, i, _dp, _dp, _dp, _dp, _dp]),
        "kda_o_verify_seq": (None, [i, i, i, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp]),
        "kda_o_verify_wy": (None, [i, i, i, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp]),
        "kda_o_commit": (i, [i, i, i, i, i, i, i, _vp, _i64p, _vp, _i64p, _vp, _i64p,
                             _fp, _fp, _i32p, _i32p, _i32p, _i32p, _i32p, _i32p,
                             d, i, _i64p, l, i]),
        "kda_o_verify": (i, [i, i, i, i, i, _u16p, _u16p, _u16p, _u16p, _u16p, _fp, _fp,
                             d, _vp, ctypes.c_int64, _i32p, i, _fp, _u16p, i, _i32p,
                             _i32p, i, _u16p, _i64p, l, i, _u16p, _fp, d, i, _u16p,
                             ctypes.c_int64, _u16p, _u16p, _u16p, ctypes.c_int64,
                             ctypes.c_int64, ctypes.c_int64, d, _i32p, _i32p, _i32p, _dp]),
        "kda_o_exp_f32": (ctypes.c_float, [ctypes.c_float]),
        "kda_o_silu_bf16": (ctypes.c_uint16, [ctypes.c_float]),
        "kda_o_conv_silu": (None, [i, _fp, _fp, ctypes.c_float, _u16p]),
        "kda_o_conv_offset": (i, [i]),
        "kda_o_gate_projection": (None, [l, i, i, _u16p, ctypes.c_int64, _u16p, _u16p]),
        "kda_o_decay_buf": (None, [l, i, i, _u16p, _fp, _fp, d, _fp]),
        "kda_o_defer": (None, [i, _i32p, _i32p, _i32p, _i32p, _i32p, i]),
        "kda_o_flush_plan": (None, [i, i, _i32p, _i32p, _i32p, _i32p, _i32p, _i32p,
                                    _i32p, i]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def default_threads() -> int:
    """Every core this process may run on, capped at 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _ptr(a, ct):
    if a is None:
        return None
    return a.ctypes.data_as(ct)


def _c(a, dtype):
    """A C-contiguous array of ``dtype`` (no copy when already one)."""
    return np.ascontiguousarray(a, dtype=dtype)


def _check_inplace(a, dtype, name):
    if not (isinstance(a, np.ndarray) and a.dtype == dtype and a.flags["C_CONTIGUOUS"]
            and a.flags["WRITEABLE"]):
        raise TypeError(f"{name} must be a writeable C-contiguous {np.dtype(dtype)} array")


# ----------------------------------------------------------------------------
# Scalars and conversions
# ----------------------------------------------------------------------------

def decay(g, a_log, dt_bias, lower_bound):
    """exp(lb * sigmoid(exp(A_log) * (g + dt_bias))) in FP64 (scalar)."""
    return _load().kda_o_decay(float(g), float(a_log), float(dt_bias), float(lower_bound))


def sigmoid(x):
    return _load().kda_o_sigmoid(float(x))


def knorm(k):
    k = _c(k, np.float64)
    out = np.empty_like(k)
    _load().kda_o_knorm(k.shape[-1], _ptr(k, _dp), _ptr(out, _dp))
    return out


def round_bf16(x):
    """FP64 values -> BF16 bit patterns (uint16), round to nearest even."""
    x = _c(x, np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().kda_o_round_bf16_buf(x.size, _ptr(x, _dp), _ptr(out, _u16p))
    return out


def bf16_to_f64(bits):
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    _load().kda_o_bf16_to_double_buf(bits.size, _ptr(bits, _u16p), _ptr(out, _dp))
    return out


# ----------------------------------------------------------------------------
# Item-level cores (double arrays): S [V, K], per-token [T, K] / [T, V]
# ----------------------------------------------------------------------------

def _commit_core(fn, S0, u, kn, d, n):
    S0 = _c(S0, np.float64)
    V, K = S0.shape
    u = _c(u, np.float64).reshape(-1, V) if n > 0 else np.zeros((1, V))
    kn = _c(kn, np.float64).reshape(-1, K) if n > 0 else np.zeros((1, K))
    d = _c(d, np.float64).reshape(-1, K) if n > 0 else np.ones((1, K))
    if n > 0 and not (u.shape[0] >= n and kn.shape[0] >= n and d.shape[0] >= n):
        raise ValueError("fewer records than n")
    S = np.empty_like(S0)
    fn(K, V, int(n), _ptr(S0, _dp), _ptr(u, _dp), _ptr(kn, _dp), _ptr(d, _dp), _ptr(S, _dp))
    return S


def commit_seq(S0, u, kn, d, n):
    """Sequential replay S <- S diag(d_t) + u_t kn_t^T for t < n."""
    return _commit_core(_load().kda_o_commit_seq, S0, u, kn, d, n)


def commit_closed(S0, u, kn, d, n):
    """CHECK-ONLY closed form S_0 diag(D_n) + sum u_t (kn_t * P_t)^T."""
    return _commit_core(_load().kda_o_commit_closed, S0, u, kn, d, n)


def commit_logspace(S0, u, kn, d, n):
    """CHECK-ONLY log-space form exp(L_{n-1}), exp(L_{n-1} - L_t)."""
    return _commit_core(_load().kda_o_commit_logspace, S0, u, kn, d, n)


def _verify_core(fn, S, q, kn, v, d, beta, inplace):
    S = _c(S, np.float64)
    if not inplace:
        S = S.copy()
    V, K = S.shape
    q = _c(q, np.float64).reshape(-1, K)
    T = q.shape[0]
    kn = _c(kn, np.float64).reshape(T, K)
    v = _c(v, np.float64).reshape(T, V)
    d = _c(d, np.float64).reshape(T, K)
    beta = _c(beta, np.float64).reshape(T)
    o = np.empty((T, V))
    u = np.empty((T, V))
    fn(K, V, T, _ptr(S, _dp), _ptr(q, _dp), _ptr(kn, _dp), _ptr(v, _dp), _ptr(d, _dp),
       _ptr(beta, _dp), _ptr(o, _dp), _ptr(u, _dp))
    return o, u, S


def verify_seq(S, q, kn, v, d, beta):
    """Stock recurrence; returns (o [T,V], u [T,V], state after the last token)."""
    return _verify_core(_load().kda_o_verify_seq, S, q, kn, v, d, beta, False)


def verify_wy(S, q, kn, v, d, beta):
    """CHECK-ONLY chunked (WY) form from an unmodified S; returns (o, u)."""
    o, u, _ = _verify_core(_load().kda_o_verify_wy, S, q, kn, v, d, beta, False)
    return o, u


# ----------------------------------------------------------------------------
# Buffer-level operations (the library's semantics on host arrays)
# ----------------------------------------------------------------------------

def _items_arg(items):
    if items is None:
        return None, 0, None
    arr = _c(items, np.int64)
    return _ptr(arr, _i64p), arr.size, arr


def commit(*, heads, window, batch, key_dim=128, value_dim=128, state_bf16,
           state_layers, state_slot_strides, corr_layers, corr_row_strides,
           kg_layers, kg_row_strides, a_log, dt_bias, sources, commit_lens,
           destinations, boundaries=None, boundary_lens=None, record_rows=None,
           lower_bound, null_slot=0, items=None, threads=None):
    """RecoverSSM commit over (layer, request, head) items, in place on the
    per-layer flat state arrays. ``items`` optionally restricts the work to
    flattened item ids ``(l*B + b)*H + h``."""
    L = len(state_layers)
    sdt = np.uint16 if state_bf16 else np.float32
    for i, s in enumerate(state_layers):
        _check_inplace(s, sdt, f"state_layers[{i}]")
    corr_layers = [_c(c, np.float32) for c in corr_layers]
    kg_layers = [_c(k, np.uint16) for k in kg_layers]
    st_addr = (ctypes.c_void_p * L)(*[s.ctypes.data for s in state_layers])
    co_addr = (ctypes.c_void_p * L)(*[c.ctypes.data for c in corr_layers])
    kg_addr = (ctypes.c_void_p * L)(*[k.ctypes.data for k in kg_layers])
    sst = _c(state_slot_strides, np.int64)
    cst = _c(corr_row_strides, np.int64)
    kst = _c(kg_row_strides, np.int64)
    a_log = _c(a_log, np.float32)
    dt_bias = _c(dt_bias, np.float32)
    src = _c(sources, np.int32)
    lens = _c(commit_lens, np.int32)
    dst = _c(destinations, np.int32)
    bnd = None if boundaries is None else _c(boundaries, np.int32)
    blen = None if boundary_lens is None else _c(boundary_lens, np.int32)
    rows = None if record_rows is None else _c(record_rows, np.int32)
    ip, ni, _keep = _items_arg(items)
    _load().kda_o_commit(
        L, heads, window, batch, key_dim, value_dim, int(bool(state_bf16)),
        ctypes.cast(st_addr, _vp), _ptr(sst, _i64p), ctypes.cast(co_addr, _vp),
        _ptr(cst, _i64p), ctypes.cast(kg_addr, _vp), _ptr(kst, _i64p),
        _ptr(a_log, _fp), _ptr(dt_bias, _fp), _ptr(src, _i32p), _ptr(lens, _i32p),
        _ptr(dst, _i32p), _ptr(bnd, _i32p), _ptr(blen, _i32p), _ptr(rows, _i32p),
        float(lower_bound), int(null_slot), ip, ni,
        default_threads() if threads is None else int(threads))


def _verify_buf(fused, *, heads, tokens, batch, q, k, v, raw_g, raw_beta, a_log,
                dt_bias, lower_bound, state, state_slot_stride, state_indices,
                corr, kg, record_tokens, record_rows, pending, out, null_slot,
                key_dim, value_dim, items, threads, gate=None, norm_weight=None,
                norm_eps=1e-5, conv=None, query_start_loc=None, boundaries=None,
                boundary_lens=None, o_raw=None):
    state_bf16 = isinstance(state, np.ndarray) and state.dtype == np.uint16
    qsl = None if query_start_loc is None else _c(query_start_loc, np.int32)
    if (boundaries is None) != (boundary_lens is None):
        raise ValueError("boundaries and boundary_lens go together")
    bnd = None if boundaries is None else _c(boundaries, np.int32)
    blen = None if boundary_lens is None else _c(boundary_lens, np.int32)
    _check_inplace(state, np.uint16 if state_bf16 else np.float32, "state")
    _check_inplace(corr, np.float32, "corr")
    _check_inplace(kg, np.uint16, "kg")
    _check_inplace(out, np.uint16, "out")
    if o_raw is not None:
        _check_inplace(o_raw, np.float64, "o_raw")
        if o_raw.shape != out.shape:
            raise ValueError("o_raw must have the shape of out")
    q, k, v, g = (None if x is None else _c(x, np.uint16) for x in (q, k, v, raw_g))
    if conv is None:
        cx = cw = cb = cs = None
        cxs = css = ccs = cts = 0
        qsc = 0.0
    else:
        cx = _c(conv["x"], np.uint16)
        cxs = int(conv["x_row_stride"])
        cw = _c(conv["weight"], np.uint16)
        cb = None if conv.get("bias") is None else _c(conv["bias"], np.uint16)
        cs = conv["state"]
        _check_inplace(cs, np.uint16, "conv state")
        css, ccs, cts = (int(conv[n]) for n in ("slot_stride", "channel_stride",
                                                "tap_stride"))
        qsc = float(conv["q_scale"])
    rb = _c(raw_beta, np.uint16)
    a_log = _c(a_log, np.float32)
    dt_bias = _c(dt_bias, np.float32)
    slots = _c(state_indices, np.int32)
    rows = None if record_rows is None else _c(record_rows, np.int32)
    pend = None if pending is None else _c(pending, np.int32)
    ip, ni, _keep = _items_arg(items)
    gt = None if gate is None else _c(gate, np.uint16)
    nw = None if norm_weight is None else _c(norm_weight, np.float32)
    _load().kda_o_verify(
        heads, tokens, batch, key_dim, value_dim, _ptr(q, _u16p), _ptr(k, _u16p),
        _ptr(v, _u16p), _ptr(g, _u16p), _ptr(rb, _u16p), _ptr(a_log, _fp),
        _ptr(dt_bias, _fp), float(lower_bound), ctypes.c_void_p(state.ctypes.data),
        int(state_slot_stride),
        _ptr(slots, _i32p), int(null_slot), _ptr(corr, _fp), _ptr(kg, _u16p),
        int(record_tokens), _ptr(rows, _i32p), _ptr(pend, _i32p), int(fused),
        _ptr(out, _u16p), ip, ni, default_threads() if threads is None else int(threads),
        _ptr(gt, _u16p), _ptr(nw, _fp), float(norm_eps), int(state_bf16),
        _ptr(cx, _u16p), cxs, _ptr(cw, _u16p), _ptr(cb, _u16p), _ptr(cs, _u16p), css, ccs,
        cts, qsc, _ptr(qsl, _i32p), _ptr(bnd, _i32p), _ptr(blen, _i32p), _ptr(o_raw, _dp))


def verify(*, heads, tokens, batch, q, k, v, raw_g, raw_beta, a_log, dt_bias,
           lower_bound, state, state_slot_stride, state_indices, corr, kg,
           record_tokens, out, record_rows=None, null_slot=0, key_dim=128,
           value_dim=128, items=None, threads=None, gate=None, norm_weight=None,
           norm_eps=1e-5, query_start_loc=None, o_raw=None):
    """Stock verify: o (or, with gate and norm_weight, the gated RMSNorm of o)
    and records; the state is never written. The pool is FP32 (float32) or
    BF16 (uint16 bits), by the dtype of ``state``. ``o_raw`` (float64, the
    shape of ``out``), when given, receives o before any rounding."""
    _verify_buf(False, heads=heads, tokens=tokens, batch=batch, q=q, k=k, v=v,
                raw_g=raw_g, raw_beta=raw_beta, a_log=a_log, dt_bias=dt_bias,
                lower_bound=lower_bound, state=state, state_slot_stride=state_slot_stride,
                state_indices=state_indices, corr=corr, kg=kg, record_tokens=record_tokens,
                record_rows=record_rows, pending=None, out=out, null_slot=null_slot,
                key_dim=key_dim, value_dim=value_dim, items=items, threads=threads,
                gate=gate, norm_weight=norm_weight, norm_eps=norm_eps,
                query_start_loc=query_start_loc, o_raw=o_raw)


def fused_replay_verify(*, heads, tokens, batch, q, k, v, raw_g, raw_beta, a_log,
                        dt_bias, lower_bound, state, state_slot_stride, state_indices,
                        corr, kg, record_tokens, record_rows, pending, out, null_slot=0,
                        key_dim=128, value_dim=128, items=None, threads=None, gate=None,
                        norm_weight=None, norm_eps=1e-5, query_start_loc=None,
                        boundaries=None, boundary_lens=None, o_raw=None):
    """Replay the pending tokens from the old records (writing S_n when n > 0,
    and S_min(m, n) to the boundary slot with boundaries), then the stock verify
    from S_n, rewriting the records."""
    if record_rows is None or pending is None:
        raise ValueError("fused replay+verify needs record_rows and pending")
    _verify_buf(True, heads=heads, tokens=tokens, batch=batch, q=q, k=k, v=v,
                raw_g=raw_g, raw_beta=raw_beta, a_log=a_log, dt_bias=dt_bias,
                lower_bound=lower_bound, state=state, state_slot_stride=state_slot_stride,
                state_indices=state_indices, corr=corr, kg=kg, record_tokens=record_tokens,
                record_rows=record_rows, pending=pending, out=out, null_slot=null_slot,
                key_dim=key_dim, value_dim=value_dim, items=items, threads=threads,
                gate=gate, norm_weight=norm_weight, norm_eps=norm_eps,
                query_start_loc=query_start_loc, boundaries=boundaries,
                boundary_lens=boundary_lens, o_raw=o_raw)


def fused_conv_replay_verify(*, heads, tokens, batch, x, x_row_stride, conv_weight,
                             conv_state, conv_slot_stride, conv_channel_stride,
                             conv_tap_stride, q_scale, raw_g, raw_beta, a_log, dt_bias,
                             lower_bound, state, state_slot_stride, state_indices, corr, kg,
                             record_tokens, record_rows, pending, out, conv_bias=None,
                             null_slot=0, key_dim=128, value_dim=128, items=None,
                             threads=None, gate=None, norm_weight=None, norm_eps=1e-5,
                             boundaries=None, boundary_lens=None, o_raw=None):
    """The fused step with the convolution prologue: q, k, v are the SiLU of a
    4-tap causal convolution of x (rows of ``x_row_stride``: q | k | v parts of
    H*K channels each) over each channel's window in ``conv_state`` (uint16 BF16,
    element [slot*slot_stride + channel*channel_stride + i*tap_stride], i < RQ+2)
    read at offset max(n - 1, 0); q is then L2-normalised and scaled by
    ``q_scale``; the window is rewritten in place. ``conv_weight`` is [3, 4, H*K]
    BF16 bits, ``conv_bias`` [3*H*K] or None."""
    if record_rows is None or pending is None:
        raise ValueError("fused replay+verify needs record_rows and pending")
    conv = dict(x=x, x_row_stride=x_row_stride, weight=conv_weight, bias=conv_bias,
                state=conv_state, slot_stride=conv_slot_stride,
                channel_stride=conv_channel_stride, tap_stride=conv_tap_stride,
                q_scale=q_scale)
    _verify_buf(True, heads=heads, tokens=tokens, batch=batch, q=None, k=None, v=None,
                raw_g=raw_g, raw_beta=raw_beta, a_log=a_log, dt_bias=dt_bias,
                lower_bound=lower_bound, state=state, state_slot_stride=state_slot_stride,
                state_indices=state_indices, corr=corr, kg=kg, record_tokens=record_tokens,
                record_rows=record_rows, pending=pending, out=out, null_slot=null_slot,
                key_dim=key_dim, value_dim=value_dim, items=items, threads=threads,
                gate=gate, norm_weight=norm_weight, norm_eps=norm_eps, conv=conv,
                boundaries=boundaries, boundary_lens=boundary_lens, o_raw=o_raw)


def exp_f32(x):
    """The prologue's FP32 exp (Cody-Waite reduction, degree-7 Taylor)."""
    return float(_load().kda_o_exp_f32(ctypes.c_float(x)))


def silu_bf16(acc):
    """BF16 bits of SiLU of an FP32 pre-activation, by the prologue's fixed steps."""
    return int(_load().kda_o_silu_bf16(ctypes.c_float(acc)))


def conv_silu(seq, w, bias=0.0):
    """One channel's causal convolution + SiLU: seq = 3 taps then T inputs (BF16
    values as float32), w the 4 weights; returns T BF16 bit patterns."""
    seq = _c(seq, np.float32)
    w = _c(w, np.float32)
    T = seq.size - 3
    y = np.zeros(T, np.uint16)
    _load().kda_o_conv_silu(T, _ptr(seq, _fp), _ptr(w, _fp), ctypes.c_float(bias),
                            _ptr(y, _u16p))
    return y


def gate_projection(f_a, f_b, f_a_row_stride=None, tokens=None):
    """raw_g [N, D] BF16 bits = BF16(F_A F_B^T), f_b uint16 [D, R]. f_a is either
    a uint16 [N, R] array, or a flat uint16 buffer whose row t starts at
    t * f_a_row_stride (then ``tokens`` gives N)."""
    f_b = _c(f_b, np.uint16)
    D, R = f_b.shape
    f_a = _c(f_a, np.uint16)
    if f_a.ndim == 2:
        N, sa = f_a.shape[0], f_a.shape[1]
        assert sa >= R
    else:
        N, sa = int(tokens), int(f_a_row_stride)
        assert f_a.size >= (N - 1) * sa + R
    flat = f_a.reshape(-1)
    out = np.zeros((N, D), np.uint16)
    _load().kda_o_gate_projection(N, D, R, _ptr(flat, _u16p), sa, _ptr(f_b, _u16p),
                                  _ptr(out, _u16p))
    return out


def conv_offset(n):
    return int(_load().kda_o_conv_offset(int(n)))


def decay_buf(raw_g, a_log, dt_bias, lower_bound):
    """FP32 decays of a [N, H, K] BF16 raw-gate tensor."""
    g = _c(raw_g, np.uint16)
    N, H, K = g.shape
    a_log = _c(a_log, np.float32)
    dt_bias = _c(dt_bias, np.float32)
    out = np.empty((N, H, K), dtype=np.float32)
    _load().kda_o_decay_buf(N, H, K, _ptr(g, _u16p), _ptr(a_log, _fp), _ptr(dt_bias, _fp),
                            float(lower_bound), _ptr(out, _fp))
    return out


def defer(state_indices, commit_lens, record_rows, pending, eager=None, null_slot=0):
    """Defer step, in place on ``commit_lens`` and ``pending`` (int32 arrays)."""
    _check_inplace(commit_lens, np.int32, "commit_lens")
    _check_inplace(pending, np.int32, "pending")
    si = _c(state_indices, np.int32)
    rr = _c(record_rows, np.int32)
    eg = None if eager is None else _c(eager, np.int32)
    _load().kda_o_defer(si.size, _ptr(si, _i32p), _ptr(commit_lens, _i32p), _ptr(rr, _i32p),
                        _ptr(pending, _i32p), _ptr(eg, _i32p), int(null_slot))


def flush_plan(state_indices, record_rows, pending, spec_query_len, null_slot=0):
    """Flush plan; returns (commit_lens, final_indices, boundaries, boundary_lens)."""
    si = _c(state_indices, np.int32)
    rr = _c(record_rows, np.int32)
    pe = _c(pending, np.int32)
    B = si.size
    outs = [np.empty(B, dtype=np.int32) for _ in range(4)]
    _load().kda_o_flush_plan(B, int(spec_query_len), _ptr(si, _i32p), _ptr(rr, _i32p),
                             _ptr(pe, _i32p), *[_ptr(o, _i32p) for o in outs],
                             int(null_slot))
    return tuple(outs)
