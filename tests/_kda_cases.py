"""GPU-vs-oracle case runners for the parity tests.

Each runner takes host inputs (from the seeded generators in ``workloads``),
runs the library on the GPU through its C ABI (via the ``spec_decode_amd``
binding), runs the FP64 oracle on host copies of the same inputs, and compares
every output: within the tolerances of ``_compare`` where the call writes, and
bit-exact everywhere else (memory the call must not touch).

Nothing produced by the GPU is ever fed to the oracle.
"""
import sys

import numpy as np
import torch

import oracle
import workloads as W
from _compare import (assert_bf16_close, assert_exact, assert_f32_close, assert_gated_close,
                      bf16_tie_distance)

K = V = 128
DEV = "cuda:0"


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- transfers

def np_of(t: torch.Tensor) -> np.ndarray:
    """Host numpy copy; BF16 tensors become uint16 bit patterns."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def to_dev(x):
    if isinstance(x, np.ndarray):
        return dev_bf16(x) if x.dtype == np.uint16 else dev(x)
    return x.to(DEV)


# ---------------------------------------------------------------- commit

def commit_written(layers, H, B, Q, lens, src, dst, bnd, blen, rows, null_slot=0):
    """(layer, slot, head) pages a commit writes, and with which length."""
    out = {}
    for l in range(layers):
        for b in range(B):
            r = b if rows is None else rows[b]
            n = int(lens[b])
            if not (n > 0 and src[b] > null_slot and dst[b] > null_slot and r >= 0):
                continue
            for h in range(H):
                out[(l, int(dst[b]), h)] = "dst"
                if bnd is not None and blen[b] > 0 and bnd[b] > null_slot:
                    out[(l, int(bnd[b]), h)] = "bnd"
    return out


def pad_record_rows(records, pad, fill):
    """Flat copy of records [rows, ...] with `pad` extra elements after each
    row, set to `fill` (a value no correct read may see); returns (flat, row
    stride in elements)."""
    rows = records.shape[0]
    n = int(np.prod(records.shape[1:]))
    flat = np.full((rows, n + pad), fill, dtype=records.dtype)
    flat[:, :n] = records.reshape(rows, n)
    return flat.reshape(-1), n + pad


def run_commit_case(*, H, B, Q, bf16, layers_state, strides, corr_layers, kg_layers, a_log,
                    dt_bias, src, lens, dst, bnd=None, blen=None, rows=None,
                    lb=W.LOWER_BOUND, null_slot=0, label="commit", corr_strides=None,
                    kg_strides=None):
    """layers_state: per-layer flat host pools (uint16 bits or float32).
    corr_strides / kg_strides: per-layer record row strides in elements
    (default dense, H*Q*128 and H*Q*256)."""
    L = len(layers_state)
    corr_strides = [H * Q * V] * L if corr_strides is None else list(corr_strides)
    kg_strides = [H * Q * 2 * K] * L if kg_strides is None else list(kg_strides)
    announce(f"{label}: L={L} H={H} B={B} Q={Q} bf16={bf16} align={bnd is not None}")
    d_state = [to_dev(s) for s in layers_state]
    d_corr = [to_dev(c) for c in corr_layers]
    d_kg = [to_dev(k) for k in kg_layers]
    i32 = lambda a: None if a is None else dev(np.asarray(a, np.int32))
    import spec_decode_amd as kda
    kda.kda_commit(heads=H, window=Q, batch=B,
                   state_dtype=kda.KDA_STATE_BF16 if bf16 else kda.KDA_STATE_F32,
                   state_addrs=[t.data_ptr() for t in d_state], state_slot_strides=strides,
                   corr_addrs=[t.data_ptr() for t in d_corr],
                   corr_row_strides=corr_strides,
                   kg_addrs=[t.data_ptr() for t in d_kg],
                   kg_row_strides=kg_strides,
                   a_log=dev(np.asarray(a_log, np.float32)),
                   dt_bias=dev(np.asarray(dt_bias, np.float32)), sources=i32(src),
                   commit_lens=i32(lens), destinations=i32(dst), boundaries=i32(bnd),
                   boundary_lens=i32(blen), record_rows=i32(rows), lower_bound=lb,
                   null_slot=null_slot)
    torch.cuda.synchronize()
    gpu = [np_of(t) for t in d_state]
    ref = [s.copy() for s in layers_state]
    oracle.commit(heads=H, window=Q, batch=B, state_bf16=bf16, state_layers=ref,
                  state_slot_strides=strides, corr_layers=corr_layers,
                  corr_row_strides=corr_strides, kg_layers=kg_layers,
                  kg_row_strides=kg_strides, a_log=a_log, dt_bias=dt_bias,
                  sources=src, commit_lens=lens, destinations=dst, boundaries=bnd,
                  boundary_lens=blen, record_rows=rows, lower_bound=lb, null_slot=null_slot)
    written = commit_written(L, H, B, Q, lens, src, dst, bnd, blen, rows, null_slot)
    for l in range(L):
        mask = np.zeros(layers_state[l].size, dtype=bool)
        for (ll, slot, h) in written:
            if ll == l:
                o = slot * strides[l] + h * V * K
                mask[o:o + V * K] = True
        if bf16:
            assert_bf16_close(f"{label} layer {l} written pages", gpu[l][mask], ref[l][mask])
        else:
            assert_f32_close(f"{label} layer {l} written pages", gpu[l][mask], ref[l][mask])
        assert_exact(f"{label} layer {l} untouched", gpu[l][~mask], layers_state[l][~mask])
    return gpu, ref, written


# ---------------------------------------------------------------- verify / fused

def run_verify_case(*, fused, H, B, T, RQ, state, slots, corr, kg, a_log, dt_bias, win,
                    rows=None, pending=None, lb=W.LOWER_BOUND, null_slot=0, label="verify",
                    stride=None, check=True, gate=None, norm_weight=None, norm_eps=1e-5,
                    qsl=None, out_rows=None, bounds=None, blens=None):
    """All host arrays: state flat, float32 or uint16 BF16 bits (the pool's
    type), corr float32 [rows,H,RQ,V], kg uint16
    [rows,H,RQ,2K], win a dict of uint16 arrays (q, k, v, raw_g, raw_beta).
    qsl: optional [B+1] token offsets (variable-length windows); out_rows the
    row count of the activations and outputs (default B*T).
    Returns (gpu results, oracle results) as dicts of host arrays."""
    stride = H * V * K if stride is None else stride
    out_rows = B * T if out_rows is None else out_rows
    announce(f"{label}: fused={fused} H={H} B={B} T={T} RQ={RQ} state={state.dtype}")
    import spec_decode_amd as kda
    d = dict(state=to_dev(state), corr=dev(corr), kg=dev_bf16(kg),
             out=torch.full((out_rows, H * V), 0, dtype=torch.bfloat16, device=DEV))
    d["out"].view(torch.int16).fill_(0x7FFF)  # a sentinel: every element must be written
    args = dict(heads=H, tokens=T, batch=B, q=dev_bf16(win["q"]), k=dev_bf16(win["k"]),
                v=dev_bf16(win["v"]), raw_g=dev_bf16(win["raw_g"]),
                raw_beta=dev_bf16(win["raw_beta"]), a_log=dev(np.asarray(a_log, np.float32)),
                dt_bias=dev(np.asarray(dt_bias, np.float32)), lower_bound=lb,
                state=d["state"], state_slot_stride=stride,
                state_indices=dev(np.asarray(slots, np.int32)), corr=d["corr"], kg=d["kg"],
                record_tokens=RQ, out=d["out"], null_slot=null_slot,
                record_rows=None if rows is None else dev(np.asarray(rows, np.int32)),
                gate=None if gate is None else dev_bf16(gate),
                norm_weight=None if norm_weight is None else dev(np.asarray(norm_weight, np.float32)),
                norm_eps=norm_eps,
                query_start_loc=None if qsl is None else dev(np.asarray(qsl, np.int32)))
    if fused:
        i32 = lambda a: None if a is None else dev(np.asarray(a, np.int32))
        kda.kda_fused_replay_verify(pending=dev(np.asarray(pending, np.int32)),
                                    boundaries=i32(bounds), boundary_lens=i32(blens), **args)
    else:
        kda.kda_verify(**args)
    torch.cuda.synchronize()
    gpu = {k: np_of(v) for k, v in d.items()}
    ref = dict(state=state.copy(), corr=corr.copy(), kg=kg.copy(),
               out=np.full((out_rows, H * V), 0x7FFF, np.uint16))
    o_raw = None if gate is None else np.zeros((out_rows, H * V), np.float64)
    oargs = dict(heads=H, tokens=T, batch=B, q=win["q"], k=win["k"], v=win["v"],
                 raw_g=win["raw_g"], raw_beta=win["raw_beta"], a_log=a_log, dt_bias=dt_bias,
                 lower_bound=lb, state=ref["state"], state_slot_stride=stride,
                 state_indices=slots, corr=ref["corr"], kg=ref["kg"], record_tokens=RQ,
                 out=ref["out"], record_rows=rows, null_slot=null_slot, gate=gate,
                 norm_weight=norm_weight, norm_eps=norm_eps, query_start_loc=qsl, o_raw=o_raw)
    if fused:
        oracle.fused_replay_verify(pending=pending, boundaries=bounds, boundary_lens=blens,
                                   **oargs)
    else:
        oracle.verify(**oargs)
    if check:
        compare_verify(gpu, ref, dict(state=state, corr=corr, kg=kg), fused=fused, H=H, B=B,
                       T=T, RQ=RQ, slots=slots, rows=rows, pending=pending, stride=stride,
                       null_slot=null_slot, label=label, o_raw=o_raw, qsl=qsl,
                       bounds=bounds, blens=blens)
    return gpu, ref


def window_lengths(B, T, qsl):
    """Each request's window length: T, or clamp(qsl[b+1] - qsl[b], 0, T)."""
    if qsl is None:
        return [T] * B
    return [min(max(int(qsl[b + 1]) - int(qsl[b]), 0), T) for b in range(B)]


def verify_written(*, fused, H, B, T, RQ, slots, rows, pending, stride, null_slot, n_state,
                   corr_shape, qsl=None, bounds=None, blens=None):
    smask = np.zeros(n_state, dtype=bool)
    cmask = np.zeros(corr_shape, dtype=bool)
    lens = window_lengths(B, T, qsl)
    for b in range(B):
        if slots[b] <= null_slot or lens[b] == 0:
            continue
        r = b if rows is None else int(rows[b])
        if r >= 0:
            cmask[r, :, :lens[b], :] = True
            if fused:
                n = min(max(int(pending[r]), 0), RQ)
                if n > 0:
                    pages = [int(slots[b])]
                    if bounds is not None and bounds[b] > null_slot and blens[b] > 0:
                        pages.append(int(bounds[b]))
                    for sl in pages:
                        for h in range(H):
                            o = sl * stride + h * V * K
                            smask[o:o + V * K] = True
    return smask, cmask


def compare_verify(gpu, ref, orig, *, fused, H, B, T, RQ, slots, rows, pending, stride,
                   null_slot, label, o_raw=None, qsl=None, bounds=None, blens=None):
    """o_raw: the oracle's unrounded o when the gated output stage ran (its
    near-tie elements are allowed a second ulp), else None."""
    smask, cmask = verify_written(fused=fused, H=H, B=B, T=T, RQ=RQ, slots=slots, rows=rows,
                                  pending=pending, stride=stride, null_slot=null_slot,
                                  n_state=orig["state"].size, corr_shape=orig["corr"].shape,
                                  qsl=qsl, bounds=bounds, blens=blens)
    if o_raw is not None:
        assert_gated_close(f"{label} gated out", gpu["out"], ref["out"], o_raw)
    else:
        assert_bf16_close(f"{label} out", gpu["out"], ref["out"])
    assert_exact(f"{label} key/gate records", gpu["kg"], ref["kg"])
    assert_f32_close(f"{label} corrections (written)", gpu["corr"][cmask], ref["corr"][cmask])
    assert_exact(f"{label} corrections (untouched)", gpu["corr"][~cmask], orig["corr"][~cmask])
    if orig["state"].dtype == np.uint16:  # a BF16 pool
        assert_bf16_close(f"{label} state (replayed)", gpu["state"][smask], ref["state"][smask])
    else:
        assert_f32_close(f"{label} state (replayed)", gpu["state"][smask], ref["state"][smask])
    assert_exact(f"{label} state (untouched)", gpu["state"][~smask], orig["state"][~smask])


def window_np(win: "W.Window"):
    return {name: np_of(getattr(win, name)) for name in ("q", "k", "v", "raw_g", "raw_beta")}


# ---------------------------------------------------------------- fused + convolution

CONV_LAYOUTS = ("dim_first", "window_major", "dim_first_padded", "dim_first_slot_pad",
                "window_major_padded", "window_major_odd")


def conv_pool_layout(S, H, W, dim_first=True, layout=None):
    """Strides (slot, channel, tap) of a window pool, in elements: [S, 3HK, W]
    (dim-first, the packed layout) or [S, W, 3HK] (window-major); layout, when
    given, also names 'dim_first_padded' (channel stride W + 1) and
    'dim_first_slot_pad' (slot stride 3HK*W + 4, not a multiple of 8), which the
    library serves with its strided code, 'window_major_padded' (rows of 3HK + 8
    elements, still 16-byte aligned: the window-major code) and
    'window_major_odd' (rows of 3HK + 3 elements: the strided code)."""
    hk3 = 3 * H * K
    layout = layout or ("dim_first" if dim_first else "window_major")
    return {"dim_first": (hk3 * W, W, 1), "window_major": (hk3 * W, 1, hk3),
            "dim_first_padded": (hk3 * (W + 1), W + 1, 1),
            "dim_first_slot_pad": (hk3 * W + 4, W, 1),
            "window_major_padded": ((hk3 + 8) * W, 1, hk3 + 8),
            "window_major_odd": ((hk3 + 3) * W, 1, hk3 + 3)}[layout]


def conv_pool_build(win, strides, seed):
    """A flat uint16 pool holding win [S, 3HK, W] (window values as BF16 bits) at
    the given strides; the elements no window covers hold seeded random bits,
    so that a test can see them stay untouched."""
    S, C, Wn = win.shape
    ss, cs, ts = strides
    n = (S - 1) * ss + (C - 1) * cs + (Wn - 1) * ts + 1
    pool = np.random.default_rng(seed).integers(0, 1 << 16, n, dtype=np.uint16)
    idx = (np.arange(S)[:, None, None] * ss + np.arange(C)[None, :, None] * cs +
           np.arange(Wn)[None, None, :] * ts)
    pool[idx] = win
    return pool


def conv_written(slots, H, RQ, T, strides, null_slot, n_elems):
    """Mask of the window entries a call rewrites: 2 + T per (live slot, column)."""
    m = np.zeros(n_elems, dtype=bool)
    ss, cs, ts = strides
    cols = np.arange(3 * H * K)
    for s in slots:
        if s <= null_slot:
            continue
        for i in range(2 + T):
            m[int(s) * ss + cols * cs + i * ts] = True
    return m


def silu_keys_plain(*, H, T, RQ, x, pitch, conv_w, conv_b, pool, strides, slot, n, tok0):
    """The recorded keys of one item by the plain definition, in FP64: the k
    part's causal convolution of its 3 window taps (at offset max(n - 1, 0))
    and T inputs, plus the bias, then SiLU(a) = a / (1 + e^-a), rounded once to
    BF16 (fused page, KdaFused.kernel and KdaFused.silu). Returns (bits [H, T,
    K], near [H, T, K]): near marks values within FP32 evaluation error of a
    BF16 rounding boundary, where the kernel's FP32 steps may round to the other
    neighbour: 2^-18 |y| for the exp and divide, plus 2^-21 times the sum of the
    absolute terms of the pre-activation for its FP32 sum (which may cancel)."""
    hk = H * K
    ss, cs, ts = strides
    off = max(n - 1, 0)
    x = np.asarray(x).reshape(-1)
    pool = np.asarray(pool).reshape(-1)
    conv_w = np.asarray(conv_w).reshape(3, 4, hk)
    conv_b = None if conv_b is None else np.asarray(conv_b).reshape(-1)
    cols = hk + np.arange(hk)  # the k part
    f = lambda b: (np.asarray(b, np.uint32) << 16).view(np.float32).astype(np.float64)
    taps = np.stack([f(pool[slot * ss + cols * cs + (off + i) * ts]) for i in range(3)])
    xin = np.stack([f(x[(tok0 + t) * pitch + cols]) for t in range(T)])
    seq = np.concatenate([taps, xin])  # [3 + T, hk]
    w = f(conv_w[1])  # [4, hk]
    bias = f(conv_b[cols]) if conv_b is not None else np.zeros(hk)
    pre = bias + sum(w[i] * seq[i:i + T] for i in range(4))  # [T, hk]
    mag = np.abs(bias) + sum(np.abs(w[i] * seq[i:i + T]) for i in range(4))
    y = pre / (1.0 + np.exp(-pre))
    bits = oracle.round_bf16(y)
    near = bf16_tie_distance(y) <= 2.0 ** -18 * np.abs(y) + 2.0 ** -21 * mag
    tr = lambda a: a.reshape(T, H, K).transpose(1, 0, 2)
    return tr(bits), tr(near)


def check_conv_keys_plain(label, gpu_kg, *, H, T, RQ, x, pitch, conv_w, conv_b, pool, strides,
                          slots, rows, pending, null_slot=0, tok_of=None):
    """The GPU's recorded keys of every live item against silu_keys_plain: bit
    for bit outside the near-tie band, within one ulp inside it. Returns the
    share of keys in the band. tok_of(b) gives request b's first token row
    (default b * T)."""
    n_near = n_all = 0
    for b in range(len(slots)):
        r = int(rows[b])
        if slots[b] <= null_slot or r < 0:
            continue
        n = min(max(int(pending[r]), 0), RQ)
        want, near = silu_keys_plain(H=H, T=T, RQ=RQ, x=x, pitch=pitch, conv_w=conv_w,
                                     conv_b=conv_b, pool=pool, strides=strides,
                                     slot=int(slots[b]), n=n,
                                     tok0=b * T if tok_of is None else tok_of(b))
        got = gpu_kg[r, :, :T, :K]
        d = np.abs(_ordered(got) - _ordered(want))
        bad = (d > 1) | ((d == 1) & ~near)
        assert not bad.any(), (f"{label} keys vs plain SiLU, request {b}: "
                               f"{int(bad.sum())} of {bad.size} differ outside the near-tie band")
        n_near += int(near.sum())
        n_all += near.size
    return n_near / max(n_all, 1)


def _ordered(bits):
    b = np.asarray(bits, np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)


def run_conv_case(*, H, B, T, RQ, state, slots, corr, kg, a_log, dt_bias, raw_g, raw_beta,
                  x, pitch, conv_w, conv_b, pool, strides, rows, pending,
                  lb=W.LOWER_BOUND, null_slot=0, label="fused conv", gate=None,
                  norm_weight=None, norm_eps=1e-5, q_scale=K ** -0.5, bounds=None, blens=None):
    """kda_fused_conv_replay_verify on the GPU and the oracle on host copies.
    Host arrays: x uint16 [B*T, pitch], conv_w uint16 [3, 4, HK], conv_b uint16
    [3HK] or None, pool uint16 flat window pool with the given strides; the
    rest as run_verify_case."""
    import spec_decode_amd as kda
    stride = H * V * K
    announce(f"{label}: H={H} B={B} T={T} RQ={RQ} state={state.dtype} strides={strides}")
    d = dict(state=to_dev(state), corr=dev(corr), kg=dev_bf16(kg), pool=dev_bf16(pool),
             out=torch.zeros((B * T, H * V), dtype=torch.bfloat16, device=DEV))
    d["out"].view(torch.int16).fill_(0x7FFF)
    kda.kda_fused_conv_replay_verify(
        heads=H, tokens=T, batch=B, x=dev_bf16(x), x_row_stride=pitch,
        conv_weight=dev_bf16(conv_w), conv_bias=None if conv_b is None else dev_bf16(conv_b),
        conv_state=d["pool"], conv_slot_stride=strides[0], conv_channel_stride=strides[1],
        conv_tap_stride=strides[2], q_scale=q_scale, raw_g=dev_bf16(raw_g),
        raw_beta=dev_bf16(raw_beta), a_log=dev(np.asarray(a_log, np.float32)),
        dt_bias=dev(np.asarray(dt_bias, np.float32)), lower_bound=lb, state=d["state"],
        state_slot_stride=stride, state_indices=dev(np.asarray(slots, np.int32)),
        corr=d["corr"], kg=d["kg"], record_tokens=RQ,
        record_rows=dev(np.asarray(rows, np.int32)),
        pending=dev(np.asarray(pending, np.int32)), out=d["out"], null_slot=null_slot,
        gate=None if gate is None else dev_bf16(gate),
        norm_weight=None if norm_weight is None else dev(np.asarray(norm_weight, np.float32)),
        norm_eps=norm_eps,
        boundaries=None if bounds is None else dev(np.asarray(bounds, np.int32)),
        boundary_lens=None if blens is None else dev(np.asarray(blens, np.int32)))
    torch.cuda.synchronize()
    gpu = {k: np_of(v) for k, v in d.items()}
    ref = dict(state=state.copy(), corr=corr.copy(), kg=kg.copy(), pool=pool.copy(),
               out=np.full((B * T, H * V), 0x7FFF, np.uint16))
    o_raw = None if gate is None else np.zeros((B * T, H * V), np.float64)
    oracle.fused_conv_replay_verify(
        heads=H, tokens=T, batch=B, x=x, x_row_stride=pitch, conv_weight=conv_w,
        conv_bias=conv_b, conv_state=ref["pool"], conv_slot_stride=strides[0],
        conv_channel_stride=strides[1], conv_tap_stride=strides[2], q_scale=q_scale,
        raw_g=raw_g, raw_beta=raw_beta, a_log=a_log, dt_bias=dt_bias, lower_bound=lb,
        state=ref["state"], state_slot_stride=stride, state_indices=slots, corr=ref["corr"],
        kg=ref["kg"], record_tokens=RQ, record_rows=rows, pending=pending, out=ref["out"],
        null_slot=null_slot, gate=gate, norm_weight=norm_weight, norm_eps=norm_eps,
        boundaries=bounds, boundary_lens=blens, o_raw=o_raw)
    compare_verify(gpu, ref, dict(state=state, corr=corr, kg=kg), fused=True, H=H, B=B, T=T,
                   RQ=RQ, slots=slots, rows=rows, pending=pending, stride=stride,
                   null_slot=null_slot, label=label, o_raw=o_raw, bounds=bounds,
                   blens=blens)
    cm = conv_written(slots, H, RQ, T, strides, null_slot, pool.size)
    assert_exact(f"{label} windows (written)", gpu["pool"][cm], ref["pool"][cm])
    assert_exact(f"{label} windows (untouched)", gpu["pool"][~cm], pool[~cm])
    share = check_conv_keys_plain(label, gpu["kg"], H=H, T=T, RQ=RQ, x=x, pitch=pitch,
                                  conv_w=conv_w, conv_b=conv_b, pool=pool, strides=strides,
                                  slots=slots, rows=rows, pending=pending, null_slot=null_slot)
    announce(f"{label}: recorded keys match the plain FP64 SiLU ({100 * share:.3f}% near a tie)")
    return gpu, ref


# ---------------------------------------------------------------- sampled full-size checks

def sampled_fused_oracle(*, R, H, T, RQ, state_pages, slots, rows, pending_row, corr, kg,
                         win, a_log, dt_bias, lb, qsl=None, bounds=None, blens=None,
                         state_dtype=np.float32):
    """The oracle on a compact copy of requests R of a large fused call: request j
    of the copy owns slot j + 1 (and, with boundaries, slot nR + 1 + j) and
    record row j. state_pages(slot) returns a slot's host page set; win holds
    the full call's activation rows (indexed through qsl when given).
    Returns the copy's (state, corr, kg, out, token rows per request)."""
    nR = len(R)
    page = H * V * K
    n_slots = nR + 1 + (nR if bounds is not None else 0)
    m_state = np.zeros(n_slots * page, state_dtype)
    m_slots = np.array([j + 1 if slots[b] > 0 else 0 for j, b in enumerate(R)], np.int32)
    m_rows = np.array([j if rows[b] >= 0 else -1 for j, b in enumerate(R)], np.int32)
    m_corr = np.zeros((nR, H, RQ, V), np.float32)
    m_kg = np.zeros((nR, H, RQ, 2 * K), np.uint16)
    m_pend = np.zeros(nR, np.int32)
    m_bnd = m_blen = None
    if bounds is not None:
        m_bnd = np.array([nR + 1 + j if bounds[b] > 0 else 0 for j, b in enumerate(R)], np.int32)
        m_blen = np.array([blens[b] for b in R], np.int32)
    for j, b in enumerate(R):
        if slots[b] > 0:
            m_state[(j + 1) * page:(j + 2) * page] = state_pages(int(slots[b]))
        if bounds is not None and bounds[b] > 0:
            m_state[(nR + 1 + j) * page:(nR + 2 + j) * page] = state_pages(int(bounds[b]))
        if rows[b] >= 0:
            m_corr[j], m_kg[j], m_pend[j] = corr[rows[b]], kg[rows[b]], pending_row[rows[b]]
    lens = window_lengths(len(slots), T, qsl)
    toks = [np.arange(b * T, b * T + T) if qsl is None else
            np.arange(int(qsl[b]), int(qsl[b]) + lens[b]) for b in R]
    m_qsl = None
    if qsl is not None:
        m_qsl = np.zeros(nR + 1, np.int32)
        m_qsl[1:] = np.cumsum([lens[b] for b in R])
    tok = np.concatenate(toks) if toks else np.zeros(0, np.int64)
    m_win = {k: np.ascontiguousarray(v[tok]) for k, v in win.items()}
    m_out = np.zeros((max(len(tok), 1), H * V), np.uint16)
    oracle.fused_replay_verify(heads=H, tokens=T, batch=nR, q=m_win["q"], k=m_win["k"],
                               v=m_win["v"], raw_g=m_win["raw_g"], raw_beta=m_win["raw_beta"],
                               a_log=a_log, dt_bias=dt_bias, lower_bound=lb, state=m_state,
                               state_slot_stride=page, state_indices=m_slots, corr=m_corr,
                               kg=m_kg, record_tokens=RQ, record_rows=m_rows, pending=m_pend,
                               out=m_out, query_start_loc=m_qsl, boundaries=m_bnd,
                               boundary_lens=m_blen)
    return dict(state=m_state, corr=m_corr, kg=m_kg, out=m_out, toks=toks, slots=m_slots,
                bounds=m_bnd)
