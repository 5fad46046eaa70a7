"""GPU parity over seeded random combinations of the verify and fused options
(window, record capacity, heads, batch, FP32/BF16 pool, gated output stage,
variable-length windows, boundary stores, padded slot strides, null slots,
missing record rows, edge pending counts, key norms, the decay's lower
bound), each against the FP64 oracle
element by element. The single-option tests cover each option alone; these
cover them together."""
import numpy as np
import pytest
import torch

import workloads as W
from _kda_cases import (CONV_LAYOUTS, conv_pool_build, conv_pool_layout, run_conv_case,
                        run_verify_case, window_np)

pytestmark = pytest.mark.gpu

K = V = 128


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import spec_decode_amd  # noqa: F401  (fails loudly without libkda.so)

    torch.cuda.init()
    yield


# The decay's lower bound, drawn apart from the other draws (so they stay as
# they were): the workloads' -5 half the time, else a degenerate end (0: no
# decay; -60: decay products underflow) or a mild -0.5.
LOWER_BOUNDS = (-5.0, -5.0, -5.0, 0.0, -0.5, -60.0)


def _lower_bound(seed):
    return float(np.random.default_rng(seed).choice(LOWER_BOUNDS))


def _draw(seed):
    r = np.random.default_rng(seed)
    T = int(r.integers(1, 9))
    RQ = int(r.integers(T, 9))
    H = int(r.integers(1, 5))
    B = int(r.integers(1, 10))
    return r, dict(T=T, RQ=RQ, H=H, B=B, bf16=bool(r.integers(2)), gated=bool(r.integers(2)),
                   fused=bool(r.integers(3) > 0), varlen=bool(r.integers(2)),
                   align=bool(r.integers(2)), pad=int(r.integers(2)))


@pytest.mark.parametrize("seed", list(range(80)))
def test_random_combination(seed):
    r, c = _draw(2000 + seed)
    T, RQ, H, B, bf16 = c["T"], c["RQ"], c["H"], c["B"], c["bf16"]
    fused, align = c["fused"], c["fused"] and c["align"]
    S = 2 * B + 3
    page = H * V * K
    stride = page + (8 * int(r.integers(1, 40)) if c["pad"] else 0)
    g = W._gen(3000 + seed)
    a_log, dtb = W.draw_gate_params(g, 1, H)
    corr, kg = W.draw_records(g, B, H, RQ)
    state = W.draw_state(4000 + seed, S * stride, torch.float32)
    state = W.bits(state.to(torch.bfloat16)) if bf16 else state.numpy().copy()
    perm = r.permutation(np.arange(1, S)).astype(np.int32)
    slots = perm[:B].copy()
    bounds = perm[B:2 * B].copy()
    for b in range(B):
        if r.random() < 0.15:
            slots[b] = 0
        if r.random() < 0.3:
            bounds[b] = 0
    rows = r.permutation(B).astype(np.int32)
    for b in range(B):
        if r.random() < 0.15:
            rows[b] = -1
    pending = r.integers(-1, RQ + 2, B).astype(np.int32)
    blens = r.integers(0, RQ + 2, B).astype(np.int32)
    qsl = None
    out_rows = B * T
    win = window_np(W.draw_window(g, B, T, H))
    # Half the combinations also rescale every key, in the window and in the
    # records, to norms from W.KEY_NORMS (drawn apart, so the other draws stay).
    keyscale = bool(np.random.default_rng(2500 + seed).integers(2))
    if keyscale:
        kg = W.rescale_record_keys(W._gen(2600 + seed), kg)
    if c["varlen"]:
        lens = r.integers(0, T + 2, B)
        qsl = np.zeros(B + 1, np.int32)
        qsl[1:] = np.cumsum(lens)
        out_rows = int(qsl[-1]) + 1
        big = window_np(W.draw_window(g, max(out_rows // T + 1, B), T, H))
        win = {k: np.ascontiguousarray(v[:out_rows]) for k, v in big.items()}
    if keyscale:
        kt = torch.from_numpy(win["k"].view(np.int16)).view(torch.bfloat16)
        win["k"] = W.bits(W.rescale_keys(W._gen(2700 + seed), kt))
        c["keyscale"] = True
    kw = {}
    if c["gated"]:
        gate, weight, eps = W.draw_output_stage(W._gen(5000 + seed), max(out_rows // T + 1, B),
                                                T, H)
        kw = dict(gate=np.ascontiguousarray(W.bits(gate)[:out_rows]),
                  norm_weight=weight.numpy(), norm_eps=eps)
    if align:
        kw.update(bounds=bounds, blens=blens)
    lb = _lower_bound(2800 + seed)
    run_verify_case(fused=fused, H=H, B=B, T=T, RQ=RQ, state=state, slots=slots,
                    corr=corr.numpy().copy(), kg=W.bits(kg), a_log=a_log[0].numpy(),
                    dt_bias=dtb[0].numpy(), win=win, rows=rows,
                    pending=pending if fused else None, stride=stride, qsl=qsl,
                    out_rows=out_rows, lb=lb, label=f"combination {seed}: {c} lb={lb}", **kw)


@pytest.mark.parametrize("seed", list(range(32)))
def test_random_conv_combination(seed):
    r, c = _draw(6000 + seed)
    T, RQ, H, B, bf16 = c["T"], c["RQ"], c["H"], c["B"], c["bf16"]
    S = 2 * B + 3
    page = H * V * K
    g = W._gen(7000 + seed)
    a_log, dtb = W.draw_gate_params(g, 1, H)
    corr, kg = W.draw_records(g, B, H, RQ)
    state = W.draw_state(8000 + seed, S * page, torch.float32)
    state = W.bits(state.to(torch.bfloat16)) if bf16 else state.numpy().copy()
    perm = r.permutation(np.arange(1, S)).astype(np.int32)
    slots = perm[:B].copy()
    bounds = perm[B:2 * B].copy()
    for b in range(B):
        if r.random() < 0.15:
            slots[b] = 0
    rows = r.permutation(B).astype(np.int32)
    for b in range(B):
        if r.random() < 0.15:
            rows[b] = -1
    pending = r.integers(-1, RQ + 2, B).astype(np.int32)
    blens = r.integers(0, RQ + 2, B).astype(np.int32)
    win = window_np(W.draw_window(g, B, T, H))
    cv = W.draw_conv_inputs(W._gen(9000 + seed), B, T, H, RQ, S)
    layout = CONV_LAYOUTS[int(r.integers(len(CONV_LAYOUTS)))]
    strides = conv_pool_layout(S, H, RQ + 2, layout=layout)
    pool = conv_pool_build(W.bits(cv.window), strides, 9700 + seed)
    kw = {}
    if c["gated"]:
        gate, weight, eps = W.draw_output_stage(W._gen(9500 + seed), B, T, H)
        kw = dict(gate=W.bits(gate), norm_weight=weight.numpy(), norm_eps=eps)
    if c["align"]:
        kw.update(bounds=bounds, blens=blens)
    run_conv_case(H=H, B=B, T=T, RQ=RQ, state=state, slots=slots, corr=corr.numpy().copy(),
                  kg=W.bits(kg), a_log=a_log[0].numpy(), dt_bias=dtb[0].numpy(),
                  raw_g=win["raw_g"], raw_beta=win["raw_beta"], x=W.bits(cv.x), pitch=cv.pitch,
                  conv_w=W.bits(cv.weight),
                  conv_b=W.bits(cv.bias) if r.integers(2) else None, pool=pool,
                  strides=strides, rows=rows, pending=pending, lb=_lower_bound(6800 + seed),
                  label=f"conv combination {seed}: {c} {layout} lb={_lower_bound(6800 + seed)}",
                  **kw)


@pytest.mark.parametrize("seed", list(range(32)))
def test_random_commit_combination(seed):
    """kda_commit over random layer counts (up to 18, more than one launch),
    windows, pool types, padded per-layer strides, padded record rows, in-place
    or src -> dst, boundaries, record rows and lengths (0, negative, above the
    window)."""
    from _kda_cases import pad_record_rows, run_commit_case
    r = np.random.default_rng(10000 + seed)
    L = int(r.choice([1, 1, 2, 3, 5, 17, 18]))
    H = int(r.integers(1, 4))
    B = int(r.integers(1, 8))
    Q = int(r.integers(1, 9))
    bf16 = bool(r.integers(2))
    inplace = bool(r.integers(2))
    align = bool(r.integers(2))
    S = 3 * B + 2
    page = H * V * K
    g = W._gen(11000 + seed)
    strides = [page + 8 * int(r.integers(0, 20)) for _ in range(L)]
    dt = torch.bfloat16 if bf16 else torch.float32
    states, corrs, kgs = [], [], []
    for l in range(L):
        st = W.draw_state(12000 + seed * 32 + l, S * strides[l], dt)
        states.append(W.bits(st) if bf16 else st.numpy().copy())
        c, k = W.draw_records(g, B, H, Q)
        corrs.append(c.numpy().copy())
        kgs.append(W.bits(k))
    a_log, dtb = W.draw_gate_params(g, L, H)
    perm = r.permutation(np.arange(1, S)).astype(np.int32)
    src = perm[:B].copy()
    dst = src.copy() if inplace else perm[B:2 * B].copy()
    bnd = perm[2 * B:3 * B].copy()
    for b in range(B):
        if r.random() < 0.15:
            src[b] = 0
        if r.random() < 0.25:
            bnd[b] = 0
    lens = r.integers(-1, Q + 3, B).astype(np.int32)
    blen = r.integers(-1, Q + 3, B).astype(np.int32)
    rows = None
    if r.integers(2):
        rows = r.permutation(B).astype(np.int32)
        for b in range(B):
            if r.random() < 0.15:
                rows[b] = -1
    # Half the combinations pad the record rows (drawn apart, so the other draws
    # stay); the padding holds NaN, which no correct read may see.
    r2 = np.random.default_rng(10900 + seed)
    corr_strides = kg_strides = None
    if r2.integers(2):
        padded = [pad_record_rows(corrs[l], 4 * int(r2.integers(1, 9)), np.float32(np.nan))
                  for l in range(L)]
        corrs, corr_strides = [x[0] for x in padded], [x[1] for x in padded]
        padded = [pad_record_rows(kgs[l], 8 * int(r2.integers(1, 9)), np.uint16(0x7FC0))
                  for l in range(L)]
        kgs, kg_strides = [x[0] for x in padded], [x[1] for x in padded]
    run_commit_case(H=H, B=B, Q=Q, bf16=bf16, layers_state=states, strides=strides,
                    corr_layers=corrs, kg_layers=kgs, a_log=a_log.numpy(), dt_bias=dtb.numpy(),
                    corr_strides=corr_strides, kg_strides=kg_strides,
                    src=src, lens=lens, dst=dst, bnd=bnd if align else None,
                    blen=blen if align else None, rows=rows, lb=_lower_bound(10800 + seed),
                    label=f"commit combination {seed}: L={L} H={H} B={B} Q={Q} bf16={bf16} "
                          f"inplace={inplace} align={align} lb={_lower_bound(10800 + seed)}")


@pytest.mark.parametrize("seed", list(range(6)))
def test_random_commit_combination_streaming(seed):
    """The same draws at a size whose FP32 source pages exceed the 256 MB MALL
    (H=64, B=66: 264 MiB per layer), so kda_commit runs its streaming FP32
    kernel (pages through LDS, folded on the matrix cores), against the full
    oracle: one or two layers, any window, in place or not, boundaries, record
    rows, padded record rows holding NaN, lengths 0, negative and above the
    window."""
    from _kda_cases import pad_record_rows, run_commit_case
    r = np.random.default_rng(13000 + seed)
    L = int(r.choice([1, 2]))
    H, B = 64, 66
    Q = int(r.integers(1, 9))
    inplace = bool(r.integers(2))
    align = bool(r.integers(2))
    S = 3 * B + 2
    page = H * V * K
    assert B * page * 4 > 256 << 20
    g = W._gen(13100 + seed)
    strides = [page + 8 * int(r.integers(0, 20)) for _ in range(L)]
    states, corrs, kgs = [], [], []
    for l in range(L):
        states.append(W.draw_state(13200 + seed * 4 + l, S * strides[l], torch.float32).numpy())
        c, k = W.draw_records(g, B, H, Q)
        corrs.append(c.numpy().copy())
        kgs.append(W.bits(k))
    a_log, dtb = W.draw_gate_params(g, L, H)
    perm = r.permutation(np.arange(1, S)).astype(np.int32)
    src = perm[:B].copy()
    dst = src.copy() if inplace else perm[B:2 * B].copy()
    bnd = perm[2 * B:3 * B].copy()
    for b in range(B):
        if r.random() < 0.15:
            src[b] = 0
        if r.random() < 0.25:
            bnd[b] = 0
    lens = r.integers(-1, Q + 3, B).astype(np.int32)
    blen = r.integers(-1, Q + 3, B).astype(np.int32)
    rows = None
    if r.integers(2):
        rows = r.permutation(B).astype(np.int32)
        for b in range(B):
            if r.random() < 0.15:
                rows[b] = -1
    corr_strides = kg_strides = None
    if r.integers(2):
        padded = [pad_record_rows(corrs[l], 4 * int(r.integers(1, 9)), np.float32(np.nan))
                  for l in range(L)]
        corrs, corr_strides = [x[0] for x in padded], [x[1] for x in padded]
        padded = [pad_record_rows(kgs[l], 8 * int(r.integers(1, 9)), np.uint16(0x7FC0))
                  for l in range(L)]
        kgs, kg_strides = [x[0] for x in padded], [x[1] for x in padded]
    lb = _lower_bound(13300 + seed)
    run_commit_case(H=H, B=B, Q=Q, bf16=False, layers_state=states, strides=strides,
                    corr_layers=corrs, kg_layers=kgs, a_log=a_log.numpy(), dt_bias=dtb.numpy(),
                    corr_strides=corr_strides, kg_strides=kg_strides,
                    src=src, lens=lens, dst=dst, bnd=bnd if align else None,
                    blen=blen if align else None, rows=rows, lb=lb,
                    label=f"streaming commit combination {seed}: L={L} Q={Q} inplace={inplace} "
                          f"align={align} lb={lb}")
