"""The step's variants at the large decode batch's size (H=64, B=512, q=8, a
2 GiB FP32 pool), in the launch configuration the benchmark times: the gated
RMSNorm output stage, the convolution prologue over a packed dim-first and
over a window-major window pool, and the stock verify. Sampled requests (null slots, a missing record row, every pending
count) are recomputed by the oracle on compact copies; pages nobody writes are
compared bit for bit over the whole pool."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _compare import assert_bf16_close, assert_exact, assert_f32_close, assert_gated_close
from _kda_cases import (DEV, announce, check_conv_keys_plain, conv_pool_layout, dev, dev_bf16,
                        np_of, window_np)

pytestmark = pytest.mark.gpu
K = V = 128
H, B, T, RQ, S = 64, 512, 8, 8, 520


def _plan(seed):
    g = W._gen(seed)
    perm = (W.permutation(g, S - 1) + 1).numpy()
    slots = perm[:B].copy()
    slots[::53] = 0
    rows = W.permutation(g, B).numpy()
    rows[5::97] = -1
    pending_row = W.uniform_int(g, 0, RQ, B).numpy()
    a_log, dtb = W.draw_gate_params(g, 1, H)
    corr, kg = W.draw_records(g, B, H, RQ)
    return g, slots, rows, pending_row, a_log[0].numpy(), dtb[0].numpy(), corr.numpy(), W.bits(kg)


def _sample(seed, slots, rows, pending_row):
    rng = np.random.default_rng(seed)
    live = [b for b in range(B) if slots[b] > 0 and rows[b] >= 0]
    by_n = {}
    for b in live:
        by_n.setdefault(int(pending_row[rows[b]]), []).append(b)
    R = [0, 53, 5] + [int(rng.choice(by_n[n])) for n in sorted(by_n)]
    R += [int(x) for x in rng.choice(live, 8, replace=False)]
    return list(dict.fromkeys(R))


def _compact(R, slots, rows, pending_row, corr, kg, pages, state_dtype=np.float32):
    nR = len(R)
    page = H * V * K
    m = dict(state=np.zeros((nR + 1) * page, state_dtype),
             slots=np.array([j + 1 if slots[b] > 0 else 0 for j, b in enumerate(R)], np.int32),
             rows=np.array([j if rows[b] >= 0 else -1 for j, b in enumerate(R)], np.int32),
             corr=np.zeros((nR, H, RQ, V), np.float32), kg=np.zeros((nR, H, RQ, 2 * K), np.uint16),
             pend=np.zeros(nR, np.int32))
    for j, b in enumerate(R):
        if slots[b] > 0:
            m["state"][(j + 1) * page:(j + 2) * page] = pages(int(slots[b]))
        if rows[b] >= 0:
            m["corr"][j], m["kg"][j], m["pend"][j] = corr[rows[b]], kg[rows[b]], pending_row[rows[b]]
    m["tok"] = np.concatenate([np.arange(b * T, (b + 1) * T) for b in R])
    return m


def _check(label, R, m, m_out, g_out, g_pages, g_corr, g_kg, slots, rows, o_raw=None,
           bf16=False):
    """o_raw: the oracle's unrounded o of the gated stage (else plain o)."""
    page = H * V * K
    close = assert_bf16_close if bf16 else assert_f32_close
    for j, b in enumerate(R):
        if o_raw is not None:
            assert_gated_close(f"{label} out request {b}", g_out[b * T:(b + 1) * T],
                               m_out[j * T:(j + 1) * T], o_raw[j * T:(j + 1) * T])
        else:
            assert_bf16_close(f"{label} out request {b}", g_out[b * T:(b + 1) * T],
                              m_out[j * T:(j + 1) * T])
        if slots[b] > 0:
            close(f"{label} page request {b}", g_pages(int(slots[b])),
                  m["state"][(j + 1) * page:(j + 2) * page])
        if slots[b] > 0 and rows[b] >= 0:
            assert_f32_close(f"{label} corrections request {b}", g_corr[rows[b]], m["corr"][j])
            assert_exact(f"{label} key/gate request {b}", g_kg[rows[b]], m["kg"][j])


def _untouched(label, d_state, before, slots, rows, pending_row):
    page = H * V * K
    touched = torch.zeros(S, dtype=torch.bool)
    for b in range(B):
        if slots[b] > 0 and rows[b] >= 0 and min(pending_row[rows[b]], RQ) > 0:
            touched[int(slots[b])] = True
    keep = (~touched).nonzero().flatten().to(DEV)
    bits = torch.int16 if d_state.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(d_state.view(S, page).index_select(0, keep).view(bits),
                       before.view(S, page).index_select(0, keep).view(bits)), label


def test_large_decode_gated_output_sampled():
    import spec_decode_amd as kda
    g, slots, rows, pending_row, a_log, dtb, corr, kg = _plan(930)
    page = H * V * K
    win = window_np(W.draw_window(g, B, T, H))
    gate, weight, eps = W.draw_output_stage(W._gen(931), B, T, H)
    gate_bits = W.bits(gate)
    d_state = W.draw_state(932, S * page, torch.float32, DEV)
    before = d_state.clone()
    d_corr, d_kg = dev(corr), dev_bf16(kg)
    out = torch.zeros((B * T, H * V), dtype=torch.bfloat16, device=DEV)
    announce("large decode, gated output stage, FP32 pool")
    kda.kda_fused_replay_verify(heads=H, tokens=T, batch=B, q=dev_bf16(win["q"]),
                                k=dev_bf16(win["k"]), v=dev_bf16(win["v"]),
                                raw_g=dev_bf16(win["raw_g"]), raw_beta=dev_bf16(win["raw_beta"]),
                                a_log=dev(a_log), dt_bias=dev(dtb), lower_bound=W.LOWER_BOUND,
                                state=d_state, state_slot_stride=page, state_indices=dev(slots),
                                corr=d_corr, kg=d_kg, record_tokens=RQ, record_rows=dev(rows),
                                pending=dev(pending_row), out=out, gate=dev_bf16(gate_bits),
                                norm_weight=weight.to(DEV), norm_eps=eps)
    torch.cuda.synchronize()
    _untouched("gated", d_state, before, slots, rows, pending_row)
    R = _sample(933, slots, rows, pending_row)
    m = _compact(R, slots, rows, pending_row, corr, kg,
                 lambda sl: np_of(before[sl * page:(sl + 1) * page]))
    m_win = {k: np.ascontiguousarray(v[m["tok"]]) for k, v in win.items()}
    m_out = np.zeros((len(R) * T, H * V), np.uint16)
    o_raw = np.zeros((len(R) * T, H * V), np.float64)
    announce(f"large decode gated: oracle on {len(R)} sampled requests")
    oracle.fused_replay_verify(heads=H, tokens=T, batch=len(R), q=m_win["q"], k=m_win["k"],
                               v=m_win["v"], raw_g=m_win["raw_g"], raw_beta=m_win["raw_beta"],
                               a_log=a_log, dt_bias=dtb, lower_bound=W.LOWER_BOUND,
                               state=m["state"], state_slot_stride=page, state_indices=m["slots"],
                               corr=m["corr"], kg=m["kg"], record_tokens=RQ,
                               record_rows=m["rows"], pending=m["pend"], out=m_out,
                               gate=np.ascontiguousarray(gate_bits[m["tok"]]),
                               norm_weight=weight.numpy(), norm_eps=eps, o_raw=o_raw)
    _check("gated", R, m, m_out, np_of(out), lambda sl: np_of(d_state[sl * page:(sl + 1) * page]),
           np_of(d_corr), np_of(d_kg), slots, rows, o_raw)
    del d_state, before
    torch.cuda.empty_cache()


@pytest.mark.parametrize("bf16", [False, True])
def test_large_decode_stock_verify_sampled(bf16):
    """kda_verify at the large decode batch's size, as the benchmark's
    --workload verify launches it (the streaming instance: half of each page
    straight into LDS on FP32 pools): o and the records of sampled requests
    against the oracle, and the pool never written."""
    import spec_decode_amd as kda
    g, slots, rows, pending_row, a_log, dtb, corr, kg = _plan(950)
    page = H * V * K
    win = window_np(W.draw_window(g, B, T, H))
    d_state = W.draw_state(952, S * page, torch.bfloat16 if bf16 else torch.float32, DEV)
    before = d_state.clone()
    d_corr, d_kg = dev(corr), dev_bf16(kg)
    out = torch.zeros((B * T, H * V), dtype=torch.bfloat16, device=DEV)
    announce(f"large decode, stock verify, {'BF16' if bf16 else 'FP32'} pool")
    kda.kda_verify(heads=H, tokens=T, batch=B, q=dev_bf16(win["q"]), k=dev_bf16(win["k"]),
                   v=dev_bf16(win["v"]), raw_g=dev_bf16(win["raw_g"]),
                   raw_beta=dev_bf16(win["raw_beta"]), a_log=dev(a_log), dt_bias=dev(dtb),
                   lower_bound=W.LOWER_BOUND, state=d_state, state_slot_stride=page,
                   state_indices=dev(slots), corr=d_corr, kg=d_kg, record_tokens=RQ,
                   record_rows=dev(rows), out=out)
    torch.cuda.synchronize()
    bits = torch.int16 if bf16 else torch.int32
    assert torch.equal(d_state.view(bits), before.view(bits)), "the stock verify wrote the pool"
    R = _sample(953, slots, rows, pending_row)
    m = _compact(R, slots, rows, pending_row, corr, kg,
                 lambda sl: np_of(before[sl * page:(sl + 1) * page]),
                 np.uint16 if bf16 else np.float32)
    m_win = {k: np.ascontiguousarray(v[m["tok"]]) for k, v in win.items()}
    m_out = np.zeros((len(R) * T, H * V), np.uint16)
    announce(f"large decode stock verify: oracle on {len(R)} sampled requests")
    oracle.verify(heads=H, tokens=T, batch=len(R), q=m_win["q"], k=m_win["k"], v=m_win["v"],
                  raw_g=m_win["raw_g"], raw_beta=m_win["raw_beta"], a_log=a_log, dt_bias=dtb,
                  lower_bound=W.LOWER_BOUND, state=m["state"], state_slot_stride=page,
                  state_indices=m["slots"], corr=m["corr"], kg=m["kg"], record_tokens=RQ,
                  record_rows=m["rows"], out=m_out)
    _check("stock verify", R, m, m_out, np_of(out),
           lambda sl: np_of(d_state[sl * page:(sl + 1) * page]), np_of(d_corr), np_of(d_kg),
           slots, rows, bf16=bf16)
    del d_state, before
    torch.cuda.empty_cache()


@pytest.mark.parametrize("layout", ["dim_first", "window_major"])
@pytest.mark.parametrize("bf16", [False, True])
def test_large_decode_conv_prologue_sampled(bf16, layout):
    """The benchmark's --conv step takes the window-major pool by default; the
    packed dim-first pool runs the packed code."""
    import spec_decode_amd as kda
    g, slots, rows, pending_row, a_log, dtb, corr, kg = _plan(940)
    page = H * V * K
    win = window_np(W.draw_window(g, B, T, H))
    cv = W.draw_conv_inputs(W._gen(941), B, T, H, RQ, S)
    x, w_bits, b_bits = W.bits(cv.x), W.bits(cv.weight), W.bits(cv.bias)
    pool = W.bits(cv.window)  # [S, 3HK, RQ + 2]: the packed dim-first layout
    strides = conv_pool_layout(S, H, RQ + 2, layout=layout)
    # The pool as the GPU holds it: [S, 3HK, RQ + 2] or [S, RQ + 2, 3HK].
    g_in = pool if layout == "dim_first" else np.ascontiguousarray(pool.transpose(0, 2, 1))
    d_state = W.draw_state(942, S * page, torch.bfloat16 if bf16 else torch.float32, DEV)
    before = d_state.clone()
    d_corr, d_kg, d_pool = dev(corr), dev_bf16(kg), dev_bf16(g_in.reshape(-1))
    out = torch.zeros((B * T, H * V), dtype=torch.bfloat16, device=DEV)
    announce(f"large decode, convolution prologue, {layout} window pool, "
             f"{'BF16' if bf16 else 'FP32'} state pool")
    kda.kda_fused_conv_replay_verify(
        heads=H, tokens=T, batch=B, x=dev_bf16(x), x_row_stride=cv.pitch,
        conv_weight=dev_bf16(w_bits), conv_bias=dev_bf16(b_bits), conv_state=d_pool,
        conv_slot_stride=strides[0], conv_channel_stride=strides[1], conv_tap_stride=strides[2],
        q_scale=K ** -0.5, raw_g=dev_bf16(win["raw_g"]), raw_beta=dev_bf16(win["raw_beta"]),
        a_log=dev(a_log), dt_bias=dev(dtb), lower_bound=W.LOWER_BOUND, state=d_state,
        state_slot_stride=page, state_indices=dev(slots), corr=d_corr, kg=d_kg,
        record_tokens=RQ, record_rows=dev(rows), pending=dev(pending_row), out=out)
    torch.cuda.synchronize()
    _untouched("conv", d_state, before, slots, rows, pending_row)
    g_pool = np_of(d_pool).reshape(g_in.shape)
    if layout == "window_major":
        g_pool = np.ascontiguousarray(g_pool.transpose(0, 2, 1))
    live_slots = set(int(s) for s in slots if s > 0)
    for s in range(S):
        if s not in live_slots:
            assert_exact(f"conv windows of unnamed slot {s}", g_pool[s], pool[s])
    R = _sample(943, slots, rows, pending_row)
    nR = len(R)
    m = _compact(R, slots, rows, pending_row, corr, kg,
                 lambda sl: np_of(before[sl * page:(sl + 1) * page]),
                 np.uint16 if bf16 else np.float32)
    m_pool = np.zeros((nR + 1, 3 * H * K, RQ + 2), np.uint16)
    for j, b in enumerate(R):
        if slots[b] > 0:
            m_pool[j + 1] = pool[int(slots[b])]
    m_strides = conv_pool_layout(nR + 1, H, RQ + 2)  # the oracle's copy stays dim-first
    m_out = np.zeros((nR * T, H * V), np.uint16)
    announce(f"large decode conv: oracle on {nR} sampled requests")
    flat = m_pool.reshape(-1)
    oracle.fused_conv_replay_verify(
        heads=H, tokens=T, batch=nR, x=np.ascontiguousarray(x[m["tok"]]), x_row_stride=cv.pitch,
        conv_weight=w_bits, conv_bias=b_bits, conv_state=flat, conv_slot_stride=m_strides[0],
        conv_channel_stride=m_strides[1], conv_tap_stride=m_strides[2], q_scale=K ** -0.5,
        raw_g=np.ascontiguousarray(win["raw_g"][m["tok"]]),
        raw_beta=np.ascontiguousarray(win["raw_beta"][m["tok"]]), a_log=a_log, dt_bias=dtb,
        lower_bound=W.LOWER_BOUND, state=m["state"], state_slot_stride=page,
        state_indices=m["slots"], corr=m["corr"], kg=m["kg"], record_tokens=RQ,
        record_rows=m["rows"], pending=m["pend"], out=m_out)
    _check("conv", R, m, m_out, np_of(out), lambda sl: np_of(d_state[sl * page:(sl + 1) * page]),
           np_of(d_corr), np_of(d_kg), slots, rows, bf16=bf16)
    m_pool = flat.reshape(nR + 1, 3 * H * K, RQ + 2)
    for j, b in enumerate(R):
        if slots[b] > 0:
            assert_exact(f"conv windows request {b}", g_pool[int(slots[b])], m_pool[j + 1])
    # The recorded keys against the plain FP64 convolution and SiLU.
    share = check_conv_keys_plain("conv", np_of(d_kg), H=H, T=T, RQ=RQ, x=x, pitch=cv.pitch,
                                  conv_w=w_bits, conv_b=b_bits, pool=g_in, strides=strides,
                                  slots=slots[R], rows=rows[R], pending=pending_row,
                                  tok_of=lambda j: R[j] * T)
    announce(f"large decode conv: keys match the plain SiLU ({100 * share:.3f}% near a tie)")
    del d_state, before
    torch.cuda.empty_cache()
