"""The streaming instances compute the same bits as the plain ones.

A launch whose state pages exceed the 256 MB MALL runs the streaming instance
(write-through, no-reuse stores at two workgroups per CU); a smaller launch
runs the plain one. Items are independent, so the same requests run as one
launch (streaming) and as two launches of half the batch (plain) must leave
the pool, the records and the outputs bit for bit equal. Neither side is the
oracle: the oracle pins both through the other GPU tests; this one pins that
the instance choice changes nothing but the cache policy. The one exception
is the commit of FP32 pages, whose streaming kernel folds on the matrix cores
and the plain one on the vector ALU: there the two agree within the FP32
tolerance, and the streaming result is checked against the oracle here.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _compare import assert_f32_close
from _kda_cases import DEV, announce

pytestmark = pytest.mark.gpu
K = V = 128
H = 64
MALL = 256 << 20


def _bits(t):
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t).cpu().numpy()


def _assert_same(a, b, names):
    for name in names:
        assert np.array_equal(_bits(a[name]), _bits(b[name])), f"{name} differs"


@pytest.mark.parametrize("gated,T,pool", [(False, 3, "f32"), (True, 3, "f32"),
                                          (False, 8, "f32"), (True, 8, "f32"),
                                          (False, 8, "bf16"), (True, 5, "bf16")])
def test_fused_streaming_instance_matches_plain(gated, T, pool):
    import spec_decode_amd as kda
    bf16 = pool == "bf16"
    es = 2 if bf16 else 4
    B, RQ = (160 if bf16 else 80), 8
    page = H * V * K
    assert B * page * es > MALL >= (B // 2) * page * es
    S = B + 9
    g = W._gen(950 + gated)
    slots = (W.permutation(g, S - 1) + 1)[:B].to(torch.int32)
    slots[[7, 45, B - 3]] = 0
    rows = W.permutation(g, B).to(torch.int32)
    rows[[12, 60, B - 7]] = -1
    pending = W.uniform_int(g, 0, RQ, B).to(torch.int32)
    corr, kg = W.draw_records(g, B, H, RQ)
    a_log, dtb = W.draw_gate_params(g, 1, H)
    w = W.draw_window(g, B, T, H).to(DEV)
    extra = {}
    if gated:
        gate, weight, eps = W.draw_output_stage(W._gen(952), B, T, H)
        extra = dict(gate=gate.to(DEV), norm_weight=weight.to(DEV), norm_eps=eps)
    state0 = W.draw_state(953 + gated, S * page, torch.bfloat16 if bf16 else torch.float32, DEV)

    def fresh():
        return dict(state=state0.clone(), corr=corr.to(DEV), kg=kg.to(DEV),
                    pending=pending.to(DEV),
                    out=torch.zeros((B * T, H * V), dtype=torch.bfloat16, device=DEV))

    def call(m, lo, hi):
        n = hi - lo
        ex = dict(extra)
        if gated:
            ex["gate"] = extra["gate"][lo * T:hi * T]
        kda.kda_fused_replay_verify(
            heads=H, tokens=T, batch=n, q=w.q[lo * T:hi * T], k=w.k[lo * T:hi * T],
            v=w.v[lo * T:hi * T], raw_g=w.raw_g[lo * T:hi * T],
            raw_beta=w.raw_beta[lo * T:hi * T], a_log=a_log[0].contiguous().to(DEV),
            dt_bias=dtb[0].contiguous().to(DEV), lower_bound=W.LOWER_BOUND, state=m["state"],
            state_slot_stride=page, state_indices=slots[lo:hi].to(DEV), corr=m["corr"],
            kg=m["kg"], record_tokens=RQ, record_rows=rows[lo:hi].to(DEV),
            pending=m["pending"], out=m["out"][lo * T:hi * T], **ex)

    announce(f"fused, streaming vs plain instance, H={H} B={B} q={T}, gated={gated}, {pool}")
    one, two = fresh(), fresh()
    call(one, 0, B)
    call(two, 0, B // 2)
    call(two, B // 2, B)
    torch.cuda.synchronize()
    assert not torch.equal(one["state"], state0)  # pages were written
    _assert_same(one, two, ("state", "corr", "kg", "out"))


@pytest.mark.parametrize("pool,Q,align", [("f32", 8, False), ("bf16", 8, False),
                                          ("f32", 3, False), ("f32", 8, True), ("f32", 5, True),
                                          ("f32", 1, False), ("f32", 4, True), ("f32", 7, True)])
def test_commit_streaming_instance_matches_plain(pool, Q, align):
    """Windows of 1, 3, 4, 5, 7 and 8 tokens, with and without boundary stores (the
    boundary pages beyond every source page, two of them null). BF16 pools:
    the same bits. FP32 pools: the two within the FP32 tolerance, and 10
    sampled requests of the streaming launch against the oracle."""
    import spec_decode_amd as kda
    bf16 = pool == "bf16"
    es = 2 if bf16 else 4
    B = 160 if bf16 else 80
    page = H * V * K
    assert B * page * es > MALL >= (B // 2) * page * es
    S = B + 5 + (B if align else 0)
    g = W._gen(960 + bf16 + 2 * Q + 20 * align)
    src = (W.permutation(g, B + 4) + 1)[:B].to(torch.int32)
    src[[3, 50]] = 0
    rows = W.permutation(g, B).to(torch.int32)
    lens = W.uniform_int(g, 0, Q, B).to(torch.int32)
    bounds = blens = None
    if align:
        # Boundary pages of their own, beyond every source page; some null.
        bounds = (B + 5 + W.permutation(g, B)).to(torch.int32)
        bounds[[7, 61]] = 0
        blens = W.uniform_int(g, 0, Q + 1, B).to(torch.int32)
    corr, kg = W.draw_records(g, B, H, Q)
    a_log, dtb = W.draw_gate_params(g, 1, H)
    state0 = W.draw_state(962 + bf16, S * page, torch.bfloat16 if bf16 else torch.float32, DEV)
    d_corr, d_kg = corr.to(DEV), kg.to(DEV)

    def call(state, lo, hi):
        s = src[lo:hi].to(DEV)
        kda.kda_commit(heads=H, window=Q, batch=hi - lo,
                       state_dtype=kda.KDA_STATE_BF16 if bf16 else kda.KDA_STATE_F32,
                       state_addrs=[state.data_ptr()], state_slot_strides=[page],
                       corr_addrs=[d_corr.data_ptr()], corr_row_strides=[H * Q * V],
                       kg_addrs=[d_kg.data_ptr()], kg_row_strides=[H * Q * 2 * K],
                       a_log=a_log.to(DEV), dt_bias=dtb.to(DEV), sources=s,
                       commit_lens=lens[lo:hi].to(DEV), destinations=s,
                       boundaries=None if bounds is None else bounds[lo:hi].to(DEV),
                       boundary_lens=None if blens is None else blens[lo:hi].to(DEV),
                       record_rows=rows[lo:hi].to(DEV), lower_bound=W.LOWER_BOUND)

    announce(f"commit, streaming vs plain instance, H={H} B={B} window {Q}, {pool} pool, "
             f"align {align}")
    one, two = state0.clone(), state0.clone()
    call(one, 0, B)
    call(two, 0, B // 2)
    call(two, B // 2, B)
    torch.cuda.synchronize()
    assert not torch.equal(one, state0)
    if align:
        assert not torch.equal(one[(B + 5) * page:], state0[(B + 5) * page:])
    if bf16:
        assert np.array_equal(_bits(one), _bits(two))
        return
    g_one, g_two = one.cpu().numpy(), two.cpu().numpy()
    assert_f32_close("streaming vs plain FP32 commit", g_one, g_two)
    # Sampled requests of the streaming launch against the oracle on a compact
    # pool: slot 1+3j source, 2+3j destination (a copy of the source: the
    # commit runs in place), 3+3j boundary.
    live = [b for b in range(B) if src[b] > 0 and lens[b] > 0]
    R = np.random.default_rng(61 + Q).choice(live, 10, replace=False)
    nR = len(R)
    m_src = (1 + 3 * np.arange(nR)).astype(np.int32)
    m_bnd = np.where((blens[R] > 0) & (bounds[R] > 0), m_src + 2, 0).astype(np.int32) \
        if align else None
    s0 = state0.cpu().numpy()
    mini = np.zeros((1 + 3 * nR) * page, np.float32)
    for j, b in enumerate(R):
        sl = int(src[b])
        mini[m_src[j] * page:(m_src[j] + 1) * page] = s0[sl * page:(sl + 1) * page]
    r_of = rows.numpy()[R]
    announce(f"commit FP32 streaming launch: oracle on {nR} sampled requests x {H} heads")
    oracle.commit(heads=H, window=Q, batch=nR, state_bf16=False, state_layers=[mini],
                  state_slot_strides=[page], corr_layers=[corr.numpy()[r_of]],
                  corr_row_strides=[H * Q * V], kg_layers=[W.bits(kg)[r_of]],
                  kg_row_strides=[H * Q * 2 * K], a_log=a_log.numpy(), dt_bias=dtb.numpy(),
                  sources=m_src, commit_lens=lens.numpy()[R], destinations=m_src,
                  boundaries=m_bnd, boundary_lens=None if blens is None else blens.numpy()[R],
                  lower_bound=W.LOWER_BOUND)
    for j, b in enumerate(R):
        sl = int(src[b])
        assert_f32_close(f"streaming commit request {b}", g_one[sl * page:(sl + 1) * page],
                         mini[m_src[j] * page:(m_src[j] + 1) * page])
        if align and m_bnd[j] > 0:
            bs = int(bounds[b])
            assert_f32_close(f"streaming commit request {b} boundary",
                             g_one[bs * page:(bs + 1) * page],
                             mini[m_bnd[j] * page:(m_bnd[j] + 1) * page])


@pytest.mark.parametrize("layout", ["dim_first", "window_major"])
def test_fused_conv_streaming_instance_matches_plain(layout):
    """The same with the convolution prologue, over the packed dim-first window
    pool and the window-major one (the strided code); the window pool, which
    the step rewrites in place, is compared too."""
    import spec_decode_amd as kda
    from _kda_cases import conv_pool_layout
    B, T, RQ = 80, 8, 8
    page = H * V * K
    S = B + 7
    g = W._gen(970)
    slots = (W.permutation(g, S - 1) + 1)[:B].to(torch.int32)
    slots[[9, 44]] = 0
    rows = W.permutation(g, B).to(torch.int32)
    rows[[21, 70]] = -1
    pending = W.uniform_int(g, 0, RQ, B).to(torch.int32)
    corr, kg = W.draw_records(g, B, H, RQ)
    a_log, dtb = W.draw_gate_params(g, 1, H)
    w = W.draw_window(g, B, T, H).to(DEV)
    cv = W.draw_conv_inputs(W._gen(971), B, T, H, RQ, S)
    pool0 = cv.window if layout == "dim_first" else cv.window.permute(0, 2, 1).contiguous()
    pool0 = pool0.reshape(-1).to(DEV)
    strides = conv_pool_layout(S, H, RQ + 2, layout=layout)
    x = cv.x.to(DEV)
    state0 = W.draw_state(972, S * page, torch.float32, DEV)

    def fresh():
        return dict(state=state0.clone(), pool=pool0.clone(), corr=corr.to(DEV), kg=kg.to(DEV),
                    pending=pending.to(DEV),
                    out=torch.zeros((B * T, H * V), dtype=torch.bfloat16, device=DEV))

    def call(m, lo, hi):
        kda.kda_fused_conv_replay_verify(
            heads=H, tokens=T, batch=hi - lo, x=x[lo * T:hi * T], x_row_stride=cv.pitch,
            conv_weight=cv.weight.to(DEV), conv_bias=cv.bias.to(DEV), conv_state=m["pool"],
            conv_slot_stride=strides[0], conv_channel_stride=strides[1],
            conv_tap_stride=strides[2], q_scale=K ** -0.5, raw_g=w.raw_g[lo * T:hi * T],
            raw_beta=w.raw_beta[lo * T:hi * T], a_log=a_log[0].contiguous().to(DEV),
            dt_bias=dtb[0].contiguous().to(DEV), lower_bound=W.LOWER_BOUND, state=m["state"],
            state_slot_stride=page, state_indices=slots[lo:hi].to(DEV), corr=m["corr"],
            kg=m["kg"], record_tokens=RQ, record_rows=rows[lo:hi].to(DEV),
            pending=m["pending"], out=m["out"][lo * T:hi * T])

    announce(f"fused conv ({layout} windows), streaming vs plain instance, H={H} B={B} q={T}")
    one, two = fresh(), fresh()
    call(one, 0, B)
    call(two, 0, B // 2)
    call(two, B // 2, B)
    torch.cuda.synchronize()
    assert not torch.equal(one["state"], state0)
    assert not torch.equal(one["pool"], pool0)
    _assert_same(one, two, ("state", "pool", "corr", "kg", "out"))


@pytest.mark.parametrize("pool", ["f32", "bf16"])
def test_verify_streaming_instance_matches_plain(pool):
    """The stock verify: above the MALL's size it writes o and the records
    through the L2; the pool is only read, on both instances."""
    import spec_decode_amd as kda
    bf16 = pool == "bf16"
    es = 2 if bf16 else 4
    B, T, RQ = (160 if bf16 else 80), 8, 8
    page = H * V * K
    assert B * page * es > MALL >= (B // 2) * page * es
    S = B + 5
    g = W._gen(980 + bf16)
    slots = (W.permutation(g, S - 1) + 1)[:B].to(torch.int32)
    slots[[4, 33]] = 0
    rows = W.permutation(g, B).to(torch.int32)
    rows[[8, 61]] = -1
    corr, kg = W.draw_records(g, B, H, RQ)
    a_log, dtb = W.draw_gate_params(g, 1, H)
    w = W.draw_window(g, B, T, H).to(DEV)
    state = W.draw_state(982 + bf16, S * page, torch.bfloat16 if bf16 else torch.float32, DEV)
    before = state.clone()

    def fresh():
        return dict(corr=corr.to(DEV), kg=kg.to(DEV),
                    out=torch.zeros((B * T, H * V), dtype=torch.bfloat16, device=DEV))

    def call(m, lo, hi):
        kda.kda_verify(
            heads=H, tokens=T, batch=hi - lo, q=w.q[lo * T:hi * T], k=w.k[lo * T:hi * T],
            v=w.v[lo * T:hi * T], raw_g=w.raw_g[lo * T:hi * T],
            raw_beta=w.raw_beta[lo * T:hi * T], a_log=a_log[0].contiguous().to(DEV),
            dt_bias=dtb[0].contiguous().to(DEV), lower_bound=W.LOWER_BOUND, state=state,
            state_slot_stride=page, state_indices=slots[lo:hi].to(DEV), corr=m["corr"],
            kg=m["kg"], record_tokens=RQ, record_rows=rows[lo:hi].to(DEV),
            out=m["out"][lo * T:hi * T])

    announce(f"verify, streaming vs plain instance, H={H} B={B} q={T}, {pool} pool")
    one, two = fresh(), fresh()
    call(one, 0, B)
    call(two, 0, B // 2)
    call(two, B // 2, B)
    torch.cuda.synchronize()
    assert torch.equal(_bits_t(state), _bits_t(before))
    assert not torch.equal(one["corr"], corr.to(DEV))  # records were written
    _assert_same(one, two, ("corr", "kg", "out"))


def _bits_t(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
