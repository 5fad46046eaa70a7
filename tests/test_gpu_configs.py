"""GPU parity on the five synthetic workloads, in the launch configuration the
benchmark times.

* tiny (verify, then commit lens {0, 3}), commit (BF16, 256 slots) and fused
  (FP32, 256 slots): every output against the full FP64 oracle.
* align commit (8 layers, 5.4 GB of BF16 pools) and large decode (2 GiB FP32
  fused, then defer, flush plan and in-place commit): the GPU runs the full
  problem; the oracle recomputes sampled requests one by one (all their heads
  and layers) from host copies of their inputs; and properties that hold at any
  size are checked over the whole pools (every page nobody writes is
  bit-identical, plan outputs bit-exact).

Records that a step replays come from the oracle's own verify of a prior
window; when the GPU and the oracle chain several calls, each side feeds its
own outputs forward.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _compare import assert_bf16_close, assert_exact, assert_f32_close
from _kda_cases import (DEV, announce, dev, dev_bf16, np_of, run_commit_case, run_verify_case,
                        sampled_fused_oracle,
                        window_np)

pytestmark = pytest.mark.gpu

K = V = 128


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import spec_decode_amd  # noqa: F401

    torch.cuda.init()
    yield
    torch.cuda.empty_cache()


def _oracle_prior_records(w, state, corr, kg, slots, rows, T, RQ, H, B):
    """The records of a verify of the prior window (oracle), written in place."""
    win = window_np(w.windows["prior"])
    out = np.zeros((B * T, H * V), np.uint16)
    oracle.verify(heads=H, tokens=T, batch=B, q=win["q"], k=win["k"], v=win["v"],
                  raw_g=win["raw_g"], raw_beta=win["raw_beta"],
                  a_log=w.arrays["a_log"][0].numpy(), dt_bias=w.arrays["dt_bias"][0].numpy(),
                  lower_bound=w.lower_bound, state=state, state_slot_stride=H * V * K,
                  state_indices=slots, corr=corr, kg=kg, record_tokens=RQ, out=out,
                  record_rows=rows)


# ---------------------------------------------------------------- config 0

def test_config0_tiny_verify_then_commit():
    import spec_decode_amd as kda

    w = W.config0()
    H, B, T = w.heads, w.batch, w.tokens
    a = w.arrays
    state0 = a["state"].numpy().copy()
    slots, rows = a["state_indices"].numpy(), a["record_rows"].numpy()
    lens = a["commit_lens"].numpy()
    a_log, dtb = a["a_log"].numpy(), a["dt_bias"].numpy()
    win = window_np(w.windows["new"])
    gpu, ref = run_verify_case(fused=False, H=H, B=B, T=T, RQ=T, state=state0,
                               slots=slots, corr=a["corr"].numpy().copy(), kg=W.bits(a["kg"]),
                               a_log=a_log[0], dt_bias=dtb[0], win=win, rows=rows,
                               label="config0 verify")
    # Commit lens {0, 3} in place; each side commits its own records.
    announce("config0: commit lens {0, 3}")
    d_state, d_corr, d_kg = dev(state0), dev(gpu["corr"]), dev_bf16(gpu["kg"])
    kda.kda_commit(heads=H, window=T, batch=B, state_dtype=kda.KDA_STATE_F32,
                   state_addrs=[d_state.data_ptr()], state_slot_strides=[H * V * K],
                   corr_addrs=[d_corr.data_ptr()], corr_row_strides=[H * T * V],
                   kg_addrs=[d_kg.data_ptr()], kg_row_strides=[H * T * 2 * K],
                   a_log=dev(a_log), dt_bias=dev(dtb), sources=dev(slots),
                   commit_lens=dev(lens), destinations=dev(slots), record_rows=dev(rows),
                   lower_bound=w.lower_bound)
    torch.cuda.synchronize()
    g_state = np_of(d_state).reshape(4, H, V, K)
    r_state = state0.copy()
    oracle.commit(heads=H, window=T, batch=B, state_bf16=False, state_layers=[r_state],
                  state_slot_strides=[H * V * K], corr_layers=[ref["corr"]],
                  corr_row_strides=[H * T * V], kg_layers=[ref["kg"]],
                  kg_row_strides=[H * T * 2 * K], a_log=a_log, dt_bias=dtb, sources=slots,
                  commit_lens=lens, destinations=slots, record_rows=rows,
                  lower_bound=w.lower_bound)
    r_state = r_state.reshape(4, H, V, K)
    s0 = state0.reshape(4, H, V, K)
    assert_f32_close("config0 committed slot 2", g_state[2], r_state[2])
    for s in (0, 1, 3):  # null slot, the lens-0 request's slot, the spare
        assert_exact(f"config0 slot {s} unchanged", g_state[s], s0[s])


# ---------------------------------------------------------------- config 1

def test_config1_commit_bf16():
    w = W.config1()
    a = w.arrays
    run_commit_case(H=w.heads, B=w.batch, Q=w.tokens, bf16=True,
                    layers_state=[W.bits(a["state"])], strides=w.slot_strides,
                    corr_layers=[a["corr"].numpy().copy()], kg_layers=[W.bits(a["kg"])],
                    a_log=a["a_log"].numpy(), dt_bias=a["dt_bias"].numpy(),
                    src=a["sources"].numpy(), lens=a["commit_lens"].numpy(),
                    dst=a["destinations"].numpy(), lb=w.lower_bound, label="config1 commit")


# ---------------------------------------------------------------- config 2

@pytest.mark.parametrize("bf16", [False, True])
def test_config2_fused_full(bf16):
    """The fused workload at full size against the full oracle; bf16 runs it
    on the same pool rounded to a BF16 pool."""
    w = W.config2()
    H, B, T, RQ = w.heads, w.batch, w.tokens, w.record_tokens
    a = w.arrays
    state = W.bits(a["state"].to(torch.bfloat16)) if bf16 else a["state"].numpy().copy()
    slots, rows = a["state_indices"].numpy(), a["record_rows"].numpy()
    corr, kg = a["corr"].numpy().copy(), W.bits(a["kg"])
    announce("config2: oracle verify of the prior window (records)")
    _oracle_prior_records(w, state, corr, kg, slots, rows, T, RQ, H, B)
    pending = np.zeros(B, np.int32)
    pending[rows] = a["pending"].numpy()  # pending is indexed by record row
    run_verify_case(fused=True, H=H, B=B, T=T, RQ=RQ, state=state, slots=slots, corr=corr,
                    kg=kg, a_log=a["a_log"][0].numpy(), dt_bias=a["dt_bias"][0].numpy(),
                    win=window_np(w.windows["new"]), rows=rows, pending=pending,
                    lb=w.lower_bound, label=f"config2 fused bf16={bf16}")


def test_config2_fused_full_gated_output():
    """The fused workload with the gated RMSNorm output stage on."""
    w = W.config2()
    H, B, T, RQ = w.heads, w.batch, w.tokens, w.record_tokens
    a = w.arrays
    state = a["state"].numpy().copy()
    slots, rows = a["state_indices"].numpy(), a["record_rows"].numpy()
    corr, kg = a["corr"].numpy().copy(), W.bits(a["kg"])
    _oracle_prior_records(w, state, corr, kg, slots, rows, T, RQ, H, B)
    pending = np.zeros(B, np.int32)
    pending[rows] = a["pending"].numpy()
    gate, weight, eps = W.draw_output_stage(W._gen(2 + 200), B, T, H)
    run_verify_case(fused=True, H=H, B=B, T=T, RQ=RQ, state=state, slots=slots, corr=corr,
                    kg=kg, a_log=a["a_log"][0].numpy(), dt_bias=a["dt_bias"][0].numpy(),
                    win=window_np(w.windows["new"]), rows=rows, pending=pending,
                    lb=w.lower_bound, gate=W.bits(gate), norm_weight=weight.numpy(),
                    norm_eps=eps, label="config2 fused gated output")


def test_config2_fused_conv_full():
    """The fused workload with the convolution prologue at full size (H=32,
    B=128, q=4): q, k, v from packed pre-activations and a dim-first window pool
    of 256 slots, against the full oracle, windows compared bit for bit."""
    from _kda_cases import conv_pool_layout, run_conv_case

    w = W.config2()
    H, B, T, RQ, S = w.heads, w.batch, w.tokens, w.record_tokens, w.slots
    a = w.arrays
    state = a["state"].numpy().copy()
    slots, rows = a["state_indices"].numpy(), a["record_rows"].numpy()
    corr, kg = a["corr"].numpy().copy(), W.bits(a["kg"])
    _oracle_prior_records(w, state, corr, kg, slots, rows, T, RQ, H, B)
    pending = np.zeros(B, np.int32)
    pending[rows] = a["pending"].numpy()
    cv = W.draw_conv_inputs(W._gen(2 + 300), B, T, H, RQ, S)
    win = window_np(w.windows["new"])
    run_conv_case(H=H, B=B, T=T, RQ=RQ, state=state, slots=slots, corr=corr, kg=kg,
                  a_log=a["a_log"][0].numpy(), dt_bias=a["dt_bias"][0].numpy(),
                  raw_g=win["raw_g"], raw_beta=win["raw_beta"], x=W.bits(cv.x), pitch=cv.pitch,
                  conv_w=W.bits(cv.weight), conv_b=W.bits(cv.bias),
                  pool=W.bits(cv.window).reshape(-1), strides=conv_pool_layout(S, H, RQ + 2),
                  rows=rows, pending=pending, lb=w.lower_bound, label="config2 fused conv")


def test_large_decode_gate_projection_sampled():
    """The gate projection at the large decode batch's size (4096 tokens, 64
    heads, F_A a column slice of packed projection rows): 64 sampled tokens
    bit-exact against the oracle (exact-grid factors), every element written."""
    import spec_decode_amd as kda
    N, H = 512 * 8, 64
    hk = H * K
    pitch = (4 * hk + 128 + H + 7) // 8 * 8
    fa, fb = W.draw_gate_factors(W._gen(4 + 400), N, H)
    packed = W.bf16(W.normal(W._gen(4 + 401), (N, pitch))).to(DEV)
    packed[:, 4 * hk:4 * hk + K] = fa.to(DEV)
    out = torch.zeros((N, hk), dtype=torch.bfloat16, device=DEV)
    out.view(torch.int16).fill_(0x7FFF)
    announce("large decode gate projection")
    kda.kda_gate_projection(tokens=N, heads=H, f_a=packed[:, 4 * hk:], f_a_row_stride=pitch,
                            f_b=fb.to(DEV), raw_g=out)
    torch.cuda.synchronize()
    got = np_of(out)
    pick = np.random.default_rng(7).choice(N, 64, replace=False)
    want = oracle.gate_projection(W.bits(fa)[pick], W.bits(fb))
    assert_exact("raw_g (sampled tokens)", got[pick], want)
    # the sentinel 0x7FFF is NaN: an unwritten element would show as one
    assert not np.any(got == 0x7FFF)


# ---------------------------------------------------------------- config 3

def test_large_decode_gate_projection_general_factors():
    """The gate projection at the large decode batch's size with general BF16
    factors, as the benchmark step draws them (F_A = BF16(N(0, 1)), F_B =
    BF16(N(0, 1) / sqrt(128))): the kernel sums in FP32 on matrix cores and
    rounds once (fused page, KdaFused.kernel, the gate projection), so an
    element whose exact sum lies within FP32 error of a BF16 rounding boundary
    may round to the other neighbour. Against the oracle on 512 sampled
    tokens: within one ulp everywhere and at least 99.9% bit-equal; every
    token against the FP64 product rounded once: within one ulp."""
    import spec_decode_amd as kda
    from _compare import bf16_mismatch
    N, H = 512 * 8, 64
    hk = H * K
    pitch = (4 * hk + 128 + H + 7) // 8 * 8
    fa, fb = W.draw_gate_factors(W._gen(4 + 410), N, H, exact=False)
    packed = W.bf16(W.normal(W._gen(4 + 411), (N, pitch))).to(DEV)
    packed[:, 4 * hk:4 * hk + K] = fa.to(DEV)
    out = torch.zeros((N, hk), dtype=torch.bfloat16, device=DEV)
    out.view(torch.int16).fill_(0x7FFF)
    announce("large decode gate projection, general factors")
    kda.kda_gate_projection(tokens=N, heads=H, f_a=packed[:, 4 * hk:], f_a_row_stride=pitch,
                            f_b=fb.to(DEV), raw_g=out)
    torch.cuda.synchronize()
    got = np_of(out)
    fa_b, fb_b = W.bits(fa), W.bits(fb)
    pick = np.random.default_rng(8).choice(N, 512, replace=False)
    want = oracle.gate_projection(fa_b[pick], fb_b)
    assert not bf16_mismatch(got[pick], want).any()
    equal = float(np.mean(got[pick] == want))
    announce(f"gate projection, general factors: {100 * equal:.4f}% bit-equal to the oracle")
    assert equal >= 0.999
    prod = oracle.bf16_to_f64(fa_b) @ oracle.bf16_to_f64(fb_b).T
    assert not bf16_mismatch(got, oracle.round_bf16(prod)).any()


@pytest.mark.parametrize("pool", ["bf16", "f32"])
def test_config3_align_commit_full_size_sampled(pool):
    """The prefix-cache align commit at full size: 8 layers of BF16 pools (the
    workload), and the same plan over 3 layers of FP32 pools, 1.5 GiB of source
    pages per launch (the streaming FP32 kernel: pages through LDS, folded on
    the matrix cores). Whole-pool property: every slot nobody writes is
    bit-identical; 12 sampled requests (6 with a boundary store) of every
    layer and head against the oracle."""
    import spec_decode_amd as kda

    bf16 = pool == "bf16"
    w = W.config3(device=DEV, layers=8 if bf16 else 3)
    a = w.arrays
    L, H, B, Q = w.layers, w.heads, w.batch, w.tokens
    strides = w.slot_strides
    page = H * V * K
    src, dst = a["sources"].numpy(), a["destinations"].numpy()
    bnd, blen, lens = a["boundaries"].numpy(), a["boundary_lens"].numpy(), a["commit_lens"].numpy()
    if bf16:
        pools = [a[f"state{l}"] for l in range(L)]
    else:
        pools = [W.draw_state(3000 + 17 + l, w.slots * strides[l], torch.float32, DEV)
                 for l in range(L)]
        for l in range(L):
            del a[f"state{l}"]
        torch.cuda.empty_cache()
    before = [p.clone() for p in pools]
    corrs = [a[f"corr{l}"].numpy().copy() for l in range(L)]
    kgs = [W.bits(a[f"kg{l}"]) for l in range(L)]
    d_corr = [dev(c) for c in corrs]
    d_kg = [dev_bf16(k) for k in kgs]
    announce(f"config3: full-size align commit L={L} H={H} B={B} Q={Q}, {pool} pools")
    kda.kda_commit(heads=H, window=Q, batch=B,
                   state_dtype=kda.KDA_STATE_BF16 if bf16 else kda.KDA_STATE_F32,
                   state_addrs=[p.data_ptr() for p in pools], state_slot_strides=strides,
                   corr_addrs=[c.data_ptr() for c in d_corr], corr_row_strides=[H * Q * V] * L,
                   kg_addrs=[k.data_ptr() for k in d_kg], kg_row_strides=[H * Q * 2 * K] * L,
                   a_log=a["a_log"].to(DEV), dt_bias=a["dt_bias"].to(DEV),
                   sources=dev(src), commit_lens=dev(lens), destinations=dev(dst),
                   boundaries=dev(bnd), boundary_lens=dev(blen), lower_bound=w.lower_bound)
    torch.cuda.synchronize()

    def bits(t):
        return t.view(torch.int16) if bf16 else t.view(torch.int32)

    # Property over the whole pools: every slot nobody writes is bit-identical.
    for l in range(L):
        written = torch.zeros(w.slots, dtype=torch.bool)
        written[torch.from_numpy(dst[lens > 0]).long()] = True
        live_b = (blen > 0) & (bnd > 0) & (lens > 0)
        written[torch.from_numpy(bnd[live_b]).long()] = True
        keep = (~written).nonzero().flatten().tolist()
        view_now = pools[l].view(w.slots, strides[l])
        view_then = before[l].view(w.slots, strides[l])
        idx = torch.tensor(keep, device=DEV)
        assert torch.equal(bits(view_now.index_select(0, idx)),
                           bits(view_then.index_select(0, idx))), f"layer {l}"
        # the padding between pages of odd layers is never written either
        if strides[l] > page:
            assert torch.equal(bits(view_now[:, page:]), bits(view_then[:, page:]))

    # Sampled requests: 6 with a boundary store and 6 without, all layers and heads.
    rng = np.random.default_rng(33)
    with_b = np.flatnonzero(blen > 0)
    without = np.flatnonzero(blen == 0)
    R = np.concatenate([rng.choice(with_b, 6, replace=False), rng.choice(without, 6, replace=False)])
    nR = len(R)
    m_stride = page  # compact mini pools: slot 1+3j source, 2+3j destination, 3+3j boundary
    m_src = (1 + 3 * np.arange(nR)).astype(np.int32)
    m_dst = m_src + 1
    m_bnd = np.where(blen[R] > 0, m_src + 2, 0).astype(np.int32)
    host = W.bits if bf16 else (lambda t: t.cpu().numpy())
    close = assert_bf16_close if bf16 else assert_f32_close
    announce(f"config3: oracle on {nR} sampled requests x {L} layers x {H} heads")
    for l in range(L):
        pool_then = before[l].view(w.slots, strides[l])[:, :page]
        mini = np.zeros((1 + 3 * nR) * page, np.uint16 if bf16 else np.float32)
        for j, b in enumerate(R):
            mini[m_src[j] * page:(m_src[j] + 1) * page] = host(pool_then[int(src[b])])
        oracle.commit(heads=H, window=Q, batch=nR, state_bf16=bf16, state_layers=[mini],
                      state_slot_strides=[m_stride], corr_layers=[corrs[l][R]],
                      corr_row_strides=[H * Q * V], kg_layers=[kgs[l][R]],
                      kg_row_strides=[H * Q * 2 * K], a_log=a["a_log"][l:l + 1].numpy(),
                      dt_bias=a["dt_bias"][l:l + 1].numpy(), sources=m_src,
                      commit_lens=lens[R], destinations=m_dst, boundaries=m_bnd,
                      boundary_lens=blen[R], lower_bound=w.lower_bound)
        pool_now = pools[l].view(w.slots, strides[l])[:, :page]
        for j, b in enumerate(R):
            close(f"config3 layer {l} request {b} destination", host(pool_now[int(dst[b])]),
                  mini[m_dst[j] * page:(m_dst[j] + 1) * page])
            if blen[b] > 0:
                close(f"config3 layer {l} request {b} boundary", host(pool_now[int(bnd[b])]),
                      mini[m_bnd[j] * page:(m_bnd[j] + 1) * page])
    del pools, before
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- config 4

def test_config4_large_decode_full_size_sampled():
    import spec_decode_amd as kda

    w = W.config4(device=DEV)
    a = w.arrays
    H, B, T, RQ = w.heads, w.batch, w.tokens, w.record_tokens
    page = H * V * K
    lb = w.lower_bound
    slots, rows = a["state_indices"].numpy(), a["record_rows"].numpy()
    pend_req, accepted = a["pending"].numpy(), a["accepted"].numpy()
    a_log, dtb = a["a_log"][0].numpy(), a["dt_bias"][0].numpy()
    d_state = a["state"]
    s0 = np_of(d_state)  # host copy of the initial 2 GiB pool
    before = d_state.clone()
    corr, kg = a["corr"].numpy().copy(), W.bits(a["kg"])
    announce("config4: oracle verify of the prior window (records), 32768 items")
    _oracle_prior_records(w, s0, corr, kg, slots, rows, T, RQ, H, B)
    pending = np.zeros(B, np.int32)
    for b in range(B):
        if rows[b] >= 0:
            pending[rows[b]] = pend_req[b]
    new = w.windows["new"]
    win = window_np(new)

    d_corr, d_kg = dev(corr), dev_bf16(kg)
    d_rows, d_slots, d_pend = dev(rows), dev(slots), dev(pending)
    out = torch.empty((B * T, H * V), dtype=torch.bfloat16, device=DEV)
    d_a, d_b = dev(a_log), dev(dtb)
    announce("config4: full-size fused replay+verify")
    kda.kda_fused_replay_verify(heads=H, tokens=T, batch=B, q=new.q.to(DEV), k=new.k.to(DEV),
                                v=new.v.to(DEV), raw_g=new.raw_g.to(DEV),
                                raw_beta=new.raw_beta.to(DEV), a_log=d_a, dt_bias=d_b,
                                lower_bound=lb, state=d_state, state_slot_stride=page,
                                state_indices=d_slots, corr=d_corr, kg=d_kg, record_tokens=RQ,
                                record_rows=d_rows, pending=d_pend, out=out)
    torch.cuda.synchronize()
    g_out = np_of(out)
    g_corr_f, g_kg_f = np_of(d_corr), np_of(d_kg)
    fused_state = d_state.clone()

    # Plan: defer the accepted counts, then the flush plan (bit-exact, full size).
    announce("config4: defer + flush plan")
    d_lens = dev(accepted.astype(np.int32))
    kda.kda_defer_commit(batch=B, state_indices=d_slots, commit_lens=d_lens, record_rows=d_rows,
                         pending=d_pend)
    fl = [torch.empty(B, dtype=torch.int32, device=DEV) for _ in range(4)]
    kda.kda_flush_plan(batch=B, spec_query_len=T, state_indices=d_slots, record_rows=d_rows,
                       pending=d_pend, commit_lens=fl[0], final_indices=fl[1], boundaries=fl[2],
                       boundary_lens=fl[3])
    torch.cuda.synchronize()
    r_lens, r_pend = accepted.astype(np.int32).copy(), pending.copy()
    oracle.defer(slots, r_lens, rows, r_pend)
    assert_exact("config4 defer commit_lens", np_of(d_lens), r_lens)
    assert_exact("config4 defer pending", np_of(d_pend), r_pend)
    r_flush = oracle.flush_plan(slots, rows, r_pend, T)
    for name, g, r in zip(("commit_lens", "final", "boundaries", "boundary_lens"), fl, r_flush):
        assert_exact(f"config4 flush {name}", np_of(g), r)
    flush_lens = r_flush[0]

    announce("config4: full-size in-place FP32 commit")
    kda.kda_commit(heads=H, window=RQ, batch=B, state_dtype=kda.KDA_STATE_F32,
                   state_addrs=[d_state.data_ptr()], state_slot_strides=[page],
                   corr_addrs=[d_corr.data_ptr()], corr_row_strides=[H * RQ * V],
                   kg_addrs=[d_kg.data_ptr()], kg_row_strides=[H * RQ * 2 * K],
                   a_log=d_a[None], dt_bias=d_b[None], sources=fl[1], commit_lens=fl[0],
                   destinations=fl[1], record_rows=d_rows, lower_bound=lb)
    torch.cuda.synchronize()

    # Property over the whole pool: pages that neither call writes are unchanged.
    touched = torch.zeros(w.slots, dtype=torch.bool)
    for b in range(B):
        if slots[b] > 0 and rows[b] >= 0 and (min(pending[rows[b]], RQ) > 0 or flush_lens[b] > 0):
            touched[int(slots[b])] = True
    keep = (~touched).nonzero().flatten().to(DEV)
    assert torch.equal(d_state.view(w.slots, page).index_select(0, keep).view(torch.int32),
                       before.view(w.slots, page).index_select(0, keep).view(torch.int32))
    # Records of rows no request names are unchanged.
    named = set(int(r) for r in rows if r >= 0)
    for r in range(B):
        if r not in named:
            assert_exact(f"config4 corr row {r}", g_corr_f[r], corr[r])

    # Sampled requests: null slots, record row -1, and live ones over all pending counts.
    rng = np.random.default_rng(44)
    live = [b for b in range(B) if slots[b] > 0 and rows[b] >= 0]
    by_n = {}
    for b in live:
        by_n.setdefault(int(pending[rows[b]]), []).append(b)
    R = [0, 7, 13, 22] + [int(rng.choice(by_n[n])) for n in sorted(by_n)]
    R += [int(x) for x in rng.choice(live, 10, replace=False) if int(x) not in R]
    nR = len(R)
    announce(f"config4: oracle on {nR} sampled requests x {H} heads")
    m_slots = np.array([j + 1 if slots[b] > 0 else 0 for j, b in enumerate(R)], np.int32)
    m_rows = np.array([j if rows[b] >= 0 else -1 for j, b in enumerate(R)], np.int32)
    m_state = np.zeros((nR + 1) * page, np.float32)
    m_corr = np.zeros((nR, H, RQ, V), np.float32)
    m_kg = np.zeros((nR, H, RQ, 2 * K), np.uint16)
    m_pend = np.zeros(nR, np.int32)
    for j, b in enumerate(R):
        if slots[b] > 0:
            m_state[(j + 1) * page:(j + 2) * page] = s0[int(slots[b]) * page:(int(slots[b]) + 1) * page]
        if rows[b] >= 0:
            m_corr[j], m_kg[j], m_pend[j] = corr[rows[b]], kg[rows[b]], pending[rows[b]]
    tok = np.concatenate([np.arange(b * T, (b + 1) * T) for b in R])
    m_win = {k: np.ascontiguousarray(v[tok]) for k, v in win.items()}
    m_out = np.zeros((nR * T, H * V), np.uint16)
    oracle.fused_replay_verify(heads=H, tokens=T, batch=nR, q=m_win["q"], k=m_win["k"],
                               v=m_win["v"], raw_g=m_win["raw_g"], raw_beta=m_win["raw_beta"],
                               a_log=a_log, dt_bias=dtb, lower_bound=lb, state=m_state,
                               state_slot_stride=page, state_indices=m_slots, corr=m_corr,
                               kg=m_kg, record_tokens=RQ, record_rows=m_rows, pending=m_pend,
                               out=m_out)
    g_fused = np_of(fused_state)
    for j, b in enumerate(R):
        assert_bf16_close(f"config4 out request {b}", g_out[b * T:(b + 1) * T],
                          m_out[j * T:(j + 1) * T])
        if slots[b] > 0:
            sl = int(slots[b])
            assert_f32_close(f"config4 fused page request {b}", g_fused[sl * page:(sl + 1) * page],
                             m_state[(j + 1) * page:(j + 2) * page])
        if rows[b] >= 0 and slots[b] > 0:
            assert_f32_close(f"config4 corrections request {b}", g_corr_f[rows[b], :, :T],
                             m_corr[j, :, :T])
            assert_exact(f"config4 key/gate request {b}", g_kg_f[rows[b]], m_kg[j])
    # The flush commit of the sampled requests, from the oracle's own fused results.
    m_lens = np.array([flush_lens[b] for b in R], np.int32)
    m_src = m_slots.copy()
    oracle.commit(heads=H, window=RQ, batch=nR, state_bf16=False, state_layers=[m_state],
                  state_slot_strides=[page], corr_layers=[m_corr], corr_row_strides=[H * RQ * V],
                  kg_layers=[m_kg], kg_row_strides=[H * RQ * 2 * K], a_log=a_log[None],
                  dt_bias=dtb[None], sources=m_src, commit_lens=m_lens, destinations=m_src,
                  record_rows=m_rows, lower_bound=lb)
    g_final = np_of(d_state)
    for j, b in enumerate(R):
        if slots[b] > 0:
            sl = int(slots[b])
            assert_f32_close(f"config4 committed page request {b}",
                             g_final[sl * page:(sl + 1) * page],
                             m_state[(j + 1) * page:(j + 2) * page])
    del d_state, before, fused_state
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- limits and variants at size

def _check_sampled(label, R, m, g_out, g_state_pages, g_corr, g_kg, slots, rows, bounds, T,
                   bf16, page):
    close = assert_bf16_close if bf16 else assert_f32_close
    nR = len(R)
    row0 = 0
    for j, b in enumerate(R):
        toks = m["toks"][j]
        n_t = len(toks)
        assert_bf16_close(f"{label} out request {b}", g_out[toks], m["out"][row0:row0 + n_t])
        row0 += n_t
        if slots[b] > 0:
            close(f"{label} page request {b}", g_state_pages(int(slots[b])),
                  m["state"][(j + 1) * page:(j + 2) * page])
            if bounds is not None and bounds[b] > 0:
                close(f"{label} boundary page request {b}", g_state_pages(int(bounds[b])),
                      m["state"][(nR + 1 + j) * page:(nR + 2 + j) * page])
        if rows[b] >= 0 and slots[b] > 0 and n_t > 0:
            assert_f32_close(f"{label} corrections request {b}", g_corr[rows[b]], m["corr"][j])
            assert_exact(f"{label} key/gate request {b}", g_kg[rows[b]], m["kg"][j])


def test_maximum_batch_grid_fused_sampled():
    """65535 requests (the largest grid the kernels take), one head, FP32 pool
    of 65536 slots (4 GiB), ragged null slots and missing record rows; 24
    sampled requests against the oracle, and every page the call must not
    write compared bit for bit."""
    import spec_decode_amd as kda
    H, B, T, RQ, S = 1, 65535, 2, 2, 65536
    page = H * V * K
    g = W._gen(900)
    slots = (W.permutation(g, S - 1) + 1).numpy()
    slots[::997] = 0
    rows = W.permutation(g, B).numpy()
    rows[5::1009] = -1
    pending_row = W.uniform_int(g, -1, RQ + 1, B).numpy()
    a_log, dtb = W.draw_gate_params(g, 1, H)
    corr, kg = W.draw_records(g, B, H, RQ)
    corr, kg = corr.numpy(), W.bits(kg)
    win = window_np(W.draw_window(g, B, T, H))
    d_state = W.draw_state(901, S * page, torch.float32, DEV)
    before = d_state.clone()
    d_corr, d_kg = dev(corr), dev_bf16(kg)
    out = torch.empty((B * T, H * V), dtype=torch.bfloat16, device=DEV)
    announce("max batch: fused H=1 B=65535 T=2")
    kda.kda_fused_replay_verify(heads=H, tokens=T, batch=B, q=dev_bf16(win["q"]),
                                k=dev_bf16(win["k"]), v=dev_bf16(win["v"]),
                                raw_g=dev_bf16(win["raw_g"]), raw_beta=dev_bf16(win["raw_beta"]),
                                a_log=dev(a_log[0].numpy()), dt_bias=dev(dtb[0].numpy()),
                                lower_bound=W.LOWER_BOUND, state=d_state, state_slot_stride=page,
                                state_indices=dev(slots), corr=d_corr, kg=d_kg, record_tokens=RQ,
                                record_rows=dev(rows), pending=dev(pending_row), out=out)
    torch.cuda.synchronize()
    n_of = lambda b: min(max(int(pending_row[rows[b]]), 0), RQ) if rows[b] >= 0 else 0
    touched = torch.zeros(S, dtype=torch.bool)
    for b in range(B):
        if slots[b] > 0 and n_of(b) > 0:
            touched[int(slots[b])] = True
    keep = (~touched).nonzero().flatten().to(DEV)
    assert torch.equal(d_state.view(S, page).index_select(0, keep).view(torch.int32),
                       before.view(S, page).index_select(0, keep).view(torch.int32))
    rng = np.random.default_rng(902)
    R = [0, 1, B - 1, 997, 5] + [int(x) for x in rng.choice(B, 19, replace=False)]
    R = list(dict.fromkeys(R))
    s_host = lambda sl: before[sl * page:(sl + 1) * page].cpu().numpy()
    m = sampled_fused_oracle(R=R, H=H, T=T, RQ=RQ, state_pages=s_host, slots=slots, rows=rows,
                             pending_row=pending_row, corr=corr, kg=kg, win=win,
                             a_log=a_log[0].numpy(), dt_bias=dtb[0].numpy(), lb=W.LOWER_BOUND)
    g_pages = lambda sl: d_state[sl * page:(sl + 1) * page].cpu().numpy()
    _check_sampled("max batch", R, m, np_of(out), g_pages, np_of(d_corr), np_of(d_kg), slots,
                   rows, None, T, False, page)
    del d_state, before
    torch.cuda.empty_cache()


@pytest.mark.parametrize("pool", ["bf16", "f32"])
def test_maximum_batch_grid_commit_sampled(pool):
    """kda_commit at 65535 requests (the largest grid the kernels take), one
    head, in place, with boundary pages of their own (two pools of 65536
    slots: 8 GiB FP32, 4 GiB BF16, so both take their streaming kernels);
    null sources, missing record
    rows, lengths 0..window+1 and boundary lengths drawn; 24 sampled requests
    against the oracle, and every page the call must not write compared bit
    for bit."""
    import spec_decode_amd as kda
    bf16 = pool == "bf16"
    H, B, Q = 1, 65535, 4
    S = 2 * 65536
    page = H * V * K
    g = W._gen(910 + bf16)
    src = (W.permutation(g, 65535) + 1).numpy().astype(np.int32)
    src[::997] = 0
    bnd = (65536 + W.permutation(g, 65536)[:B]).numpy().astype(np.int32)
    bnd[3::5] = 0
    rows = W.permutation(g, B).numpy().astype(np.int32)
    rows[5::1009] = -1
    lens = W.uniform_int(g, 0, Q + 1, B).numpy()
    blen = W.uniform_int(g, 0, Q + 1, B).numpy()
    a_log, dtb = W.draw_gate_params(g, 1, H)
    corr, kg = W.draw_records(g, B, H, Q)
    corr, kg = corr.numpy(), W.bits(kg)
    d_state = W.draw_state(911 + bf16, S * page, torch.bfloat16 if bf16 else torch.float32, DEV)
    before = d_state.clone()
    d_corr, d_kg = dev(corr), dev_bf16(kg)
    announce(f"max batch: commit H=1 B=65535 window {Q}, {pool} pool with boundaries")
    kda.kda_commit(heads=H, window=Q, batch=B,
                   state_dtype=kda.KDA_STATE_BF16 if bf16 else kda.KDA_STATE_F32,
                   state_addrs=[d_state.data_ptr()], state_slot_strides=[page],
                   corr_addrs=[d_corr.data_ptr()], corr_row_strides=[H * Q * V],
                   kg_addrs=[d_kg.data_ptr()], kg_row_strides=[H * Q * 2 * K],
                   a_log=a_log.to(DEV), dt_bias=dtb.to(DEV), sources=dev(src),
                   commit_lens=dev(lens), destinations=dev(src), boundaries=dev(bnd),
                   boundary_lens=dev(blen), record_rows=dev(rows), lower_bound=W.LOWER_BOUND)
    torch.cuda.synchronize()
    live = (lens > 0) & (src > 0) & (rows >= 0)
    touched = torch.zeros(S, dtype=torch.bool)
    touched[torch.from_numpy(src[live]).long()] = True
    bl = live & (blen > 0) & (bnd > 0)
    touched[torch.from_numpy(bnd[bl]).long()] = True
    keep = (~touched).nonzero().flatten().to(DEV)
    bits = torch.int16 if bf16 else torch.int32
    for part in torch.split(keep, 16384):
        assert torch.equal(d_state.view(S, page).index_select(0, part).view(bits),
                           before.view(S, page).index_select(0, part).view(bits))
    rng = np.random.default_rng(912)
    cand = np.flatnonzero(live)
    R = [int(x) for x in np.concatenate([np.flatnonzero(bl)[:6], [B - 1, 0, 5, 997],
                                         rng.choice(cand, 14, replace=False)])]
    R = list(dict.fromkeys(R))
    nR = len(R)
    host = (lambda t: W.bits(t)) if bf16 else (lambda t: t.cpu().numpy())
    m_src = (1 + 2 * np.arange(nR)).astype(np.int32)  # slot 1+2j the page, 2+2j its boundary
    m_bnd = np.where(bl[R], m_src + 1, 0).astype(np.int32)
    mini = np.zeros((1 + 2 * nR) * page, np.uint16 if bf16 else np.float32)
    for j, b in enumerate(R):
        if src[b] > 0:
            mini[m_src[j] * page:(m_src[j] + 1) * page] = host(before[int(src[b]) * page:
                                                                  (int(src[b]) + 1) * page])
    r_of = np.where(rows[R] >= 0, rows[R], 0)
    announce(f"max batch commit: oracle on {nR} sampled requests")
    oracle.commit(heads=H, window=Q, batch=nR, state_bf16=bf16, state_layers=[mini],
                  state_slot_strides=[page], corr_layers=[corr[r_of]],
                  corr_row_strides=[H * Q * V], kg_layers=[kg[r_of]],
                  kg_row_strides=[H * Q * 2 * K], a_log=a_log.numpy(), dt_bias=dtb.numpy(),
                  sources=np.where(src[R] > 0, m_src, 0).astype(np.int32),
                  commit_lens=lens[R], destinations=np.where(src[R] > 0, m_src, 0).astype(np.int32),
                  boundaries=m_bnd, boundary_lens=blen[R],
                  record_rows=np.where(rows[R] >= 0, np.arange(nR), -1).astype(np.int32),
                  lower_bound=W.LOWER_BOUND)
    close = assert_bf16_close if bf16 else assert_f32_close
    for j, b in enumerate(R):
        if src[b] > 0:
            close(f"max batch commit request {b}",
                  host(d_state[int(src[b]) * page:(int(src[b]) + 1) * page]),
                  mini[m_src[j] * page:(m_src[j] + 1) * page])
        if m_bnd[j] > 0:
            close(f"max batch commit request {b} boundary",
                  host(d_state[int(bnd[b]) * page:(int(bnd[b]) + 1) * page]),
                  mini[m_bnd[j] * page:(m_bnd[j] + 1) * page])
    del d_state, before
    torch.cuda.empty_cache()


@pytest.mark.parametrize("pool", ["bf16", "f32"])
def test_large_decode_ragged_windows_and_boundaries_sampled(pool):
    """The large decode shape (H=64, B=512, q=8) on a pool of 1040 slots (2 GiB
    BF16, 4 GiB FP32: the FP32 launch takes the streaming instance, whose S_n
    stores write through): window lengths 0..8 through query_start_loc and
    boundary stores for half the requests (m in 1..9); 30 sampled requests
    against the oracle and the pages nobody writes compared bit for bit."""
    import spec_decode_amd as kda
    bf16 = pool == "bf16"
    H, B, T, RQ, S = 64, 512, 8, 8, 1040
    page = H * V * K
    g = W._gen(910)
    perm = (W.permutation(g, S - 1) + 1).numpy()
    slots = perm[:B].copy()
    slots[::41] = 0
    bounds = perm[B:2 * B].copy()
    bounds[1::2] = 0
    assert slots.size == B and bounds.size == B
    blens = W.uniform_int(g, 1, RQ + 1, B).numpy()
    rows = W.permutation(g, B).numpy()
    rows[3::37] = -1
    pending_row = W.uniform_int(g, 0, RQ, B).numpy()
    lens = W.uniform_int(g, 0, T, B).numpy()
    qsl = np.zeros(B + 1, np.int32)
    qsl[1:] = np.cumsum(lens)
    total = int(qsl[-1])
    a_log, dtb = W.draw_gate_params(g, 1, H)
    corr, kg = W.draw_records(g, B, H, RQ)
    corr, kg = corr.numpy(), W.bits(kg)
    win = {k: np.ascontiguousarray(v[:total]) for k, v in window_np(W.draw_window(g, B, T, H)).items()}
    d_state = W.draw_state(911, S * page, torch.bfloat16 if bf16 else torch.float32, DEV)
    before = d_state.clone()
    d_corr, d_kg = dev(corr), dev_bf16(kg)
    out = torch.zeros((total, H * V), dtype=torch.bfloat16, device=DEV)
    announce(f"large decode ragged + boundaries, {pool} pool")
    kda.kda_fused_replay_verify(heads=H, tokens=T, batch=B, q=dev_bf16(win["q"]),
                                k=dev_bf16(win["k"]), v=dev_bf16(win["v"]),
                                raw_g=dev_bf16(win["raw_g"]), raw_beta=dev_bf16(win["raw_beta"]),
                                a_log=dev(a_log[0].numpy()), dt_bias=dev(dtb[0].numpy()),
                                lower_bound=W.LOWER_BOUND, state=d_state, state_slot_stride=page,
                                state_indices=dev(slots), corr=d_corr, kg=d_kg, record_tokens=RQ,
                                record_rows=dev(rows), pending=dev(pending_row),
                                query_start_loc=dev(qsl), boundaries=dev(bounds),
                                boundary_lens=dev(blens), out=out)
    torch.cuda.synchronize()
    touched = torch.zeros(S, dtype=torch.bool)
    for b in range(B):
        n = min(pending_row[rows[b]], RQ) if rows[b] >= 0 else 0
        if slots[b] > 0 and lens[b] > 0 and n > 0:
            touched[int(slots[b])] = True
            if bounds[b] > 0:
                touched[int(bounds[b])] = True
    keep = (~touched).nonzero().flatten().to(DEV)
    bits = torch.int16 if bf16 else torch.int32
    assert torch.equal(d_state.view(S, page).index_select(0, keep).view(bits),
                       before.view(S, page).index_select(0, keep).view(bits))
    rng = np.random.default_rng(912)
    live = [b for b in range(B) if slots[b] > 0 and rows[b] >= 0]
    by_len = {}
    for b in live:
        by_len.setdefault(int(lens[b]), []).append(b)
    R = [0, 41, 3] + [int(rng.choice(by_len[l])) for l in sorted(by_len)]
    R += [int(x) for x in rng.choice(live, 16, replace=False)]
    R = list(dict.fromkeys(R))
    s_host = lambda sl: np_of(before[sl * page:(sl + 1) * page])
    m = sampled_fused_oracle(R=R, H=H, T=T, RQ=RQ, state_pages=s_host, slots=slots, rows=rows,
                             pending_row=pending_row, corr=corr, kg=kg, win=win,
                             a_log=a_log[0].numpy(), dt_bias=dtb[0].numpy(), lb=W.LOWER_BOUND,
                             qsl=qsl, bounds=bounds, blens=blens,
                             state_dtype=np.uint16 if bf16 else np.float32)
    g_pages = lambda sl: np_of(d_state[sl * page:(sl + 1) * page])
    _check_sampled("ragged+bnd", R, m, np_of(out), g_pages, np_of(d_corr), np_of(d_kg), slots,
                   rows, bounds, T, bf16, page)
    del d_state, before
    torch.cuda.empty_cache()
