"""GPU parity on small seeded cases that span every template instance (window
1..8, BF16/FP32 state, align on/off, verify/fused) plus the edge cases: null
slots, record row -1, n = 0, n above the capacity, negative pending, m > n,
in-place commits, per-layer stride tables and more layers than one launch
holds. Every output is compared with the FP64 oracle element by element."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _compare import assert_exact, assert_f32_close
from _kda_cases import (CONV_LAYOUTS, DEV, announce, conv_pool_build, conv_pool_layout, dev,
                        dev_bf16, np_of, run_commit_case, run_conv_case, run_verify_case,
                        window_np)

pytestmark = pytest.mark.gpu

K = V = 128


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import spec_decode_amd  # noqa: F401  (fails loudly without libkda.so)

    torch.cuda.init()
    yield


# ---------------------------------------------------------------- plan steps

@pytest.mark.parametrize("null_slot", [0, 2])
@pytest.mark.parametrize("eager", [False, True])
def test_plan_steps_bit_exact(eager, null_slot):
    import spec_decode_amd as kda

    rng = np.random.default_rng(3)
    B, rows_n = 777, 900
    si = rng.integers(-2, 5, B).astype(np.int32)
    rows = rng.permutation(rows_n)[:B].astype(np.int32)
    rows[rng.random(B) < 0.1] = -1
    lens = rng.integers(-3, 12, B).astype(np.int32)
    pending = rng.integers(-5, 20, rows_n).astype(np.int32)
    eg = (rng.random(B) < 0.3).astype(np.int32) if eager else None
    announce(f"plan: defer B={B} eager={eager} null_slot={null_slot}")
    d_lens, d_pend = dev(lens), dev(pending)
    kda.kda_defer_commit(batch=B, state_indices=dev(si), commit_lens=d_lens,
                         record_rows=dev(rows), pending=d_pend,
                         eager=None if eg is None else dev(eg), null_slot=null_slot)
    torch.cuda.synchronize()
    r_lens, r_pend = lens.copy(), pending.copy()
    oracle.defer(si, r_lens, rows, r_pend, eg, null_slot=null_slot)
    assert_exact("defer commit_lens", np_of(d_lens), r_lens)
    assert_exact("defer pending", np_of(d_pend), r_pend)
    for q in (1, 4, 8):
        announce(f"plan: flush B={B} q={q}")
        outs = [torch.full((B,), -99, dtype=torch.int32, device=DEV) for _ in range(4)]
        kda.kda_flush_plan(batch=B, spec_query_len=q, state_indices=dev(si),
                           record_rows=dev(rows), pending=dev(r_pend), commit_lens=outs[0],
                           final_indices=outs[1], boundaries=outs[2], boundary_lens=outs[3],
                           null_slot=null_slot)
        torch.cuda.synchronize()
        ref = oracle.flush_plan(si, rows, r_pend, q, null_slot=null_slot)
        for name, g, r in zip(("commit_lens", "final", "boundaries", "boundary_lens"), outs, ref):
            assert_exact(f"flush {name} q={q}", np_of(g), r)


# ---------------------------------------------------------------- decay

@pytest.mark.parametrize("lb", [-5.0, 0.0, -0.5])
def test_decay(lb):
    import spec_decode_amd as kda

    g = W._gen(5)
    N, H = 37, 5
    raw = W.bf16(W.normal(g, (N, H, K)) * 3.0)
    raw[0, 0, :4] = torch.tensor([60.0, -60.0, 0.0, -0.0]).to(torch.bfloat16)
    a_log, dtb = W.draw_gate_params(g, 1, H)
    announce(f"decay N={N} H={H} lb={lb}")
    out = torch.empty((N, H, K), dtype=torch.float32, device=DEV)
    kda.kda_decay(raw.to(DEV), a_log[0].to(DEV), dtb[0].to(DEV), lb, out)
    torch.cuda.synchronize()
    ref = oracle.decay_buf(W.bits(raw), a_log[0].numpy(), dtb[0].numpy(), lb)
    assert_f32_close("decay", np_of(out), ref)
    if lb == 0.0:
        assert np.all(np_of(out) == 1.0)


@pytest.mark.parametrize("N", [4096, 4099])
def test_decay_full_size(N):
    """The large decode batch's raw gates (4096 tokens x 64 heads x 128, as the
    benchmark's decay workload), and 3 tokens more: more 8-byte chunks than the
    capped grid has threads, so every thread takes a second chunk, the last
    pass ragged. Every element against the oracle."""
    import spec_decode_amd as kda

    g = W._gen(6)
    H = 64
    assert N * H * K // 4 > 256 * 64 * 256
    raw = W.bf16(W.normal(g, (N, H, K)) * 3.0)
    a_log, dtb = W.draw_gate_params(g, 1, H)
    announce(f"decay N={N} H={H} (grid-stride)")
    out = torch.full((N, H, K), float("nan"), dtype=torch.float32, device=DEV)
    kda.kda_decay(raw.to(DEV), a_log[0].to(DEV), dtb[0].to(DEV), W.LOWER_BOUND, out)
    torch.cuda.synchronize()
    ref = oracle.decay_buf(W.bits(raw), a_log[0].numpy(), dtb[0].numpy(), W.LOWER_BOUND)
    assert_f32_close("decay full size", np_of(out), ref)


# ---------------------------------------------------------------- commit

def _commit_inputs(seed, L, H, B, Q, bf16, slots, pad=(0,)):
    g = W._gen(seed)
    page = H * V * K
    strides = [page + pad[l % len(pad)] for l in range(L)]
    dt = torch.bfloat16 if bf16 else torch.float32
    states, corrs, kgs = [], [], []
    for l in range(L):
        s = W.draw_state(seed * 31 + l, slots * strides[l], dt)
        states.append(W.bits(s) if bf16 else s.numpy().copy())
        c, k = W.draw_records(g, B, H, Q)
        corrs.append(c.numpy().copy())
        kgs.append(W.bits(k))
    a_log, dtb = W.draw_gate_params(g, L, H)
    return states, strides, corrs, kgs, a_log.numpy(), dtb.numpy()


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("Q", [1, 2, 3, 4, 5, 6, 7, 8])
def test_commit_windows(bf16, Q):
    H, B, L, S = 3, 7, 1, 16
    states, strides, corrs, kgs, a_log, dtb = _commit_inputs(100 + Q, L, H, B, Q, bf16, S)
    rng = np.random.default_rng(Q)
    perm = rng.permutation(np.arange(1, S))
    src = perm[:B].astype(np.int32)
    dst = perm[B:2 * B].astype(np.int32)
    lens = rng.integers(0, Q + 3, B).astype(np.int32)  # includes 0 and > Q
    lens[0], lens[1] = 0, Q + 2
    src[2] = 0  # null source: no-op
    dst[3] = 0  # null destination: no-op
    run_commit_case(H=H, B=B, Q=Q, bf16=bf16, layers_state=states, strides=strides,
                    corr_layers=corrs, kg_layers=kgs, a_log=a_log, dt_bias=dtb, src=src,
                    lens=lens, dst=dst, label=f"commit Q={Q} bf16={bf16}")


@pytest.mark.parametrize("bf16", [True, False])
def test_commit_align_multilayer_strides(bf16):
    H, B, L, Q, S = 2, 6, 3, 8, 24
    states, strides, corrs, kgs, a_log, dtb = _commit_inputs(7, L, H, B, Q, bf16, S,
                                                             pad=(0, 64, 128))
    rng = np.random.default_rng(8)
    perm = rng.permutation(np.arange(1, S))
    src, dst, bnd = (perm[i * B:(i + 1) * B].astype(np.int32) for i in range(3))
    lens = np.array([8, 5, 3, 1, 6, 0], np.int32)
    blen = np.array([3, 0, 7, 1, 6, 2], np.int32)  # m = 0, m > n, m = n, lens 0
    bnd[4] = 0  # null boundary: no boundary store
    rows = rng.permutation(B).astype(np.int32)
    run_commit_case(H=H, B=B, Q=Q, bf16=bf16, layers_state=states, strides=strides,
                    corr_layers=corrs, kg_layers=kgs, a_log=a_log, dt_bias=dtb, src=src,
                    lens=lens, dst=dst, bnd=bnd, blen=blen, rows=rows,
                    label=f"commit align L={L} bf16={bf16}")


def test_commit_inplace_record_rows_fp32():
    H, B, L, Q, S = 4, 5, 1, 8, 8
    states, strides, corrs, kgs, a_log, dtb = _commit_inputs(9, L, H, B, Q, False, S)
    src = np.array([1, 2, 3, 4, 5], np.int32)
    lens = np.array([8, 1, 0, 4, 7], np.int32)
    rows = np.array([4, -1, 2, 0, 1], np.int32)  # row -1: no-op
    run_commit_case(H=H, B=B, Q=Q, bf16=False, layers_state=states, strides=strides,
                    corr_layers=corrs, kg_layers=kgs, a_log=a_log, dt_bias=dtb, src=src,
                    lens=lens, dst=src.copy(), rows=rows, label="commit in-place fp32")


def test_commit_more_layers_than_one_launch():
    H, B, L, Q, S = 1, 2, 18, 3, 5
    states, strides, corrs, kgs, a_log, dtb = _commit_inputs(11, L, H, B, Q, True, S, pad=(0, 8))
    src = np.array([1, 2], np.int32)
    dst = np.array([3, 4], np.int32)
    lens = np.array([3, 2], np.int32)
    run_commit_case(H=H, B=B, Q=Q, bf16=True, layers_state=states, strides=strides,
                    corr_layers=corrs, kg_layers=kgs, a_log=a_log, dt_bias=dtb, src=src,
                    lens=lens, dst=dst, label="commit L=18")


# ---------------------------------------------------------------- verify / fused

def _vf_case(seed, H, B, T, RQ, S, null_rows=(), norec_rows=(), bf16=False):
    """A small verify/fused case; bf16 gives the pool as BF16 bits (the FP32
    draw rounded to nearest even)."""
    c = W.small_fused_case(seed, H, B, T, RQ, S, null_rows=null_rows, no_record_rows=norec_rows)
    state = W.bits(c["state"].to(torch.bfloat16)) if bf16 else c["state"].numpy().copy()
    return dict(state=state, slots=c["state_indices"].numpy().copy(),
                rows=c["record_rows"].numpy().copy(), corr=c["corr"].numpy().copy(),
                kg=W.bits(c["kg"]), a_log=c["a_log"][0].numpy(), dt_bias=c["dt_bias"][0].numpy(),
                win=window_np(c["window"]))


def _rescaled(bits_np, seed, records=False):
    """Window keys [N, H, K] or key/gate records [..., 2K] (uint16 bits) with
    each key rescaled to a norm from W.KEY_NORMS (0, 1e-4, 1e-2, 1, 30)."""
    t = torch.from_numpy(bits_np.view(np.int16)).view(torch.bfloat16)
    g = W._gen(seed)
    return W.bits(W.rescale_record_keys(g, t) if records else W.rescale_keys(g, t))


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("kind", ["verify", "fused", "commit"])
def test_key_norm_edge(kind, bf16):
    """Keys of norm 0, 1e-4, 1e-2, 1 and 30, in the window and in the records:
    every use normalises k by (sum k^2 + 1e-6)^-1/2 (commit page, KdaCommit
    kernel; fused page, KdaFused.kernel, the new and the recorded keys), so the
    eps dominates at 1e-4, matters at 1e-2, and a zero key contributes nothing."""
    H, T, RQ = 3, 8, 8
    if kind == "commit":
        B, L, S = 6, 1, 16
        states, strides, corrs, kgs, a_log, dtb = _commit_inputs(1300, L, H, B, RQ, bf16, S)
        kgs = [_rescaled(kgs[0], 1301, records=True)]
        src = np.arange(1, B + 1, dtype=np.int32)
        lens = np.array([8, 8, 5, 3, 1, 8], np.int32)
        run_commit_case(H=H, B=B, Q=RQ, bf16=bf16, layers_state=states, strides=strides,
                        corr_layers=corrs, kg_layers=kgs, a_log=a_log, dt_bias=dtb, src=src,
                        lens=lens, dst=src.copy(), label=f"commit key norms bf16={bf16}")
        return
    B = 6
    c = _vf_case(1310 + bf16, H, B, T, RQ, 10, bf16=bf16)
    win = dict(c["win"])
    win["k"] = _rescaled(win["k"], 1320)
    kg = _rescaled(c["kg"], 1321, records=True)
    pending = np.full(B, RQ, np.int32)
    pending[:3] = [0, 3, 5]
    run_verify_case(fused=kind == "fused", H=H, B=B, T=T, RQ=RQ, state=c["state"],
                    slots=c["slots"], corr=c["corr"], kg=kg, a_log=c["a_log"],
                    dt_bias=c["dt_bias"], win=win, rows=c["rows"],
                    pending=pending if kind == "fused" else None,
                    label=f"{kind} key norms bf16={bf16}")


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("lb", [0.0, -0.5, -60.0])
@pytest.mark.parametrize("kind", ["verify", "fused", "commit", "fused_conv"])
def test_lower_bound_edges(kind, lb, bf16):
    """The decay's lower bound at its degenerate ends, through every kernel that
    forms decays (fused page, KdaFused.decay; commit page, KdaCommit): lb = 0
    gives d = 1 (the plain delta rule, nothing decays), lb = -60 drives d to
    about e^-30 or below, so the decay products underflow within a window, and
    -0.5 sits between. The workloads use -5 only."""
    H, T, RQ = 3, 8, 8
    if kind == "commit":
        B, L, S = 6, 1, 16
        states, strides, corrs, kgs, a_log, dtb = _commit_inputs(1400, L, H, B, RQ, bf16, S)
        src = np.arange(1, B + 1, dtype=np.int32)
        lens = np.array([8, 8, 5, 3, 1, 2], np.int32)
        run_commit_case(H=H, B=B, Q=RQ, bf16=bf16, layers_state=states, strides=strides,
                        corr_layers=corrs, kg_layers=kgs, a_log=a_log, dt_bias=dtb, src=src,
                        lens=lens, dst=(src + B).astype(np.int32), lb=lb,
                        label=f"commit lb={lb} bf16={bf16}")
        return
    B = 6
    pending = np.array([0, 8, 3, 5, 1, 8], np.int32)
    if kind == "fused_conv":
        c = _conv_case(1410 + bf16, H, B, T, RQ, 10, bf16=bf16)
        _run_conv(c, H, B, T, RQ, pending, f"fused conv lb={lb} bf16={bf16}", lb=lb)
        return
    c = _vf_case(1420 + bf16, H, B, T, RQ, 10, bf16=bf16)
    run_verify_case(fused=kind == "fused", H=H, B=B, T=T, RQ=RQ, state=c["state"],
                    slots=c["slots"], corr=c["corr"], kg=c["kg"], a_log=c["a_log"],
                    dt_bias=c["dt_bias"], win=c["win"], rows=c["rows"],
                    pending=pending if kind == "fused" else None, lb=lb,
                    label=f"{kind} lb={lb} bf16={bf16}")


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("kind", ["verify", "fused", "commit", "fused_conv"])
def test_nonzero_null_slot(kind, bf16):
    """The null slot is an argument (the kernels page's plan steps and the
    verify/commit operands compare slots against it): with null_slot = 3,
    every slot 1..3 marks padding just as 0 does, so those items write zeros
    to o (verify, fused) or nothing at all (commit), and their pages, records
    and windows stay untouched."""
    H, T, RQ, NULL = 3, 8, 8, 3
    if kind == "commit":
        B, L, S = 8, 1, 20
        states, strides, corrs, kgs, a_log, dtb = _commit_inputs(1500, L, H, B, RQ, bf16, S)
        src = np.array([1, 4, 3, 5, 6, 7, 2, 8], np.int32)   # 1, 3, 2: null sources
        dst = np.array([9, 10, 11, 2, 12, 13, 14, 15], np.int32)  # 2: a null destination
        bnd = np.array([16, 3, 17, 18, 19, 0, 1, 16], np.int32)
        blen = np.array([2, 3, 1, 2, 4, 1, 1, 0], np.int32)
        lens = np.array([4, 5, 3, 6, 8, 2, 7, 3], np.int32)
        bnd[7] = 0  # (16 is request 0's boundary)
        run_commit_case(H=H, B=B, Q=RQ, bf16=bf16, layers_state=states, strides=strides,
                        corr_layers=corrs, kg_layers=kgs, a_log=a_log, dt_bias=dtb, src=src,
                        lens=lens, dst=dst, bnd=bnd, blen=blen, null_slot=NULL,
                        label=f"commit null_slot={NULL} bf16={bf16}")
        return
    B = 8
    pending = np.array([0, 8, 3, 5, 1, 8, 2, 6], np.int32)
    if kind == "fused_conv":
        c = _conv_case(1510 + bf16, H, B, T, RQ, 12, bf16=bf16)
        assert (c["slots"] <= NULL).any() and (c["slots"] > NULL).sum() >= 4
        _run_conv(c, H, B, T, RQ, pending, f"fused conv null_slot={NULL} bf16={bf16}",
                  null_slot=NULL)
        return
    c = _vf_case(1520 + bf16, H, B, T, RQ, 12, bf16=bf16)
    assert (c["slots"] <= NULL).any() and (c["slots"] > NULL).sum() >= 4
    run_verify_case(fused=kind == "fused", H=H, B=B, T=T, RQ=RQ, state=c["state"],
                    slots=c["slots"], corr=c["corr"], kg=c["kg"], a_log=c["a_log"],
                    dt_bias=c["dt_bias"], win=c["win"], rows=c["rows"],
                    pending=pending if kind == "fused" else None, null_slot=NULL,
                    label=f"{kind} null_slot={NULL} bf16={bf16}")


@pytest.mark.parametrize("q_scale", [1.0, 0.05])
def test_fused_conv_q_scale(q_scale):
    """The query scale of the convolution prologue is an argument (fused page,
    KdaFused.kernel: q is normalised, then scaled); the workloads pass 128^-1/2."""
    H, B, T, RQ = 3, 5, 8, 8
    c = _conv_case(1530, H, B, T, RQ, 9, null_rows=(2,), norec_rows=(4,))
    pending = np.array([0, 8, 3, 5, 1], np.int32)
    _run_conv(c, H, B, T, RQ, pending, f"fused conv q_scale={q_scale}", q_scale=q_scale)


@pytest.mark.parametrize("norm_eps", [0.0, 1e-3, 1.0])
@pytest.mark.parametrize("fused", [False, True])
def test_gated_output_norm_eps(fused, norm_eps):
    """The gated RMSNorm's eps is an argument (fused page, KdaFused.kernel,
    output stage: rstd = (mean(o^2) + eps)^-1/2); the workloads pass 1e-5."""
    H, B, T, RQ = 3, 5, 8, 8
    c = _vf_case(1540, H, B, T, RQ, 9, null_rows=(1,), norec_rows=(3,))
    gate, weight, _ = W.draw_output_stage(W._gen(1541), B, T, H)
    pending = np.array([0, 8, 3, 5, 1], np.int32)
    run_verify_case(fused=fused, H=H, B=B, T=T, RQ=RQ, state=c["state"], slots=c["slots"],
                    corr=c["corr"], kg=c["kg"], a_log=c["a_log"], dt_bias=c["dt_bias"],
                    win=c["win"], rows=c["rows"], pending=pending if fused else None,
                    gate=W.bits(gate), norm_weight=weight.numpy(), norm_eps=norm_eps,
                    label=f"gated output fused={fused} eps={norm_eps}")


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 6, 7, 8])
def test_verify_windows(T, bf16):
    H, B = 3, 5
    for RQ in sorted({T, 8}):
        c = _vf_case(200 + T, H, B, T, RQ, 9, null_rows=(1,), norec_rows=(3,), bf16=bf16)
        run_verify_case(fused=False, H=H, B=B, T=T, RQ=RQ, state=c["state"], slots=c["slots"],
                        corr=c["corr"], kg=c["kg"], a_log=c["a_log"], dt_bias=c["dt_bias"],
                        win=c["win"], rows=c["rows"], label=f"verify T={T} RQ={RQ}")
    # record_rows = NULL: request b writes row b
    c = _vf_case(300 + T, H, B, T, T, 9, bf16=bf16)
    run_verify_case(fused=False, H=H, B=B, T=T, RQ=T, state=c["state"], slots=c["slots"],
                    corr=c["corr"], kg=c["kg"], a_log=c["a_log"], dt_bias=c["dt_bias"],
                    win=c["win"], rows=None, label=f"verify T={T} rows=NULL")


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 6, 7, 8])
def test_fused_windows(T, bf16):
    H, B = 3, 6
    for RQ in sorted({T, 8}):
        c = _vf_case(400 + T, H, B, T, RQ, 10, null_rows=(1,), norec_rows=(3,), bf16=bf16)
        rng = np.random.default_rng(T * 10 + RQ)
        pending = rng.integers(0, RQ + 1, B).astype(np.int32)
        rows = c["rows"]
        # edge pending values on live rows: 0, RQ, above RQ, negative, 1..4 and 5..8
        live = [b for b in range(B) if b not in (1, 3)]
        edge = [0, RQ, RQ + 3, -2]
        for b, e in zip(live, edge):
            pending[rows[b]] = e
        run_verify_case(fused=True, H=H, B=B, T=T, RQ=RQ, state=c["state"], slots=c["slots"],
                        corr=c["corr"], kg=c["kg"], a_log=c["a_log"], dt_bias=c["dt_bias"],
                        win=c["win"], rows=rows, pending=pending, label=f"fused T={T} RQ={RQ}")


@pytest.mark.parametrize("bf16", [False, True])
def test_fused_every_pending_count(bf16):
    """One request per n = 0..8 (the replay's one- and two-MFMA paths)."""
    H, B, T, RQ = 2, 9, 4, 8
    c = _vf_case(77, H, B, T, RQ, 12, bf16=bf16)
    pending = np.zeros(B, np.int32)
    for b in range(B):
        pending[c["rows"][b]] = b
    run_verify_case(fused=True, H=H, B=B, T=T, RQ=RQ, state=c["state"], slots=c["slots"],
                    corr=c["corr"], kg=c["kg"], a_log=c["a_log"], dt_bias=c["dt_bias"],
                    win=c["win"], rows=c["rows"], pending=pending, label="fused n=0..8")


@pytest.mark.parametrize("bf16", [False, True])
def test_fused_padded_slot_stride(bf16):
    H, B, T, RQ, S = 2, 4, 3, 4, 6
    stride = H * V * K + 264 if bf16 else H * V * K + 260  # 16-byte slots, not 256-byte
    g = W._gen(55)
    state = W.draw_state(56, S * stride, torch.float32)
    state = W.bits(state.to(torch.bfloat16)) if bf16 else state.numpy().copy()
    a_log, dtb = W.draw_gate_params(g, 1, H)
    corr, kg = W.draw_records(g, B, H, RQ)
    win = window_np(W.draw_window(g, B, T, H))
    slots = np.array([5, 2, 0, 3], np.int32)
    rows = np.array([1, 3, 0, 2], np.int32)
    pending = np.array([2, 4, 1, 3], np.int32)
    run_verify_case(fused=True, H=H, B=B, T=T, RQ=RQ, state=state, slots=slots,
                    corr=corr.numpy().copy(), kg=W.bits(kg), a_log=a_log[0].numpy(),
                    dt_bias=dtb[0].numpy(), win=win, rows=rows, pending=pending, stride=stride,
                    label="fused padded stride")


def test_page_rw_probe_leaves_pool_unchanged():
    import spec_decode_amd as kda

    H, B, S = 3, 5, 8
    g = W._gen(66)
    state = W.draw_state(67, S * H * V * K, torch.float32).to(DEV)
    before = state.clone()
    slots = dev(np.array([3, 0, 7, 1, 5], np.int32))
    announce("page_rw_probe H=3 B=5")
    kda.kda_page_rw_probe(heads=H, batch=B, state=state, state_slot_stride=H * V * K,
                          state_indices=slots)
    torch.cuda.synchronize()
    assert torch.equal(state.view(torch.int32), before.view(torch.int32))


@pytest.mark.parametrize("T,bf16", [(1, False), (3, False), (4, False), (8, False), (3, True),
                                    (8, True)])
@pytest.mark.parametrize("fused", [False, True])
def test_gated_output_stage(T, fused, bf16):
    H, B, RQ = 3, 5, 8
    c = _vf_case(500 + T, H, B, T, RQ, 9, null_rows=(1,), norec_rows=(3,), bf16=bf16)
    gate, weight, eps = W.draw_output_stage(W._gen(600 + T), B, T, H)
    rng = np.random.default_rng(T)
    pending = rng.integers(0, RQ + 1, B).astype(np.int32)
    run_verify_case(fused=fused, H=H, B=B, T=T, RQ=RQ, state=c["state"], slots=c["slots"],
                    corr=c["corr"], kg=c["kg"], a_log=c["a_log"], dt_bias=c["dt_bias"],
                    win=c["win"], rows=c["rows"], pending=pending if fused else None,
                    gate=W.bits(gate), norm_weight=weight.numpy(), norm_eps=eps,
                    label=f"gated output fused={fused} T={T}")


@pytest.mark.parametrize("fused", [False, True])
def test_gated_output_rounding_point_exact(fused):
    """The hand-derived case whose gated output depends on rounding o to BF16
    both in the sum of squares and in the product (fused page, KdaFused.kernel,
    the output stage): the kernel must give the closed-form bits exactly."""
    import spec_decode_amd as kda
    from _pinned_cases import gated_rounding_case
    args, want, _ = gated_rounding_case()
    announce(f"gated output rounding point, fused={fused}")
    out = torch.zeros((1, V), dtype=torch.bfloat16, device=DEV)
    out.view(torch.int16).fill_(0x7FFF)
    d = {}
    for name, val in args.items():
        if isinstance(val, np.ndarray):
            d[name] = dev_bf16(val) if val.dtype == np.uint16 else dev(val)
        else:
            d[name] = val
    if fused:
        kda.kda_fused_replay_verify(out=out, pending=dev(np.zeros(1, np.int32)), **d)
    else:
        kda.kda_verify(out=out, **d)
    torch.cuda.synchronize()
    assert_exact("gated rounding-point output", np_of(out)[0], want)


# ---------------------------------------------------------------- fused + convolution

def _conv_case(seed, H, B, T, RQ, S, bf16=False, dim_first=True, null_rows=(), norec_rows=(),
               layout=None):
    c = _vf_case(seed, H, B, T, RQ, S, null_rows=null_rows, norec_rows=norec_rows, bf16=bf16)
    cv = W.draw_conv_inputs(W._gen(seed + 7), B, T, H, RQ, S)
    win = W.bits(cv.window)  # [S, 3HK, RQ + 2]
    c["strides"] = conv_pool_layout(S, H, RQ + 2, dim_first, layout)
    c["pool"] = conv_pool_build(win, c["strides"], seed + 11)
    c.update(x=W.bits(cv.x), pitch=cv.pitch, conv_w=W.bits(cv.weight), conv_b=W.bits(cv.bias))
    return c


def _run_conv(c, H, B, T, RQ, pending, label, bias=True, **kw):
    return run_conv_case(H=H, B=B, T=T, RQ=RQ, state=c["state"], slots=c["slots"],
                         corr=c["corr"], kg=c["kg"], a_log=c["a_log"], dt_bias=c["dt_bias"],
                         raw_g=c["win"]["raw_g"], raw_beta=c["win"]["raw_beta"], x=c["x"],
                         pitch=c["pitch"], conv_w=c["conv_w"],
                         conv_b=c["conv_b"] if bias else None, pool=c["pool"],
                         strides=c["strides"], rows=c["rows"], pending=pending, label=label,
                         **kw)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 6, 7, 8])
def test_fused_conv_windows(T, bf16):
    H, B = 3, 6
    for RQ in sorted({T, 8}):
        c = _conv_case(700 + T, H, B, T, RQ, 10, bf16=bf16, dim_first=(T + RQ) % 2 == 0,
                       null_rows=(1,), norec_rows=(3,))
        rng = np.random.default_rng(T * 10 + RQ)
        pending = rng.integers(0, RQ + 1, B).astype(np.int32)
        live = [b for b in range(B) if b not in (1, 3)]
        for b, e in zip(live, [0, RQ, RQ + 3, -2]):
            pending[c["rows"][b]] = e
        _run_conv(c, H, B, T, RQ, pending, f"fused conv T={T} RQ={RQ}")


@pytest.mark.parametrize("dim_first", [True, False])
def test_fused_conv_every_pending_count(dim_first):
    """One request per n = 0..8: every window offset 0..7, no convolution bias."""
    H, B, T, RQ = 2, 9, 4, 8
    c = _conv_case(777, H, B, T, RQ, 12, dim_first=dim_first)
    pending = np.zeros(B, np.int32)
    for b in range(B):
        pending[c["rows"][b]] = b
    _run_conv(c, H, B, T, RQ, pending, "fused conv n=0..8", bias=False)


@pytest.mark.parametrize("layout", CONV_LAYOUTS)
@pytest.mark.parametrize("T,RQ,bf16", [(8, 8, False), (3, 8, True), (2, 3, False), (5, 6, True)])
def test_fused_conv_pool_layouts(layout, T, RQ, bf16):
    """Every window pool layout: the packed dim-first blocks (including windows
    of 5 and 8 entries, whose blocks are not a whole number of 64 chunks) and
    the strided forms, with the padding between windows left alone."""
    H, B = 3, 6
    c = _conv_case(950 + T + RQ, H, B, T, RQ, 9, bf16=bf16, null_rows=(2,), norec_rows=(4,),
                   layout=layout)
    pending = np.random.default_rng(T + RQ).integers(0, RQ + 1, B).astype(np.int32)
    pending[c["rows"][0]] = RQ
    _run_conv(c, H, B, T, RQ, pending, f"fused conv {layout} T={T} RQ={RQ}")


@pytest.mark.parametrize("layout", ["window_major", "window_major_padded"])
def test_fused_conv_unaligned_input_rows(layout):
    """Input rows whose pitch is not a multiple of 8 elements: a window-major
    pool then goes through the strided code instead of the 16-byte stage."""
    H, B, T, RQ = 3, 6, 8, 8
    c = _conv_case(960, H, B, T, RQ, 9, null_rows=(2,), norec_rows=(4,), layout=layout)
    pitch2 = c["pitch"] + 3
    x2 = np.zeros((B * T, pitch2), np.uint16)
    x2[:, :c["pitch"]] = c["x"].reshape(B * T, c["pitch"])
    c.update(x=x2, pitch=pitch2)
    pending = np.array([0, 8, 3, 5, 1, 7], np.int32)
    _run_conv(c, H, B, T, RQ, pending, f"fused conv {layout} pitch={pitch2}")


@pytest.mark.parametrize("bf16", [False, True])
def test_fused_conv_window_major_matches_strided(bf16):
    """The window-major 16-byte stage and the strided code give the same bits:
    the same inputs through a window-major pool (rows of 3HK) and through one
    with rows of 3HK + 3 (the strided code), every output compared exactly,
    the windows by their logical entries."""
    H, B, T, RQ, S = 3, 6, 8, 8, 9
    pending = np.array([0, 8, 3, 5, 1, 7], np.int32)
    res = []
    for layout in ("window_major", "window_major_odd"):
        c = _conv_case(970 + bf16, H, B, T, RQ, S, bf16=bf16, null_rows=(2,), norec_rows=(4,),
                       layout=layout)
        gpu, _ = _run_conv(c, H, B, T, RQ, pending, f"fused conv {layout} bf16={bf16}")
        ss, cs, ts = c["strides"]
        idx = (np.arange(S)[:, None, None] * ss + np.arange(3 * H * K)[None, :, None] * cs +
               np.arange(RQ + 2)[None, None, :] * ts)
        res.append(dict(gpu, pool=gpu["pool"][idx]))
    for name in ("out", "state", "corr", "kg", "pool"):
        assert_exact(f"window-major stage vs strided code: {name}", res[0][name], res[1][name])


@pytest.mark.parametrize("T,bf16", [(3, False), (8, False), (4, True)])
def test_fused_conv_gated_output(T, bf16):
    H, B, RQ = 3, 5, 8
    c = _conv_case(800 + T, H, B, T, RQ, 9, bf16=bf16, null_rows=(2,), norec_rows=(4,))
    gate, weight, eps = W.draw_output_stage(W._gen(900 + T), B, T, H)
    pending = np.random.default_rng(T).integers(0, RQ + 1, B).astype(np.int32)
    _run_conv(c, H, B, T, RQ, pending, f"fused conv gated T={T}", gate=W.bits(gate),
              norm_weight=weight.numpy(), norm_eps=eps)


# ---------------------------------------------------------------- gate projection

def _gate_proj_gpu(fa_bits, pitch, col0, fb_bits, N, H):
    """Runs kda_gate_projection with F_A as columns col0.. of packed rows of
    width pitch; returns raw_g bits [N, H*128]."""
    import spec_decode_amd as kda
    packed = np.zeros((N, pitch), np.uint16)
    packed[:, col0:col0 + K] = fa_bits
    d_packed = dev_bf16(packed)
    out = torch.zeros((N, H * K), dtype=torch.bfloat16, device=DEV)
    out.view(torch.int16).fill_(0x7FFF)
    kda.kda_gate_projection(tokens=N, heads=H, f_a=d_packed[:, col0:], f_a_row_stride=pitch,
                            f_b=dev_bf16(fb_bits), raw_g=out)
    torch.cuda.synchronize()
    return np_of(out)


@pytest.mark.parametrize("N,H,pitch,col0", [(1, 1, 128, 0), (17, 3, 136, 8), (64, 2, 128, 0),
                                            (100, 3, 1000, 600), (257, 2, 264, 128),
                                            (130, 5, 256, 64), (129, 9, 128, 0)])
def test_gate_projection_exact_grid(N, H, pitch, col0):
    """On the generator's exact grid every FP32 partial sum is exact, so the
    BF16 result is bit-identical to the oracle's."""
    announce(f"gate projection exact N={N} H={H} pitch={pitch}")
    fa, fb = W.draw_gate_factors(W._gen(1000 + N), N, H)
    got = _gate_proj_gpu(W.bits(fa), pitch, col0, W.bits(fb), N, H)
    want = oracle.gate_projection(W.bits(fa), W.bits(fb))
    assert_exact("raw_g", got, want)


def test_gate_projection_general_inputs():
    """General BF16 factors: within one BF16 ulp of the FP64 product rounded
    once (a different FP32 summation order can cross a rounding boundary),
    and equal almost everywhere."""
    from _compare import bf16_mismatch
    N, H = 200, 4
    announce(f"gate projection general N={N} H={H}")
    fa, fb = W.draw_gate_factors(W._gen(2000), N, H, exact=False)
    got = _gate_proj_gpu(W.bits(fa), 128, 0, W.bits(fb), N, H)
    want = oracle.gate_projection(W.bits(fa), W.bits(fb))
    assert not bf16_mismatch(got, want, ulps=1).any()
    assert (got == want).mean() > 0.999


# ---------------------------------------------------------------- variable-length windows

@pytest.mark.parametrize("T,fused,bf16,gated", [(3, False, False, False), (8, False, True, False),
                                                (4, True, False, False), (8, True, False, False),
                                                (5, True, True, True), (2, True, False, True)])
def test_variable_length_windows(T, fused, bf16, gated):
    """Request lengths 0..T (one above T, clamped) through query_start_loc, with
    a null slot, a request without a record row and rows nobody owns."""
    H, B, RQ = 3, 7, 8
    c = _vf_case(1100 + T, H, B, T, RQ, 10, null_rows=(5,), norec_rows=(4,), bf16=bf16)
    lens = [T, 0, 1, T + 2, T - 1, 2, 0]
    qsl = np.zeros(B + 1, np.int32)
    qsl[1:] = np.cumsum(lens)
    rows_total = int(qsl[-1]) + 2
    win = {n: np.ascontiguousarray(a[:rows_total]) for n, a in c["win"].items()}
    assert all(a.shape[0] == rows_total for a in win.values())
    pending = np.random.default_rng(T).integers(0, RQ + 1, B).astype(np.int32)
    kw = {}
    if gated:
        gate, weight, eps = W.draw_output_stage(W._gen(1200 + T), B, T, H)
        kw = dict(gate=np.ascontiguousarray(W.bits(gate)[:rows_total]),
                  norm_weight=weight.numpy(), norm_eps=eps)
    run_verify_case(fused=fused, H=H, B=B, T=T, RQ=RQ, state=c["state"], slots=c["slots"],
                    corr=c["corr"], kg=c["kg"], a_log=c["a_log"], dt_bias=c["dt_bias"],
                    win=win, rows=c["rows"], pending=pending if fused else None, qsl=qsl,
                    out_rows=rows_total, label=f"varlen T={T} fused={fused}", **kw)


# ---------------------------------------------------------------- align inside the fused replay

@pytest.mark.parametrize("T,bf16", [(2, False), (4, False), (8, False), (3, True), (8, True)])
def test_fused_boundary_stores(T, bf16):
    """Boundary slots with m = 1, n - 1, n, above n, 0, and a null boundary;
    pending counts across both MFMA stages (m and n on each side of 4)."""
    H, B, RQ, S = 3, 8, 8, 20
    c = _vf_case(1300 + T, H, B, T, RQ, S, null_rows=(7,), norec_rows=(6,), bf16=bf16)
    slots, rows = c["slots"], c["rows"]
    n_req = [8, 6, 5, 3, 7, 4, 2, 5]
    m_req = [5, 5, 5, 9, 0, 1, 2, 3]
    pending = np.zeros(B, np.int32)
    for b in range(B):
        if rows[b] >= 0:
            pending[rows[b]] = n_req[b]
    free = [sl for sl in range(1, S) if sl not in set(slots.tolist())]
    bounds = np.array(free[:B], np.int32)
    bounds[2] = 0  # a null boundary
    blens = np.array(m_req, np.int32)
    run_verify_case(fused=True, H=H, B=B, T=T, RQ=RQ, state=c["state"], slots=slots,
                    corr=c["corr"], kg=c["kg"], a_log=c["a_log"], dt_bias=c["dt_bias"],
                    win=c["win"], rows=rows, pending=pending, bounds=bounds, blens=blens,
                    label=f"fused align T={T} bf16={bf16}")
