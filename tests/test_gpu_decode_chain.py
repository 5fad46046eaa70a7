"""Several decode steps in a row through deferred RecoverSSM, on the GPU and in
the oracle side by side (kernels page: the deferred RecoverSSM plan steps;
fused page: KdaFused, replay of the pending commit before the verify).

Each step runs the fused replay+verify (it replays what the previous step
accepted from the records that step wrote, then verifies a new window and
rewrites the records), the defer step over that step's accepted counts with a
mix of eager and deferred requests, and the commit of the eager requests. A
flush (plan, then commit) ends the run. The GPU chain and the oracle chain run
independently from the same seeded inputs: nothing the GPU produces is fed to
the oracle. The pool is FP32, where the two chains stay within FP32 rounding
of each other from step to step; a BF16 pool's legitimate one-ulp differences
are scaled by the decays and can cancel in the next fold, so no per-step ulp
bound holds over a chain of BF16 pages. With the convolution prologue the
chain also carries each slot's window pool from step to step: a step reads its
taps at the offset that the previous step's accepted count sets and writes the
window back, so the next step's inputs depend on it.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _compare import assert_bf16_close, assert_exact, assert_f32_close
from _kda_cases import (DEV, announce, conv_pool_build, conv_pool_layout, dev, dev_bf16,
                        np_of, window_np)

pytestmark = pytest.mark.gpu

K = V = 128


def _commit_args(kda, H, RQ, B, d, sources, lens, rows):
    return dict(heads=H, window=RQ, batch=B, state_dtype=kda.KDA_STATE_F32,
                state_addrs=[d["state"].data_ptr()], state_slot_strides=[H * V * K],
                corr_addrs=[d["corr"].data_ptr()], corr_row_strides=[H * RQ * V],
                kg_addrs=[d["kg"].data_ptr()], kg_row_strides=[H * RQ * 2 * K],
                a_log=d["a_log"][None], dt_bias=d["dt_bias"][None], sources=sources,
                commit_lens=lens, destinations=sources, record_rows=rows,
                lower_bound=W.LOWER_BOUND)


def _run_chain(seed, conv_layout=None):
    import spec_decode_amd as kda

    H, B, T, RQ, S, STEPS = 4, 24, 8, 8, 32, 4
    page = H * V * K
    c = W.small_fused_case(seed, H, B, T, RQ, S, null_rows=(3, 17), no_record_rows=(5, 20))
    slots = c["state_indices"].numpy().astype(np.int32)
    rows = c["record_rows"].numpy().astype(np.int32)
    a_log = c["a_log"][0].numpy()
    dtb = c["dt_bias"][0].numpy()
    g = W._gen(seed + 1000)
    windows = [window_np(c["window"])] + [window_np(W.draw_window(W._gen(seed + 100 + i), B, T, H))
                                          for i in range(1, STEPS)]
    accepted = [W.uniform_int(g, 0, T, B).numpy().astype(np.int32) for _ in range(STEPS)]
    eager = [(W.uniform_int(g, 0, 2, B).numpy() == 0).astype(np.int32) for _ in range(STEPS)]

    # The oracle chain's buffers and the GPU chain's, from the same host inputs.
    ref = dict(state=c["state"].numpy().astype(np.float32).copy(),
               corr=c["corr"].numpy().copy(), kg=W.bits(c["kg"]).copy(),
               pending=c["pending"].numpy().astype(np.int32).copy())
    d = dict(state=dev(ref["state"]), corr=dev(ref["corr"]), kg=dev_bf16(ref["kg"]),
             pending=dev(ref["pending"]), a_log=dev(a_log), dt_bias=dev(dtb))
    d_slots, d_rows = dev(slots), dev(rows)
    out = torch.empty((B * T, H * V), dtype=torch.bfloat16, device=DEV)
    first = ref["state"].copy()
    if conv_layout is not None:
        cv = W.draw_conv_inputs(W._gen(seed + 7), B, T, H, RQ, S)
        strides = conv_pool_layout(S, H, RQ + 2, layout=conv_layout)
        ref["pool"] = conv_pool_build(W.bits(cv.window), strides, seed + 11)
        d["pool"] = dev_bf16(ref["pool"])
        conv_w, conv_b, pitch = W.bits(cv.weight), W.bits(cv.bias), cv.pitch
        xs = [W.bits(cv.x)] + [W.bits(W.draw_conv_inputs(W._gen(seed + 200 + i), B, T, H, RQ,
                                                         S).x) for i in range(1, STEPS)]
        d_conv_w, d_conv_b = dev_bf16(conv_w), dev_bf16(conv_b)
        pool0 = ref["pool"].copy()

    def compare(label):
        assert_f32_close(f"{label} state pool", np_of(d["state"]), ref["state"])
        assert_f32_close(f"{label} corrections", np_of(d["corr"]), ref["corr"])
        assert_exact(f"{label} key/gate records", np_of(d["kg"]), ref["kg"])
        assert_exact(f"{label} pending", np_of(d["pending"]), ref["pending"])
        if conv_layout is not None:
            assert_exact(f"{label} window pool", np_of(d["pool"]), ref["pool"])

    replayed = eager_commits = 0
    for i in range(STEPS):
        win = windows[i]
        live = [b for b in range(B) if slots[b] > 0 and rows[b] >= 0]
        replayed += sum(int(min(ref["pending"][rows[b]], RQ) > 0) for b in live)
        announce(f"decode chain seed={seed} step {i}: fused H={H} B={B} T={T} RQ={RQ} "
                 f"FP32 pool, convolution prologue {conv_layout}")
        common = dict(heads=H, tokens=T, batch=B, lower_bound=W.LOWER_BOUND,
                      state_slot_stride=page, record_tokens=RQ)
        g_io = dict(raw_g=dev_bf16(win["raw_g"]), raw_beta=dev_bf16(win["raw_beta"]),
                    a_log=d["a_log"], dt_bias=d["dt_bias"], state=d["state"],
                    state_indices=d_slots, corr=d["corr"], kg=d["kg"], record_rows=d_rows,
                    pending=d["pending"], out=out)
        r_out = np.zeros((B * T, H * V), np.uint16)
        r_io = dict(raw_g=win["raw_g"], raw_beta=win["raw_beta"], a_log=a_log, dt_bias=dtb,
                    state=ref["state"], state_indices=slots, corr=ref["corr"], kg=ref["kg"],
                    record_rows=rows, pending=ref["pending"], out=r_out)
        if conv_layout is None:
            kda.kda_fused_replay_verify(q=dev_bf16(win["q"]), k=dev_bf16(win["k"]),
                                        v=dev_bf16(win["v"]), **common, **g_io)
            oracle.fused_replay_verify(q=win["q"], k=win["k"], v=win["v"], **common, **r_io)
        else:
            conv = dict(x_row_stride=pitch, conv_slot_stride=strides[0],
                        conv_channel_stride=strides[1], conv_tap_stride=strides[2],
                        q_scale=K ** -0.5)
            kda.kda_fused_conv_replay_verify(x=dev_bf16(xs[i]), conv_weight=d_conv_w,
                                             conv_bias=d_conv_b, conv_state=d["pool"],
                                             **conv, **common, **g_io)
            oracle.fused_conv_replay_verify(x=xs[i], conv_weight=conv_w, conv_bias=conv_b,
                                            conv_state=ref["pool"], **conv, **common, **r_io)
        torch.cuda.synchronize()
        assert_bf16_close(f"step {i} out", np_of(out), r_out)
        compare(f"step {i} fused")

        announce(f"decode chain seed={seed} step {i}: defer + eager commit")
        d_lens = dev(accepted[i])
        kda.kda_defer_commit(batch=B, state_indices=d_slots, commit_lens=d_lens,
                             record_rows=d_rows, pending=d["pending"], eager=dev(eager[i]))
        r_lens = accepted[i].copy()
        oracle.defer(slots, r_lens, rows, ref["pending"], eager=eager[i])
        torch.cuda.synchronize()
        assert_exact(f"step {i} defer commit_lens", np_of(d_lens), r_lens)
        eager_commits += sum(int(r_lens[b] > 0) for b in live)
        kda.kda_commit(**_commit_args(kda, H, RQ, B, d, d_slots, d_lens, d_rows))
        oracle.commit(heads=H, window=RQ, batch=B, state_bf16=False, state_layers=[ref["state"]],
                      state_slot_strides=[page], corr_layers=[ref["corr"]],
                      corr_row_strides=[H * RQ * V], kg_layers=[ref["kg"]],
                      kg_row_strides=[H * RQ * 2 * K], a_log=a_log[None], dt_bias=dtb[None],
                      sources=slots, commit_lens=r_lens, destinations=slots, record_rows=rows,
                      lower_bound=W.LOWER_BOUND)
        torch.cuda.synchronize()
        compare(f"step {i} eager commit")

    announce(f"decode chain seed={seed}: flush plan + commit")
    fl = [torch.empty(B, dtype=torch.int32, device=DEV) for _ in range(4)]
    kda.kda_flush_plan(batch=B, spec_query_len=T, state_indices=d_slots, record_rows=d_rows,
                       pending=d["pending"], commit_lens=fl[0], final_indices=fl[1],
                       boundaries=fl[2], boundary_lens=fl[3])
    r_flush = oracle.flush_plan(slots, rows, ref["pending"], T)
    torch.cuda.synchronize()
    for name, got, want in zip(("commit_lens", "final", "boundaries", "boundary_lens"), fl,
                               r_flush):
        assert_exact(f"flush {name}", np_of(got), want)
    kda.kda_commit(**_commit_args(kda, H, RQ, B, d, fl[1], fl[0], d_rows))
    oracle.commit(heads=H, window=RQ, batch=B, state_bf16=False, state_layers=[ref["state"]],
                  state_slot_strides=[page], corr_layers=[ref["corr"]],
                  corr_row_strides=[H * RQ * V], kg_layers=[ref["kg"]],
                  kg_row_strides=[H * RQ * 2 * K], a_log=a_log[None], dt_bias=dtb[None],
                  sources=r_flush[1], commit_lens=r_flush[0], destinations=r_flush[1],
                  record_rows=rows, lower_bound=W.LOWER_BOUND)
    torch.cuda.synchronize()
    compare("flush commit")

    # The chain did what it is meant to exercise: replays in later steps, eager
    # commits and a non-empty flush. A page moved iff its request had tokens to
    # fold (pending at the start, or accepted in some step); the null slot's
    # page and the pages of requests without a record row never change.
    assert replayed > B and eager_commits > 0 and int(r_flush[0].sum()) > 0
    final, start = np_of(d["state"]).reshape(S, page), first.reshape(S, page)
    pend0, moved = c["pending"].numpy(), set()
    for b in range(B):
        if slots[b] > 0 and rows[b] >= 0 and (
                pend0[rows[b]] > 0 or any(acc[b] > 0 for acc in accepted)):
            moved.add(int(slots[b]))
    assert len(moved) > B // 2
    for s in range(S):
        if s in moved:
            assert not np.array_equal(final[s], start[s]), f"slot {s} did not move"
        else:
            assert_exact(f"slot {s} (nothing to fold)", final[s], start[s])
    if conv_layout is not None:
        # every step rewrote the windows of the live slots, and only theirs
        rewritten = np_of(d["pool"]) != pool0
        assert rewritten.any()
        ss, cs, ts = strides
        idx = np.arange(pool0.size)
        slot_of = idx // ss
        assert set(np.unique(slot_of[rewritten])) <= set(int(x) for x in slots if x > 0)


@pytest.mark.parametrize("seed", [11, 12])
def test_decode_steps_chain_against_oracle(seed):
    _run_chain(seed)


@pytest.mark.parametrize("layout", ["dim_first", "window_major"])
def test_decode_steps_chain_convolution_prologue(layout):
    _run_chain(21 if layout == "dim_first" else 22, conv_layout=layout)
