"""The entry points under HIP graph capture: one whole decode step (the
accepted-count copy, the fused replay+verify, defer, flush plan and the
in-place commit) captured once and replayed three times, with the program's
own eager work and synchronisations between the replays, matches the same
steps run eagerly, bit for bit, after every replay. The calls read no device
memory on the host, so they can be captured; none of them records a memset."""
import numpy as np
import pytest
import torch

import workloads as W
from _kda_cases import DEV, announce

pytestmark = pytest.mark.gpu
K = V = 128


def _case(bf16, seed=31, large=False):
    # large: 64 heads x 80 requests of FP32 pages (320 MiB, above the MALL's
    # 256 MB), so the fused step and the commit run their streaming instances.
    H, B, T, RQ, S = (64, 80, 8, 8, 90) if large else (4, 24, 8, 8, 40)
    g = W._gen(seed)
    page = H * V * K
    state = W.draw_state(seed + 1, S * page, torch.float32)
    if bf16:
        state = state.to(torch.bfloat16)
    perm = W.permutation(g, S - 1) + 1
    slots = perm[:B].to(torch.int32)
    slots[[3, 11]] = 0
    rows = W.permutation(g, B).to(torch.int32)
    rows[[5, 17]] = -1
    corr, kg = W.draw_records(g, B, H, RQ)
    a_log, dt_bias = W.draw_gate_params(g, 1, H)
    win = W.draw_window(g, B, T, H)
    pending = W.uniform_int(g, 0, RQ, B).to(torch.int32)
    accepted = W.uniform_int(g, 0, T, B).to(torch.int32)
    fixed = dict(H=H, B=B, T=T, RQ=RQ, page=page, bf16=bf16,
                 slots=slots.to(DEV), rows=rows.to(DEV), accepted=accepted.to(DEV),
                 a_log=a_log[0].contiguous().to(DEV), dt_bias=dt_bias[0].contiguous().to(DEV),
                 win=win.to(DEV))
    mutable = dict(state=state.to(DEV), corr=corr.to(DEV), kg=kg.to(DEV),
                   pending=pending.to(DEV),
                   out=torch.zeros((B * T, H * V), dtype=torch.bfloat16, device=DEV),
                   commit_lens=torch.zeros(B, dtype=torch.int32, device=DEV),
                   flush=torch.zeros((4, B), dtype=torch.int32, device=DEV))
    return fixed, mutable


def _step(f, m):
    import spec_decode_amd as kda
    H, B, T, RQ, w = f["H"], f["B"], f["T"], f["RQ"], f["win"]
    m["commit_lens"].copy_(f["accepted"])
    kda.kda_fused_replay_verify(heads=H, tokens=T, batch=B, q=w.q, k=w.k, v=w.v,
                                raw_g=w.raw_g, raw_beta=w.raw_beta, a_log=f["a_log"],
                                dt_bias=f["dt_bias"], lower_bound=W.LOWER_BOUND,
                                state=m["state"], state_slot_stride=f["page"],
                                state_indices=f["slots"], corr=m["corr"], kg=m["kg"],
                                record_tokens=RQ, record_rows=f["rows"],
                                pending=m["pending"], out=m["out"])
    kda.kda_defer_commit(batch=B, state_indices=f["slots"], commit_lens=m["commit_lens"],
                         record_rows=f["rows"], pending=m["pending"])
    fl = m["flush"]
    kda.kda_flush_plan(batch=B, spec_query_len=T, state_indices=f["slots"],
                       record_rows=f["rows"], pending=m["pending"], commit_lens=fl[0],
                       final_indices=fl[1], boundaries=fl[2], boundary_lens=fl[3])
    kda.kda_commit(heads=H, window=RQ, batch=B,
                   state_dtype=kda.KDA_STATE_BF16 if f["bf16"] else kda.KDA_STATE_F32,
                   state_addrs=[m["state"].data_ptr()], state_slot_strides=[f["page"]],
                   corr_addrs=[m["corr"].data_ptr()], corr_row_strides=[H * RQ * V],
                   kg_addrs=[m["kg"].data_ptr()], kg_row_strides=[H * RQ * 2 * K],
                   a_log=f["a_log"], dt_bias=f["dt_bias"], sources=fl[1],
                   commit_lens=fl[0], destinations=fl[1], record_rows=f["rows"],
                   lower_bound=W.LOWER_BOUND)


def _snapshot(m):
    return {k: (v.view(torch.int16) if v.dtype == torch.bfloat16 else v).cpu().numpy().copy()
            for k, v in m.items()}


@pytest.mark.parametrize("bf16,large", [(False, False), (True, False), (False, True)])
def test_captured_step_replays_match_eager_steps(bf16, large):
    announce(f"graph capture: step of {'H=64 B=80' if large else 'H=4 B=24'} q=8, "
             f"{'BF16' if bf16 else 'FP32'} pool")
    fixed, eager = _case(bf16, large=large)
    _, graphed = _case(bf16, large=large)
    ref = []
    for _ in range(3):
        _step(fixed, eager)
        torch.cuda.synchronize()
        ref.append(_snapshot(eager))
    # The steps move the state, the records and the outputs: equal replays mean something.
    for name in ("state", "corr", "out"):
        assert not np.array_equal(ref[0][name], ref[1][name]), name
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _step(fixed, graphed)
    torch.cuda.synchronize()
    # Capture executes nothing: the graphed buffers still hold their inputs.
    assert np.array_equal(_snapshot(graphed)["pending"],
                          _case(bf16, large=large)[1]["pending"].cpu().numpy())
    scratch = torch.ones(1 << 20, device=DEV)
    for r in range(3):
        graph.replay()
        torch.cuda.synchronize()
        scratch.mul_(1.5).add_(float(r))  # eager work of the program between replays
        torch.cuda.synchronize()
        got = _snapshot(graphed)
        for name, want in ref[r].items():
            assert np.array_equal(got[name], want), f"replay {r + 1}: {name} differs"
