"""The benchmark's host-side accounting, checked on CPU: algorithmic bytes
against hand counts of tiny plans, its plan simulation against the oracle's
defer and flush-plan steps, the percentile helper, and the one-GPU rule."""
import importlib.util
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_fused_bytes_hand_count():
    b = _bench()
    K = V = 128
    H, T, RQ = 2, 3, 4
    # request 0: null slot; 1: rec row -1 (no replay, no records);
    # 2: pending 9 clamped to RQ = 4; 3: pending 0 (page read only).
    slots = [0, 5, 6, 7]
    rows = [0, -1, 1, 2]
    pending = np.array([1, 9, 0], np.int32)  # by record row
    st, tot = b.fused_bytes(slots, rows, pending, T, RQ, H)
    page = V * K * 4
    rec_tok = V * 4 + 2 * K * 2          # one token's correction + key/gate record
    inputs = T * (3 * K * 2 + V * 2) + T * 2
    out = T * V * 2
    want_state = H * (page + (page + page) + page)
    want_tot = (H * out                                   # null slot: zero outputs
                + H * (page + inputs + out)                # no record row
                + H * (2 * page + 4 * rec_tok + T * rec_tok + inputs + out)
                + H * (page + T * rec_tok + inputs + out))
    assert (st, tot) == (want_state, want_tot)
    # BF16 pages halve the page terms; the gated stage adds T*256 B per live item.
    st16, _ = b.fused_bytes(slots, rows, pending, T, RQ, H, es=2)
    assert st16 == want_state // 2
    _, tot_g = b.fused_bytes(slots, rows, pending, T, RQ, H, gated=True)
    assert tot_g - tot == 3 * H * T * V * 2
    # The convolution adds, per live item, the 3 taps read and T + 2 entries
    # written for 3*128 channels, and the weights and bias once.
    _, tot_c = b.fused_bytes(slots, rows, pending, T, RQ, H, conv=True)
    assert tot_c - tot == 3 * H * (3 * K * 3 * 2 + 3 * K * (T + 2) * 2) + 3 * 4 * H * K * 2 + 3 * H * K * 2


def test_commit_bytes_hand_count():
    b = _bench()
    K = V = 128
    H, Q = 3, 4
    slots = [0, 4, 5, 6, 7]
    lens = [2, 0, 9, 1, 3]
    rows = [0, 1, 2, -1, 3]
    st, tot = b.commit_bytes(slots, lens, rows, H, Q)
    page = V * K * 4
    rec_tok = V * 4 + 2 * K * 2
    # live: request 2 (n = 4 after the clamp) and request 4 (n = 3)
    assert st == H * 2 * page * 2
    assert tot == H * (2 * page + 4 * rec_tok) + H * (2 * page + 3 * rec_tok)


def test_plan_simulation_matches_the_oracle():
    import oracle
    b = _bench()
    rng = np.random.default_rng(3)
    B, q, null = 40, 8, 0
    slots = rng.integers(0, 30, B).astype(np.int32)
    rows = rng.permutation(B).astype(np.int32)
    rows[rng.random(B) < 0.2] = -1
    pending0 = rng.integers(-2, q + 3, B).astype(np.int32)
    accepted = rng.integers(0, q + 1, B).astype(np.int32)
    sim = b.simulate_plan(slots, rows, pending0, accepted, 3, q, null)
    pending = pending0.copy()
    for fused_pending, lens in sim:
        assert np.array_equal(np.asarray(fused_pending), pending)
        commit_lens = accepted.copy()
        oracle.defer(slots, commit_lens, rows, pending, null_slot=null)
        flush = oracle.flush_plan(slots, rows, pending, q, null_slot=null)
        assert list(flush[0]) == list(lens)


def test_spread():
    b = _bench()
    assert b.spread([3.0]) == {"median_ms": 3.0, "p90_ms": 3.0}
    assert b.spread(list(range(10, 0, -1))) == {"median_ms": 5, "p90_ms": 9}
    assert b.spread(list(range(20))) == {"median_ms": 9, "p90_ms": 17}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_trace_summary_averages_the_timed_launches(tmp_path):
    """bench.py --trace-summary: per kernel, the mean over its last N launches
    (in start-time order, whatever the CSV's row order), and counter values
    summed per dispatch before they are averaged."""
    import csv
    b = _bench()
    trace = tmp_path / "kda_kernel_trace.csv"
    rows = []
    # kernel A: 4 warm-up launches of 10 us, then 3 timed ones of 2, 4, 6 us;
    # rows written out of order
    t = 0
    for d in [10, 10, 10, 10, 2, 4, 6]:
        rows.append({"Kernel_Name": "A", "Dispatch_Id": str(len(rows)), "Start_Timestamp": str(t),
                     "End_Timestamp": str(t + d * 1000)})
        t += 100000
    rows.append({"Kernel_Name": "B", "Dispatch_Id": "99", "Start_Timestamp": "5",
                 "End_Timestamp": "1005"})
    with open(trace, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        for r in reversed(rows):
            w.writerow(r)
    s = b.trace_summary(str(trace), 3)
    assert s["A"]["launches"] == 7 and s["A"]["timed_launches"] == 3
    assert s["A"]["timed_mean_us"] == 4.0 and s["A"]["timed_min_us"] == 2.0
    assert s["A"]["all_mean_us"] == round((40 + 12) / 7, 2)
    assert s["B"]["timed_mean_us"] == 1.0
    # counters: two counter rows per dispatch (e.g. per XCD) are summed first
    ctr = tmp_path / "kda_counter_collection.csv"
    with open(ctr, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Dispatch_Id", "Start_Timestamp",
                                          "End_Timestamp", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for did, (t0, v) in enumerate([(0, 100.0), (10, 200.0), (20, 300.0)]):
            for part in (0.25, 0.75):
                w.writerow({"Kernel_Name": "A", "Dispatch_Id": str(did),
                            "Start_Timestamp": str(t0), "End_Timestamp": str(t0 + 1000),
                            "Counter_Name": "FETCH_SIZE", "Counter_Value": str(v * part)})
    c = b.trace_summary(str(ctr), 2)
    assert c["A"]["counters_timed_mean"]["FETCH_SIZE"] == 250.0


def test_source_digest_follows_code_not_comments(tmp_path, monkeypatch):
    b = _bench()
    src = ('#include "a.h"  // header\n'
           '/* block\n   comment */ int f(int x) {\n'
           '  const char* s = "http://not/a/comment";  // trailing\n'
           "  return x + '/';\n}\n")
    stripped = b.strip_comments(src)
    assert "header" not in stripped and "block" not in stripped and "trailing" not in stripped
    assert '"http://not/a/comment"' in stripped and "'/'" in stripped
    assert '#include "a.h"' in stripped.splitlines()

    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    path = tmp_path / "k.hip"

    def digest(text):
        path.write_text(text)
        return b.source_digest(["k.hip"])

    base = digest(src)
    # a comment edit, a new comment line, blank lines and indentation: same code
    assert digest(src.replace("// trailing", "// reworded note")) == base
    assert digest("// new first line\n\n" + src.replace("  return", "      return")) == base
    # any code edit changes it, also one inside a string literal
    assert digest(src.replace("x + '/'", "x - '/'")) != base
    assert digest(src.replace("not/a", "not/b")) != base


def test_sampled_cpu_baseline_runners_match_the_oracle():
    """The single-kernel workloads' CPU-baseline runners pass the workload to the
    oracle unchanged: on all items each equals a direct oracle call, and their
    state-byte counts equal the bench's accounting."""
    import torch
    import oracle
    import workloads as W
    b = _bench()
    H, B, T, RQ, S = 2, 5, 4, 4, 8
    c = W.small_fused_case(3, H, B, T, RQ, S, null_rows=(1,), no_record_rows=(2,))
    run, state_bytes = b._verify_cpu_runner(
        True, H, B, T, RQ, c["state"], c["state_indices"], c["record_rows"], c["pending"],
        c["corr"], c["kg"], c["a_log"][0], c["dt_bias"][0], W.LOWER_BOUND, c["window"])
    run(np.arange(B * H, dtype=np.int64), 1)
    state = c["state"].numpy().copy()
    corr, kg = c["corr"].numpy().copy(), W.bits(c["kg"])
    win = {n: W.bits(getattr(c["window"], n)) for n in ("q", "k", "v", "raw_g", "raw_beta")}
    out = np.zeros((B * T, H * 128), np.uint16)
    slots = c["state_indices"].numpy().astype(np.int32)
    rows = c["record_rows"].numpy().astype(np.int32)
    pend = c["pending"].numpy().astype(np.int32)
    oracle.fused_replay_verify(heads=H, tokens=T, batch=B, a_log=c["a_log"][0].numpy(),
                               dt_bias=c["dt_bias"][0].numpy(), lower_bound=W.LOWER_BOUND,
                               state=state, state_slot_stride=H * 128 * 128,
                               state_indices=slots, corr=corr, kg=kg, record_tokens=RQ,
                               record_rows=rows, pending=pend, out=out, threads=1, **win)
    rec = run.__closure__  # the runner's host copies, reached through its free variables
    h = next(cell.cell_contents for cell in rec if isinstance(cell.cell_contents, dict))
    assert np.array_equal(h["state"], state) and np.array_equal(h["corr"], corr)
    assert np.array_equal(h["kg"], kg)
    assert state_bytes(range(B * H)) == b.fused_bytes(slots, rows, pend, T, RQ, H)[0]
    res = b.sampled_cpu_baseline(run, B * H, state_bytes, seconds=0.01)
    assert res["kind"] == "oracle" and res["cores"] >= 1 and res["value"] > 0
    assert res["single_thread"]["items_per_s"] > 0

    # commit: two BF16 layers, src -> dst (disjoint), one boundary store
    L, Q, S = 2, 4, 10
    page = H * 128 * 128  # elements per slot
    g = W._gen(5)
    states = [W.bf16(W.normal(g, (S * page,), 0.1)) for _ in range(L)]
    recs = [W.draw_records(g, B, H, Q) for _ in range(L)]
    a_log, dt_bias = W.draw_gate_params(g, L, H)
    src = np.array([1, 2, 0, 3, 4], np.int32)
    dst = np.array([5, 6, 0, 7, 0], np.int32)
    lens = np.array([2, 0, 3, 4, 1], np.int32)
    bnd = np.array([8, 0, 0, 0, 0], np.int32)
    blen = np.array([1, 0, 0, 0, 0], np.int32)
    run, state_bytes = b._commit_cpu_runner(H, B, Q, states, [page] * L,
                                            [r[0] for r in recs], [r[1] for r in recs], a_log,
                                            dt_bias, src, lens, dst, bnd, blen, W.LOWER_BOUND)
    run(np.arange(L * B * H, dtype=np.int64), 1)
    want = [W.bits(t) for t in states]
    oracle.commit(heads=H, window=Q, batch=B, state_bf16=True, state_layers=want,
                  state_slot_strides=[page] * L,
                  corr_layers=[r[0].numpy() for r in recs], corr_row_strides=[H * Q * 128] * L,
                  kg_layers=[W.bits(r[1]) for r in recs], kg_row_strides=[H * Q * 256] * L,
                  a_log=a_log.numpy(), dt_bias=dt_bias.numpy(), sources=src, commit_lens=lens,
                  destinations=dst, boundaries=bnd, boundary_lens=blen,
                  lower_bound=W.LOWER_BOUND, threads=1)
    h_st = next(cell.cell_contents for cell in run.__closure__
                if isinstance(cell.cell_contents, list)
                and isinstance(cell.cell_contents[0], np.ndarray)
                and cell.cell_contents[0].size == S * page)
    for l in range(L):
        assert np.array_equal(h_st[l], want[l]), l
        assert not np.array_equal(h_st[l], W.bits(states[l])), l  # the pools moved
    # live: requests 0 (with its boundary page) and 3; request 4 has a null destination
    page_bytes = 128 * 128 * 2
    assert state_bytes(range(L * B * H)) == L * H * (3 + 2) * page_bytes
