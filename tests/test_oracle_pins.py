"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these tests re-types the oracle's recurrence: each checks it against
an independent statement (the scalar worked example of "Mamba Streaming State
That Survives Chunking", brute-force unrolled products, the SSD quadratic
form, closed forms, and the page's chunking/reset/reorder invariants).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from streaming_state_amd import inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden", "scalar_artifact.json")


# ---------------------------------------------------------------------------
# the scalar worked example ("Runnable artifact")
# ---------------------------------------------------------------------------
def _scalar_inputs(tokens):
    """Map the scalar program onto the Mamba-2 form: H=P=N=G=1, B=C=1, dt=1,
    x = the token, D = 0, decay injected exactly as 3/4."""
    L = len(tokens)
    x = np.array(tokens, dtype=np.float64).reshape(L, 1, 1)
    one = np.ones((L, 1, 1))
    return dict(x=x, dt=np.ones((L, 1)), B=one, C=one, A=np.zeros(1), D=np.zeros(1),
                decay=np.full((L, 1), 0.75))


def _scan_chunks(chunks, reset_before=()):
    """Scan chunk by chunk, resetting the stream before the listed chunk indices."""
    st, pos, out = None, 0, []
    for i, ch in enumerate(chunks):
        if i in reset_before:
            st, pos = None, 0
        inp = _scalar_inputs(ch)
        r = oracle.scan(inp["x"], inp["dt"], inp["B"], inp["C"], inp["A"], inp["D"], state=st,
                        pos=pos, decay=inp["decay"])
        out.extend(r["y"].reshape(-1).tolist())
        st, pos = r["state"], r["pos"]
    value = 0.0 if st is None else float(st.reshape(-1)[0])
    return out, value, pos


def _exact_outputs(tokens, decay=Fraction(3, 4)):
    """Exact outputs by the unrolled sum v_t = sum_{s<=t} decay^(t-s) * token_s."""
    return [sum(decay ** (t - s) * tokens[s] for s in range(t + 1)) for t in range(len(tokens))]


@pytest.fixture(scope="module")
def gold():
    with open(GOLD) as f:
        return json.load(f)


def test_artifact_full_scan_exact(gold):
    toks = gold["tokens"]
    out, value, pos = _scan_chunks([toks])
    exact = _exact_outputs(toks, Fraction(gold["decay"]))
    assert [Fraction(v) for v in out] == exact  # dyadic rationals: exact in fp64
    assert exact[1] == Fraction(11, 4) and exact[8] == Fraction(210601, 65536)
    assert Fraction(value) == exact[-1]
    assert pos == gold["final_position"] == len(toks)


def test_artifact_chunked_equals_full(gold):
    toks = gold["tokens"]
    a, b = gold["chunked_split"]
    full = _scan_chunks([toks])
    chunked = _scan_chunks([toks[:a], toks[a:b], toks[b:]])
    assert chunked[0] == full[0]            # outputs
    assert chunked[1:] == full[1:]          # state value and position


def test_artifact_empty_chunk_neutral(gold):
    toks = gold["tokens"]
    assert _scan_chunks([[], toks])[0] == _scan_chunks([toks])[0]


def test_artifact_reset_differs_and_restarts(gold):
    toks = gold["tokens"]
    k = gold["reset_split"]
    out, _, pos = _scan_chunks([toks[:k], toks[k:]], reset_before={gold["reset_before_chunk"]})
    full = _scan_chunks([toks])[0]
    assert out != full
    assert [Fraction(v) for v in out[k:]] == _exact_outputs(toks[k:])
    assert out[k:k + 3] == [3.0, 2.25, 5.6875]
    assert pos == len(toks) - k


def test_artifact_reorder_differs(gold):
    toks = gold["tokens"]
    assert _scan_chunks([toks[3:], toks[:3]])[0] != _scan_chunks([toks])[0]


def test_artifact_invalid_chunk_rejected():
    inp = _scalar_inputs([1.0, float("nan")])
    st = np.full((1, 1, 1), 5.0)
    with pytest.raises(oracle.OracleError) as e:
        oracle.scan(inp["x"], inp["dt"], inp["B"], inp["C"], inp["A"], inp["D"], state=st,
                    decay=inp["decay"])
    assert e.value.code == oracle.ORC_E_INVALID_CHUNK


def test_artifact_two_chunkings_identical(gold):
    c1, c2 = gold["equal_chunkings"]
    assert _scan_chunks(c1) == _scan_chunks(c2)


# ---------------------------------------------------------------------------
# brute force: unrolled products on tiny inputs
# ---------------------------------------------------------------------------
def _tiny(seed, L=11, H=2, P=2, N=3, G=1):
    r = np.random.default_rng(seed)
    x = r.standard_normal((L, H, P))
    dt = np.log1p(np.exp(r.normal(-1.0, 0.5, (L, H))))
    B = r.standard_normal((L, G, N))
    C = r.standard_normal((L, G, N))
    A = -np.exp(r.uniform(0, np.log(16), H))
    D = r.standard_normal(H)
    h0 = r.standard_normal((H, P, N))
    return x, dt, B, C, A, D, h0


@pytest.mark.parametrize("G", [1, 2])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_bruteforce_unrolled(seed, G):
    """h_t = (prod_{i<=t} a_i) h0 + sum_{s<=t} (prod_{s<i<=t} a_i) dt_s x_s B_s^T,
    y_t = h_t C_t + D x_t, evaluated with explicit products."""
    x, dt, B, C, A, D, h0 = _tiny(seed, H=2 * G, G=G)
    L, H, P = x.shape
    N = B.shape[2]
    r = oracle.scan(x, dt, B, C, A, D, state=h0)
    for h in range(H):
        g = h // (H // G)
        a = [math.exp(dt[t, h] * A[h]) for t in range(L)]
        for t in range(L):
            h_t = np.prod(a[:t + 1]) * h0[h]
            for s in range(t + 1):
                w = np.prod(a[s + 1:t + 1]) if s < t else 1.0
                h_t = h_t + w * dt[s, h] * np.outer(x[s, h], B[s, g])
            y = h_t @ C[t, g] + D[h] * x[t, h]
            np.testing.assert_allclose(r["y"][t, h], y, rtol=1e-12, atol=1e-12)
            if t == L - 1:
                np.testing.assert_allclose(r["state"][h], h_t, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", [3, 4])
def test_ssd_quadratic_form(seed):
    """Matrix (SSD) view: y = (Lmask o C B^T)(dt o x) + decay-to-start * C h0 + D x."""
    x, dt, B, C, A, D, h0 = _tiny(seed, L=12)
    L, H, P = x.shape
    r = oracle.scan(x, dt, B, C, A, D, state=h0)
    for h in range(H):
        logs = dt[:, h] * A[h]
        Lm = np.zeros((L, L))
        for t in range(L):
            for s in range(t + 1):
                Lm[t, s] = math.exp(sum(logs[s + 1:t + 1]))
        CB = C[:, 0, :] @ B[:, 0, :].T
        start = np.array([math.exp(sum(logs[:t + 1])) for t in range(L)])
        y = (Lm * CB) @ (dt[:, h:h + 1] * x[:, h, :]) + start[:, None] * (C[:, 0, :] @ h0[h].T)
        y = y + D[h] * x[:, h, :]
        np.testing.assert_allclose(r["y"][:, h, :], y, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# closed forms and special cases
# ---------------------------------------------------------------------------
def test_A_zero_is_prefix_sum_exact():
    """A = 0 gives a = 1: the state is the inclusive prefix sum of dt x B^T
    (small integers, so every value is exact)."""
    r = np.random.default_rng(7)
    L, H, P, N = 20, 3, 2, 4
    x = r.integers(-3, 4, (L, H, P)).astype(np.float64)
    B = r.integers(-2, 3, (L, 1, N)).astype(np.float64)
    C = r.integers(-2, 3, (L, 1, N)).astype(np.float64)
    dt = r.integers(1, 3, (L, H)).astype(np.float64)
    out = oracle.scan(x, dt, B, C, np.zeros(H), np.zeros(H))
    pref = np.cumsum(dt[:, :, None, None] * x[:, :, :, None] * B[:, None, 0, None, :], axis=0)
    y = np.einsum("thpn,tn->thp", pref, C[:, 0, :])
    assert np.array_equal(out["y"], y)
    assert np.array_equal(out["state"], pref[-1])


def test_geometric_closed_form():
    """Constant a and u = dt x B: h_t = a^(t+1) h0 + u (1 - a^(t+1)) / (1 - a)."""
    L, P, N = 40, 2, 2
    A, dtv = -0.7, 0.3
    a = math.exp(dtv * A)
    x = np.full((L, 1, P), 1.5)
    B = np.full((L, 1, N), 0.25)
    C = np.full((L, 1, N), 1.0)
    h0 = np.full((1, P, N), 2.0)
    out = oracle.scan(x, np.full((L, 1), dtv), B, C, np.array([A]), np.array([0.0]), state=h0)
    u = dtv * 1.5 * 0.25
    for t in range(L):
        k = t + 1
        h = a ** k * 2.0 + u * (1 - a ** k) / (1 - a)
        np.testing.assert_allclose(out["y"][t, 0], np.full(P, h * N), rtol=1e-13)


def test_memoryless_at_large_negative_decay():
    """dt*A = -800 underflows exp to 0: h_t = dt_t x_t B_t^T exactly."""
    x, _, B, C, _, D, h0 = _tiny(5, L=6)
    L, H, P = x.shape
    dt = np.full((L, H), 50.0)
    A = np.full(H, -16.0)
    out = oracle.scan(x, dt, B, C, A, D, state=h0)
    for t in range(L):
        for h in range(H):
            h_t = dt[t, h] * np.outer(x[t, h], B[t, 0])
            y = h_t @ C[t, 0] + D[h] * x[t, h]
            np.testing.assert_allclose(out["y"][t, h], y, rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------------------
# chunk equivalence, reset, reorder (the page's invariants, workload 0)
# ---------------------------------------------------------------------------
def _chunked(w, sizes, reset=None):
    st, pos, ys = None, 0, []
    t0 = 0
    for s in sizes:
        sl = slice(t0, t0 + s)
        r = oracle.scan(w["x"][sl], w["dt"][sl], w["B"][sl], w["C"][sl], w["A"], w["D"],
                        state=st, pos=pos, reset=None if reset is None else reset[sl])
        ys.append(r["y"])
        st, pos = r["state"], r["pos"]
        t0 += s
    assert t0 == w["L"]
    return np.concatenate(ys), st, pos


def test_chunk_equivalence_bitwise_all_partitions():
    w = inputs.workload0()
    reset = np.zeros(w["L"], np.uint8)
    reset[w["reset_at"]] = 1
    for rs in (None, reset):
        full = _chunked(w, [w["L"]], rs)
        for sizes in inputs.partitions0(w["L"]):
            ch = _chunked(w, sizes, rs)
            assert np.array_equal(ch[0], full[0]), sizes
            assert np.array_equal(ch[1], full[1]), sizes
            assert ch[2] == full[2]
    assert full[2] == w["L"] - w["reset_at"]


def test_reset_then_B_equals_fresh_B_and_differs_without_reset():
    w = inputs.workload0()
    k = w["reset_at"]
    reset = np.zeros(w["L"], np.uint8)
    reset[k] = 1
    with_reset = oracle.scan(w["x"], w["dt"], w["B"], w["C"], w["A"], w["D"], reset=reset)
    fresh = oracle.scan(w["x"][k:], w["dt"][k:], w["B"][k:], w["C"][k:], w["A"], w["D"])
    assert np.array_equal(with_reset["y"][k:], fresh["y"])
    assert np.array_equal(with_reset["state"], fresh["state"])
    assert with_reset["pos"] == fresh["pos"] == w["L"] - k
    no_reset = oracle.scan(w["x"], w["dt"], w["B"], w["C"], w["A"], w["D"])
    # inequality control near the boundary: the prefix still shows in the output
    assert np.max(np.abs(no_reset["y"][k] - with_reset["y"][k])) > 1e-5


def test_reorder_and_double_apply_differ():
    w = inputs.workload0()
    full = _chunked(w, [w["L"]])
    sl1, sl2 = slice(0, 20), slice(20, 64)

    def run(order):
        st, ys = None, []
        for sl in order:
            r = oracle.scan(w["x"][sl], w["dt"][sl], w["B"][sl], w["C"][sl], w["A"], w["D"],
                            state=st)
            ys.append(r["y"])
            st = r["state"]
        return np.concatenate(ys), st

    swapped = run([sl2, sl1])
    assert not np.array_equal(swapped[1], full[1])
    assert np.max(np.abs(swapped[0][:20] - full[0][:20])) > 1e-5
    # applying the first chunk twice: the repeated chunk sees the first copy's
    # state, so its outputs differ from the single application near its start
    # (both heads of this fixture decay fast, so the third chunk barely changes)
    twice = run([sl1, sl1, sl2])
    assert np.max(np.abs(twice[0][20:24] - full[0][0:4])) > 1e-3


def test_nonfinite_leaves_state_untouched():
    w = inputs.workload0()
    st0 = np.random.default_rng(1).standard_normal((w["H"], w["P"], w["N"]))
    for name in ("x", "dt", "B", "C"):
        bad = {k: np.array(w[k], dtype=np.float64) for k in ("x", "dt", "B", "C")}
        bad[name].reshape(-1)[5] = np.inf if name != "x" else np.nan
        st = st0.copy()
        with pytest.raises(oracle.OracleError) as e:
            oracle.scan(bad["x"], bad["dt"], bad["B"], bad["C"], w["A"], w["D"], state=st)
        assert e.value.code == oracle.ORC_E_INVALID_CHUNK
        assert np.array_equal(st, st0)


def test_checkpoints_match_split_scan_and_threads_do_not_matter():
    w = inputs.workload1(L=96)
    ck = [10, 47, 95]
    r1 = oracle.scan(w["x"], w["dt"], w["B"], w["C"], w["A"], w["D"], ckpt_at=ck, n_threads=1)
    r4 = oracle.scan(w["x"], w["dt"], w["B"], w["C"], w["A"], w["D"], ckpt_at=ck, n_threads=4)
    assert np.array_equal(r1["y"], r4["y"]) and np.array_equal(r1["ckpt"], r4["ckpt"])
    for i, e in enumerate(ck):
        part = oracle.scan(w["x"][:e + 1], w["dt"][:e + 1], w["B"][:e + 1], w["C"][:e + 1],
                           w["A"], w["D"])
        assert np.array_equal(part["state"], r1["ckpt"][i])
    assert np.array_equal(r1["ckpt"][-1], r1["state"])


def test_hydration_bitwise():
    """Checkpoint after k tokens, restore into a fresh record, continue: bit-identical
    to the uninterrupted run (the determinism behind the pion page's hydration check)."""
    w = inputs.workload1(L=80)
    full = oracle.scan(w["x"], w["dt"], w["B"], w["C"], w["A"], w["D"])
    k = 33
    a = oracle.scan(w["x"][:k], w["dt"][:k], w["B"][:k], w["C"][:k], w["A"], w["D"])
    snapshot = a["state"].copy()
    b = oracle.scan(w["x"][k:], w["dt"][k:], w["B"][k:], w["C"][k:], w["A"], w["D"],
                    state=snapshot, pos=a["pos"])
    assert np.array_equal(np.concatenate([a["y"], b["y"]]), full["y"])
    assert np.array_equal(b["state"], full["state"]) and b["pos"] == full["pos"]


# ---------------------------------------------------------------------------
# decode and speculative verify
# ---------------------------------------------------------------------------
def test_decode_matches_per_slot_scan_and_handles_reset():
    S, H, P, N, b = 6, 3, 4, 5, 4
    r = np.random.default_rng(11)
    state = r.standard_normal((S, H, P, N))
    pos = np.arange(S, dtype=np.int64) + 100
    slots = np.array([4, 0, 5, 2], np.int32)
    x, dt, B, C = inputs.tokens(2, b, H, P, N, 1, 0)
    A, D = inputs.params(2, H)
    reset = np.array([0, 1, 0, 1], np.uint8)
    ref_states = state.copy()
    y = oracle.decode(state, pos, slots, x, dt, B, C, A, D, reset=reset)
    for i, s in enumerate(slots):
        st0 = np.zeros((H, P, N)) if reset[i] else ref_states[s]
        one = oracle.scan(x[i:i + 1], dt[i:i + 1], B[i:i + 1], C[i:i + 1], A, D, state=st0)
        assert np.array_equal(one["y"][0], y[i])
        assert np.array_equal(one["state"], state[s])
    untouched = [s for s in range(S) if s not in slots]
    assert np.array_equal(state[untouched], ref_states[untouched])
    assert pos[0] == 1 and pos[2] == 1 and pos[4] == 105 and pos[5] == 106 and pos[1] == 101


def test_spec_step_keeps_accepted_prefix():
    S, H, P, N, n_in = 3, 2, 3, 4, 5
    r = np.random.default_rng(12)
    state = r.standard_normal((S, H, P, N))
    pos = np.zeros(S, np.int64)
    slots = np.array([2, 0], np.int32)
    x, dt, B, C = inputs.spec_step_inputs(0, batch=2, n_in=n_in, H=H, P=P, N=N)
    A, D = inputs.params(3, H)
    acc = np.array([3, 1], np.int32)
    before = state.copy()
    y = oracle.spec_step(state, pos, slots, x, dt, B, C, A, D, acc)
    for i, s in enumerate(slots):
        run = oracle.scan(x[i], dt[i], B[i], C[i], A, D, state=before[s])
        assert np.array_equal(run["y"], y[i])
        keep = oracle.scan(x[i, :acc[i]], dt[i, :acc[i]], B[i, :acc[i]], C[i, :acc[i]], A, D,
                           state=before[s])
        assert np.array_equal(keep["state"], state[s])
    assert list(pos) == [1, 0, 3]


@pytest.mark.parametrize("W", [8, 16])
def test_replay_form_equals_recurrence(W):
    """Outputs from checkpoint + log (rearranged math) equal the step-by-step
    recurrence with rollback, within 1e-12, over random drafts and rejections
    (section "The Fix: Log the Inputs, Checkpoint the State": the rearranged
    form agrees with the recurrence to within 1e-12)."""
    H, P, N, n_in, steps = 2, 3, 4, 5, 14
    A, D = inputs.params(3, H)
    r = np.random.default_rng(W)
    ckpt = r.standard_normal((H, P, N)) * 0.1
    state = ckpt[None].copy()
    pos = np.zeros(1, np.int64)
    acc = inputs.acceptances(steps, 1, T=n_in - 1, p=0.7)
    sched = oracle.replay_schedule(acc, W, n_in)
    log = {"dt": [], "x": [], "B": []}
    worst = 0.0
    for s in range(steps):
        x, dt, B, C = inputs.spec_step_inputs(s, batch=1, n_in=n_in, H=H, P=P, N=N)
        if sched["flush"][s, 0]:
            n_log = len(log["dt"])
            M = n_log
            _, ckpt = oracle.replay_unrolled(ckpt, np.array(log["dt"]).reshape(M, H),
                                             np.array(log["x"]).reshape(M, H, P),
                                             np.array(log["B"]).reshape(M, 1, N),
                                             np.zeros((M, 1, N)), A, D, n_log)
            log = {"dt": [], "x": [], "B": []}
            np.testing.assert_allclose(ckpt, state[0], rtol=1e-12, atol=1e-12)
        assert len(log["dt"]) == sched["len_before"][s, 0]
        n_log = len(log["dt"])
        dt_all = np.concatenate([np.array(log["dt"]).reshape(n_log, H), dt[0]])
        x_all = np.concatenate([np.array(log["x"]).reshape(n_log, H, P), x[0]])
        B_all = np.concatenate([np.array(log["B"]).reshape(n_log, 1, N), B[0]])
        C_all = np.concatenate([np.zeros((n_log, 1, N)), C[0]])
        y_rep, _ = oracle.replay_unrolled(ckpt, dt_all, x_all, B_all, C_all, A, D, n_log)
        y_rec = oracle.spec_step(state, pos, [0], x, dt, B, C, A, D, acc[s])
        worst = max(worst, float(np.max(np.abs(y_rep - y_rec[0]))))
        a = int(acc[s, 0])
        for k in range(a):
            log["dt"].append(dt[0, k])
            log["x"].append(x[0, k])
            log["B"].append(B[0, k])
    assert worst < 1e-12
    assert sched["flushes"][0] >= 1


# ---------------------------------------------------------------------------
# acceptance model and flush schedule
# ---------------------------------------------------------------------------
def test_copy_rule_matches_printed_values():
    # "Implementing It", Role 1: 0.92 at p=0.6 and 1.34 at p=0.8, T=4
    assert round(oracle.copy_rule(0.6, 4), 2) == 0.92
    assert round(oracle.copy_rule(0.8, 4), 2) == 1.34
    assert abs(oracle.copy_rule(0.6, 4) - 0.92224) < 1e-12
    assert abs(oracle.copy_rule(0.8, 4) - 1.34464) < 1e-12
    # brute force over all accept/reject patterns of 4 drafts
    for p in (0.3, 0.7):
        tot = 0.0
        for mask in range(16):
            bits = [(mask >> i) & 1 for i in range(4)]
            prob = np.prod([p if b else 1 - p for b in bits])
            lead = 0
            while lead < 4 and bits[lead]:
                lead += 1
            tot += prob * (1 + lead)
        assert abs(tot - oracle.tokens_kept(p, 4)) < 1e-12


def test_sampled_acceptance_mean():
    acc = inputs.acceptances(128, 256, T=4, p=0.7)
    mean = oracle.expected_kept(0.7, 4)
    assert abs(mean - 2.7731) < 1e-12
    var = sum((1 + k) ** 2 * (0.7 ** k) * (0.3 if k < 4 else 1.0) for k in range(5)) - mean ** 2
    sigma = math.sqrt(var / acc.size)
    assert abs(acc.mean() - mean) < 4 * sigma
    assert acc.min() >= 1 and acc.max() <= 5


def test_flush_schedule_hand_cases():
    # one token per step, W=16: a flush before step 16, 32, ... (once every 16 steps)
    s = oracle.replay_schedule(np.ones((48, 1), np.int32), 16, 1)
    assert list(np.nonzero(s["flush"][:, 0])[0]) == [16, 32]
    # n_in = 5, W = 8, accepting 3, 2, 5, 1: lengths seen 0, 3 (3+5 fits), then
    # 5+5 > 8 flushes before step 2 and again before step 3
    acc = np.array([[3], [2], [5], [1]], np.int32)
    s = oracle.replay_schedule(acc, 8, 5)
    assert s["flush"][:, 0].tolist() == [False, False, True, True]
    assert s["len_before"][:, 0].tolist() == [0, 3, 0, 0]
    assert s["final_len"].tolist() == [1]
