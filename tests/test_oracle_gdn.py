"""Pins of the Gated DeltaNet oracle (oracle/gdn_oracle.c) against statements
independent of its loops: the recurrence as explicit matrix products, the
delta rule's key-value overwrite with one-hot keys (exact), the read-back
property (after a full-strength write of (k, v) the state maps k to v), the
beta = 0 case (a pure scalar decay), chunked == full bitwise with resets, and
the replay form (checkpoint plus logged factors) against the step-by-step
recurrence with rollback to 1e-12 over random drafts and rejections."""
import numpy as np
import pytest

import oracle
from oracle import gdn
from streaming_state_amd import inputs


def _rand(seed, L, H, P, N, G, unit_k=False):
    r = np.random.default_rng(seed)
    v = r.standard_normal((L, H, P))
    dt = np.log1p(np.exp(r.normal(-2.0, 0.5, (L, H))))
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((L, H))))
    k = r.standard_normal((L, G, N))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = r.standard_normal((L, G, N)) * 0.3
    A = -np.exp(r.uniform(0, np.log(16), H))
    S0 = r.standard_normal((H, P, N)) * 0.1
    return v, dt, beta, k, q, A, S0


@pytest.mark.parametrize("H,P,N,G", [(3, 3, 4, 1), (4, 2, 5, 2), (2, 5, 3, 2)])
def test_matches_explicit_matrix_products(H, P, N, G):
    """S_t = S_{t-1} A_t + beta_t v_t k_t^T with A_t = alpha_t (I - beta_t k_t k_t^T)
    formed as an N x N matrix, o_t = S_t q_t; keys are not normalised here."""
    L = 11
    v, dt, beta, k, q, A, S0 = _rand(H * 100 + N, L, H, P, N, G)
    r = gdn.scan(v, dt, beta, k, q, A, state=S0, pos=3)
    S = S0.copy()
    for t in range(L):
        for h in range(H):
            g = h // (H // G)
            alpha = np.exp(dt[t, h] * A[h])
            At = alpha * (np.eye(N) - beta[t, h] * np.outer(k[t, g], k[t, g]))
            S[h] = S[h] @ At + beta[t, h] * np.outer(v[t, h], k[t, g])
            np.testing.assert_allclose(r["o"][t, h], S[h] @ q[t, g], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["state"], S, rtol=1e-12, atol=1e-12)
    assert r["pos"] == 3 + L


def test_one_hot_keys_overwrite_columns_exactly():
    """alpha = 1 (dt = 0), beta = 1 and one-hot keys e_i: each token replaces
    column i of the state by v_t and leaves the rest; o_t = S_t q_t.  Every
    value is a small dyadic number, so the results are exact."""
    H, P, N, G, L = 2, 3, 4, 1, 9
    r = np.random.default_rng(7)
    cols = [2, 0, 2, 3, 1, 1, 0, 3, 2]
    v = r.integers(-8, 9, (L, H, P)) / 4.0
    k = np.zeros((L, G, N))
    k[np.arange(L), 0, cols] = 1.0
    q = r.integers(-4, 5, (L, G, N)) / 2.0
    S0 = r.integers(-8, 9, (H, P, N)) / 8.0
    out = gdn.scan(v, np.zeros((L, H)), np.ones((L, H)), k, q, np.full(H, -3.0), state=S0)
    table = S0.copy()
    for t in range(L):
        table[:, :, cols[t]] = v[t]
        for h in range(H):
            assert np.array_equal(out["o"][t, h], table[h] @ q[t, 0])
    assert np.array_equal(out["state"], table)


def test_full_write_reads_back_its_value():
    """With beta = 1 and alpha = 1 the write makes the state return v_t at the
    unit key k_t, whatever it held before: S_t k_t = v_t."""
    H, P, N, G, L = 3, 4, 6, 1, 7
    v, _, _, k, q, A, S0 = _rand(11, L, H, P, N, G, unit_k=True)
    st, pos = S0, 0
    for t in range(L):
        r = gdn.scan(v[t:t + 1], np.zeros((1, H)), np.ones((1, H)), k[t:t + 1], q[t:t + 1], A,
                     state=st, pos=pos)
        st, pos = r["state"], r["pos"]
        for h in range(H):
            np.testing.assert_allclose(st[h] @ k[t, 0], v[t, h], rtol=0, atol=1e-12)


def test_beta_zero_is_a_pure_decay():
    """beta = 0: nothing is written or erased, S_t = (prod alpha) S_0 and
    o_t = (prod_{i<=t} alpha_i) S_0 q_t."""
    H, P, N, G, L = 2, 3, 5, 1, 10
    v, dt, _, k, q, A, S0 = _rand(12, L, H, P, N, G)
    r = gdn.scan(v, dt, np.zeros((L, H)), k, q, A, state=S0)
    for h in range(H):
        for t in range(L):
            lam = np.exp(A[h] * dt[:t + 1, h].sum())
            np.testing.assert_allclose(r["o"][t, h], lam * (S0[h] @ q[t, 0]), rtol=1e-13,
                                       atol=1e-15)
        np.testing.assert_allclose(r["state"][h], np.exp(A[h] * dt[:, h].sum()) * S0[h],
                                   rtol=1e-13, atol=1e-15)


def test_chunked_equals_full_and_reset_separates():
    """Chunked == full bitwise for several partitions; a reset restarts from
    zero (reset-then-B == fresh-B bitwise) and differs from no reset."""
    H, P, N, G, L = 2, 3, 8, 2, 40
    v, dt, beta, k, q, A, _ = _rand(13, L, H, P, N, G, unit_k=True)
    reset = np.zeros(L, np.uint8)
    reset[17] = 1
    full = gdn.scan(v, dt, beta, k, q, A, reset=reset)
    for sizes in ([1] * L, [3, 0, 14, 23], [17, 23], [5, 7, 11, 13, 4]):
        st, pos, outs, t0 = None, 0, [], 0
        for sz in sizes:
            sl = slice(t0, t0 + sz)
            r = gdn.scan(v[sl], dt[sl], beta[sl], k[sl], q[sl], A, state=st, pos=pos,
                         reset=reset[sl])
            outs.append(r["o"])
            st, pos, t0 = r["state"], r["pos"], t0 + sz
        assert np.array_equal(np.concatenate(outs), full["o"]), sizes
        assert np.array_equal(st, full["state"]) and pos == full["pos"] == L - 17
    fresh = gdn.scan(v[17:], dt[17:], beta[17:], k[17:], q[17:], A)
    assert np.array_equal(fresh["o"], full["o"][17:])
    none = gdn.scan(v, dt, beta, k, q, A)
    assert np.abs(none["o"][17] - full["o"][17]).max() > 1e-6


def test_nonfinite_input_rejected():
    H, P, N, G, L = 2, 2, 4, 1, 5
    v, dt, beta, k, q, A, S0 = _rand(14, L, H, P, N, G)
    beta[3, 1] = np.nan
    with pytest.raises(oracle.OracleError) as e:
        gdn.scan(v, dt, beta, k, q, A, state=S0)
    assert e.value.code == oracle.ORC_E_INVALID_CHUNK


@pytest.mark.parametrize("W,n_in,G", [(8, 5, 1), (16, 5, 2), (5, 5, 1), (6, 1, 1)])
def test_replay_form_equals_recurrence(W, n_in, G):
    """ReplaySSM for the gated delta rule: outputs from the checkpoint and the
    logged entries (each query carried back through the entries' rank-1
    factors) and the fold (an explicit product of the factors) equal the
    step-by-step recurrence with rollback within 1e-12 over 30 steps of random
    drafts and rejections, with the flush rule of the Mamba-2 path."""
    S_, H, P, N, steps = 3, 4, 5, 8, 30
    A = inputs.params(70, H)[0].astype(np.float64)
    r = np.random.default_rng(W * 10 + n_in)
    state = r.standard_normal((S_, H, P, N)) * 0.1
    ckpt = state.copy()
    pos = np.zeros(S_, np.int64)
    logs = [[] for _ in range(S_)]
    slots = np.arange(S_)
    acc = inputs.acceptances(steps, S_, T=n_in - 1, p=0.7) if n_in > 1 else \
        np.ones((steps, S_), np.int32)
    n_fold = 0
    for s in range(steps):
        v, dt, beta, k, q = inputs.gdn_tokens(70, S_ * n_in, H, P, N, G, s)
        v, dt, beta = v.reshape(S_, n_in, H, P), dt.reshape(S_, n_in, H), beta.reshape(S_, n_in, H)
        k, q = k.reshape(S_, n_in, G, N), q.reshape(S_, n_in, G, N)
        o_rec = gdn.spec_step(state, pos, slots, v, dt, beta, k, q, A, acc[s])
        for b in range(S_):
            if len(logs[b]) + n_in > W:  # the log is full: fold it into the checkpoint
                ent = logs[b]
                _, ckpt[b] = gdn.replay_unrolled(
                    ckpt[b], np.array([e[1] for e in ent]), np.array([e[2] for e in ent]),
                    np.array([e[0] for e in ent]), np.array([e[3] for e in ent]),
                    np.array([e[4] for e in ent]), A, n_log=len(ent))
                logs[b] = []
                n_fold += 1
            new = [(v[b, i], dt[b, i], beta[b, i], k[b, i], q[b, i]) for i in range(n_in)]
            ent = logs[b] + new
            o_rep, _ = gdn.replay_unrolled(
                ckpt[b], np.array([e[1] for e in ent]), np.array([e[2] for e in ent]),
                np.array([e[0] for e in ent]), np.array([e[3] for e in ent]),
                np.array([e[4] for e in ent]), A, n_log=len(logs[b]))
            np.testing.assert_allclose(o_rep, o_rec[b], rtol=0, atol=1e-12)
            logs[b] += new[:acc[s, b]]
    assert n_fold > 0
    for b in range(S_):
        ent = logs[b]
        if ent:
            _, ckpt[b] = gdn.replay_unrolled(
                ckpt[b], np.array([e[1] for e in ent]), np.array([e[2] for e in ent]),
                np.array([e[0] for e in ent]), np.array([e[3] for e in ent]),
                np.array([e[4] for e in ent]), A, n_log=len(ent))
    np.testing.assert_allclose(ckpt, state, rtol=0, atol=1e-12)
    assert (pos == acc.sum(axis=0)).all()
