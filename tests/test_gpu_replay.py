"""Replay and copy-baseline parity: ReplaySSM verify (checkpoint + log, fused
fold when the log fills) and the copy-state-per-draft baseline, through the C
ABI, vs the oracle's step-by-step recurrence with rollback.  Flush counts and
positions must match the oracle's schedule exactly."""
import numpy as np
import pytest

import oracle
from streaming_state_amd import inputs
from tests.gpu_helpers import F32_TOL, assert_close, bf16_dev, bf16_tol, host, say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ssm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from streaming_state_amd import ssm as m
    return m


@pytest.mark.parametrize("W,n_in,H,P,N,G,io,neg", [
    (8, 5, 2, 8, 16, 1, "f32", False),
    (16, 5, 3, 40, 20, 1, "f32", False),
    (32, 5, 4, 72, 128, 2, "f32", False),
    (8, 1, 2, 64, 128, 1, "f32", False),   # one token per step: the plain-decode case
    (16, 5, 2, 64, 128, 1, "bf16", False),
    (5, 5, 2, 16, 32, 1, "f32", False),    # every step flushes a full window
    (64, 16, 2, 64, 128, 1, "f32", False),  # the largest window and in-flight count (>64 KiB LDS)
    (8, 5, 2, 64, 128, 1, "f32", True),    # some dt negative (accepted input)
    # rows that are not whole 16-byte chunks: the element-copy staging, whose
    # x rows sit at a stride rounded up to 8 (fp32 P=6, bf16 P=12)
    (8, 5, 2, 6, 16, 1, "f32", False),
    (8, 5, 3, 12, 32, 1, "bf16", False),
    (16, 5, 2, 70, 128, 1, "f32", False),  # a 6-row second tile
    (16, 5, 2, 64, 128, 1, "f32", "xoff"),  # x 4 bytes past a 16-byte boundary
])
def test_replay_and_copy_vs_oracle(ssm, W, n_in, H, P, N, G, io, neg):
    S, b, steps = 6, 4, 40
    say("replay small", W, n_in, H, P, N, G, io, neg)
    A, D = inputs.params(40, H)
    st0 = np.random.default_rng(W).standard_normal((S, H, P, N)).astype(np.float32) * 0.1
    rep = ssm.StreamState(H, P, N, S, to_dev(A), to_dev(D), G=G, io_dtype=io)
    cop = ssm.StreamState(H, P, N, S, to_dev(A), to_dev(D), G=G, io_dtype=io)
    rep.init(np.arange(S), to_dev(st0))
    cop.init(np.arange(S), to_dev(st0))
    rep.replay_attach(W)
    cop.copy_attach(n_in)
    slots = np.array([5, 1, 2, 0], np.int32)
    ref_state = st0.astype(np.float64).copy()
    ref_pos = np.zeros(S, np.int64)
    acc = inputs.acceptances(steps, b, T=n_in - 1, p=0.7) if n_in > 1 else \
        np.ones((steps, b), np.int32)
    sched = oracle.replay_schedule(acc, W, n_in)
    for s in range(steps):
        x, dt, B, C = inputs.spec_step_inputs(s, batch=b, n_in=n_in, H=H, P=P, N=N, G=G,
                                              workload=40)
        if neg is True:
            dt = dt.copy()
            dt[:, s % n_in, s % H] = -0.02
        if io == "bf16":
            bits = [inputs.bf16_bits(a) for a in (x, dt, B, C)]
            x, dt, B, C = [inputs.bf16_to_f32(a) for a in bits]
            dev = [bf16_dev(a) for a in bits]
        else:
            dev = [to_dev(a) for a in (x, dt, B, C)]
        if neg == "xoff":  # the same x values behind a one-element offset
            buf = torch.zeros(x.size + 1, dtype=torch.float32, device="cuda")
            buf[1:] = dev[0].reshape(-1)
            dev[0] = buf[1:].view(x.shape)
            assert dev[0].data_ptr() % 16 != 0
        y_rep = rep.replay_step(slots, *dev)
        y_cop = cop.copy_step(slots, *dev)
        ref_y = oracle.spec_step(ref_state, ref_pos, slots, x, dt, B, C, A, D, acc[s])
        torch.cuda.synchronize()
        tol = bf16_tol(ref_y) if io == "bf16" else F32_TOL
        assert_close(host(y_rep), ref_y, what=f"replay y step {s}", **tol)
        assert_close(host(y_cop), ref_y, what=f"copy y step {s}", **tol)
        rep.replay_commit(slots, acc[s])
        cop.copy_commit(slots, acc[s])
        for i, sl in enumerate(slots):
            assert rep.log_state(int(sl))[0] == sched["len_before"][s, i] + acc[s, i]
    c = rep.counters()
    assert c["replay_flushes"] == int(sched["flushes"].sum())
    rep.materialize(slots)
    cop.materialize(slots)
    torch.cuda.synchronize()
    stol = bf16_tol(ref_state) if io == "bf16" else F32_TOL
    assert_close(host(rep.state), ref_state, what="replay state", **stol)
    assert_close(host(cop.state), ref_state, what="copy state", **stol)
    for sl in range(S):
        assert rep.position(sl)[0] == ref_pos[sl] == cop.position(sl)[0]
    rep.destroy()
    cop.destroy()


@pytest.mark.parametrize("W", [8, 16, 32])
def test_replay_workload3_full_batch(ssm, W):
    """B=256, H=128, P=64, N=128, T=4 drafts accepted with p=0.7, 128 steps:
    ReplaySSM and the copy-state-per-draft baseline on the same seeded inputs,
    every output of every slot and step against the threaded oracle, the
    flush count against the oracle's schedule, positions and final states."""
    Wc = inputs.W3
    B_, H, P, N, G = Wc["batch"], Wc["H"], Wc["P"], Wc["N"], Wc["G"]
    n_in, steps = Wc["T"] + 1, Wc["steps"]
    say("replay workload3", W, steps)
    A, D = inputs.params(3, H)
    init = inputs.device_state(3, B_, H, P, N)
    h = ssm.StreamState(H, P, N, B_, to_dev(A), to_dev(D), G=G)
    h.init(np.arange(B_), init)
    h.replay_attach(W)
    c = ssm.StreamState(H, P, N, B_, to_dev(A), to_dev(D), G=G)
    c.init(np.arange(B_), init)
    c.copy_attach(n_in)
    slots = np.arange(B_, dtype=np.int32)
    acc = inputs.acceptances(steps, B_, T=Wc["T"], p=Wc["p"])
    sched = oracle.replay_schedule(acc, W, n_in)
    ref_state = host(init)
    del init
    ref_pos = np.zeros(B_, np.int64)
    for s in range(steps):
        x, dt, B, C = inputs.device_tokens(3, B_ * n_in, H, P, N, G, seed_extra=s)
        x, dt = x.view(B_, n_in, H, P), dt.view(B_, n_in, H)
        B, C = B.view(B_, n_in, G, N), C.view(B_, n_in, G, N)
        y = h.replay_step(slots, x, dt, B, C)
        yc = c.copy_step(slots, x, dt, B, C)
        ref_y = oracle.spec_step(ref_state, ref_pos, slots, host(x), host(dt), host(B),
                                 host(C), A, D, acc[s], n_threads=None)
        assert_close(host(y), ref_y, what=f"replay y step {s}", **F32_TOL)
        assert_close(host(yc), ref_y, what=f"copy y step {s}", **F32_TOL)
        h.replay_commit(slots, acc[s])
        c.copy_commit(slots, acc[s])
        for b in range(B_):
            assert h.log_state(b)[0] == sched["len_before"][s, b] + acc[s, b]
    assert h.counters()["replay_flushes"] == int(sched["flushes"].sum())
    h.materialize(slots)
    c.materialize(slots)
    assert_close(host(h.state), ref_state, what="replay state", **F32_TOL)
    assert_close(host(c.state), ref_state, what="copy state", **F32_TOL)
    for b in range(B_):
        assert h.position(b)[0] == c.position(b)[0] == ref_pos[b]
    h.destroy()
    c.destroy()


def test_replay_alone_matches_decode(ssm):
    """One token per step through ReplaySSM (no drafts, W=16) against plain
    decode on the same inputs: equal outputs every step, and after the log is
    folded back the same state, over 40 steps (two folds).  Both also agree
    with the oracle's decode."""
    S, H, P, N, G, W, steps = 12, 3, 64, 128, 1, 16, 40
    say("replay alone vs decode", S, H, P, N, W, steps)
    A, D = inputs.params(2, H)
    r = np.random.default_rng(7)
    st0 = (r.standard_normal((S, H, P, N)) * 0.05).astype(np.float32)
    dec = ssm.StreamState(H, P, N, S, to_dev(A), to_dev(D), G=G)
    rep = ssm.StreamState(H, P, N, S, to_dev(A), to_dev(D), G=G)
    slots = np.arange(S, dtype=np.int32)
    dec.init(slots, to_dev(st0))
    rep.init(slots, to_dev(st0))
    rep.replay_attach(W)
    ref_state = st0.astype(np.float64)
    ref_pos = np.zeros(S, np.int64)
    ones = np.ones(S, np.int32)
    for step in range(steps):
        x, dt, B, C = inputs.tokens(33, S, H, P, N, G, step)
        dev = [to_dev(a) for a in (x, dt, B, C)]
        yd = dec.decode_step(slots, *dev)
        yr = rep.replay_step(slots, dev[0][:, None], dev[1][:, None], dev[2][:, None],
                             dev[3][:, None])
        rep.replay_commit(slots, ones)
        ref = oracle.decode(ref_state, ref_pos, slots, x, dt, B, C, A, D)
        torch.cuda.synchronize()
        assert_close(host(yr[:, 0]), host(yd), what=f"replay vs decode step {step}", **F32_TOL)
        assert_close(host(yd), ref, what=f"decode vs oracle step {step}", **F32_TOL)
    # the log fills after W steps: the folds come before steps W and 2W
    assert rep.counters()["replay_flushes"] == 2 * S
    rep.materialize(slots)
    torch.cuda.synchronize()
    assert_close(host(rep.state), host(dec.state), what="materialized state", **F32_TOL)
    assert_close(host(dec.state), ref_state, what="state vs oracle", **F32_TOL)
    for b in range(S):
        assert rep.position(b)[0] == dec.position(b)[0] == steps
    dec.destroy()
    rep.destroy()
