"""Gated DeltaNet replay and copy-baseline parity: ReplaySSM verify of the
gated delta rule (checkpoint + log, queries carried back through the logged
rank-1 factors, fold when the log fills) and the copy-state-per-draft
baseline, through the C ABI, vs the fp64 oracle's step-by-step recurrence
with rollback.  Flush counts, log lengths and positions must match the
oracle's schedule exactly."""
import numpy as np
import pytest

import oracle
from oracle import gdn
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


@pytest.mark.parametrize("W,n_in,H,P,N,G,io,var", [
    (8, 5, 2, 64, 128, 1, "f32", None),
    (16, 5, 4, 64, 128, 2, "f32", None),    # two key groups
    (32, 5, 2, 128, 128, 1, "f32", None),   # two row tiles per head
    (8, 1, 2, 64, 128, 1, "f32", None),     # one token per step (plain decode through replay)
    (16, 5, 2, 64, 128, 1, "bf16", None),
    (5, 5, 2, 16, 32, 1, "f32", None),      # every step folds a full window
    (8, 5, 3, 40, 20, 1, "f32", None),      # ragged tile, N not a multiple of 32
    (64, 16, 2, 64, 128, 1, "f32", None),   # the largest window and in-flight count
    (8, 5, 2, 6, 16, 1, "f32", None),       # rows not whole 16-byte chunks
    (8, 5, 2, 12, 32, 1, "bf16", None),
    (16, 5, 2, 64, 128, 1, "f32", "xoff"),  # v 4 bytes past a 16-byte boundary
    (8, 5, 2, 200, 48, 1, "f32", None),     # 128-row tiles, the second ragged
    (16, 5, 2, 136, 128, 1, "bf16", None),  # 128-row tiles, an 8-row second tile
    (8, 3, 2, 130, 32, 1, "f32", None),     # 128-row tiles, rows not whole 16-byte chunks
    (16, 5, 2, 128, 128, 1, "f32", "strong"),  # dt x 25: gates down to e^-50 and below
    (64, 16, 2, 128, 128, 1, "f32", None),  # 128-row tile at the largest window and in-flight count
    (8, 5, 4, 256, 64, 2, "bf16", None),    # two 128-row tiles per head, two key groups
    (8, 5, 16, 64, 128, 8, "f32", None),    # two value heads per group, 16 heads (XCD-paired order)
    (16, 5, 32, 128, 64, 16, "f32", None),  # the same with 128-row tiles
])
def test_gdn_replay_and_copy_vs_oracle(ssm, W, n_in, H, P, N, G, io, var):
    S, b, steps = 6, 4, 40
    say("gdn replay small", W, n_in, H, P, N, G, io, var)
    A = inputs.params(45, H)[0]
    st0 = (np.random.default_rng(W + n_in).standard_normal((S, H, P, N)) * 0.1).astype(np.float32)
    kw = dict(G=G, io_dtype=io, recurrence="gated_delta")
    rep = ssm.StreamState(H, P, N, S, to_dev(A), None, **kw)
    cop = ssm.StreamState(H, P, N, S, to_dev(A), None, **kw)
    rep.init(np.arange(S), to_dev(st0))
    cop.init(np.arange(S), to_dev(st0))
    rep.replay_attach(W)
    cop.copy_attach(n_in)
    slots = np.array([5, 1, 2, 0], np.int32)
    ref_state = st0.astype(np.float64)
    ref_pos = np.zeros(S, np.int64)
    acc = inputs.acceptances(steps, b, T=n_in - 1, p=0.7) if n_in > 1 else \
        np.ones((steps, b), np.int32)
    sched = oracle.replay_schedule(acc, W, n_in)
    for s in range(steps):
        v, dt, beta, k, q = inputs.gdn_tokens(45, b * n_in, H, P, N, G, s)
        if var == "strong":  # products of gates that underflow fp32 within a window
            dt = dt * np.float32(25.0)
        arrs = [v.reshape(b, n_in, H, P), dt.reshape(b, n_in, H), beta.reshape(b, n_in, H),
                k.reshape(b, n_in, G, N), q.reshape(b, n_in, G, N)]
        if io == "bf16":
            bits = [inputs.bf16_bits(a) for a in arrs]
            arrs = [inputs.bf16_to_f32(a) for a in bits]
            dev = [bf16_dev(a) for a in bits]
        else:
            dev = [to_dev(a) for a in arrs]
        if var == "xoff":  # the same v values behind a one-element offset
            buf = torch.zeros(dev[0].numel() + 1, dtype=torch.float32, device="cuda")
            buf[1:] = dev[0].reshape(-1)
            dev[0] = buf[1:].view(dev[0].shape)
            assert dev[0].data_ptr() % 16 != 0
        y_rep = rep.gdn_replay_step(slots, *dev)
        y_cop = cop.gdn_copy_step(slots, *dev)
        ref_y = gdn.spec_step(ref_state, ref_pos, slots, *arrs, A, acc[s])
        torch.cuda.synchronize()
        tol = bf16_tol(ref_y) if io == "bf16" else F32_TOL
        assert_close(host(y_rep), ref_y, what=f"replay o step {s}", **tol)
        assert_close(host(y_cop), ref_y, what=f"copy o step {s}", **tol)
        rep.replay_commit(slots, acc[s])
        cop.copy_commit(slots, acc[s])
        for i, sl in enumerate(slots):
            assert rep.log_state(int(sl))[0] == sched["len_before"][s, i] + acc[s, i]
    assert rep.counters()["replay_flushes"] == int(sched["flushes"].sum())
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
def test_gdn_workload_full_batch(ssm, W):
    """B=256 slots, 32 value heads over 16 key groups, P = N = 128 (2 MiB of
    fp32 state per slot), T=4 drafts accepted with p=0.7, 128 steps: replay and
    the copy baseline on the same seeded inputs, every output of every slot
    against the threaded oracle; flush count, positions and final states."""
    Wc = inputs.W5
    B_, H, P, N, G = Wc["batch"], Wc["H"], Wc["P"], Wc["N"], Wc["G"]
    n_in, steps = Wc["T"] + 1, Wc["steps"]
    say("gdn workload", W, steps)
    A = inputs.params(5, H)[0]
    init = inputs.device_state(5, B_, H, P, N)
    kw = dict(G=G, recurrence="gated_delta")
    h = ssm.StreamState(H, P, N, B_, to_dev(A), None, **kw)
    c = ssm.StreamState(H, P, N, B_, to_dev(A), None, **kw)
    h.init(np.arange(B_), init)
    c.init(np.arange(B_), init)
    h.replay_attach(W)
    c.copy_attach(n_in)
    slots = np.arange(B_, dtype=np.int32)
    acc = inputs.acceptances(steps, B_, T=Wc["T"], p=Wc["p"], workload=5)
    sched = oracle.replay_schedule(acc, W, n_in)
    ref_state = host(init)
    del init
    ref_pos = np.zeros(B_, np.int64)
    for s in range(steps):
        v, dt, beta, k, q = inputs.device_gdn_tokens(5, B_ * n_in, H, P, N, G, seed_extra=s)
        dev = [v.view(B_, n_in, H, P), dt.view(B_, n_in, H), beta.view(B_, n_in, H),
               k.view(B_, n_in, G, N), q.view(B_, n_in, G, N)]
        y = h.gdn_replay_step(slots, *dev)
        yc = c.gdn_copy_step(slots, *dev)
        ref_y = gdn.spec_step(ref_state, ref_pos, slots, *[host(t) for t in dev], A, acc[s],
                              n_threads=None)
        assert_close(host(y), ref_y, what=f"replay o step {s}", **F32_TOL)
        assert_close(host(yc), ref_y, what=f"copy o step {s}", **F32_TOL)
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


def test_gdn_checkpoint_restore_and_recurrence_guard(ssm):
    """A Gated DeltaNet slot's checkpoint (with a replay log folded in)
    restores bit for bit and continues identically; its receipt names the
    recurrence, so a Mamba-2 handle of the same shape refuses it, and each
    recurrence's calls refuse the other's handles."""
    H, P, N, G, S, W = 2, 64, 128, 1, 3, 8
    say("gdn checkpoint")
    A = inputs.params(46, H)[0]
    h = ssm.StreamState(H, P, N, S, to_dev(A), None, G=G, recurrence="gated_delta")
    h.reset(range(S))
    h.replay_attach(W)
    slots = np.array([0], np.int32)
    for s in range(3):
        v, dt, beta, k, q = inputs.gdn_tokens(46, 2, H, P, N, G, s)
        dev = [to_dev(a.reshape((1, 2) + a.shape[1:])) for a in (v, dt, beta, k, q)]
        h.gdn_replay_step(slots, *dev)
        h.replay_commit(slots, [2])
    ck, rc = h.checkpoint(0)
    torch.cuda.synchronize()
    assert rc["recurrence"] == ssm.SSM_GATED_DELTA and rc["position"] == 6
    h.restore(1, ck, rc)
    v, dt, beta, k, q = inputs.gdn_tokens(46, 2, H, P, N, G, 9)
    outs = []
    for sl in (0, 1):
        dev = [to_dev(a.reshape((1, 2) + a.shape[1:])) for a in (v, dt, beta, k, q)]
        outs.append(h.gdn_replay_step([sl], *dev))
        h.replay_commit([sl], [2])
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    m = ssm.StreamState(H, P, N, 1, to_dev(A), to_dev(np.zeros(H, np.float32)), G=G)
    with pytest.raises(ssm.SSMError) as e:
        m.restore(0, ck, rc)
    assert e.value.code == ssm.SSM_E_SCHEMA and "recurrence" in str(e.value)
    z = lambda *shape: torch.zeros(shape, device="cuda")  # noqa: E731
    m.replay_attach(W)
    with pytest.raises(ssm.SSMError) as e:
        m.gdn_replay_step([0], z(1, 1, H, P), z(1, 1, H), z(1, 1, H), z(1, 1, G, N), z(1, 1, G, N))
    assert e.value.code == ssm.SSM_E_INVALID_ARG and "Mamba-2" in str(e.value)
    with pytest.raises(ssm.SSMError) as e:
        h.decode_step([2], z(1, H, P), z(1, H), z(1, G, N), z(1, G, N))
    assert e.value.code == ssm.SSM_E_INVALID_ARG and "Gated DeltaNet" in str(e.value)
    h.destroy()
    m.destroy()
