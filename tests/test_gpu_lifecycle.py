"""Lifecycle on the GPU: checkpoint/restore receipts with bit-exact
continuation, slot reuse after reset, non-finite rejection, reordering and
duplicates rejected with the state untouched, and determinism."""
import numpy as np
import pytest

from streaming_state_amd import inputs
from tests.gpu_helpers import say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ssm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from streaming_state_amd import ssm as m
    return m


def _layer(ssm, S=4, H=4, P=64, N=128, **kw):
    A, D = inputs.params(50, H)
    h = ssm.StreamState(H, P, N, S, to_dev(A), to_dev(D), **kw)
    h.reset(np.arange(S))
    return h


def test_checkpoint_restore_bit_exact_continuation(ssm):
    """Decode 40 tokens, checkpoint, decode 60 more; restoring the checkpoint
    into another slot and decoding the same 60 gives bit-identical outputs and
    state (hydration as in the pion page's validation)."""
    say("checkpoint/restore")
    H, P, N = 4, 64, 128
    h = _layer(ssm, S=3, H=H, P=P, N=N, schema_version=7, model_rev=11)
    toks = [inputs.device_tokens(51, 1, H, P, N, 1, seed_extra=s) for s in range(100)]
    for s in range(40):
        h.decode_step([0], *toks[s])
    snap, receipt = h.checkpoint(0)
    assert receipt["position"] == 40 and receipt["schema_version"] == 7
    assert receipt["H"] == H and receipt["model_rev"] == 11
    ya = [h.decode_step([0], *toks[s]) for s in range(40, 100)]
    h.restore(2, snap, receipt)
    assert h.position(2)[0] == 40
    yb = [h.decode_step([2], *toks[s]) for s in range(40, 100)]
    torch.cuda.synchronize()
    for a, b in zip(ya, yb):
        assert torch.equal(a, b)
    assert torch.equal(h.state[0], h.state[2])
    # a corrupted state or an incompatible receipt is rejected, slot untouched
    before = h.state[1].clone()
    bad = snap.clone()
    bad[0, 0, 0] += 1.0
    with pytest.raises(ssm.SSMError) as e:
        h.restore(1, bad, receipt)
    assert e.value.code == ssm.SSM_E_SCHEMA
    with pytest.raises(ssm.SSMError) as e:
        h.restore(1, snap, dict(receipt, schema_version=8))
    assert e.value.code == ssm.SSM_E_SCHEMA
    assert torch.equal(before, h.state[1])
    h.destroy()


def test_checkpoint_flushes_replay_log(ssm):
    say("checkpoint after replay")
    H, P, N = 2, 64, 128
    h = _layer(ssm, S=2, H=H, P=P, N=N)
    ref = _layer(ssm, S=2, H=H, P=P, N=N)
    h.replay_attach(16)
    x, dt, B, C = inputs.device_tokens(52, 5, H, P, N, 1, seed_extra=0)
    h.replay_step([1], x[None], dt[None], B[None], C[None])
    h.replay_commit([1], [3])
    snap, r = h.checkpoint(1)
    assert r["position"] == 3 and h.log_state(1) == (0, 0)
    ref.scan_chunk(1, 0, x[:3], dt[:3], B[:3], C[:3])
    torch.cuda.synchronize()
    assert torch.allclose(snap, ref.state[1], rtol=1e-5, atol=1e-6)


def test_slot_reuse_reset_flag(ssm):
    """A decode reset flag makes the slot's next occupant start from zero: its
    output equals that of a freshly reset slot."""
    say("slot reuse")
    H, P, N = 4, 64, 128
    h = _layer(ssm, S=2, H=H, P=P, N=N)
    for s in range(10):
        h.decode_step([0], *inputs.device_tokens(53, 1, H, P, N, 1, seed_extra=s))
    t = inputs.device_tokens(53, 1, H, P, N, 1, seed_extra=99)
    y_reuse = h.decode_step([0], *t, reset=[1])
    y_fresh = h.decode_step([1], *t)
    torch.cuda.synchronize()
    assert torch.equal(y_reuse, y_fresh)
    assert h.position(0)[0] == 1


def test_nonfinite_rejected_state_untouched(ssm):
    say("non-finite")
    H, P, N = 2, 64, 128
    h = _layer(ssm, S=2, H=H, P=P, N=N, check_finite=True)
    x, dt, B, C = inputs.device_tokens(54, 8, H, P, N, 1, seed_extra=0)
    h.scan_chunk(0, 0, x, dt, B, C)
    before = h.state.clone()
    bad = x.clone()
    bad[3, 1, 7] = float("nan")
    with pytest.raises(ssm.SSMError) as e:
        h.scan_chunk(0, 1, bad, dt, B, C)
    assert e.value.code == ssm.SSM_E_INVALID_CHUNK
    bad_dt = dt[:1].clone()
    bad_dt[0, 0] = float("inf")
    with pytest.raises(ssm.SSMError):
        h.decode_step([1], x[:1], bad_dt, B[:1], C[:1])
    torch.cuda.synchronize()
    assert torch.equal(before, h.state)
    assert h.position(0) == (8, 1) and h.position(1) == (0, 0)
    h.scan_chunk(0, 1, x, dt, B, C)  # the same chunk number is still accepted


def test_duplicate_and_reordered_chunks_rejected(ssm):
    say("chunk order")
    H, P, N = 2, 64, 128
    h = _layer(ssm, S=1, H=H, P=P, N=N)
    x, dt, B, C = inputs.device_tokens(55, 16, H, P, N, 1, seed_extra=0)
    h.scan_chunk(0, 0, x[:8], dt[:8], B[:8], C[:8])
    snap = h.state.clone()
    for seq in (0, 2):
        with pytest.raises(ssm.SSMError) as e:
            h.scan_chunk(0, seq, x[8:], dt[8:], B[8:], C[8:])
        assert e.value.code == ssm.SSM_E_SEQUENCE
    torch.cuda.synchronize()
    assert torch.equal(snap, h.state)


def test_runs_are_deterministic(ssm):
    say("determinism")
    H, P, N = 4, 64, 128
    outs = []
    for _ in range(2):
        h = _layer(ssm, S=1, H=H, P=P, N=N)
        x, dt, B, C = inputs.device_tokens(56, 300, H, P, N, 1, seed_extra=0)
        y = h.scan_chunk(0, 0, x, dt, B, C)
        torch.cuda.synchronize()
        outs.append((y.clone(), h.state.clone()))
        h.destroy()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
