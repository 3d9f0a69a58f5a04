"""State blobs on the GPU: serialization in the reference format of the
recurrent-state companion store ("SSM.PREFIX.* -- recurrent-state companion",
pion docs) and bit-exact hydration.

The page validates hydration as bit-perfect: a Mamba-130M fp32 stream decoded
for 2048 tokens through a snapshot agrees with the run that took no snapshot,
with a maximum absolute difference of zero.  Here one Mamba-130M layer's state
shape (24 heads of P=64, N=128) is decoded for 1024 tokens, serialized,
hydrated into another slot, and both slots decode the remaining 1024 tokens.
Blob bytes are read back with the oracle's independent reader; the state it
holds and the outputs after hydration are also checked against the fp64
oracle.
"""
import numpy as np
import pytest

import oracle
from oracle import blob as oblob
from streaming_state_amd import inputs
from tests.gpu_helpers import F32_TOL, assert_close, host, receipt_checksum, say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ssm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from streaming_state_amd import ssm as m
    return m


def _layer(ssm, workload, S, H, P, N, **kw):
    A, D = inputs.params(workload, H)
    h = ssm.StreamState(H, P, N, S, to_dev(A), to_dev(D), **kw)
    h.reset(np.arange(S))
    return h, A, D


def test_hydration_bit_exact_over_2048_decode_tokens(ssm):
    H, P, N, L, half = 24, 64, 128, 2048, 1024
    say("blob hydration", dict(H=H, P=P, N=N, L=L))
    h, A, D = _layer(ssm, 61, 2, H, P, N, schema_version=1, model_rev=130)
    x, dt, B, C = inputs.tokens(61, L, H, P, N)
    xd, dtd, Bd, Cd = (to_dev(a) for a in (x, dt, B, C))
    for t in range(half):
        h.decode_step([0], xd[t:t + 1], dtd[t:t + 1], Bd[t:t + 1], Cd[t:t + 1])
    blob, rec = h.serialize(0)
    assert len(blob) == h.blob_bytes() == 28 + H * P * N * 4
    assert rec["position"] == half and rec["model_rev"] == 130

    # the bytes follow the page's layout and hold the slot's state
    arrays = oblob.read(blob)
    assert len(arrays) == 1 and arrays[0][0] == oblob.F32
    snap = arrays[0][1]
    assert snap.shape == (H, P, N)
    assert snap.tobytes() == h.state[0].cpu().numpy().tobytes()
    assert rec["checksum"] == receipt_checksum(snap)
    ref = oracle.scan(x, dt, B, C, A, D)
    assert_close(snap, oracle.scan(x[:half], dt[:half], B[:half], C[:half], A, D)["state"],
                 **F32_TOL, what="serialized state vs oracle")

    # hydrate into slot 1, then both slots take the same second half
    h.deserialize(1, blob, rec)
    assert h.position(1) == h.position(0)
    ys = []
    for t in range(half, L):
        two = lambda a: a[t:t + 1].expand(2, *a.shape[1:]).contiguous()
        ys.append(h.decode_step([0, 1], two(xd), two(dtd), two(Bd), two(Cd)).clone())
    torch.cuda.synchronize()
    y = torch.stack(ys)
    diff = (y[:, 0] - y[:, 1]).abs().max().item()
    assert diff == 0.0 and torch.equal(y[:, 0], y[:, 1])
    assert torch.equal(h.state[0], h.state[1])
    b0, r0 = h.serialize(0)
    b1, r1 = h.serialize(1)
    assert b0 == b1 and r0 == r1 and r1["position"] == L
    assert_close(host(y[:, 1]), ref["y"][half:], **F32_TOL, what="outputs after hydration")
    assert_close(host(h.state[1]), ref["state"], **F32_TOL, what="final state")
    h.destroy()


def test_hydrate_blobs_written_by_the_oracle(ssm):
    """fp16 (widened exactly), bf16-as-fp32, and a Mamba pair
    [conv_state, ssm_state] whose second array is the state; decoding then
    continues from exactly those values."""
    H, P, N = 4, 64, 128
    say("oracle-written blobs", dict(H=H, P=P, N=N))
    h, A, D = _layer(ssm, 62, 4, H, P, N, schema_version=2, model_rev=9)
    _, base = h.serialize(0)
    rng = np.random.default_rng(62)
    s16 = (rng.standard_normal((1, H, P, N)) * 0.5).astype(np.float16)
    sbf = inputs.bf16_to_f32(inputs.bf16_bits(rng.standard_normal((H, P, N)) * 0.1))
    s32 = (rng.standard_normal((H, P, N)) * 0.1).astype(np.float32)
    conv = rng.standard_normal((1, H * P + 2 * N, 4)).astype(np.float32)
    cases = {1: (oblob.write([(oblob.F16, s16)]), s16.astype(np.float32).reshape(H, P, N)),
             2: (oblob.write([(oblob.BF16, sbf)]), sbf),
             3: (oblob.write([(oblob.F32, conv), (oblob.F32, s32)]), s32)}
    for slot, (b, want) in cases.items():
        rec = dict(base, position=100 + slot, chunk_seq=slot, checksum=receipt_checksum(want))
        h.deserialize(slot, b, rec)
        assert h.position(slot) == (100 + slot, slot)
        assert h.state[slot].cpu().numpy().tobytes() == want.tobytes(), slot
    # continuing from the hydrated values matches the oracle started from them
    x, dt, B, C = inputs.tokens(62, 8, H, P, N)
    slots = list(cases)
    st = np.stack([cases[s][1] for s in slots]).astype(np.float64)
    pos = np.zeros(len(slots), np.int64)
    for t in range(8):
        rep = lambda a: np.repeat(a[t:t + 1], len(slots), axis=0)
        yg = h.decode_step(slots, to_dev(rep(x)), to_dev(rep(dt)), to_dev(rep(B)),
                           to_dev(rep(C)))
        yr = oracle.decode(st, pos, np.arange(len(slots)), rep(x), rep(dt), rep(B), rep(C), A, D)
        assert_close(host(yg), yr, **F32_TOL, what=f"decode {t} after hydration")
    assert_close(host(h.state[slots]), st, **F32_TOL, what="state after hydration")
    h.destroy()


def test_serialize_folds_replay_log_and_respects_pending_steps(ssm):
    H, P, N = 2, 64, 128
    say("serialize with replay log", dict(H=H, P=P, N=N))
    h, A, D = _layer(ssm, 63, 2, H, P, N)
    h.replay_attach(16)
    x, dt, B, C = inputs.tokens(63, 5, H, P, N)
    xd, dtd, Bd, Cd = (to_dev(a)[None] for a in (x, dt, B, C))
    h.replay_step([1], xd, dtd, Bd, Cd)
    with pytest.raises(ssm.SSMError) as e:
        h.serialize(1)
    assert e.value.code == ssm.SSM_E_LOG
    with pytest.raises(ssm.SSMError) as e:
        h.deserialize(1, b"", {f: 0 for f, _ in ssm.Receipt._fields_})
    assert e.value.code == ssm.SSM_E_LOG
    h.replay_commit([1], [3])
    blob, rec = h.serialize(1)  # folds the 3 committed log entries first
    assert rec["position"] == 3 and h.log_state(1) == (0, 0)
    snap, rck = h.checkpoint(1)
    assert oblob.read(blob)[0][1].tobytes() == snap.cpu().numpy().tobytes()
    assert rck["checksum"] == rec["checksum"]
    ref = oracle.scan(x[:3], dt[:3], B[:3], C[:3], A, D)["state"]
    assert_close(oblob.read(blob)[0][1], ref, **F32_TOL, what="folded state")
    h.destroy()


def test_rejected_blob_leaves_slot_untouched(ssm):
    H, P, N = 2, 64, 128
    say("blob rejection", dict(H=H, P=P, N=N))
    h, _, _ = _layer(ssm, 64, 2, H, P, N)
    x, dt, B, C = inputs.tokens(64, 6, H, P, N)
    for t in range(6):
        h.decode_step([0, 1], *(to_dev(np.repeat(a[t:t + 1], 2, axis=0)) for a in (x, dt, B, C)))
    blob, rec = h.serialize(0)
    before, pos = h.state[1].clone(), h.position(1)
    flipped = bytearray(blob)
    flipped[100] ^= 0x01  # one payload bit
    for b, r in ((bytes(flipped), rec), (blob, dict(rec, G=2)), (blob[:-1], rec)):
        with pytest.raises(ssm.SSMError) as e:
            h.deserialize(1, b, r)
        assert e.value.code == ssm.SSM_E_SCHEMA
    torch.cuda.synchronize()
    assert torch.equal(before, h.state[1]) and h.position(1) == pos
    assert h.counters()["restores_rejected"] == 3
    h.destroy()


def test_mamba_pair_blob_with_conv_state(ssm):
    """With the conv attached a slot's state is the pair [conv_state, ssm_state]
    (the page's Mamba blob).  A layer step: the conv (SiLU) over the channels
    [x | B | C], then the scan decode on its output.  Serialize after 48 steps,
    hydrate another slot, continue both 48 more: bitwise equal."""
    H, P, N, G, K = 4, 64, 128, 1, 4
    Cc = H * P + 2 * G * N
    say("mamba pair blob", dict(H=H, P=P, N=N, C=Cc, K=K))
    h, A, D = _layer(ssm, 65, 2, H, P, N, schema_version=3, model_rev=5)
    r = np.random.default_rng(65)
    w = to_dev((r.standard_normal((Cc, K)) * 0.5).astype(np.float32))
    b = to_dev((r.standard_normal(Cc) * 0.1).astype(np.float32))
    h.conv_attach(Cc, K, w, b, act=True)
    steps = 96
    xbc = to_dev(r.standard_normal((steps, Cc)).astype(np.float32))
    _, dt, _, _ = inputs.tokens(65, steps, H, P, N)
    dtd = to_dev(dt)

    def layer_step(slots, t):
        n = len(slots)
        u = h.conv_decode(slots, xbc[t:t + 1].expand(n, Cc).contiguous())
        x = u[:, :H * P].reshape(n, H, P).contiguous()
        Bm = u[:, H * P:H * P + G * N].reshape(n, G, N).contiguous()
        Cm = u[:, H * P + G * N:].reshape(n, G, N).contiguous()
        y = h.decode_step(slots, x, dtd[t:t + 1].expand(n, H).contiguous(), Bm, Cm)
        return u, y

    for t in range(48):
        layer_step([0], t)
    blob, rec = h.serialize(0)
    assert len(blob) == h.blob_bytes() == 8 + 16 + Cc * (K - 1) * 4 + 20 + H * P * N * 4
    arrays = oblob.read(blob)
    assert [a.shape for _, a in arrays] == [(Cc, K - 1), (H, P, N)]
    assert arrays[0][1].tobytes() == h.conv_state[0].cpu().numpy().tobytes()
    assert arrays[1][1].tobytes() == h.state[0].cpu().numpy().tobytes()
    # a blob without the conv state is refused by a handle that carries one
    with pytest.raises(ssm.SSMError) as e:
        h.deserialize(1, oblob.write([arrays[1]]), rec)
    assert e.value.code == ssm.SSM_E_SCHEMA
    h.deserialize(1, blob, rec)
    outs = [layer_step([0, 1], t) for t in range(48, steps)]
    torch.cuda.synchronize()
    for u, y in outs:
        assert torch.equal(u[0], u[1]) and torch.equal(y[0], y[1])
    assert torch.equal(h.state[0], h.state[1])
    assert torch.equal(h.conv_state[0], h.conv_state[1])
    h.destroy()
