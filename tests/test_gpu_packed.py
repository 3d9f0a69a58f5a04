"""Packed prefill into per-sequence slots (ssm_scan_packed) against the fp64
oracle: every sequence's outputs, its final state landing in its own slot
with its exact position, chunk number and a fresh stream id, a copy of each
final state with a receipt that restores the stream, and decode continuing
every slot from there.  A continuing sequence carries its slot's state and
chunk number in; empty sequences are legal."""
import numpy as np
import pytest

import oracle
from streaming_state_amd import inputs
from tests.gpu_helpers import (F32_TOL, assert_close, bf16_dev, bf16_tol, host, receipt_checksum,
                               say, to_dev)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ssm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from streaming_state_amd import ssm as m
    return m


def _io(io, arrays):
    """bf16: round once on the host; both sides use the same bits."""
    if io == "bf16":
        bits = [inputs.bf16_bits(a) for a in arrays]
        return [inputs.bf16_to_f32(b) for b in bits], [bf16_dev(b) for b in bits]
    return list(arrays), [to_dev(a) for a in arrays]


@pytest.mark.parametrize("H,P,N,G,io", [
    (4, 64, 128, 1, "bf16"),   # head-pair MFMA kernel
    (3, 64, 128, 1, "bf16"),   # one-head MFMA kernel (odd head count)
    (3, 40, 20, 1, "f32"),     # recurrent kernel
    (4, 16, 64, 2, "bf16"),    # recurrent kernel, two groups
])
def test_packed_sequences_land_in_their_slots_then_decode(ssm, H, P, N, G, io):
    say("packed into slots", H, P, N, G, io)
    lengths = [137, 0, 1, 300, 64, 65, 29, 203]
    slots = [5, 0, 9, 2, 7, 3, 8, 1]
    cont = [0, 0, 0, 0, 1, 0, 0, 1]     # sequences 4 and 7 continue their slot's stream
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    L, S = int(cu[-1]), 10
    A, D = inputs.params(50, H)
    (x, dt, B, C), dev = _io(io, inputs.tokens(50, L, H, P, N, G))
    tol = (lambda a: bf16_tol(a)) if io == "bf16" else (lambda a: F32_TOL)
    h = ssm.StreamState(H, P, N, S, to_dev(A), to_dev(D), G=G, io_dtype=io)
    r = np.random.default_rng(50)
    st0 = (r.standard_normal((S, H, P, N)) * 0.05).astype(np.float32)
    h.init(np.arange(S), to_dev(st0))
    # slot 1 (sequence 7's) first takes a short chunk of its own: position 5, chunk 1
    (xp, dtp, Bp, Cp), devp = _io(io, inputs.tokens(51, 5, H, P, N, G))
    h.scan_chunk(1, 0, *devp)
    pre = oracle.scan(xp, dtp, Bp, Cp, A, D, state=st0[1])
    stream_before = {}
    for s_ in range(S):
        stream_before[s_] = h.checkpoint(s_)[1]["stream_id"]
    chunk_seq = [0] * 8
    chunk_seq[4] = 0   # slot 7: fresh from init, chunk 0
    chunk_seq[7] = 1   # slot 1: after its own chunk
    y, final, recs = h.scan_packed(cu, slots, *dev, final=True, receipts=True, cont=cont,
                                   chunk_seq=np.array(chunk_seq, np.uint64))
    torch.cuda.synchronize()
    yh = host(y)
    ref_states, ref_pos = [], []
    for i in range(8):
        t0, t1 = cu[i], cu[i + 1]
        if cont[i]:
            init = pre["state"] if slots[i] == 1 else st0[slots[i]]
            pos0 = pre["pos"] if slots[i] == 1 else 0
        else:
            init, pos0 = None, 0
        ref = oracle.scan(x[t0:t1], dt[t0:t1], B[t0:t1], C[t0:t1], A, D, state=init, pos=pos0)
        if t1 > t0:
            assert_close(yh[t0:t1], ref["y"], what=f"y seq {i}", **tol(ref["y"]))
        assert_close(host(h.state[slots[i]]), ref["state"], what=f"slot state seq {i}",
                     **tol(ref["state"]))
        ref_states.append(ref["state"])
        ref_pos.append(ref["pos"])
        # the emitted copy is the slot's state, bit for bit
        assert torch.equal(final[i], h.state[slots[i]]), i
        pos, cs = h.position(slots[i])
        assert pos == ref["pos"] == (pos0 + t1 - t0), i
        assert cs == (chunk_seq[i] + 1 if cont[i] else 1), i
        rc = recs[i]
        assert rc["position"] == pos and rc["chunk_seq"] == cs
        assert rc["checksum"] == receipt_checksum(host(final[i]).astype(np.float32))
        if cont[i]:
            assert rc["stream_id"] == stream_before[slots[i]]
        else:
            assert rc["stream_id"] != stream_before[slots[i]]
    assert len({rc["stream_id"] for rc in recs}) == 8
    # the untouched slots keep their state
    for s_ in (4, 6):
        assert torch.equal(h.state[s_], to_dev(st0[s_]))
    # decode 16 tokens on all eight slots from where each prefill ended
    st = np.stack(ref_states)
    pos = np.array(ref_pos, np.int64)
    for k in range(16):
        (xd, dtd, Bd, Cd), devd = _io(io, inputs.tokens(52, 8, H, P, N, G, k))
        yd = h.decode_step(slots, *devd)
        ry = oracle.decode(st, pos, np.arange(8), xd, dtd, Bd, Cd, A, D)
        torch.cuda.synchronize()
        assert_close(host(yd), ry, what=f"decode {k}", **tol(ry))
    for i in range(8):
        assert h.position(slots[i])[0] == pos[i] == ref_pos[i] + 16
        assert_close(host(h.state[slots[i]]), st[i], what=f"state after decode {i}",
                     **tol(st[i]))
    # a copy and its receipt restore the stream into another slot
    h.restore(6, final[3], recs[3])
    torch.cuda.synchronize()
    assert torch.equal(h.state[6], final[3])
    assert h.position(6) == (recs[3]["position"], recs[3]["chunk_seq"])
    h.destroy()


def test_packed_matches_single_slot_scan(ssm):
    """The same packed batch through ssm_scan_packed and through ssm_scan_chunk
    on one slot with resets at sequence starts: identical outputs and final
    states (the same kernel runs the same segments)."""
    H, P, N, G = 4, 64, 128, 1
    lengths = [190, 77, 1, 400]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    L = int(cu[-1])
    say("packed vs single slot", lengths)
    A, D = inputs.params(53, H)
    _, dev = _io("bf16", inputs.tokens(53, L, H, P, N, G))
    a = ssm.StreamState(H, P, N, 4, to_dev(A), to_dev(D), G=G, io_dtype="bf16")
    b = ssm.StreamState(H, P, N, 1, to_dev(A), to_dev(D), G=G, io_dtype="bf16")
    a.reset(range(4))
    b.reset([0])
    ya, fa, _ = a.scan_packed(cu, [3, 1, 0, 2], *dev, final=True)
    reset = np.zeros(L, np.uint8)
    reset[cu[:-1]] = 1
    yb, cb = b.scan_chunk(0, 0, *dev, reset=reset, ckpt_at=cu[1:] - 1)
    torch.cuda.synchronize()
    assert torch.equal(ya, yb)
    assert torch.equal(fa, cb)
    assert torch.equal(a.state[2], b.state[0])


def test_workload4_packed_into_eight_slots(ssm):
    """The 65,536-token packed prefill (8 sequences, H=128, P=64, N=128, bf16)
    scanned into 8 slots with receipts; the oracle runs 8 sampled heads (both
    heads of three pairs and two more, spread over the head range) over every
    token, and each slot's position equals its sequence length."""
    W = inputs.W4
    L, H, P, N, G = W["L"], W["H"], W["P"], W["N"], W["G"]
    lengths = inputs.sequence_lengths()
    _, cu, ends = inputs.packed_layout(lengths)
    reset = np.zeros(L, np.uint8)
    reset[cu[:-1]] = 1
    say("workload4 packed into slots", lengths.tolist())
    d = inputs.device_prefill(L, H, P, N, G)
    slots = [6, 2, 7, 0, 5, 1, 4, 3]
    h = ssm.StreamState(H, P, N, 8, d["A"], d["D"], G=G, io_dtype="bf16")
    h.reset(range(8))
    y, final, recs = h.scan_packed(cu.astype(np.int32), slots, d["x"], d["dt"], d["B"], d["C"],
                                   final=True, receipts=True)
    torch.cuda.synchronize()
    heads = [0, 1, 40, 41, 86, 87, 100, 127]
    A, D = inputs.params(4, H)
    hs = torch.as_tensor(heads).long().cuda()
    ref = oracle.scan(host(d["x"][:, hs]), host(d["dt"][:, hs]), host(d["B"]), host(d["C"]),
                      A[heads], D[heads], reset=reset, ckpt_at=ends, n_threads=None)
    assert_close(host(y[:, hs]), ref["y"], what="y", **bf16_tol(ref["y"]))
    for i in range(8):
        ck = ref["ckpt"][i]
        assert_close(host(h.state[slots[i]][hs]), ck, what=f"slot state seq {i}", **bf16_tol(ck))
        assert torch.equal(final[i], h.state[slots[i]])
        assert h.position(slots[i]) == (int(lengths[i]), 1)
        assert recs[i]["position"] == int(lengths[i])
        assert recs[i]["checksum"] == receipt_checksum(host(final[i]).astype(np.float32))
    h.destroy()
