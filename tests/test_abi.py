"""C ABI checks that need no GPU: the library loads, exports every entry point
the header declares, and rejects bad calls on the host before any device work
(sequence numbers, slot ids, lifecycle misuse, incompatible receipts).

Pointers passed here are never dereferenced: every call below fails (or, for
an empty chunk, succeeds) before anything is enqueued.
"""
import ctypes
import re

import numpy as np
import pytest

from tests.gpu_helpers import receipt_checksum

ssm = pytest.importorskip("streaming_state_amd.ssm",
                          reason="libssm_stream.so not built (python -m streaming_state_amd.build)")

FAKE = ctypes.c_void_p(0x1000)  # a non-null device pointer that is never used


def declared_functions():
    text = open(ssm.HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = declared_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(ssm.lib(), n), f"{n} declared in ssm_stream.h but not exported"


def _desc(H=4, P=8, N=16, G=1, io=ssm.SSM_F32):
    return ssm.LayerDesc(H, P, N, G, io, 3, 77)


def _create(S=4, desc=None, flags=0):
    d = desc or _desc()
    h = ctypes.c_int64(0)
    rc = ssm.lib().ssm_create(ctypes.byref(d), S, FAKE, FAKE, FAKE, flags, ctypes.byref(h))
    return rc, h.value


def _err():
    return ssm.lib().ssm_last_error().decode()


def test_create_validates_layer():
    for bad in (_desc(N=6), _desc(N=256), _desc(H=6, G=4), _desc(io=ssm.SSM_F16), _desc(P=0)):
        rc, _ = _create(desc=bad)
        assert rc == ssm.SSM_E_INVALID_ARG
    rc, h = _create()
    assert rc == ssm.SSM_OK and h > 0
    assert ssm.lib().ssm_destroy(h) == ssm.SSM_OK


def test_destroyed_handle_is_invalid_and_ids_not_reused():
    rc, h = _create()
    assert ssm.lib().ssm_destroy(h) == ssm.SSM_OK
    assert ssm.lib().ssm_destroy(h) == ssm.SSM_E_INVALID_STATE
    pos = ctypes.c_int64(0)
    assert ssm.lib().ssm_get_position(h, 0, ctypes.byref(pos), None) == ssm.SSM_E_INVALID_STATE
    rc, h2 = _create()
    assert h2 != h
    ssm.lib().ssm_destroy(h2)


def _scan(h, slot, seq, L, reset=None, ckpt=None, ws=None):
    rs = None if reset is None else (ctypes.c_uint8 * len(reset))(*reset)
    ck = None if ckpt is None else (ctypes.c_int64 * len(ckpt))(*ckpt)
    return ssm.lib().ssm_scan_chunk(h, slot, seq, L, FAKE, FAKE, FAKE, FAKE, rs, FAKE,
                                    0 if ckpt is None else len(ckpt), ck,
                                    FAKE if ckpt else None, ws, 0, None)


def test_chunk_sequence_rules():
    rc, h = _create()
    lib = ssm.lib()
    # an empty chunk is admitted and only advances the sequence number
    assert _scan(h, 1, 0, 0) == ssm.SSM_OK
    pos, seq = ctypes.c_int64(-1), ctypes.c_uint64(0)
    lib.ssm_get_position(h, 1, ctypes.byref(pos), ctypes.byref(seq))
    assert (pos.value, seq.value) == (0, 1)
    # duplicate and reordered chunks are rejected with nothing changed
    assert _scan(h, 1, 0, 5) == ssm.SSM_E_SEQUENCE
    assert "duplicate" in _err()
    assert _scan(h, 1, 2, 5) == ssm.SSM_E_SEQUENCE
    assert _scan(h, 1, 7, 0) == ssm.SSM_E_SEQUENCE
    lib.ssm_get_position(h, 1, ctypes.byref(pos), ctypes.byref(seq))
    assert (pos.value, seq.value) == (0, 1)
    c = ssm.Counters()
    lib.ssm_get_counters(h, ctypes.byref(c))
    assert c.chunks_admitted == 1 and c.chunks_rejected == 3
    lib.ssm_destroy(h)


def test_scan_argument_checks():
    rc, h = _create()
    assert _scan(h, 9, 0, 4) == ssm.SSM_E_INVALID_ARG             # slot out of range
    assert _scan(h, 0, 0, -1) == ssm.SSM_E_INVALID_ARG            # negative length
    assert _scan(h, 0, 0, 4, ckpt=[2, 2]) == ssm.SSM_E_INVALID_ARG  # not increasing
    assert _scan(h, 0, 0, 4, ckpt=[4]) == ssm.SSM_E_INVALID_ARG     # outside [0, L)
    # carries state in and resets later: needs the workspace
    assert _scan(h, 0, 0, 4, reset=[0, 0, 1, 0]) == ssm.SSM_E_INVALID_ARG
    assert "workspace" in _err()
    ssm.lib().ssm_destroy(h)


def test_batch_slot_checks():
    rc, h = _create(S=4)
    lib = ssm.lib()
    ids = (ctypes.c_int32 * 3)(0, 2, 0)
    assert lib.ssm_decode_step(h, 3, ids, FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == \
        ssm.SSM_E_INVALID_ARG
    assert "repeated" in _err()
    ids = (ctypes.c_int32 * 2)(0, 4)
    assert lib.ssm_decode_step(h, 2, ids, FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == \
        ssm.SSM_E_INVALID_ARG
    assert lib.ssm_state_reset(h, 2, ids, None) == ssm.SSM_E_INVALID_ARG
    lib.ssm_destroy(h)


def test_replay_and_copy_bookkeeping_misuse():
    rc, h = _create(S=4)
    lib = ssm.lib()
    ids = (ctypes.c_int32 * 1)(1)
    acc = (ctypes.c_int32 * 1)(1)
    # no log attached / nothing to commit
    assert lib.ssm_replay_step(h, 1, ids, 2, FAKE, FAKE, FAKE, FAKE, FAKE, None) == ssm.SSM_E_LOG
    assert lib.ssm_replay_commit(h, 1, ids, acc) == ssm.SSM_E_LOG
    assert lib.ssm_copy_commit(h, 1, ids, acc) == ssm.SSM_E_LOG
    d = _desc()
    nb = lib.ssm_replay_log_bytes(ctypes.byref(d), 4, 8)
    assert nb > 0
    assert lib.ssm_replay_log_bytes(ctypes.byref(d), 4, 65) == 0  # window above the limit
    assert lib.ssm_replay_attach(h, 8, FAKE, nb - 1) == ssm.SSM_E_INVALID_ARG
    assert lib.ssm_replay_attach(h, 8, FAKE, nb) == ssm.SSM_OK
    assert lib.ssm_replay_step(h, 1, ids, 9, FAKE, FAKE, FAKE, FAKE, FAKE, None) == \
        ssm.SSM_E_INVALID_ARG  # n_in above W
    assert lib.ssm_copy_step(h, 1, ids, 2, FAKE, FAKE, FAKE, FAKE, FAKE, None) == ssm.SSM_E_LOG
    lib.ssm_destroy(h)


def test_restore_rejects_incompatible_receipts():
    rc, h = _create(desc=_desc())
    lib = ssm.lib()
    good = dict(stream_id=5, model_rev=77, code_rev=ssm.code_rev(), schema_version=3,
                state_dtype=0, H=4, P=8, N=16, G=1, position=10, chunk_seq=2, checksum=0)
    for field, value in (("schema_version", 4), ("model_rev", 78), ("code_rev", 999),
                         ("N", 32), ("H", 2), ("state_dtype", 2)):
        r = ssm.Receipt.from_dict(dict(good, **{field: value}))
        assert lib.ssm_state_restore(h, 0, FAKE, ctypes.byref(r), None) == ssm.SSM_E_SCHEMA, field
    c = ssm.Counters()
    lib.ssm_get_counters(h, ctypes.byref(c))
    assert c.restores_rejected == 6
    lib.ssm_destroy(h)


def test_size_queries():
    lib = ssm.lib()
    d = _desc(H=128, P=64, N=128)
    state = 128 * 64 * 128 * 4
    # fp32 io at P=64, N=128: the tile-parallel form needs one state per
    # 64-token tile (at most 64 tiles at a time) plus 64 decays per head
    ws = lib.ssm_scan_workspace_bytes
    assert ws(ctypes.byref(d), 1) == state
    assert ws(ctypes.byref(d), 2048) == 32 * state + 64 * 128 * 4
    assert ws(ctypes.byref(d), 65536) == 64 * state + 64 * 128 * 4
    assert ws(ctypes.byref(d), -1) == 0
    # bf16 at P=64, N=128 takes the SSD form; P=4 only the recurrent form
    assert ws(ctypes.byref(_desc(H=128, P=64, N=128, io=ssm.SSM_BF16)), 65536) == state
    assert ws(ctypes.byref(_desc(H=2, P=4, N=8)), 4096) == 2 * 4 * 8 * 4
    assert lib.ssm_copy_buffer_bytes(ctypes.byref(d), 256, 5) == 256 * 5 * 4 * 1024 * 1024
    # the log holds two halves of W entries of dt[H], x[H,P], B[G,N] per slot
    entry = (128 + 128 * 64 + 128) * 4
    assert lib.ssm_replay_log_bytes(ctypes.byref(d), 256, 16) >= 256 * 2 * 16 * entry


def test_blob_size_and_serialize_argument_checks():
    lib = ssm.lib()
    d = _desc(H=4, P=8, N=16)
    assert lib.ssm_blob_bytes(ctypes.byref(d)) == 28 + 4 * 8 * 16 * 4
    assert lib.ssm_blob_bytes(ctypes.byref(_desc(N=6))) == 0
    rc, h = _create(desc=d)
    n, r = ctypes.c_size_t(0), ssm.Receipt()
    buf = ctypes.create_string_buffer(64)
    assert lib.ssm_state_serialize(h, 0, buf, 64, ctypes.byref(n), ctypes.byref(r),
                                   None) == ssm.SSM_E_INVALID_ARG
    assert "capacity" in _err()
    assert lib.ssm_state_serialize(h, 9, buf, 64, ctypes.byref(n), ctypes.byref(r),
                                   None) == ssm.SSM_E_INVALID_ARG
    lib.ssm_destroy(h)


def test_deserialize_rejects_before_any_device_work():
    """Every rejection below happens on the host; the slot and counters show it."""
    from oracle import blob
    lib = ssm.lib()
    d = _desc(H=4, P=8, N=16)
    rc, h = _create(desc=d)
    state = np.arange(4 * 8 * 16, dtype=np.float32).reshape(4, 8, 16) / 64
    good_r = dict(stream_id=5, model_rev=77, code_rev=ssm.code_rev(), schema_version=3,
                  state_dtype=0, H=4, P=8, N=16, G=1, position=10, chunk_seq=2,
                  checksum=receipt_checksum(state))
    conv = np.zeros((1, 8, 4), np.float32)
    ok = blob.write([(0, state)])
    off = state + np.float32(2.0 ** -20)  # not bf16 numbers
    off_b = blob.write([(0, off)])
    cases = [
        ("receipt model revision", ok, dict(good_r, model_rev=1)),
        ("checksum mismatch", ok, dict(good_r, checksum=1)),
        ("not [H, P, N]", blob.write([(0, state.reshape(4, 16, 8))]), good_r),
        ("not [H, P, N]", blob.write([(0, state.reshape(32, 16))]), good_r),
        ("not [H, P, N]", blob.write([(0, np.stack([state, state]))]), good_r),
        ("not [H, P, N]", blob.write([(0, state), (0, conv)]), good_r),
        ("truncated", ok[:-4], good_r),
        ("trailing bytes", ok + b"\0\0\0\0", good_r),
        ("version", b"\x02\0\0\0" + ok[4:], good_r),
        ("unknown dtype code", ok[:24] + b"\x05\0\0\0" + ok[28:], good_r),
        ("bf16 cannot represent", off_b[:24] + b"\x02\0\0\0" + off_b[28:],
         dict(good_r, checksum=receipt_checksum(off))),
        ("shorter than its header", b"", good_r),
    ]
    for what, b, rd in cases:
        r = ssm.Receipt.from_dict(rd)
        assert lib.ssm_state_deserialize(h, 1, b, len(b), ctypes.byref(r),
                                         None) == ssm.SSM_E_SCHEMA, what
        assert what in _err(), (what, _err())
    c = ssm.Counters()
    lib.ssm_get_counters(h, ctypes.byref(c))
    assert c.restores_rejected == len(cases) and c.restores == 0
    pos, seq = ctypes.c_int64(-1), ctypes.c_uint64(9)
    lib.ssm_get_position(h, 1, ctypes.byref(pos), ctypes.byref(seq))
    assert pos.value == 0 and seq.value == 0
    r = ssm.Receipt.from_dict(good_r)
    assert lib.ssm_state_deserialize(h, 1, None, 0, ctypes.byref(r),
                                     None) == ssm.SSM_E_INVALID_ARG
    lib.ssm_destroy(h)


def test_conv_and_gate_argument_checks():
    lib = ssm.lib()
    assert lib.ssm_conv_state_bytes(4, 10, 4) == 4 * 10 * 3 * 4
    assert lib.ssm_conv_state_bytes(4, 10, 5) == 0 and lib.ssm_conv_state_bytes(4, 0, 4) == 0
    rc, h = _create(desc=_desc())
    # no conv attached yet
    assert lib.ssm_conv_chunk(h, 0, 8, FAKE, None, FAKE, None) == ssm.SSM_E_INVALID_STATE
    assert lib.ssm_conv_decode(h, 1, (ctypes.c_int32 * 1)(0), FAKE, None, FAKE,
                               None) == ssm.SSM_E_INVALID_STATE
    for C, K, act in ((0, 4, 1), (8, 0, 1), (8, 5, 1), (8, 4, 2)):
        assert lib.ssm_conv_attach(h, C, K, act, FAKE, FAKE, None) == ssm.SSM_E_INVALID_ARG
    assert lib.ssm_conv_attach(h, 8, 4, 1, None, FAKE, None) == ssm.SSM_E_INVALID_ARG  # no state
    assert lib.ssm_conv_attach(h, 8, 4, 1, FAKE, FAKE, None) == ssm.SSM_OK
    assert lib.ssm_conv_chunk(h, 9, 8, FAKE, None, FAKE, None) == ssm.SSM_E_INVALID_ARG
    assert lib.ssm_conv_chunk(h, 0, -1, FAKE, None, FAKE, None) == ssm.SSM_E_INVALID_ARG
    assert lib.ssm_conv_chunk(h, 0, 0, None, None, None, None) == ssm.SSM_OK  # empty chunk
    # y overlapping x is refused (the window reads inputs other threads overwrite)
    x = ctypes.c_void_p(0x10000)
    y = ctypes.c_void_p(0x10000 + 4 * 8 * 3)
    assert lib.ssm_conv_chunk(h, 0, 8, x, None, y, None) == ssm.SSM_E_INVALID_ARG
    assert "overlap" in _err()
    dup = (ctypes.c_int32 * 2)(1, 1)
    assert lib.ssm_conv_decode(h, 2, dup, FAKE, None, FAKE, None) == ssm.SSM_E_INVALID_ARG
    lib.ssm_destroy(h)
    gate = lib.ssm_gate
    assert gate(ssm.SSM_F16, 4, 8, 8, FAKE, FAKE, None, 0.0, FAKE, None) == ssm.SSM_E_INVALID_ARG
    assert gate(ssm.SSM_F32, 4, 8, 3, FAKE, FAKE, FAKE, 1e-6, FAKE, None) == ssm.SSM_E_INVALID_ARG
    assert gate(ssm.SSM_F32, 4, 8, 4, FAKE, FAKE, FAKE, -1.0, FAKE, None) == ssm.SSM_E_INVALID_ARG
    assert gate(ssm.SSM_F32, 0, 8, 8, None, None, None, 0.0, None, None) == ssm.SSM_OK


def _packed(h, cu, slots, cont=None, seqs=None, receipts=None):
    lib = ssm.lib()
    n = len(slots)
    cu_ = (ctypes.c_int32 * len(cu))(*cu)
    sl_ = (ctypes.c_int32 * max(n, 1))(*slots)
    ct_ = None if cont is None else (ctypes.c_uint8 * n)(*cont)
    sq_ = None if seqs is None else (ctypes.c_uint64 * n)(*seqs)
    return lib.ssm_scan_packed(h, n, cu_, sl_, ct_, sq_, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                               receipts, None)


def test_scan_packed_rejects_on_the_host():
    """Packed sequences into their own slots: malformed cu_seqlens, repeated or
    out-of-range slots, a continuing sequence whose chunk number is stale or
    ahead, and a continuation without chunk numbers are refused with every
    slot unchanged."""
    lib = ssm.lib()
    rc, h = _create(S=4)
    pos, seq = ctypes.c_int64(-1), ctypes.c_uint64(9)

    def meta(slot):
        lib.ssm_get_position(h, slot, ctypes.byref(pos), ctypes.byref(seq))
        return pos.value, seq.value

    assert lib.ssm_scan_packed(h, -1, None, None, None, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                               None, None, None) == ssm.SSM_E_INVALID_ARG
    assert lib.ssm_scan_packed(h, 0, None, None, None, None, None, None, None, None, None,
                               None, None, None) == ssm.SSM_OK  # nothing to do
    assert _packed(h, [1, 4, 9], [0, 1]) == ssm.SSM_E_INVALID_ARG  # cu[0] != 0
    assert _packed(h, [0, 5, 3], [0, 1]) == ssm.SSM_E_INVALID_ARG  # decreasing
    assert "decreases" in _err()
    assert _packed(h, [0, 3, 6], [2, 2]) == ssm.SSM_E_INVALID_ARG  # repeated slot
    assert "repeated" in _err()
    assert _packed(h, [0, 3, 6], [0, 4]) == ssm.SSM_E_INVALID_ARG  # out of range
    assert _packed(h, [0, 3, 6], [0, 1], cont=[0, 1]) == ssm.SSM_E_INVALID_ARG  # no chunk seqs
    assert _packed(h, [0, 3, 6], [0, 1], cont=[0, 1], seqs=[0, 1]) == ssm.SSM_E_SEQUENCE
    assert "reordered" in _err()
    # empty sequences only: admitted on the host with no device work (a fresh
    # empty sequence zeroes its slot on the device, so use continuations)
    assert _packed(h, [0, 0, 0], [0, 1], cont=[1, 1], seqs=[0, 0]) == ssm.SSM_OK
    assert meta(0) == (0, 1) and meta(1) == (0, 1)
    assert _packed(h, [0, 0], [1], cont=[1], seqs=[0]) == ssm.SSM_E_SEQUENCE  # duplicate
    assert "duplicate" in _err()
    c = ssm.Counters()
    lib.ssm_get_counters(h, ctypes.byref(c))
    assert c.chunks_admitted == 2 and c.chunks_rejected == 2
    for s_ in range(4):
        assert meta(s_)[0] == 0
    lib.ssm_destroy(h)


def test_recurrence_guards_on_the_host():
    """Gated DeltaNet handles: D may be NULL (Mamba-2 needs it); each
    recurrence's calls refuse the other's handles; a receipt of the other
    recurrence is refused; an unknown recurrence is refused."""
    lib = ssm.lib()
    g = _desc(H=4, P=8, N=16)
    g.recurrence = ssm.SSM_GATED_DELTA
    h = ctypes.c_int64(0)
    assert lib.ssm_create(ctypes.byref(g), 2, FAKE, FAKE, None, 0, ctypes.byref(h)) == ssm.SSM_OK
    hm = ctypes.c_int64(0)
    assert lib.ssm_create(ctypes.byref(_desc()), 2, FAKE, FAKE, None, 0,
                          ctypes.byref(hm)) == ssm.SSM_E_INVALID_ARG
    rc, hm = _create()
    bad = _desc()
    bad.recurrence = 7
    assert lib.ssm_create(ctypes.byref(bad), 2, FAKE, FAKE, FAKE, 0,
                          ctypes.byref(ctypes.c_int64(0))) == ssm.SSM_E_INVALID_ARG
    ids = (ctypes.c_int32 * 1)(0)
    assert lib.ssm_decode_step(h.value, 1, ids, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                               None) == ssm.SSM_E_INVALID_ARG
    assert "Gated DeltaNet" in _err()
    assert _scan(h.value, 0, 0, 4) == ssm.SSM_E_INVALID_ARG
    assert lib.ssm_gdn_replay_step(hm, 1, ids, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   None) == ssm.SSM_E_INVALID_ARG
    assert lib.ssm_gdn_copy_step(hm, 1, ids, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 None) == ssm.SSM_E_INVALID_ARG
    assert "Mamba-2" in _err()
    # a Gated DeltaNet log holds beta too
    assert lib.ssm_replay_log_bytes(ctypes.byref(g), 4, 8) != \
        lib.ssm_replay_log_bytes(ctypes.byref(_desc(H=4, P=8, N=16)), 4, 8)
    good = dict(stream_id=5, model_rev=77, code_rev=ssm.code_rev(), schema_version=3,
                state_dtype=0, H=4, P=8, N=16, G=1, position=10, chunk_seq=2, checksum=0,
                recurrence=ssm.SSM_MAMBA2)
    r = ssm.Receipt.from_dict(good)
    assert lib.ssm_state_restore(h.value, 0, FAKE, ctypes.byref(r), None) == ssm.SSM_E_SCHEMA
    assert "recurrence" in _err()
    lib.ssm_destroy(h.value)
    lib.ssm_destroy(hm)
