"""Pins of the state-blob reader/writer against a hand-written byte fixture.

The fixture (``tests/golden/state_blob_v1.txt``) spells out a blob field by
field in the reference serialization of the recurrent-state companion store
("SSM.PREFIX.* -- recurrent-state companion", pion docs), with every value's
IEEE 754 encoding derived by hand.  A swapped field, a wrong byte order, a
wrong element width for any dtype code or a skipped rank would fail here.
"""
import os
import struct

import numpy as np
import pytest

from oracle import blob

GOLD = os.path.join(os.path.dirname(__file__), "golden", "state_blob_v1.txt")


def _fixture():
    raw, expect = bytearray(), []
    for line in open(GOLD):
        line = line.split("#", 1)[0].split()
        if not line:
            continue
        if line[0] == "hex":
            raw += bytes(int(b, 16) for b in line[1:])
        elif line[0] == "expect":
            idx, code = int(line[1]), int(line[2])
            shape = tuple(int(s) for s in line[3].split(","))
            vals = np.array([float(v) for v in line[4:]]).reshape(shape)
            expect.append((idx, code, vals))
    return bytes(raw), expect


def test_reader_decodes_hand_written_blob():
    raw, expect = _fixture()
    arrays = blob.read(raw)
    assert len(arrays) == len(expect) == 3
    for idx, code, vals in expect:
        got_code, got = arrays[idx]
        assert got_code == code
        assert got.shape == vals.shape
        assert np.array_equal(got.astype(np.float64), vals), idx
    assert arrays[1][1].dtype == np.float16
    assert arrays[0][1].dtype == arrays[2][1].dtype == np.float32


def test_writer_reproduces_hand_written_bytes():
    raw, expect = _fixture()
    dtypes = {0: np.float32, 1: np.float16, 2: np.float32}
    arrays = [(code, vals.astype(dtypes[code])) for _, code, vals in expect]
    assert blob.write(arrays) == raw


def test_round_trip_of_mamba_shaped_state():
    # a Mamba blob lists [conv_state, ssm_state]; sizes of one Mamba-130M layer
    rng = np.random.default_rng(7)
    conv = rng.standard_normal((1, 1536 + 2 * 128, 4)).astype(np.float32)
    ssm = rng.standard_normal((24, 64, 128)).astype(np.float32)
    b = blob.write([(blob.F32, conv), (blob.F32, ssm)])
    assert len(b) == 8 + (4 + 12 + 4) + conv.nbytes + (4 + 12 + 4) + ssm.nbytes
    (c0, conv2), (c1, ssm2) = blob.read(b)
    assert c0 == c1 == blob.F32
    assert conv2.tobytes() == conv.tobytes() and ssm2.tobytes() == ssm.tobytes()


def test_fp16_width_and_bf16_widening():
    h = np.array([0.5, -3.0], dtype=np.float16)
    b = blob.write([(blob.F16, h)])
    assert len(b) == 8 + 4 + 4 + 4 + 2 * 2
    # code 2 takes 4 bytes per element and only values bf16 can hold
    w = np.array([1.0, 2.0 ** -7], dtype=np.float32)
    assert len(blob.write([(blob.BF16, w)])) == 8 + 4 + 4 + 4 + 2 * 4
    with pytest.raises(blob.BlobError):
        blob.write([(blob.BF16, np.array([1.0 + 2.0 ** -20], dtype=np.float32))])


@pytest.mark.parametrize("mutate, what", [
    (lambda r: r[:-1], "truncated data"),
    (lambda r: r + b"\0", "trailing byte"),
    (lambda r: struct.pack("<I", 2) + r[4:], "version 2"),
    (lambda r: r[:4] + struct.pack("<I", 0) + r[8:], "no arrays"),
    (lambda r: r[:4] + struct.pack("<I", 4) + r[8:], "array count too high"),
    (lambda r: r[:16] + struct.pack("<I", 7) + r[20:], "shape extent changed"),
    (lambda r: r[:20] + struct.pack("<I", 3) + r[24:], "dtype code 3"),
])
def test_reader_rejects_malformed(mutate, what):
    raw, _ = _fixture()
    with pytest.raises(blob.BlobError):
        blob.read(mutate(raw))
