"""State-blob reader and writer (bytes only, no arithmetic on values).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Format: the reference serialization of the recurrent-state companion store on
the page "SSM.PREFIX.* -- recurrent-state companion" (pion docs, command
reference, section on the state blob).  A blob is a little-endian u32 version
(1), a u32 array count, and then for each array: u32 rank, u32 extents, u32
dtype code, raw element bytes.  Dtype codes: 0 fp32, 1 fp16, 2 bf16.

Reading of the page taken here: the remark that bf16 is carried as fp32
belongs to code 2 alone (a bf16 array is widened to fp32 on write, losing
nothing, so it takes 4 bytes per element); an fp16 array keeps its 2-byte
halves.  A Mamba blob lists ``[conv_state, ssm_state]`` in that order.

Arrays are returned and taken as ``(code, ndarray)``; fp16 decodes through
numpy's IEEE binary16 type.  Any malformation raises ``BlobError``.
"""
import struct

import numpy as np

VERSION = 1
F32, F16, BF16 = 0, 1, 2
_ITEM = {F32: ("<f4", 4), F16: ("<f2", 2), BF16: ("<f4", 4)}


class BlobError(ValueError):
    pass


def write(arrays):
    """arrays: list of (code, ndarray) -> bytes.  For code 2 the array's values
    must be bf16 numbers (fp32 words whose low 16 bits are zero)."""
    out = [struct.pack("<II", VERSION, len(arrays))]
    for code, a in arrays:
        if code not in _ITEM:
            raise BlobError(f"unknown dtype code {code}")
        a = np.asarray(a)
        out.append(struct.pack("<I", a.ndim))
        out.append(struct.pack(f"<{a.ndim}I", *a.shape))
        out.append(struct.pack("<I", code))
        payload = np.ascontiguousarray(a, dtype=_ITEM[code][0])
        if code == BF16 and np.any(payload.view("<u4") & 0xFFFF):
            raise BlobError("code 2 array holds values that are not bf16")
        out.append(payload.tobytes())
    return b"".join(out)


def read(blob):
    """bytes -> list of (code, ndarray); fp16 stays float16, codes 0 and 2 are
    float32."""
    blob = bytes(blob)
    at = 0

    def take(n):
        nonlocal at
        if at + n > len(blob):
            raise BlobError("truncated")
        piece = blob[at:at + n]
        at += n
        return piece

    version, n_arrays = struct.unpack("<II", take(8))
    if version != VERSION:
        raise BlobError(f"version {version}")
    if n_arrays == 0:
        raise BlobError("no arrays")
    arrays = []
    for _ in range(n_arrays):
        (rank,) = struct.unpack("<I", take(4))
        shape = struct.unpack(f"<{rank}I", take(4 * rank))
        (code,) = struct.unpack("<I", take(4))
        if code not in _ITEM:
            raise BlobError(f"unknown dtype code {code}")
        dtype, size = _ITEM[code]
        count = int(np.prod(shape, dtype=np.int64)) if rank else 1
        a = np.frombuffer(take(count * size), dtype=dtype).reshape(shape)
        if code == BF16 and np.any(a.view("<u4") & 0xFFFF):
            raise BlobError("code 2 array holds values that are not bf16")
        arrays.append((code, a.copy()))
    if at != len(blob):
        raise BlobError("trailing bytes")
    return arrays
