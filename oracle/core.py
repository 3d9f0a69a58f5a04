"""ctypes marshalling for ``liboracle.so`` (built from ``ssm_oracle.c``).

TEST INFRASTRUCTURE ONLY (see the package docstring).  All arithmetic lives in
the C file; this module converts arrays to contiguous fp64 and back.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_LIB = os.environ.get("SSM_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

ORC_OK = 0
ORC_E_ARG = -1
ORC_E_INVALID_CHUNK = -2


class OracleError(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"oracle {what} returned {code}")
        self.code = code


def lib_path():
    return _LIB


def build(force=True):
    """Compile the oracle with gcc (plain C, no fast-math, no FMA contraction)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-o", tmp, _SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int, ctypes.c_int64
        lib.oracle_scan.argtypes = [i32, i32, i32, i32, i64, P, P, P, P, P, P, P, P, P, P, P,
                                    i32, P, P, i32]
        lib.oracle_decode.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P,
                                      P, P, P, i32]
        lib.oracle_spec_step.argtypes = [i32, i32, i32, i32, i32, i32, P, i32, P, P, P, P, P,
                                         P, P, P, P, P, i32]
        lib.oracle_replay_unrolled.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P, P,
                                               P, P, P]
        for f in (lib.oracle_scan, lib.oracle_decode, lib.oracle_spec_step,
                  lib.oracle_replay_unrolled):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a, shape=None):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if shape is not None:
        a = a.reshape(shape)
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _threads(n):
    if n is None:
        n = len(os.sched_getaffinity(0))
    return int(max(1, n))


def scan(x, dt, B, C, A, D, state=None, pos=0, reset=None, ckpt_at=None, decay=None,
         n_threads=1):
    """Advance one stream by L tokens.

    x[L,H,P] dt[L,H] B,C[L,G,N] A,D[H]; state[H,P,N] carry-in (zeros if None);
    reset: u8[L] or None; ckpt_at: increasing token indices whose post-token
    state is returned; decay[L,H]: test-only direct a_t.
    Returns dict(y[L,H,P], state[H,P,N], pos, ckpt[n,H,P,N]).  Raises
    OracleError(ORC_E_INVALID_CHUNK) on non-finite input (nothing changed).
    """
    x = _f64(x)
    L, H, P = x.shape
    B = _f64(B)
    G, N = B.shape[1], B.shape[2]
    dt = _f64(dt, (L, H))
    C = _f64(C, (L, G, N))
    B = B.reshape(L, G, N)
    A = _f64(A, (H,))
    D = _f64(D, (H,))
    st = np.zeros((H, P, N)) if state is None else _f64(state, (H, P, N)).copy()
    y = np.zeros((L, H, P))
    rs = None if reset is None else np.ascontiguousarray(np.asarray(reset, dtype=np.uint8))
    if rs is not None and rs.shape != (L,):
        raise ValueError("reset must be u8[L]")
    ck = np.zeros(0, dtype=np.int64) if ckpt_at is None else np.ascontiguousarray(
        np.asarray(ckpt_at, dtype=np.int64))
    ck_out = np.zeros((max(len(ck), 1), H, P, N))
    dc = None if decay is None else _f64(decay, (L, H))
    p = ctypes.c_int64(int(pos))
    rc = _load().oracle_scan(H, P, N, G, L, _ptr(x), _ptr(dt), _ptr(B), _ptr(C), _ptr(A),
                             _ptr(D), _ptr(dc), _ptr(rs), _ptr(st), ctypes.byref(p), _ptr(y),
                             len(ck), _ptr(ck), _ptr(ck_out), _threads(n_threads))
    if rc != ORC_OK:
        raise OracleError(rc, "scan")
    return {"y": y, "state": st, "pos": p.value, "ckpt": ck_out[:len(ck)]}


def decode(state, pos, slot_ids, x, dt, B, C, A, D, reset=None, n_threads=1):
    """One token per slot, in place on ``state[S,H,P,N]`` (fp64) and ``pos[S]`` (int64).

    x[b,H,P] dt[b,H] B,C[b,G,N]; reset u8[b] or None.  Returns y[b,H,P].
    """
    assert state.dtype == np.float64 and state.flags.c_contiguous
    assert pos.dtype == np.int64 and pos.flags.c_contiguous
    S, H, P, N = state.shape
    slots = np.ascontiguousarray(np.asarray(slot_ids, dtype=np.int32))
    b = len(slots)
    x = _f64(x, (b, H, P))
    G = np.asarray(B).shape[-2] if np.asarray(B).ndim == 3 else 1
    B = _f64(B, (b, G, N))
    C = _f64(C, (b, G, N))
    dt = _f64(dt, (b, H))
    A = _f64(A, (H,))
    D = _f64(D, (H,))
    rs = None if reset is None else np.ascontiguousarray(np.asarray(reset, dtype=np.uint8))
    y = np.zeros((b, H, P))
    rc = _load().oracle_decode(S, H, P, N, G, b, _ptr(slots), _ptr(x), _ptr(dt), _ptr(B),
                               _ptr(C), _ptr(A), _ptr(D), _ptr(rs), _ptr(state), _ptr(pos),
                               _ptr(y), _threads(n_threads))
    if rc != ORC_OK:
        raise OracleError(rc, "decode")
    return y


def spec_step(state, pos, slot_ids, x, dt, B, C, A, D, accepted, n_threads=1):
    """Speculative verify with rollback, in place on ``state``/``pos``.

    x[b,n_in,H,P] dt[b,n_in,H] B,C[b,n_in,G,N]; accepted[b] in 1..n_in.
    Returns y[b,n_in,H,P] (outputs of every in-flight token).
    """
    assert state.dtype == np.float64 and state.flags.c_contiguous
    assert pos.dtype == np.int64 and pos.flags.c_contiguous
    S, H, P, N = state.shape
    slots = np.ascontiguousarray(np.asarray(slot_ids, dtype=np.int32))
    b = len(slots)
    x = _f64(x)
    n_in = x.shape[1]
    x = x.reshape(b, n_in, H, P)
    G = np.asarray(B).shape[-2]
    B = _f64(B, (b, n_in, G, N))
    C = _f64(C, (b, n_in, G, N))
    dt = _f64(dt, (b, n_in, H))
    A = _f64(A, (H,))
    D = _f64(D, (H,))
    acc = np.ascontiguousarray(np.asarray(accepted, dtype=np.int32))
    y = np.zeros((b, n_in, H, P))
    rc = _load().oracle_spec_step(S, H, P, N, G, b, _ptr(slots), n_in, _ptr(x), _ptr(dt),
                                  _ptr(B), _ptr(C), _ptr(A), _ptr(D), _ptr(acc), _ptr(state),
                                  _ptr(pos), _ptr(y), _threads(n_threads))
    if rc != ORC_OK:
        raise OracleError(rc, "spec_step")
    return y


def replay_unrolled(ckpt, dt_all, x_all, B_all, C_all, A, D, n_log):
    """Test-only replay form: outputs of the in-flight entries and the folded state.

    ckpt[H,P,N]; dt_all[M,H] x_all[M,H,P] B_all,C_all[M,G,N] with M = n_log + n_in.
    Returns (y[n_in,H,P], fold[H,P,N]).
    """
    ckpt = _f64(ckpt)
    H, P, N = ckpt.shape
    x_all = _f64(x_all)
    M = x_all.shape[0]
    G = np.asarray(B_all).shape[1]
    dt_all = _f64(dt_all, (M, H))
    B_all = _f64(B_all, (M, G, N))
    C_all = _f64(C_all, (M, G, N))
    A = _f64(A, (H,))
    D = _f64(D, (H,))
    n_in = M - n_log
    y = np.zeros((max(n_in, 1), H, P))
    fold = np.zeros((H, P, N))
    rc = _load().oracle_replay_unrolled(H, P, N, G, n_log, n_in, _ptr(ckpt), _ptr(dt_all),
                                        _ptr(x_all), _ptr(B_all), _ptr(C_all), _ptr(A),
                                        _ptr(D), _ptr(y), _ptr(fold))
    if rc != ORC_OK:
        raise OracleError(rc, "replay_unrolled")
    return y[:n_in], fold
