"""ctypes marshalling for ``liboracle_gdn.so`` (built from ``gdn_oracle.c``):
the Gated DeltaNet recurrence in plain fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).  All arithmetic lives in
the C file; this module converts arrays to contiguous fp64 and back.
"""
import ctypes
import os
import subprocess

import numpy as np

from .core import ORC_OK, OracleError, _f64, _ptr, _threads

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.environ.get("SSM_GDN_ORACLE_LIB") or os.path.join(_HERE, "liboracle_gdn.so")


def lib_path():
    return _LIB


def build():
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
        lib.oracle_gdn_scan.argtypes = [i32, i32, i32, i32, i64, P, P, P, P, P, P, P, P, P, P,
                                        i32]
        lib.oracle_gdn_spec_step.argtypes = [i32, i32, i32, i32, i32, i32, P, i32, P, P, P, P,
                                             P, P, P, P, P, P, i32]
        lib.oracle_gdn_replay_unrolled.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P,
                                                   P, P, P, P]
        for f in (lib.oracle_gdn_scan, lib.oracle_gdn_spec_step, lib.oracle_gdn_replay_unrolled):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def scan(v, dt, beta, k, q, A, state=None, pos=0, reset=None, n_threads=1):
    """Advance one stream by L tokens: v[L,H,P] dt,beta[L,H] k,q[L,G,N] A[H];
    state[H,P,N] carry-in (zeros if None).  Returns dict(o, state, pos)."""
    v = _f64(v)
    L, H, P = v.shape
    k = _f64(k)
    G, N = k.shape[1], k.shape[2]
    q = _f64(q, (L, G, N))
    dt = _f64(dt, (L, H))
    beta = _f64(beta, (L, H))
    A = _f64(A, (H,))
    st = np.zeros((H, P, N)) if state is None else _f64(state, (H, P, N)).copy()
    o = np.zeros((L, H, P))
    rs = None if reset is None else np.ascontiguousarray(np.asarray(reset, dtype=np.uint8))
    p = ctypes.c_int64(int(pos))
    rc = _load().oracle_gdn_scan(H, P, N, G, L, _ptr(v), _ptr(dt), _ptr(beta), _ptr(k), _ptr(q),
                                 _ptr(A), _ptr(rs), _ptr(st), ctypes.byref(p), _ptr(o),
                                 _threads(n_threads))
    if rc != ORC_OK:
        raise OracleError(rc, "gdn_scan")
    return {"o": o, "state": st, "pos": p.value}


def spec_step(state, pos, slot_ids, v, dt, beta, k, q, A, accepted, n_threads=1):
    """Speculative verify with rollback, in place on ``state[S,H,P,N]`` (fp64)
    and ``pos[S]``.  v[b,n_in,H,P] dt,beta[b,n_in,H] k,q[b,n_in,G,N].
    Returns o[b,n_in,H,P]."""
    assert state.dtype == np.float64 and state.flags.c_contiguous
    assert pos.dtype == np.int64 and pos.flags.c_contiguous
    S, H, P, N = state.shape
    slots = np.ascontiguousarray(np.asarray(slot_ids, dtype=np.int32))
    b = len(slots)
    v = _f64(v)
    n_in = v.shape[1]
    v = v.reshape(b, n_in, H, P)
    G = np.asarray(k).shape[-2]
    k = _f64(k, (b, n_in, G, N))
    q = _f64(q, (b, n_in, G, N))
    dt = _f64(dt, (b, n_in, H))
    beta = _f64(beta, (b, n_in, H))
    A = _f64(A, (H,))
    acc = np.ascontiguousarray(np.asarray(accepted, dtype=np.int32))
    o = np.zeros((b, n_in, H, P))
    rc = _load().oracle_gdn_spec_step(S, H, P, N, G, b, _ptr(slots), n_in, _ptr(v), _ptr(dt),
                                      _ptr(beta), _ptr(k), _ptr(q), _ptr(A), _ptr(acc),
                                      _ptr(state), _ptr(pos), _ptr(o), _threads(n_threads))
    if rc != ORC_OK:
        raise OracleError(rc, "gdn_spec_step")
    return o


def replay_unrolled(ckpt, dt_all, beta_all, v_all, k_all, q_all, A, n_log):
    """Test-only replay form of one slot: (o[n_in,H,P], fold[H,P,N])."""
    ckpt = _f64(ckpt)
    H, P, N = ckpt.shape
    v_all = _f64(v_all)
    M = v_all.shape[0]
    G = np.asarray(k_all).shape[1]
    dt_all = _f64(dt_all, (M, H))
    beta_all = _f64(beta_all, (M, H))
    k_all = _f64(k_all, (M, G, N))
    q_all = _f64(q_all, (M, G, N))
    A = _f64(A, (H,))
    n_in = M - n_log
    o = np.zeros((max(n_in, 1), H, P))
    fold = np.zeros((H, P, N))
    rc = _load().oracle_gdn_replay_unrolled(H, P, N, G, n_log, n_in, _ptr(ckpt), _ptr(dt_all),
                                            _ptr(beta_all), _ptr(v_all), _ptr(k_all),
                                            _ptr(q_all), _ptr(A), _ptr(o), _ptr(fold))
    if rc != ORC_OK:
        raise OracleError(rc, "gdn_replay_unrolled")
    return o[:n_in], fold
