"""Python binding of ``libssm_stream.so`` (the C ABI in ``include/ssm_stream.h``).

Argument marshalling only: every step of every path runs in the library's HIP
kernels.  Device buffers are torch tensors (PyTorch supplies device memory and
the current stream); host metadata (slot ids, reset flags, accepted counts,
checkpoint token indices) is passed as host arrays.  Importing this module
raises ImportError when the library has not been built; there is no fallback.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssm_stream.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "ssm_stream.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m streaming_state_amd.build`")

# torch must be loaded first: the library then binds to the HIP runtime torch
# already mapped (same soname), so device pointers and streams from torch are
# valid inside it.  Loading it first would map a second runtime.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes():
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for ln in f:
                if "libamdhip64" in ln:
                    paths.add(os.path.realpath(ln.split()[-1]))
    except OSError:
        pass
    return paths


if len(_hip_runtimes()) > 1:
    raise ImportError(f"two HIP runtimes are mapped ({sorted(_hip_runtimes())}); import torch "
                      "before loading libssm_stream.so")

SSM_OK = 0
SSM_E_INVALID_ARG = -1
SSM_E_INVALID_CHUNK = -2
SSM_E_INVALID_STATE = -3
SSM_E_SEQUENCE = -4
SSM_E_SCHEMA = -5
SSM_E_LOG = -6
SSM_E_HIP = -7
SSM_F32, SSM_F16, SSM_BF16 = 0, 1, 2
SSM_MAMBA2, SSM_GATED_DELTA = 0, 1
SSM_FLAG_CHECK_FINITE = 1
SSM_STATIC_WORKSPACE_BYTES = 16 << 20

_NAMES = {0: "SSM_OK", -1: "SSM_E_INVALID_ARG", -2: "SSM_E_INVALID_CHUNK",
          -3: "SSM_E_INVALID_STATE", -4: "SSM_E_SEQUENCE", -5: "SSM_E_SCHEMA", -6: "SSM_E_LOG",
          -7: "SSM_E_HIP"}


class LayerDesc(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("P", ctypes.c_int32), ("N", ctypes.c_int32),
                ("G", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
                ("schema_version", ctypes.c_uint32), ("model_rev", ctypes.c_uint64),
                ("recurrence", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class Receipt(ctypes.Structure):
    _fields_ = [("stream_id", ctypes.c_uint64), ("model_rev", ctypes.c_uint64),
                ("code_rev", ctypes.c_uint64), ("schema_version", ctypes.c_uint32),
                ("state_dtype", ctypes.c_uint32), ("H", ctypes.c_int32), ("P", ctypes.c_int32),
                ("N", ctypes.c_int32), ("G", ctypes.c_int32), ("position", ctypes.c_int64),
                ("chunk_seq", ctypes.c_uint64), ("checksum", ctypes.c_uint64),
                ("recurrence", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_ if f != "reserved"}

    @classmethod
    def from_dict(cls, d):
        """Fields missing from d (recurrence, reserved) are 0."""
        r = cls()
        for f, _ in cls._fields_:
            setattr(r, f, d.get(f, 0))
        return r


class Counters(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "chunks_admitted", "chunks_rejected", "tokens_scanned", "decode_tokens", "resets",
        "replay_steps", "replay_flushes", "replay_tokens_committed", "copy_steps", "checkpoints",
        "restores", "restores_rejected", "state_bytes_read", "state_bytes_written")]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


_V = ctypes.c_void_p
_I32, _I64, _U32, _U64, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64, \
    ctypes.c_size_t
_H = ctypes.c_int64
_SIGS = {
    "ssm_create": [ctypes.POINTER(LayerDesc), _I32, _V, _V, _V, _U32, ctypes.POINTER(_H)],
    "ssm_destroy": [_H],
    "ssm_state_reset": [_H, _I32, _V, _V],
    "ssm_state_init": [_H, _I32, _V, _V, _V],
    "ssm_scan_workspace_bytes": [ctypes.POINTER(LayerDesc), _I64],
    "ssm_scan_chunk": [_H, _I32, _U64, _I64, _V, _V, _V, _V, _V, _V, _I32, _V, _V, _V, _SZ, _V],
    "ssm_scan_chunk_static": [_H, _I32, _U64, _I64, _V, _V, _V, _V, _V, _V, _I32, _V, _V, _V],
    "ssm_scan_packed": [_H, _I32, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V,
                        ctypes.POINTER(Receipt), _V],
    "ssm_decode_step": [_H, _I32, _V, _V, _V, _V, _V, _V, _V, _V],
    "ssm_replay_log_bytes": [ctypes.POINTER(LayerDesc), _I32, _I32],
    "ssm_replay_attach": [_H, _I32, _V, _SZ],
    "ssm_replay_step": [_H, _I32, _V, _I32, _V, _V, _V, _V, _V, _V],
    "ssm_replay_commit": [_H, _I32, _V, _V],
    "ssm_gdn_replay_step": [_H, _I32, _V, _I32, _V, _V, _V, _V, _V, _V, _V],
    "ssm_gdn_copy_step": [_H, _I32, _V, _I32, _V, _V, _V, _V, _V, _V, _V],
    "ssm_copy_buffer_bytes": [ctypes.POINTER(LayerDesc), _I32, _I32],
    "ssm_copy_attach": [_H, _I32, _V, _SZ],
    "ssm_copy_step": [_H, _I32, _V, _I32, _V, _V, _V, _V, _V, _V],
    "ssm_copy_commit": [_H, _I32, _V, _V],
    "ssm_state_materialize": [_H, _I32, _V, _V],
    "ssm_state_checkpoint": [_H, _I32, _V, ctypes.POINTER(Receipt), _V],
    "ssm_state_restore": [_H, _I32, _V, ctypes.POINTER(Receipt), _V],
    "ssm_blob_bytes": [ctypes.POINTER(LayerDesc)],
    "ssm_state_blob_bytes": [_H],
    "ssm_state_serialize": [_H, _I32, _V, _SZ, ctypes.POINTER(_SZ), ctypes.POINTER(Receipt), _V],
    "ssm_state_deserialize": [_H, _I32, _V, _SZ, ctypes.POINTER(Receipt), _V],
    "ssm_conv_state_bytes": [_I32, _I32, _I32],
    "ssm_conv_attach": [_H, _I32, _I32, _I32, _V, _V, _V],
    "ssm_conv_chunk": [_H, _I32, _I64, _V, _V, _V, _V],
    "ssm_conv_decode": [_H, _I32, _V, _V, _V, _V, _V],
    "ssm_gate": [_I32, _I64, _I32, _I32, _V, _V, _V, ctypes.c_float, _V, _V],
    "ssm_get_position": [_H, _I32, ctypes.POINTER(_I64), ctypes.POINTER(_U64)],
    "ssm_get_log_state": [_H, _I32, ctypes.POINTER(_I32), ctypes.POINTER(_I32)],
    "ssm_get_counters": [_H, ctypes.POINTER(Counters)],
    "ssm_last_error": [],
    "ssm_code_rev": [],
}
for _name, _args in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    if _name.endswith("_bytes"):
        _f.restype = ctypes.c_size_t
    elif _name == "ssm_last_error":
        _f.restype = ctypes.c_char_p
    elif _name == "ssm_code_rev":
        _f.restype = ctypes.c_uint64
    else:
        _f.restype = ctypes.c_int


def lib():
    return _lib


class SSMError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{_NAMES.get(code, code)}: {msg}")
        self.code = code


def _check(rc):
    if rc != SSM_OK:
        raise SSMError(rc, _lib.ssm_last_error().decode(errors="replace"))


def code_rev():
    return int(_lib.ssm_code_rev())


# ------------------------------------------------------------ marshalling
def _torch():
    import torch
    return torch


def _io_torch_dtype(io):
    torch = _torch()
    return torch.bfloat16 if io == SSM_BF16 else torch.float32


def _dev_ptr(t, dtype=None, shape=None, name="tensor"):
    """Device pointer of a contiguous CUDA/HIP tensor (None passes NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _host(a, dtype):
    if a is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(a, dtype=dtype))
    return arr, arr.ctypes.data_as(ctypes.c_void_p)


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def conv_state_bytes(n_slots, C, K):
    return int(_lib.ssm_conv_state_bytes(n_slots, C, K))


def gate(y, z, norm_w=None, group=None, eps=1e-6, out=None, stream=None):
    """out = y * SiLU(z) over [rows, C] (fp32 or bf16 device tensors); with
    norm_w [C] fp32, each group of `group` channels is RMS-normalised."""
    torch = _torch()
    if y.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("gate: y must be float32 or bfloat16")
    io = SSM_BF16 if y.dtype == torch.bfloat16 else SSM_F32
    rows, C = y.shape
    group = C if group is None else group
    if out is None:
        out = torch.empty_like(y)
    _check(_lib.ssm_gate(io, rows, C, group, _dev_ptr(y, y.dtype, (rows, C), "y"),
                         _dev_ptr(z, y.dtype, (rows, C), "z"),
                         None if norm_w is None else _dev_ptr(norm_w, torch.float32, (C,), "norm_w"),
                         float(eps), _dev_ptr(out, y.dtype, (rows, C), "out"), _stream(stream)))
    return out


class StreamState:
    """Handle over ``n_slots`` stream slots whose fp32 state is a torch tensor
    ``state[n_slots, H, P, N]`` on the device.  ``A`` and ``D`` are fp32 [H]
    device tensors that must outlive the handle."""

    def __init__(self, H, P, N, n_slots, A, D, G=1, io_dtype="f32", state=None,
                 check_finite=False, schema_version=1, model_rev=0, recurrence="mamba2"):
        torch = _torch()
        self.io = {"f32": SSM_F32, "fp32": SSM_F32, "bf16": SSM_BF16}[io_dtype]
        self.io_dtype = _io_torch_dtype(self.io)
        self.H, self.P, self.N, self.G, self.S = H, P, N, G, n_slots
        self.rec = {"mamba2": SSM_MAMBA2, "gated_delta": SSM_GATED_DELTA}[recurrence]
        self.desc = LayerDesc(H, P, N, G, self.io, schema_version, model_rev, self.rec, 0)
        if state is None:
            state = torch.zeros((n_slots, H, P, N), dtype=torch.float32, device="cuda")
        self.state = state
        self.A, self.D = A, D
        h = _H(0)
        flags = SSM_FLAG_CHECK_FINITE if check_finite else 0
        _check(_lib.ssm_create(ctypes.byref(self.desc), n_slots,
                               _dev_ptr(state, torch.float32, (n_slots, H, P, N), "state"),
                               _dev_ptr(A, torch.float32, (H,), "A"),
                               None if D is None else _dev_ptr(D, torch.float32, (H,), "D"),
                               flags, ctypes.byref(h)))
        self.handle = h.value
        self.log = None
        self.copies = None
        self.workspace = None
        self._ws_serial = None

    # -------------------------------------------------------------- lifecycle
    def destroy(self):
        _check(_lib.ssm_destroy(self.handle))

    def reset(self, slots, stream=None):
        arr, p = _host(slots, np.int32)
        _check(_lib.ssm_state_reset(self.handle, len(arr), p, _stream(stream)))

    def init(self, slots, init, stream=None):
        torch = _torch()
        arr, p = _host(slots, np.int32)
        _check(_lib.ssm_state_init(self.handle, len(arr), p,
                                   _dev_ptr(init, torch.float32,
                                            (len(arr), self.H, self.P, self.N), "init"),
                                   _stream(stream)))

    # ------------------------------------------------------------------ scan
    def scan_workspace_bytes(self, L):
        return int(_lib.ssm_scan_workspace_bytes(ctypes.byref(self.desc), int(L)))

    def _scan_workspace(self, L, workspace, device):
        """None: a cached buffer sized for L (the fastest form); "serial": one
        state's worth (the recurrent form); a tensor: used as given."""
        torch = _torch()
        if workspace is not None and not isinstance(workspace, str):
            return workspace
        if workspace == "serial":
            nb = self.H * self.P * self.N * 4
            if self._ws_serial is None:
                self._ws_serial = torch.empty(nb, dtype=torch.uint8, device=device)
            return self._ws_serial
        if workspace is not None:
            raise ValueError(f"unknown workspace mode {workspace!r}")
        nb = self.scan_workspace_bytes(L)
        if self.workspace is None or self.workspace.numel() < nb:
            self.workspace = torch.empty(nb, dtype=torch.uint8, device=device)
        return self.workspace

    def scan_chunk(self, slot, chunk_seq, x, dt, B, C, y=None, reset=None, ckpt_at=None,
                   ckpt_out=None, stream=None, workspace=None):
        torch = _torch()
        L = x.shape[0]
        H, P, N, G = self.H, self.P, self.N, self.G
        if y is None:
            y = torch.empty((L, H, P), dtype=self.io_dtype, device=x.device)
        rs, rp = _host(reset, np.uint8)
        if rs is not None and rs.shape != (L,):
            raise ValueError("reset must be u8[L]")
        ck, ckp = _host(ckpt_at if ckpt_at is not None else [], np.int64)
        n_ck = len(ck)
        if n_ck and ckpt_out is None:
            ckpt_out = torch.empty((n_ck, H, P, N), dtype=torch.float32, device=x.device)
        ws = self._scan_workspace(L, workspace, x.device)
        dt_ = self.io_dtype
        _check(_lib.ssm_scan_chunk(
            self.handle, int(slot), int(chunk_seq), int(L),
            _dev_ptr(x, dt_, (L, H, P), "x"), _dev_ptr(dt, dt_, (L, H), "dt"),
            _dev_ptr(B, dt_, (L, G, N), "B"), _dev_ptr(C, dt_, (L, G, N), "C"), rp,
            _dev_ptr(y, dt_, (L, H, P), "y"), n_ck, ckp if n_ck else None,
            _dev_ptr(ckpt_out, torch.float32, (n_ck, H, P, N), "ckpt_out") if n_ck else None,
            _dev_ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
        return (y, ckpt_out) if n_ck else y

    def scan_chunk_static(self, slot, chunk_seq, x, dt, B, C, y=None, reset=None, ckpt_at=None,
                          ckpt_out=None, stream=None):
        """scan_chunk with the library's static device scratch as workspace
        (no device memory is allocated by the call)."""
        torch = _torch()
        L = x.shape[0]
        H, P, N, G = self.H, self.P, self.N, self.G
        if y is None:
            y = torch.empty((L, H, P), dtype=self.io_dtype, device=x.device)
        rs, rp = _host(reset, np.uint8)
        if rs is not None and rs.shape != (L,):
            raise ValueError("reset must be u8[L]")
        ck, ckp = _host(ckpt_at if ckpt_at is not None else [], np.int64)
        n_ck = len(ck)
        if n_ck and ckpt_out is None:
            ckpt_out = torch.empty((n_ck, H, P, N), dtype=torch.float32, device=x.device)
        dt_ = self.io_dtype
        _check(_lib.ssm_scan_chunk_static(
            self.handle, int(slot), int(chunk_seq), int(L),
            _dev_ptr(x, dt_, (L, H, P), "x"), _dev_ptr(dt, dt_, (L, H), "dt"),
            _dev_ptr(B, dt_, (L, G, N), "B"), _dev_ptr(C, dt_, (L, G, N), "C"), rp,
            _dev_ptr(y, dt_, (L, H, P), "y"), n_ck, ckp if n_ck else None,
            _dev_ptr(ckpt_out, torch.float32, (n_ck, H, P, N), "ckpt_out") if n_ck else None,
            _stream(stream)))
        return (y, ckpt_out) if n_ck else y

    def scan_packed(self, cu_seqlens, seq_slots, x, dt, B, C, y=None, final=None,
                    receipts=False, cont=None, chunk_seq=None, stream=None):
        """Scan packed sequences into their own slots.  cu_seqlens int[nseq+1];
        seq_slots int[nseq]; cont u8[nseq] (continue the slot's stream) with
        chunk_seq u64[nseq].  final: None, True (allocate [nseq,H,P,N]) or a
        tensor.  Returns (y, final, receipts) with receipts a list of dicts
        when requested."""
        torch = _torch()
        cu, cup = _host(cu_seqlens, np.int32)
        sl, slp = _host(seq_slots, np.int32)
        nseq = len(sl)
        if cu.shape != (nseq + 1,):
            raise ValueError("cu_seqlens must have nseq + 1 entries")
        L = int(cu[-1]) if nseq else 0
        H, P, N, G = self.H, self.P, self.N, self.G
        if y is None:
            y = torch.empty((L, H, P), dtype=self.io_dtype, device=x.device)
        if final is True:
            final = torch.empty((nseq, H, P, N), dtype=torch.float32, device=x.device)
        ct, ctp = _host(cont, np.uint8)
        cs, csp = _host(chunk_seq, np.uint64)
        recs = (Receipt * max(nseq, 1))() if receipts else None
        dt_ = self.io_dtype
        _check(_lib.ssm_scan_packed(
            self.handle, nseq, cup, slp, ctp, csp,
            _dev_ptr(x, dt_, (L, H, P), "x"), _dev_ptr(dt, dt_, (L, H), "dt"),
            _dev_ptr(B, dt_, (L, G, N), "B"), _dev_ptr(C, dt_, (L, G, N), "C"),
            _dev_ptr(y, dt_, (L, H, P), "y"),
            None if final is None else _dev_ptr(final, torch.float32, (nseq, H, P, N), "final"),
            recs, _stream(stream)))
        return y, final, ([recs[i].as_dict() for i in range(nseq)] if receipts else None)

    # ---------------------------------------------------------------- decode
    def decode_step(self, slot_ids, x, dt, B, C, reset=None, y=None, stream=None):
        torch = _torch()
        ids, ip = _host(slot_ids, np.int32)
        b = len(ids)
        H, P, N, G = self.H, self.P, self.N, self.G
        if y is None:
            y = torch.empty((b, H, P), dtype=self.io_dtype, device=x.device)
        rs, rp = _host(reset, np.uint8)
        dt_ = self.io_dtype
        _check(_lib.ssm_decode_step(
            self.handle, b, ip, _dev_ptr(x, dt_, (b, H, P), "x"), _dev_ptr(dt, dt_, (b, H), "dt"),
            _dev_ptr(B, dt_, (b, G, N), "B"), _dev_ptr(C, dt_, (b, G, N), "C"), rp,
            _dev_ptr(y, dt_, (b, H, P), "y"), _stream(stream)))
        return y

    # ---------------------------------------------------------------- replay
    def replay_log_bytes(self, W):
        return int(_lib.ssm_replay_log_bytes(ctypes.byref(self.desc), self.S, W))

    def replay_attach(self, W, log=None):
        torch = _torch()
        nb = self.replay_log_bytes(W)
        if nb == 0:
            raise SSMError(SSM_E_INVALID_ARG, f"unsupported window {W}")
        if log is None:
            log = torch.empty(nb, dtype=torch.uint8, device=self.state.device)
        _check(_lib.ssm_replay_attach(self.handle, W, _dev_ptr(log, name="log"), log.numel()))
        self.log = log
        self.W = W

    def replay_step(self, slot_ids, x, dt, B, C, y=None, stream=None):
        torch = _torch()
        ids, ip = _host(slot_ids, np.int32)
        b = len(ids)
        n_in = x.shape[1]
        H, P, N, G = self.H, self.P, self.N, self.G
        if y is None:
            y = torch.empty((b, n_in, H, P), dtype=self.io_dtype, device=x.device)
        dt_ = self.io_dtype
        _check(_lib.ssm_replay_step(
            self.handle, b, ip, n_in, _dev_ptr(x, dt_, (b, n_in, H, P), "x"),
            _dev_ptr(dt, dt_, (b, n_in, H), "dt"), _dev_ptr(B, dt_, (b, n_in, G, N), "B"),
            _dev_ptr(C, dt_, (b, n_in, G, N), "C"), _dev_ptr(y, dt_, (b, n_in, H, P), "y"),
            _stream(stream)))
        return y

    def _gdn_step(self, fn, slot_ids, v, dt, beta, k, q, y, stream):
        torch = _torch()
        ids, ip = _host(slot_ids, np.int32)
        b = len(ids)
        n_in = v.shape[1]
        H, P, N, G = self.H, self.P, self.N, self.G
        if y is None:
            y = torch.empty((b, n_in, H, P), dtype=self.io_dtype, device=v.device)
        dt_ = self.io_dtype
        _check(fn(self.handle, b, ip, n_in, _dev_ptr(v, dt_, (b, n_in, H, P), "v"),
                  _dev_ptr(dt, dt_, (b, n_in, H), "dt"), _dev_ptr(beta, dt_, (b, n_in, H), "beta"),
                  _dev_ptr(k, dt_, (b, n_in, G, N), "k"), _dev_ptr(q, dt_, (b, n_in, G, N), "q"),
                  _dev_ptr(y, dt_, (b, n_in, H, P), "y"), _stream(stream)))
        return y

    def gdn_replay_step(self, slot_ids, v, dt, beta, k, q, y=None, stream=None):
        """ReplaySSM verify of a Gated DeltaNet handle: v[b,n_in,H,P],
        dt/beta[b,n_in,H], k/q[b,n_in,G,N]; returns o[b,n_in,H,P]."""
        return self._gdn_step(_lib.ssm_gdn_replay_step, slot_ids, v, dt, beta, k, q, y, stream)

    def gdn_copy_step(self, slot_ids, v, dt, beta, k, q, y=None, stream=None):
        """The copy-state-per-draft baseline of gdn_replay_step."""
        return self._gdn_step(_lib.ssm_gdn_copy_step, slot_ids, v, dt, beta, k, q, y, stream)

    def replay_commit(self, slot_ids, accepted):
        ids, ip = _host(slot_ids, np.int32)
        acc, ap = _host(accepted, np.int32)
        if acc.shape != ids.shape:
            raise ValueError("accepted must match slot_ids")
        _check(_lib.ssm_replay_commit(self.handle, len(ids), ip, ap))

    # ---------------------------------------------------------- copy baseline
    def copy_attach(self, n_in_max, buf=None):
        torch = _torch()
        nb = int(_lib.ssm_copy_buffer_bytes(ctypes.byref(self.desc), self.S, n_in_max))
        if buf is None:
            buf = torch.empty(nb // 4, dtype=torch.float32, device=self.state.device)
        _check(_lib.ssm_copy_attach(self.handle, n_in_max, _dev_ptr(buf, name="copies"),
                                    buf.numel() * buf.element_size()))
        self.copies = buf

    def copy_step(self, slot_ids, x, dt, B, C, y=None, stream=None):
        torch = _torch()
        ids, ip = _host(slot_ids, np.int32)
        b = len(ids)
        n_in = x.shape[1]
        H, P, N, G = self.H, self.P, self.N, self.G
        if y is None:
            y = torch.empty((b, n_in, H, P), dtype=self.io_dtype, device=x.device)
        dt_ = self.io_dtype
        _check(_lib.ssm_copy_step(
            self.handle, b, ip, n_in, _dev_ptr(x, dt_, (b, n_in, H, P), "x"),
            _dev_ptr(dt, dt_, (b, n_in, H), "dt"), _dev_ptr(B, dt_, (b, n_in, G, N), "B"),
            _dev_ptr(C, dt_, (b, n_in, G, N), "C"), _dev_ptr(y, dt_, (b, n_in, H, P), "y"),
            _stream(stream)))
        return y

    def copy_commit(self, slot_ids, accepted):
        ids, ip = _host(slot_ids, np.int32)
        acc, ap = _host(accepted, np.int32)
        _check(_lib.ssm_copy_commit(self.handle, len(ids), ip, ap))

    # ------------------------------------------------------------- state ops
    def materialize(self, slots, stream=None):
        arr, p = _host(slots, np.int32)
        _check(_lib.ssm_state_materialize(self.handle, len(arr), p, _stream(stream)))

    def checkpoint(self, slot, dst=None, stream=None):
        torch = _torch()
        if dst is None:
            dst = torch.empty((self.H, self.P, self.N), dtype=torch.float32,
                              device=self.state.device)
        r = Receipt()
        _check(_lib.ssm_state_checkpoint(self.handle, int(slot),
                                         _dev_ptr(dst, torch.float32,
                                                  (self.H, self.P, self.N), "dst"),
                                         ctypes.byref(r), _stream(stream)))
        return dst, r.as_dict()

    def restore(self, slot, src, receipt, stream=None):
        torch = _torch()
        r = Receipt.from_dict(receipt)
        _check(_lib.ssm_state_restore(self.handle, int(slot),
                                      _dev_ptr(src, torch.float32,
                                               (self.H, self.P, self.N), "src"),
                                      ctypes.byref(r), _stream(stream)))

    def blob_bytes(self):
        return int(_lib.ssm_state_blob_bytes(self.handle))

    def serialize(self, slot, stream=None):
        """The slot's state as a state blob (bytes) and its receipt."""
        cap = self.blob_bytes()
        buf = ctypes.create_string_buffer(cap)
        n, r = _SZ(0), Receipt()
        _check(_lib.ssm_state_serialize(self.handle, int(slot), buf, cap, ctypes.byref(n),
                                        ctypes.byref(r), _stream(stream)))
        return buf.raw[:n.value], r.as_dict()

    def deserialize(self, slot, blob, receipt, stream=None):
        blob = bytes(blob)
        r = Receipt.from_dict(receipt)
        _check(_lib.ssm_state_deserialize(self.handle, int(slot), blob, len(blob),
                                          ctypes.byref(r), _stream(stream)))

    # ------------------------------------------------------ conv1d (before the scan)
    def conv_attach(self, C, K, w, bias=None, act=True, state=None):
        """Causal depthwise conv of C channels and width K: w [C, K] and bias
        [C] fp32 device tensors; the conv state [S, C, K-1] fp32 (zeroed here
        when allocated)."""
        torch = _torch()
        if state is None and K > 1:
            state = torch.zeros((self.S, C, K - 1), dtype=torch.float32,
                                device=self.state.device)
        _check(_lib.ssm_conv_attach(
            self.handle, int(C), int(K), 1 if act else 0,
            None if K == 1 else _dev_ptr(state, torch.float32, (self.S, C, K - 1), "conv state"),
            _dev_ptr(w, torch.float32, (C, K), "w"),
            None if bias is None else _dev_ptr(bias, torch.float32, (C,), "bias")))
        self.conv_C, self.conv_K, self.conv_w, self.conv_b = C, K, w, bias
        self.conv_state = state

    def conv_chunk(self, slot, x, reset=None, y=None, stream=None):
        torch = _torch()
        L = x.shape[0]
        if y is None:
            y = torch.empty((L, self.conv_C), dtype=self.io_dtype, device=x.device)
        rs, rp = _host(reset, np.uint8)
        if rs is not None and len(rs) != L:
            raise ValueError("reset must have one flag per token")
        _check(_lib.ssm_conv_chunk(self.handle, int(slot), L,
                                   _dev_ptr(x, self.io_dtype, (L, self.conv_C), "x"), rp,
                                   _dev_ptr(y, self.io_dtype, (L, self.conv_C), "y"),
                                   _stream(stream)))
        return y

    def conv_decode(self, slot_ids, x, reset=None, y=None, stream=None):
        torch = _torch()
        ids, ip = _host(slot_ids, np.int32)
        b = len(ids)
        if y is None:
            y = torch.empty((b, self.conv_C), dtype=self.io_dtype, device=x.device)
        rs, rp = _host(reset, np.uint8)
        _check(_lib.ssm_conv_decode(self.handle, b, ip,
                                    _dev_ptr(x, self.io_dtype, (b, self.conv_C), "x"), rp,
                                    _dev_ptr(y, self.io_dtype, (b, self.conv_C), "y"),
                                    _stream(stream)))
        return y

    def position(self, slot):
        p, c = _I64(0), _U64(0)
        _check(_lib.ssm_get_position(self.handle, int(slot), ctypes.byref(p), ctypes.byref(c)))
        return p.value, c.value

    def log_state(self, slot):
        n, pend = _I32(0), _I32(0)
        _check(_lib.ssm_get_log_state(self.handle, int(slot), ctypes.byref(n), ctypes.byref(pend)))
        return n.value, pend.value

    def counters(self):
        c = Counters()
        _check(_lib.ssm_get_counters(self.handle, ctypes.byref(c)))
        return c.as_dict()
