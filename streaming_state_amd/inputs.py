"""Seeded synthetic inputs for the five workloads (no method arithmetic here).

This module is the only code shared by the HIP-path tests and the oracle
tests: it draws random numbers with the value distributions of the workloads
and nothing else.  It never computes any part of the recurrence.

Distributions (same for every workload):
  x ~ N(0, 1)                     per token, head and head-dim
  B, C ~ N(0, 1/N)                per token and group
  dt = softplus(z), z ~ N(-2, 0.5)   (dt arrives positive; the path applies no
                                    bias, softplus or clamp of its own)
  A_h = -exp(u), u ~ U(0, ln 16)  so A_h lies in [-16, -1]
  D_h ~ N(0, 1)
Decode and replay workloads start from a seeded fp32 state N(0, 0.02^2) at
position 0, loaded as a learned initial state (the pages leave the initial
state open; this is the reading used).

Seeds: numpy PCG64 seeded from SeedSequence([20261202 + workload, tensor id,
extra...]); each tensor (and each step of per-step tensors) has its own
stream, so any slice can be regenerated alone.

bf16 inputs are drawn in fp32 and rounded once, round-to-nearest-even; both
sides consume the same bf16 bits (``bf16_bits`` / ``bf16_to_f32``).

For the 65,536-token prefill workload the draws are made on the GPU with a
seeded torch generator (``device_prefill``) because host generation of 0.5 G
normals takes minutes; the oracle then reads a host copy of the sampled
heads' inputs.
"""
import numpy as np

BASE_SEED = 20261202
_TENSOR_IDS = {"x": 1, "dt": 2, "B": 3, "C": 4, "A": 5, "D": 6, "state": 7, "reset": 8,
               "accept": 9, "lengths": 10, "slots": 11, "beta": 12, "k": 13, "q": 14}


def rng(workload, tensor, *extra):
    ss = np.random.SeedSequence([BASE_SEED + int(workload), _TENSOR_IDS[tensor]] +
                                [int(e) for e in extra])
    return np.random.Generator(np.random.PCG64(ss))


def _softplus(z):
    # log(1 + e^z) written stably; an input transform of the draw
    return np.where(z > 20.0, z, np.log1p(np.exp(np.minimum(z, 20.0))))


# ---------------------------------------------------------------------------
# bf16 bit handling (round-to-nearest-even from fp32)
# ---------------------------------------------------------------------------
def bf16_bits(a):
    """fp32 array -> uint16 bf16 bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


# ---------------------------------------------------------------------------
# parameters and per-token tensors
# ---------------------------------------------------------------------------
def params(workload, H):
    """A[H], D[H] fp32."""
    A = -np.exp(rng(workload, "A").uniform(0.0, np.log(16.0), size=H))
    D = rng(workload, "D").standard_normal(H)
    return A.astype(np.float32), D.astype(np.float32)


def tokens(workload, L, H, P, N, G=1, *extra):
    """x[L,H,P], dt[L,H], B[L,G,N], C[L,G,N] fp32."""
    x = rng(workload, "x", *extra).standard_normal((L, H, P), dtype=np.float32)
    z = rng(workload, "dt", *extra).normal(-2.0, 0.5, size=(L, H))
    dt = _softplus(z).astype(np.float32)
    s = 1.0 / np.sqrt(N)
    B = (rng(workload, "B", *extra).standard_normal((L, G, N)) * s).astype(np.float32)
    C = (rng(workload, "C", *extra).standard_normal((L, G, N)) * s).astype(np.float32)
    return x, dt, B, C


def initial_state(workload, S, H, P, N):
    return (rng(workload, "state").standard_normal((S, H, P, N), dtype=np.float32) *
            np.float32(0.02))


# ---------------------------------------------------------------------------
# workload 0: tiny chunk-equivalence fixture
# ---------------------------------------------------------------------------
W0 = dict(L=64, H=2, P=4, N=8, G=1, reset_at=32)


def workload0():
    d = W0
    x, dt, B, C = tokens(0, d["L"], d["H"], d["P"], d["N"], d["G"])
    A, D = params(0, d["H"])
    return dict(x=x, dt=dt, B=B, C=C, A=A, D=D, **d)


def partitions0(L=64, n_random=8):
    """Chunkings of L tokens: uniform sizes 1, 3, 7, 13, 64 with a short final
    chunk; a partition with empty chunks at the start, at t=32 and at the end;
    and seeded random partitions into prime sizes (with a short final chunk)."""
    parts = []
    for s in (1, 3, 7, 13, 64):
        sizes = [s] * (L // s) + ([L % s] if L % s else [])
        parts.append(sizes)
    parts.append([0, 32, 0, L - 32, 0])
    primes = [2, 3, 5, 7, 11, 13, 17, 19, 23]
    r = rng(0, "lengths", 99)
    for _ in range(n_random):
        sizes, tot = [], 0
        while tot < L:
            s = int(primes[r.integers(len(primes))])
            s = min(s, L - tot)
            sizes.append(s)
            tot += s
        parts.append(sizes)
    return parts


# ---------------------------------------------------------------------------
# workload 1: Mamba-130M-shaped single layer, fp32
# ---------------------------------------------------------------------------
W1 = dict(L=2048, H=24, P=64, N=128, G=1, chunk_sizes=(1, 17, 64, 256))


def workload1(L=None):
    d = dict(W1)
    if L is not None:
        d["L"] = L
    x, dt, B, C = tokens(1, d["L"], d["H"], d["P"], d["N"], d["G"])
    A, D = params(1, d["H"])
    return dict(x=x, dt=dt, B=B, C=C, A=A, D=D, **d)


# ---------------------------------------------------------------------------
# workload 2: batched decode, 256 requests, 64 steps, reset p = 0.02
# ---------------------------------------------------------------------------
W2 = dict(batch=256, H=128, P=64, N=128, G=1, steps=64, reset_p=0.02)


def decode_step_inputs(step, batch=256, H=128, P=64, N=128, G=1, workload=2):
    """Inputs of one decode step: x[b,H,P], dt[b,H], B,C[b,G,N], reset u8[b]."""
    x, dt, B, C = tokens(workload, batch, H, P, N, G, step)
    reset = (rng(workload, "reset", step).random(batch) < 0.02).astype(np.uint8)
    return x, dt, B, C, reset


def slot_permutation(workload, S, batch):
    """Seeded distinct slot ids (exercises the slot indirection)."""
    return rng(workload, "slots").permutation(S)[:batch].astype(np.int32)


# ---------------------------------------------------------------------------
# workload 3: speculative verify, T = 4 drafts accepted i.i.d. p = 0.7
# ---------------------------------------------------------------------------
W3 = dict(batch=256, H=128, P=64, N=128, G=1, steps=128, T=4, p=0.7, windows=(8, 16, 32))


def spec_step_inputs(step, batch=256, n_in=5, H=128, P=64, N=128, G=1, workload=3):
    """Inputs of the n_in in-flight tokens: x[b,n_in,H,P], dt[b,n_in,H], B,C[b,n_in,G,N]."""
    x, dt, B, C = tokens(workload, batch * n_in, H, P, N, G, step)
    return (x.reshape(batch, n_in, H, P), dt.reshape(batch, n_in, H),
            B.reshape(batch, n_in, G, N), C.reshape(batch, n_in, G, N))


def acceptances(steps, batch, T=4, p=0.7, workload=3):
    """a[steps, batch] = 1 + number of leading accepted drafts (each Bernoulli(p),
    truncated at the first miss)."""
    r = rng(workload, "accept")
    ok = r.random((steps, batch, T)) < p
    lead = np.cumprod(ok, axis=2).sum(axis=2)
    return (1 + lead).astype(np.int32)


# ---------------------------------------------------------------------------
# workload 4: packed prefill, 8 sequences, 65,536 tokens, bf16 inputs
# ---------------------------------------------------------------------------
W4 = dict(L=65536, H=128, P=64, N=128, G=1, nseq=8, lo=1024, hi=15360, chunk=256)


def sequence_lengths(total=65536, nseq=8, lo=1024, hi=15360, workload=4):
    """nseq lengths in [lo, hi] summing to total: draw nseq-1 uniformly and let
    the last be the remainder, redrawing until it is in range."""
    r = rng(workload, "lengths")
    while True:
        head = r.integers(lo, hi + 1, size=nseq - 1)
        last = total - int(head.sum())
        if lo <= last <= hi:
            return np.concatenate([head, [last]]).astype(np.int64)


def packed_layout(lengths):
    """Return (reset u8[L], cu_seqlens int64[nseq+1], seq_end int64[nseq])."""
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    L = int(cu[-1])
    reset = np.zeros(L, dtype=np.uint8)
    reset[cu[:-1]] = 1
    return reset, cu, cu[1:] - 1


def host_prefill(L, H, P, N, G=1, workload=4, heads=None):
    """Host draws for a prefill workload, rounded to bf16.

    Returns bf16 bits (uint16) for x[L,H,P] (or only ``heads``), dt[L,H],
    B[L,G,N], C[L,G,N] and fp32 A[H], D[H].
    """
    x, dt, B, C = tokens(workload, L, H, P, N, G)
    if heads is not None:
        x = x[:, heads]
        dt = dt[:, heads]
    A, D = params(workload, H)
    return dict(x=bf16_bits(x), dt=bf16_bits(dt), B=bf16_bits(B), C=bf16_bits(C), A=A, D=D)


def device_prefill(L, H, P, N, G=1, workload=4, device="cuda", dtype=None):
    """Device draws (seeded torch generator) with the same distributions.

    Returns torch tensors x[L,H,P], dt[L,H], B[L,G,N], C[L,G,N] in ``dtype``
    (default bfloat16, rounded RNE from fp32 by the device conversion) and fp32
    A[H], D[H] from the host parameter draw.
    """
    import torch
    if dtype is None:
        dtype = torch.bfloat16
    g = torch.Generator(device=device)
    g.manual_seed(BASE_SEED + workload)
    x = torch.randn((L, H, P), generator=g, device=device, dtype=torch.float32)
    z = torch.randn((L, H), generator=g, device=device, dtype=torch.float32) * 0.5 - 2.0
    dt = torch.nn.functional.softplus(z)
    s = 1.0 / float(np.sqrt(N))
    B = torch.randn((L, G, N), generator=g, device=device, dtype=torch.float32) * s
    C = torch.randn((L, G, N), generator=g, device=device, dtype=torch.float32) * s
    A, D = params(workload, H)
    return dict(x=x.to(dtype), dt=dt.to(dtype), B=B.to(dtype), C=C.to(dtype),
                A=torch.from_numpy(A).to(device), D=torch.from_numpy(D).to(device))


def device_tokens(workload, L, H, P, N, G=1, seed_extra=0, device="cuda", dtype=None):
    """Device draws for per-step decode/replay tensors (fp32 by default)."""
    import torch
    if dtype is None:
        dtype = torch.float32
    g = torch.Generator(device=device)
    g.manual_seed((BASE_SEED + workload) * 1000003 + int(seed_extra))
    x = torch.randn((L, H, P), generator=g, device=device, dtype=torch.float32)
    z = torch.randn((L, H), generator=g, device=device, dtype=torch.float32) * 0.5 - 2.0
    dt = torch.nn.functional.softplus(z)
    s = 1.0 / float(np.sqrt(N))
    B = torch.randn((L, G, N), generator=g, device=device, dtype=torch.float32) * s
    C = torch.randn((L, G, N), generator=g, device=device, dtype=torch.float32) * s
    return x.to(dtype), dt.to(dtype), B.to(dtype), C.to(dtype)


def device_state(workload, S, H, P, N, std=0.02, device="cuda"):
    """Seeded fp32 initial state N(0, std^2) drawn on the device ([S,H,P,N])."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((BASE_SEED + workload) * 7919 + 17)
    return torch.randn((S, H, P, N), generator=g, device=device, dtype=torch.float32) * std


def device_resets(workload, step, batch, p=0.02):
    """Per-slot reset flags of one decode step (host u8[batch])."""
    return (rng(workload, "reset", step).random(batch) < p).astype(np.uint8)


# ---------------------------------------------------------------------------
# Gated DeltaNet verify workload (the pages name the recurrence but give no
# workload): B=256 slots of one layer with 32 value heads over 16 key groups,
# head dims 128 x 128 (2 MiB of fp32 state per slot), T = 4 drafts, p = 0.7,
# windows 8, 16, 32.
# ---------------------------------------------------------------------------
W5 = dict(batch=256, H=32, G=16, P=128, N=128, steps=128, T=4, p=0.7, windows=(8, 16, 32))


def gdn_tokens(workload, L, H, P, N, G=1, *extra):
    """v[L,H,P] ~ N(0,1); k[L,G,N] unit-norm (a N(0,I) draw divided by its
    norm) and q[L,G,N] unit-norm times N^-1/2 (how such layers feed keys and
    queries); beta[L,H] = sigmoid(N(0,1)); dt[L,H] = softplus(N(-2, 0.5)), the
    gate's step as for Mamba-2.  fp32."""
    v = rng(workload, "x", *extra).standard_normal((L, H, P), dtype=np.float32)
    z = rng(workload, "dt", *extra).normal(-2.0, 0.5, size=(L, H))
    dt = _softplus(z).astype(np.float32)
    bz = rng(workload, "beta", *extra).standard_normal((L, H))
    beta = (1.0 / (1.0 + np.exp(-bz))).astype(np.float32)
    k = rng(workload, "k", *extra).standard_normal((L, G, N))
    k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)
    q = rng(workload, "q", *extra).standard_normal((L, G, N))
    q = (q / np.linalg.norm(q, axis=-1, keepdims=True) / np.sqrt(N)).astype(np.float32)
    return v, dt, beta, k, q


def device_gdn_tokens(workload, L, H, P, N, G=1, seed_extra=0, device="cuda"):
    """The same distributions drawn on the device with a seeded torch
    generator (fp32): v, dt, beta, k, q."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((BASE_SEED + workload) * 1000003 + int(seed_extra))
    v = torch.randn((L, H, P), generator=g, device=device)
    dt = torch.nn.functional.softplus(torch.randn((L, H), generator=g, device=device) * 0.5 - 2.0)
    beta = torch.sigmoid(torch.randn((L, H), generator=g, device=device))
    k = torch.randn((L, G, N), generator=g, device=device)
    k = k / k.norm(dim=-1, keepdim=True)
    q = torch.randn((L, G, N), generator=g, device=device)
    q = q / q.norm(dim=-1, keepdim=True) / float(np.sqrt(N))
    return v, dt, beta, k, q
