"""The conv1d before the scan and the gated output, on the GPU against the
fp64 oracle (oracle/conv.py): chunks with resets (including more resets than
one launch holds), a stream cut into chunks against the whole, batched
decode, the state reset, the gate with and without the group RMS norm, and
the 65,536-token packed-prefill shape on sampled channels.

Tolerances: fp32 io rtol = atol = 1e-5; bf16 io (outputs rounded to bf16)
rtol = 2e-2 with atol = 2e-2 * RMS(ref).  The carried conv state holds copies
of inputs, so it is compared bit for bit.
"""
import numpy as np
import pytest

from oracle import conv as oconv
from streaming_state_amd import inputs
from tests.gpu_helpers import F32_TOL, assert_close, bf16_tol, host, say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ssm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from streaming_state_amd import ssm as m
    return m


def _tol(io, ref):
    return F32_TOL if io == "f32" else bf16_tol(ref)


def _handle(ssm, S, C, K, io, act, seed):
    A, D = inputs.params(70, 2)
    h = ssm.StreamState(2, 8, 16, S, to_dev(A), to_dev(D), io_dtype=io)
    r = np.random.default_rng(seed)
    w = r.standard_normal((C, K)).astype(np.float32) * 0.5
    b = r.standard_normal(C).astype(np.float32) * 0.1
    h.conv_attach(C, K, to_dev(w), to_dev(b), act=act)
    return h, w, b


def _x(io, L, C, seed):
    x = np.random.default_rng(seed).standard_normal((L, C)).astype(np.float32)
    if io == "bf16":
        x = inputs.bf16_to_f32(inputs.bf16_bits(x))
    dev = to_dev(x) if io == "f32" else to_dev(x).to(torch.bfloat16)
    return x, dev


@pytest.mark.parametrize("L,C,K,io,act,resets", [
    (300, 50, 4, "f32", True, [37, 38, 250]),     # one channel per thread
    (300, 52, 4, "f32", True, [0, 37, 38, 299]),  # four channels per thread
    (1000, 512, 4, "bf16", True, [100, 613]),
    (77, 64, 1, "f32", False, [5]),
    (77, 64, 2, "f32", False, []),
    (77, 33, 3, "bf16", True, [0]),
    (400, 16, 4, "f32", True, list(range(3, 400, 7))),  # 57 resets: several launches
    (2, 8, 4, "f32", True, []),                   # shorter than the window
])
def test_conv_chunk_vs_oracle(ssm, L, C, K, io, act, resets):
    say("conv chunk", L, C, K, io, act, len(resets))
    h, w, b = _handle(ssm, 3, C, K, io, act, L + C)
    r = np.random.default_rng(C)
    st0 = r.standard_normal((C, K - 1)).astype(np.float32)
    if K > 1:
        h.conv_state[1] = to_dev(st0)
    x, xd = _x(io, L, C, L)
    rs = np.zeros(L, np.uint8)
    rs[resets] = 1
    y = h.conv_chunk(1, xd, reset=rs)
    torch.cuda.synchronize()
    yr, sr = oconv.conv_chunk(x, w, b, st0, rs, act)
    assert_close(host(y), yr, **_tol(io, yr), what="conv y")
    if K > 1:
        np.testing.assert_array_equal(h.conv_state[1].cpu().numpy(), sr.astype(np.float32))
        assert not h.conv_state[0].any() and not h.conv_state[2].any()  # other slots untouched
    h.destroy()


def test_chunked_stream_matches_whole(ssm):
    L, C, K = 256, 64, 4
    say("conv chunked stream", L, C, K)
    h, w, b = _handle(ssm, 2, C, K, "f32", True, 5)
    x, xd = _x("f32", L, C, 6)
    rs = np.zeros(L, np.uint8)
    rs[[40, 41, 200]] = 1
    ys, t0 = [], 0
    for n in (1, 3, 17, 64, 171):
        ys.append(h.conv_chunk(0, xd[t0:t0 + n], reset=rs[t0:t0 + n]))
        t0 += n
    torch.cuda.synchronize()
    yr, sr = oconv.conv_chunk(x, w, b, None, rs)
    assert_close(host(torch.cat(ys)), yr, **F32_TOL, what="chunked conv y")
    np.testing.assert_array_equal(h.conv_state[0].cpu().numpy(), sr.astype(np.float32))
    h.destroy()


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_conv_decode_vs_oracle(ssm, io):
    S, b, C, K, steps = 6, 4, 96, 4, 20
    say("conv decode", io)
    h, w, bias = _handle(ssm, S, C, K, io, True, 11)
    states = np.zeros((S, C, K - 1))
    r = np.random.default_rng(12)
    for t in range(steps):
        slots = r.permutation(S)[:b].astype(np.int32)
        rs = (r.random(b) < 0.2).astype(np.uint8)
        x, xd = _x(io, b, C, 100 + t)
        y = h.conv_decode(slots, xd, reset=rs)
        yr = oconv.conv_decode(states, slots, x, w, bias, rs)
        torch.cuda.synchronize()
        assert_close(host(y), yr, **_tol(io, yr), what=f"conv decode step {t}")
    np.testing.assert_array_equal(h.conv_state.cpu().numpy(), states.astype(np.float32))
    # reset clears both halves of a slot's state
    h.reset([1, 4])
    torch.cuda.synchronize()
    assert not h.conv_state[1].any() and not h.conv_state[4].any()
    assert h.conv_state[0].abs().sum() > 0
    h.destroy()


@pytest.mark.parametrize("rows,C,group,io,norm", [
    (33, 96, 96, "f32", False),
    (64, 512, 128, "bf16", True),
    (7, 50, 25, "f32", True),     # one element per thread
    (16, 1536, 1536, "f32", True),
    (5, 24, 8, "bf16", True),        # 16-byte vectors, one per group
    (4, 16384, 16384, "bf16", True),  # 16-byte vectors, a group past the registers: two passes
])
def test_gate_vs_oracle(ssm, rows, C, group, io, norm):
    say("gate", rows, C, group, io, norm)
    r = np.random.default_rng(rows * C)
    y, yd = _x(io, rows, C, rows)
    z, zd = _x(io, rows, C, rows + 1)
    w = r.standard_normal(C).astype(np.float32) if norm else None
    out = ssm.gate(yd, zd, None if w is None else to_dev(w), group=group, eps=1e-5)
    ref = oconv.gate(y, z, w, group, eps=1e-5)
    torch.cuda.synchronize()
    assert_close(host(out), ref, **_tol(io, ref), what="gate")
    # in place
    out2 = ssm.gate(yd, zd, None if w is None else to_dev(w), group=group, eps=1e-5, out=yd)
    torch.cuda.synchronize()
    assert out2.data_ptr() == yd.data_ptr()
    assert torch.equal(out2, out)


def test_conv_packed_prefill_shape_sampled(ssm):
    """The packed-prefill workload's shape: 65,536 bf16 tokens of the conv's
    C = H*P + 2*G*N = 8,448 channels (H=128, P=64, N=128), K = 4, a reset at
    each of the 8 sequence starts; 64 sampled channels against the oracle."""
    L, C, K = 65536, 128 * 64 + 2 * 128, 4
    say("conv packed prefill", L, C, K)
    h, w, b = _handle(ssm, 1, C, K, "bf16", True, 21)
    g = torch.Generator(device="cuda")
    g.manual_seed(22)
    xd = torch.randn((L, C), generator=g, device="cuda").to(torch.bfloat16)
    lengths = inputs.sequence_lengths()
    rs = np.zeros(L, np.uint8)
    rs[np.concatenate([[0], np.cumsum(lengths)[:-1]])] = 1
    y = h.conv_chunk(0, xd, reset=rs)
    torch.cuda.synchronize()
    idx = np.sort(np.random.default_rng(23).choice(C, 64, replace=False))
    xs = host(xd[:, idx])
    yr, sr = oconv.conv_chunk(xs, w[idx], b[idx], None, rs)
    assert_close(host(y[:, idx]), yr, **bf16_tol(yr), what="packed conv y")
    np.testing.assert_array_equal(h.conv_state[0].cpu().numpy()[idx], sr.astype(np.float32))
    h.destroy()
