"""Decode parity: the HIP decode kernel through the C ABI vs the fp64 oracle."""
import numpy as np
import pytest

import oracle
from streaming_state_amd import inputs
from tests.gpu_helpers import F32_TOL, assert_close, bf16_dev, bf16_tol, host, say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ssm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from streaming_state_amd import ssm as m
    return m


@pytest.mark.parametrize("H,P,N,G,io", [
    (3, 40, 20, 1, "f32"),   # ragged row tile, ragged float4 groups
    (4, 72, 128, 2, "f32"),  # two row tiles (second ragged), two groups
    (2, 64, 128, 1, "bf16"),
    (1, 1, 4, 1, "f32"),     # smallest shape
])
def test_decode_small_shapes(ssm, H, P, N, G, io):
    say("decode small", H, P, N, G, io)
    S, b, steps = 7, 5, 6
    A, D = inputs.params(20, H)
    st0 = np.random.default_rng(1).standard_normal((S, H, P, N)).astype(np.float32) * 0.1
    h = ssm.StreamState(H, P, N, S, to_dev(A), to_dev(D), G=G, io_dtype=io)
    h.init(np.arange(S), to_dev(st0))
    ref_state = st0.astype(np.float64).copy()
    ref_pos = np.zeros(S, np.int64)
    slots = np.array([6, 0, 3, 2, 5], np.int32)
    for s in range(steps):
        x, dt, B, C = inputs.tokens(20, b, H, P, N, G, s)
        reset = np.array([s % 3 == 0, 0, s == 4, 0, 1], np.uint8)
        if io == "bf16":
            bits = [inputs.bf16_bits(a) for a in (x, dt, B, C)]
            x, dt, B, C = [inputs.bf16_to_f32(a) for a in bits]
            dev = [bf16_dev(a) for a in bits]
        else:
            dev = [to_dev(a) for a in (x, dt, B, C)]
        y = h.decode_step(slots, *dev, reset=reset)
        ref_y = oracle.decode(ref_state, ref_pos, slots, x, dt, B, C, A, D, reset=reset)
        torch.cuda.synchronize()
        tol = bf16_tol(ref_y) if io == "bf16" else F32_TOL
        assert_close(host(y), ref_y, what=f"y step {s}", **tol)
    assert_close(host(h.state), ref_state, what="state",
                 **(bf16_tol(ref_state) if io == "bf16" else F32_TOL))
    for sl in range(S):
        assert h.position(sl)[0] == ref_pos[sl]
    h.destroy()


def test_decode_workload2_full_batch(ssm):
    """B=256, H=128, P=64, N=128, 64 steps, per-slot resets p=0.02, seeded
    learned initial state, slots in a permuted order; the threaded oracle
    follows every slot: all outputs of every step and all final states."""
    W = inputs.W2
    B_, H, P, N, G = W["batch"], W["H"], W["P"], W["N"], W["G"]
    steps = W["steps"]
    say("decode workload2", B_, H, P, N, steps)
    A, D = inputs.params(2, H)
    init = inputs.device_state(2, B_, H, P, N)
    h = ssm.StreamState(H, P, N, B_, to_dev(A), to_dev(D), G=G)
    slots = inputs.slot_permutation(2, B_, B_)
    h.init(np.arange(B_), init)
    order = torch.as_tensor(slots).long().cuda()
    ref_state = host(init[order])          # ref entry i is slot slots[i]
    ref_pos = np.zeros(B_, np.int64)
    n_reset = 0
    for s in range(steps):
        x, dt, B, C = inputs.device_tokens(2, B_, H, P, N, G, seed_extra=s)
        reset = inputs.device_resets(2, s, B_)
        n_reset += int(reset.sum())
        y = h.decode_step(slots, x, dt, B, C, reset=reset)
        ref_y = oracle.decode(ref_state, ref_pos, np.arange(B_), host(x), host(dt), host(B),
                              host(C), A, D, reset=reset, n_threads=None)
        assert_close(host(y), ref_y, what=f"y step {s}", **F32_TOL)
    assert n_reset > 0
    assert_close(host(h.state[order]), ref_state, what="final states", **F32_TOL)
    for i in range(B_):
        assert h.position(int(slots[i]))[0] == ref_pos[i]
    h.destroy()


def test_decode_equals_scan_of_one_token(ssm):
    """Cross-path: a decode step equals a one-token chunk scan of the same slot."""
    H, P, N = 4, 64, 128
    say("decode vs scan L=1")
    A, D = inputs.params(21, H)
    st0 = inputs.device_state(21, 1, H, P, N).repeat(2, 1, 1, 1)  # same state in both slots
    h = ssm.StreamState(H, P, N, 2, to_dev(A), to_dev(D))
    h.init([0, 1], st0)
    x, dt, B, C = inputs.device_tokens(21, 1, H, P, N, 1, seed_extra=0)
    y_dec = h.decode_step([0], x, dt, B, C)
    y_scan = h.scan_chunk(1, 0, x, dt, B, C)
    torch.cuda.synchronize()
    assert_close(host(y_dec), host(y_scan), what="y", **F32_TOL)
    assert_close(host(h.state[0]), host(h.state[1]), what="state", **F32_TOL)
    h.destroy()


def test_decode_large_batch_split_launches(ssm):
    """More slots than one launch carries (the host splits the batch)."""
    H, P, N, S = 2, 64, 32, 600
    say("decode batch 600")
    A, D = inputs.params(22, H)
    h = ssm.StreamState(H, P, N, S, to_dev(A), to_dev(D))
    h.reset(np.arange(S))
    slots = np.random.default_rng(3).permutation(S).astype(np.int32)
    x, dt, B, C = inputs.tokens(22, S, H, P, N, 1, 0)
    ref_state = np.zeros((S, H, P, N))
    ref_pos = np.zeros(S, np.int64)
    y = h.decode_step(slots, to_dev(x), to_dev(dt), to_dev(B), to_dev(C))
    ref = oracle.decode(ref_state, ref_pos, slots, x, dt, B, C, A, D)
    torch.cuda.synchronize()
    assert_close(host(y), ref, what="y", **F32_TOL)
    assert_close(host(h.state), ref_state, what="state", **F32_TOL)
    h.destroy()
