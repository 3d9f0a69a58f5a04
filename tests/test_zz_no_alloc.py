"""ssm_scan_chunk_static (the chunk scan with the library's static device
scratch as its workspace, for callers that cannot allocate) against
ssm_scan_chunk given a workspace of the same size, through the C ABI: two
calls in a row, the second with a smaller input, on every form the static
workspace selects (tile-parallel, recurrent, SSD with the carry through the
workspace), plus the finite check and the size refusal."""
import numpy as np
import pytest

from streaming_state_amd import inputs
from tests.gpu_helpers import bf16_dev, say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ssm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from streaming_state_amd import ssm as m
    return m


def _dev(io, arrays):
    if io == "bf16":
        return [bf16_dev(inputs.bf16_bits(a)) for a in arrays]
    return [to_dev(a) for a in arrays]


# (H, P, N, io, first call (L, resets, checkpoints), second call (smaller))
CASES = [
    # fp32, Mamba-130M-shaped heads: 1,024 tokens take the tile-parallel form
    # (16 tile states fit 16 MiB), then 300 tokens with resets inside tiles
    (24, 64, 128, "f32", (1024, [], [100, 1023]), (300, [70, 71, 200], [69, 299])),
    # fp32, 2,048 tokens need 25 MB of tile states: the recurrent form; then a
    # short chunk carrying state in with a reset later (the workspace carry)
    (24, 64, 128, "f32", (2048, [1500], [10, 2047]), (40, [20], [19, 39])),
    # bf16 head pairs on the MFMA form, carry-in and resets later (workspace)
    (4, 64, 128, "bf16", (700, [300, 301, 650], [299, 699]), (90, [45], [44])),
]


@pytest.mark.parametrize("H,P,N,io,first,second", CASES)
def test_static_scratch_matches_workspace_entry(ssm, H, P, N, io, first, second):
    say("scan static scratch", H, P, N, io, first[0], second[0])
    A, D = inputs.params(60, H)
    r = np.random.default_rng(60 + H)
    st0 = (r.standard_normal((H, P, N)) * 0.05).astype(np.float32)
    a = ssm.StreamState(H, P, N, 1, to_dev(A), to_dev(D), io_dtype=io)
    b = ssm.StreamState(H, P, N, 1, to_dev(A), to_dev(D), io_dtype=io)
    a.init([0], to_dev(st0[None]))
    b.init([0], to_dev(st0[None]))
    ws = torch.empty(ssm.SSM_STATIC_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    for q, (L, resets, ck) in enumerate((first, second)):
        dev = _dev(io, inputs.tokens(61 + q, L, H, P, N))
        reset = np.zeros(L, np.uint8)
        reset[resets] = 1
        ya, ca = a.scan_chunk_static(0, q, *dev, reset=reset, ckpt_at=ck)
        yb, cb = b.scan_chunk(0, q, *dev, reset=reset, ckpt_at=ck, workspace=ws)
        torch.cuda.synchronize()
        # the same form over the same inputs: identical bits
        assert torch.equal(ya, yb), f"y, call {q}"
        assert torch.equal(ca, cb), f"checkpoints, call {q}"
        assert torch.equal(a.state, b.state), f"state, call {q}"
        assert a.position(0) == b.position(0)
    a.destroy()
    b.destroy()


def test_static_scratch_finite_check_and_refusal(ssm):
    H, P, N = 2, 64, 128
    say("scan static scratch finite check")
    A, D = inputs.params(62, H)
    h = ssm.StreamState(H, P, N, 1, to_dev(A), to_dev(D), check_finite=True)
    h.reset([0])
    x, dt, B, C = inputs.tokens(62, 80, H, P, N)
    y = h.scan_chunk_static(0, 0, *(to_dev(v) for v in (x, dt, B, C)))
    torch.cuda.synchronize()
    before = h.state.clone()
    x[5, 1, 3] = np.nan
    with pytest.raises(ssm.SSMError) as e:
        h.scan_chunk_static(0, 1, *(to_dev(v) for v in (x, dt, B, C)))
    assert e.value.code == ssm.SSM_E_INVALID_CHUNK
    assert torch.equal(before, h.state) and h.position(0) == (80, 1)
    assert torch.isfinite(y).all()
    h.destroy()
    # a layer whose state exceeds the static scratch cannot carry a state
    # through it: refused before any work, nothing changed
    H = 1024  # 32 MiB of state
    A, D = np.full(H, -1.0, np.float32), np.zeros(H, np.float32)
    g = ssm.StreamState(H, 64, 128, 1, to_dev(A), to_dev(D), io_dtype="bf16")
    g.reset([0])
    L = 4
    xb = torch.zeros((L, H, 64), dtype=torch.bfloat16, device="cuda")
    dtb = torch.zeros((L, H), dtype=torch.bfloat16, device="cuda")
    Bb = torch.zeros((L, 1, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ssm.SSMError) as e:
        g.scan_chunk_static(0, 0, xb, dtb, Bb, Bb, reset=np.array([0, 0, 1, 0], np.uint8))
    assert e.value.code == ssm.SSM_E_INVALID_ARG and "static scratch" in str(e.value)
    assert g.position(0) == (0, 0)
    g.destroy()
