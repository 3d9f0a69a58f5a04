"""Chunk-scan parity: the HIP scan through the C ABI vs the fp64 oracle, over
every chunking of the tiny fixture, the Mamba-130M-shaped layer streamed in
chunks, ragged shapes with resets and checkpoints, and the 65,536-token packed
bf16 prefill (sampled heads)."""
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


def _stream_chunks(h, slot, sizes, dev, reset=None, workspace=None):
    """Scan dev tensors chunk by chunk; return concatenated y."""
    ys, t0 = [], 0
    for seq, s in enumerate(sizes):
        sl = slice(t0, t0 + s)
        y = h.scan_chunk(slot, seq, dev[0][sl], dev[1][sl], dev[2][sl], dev[3][sl],
                         reset=None if reset is None else reset[sl], workspace=workspace)
        ys.append(y)
        t0 += s
    return torch.cat(ys) if ys else None


def test_workload0_every_chunking(ssm):
    w = inputs.workload0()
    L, H, P, N = w["L"], w["H"], w["P"], w["N"]
    reset = np.zeros(L, np.uint8)
    reset[w["reset_at"]] = 1
    ref = oracle.scan(w["x"], w["dt"], w["B"], w["C"], w["A"], w["D"], reset=reset)
    dev = [to_dev(w[k]) for k in ("x", "dt", "B", "C")]
    for pi, sizes in enumerate(inputs.partitions0(L)):
        say("workload0 partition", pi, sizes)
        h = ssm.StreamState(H, P, N, 2, to_dev(w["A"]), to_dev(w["D"]))
        h.reset([0, 1])
        y = _stream_chunks(h, 1, sizes, dev, reset)
        torch.cuda.synchronize()
        assert_close(host(y), ref["y"], what=f"y {sizes}", **F32_TOL)
        assert_close(host(h.state[1]), ref["state"], what=f"state {sizes}", **F32_TOL)
        assert h.position(1) == (ref["pos"], len(sizes))
        assert float(h.state[0].abs().max()) == 0.0  # the other slot is untouched
        h.destroy()


def test_workload0_reset_separation(ssm):
    """Prefix, reset, then B equals B from a fresh state; without the reset it
    differs (inequality control near the boundary)."""
    w = inputs.workload0()
    L, H, P, N, k = w["L"], w["H"], w["P"], w["N"], w["reset_at"]
    dev = [to_dev(w[n]) for n in ("x", "dt", "B", "C")]
    h = ssm.StreamState(H, P, N, 3, to_dev(w["A"]), to_dev(w["D"]))
    h.reset([0, 1, 2])
    say("workload0 reset separation")
    reset = np.zeros(L, np.uint8)
    reset[k] = 1
    y_r = h.scan_chunk(0, 0, *dev, reset=reset)
    y_f = h.scan_chunk(1, 0, *[d[k:] for d in dev])
    y_n = h.scan_chunk(2, 0, *dev)
    torch.cuda.synchronize()
    assert_close(host(y_r[k:]), host(y_f), what="reset vs fresh", rtol=1e-6, atol=1e-6)
    assert_close(host(h.state[0]), host(h.state[1]), what="state", rtol=1e-6, atol=1e-6)
    assert np.abs(host(y_r[k]) - host(y_n[k])).max() > 1e-5
    assert h.position(0)[0] == L - k


@pytest.mark.parametrize("chunk,ws", [(None, None), (None, "serial"), (256, None), (64, None),
                                      (17, None), (1, None)])
def test_workload1_streaming(ssm, chunk, ws):
    """Mamba-130M-shaped layer (H=24, P=64, N=128, L=2048, fp32): full scan and
    chunked streaming with the state carried across chunks.  Chunks of 64
    tokens or more take the tile-parallel form; ws="serial" forces the
    recurrent form on the full scan."""
    w = inputs.workload1()
    L, H, P, N = w["L"], w["H"], w["P"], w["N"]
    say("workload1 chunk", chunk, ws)
    ref = oracle.scan(w["x"], w["dt"], w["B"], w["C"], w["A"], w["D"], n_threads=None)
    dev = [to_dev(w[k]) for k in ("x", "dt", "B", "C")]
    h = ssm.StreamState(H, P, N, 1, to_dev(w["A"]), to_dev(w["D"]))
    h.reset([0])
    sizes = [L] if chunk is None else [chunk] * (L // chunk) + ([L % chunk] if L % chunk else [])
    y = _stream_chunks(h, 0, sizes, dev, workspace=ws)
    torch.cuda.synchronize()
    assert_close(host(y), ref["y"], what="y", **F32_TOL)
    assert_close(host(h.state[0]), ref["state"], what="state", **F32_TOL)
    assert h.position(0) == (L, len(sizes))


@pytest.mark.parametrize("H,P,N,G,io,L", [
    (3, 40, 20, 1, "f32", 97),
    (4, 72, 128, 2, "f32", 130),
    (2, 64, 128, 1, "bf16", 301),
    (4, 16, 64, 4, "bf16", 77),
    # the MFMA form: head pairs sharing a group, an odd head count (one head
    # per workgroup), pairs over two groups, one head per group
    (6, 64, 128, 1, "bf16", 203),
    (3, 64, 128, 1, "bf16", 150),
    (4, 64, 128, 2, "bf16", 200),
    (4, 64, 128, 4, "bf16", 90),
])
def test_ragged_resets_checkpoints(ssm, H, P, N, G, io, L):
    say("scan ragged", H, P, N, G, io, L)
    r = np.random.default_rng(L)
    x, dt, B, C = inputs.tokens(30, L, H, P, N, G)
    A, D = inputs.params(30, H)
    if io == "bf16":
        bits = [inputs.bf16_bits(a) for a in (x, dt, B, C)]
        x, dt, B, C = [inputs.bf16_to_f32(a) for a in bits]
        dev = [bf16_dev(a) for a in bits]
    else:
        dev = [to_dev(a) for a in (x, dt, B, C)]
    st0 = r.standard_normal((H, P, N)).astype(np.float32) * 0.05
    reset = np.zeros(L, np.uint8)
    reset[[L // 3, L // 3 + 1, (2 * L) // 3]] = 1
    ck = sorted({0, L // 3 - 1, L // 3, L // 2, L - 1})
    ref = oracle.scan(x, dt, B, C, A, D, state=st0, pos=5, reset=reset, ckpt_at=ck)
    h = ssm.StreamState(H, P, N, 2, to_dev(A), to_dev(D), G=G, io_dtype=io)
    h.init([1], to_dev(st0[None]))
    y, cko = h.scan_chunk(1, 0, *dev, reset=reset, ckpt_at=ck)
    torch.cuda.synchronize()
    tol = (lambda a: bf16_tol(a)) if io == "bf16" else (lambda a: F32_TOL)
    assert_close(host(y), ref["y"], what="y", **tol(ref["y"]))
    assert_close(host(cko), ref["ckpt"], what="checkpoints", **tol(ref["ckpt"]))
    assert_close(host(h.state[1]), ref["state"], what="carry-out", **tol(ref["state"]))
    # the last reset fixes the position: tokens after it
    assert h.position(1) == (ref["pos"], 1) and ref["pos"] == L - (2 * L) // 3


def test_mfma_form_dt_not_word_aligned(ssm):
    """The head-pair MFMA kernel reads dt of a head pair as one 32-bit word;
    a dt buffer that starts on an odd bf16 element takes the one-head kernel.
    Both forms must give the oracle's results (here with a reset and
    checkpoints), and the outputs of the two must agree closely."""
    H, P, N, G, L = 4, 64, 128, 1, 150
    say("scan dt offset by one element", H, L)
    x, dt, B, C = inputs.tokens(32, L, H, P, N, G)
    A, D = inputs.params(32, H)
    bits = [inputs.bf16_bits(a) for a in (x, dt, B, C)]
    x, dt, B, C = [inputs.bf16_to_f32(a) for a in bits]
    dx, ddt, dB, dC = [bf16_dev(a) for a in bits]
    # the same dt values behind a one-element offset: 2-byte but not 4-byte aligned
    padded = torch.zeros(L * H + 1, dtype=torch.bfloat16, device="cuda")
    padded[1:] = ddt.reshape(-1)
    ddt_odd = padded[1:].view(L, H)
    assert ddt_odd.data_ptr() % 4 == 2 and ddt.data_ptr() % 4 == 0
    reset = np.zeros(L, np.uint8)
    reset[70] = 1
    ck = [10, 69, 149]
    ref = oracle.scan(x, dt, B, C, A, D, reset=reset, ckpt_at=ck)
    outs = []
    for d_ in (ddt, ddt_odd):
        h = ssm.StreamState(H, P, N, 1, to_dev(A), to_dev(D), G=G, io_dtype="bf16")
        h.reset([0])
        y, cko = h.scan_chunk(0, 0, dx, d_, dB, dC, reset=reset, ckpt_at=ck)
        torch.cuda.synchronize()
        assert_close(host(y), ref["y"], what="y", **bf16_tol(ref["y"]))
        assert_close(host(cko), ref["ckpt"], what="checkpoints", **bf16_tol(ref["ckpt"]))
        outs.append((host(y), host(h.state[0])))
        h.destroy()
    assert_close(outs[0][0], outs[1][0], what="pair vs one-head y", **bf16_tol(outs[1][0]))
    assert_close(outs[0][1], outs[1][1], what="pair vs one-head state", **bf16_tol(outs[1][1]))


@pytest.mark.parametrize("ws", [None, "serial"])
def test_fp32_forms_negative_dt(ssm, ws):
    """fp32 scan with some negative dt values: the tile-parallel form (ws
    None) and the recurrent form ("serial") against the oracle, then decode
    steps with negative dt from the carried state."""
    H, P, N, G, L = 2, 64, 128, 1, 300
    say("fp32 negative dt", ws)
    x, dt, B, C = inputs.tokens(35, L + 4, H, P, N, G)
    A, D = inputs.params(35, H)
    dt = dt.copy()
    dt[20:26, 0] = -0.02
    dt[100:140, :] = -0.01
    dt[L + 1:, 1] = -0.02
    h = ssm.StreamState(H, P, N, 1, to_dev(A), to_dev(D))
    h.reset([0])
    y = h.scan_chunk(0, 0, *(to_dev(a[:L]) for a in (x, dt, B, C)), workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.scan(x[:L], dt[:L], B[:L], C[:L], A, D)
    assert_close(host(y), ref["y"], what="y", **F32_TOL)
    assert_close(host(h.state[0]), ref["state"], what="state", **F32_TOL)
    st = ref["state"][None].copy()
    pos = np.array([L], np.int64)
    for t in range(L, L + 4):
        yd = h.decode_step([0], *(to_dev(a[t:t + 1]) for a in (x, dt, B, C)))
        yr = oracle.decode(st, pos, np.zeros(1, np.int64), x[t:t + 1], dt[t:t + 1], B[t:t + 1],
                           C[t:t + 1], A, D)
        torch.cuda.synchronize()
        assert_close(host(yd), yr, what=f"decode {t}", **F32_TOL)
    assert_close(host(h.state[0]), st[0], what="state after decode", **F32_TOL)
    h.destroy()


@pytest.mark.parametrize("one_head", [False, True])
def test_mfma_form_negative_dt(ssm, one_head):
    """A finite negative dt is accepted (the pages give no rule against it):
    the head-pair kernel carries |dt| in the mask's exponent and takes the
    sign from dt itself; the one-head kernel (dt behind a one-element offset)
    multiplies by dt.  Negative runs in one head only, in both heads, and
    across a block boundary, with a reset and checkpoints."""
    H, P, N, G, L = 4, 64, 128, 1, 300
    say("scan negative dt", H, L)
    x, dt, B, C = inputs.tokens(34, L, H, P, N, G)
    A, D = inputs.params(34, H)
    dt = dt.copy()
    dt[10:15, 1] = -0.02          # head 1 of the first pair only
    dt[60:70, 2:4] = -0.02        # both heads of the second pair, across blocks 0 and 1
    dt[130, :] = -0.02            # every head, one token
    dt[200:204, 0] = -0.02        # right after the reset below
    bits = [inputs.bf16_bits(a) for a in (x, dt, B, C)]
    x, dt, B, C = [inputs.bf16_to_f32(a) for a in bits]
    assert (dt < 0).sum() == 5 + 20 + 4 + 4
    dev = [bf16_dev(a) for a in bits]
    if one_head:  # the same dt values, 2-byte but not 4-byte aligned
        padded = torch.zeros(L * H + 1, dtype=torch.bfloat16, device="cuda")
        padded[1:] = dev[1].reshape(-1)
        dev[1] = padded[1:].view(L, H)
        assert dev[1].data_ptr() % 4 == 2
    reset = np.zeros(L, np.uint8)
    reset[200] = 1
    ck = [14, 69, 130, 199, 203, 299]
    ref = oracle.scan(x, dt, B, C, A, D, reset=reset, ckpt_at=ck)
    h = ssm.StreamState(H, P, N, 1, to_dev(A), to_dev(D), G=G, io_dtype="bf16")
    h.reset([0])
    y, cko = h.scan_chunk(0, 0, *dev, reset=reset, ckpt_at=ck)
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all()
    assert_close(host(y), ref["y"], what="y", **bf16_tol(ref["y"]))
    assert_close(host(cko), ref["ckpt"], what="checkpoints", **bf16_tol(ref["ckpt"]))
    assert_close(host(h.state[0]), ref["state"], what="carry-out", **bf16_tol(ref["state"]))
    h.destroy()


@pytest.mark.parametrize("carry", [True, False])
def test_mfma_form_many_segments_across_launches(ssm, carry):
    """The head-pair MFMA kernel over more segments than one launch takes
    (40 resets: runs of one token, back-to-back resets, a reset on the last
    token), with checkpoints on both sides of the launch split and just before
    resets.  With a carried-in state and resets later in the chunk the carry
    goes through the workspace; without, the chunk opens with a reset."""
    H, P, N, G, L = 4, 64, 128, 1, 700
    say("scan many segments", carry)
    x, dt, B, C = inputs.tokens(33, L, H, P, N, G)
    A, D = inputs.params(33, H)
    bits = [inputs.bf16_bits(a) for a in (x, dt, B, C)]
    x, dt, B, C = [inputs.bf16_to_f32(a) for a in bits]
    dev = [bf16_dev(a) for a in bits]
    r = np.random.default_rng(33)
    rs = set(r.choice(np.arange(2, L - 1), 34, replace=False).tolist())
    rs |= {5, 6, 7, 300, 301, L - 1}
    if not carry:
        rs.add(0)
    reset = np.zeros(L, np.uint8)
    reset[sorted(rs)] = 1
    assert int(reset.sum()) >= 40
    ck = sorted({4, 6, 299, 300, 450, 698, L - 1} | {int(t) for t in r.choice(L, 12, replace=False)})
    st0 = (r.standard_normal((H, P, N)) * 0.05).astype(np.float32)
    ref = oracle.scan(x, dt, B, C, A, D, state=st0 if carry else None, reset=reset, ckpt_at=ck)
    h = ssm.StreamState(H, P, N, 2, to_dev(A), to_dev(D), G=G, io_dtype="bf16")
    h.init([1], to_dev(st0[None]))
    y, cko = h.scan_chunk(1, 0, *dev, reset=reset, ckpt_at=ck)
    torch.cuda.synchronize()
    assert_close(host(y), ref["y"], what="y", **bf16_tol(ref["y"]))
    assert_close(host(cko), ref["ckpt"], what="checkpoints", **bf16_tol(ref["ckpt"]))
    assert_close(host(h.state[1]), ref["state"], what="carry-out", **bf16_tol(ref["state"]))
    h.destroy()


@pytest.mark.parametrize("H,P,N,G,io,L,resets,ck", [
    # resets inside tiles (one doubled, one on a checkpoint token), checkpoints
    # on tile edges and on the last token
    (3, 64, 128, 1, "f32", 300, [70, 100, 101, 190], [5, 63, 64, 100, 150, 299]),
    # more than 64 tiles: two launches, the carry passing through the slot
    (4, 32, 64, 2, "f32", 4200, [1000, 4096, 4100], [4095, 4096, 4199]),
    # bf16 io outside the SSD form's shape
    (2, 32, 96, 1, "bf16", 257, [128], [0, 127, 256]),
    # one full tile that starts with a reset: the carried-in state is dropped
    (2, 64, 128, 1, "f32", 64, [0, 40], [63]),
    # a reset on a tile's first token, ragged last tile
    (5, 64, 32, 5, "f32", 200, [64, 128], [199]),
])
def test_tile_parallel_form(ssm, H, P, N, G, io, L, resets, ck):
    """The tile-parallel scan (fp32 MFMA) against the oracle: carry-in from a
    learned state, per-token resets inside and on tile edges, checkpoints."""
    say("scan tile-parallel", H, P, N, G, io, L)
    r = np.random.default_rng(L + P)
    x, dt, B, C = inputs.tokens(31, L, H, P, N, G)
    A, D = inputs.params(31, H)
    if io == "bf16":
        bits = [inputs.bf16_bits(a) for a in (x, dt, B, C)]
        x, dt, B, C = [inputs.bf16_to_f32(a) for a in bits]
        dev = [bf16_dev(a) for a in bits]
    else:
        dev = [to_dev(a) for a in (x, dt, B, C)]
    st0 = r.standard_normal((H, P, N)).astype(np.float32) * 0.05
    reset = np.zeros(L, np.uint8)
    reset[resets] = 1
    ref = oracle.scan(x, dt, B, C, A, D, state=st0, pos=5, reset=reset, ckpt_at=ck,
                      n_threads=None)
    h = ssm.StreamState(H, P, N, 2, to_dev(A), to_dev(D), G=G, io_dtype=io)
    h.init([1], to_dev(st0[None]))
    assert h.scan_workspace_bytes(L) > H * P * N * 4
    y, cko = h.scan_chunk(1, 0, *dev, reset=reset, ckpt_at=ck)
    torch.cuda.synchronize()
    tol = (lambda a: bf16_tol(a)) if io == "bf16" else (lambda a: F32_TOL)
    assert_close(host(y), ref["y"], what="y", **tol(ref["y"]))
    assert_close(host(cko), ref["ckpt"], what="checkpoints", **tol(ref["ckpt"]))
    assert_close(host(h.state[1]), ref["state"], what="carry-out", **tol(ref["state"]))
    assert h.position(1) == (ref["pos"], 1)
    # deterministic: the same chunk again from the same state gives the same bits
    h.init([0], to_dev(st0[None]))
    y2, cko2 = h.scan_chunk(0, 0, *dev, reset=reset, ckpt_at=ck)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(cko, cko2) and torch.equal(h.state[0], h.state[1])


def test_empty_chunk_is_neutral(ssm):
    w = inputs.workload0()
    H, P, N = w["H"], w["P"], w["N"]
    say("empty chunk")
    dev = [to_dev(w[k]) for k in ("x", "dt", "B", "C")]
    h = ssm.StreamState(H, P, N, 1, to_dev(w["A"]), to_dev(w["D"]))
    h.reset([0])
    h.scan_chunk(0, 0, *[d[:10] for d in dev])
    before = h.state.clone()
    e = [d[:0] for d in dev]
    y = h.scan_chunk(0, 1, *e)
    torch.cuda.synchronize()
    assert y.shape[0] == 0
    assert torch.equal(before, h.state)
    assert h.position(0) == (10, 2)


def test_workload4_packed_prefill_sampled_heads(ssm):
    """8 packed sequences, 65,536 tokens, H=128, P=64, N=128, bf16 inputs, fp32
    state, reset at every sequence start, final states emitted as checkpoints.
    The oracle runs three sampled heads over all tokens."""
    W = inputs.W4
    L, H, P, N, G = W["L"], W["H"], W["P"], W["N"], W["G"]
    lengths = inputs.sequence_lengths()
    reset, cu, ends = inputs.packed_layout(lengths)
    say("workload4", lengths.tolist())
    d = inputs.device_prefill(L, H, P, N, G)
    h = ssm.StreamState(H, P, N, 1, d["A"], d["D"], G=G, io_dtype="bf16")
    h.reset([0])
    y, cko = h.scan_chunk(0, 0, d["x"], d["dt"], d["B"], d["C"], reset=reset, ckpt_at=ends)
    torch.cuda.synchronize()
    heads = [0, 61, 127]
    A, D = inputs.params(4, H)
    hs = torch.as_tensor(heads).long().cuda()
    ref = oracle.scan(host(d["x"][:, hs]), host(d["dt"][:, hs]), host(d["B"]), host(d["C"]),
                      A[heads], D[heads], reset=reset, ckpt_at=ends, n_threads=None)
    ys = host(y[:, hs])
    assert_close(ys, ref["y"], what="y", **bf16_tol(ref["y"]))
    ck = host(cko[:, hs])
    assert_close(ck, ref["ckpt"], what="checkpoints", **bf16_tol(ref["ckpt"]))
    assert_close(host(h.state[0][hs]), ref["state"], what="carry-out", **bf16_tol(ref["state"]))
    assert h.position(0)[0] == lengths[-1]


@pytest.mark.parametrize("sizes", [[700], [1] * 20 + [680], [37] * 18 + [34], [64, 129, 3, 504],
                                   [0, 300, 0, 400]])
def test_bf16_mfma_path_chunked_with_reset(ssm, sizes):
    """bf16, P=64, N=128 (the MFMA path): streamed in chunks with the state
    carried across, a reset at t=300 inside a chunk, checkpoints mid-chunk."""
    H, P, N, L = 4, 64, 128, 700
    say("bf16 chunked", sizes[:4])
    x, dt, B, C = inputs.tokens(31, L, H, P, N, 1)
    A, D = inputs.params(31, H)
    bits = [inputs.bf16_bits(a) for a in (x, dt, B, C)]
    x, dt, B, C = [inputs.bf16_to_f32(a) for a in bits]
    dev = [bf16_dev(a) for a in bits]
    reset = np.zeros(L, np.uint8)
    reset[300] = 1
    st0 = np.random.default_rng(5).standard_normal((H, P, N)).astype(np.float32) * 0.05
    ref = oracle.scan(x, dt, B, C, A, D, state=st0, reset=reset)
    h = ssm.StreamState(H, P, N, 1, to_dev(A), to_dev(D), io_dtype="bf16")
    h.init([0], to_dev(st0[None]))
    ys, t0 = [], 0
    for q, s in enumerate(sizes):
        sl = slice(t0, t0 + s)
        ys.append(h.scan_chunk(0, q, *[d_[sl] for d_ in dev], reset=reset[sl]))
        t0 += s
    torch.cuda.synchronize()
    y = torch.cat(ys)
    assert_close(host(y), ref["y"], what="y", **bf16_tol(ref["y"]))
    assert_close(host(h.state[0]), ref["state"], what="state", **bf16_tol(ref["state"]))
    assert h.position(0) == (L - 300, len(sizes))
