"""Pins of the conv / gate oracle against independent statements: numpy's
convolution (which flips the filter itself), identity and shift filters,
chunked == full bitwise with resets, the reset rule, and closed forms of the
SiLU gate and the group RMS norm.  A reversed filter, a dropped bias, a state
kept newest-first or a reset that leaks the old window fails one of these."""
import numpy as np
import pytest
from scipy.special import expit

from oracle import conv


def _rand(seed, L, C, K):
    r = np.random.default_rng(seed)
    return (r.standard_normal((L, C)), r.standard_normal((C, K)), r.standard_normal(C),
            r.standard_normal((C, K - 1)))


@pytest.mark.parametrize("K", [1, 2, 4, 7])
def test_matches_numpy_convolution(K):
    x, w, b, _ = _rand(K, 37, 5, K)
    y, st = conv.conv_chunk(x, w, b, None, act=False)
    for c in range(5):
        ref = np.convolve(x[:, c], w[c, ::-1], mode="full")[:37] + b[c]
        np.testing.assert_allclose(y[:, c], ref, rtol=1e-13, atol=1e-13)
    if K > 1:  # the state is the last K-1 inputs, oldest first
        np.testing.assert_array_equal(st, x[-(K - 1):].T)


def test_carried_state_is_the_previous_inputs():
    x, w, b, _ = _rand(3, 20, 4, 4)
    full, _ = conv.conv_chunk(x, w, b, None, act=False)
    # feeding tokens 0..9 as the state-producing prefix equals a state built by hand
    _, st = conv.conv_chunk(x[:10], w, b, None, act=False)
    np.testing.assert_array_equal(st, x[7:10].T)
    y2, _ = conv.conv_chunk(x[10:], w, b, x[7:10].T, act=False)
    np.testing.assert_array_equal(y2, full[10:])


def test_identity_and_shift_filters():
    x, _, _, s0 = _rand(5, 12, 3, 4)
    ident = np.zeros((3, 4))
    ident[:, 3] = 1.0
    y, st = conv.conv_chunk(x, ident, None, s0, act=False)
    np.testing.assert_array_equal(y, x)
    shift = np.zeros((3, 4))
    shift[:, 0] = 1.0  # the oldest tap: y[t] = x[t - 3], from the state for t < 3
    y, _ = conv.conv_chunk(x, shift, None, s0, act=False)
    np.testing.assert_array_equal(y[:3], s0.T)
    np.testing.assert_array_equal(y[3:], x[:-3])


def test_short_chunks_shift_the_state():
    x, w, b, s0 = _rand(6, 2, 3, 4)  # L = 2 < K - 1 = 3
    _, st = conv.conv_chunk(x, w, b, s0, act=False)
    np.testing.assert_array_equal(st[:, 0], s0[:, 2])
    np.testing.assert_array_equal(st[:, 1:], x.T)


@pytest.mark.parametrize("act", [False, True])
def test_chunked_equals_full_bitwise_with_resets(act):
    L, C, K = 50, 6, 4
    x, w, b, s0 = _rand(7, L, C, K)
    reset = np.zeros(L, np.uint8)
    reset[[0, 17, 18, 41]] = 1
    full, sf = conv.conv_chunk(x, w, b, s0, reset, act)
    for cuts in ([0, 1, 2, 3, 50], [0, 17, 18, 41, 50], [0, 0, 5, 5, 50, 50],
                 [0] + list(range(1, 50)) + [50], [0, 13, 26, 39, 50]):
        st, ys = s0, []
        for a, e in zip(cuts[:-1], cuts[1:]):
            y, st = conv.conv_chunk(x[a:e], w, b, st, reset[a:e], act)
            ys.append(y)
        np.testing.assert_array_equal(np.concatenate(ys), full)
        np.testing.assert_array_equal(st, sf)


def test_reset_starts_a_fresh_window():
    L, C, K = 30, 4, 4
    x, w, b, s0 = _rand(8, L, C, K)
    reset = np.zeros(L, np.uint8)
    reset[12] = 1
    y, st = conv.conv_chunk(x, w, b, s0, reset)
    fresh, st2 = conv.conv_chunk(x[12:], w, b, None)
    np.testing.assert_array_equal(y[12:], fresh)
    np.testing.assert_array_equal(st, st2)
    # inequality control: without the reset the first tokens after it differ
    y0, _ = conv.conv_chunk(x, w, b, s0)
    assert np.abs(y0[12] - y[12]).min() > 1e-6
    # a reset on the last token leaves only that token in the state
    r = np.zeros(L, np.uint8)
    r[-1] = 1
    _, st = conv.conv_chunk(x, w, b, s0, r)
    np.testing.assert_array_equal(st[:, :2], 0.0)
    np.testing.assert_array_equal(st[:, 2], x[-1])


def test_decode_is_one_token_chunks():
    S, C, K, steps = 3, 5, 4, 9
    x, w, b, _ = _rand(9, steps * S, C, K)
    states = np.zeros((S, C, K - 1))
    ref = [np.zeros((C, K - 1)) for _ in range(S)]
    r = np.random.default_rng(1)
    for t in range(steps):
        rs = (r.random(S) < 0.2).astype(np.uint8)
        xt = x[t * S:(t + 1) * S]
        y = conv.conv_decode(states, [2, 0, 1], xt, w, b, rs)
        for i, s in enumerate([2, 0, 1]):
            yr, ref[s] = conv.conv_chunk(xt[i:i + 1], w, b, ref[s], rs[i:i + 1])
            np.testing.assert_array_equal(y[i], yr[0])
    for s in range(S):
        np.testing.assert_array_equal(states[s], ref[s])


def test_silu_and_gate_closed_forms():
    v = np.linspace(-30, 30, 121)
    np.testing.assert_allclose(conv.silu(v), v * expit(v), rtol=1e-14, atol=1e-300)
    assert conv.silu(0.0) == 0.0
    y = np.array([[3.0, 4.0, -1.0, 2.0]])
    z = np.array([[0.5, -2.0, 1.0, 7.0]])
    np.testing.assert_allclose(conv.gate(y, z), y * z * expit(z), rtol=1e-15)
    # the norm divides each group by its RMS: for g = (3, 4) the RMS is sqrt(12.5)
    zz = np.full((1, 2), 40.0)  # SiLU(40) = 40 (1 - e^-40) ~ 40
    out = conv.gate(np.array([[3.0, 4.0]]), zz, w=np.ones(2), group=2, eps=0.0)
    np.testing.assert_allclose(out, [[3 / np.sqrt(12.5), 4 / np.sqrt(12.5)]], rtol=1e-14)
    # per-group RMS of the normalised output is 1 (weights 1, eps 0)
    r = np.random.default_rng(2)
    yy, zz, w = r.standard_normal((5, 12)), r.standard_normal((5, 12)), r.standard_normal(12)
    o = conv.gate(yy, zz, np.ones(12), group=4, eps=0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(o.reshape(5, 3, 4) ** 2, axis=-1)), 1.0,
                               rtol=1e-13)
    o2 = conv.gate(yy, zz, w, group=4, eps=0.0)
    np.testing.assert_allclose(o2, o * w, rtol=1e-14)


# ---------------------------------------------------------------------------
# planted mistakes: each mutant of the oracle's source must fail a pin
# ---------------------------------------------------------------------------
MUTANTS = {
    "reversed taps": ("acc = acc + w[:, k] * hist[src + K - 1]",
                      "acc = acc + w[:, K - 1 - k] * hist[src + K - 1]"),
    "dropped bias": ("acc = b.copy()", "acc = np.zeros(C)"),
    "state newest first": ("hist = np.concatenate([st.T, x], axis=0)",
                           "hist = np.concatenate([st.T[::-1], x], axis=0)"),
    "reset ignored": ("            first = t\n", "            first = first\n"),
    "window off by one": ("            src = t - (K - 1) + k\n", "            src = t - K + k\n"),
    "state kept across reset": ("        src = L - (K - 1) + j\n        if src >= first:",
                                "        src = L - (K - 1) + j\n        if True:"),
    "gate without silu": ("g = np.asarray(y, dtype=np.float64) * silu(z)",
                          "g = np.asarray(y, dtype=np.float64) * np.asarray(z)"),
    "norm without mean": ("ms = np.mean(gg * gg, axis=-1, keepdims=True)",
                          "ms = np.sum(gg * gg, axis=-1, keepdims=True)"),
}


def _mutant(name):
    import types
    src = open(conv.__file__).read()
    a, b = MUTANTS[name]
    assert src.count(a) == 1, name
    mod = types.ModuleType("conv_mutant")
    exec(compile(src.replace(a, b), "conv_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_fail_a_pin(name, monkeypatch):
    mod = _mutant(name)
    monkeypatch.setattr(conv, "conv_chunk", mod.conv_chunk)
    monkeypatch.setattr(conv, "conv_decode", mod.conv_decode)
    monkeypatch.setattr(conv, "gate", mod.gate)
    pins = [lambda: test_matches_numpy_convolution(4), test_carried_state_is_the_previous_inputs,
            test_identity_and_shift_filters, test_short_chunks_shift_the_state,
            lambda: test_chunked_equals_full_bitwise_with_resets(True),
            test_reset_starts_a_fresh_window, test_silu_and_gate_closed_forms]
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"mutant '{name}' passes every pin"
