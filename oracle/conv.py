"""The steps on either side of the scan: causal depthwise conv1d with its
carried conv_state, and the gated output (fp64, numpy).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name the conv state as half of a Mamba layer's recurrent state (the
state blob of "SSM.PREFIX.* -- recurrent-state companion" lists a Mamba layer
as [conv_state, ssm_state]) but define neither the convolution nor the output
gate.  The definitions below are the Mamba-2 block's (Dao and Gu, 2024):

  conv:  y[t, c] = act( b[c] + sum_{k=0}^{K-1} w[c, k] * x[t - (K-1) + k, c] )
         a per-channel causal filter of width K over the token axis; tap K-1
         meets the current token, act is SiLU (v * sigmoid(v)) or the identity.
  state: conv_state[c, j], j = 0..K-2, holds the K-1 inputs before the next
         token, oldest first; a fresh stream holds zeros.
  reset: a reset flag on token t starts a fresh stream at t, so the windows of
         t and later tokens see zeros for every input before t (the same rule
         as the scan's reset).
  gate:  g = y * SiLU(z); with a norm weight, each group of `group` channels
         is divided by its root mean square: out = g / sqrt(mean(g^2) + eps)
         * w[c] (the gated RMS norm of the Mamba-2 block).

Sums run over k in increasing order after the bias, so a chunked run is
bit-identical to the full run.
"""
import numpy as np


def silu(v):
    v = np.asarray(v, dtype=np.float64)
    return v / (1.0 + np.exp(-v))


def conv_chunk(x, w, bias=None, state=None, reset=None, act=True):
    """One chunk of one stream.  x[L, C], w[C, K], bias[C] or None,
    state[C, K-1] (None: zeros), reset u8[L] or None.
    Returns (y[L, C], new state[C, K-1])."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    L, C = x.shape
    K = w.shape[1]
    b = np.zeros(C) if bias is None else np.asarray(bias, dtype=np.float64)
    st = np.zeros((C, K - 1)) if state is None else np.asarray(state, dtype=np.float64)
    assert w.shape == (C, K) and st.shape == (C, K - 1) and b.shape == (C,)
    # history row i holds the input of token i - (K - 1) (rows 0..K-2: the state)
    hist = np.concatenate([st.T, x], axis=0)
    first = -(K - 1)  # earliest token index the windows may see
    y = np.zeros((L, C))
    for t in range(L):
        if reset is not None and reset[t]:
            first = t
        acc = b.copy()
        for k in range(K):
            src = t - (K - 1) + k
            if src >= first:
                acc = acc + w[:, k] * hist[src + K - 1]
        y[t] = silu(acc) if act else acc
    new = np.zeros((C, K - 1))
    for j in range(K - 1):
        src = L - (K - 1) + j
        if src >= first:
            new[:, j] = hist[src + K - 1]
    return y, new


def conv_decode(states, slot_ids, x, w, bias=None, reset=None, act=True):
    """One token for each of a batch of streams: states[S, C, K-1] is updated
    in place for the listed slots; x[b, C]; returns y[b, C]."""
    x = np.asarray(x, dtype=np.float64)
    y = np.zeros_like(x)
    for i, s in enumerate(slot_ids):
        r = None if reset is None else np.array([reset[i]], dtype=np.uint8)
        yi, states[s] = conv_chunk(x[i:i + 1], w, bias, states[s], r, act)
        y[i] = yi[0]
    return y


def gate(y, z, w=None, group=None, eps=1e-6):
    """y, z [R, C]; w [C] or None (no norm); group divides C."""
    g = np.asarray(y, dtype=np.float64) * silu(z)
    if w is None:
        return g
    R, C = g.shape
    group = C if group is None else group
    gg = g.reshape(R, C // group, group)
    ms = np.mean(gg * gg, axis=-1, keepdims=True)
    return (gg / np.sqrt(ms + eps)).reshape(R, C) * np.asarray(w, dtype=np.float64)
