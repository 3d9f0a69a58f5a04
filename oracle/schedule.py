"""Replay-log flush schedule (integers only).

TEST INFRASTRUCTURE ONLY (see the package docstring).

ReplaySSM keeps a checkpoint and a log of per-token inputs; the full state is
written only when the log fills ("Why Speculative Decoding Slows Hybrid Mamba
Models at Large Batch Sizes", section "The Fix: Log the Inputs, Checkpoint the
State", and the Glossary's checkpoint entry: a whole-state copy refreshed
once per window).  Reading used here: the log holds committed entries plus the n_in
in-flight entries of the current step, capacity W.  Before a step, if the
committed length plus n_in would exceed W, the log is folded into the
checkpoint (a flush) and the length restarts at 0; after the step the length
grows by the number of accepted tokens.  With one token per step and W = 16
that is one flush every 16 steps, as the page says.
"""
import numpy as np


def replay_schedule(accepted, W, n_in, len0=None):
    """accepted[steps, batch] (1..n_in) -> dict of flush mask, counts, lengths.

    Returns:
      flush[steps, batch]  bool, a flush happens before that step
      len_before[steps, batch]  committed log length seen by the step (after any flush)
      flushes[batch]  number of flushes
      final_len[batch]  committed length after the last step
    """
    acc = np.asarray(accepted, dtype=np.int64)
    if acc.ndim != 2:
        raise ValueError("accepted must be [steps, batch]")
    if W < n_in or n_in < 1:
        raise ValueError("need 1 <= n_in <= W")
    if ((acc < 1) | (acc > n_in)).any():
        raise ValueError("accepted counts must lie in 1..n_in")
    steps, batch = acc.shape
    length = np.zeros(batch, dtype=np.int64) if len0 is None else np.array(len0, np.int64)
    flush = np.zeros((steps, batch), dtype=bool)
    len_before = np.zeros((steps, batch), dtype=np.int64)
    for s in range(steps):
        for b in range(batch):
            if length[b] + n_in > W:
                flush[s, b] = True
                length[b] = 0
            len_before[s, b] = length[b]
            length[b] += acc[s, b]
    return {"flush": flush, "len_before": len_before, "flushes": flush.sum(axis=0),
            "final_len": length}
