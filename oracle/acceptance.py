"""Acceptance model of speculative decoding (host-side integers and reals).

TEST INFRASTRUCTURE ONLY (see the package docstring).

A verify step handles the real token plus T drafts; the tokens kept are the
real token plus the drafts up to the first rejected one ("Why Speculative
Decoding Slows Hybrid Mamba Models at Large Batch Sizes", section
"Implementing It", Role 1).  With each draft accepted independently with
probability p, the expected number kept is the geometric sum
1 + p + ... + p**T.  The copy rule compares that with the state traffic of a
step that writes a state copy per draft, about (1 + T) / 2 plain steps
(section "What This Means for You").
"""


def tokens_kept(p, T):
    """Expected tokens kept per verify step: 1 + p + ... + p**T (closed form)."""
    p = float(p)
    T = int(T)
    if T < 0:
        raise ValueError("T must be >= 0")
    if p == 1.0:
        return float(T + 1)
    return (1.0 - p ** (T + 1)) / (1.0 - p)


expected_kept = tokens_kept


def copy_rule(p, T):
    """Tokens kept per unit of copy-path state traffic; above 1 speculation still wins."""
    return tokens_kept(p, T) / ((1.0 + T) / 2.0)
