"""fp64 CPU oracle for the Mamba-2 streaming-state recurrence.

TEST INFRASTRUCTURE ONLY: this package is imported by ``tests/``, by the
smoke check in ``__graft_entry__.py`` and by the CPU-baseline leg of
``bench.py``, and by nothing in the product path.  It shares no code with the
HIP library (``streaming_state_amd``); neither imports the other.

``ssm_oracle.c`` holds the recurrence (plain sequential fp64 loops); this
module only marshals numpy arrays into it.  ``acceptance.py`` and
``schedule.py`` hold the integer/host-side model of speculative decoding and
of the replay flush schedule; ``blob.py`` reads and writes the state-blob byte
format of the recurrent-state companion store; ``conv.py`` holds the causal
depthwise conv1d with its carried conv state and the gated output (numpy,
fp64).  ``gdn_oracle.c`` (marshalled by ``gdn.py``) holds the Gated DeltaNet
recurrence and its replay form.

Every function is pinned by ``tests/test_oracle_*.py`` against the pages and
the mathematics (worked example, closed forms, brute force); none is "parity
unpinned".
"""
from .core import (  # noqa: F401
    ORC_OK, ORC_E_ARG, ORC_E_INVALID_CHUNK, OracleError,
    build, lib_path, scan, decode, spec_step, replay_unrolled,
)
from .acceptance import tokens_kept, copy_rule, expected_kept  # noqa: F401
from .schedule import replay_schedule  # noqa: F401
from . import gdn  # noqa: F401


def build_all():
    """Compile every C part of the oracle."""
    build()
    gdn.build()
