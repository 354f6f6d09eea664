"""fp64 CPU oracle of the gated-delta-rule mixer -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never uses it, and it
never uses the HIP library: the two share no code.  The library itself is
``gdn_oracle.c``; this module marshals numpy arrays into it.

Parity status of each function (what pins it is in ``tests/test_oracle.py``):
every exported function is pinned by closed forms, special cases, brute force
or an independent formulation; the model-level conventions that the pages leave
open (tap order, channel order, key-head mapping, eps placement) are fixed by
stated readings and are, as conventions, parity unpinned.
"""
from .gdn_oracle import (  # noqa: F401
    OracleShape, lib, gates, conv_silu, raw_recurrence, window, tree, prefill, commit,
    replay, commit_replay, max_threads,
)
from . import inproj  # noqa: F401  (the affine 4-bit in-projection, numpy fp64)
