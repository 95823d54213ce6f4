"""CPU oracle for the paged-KV hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or run anything in this package.  The product
(the HIP library and its Python binding) never routes through it, and the two
share no code: this package imports nothing from the library, the binding or
the workload generator.

Everything here is plain, slow and meant to be checked by eye against the
pages it cites:

* ``codecs``  -- bfloat16 and OCP FP8 E4M3 (e4m3fn) codecs written from the
  formats' bit-level definitions (no ml_dtypes, no torch).
* ``paged``   -- the block-table address map, the KV append scatter, the
  materialisation of a sequence's contiguous K/V from its block table, and
  attention computed by the two-pass softmax definition in float64, for
  single-token decode and for causal prefill chunks.  It also holds the
  online (block-by-block) softmax recurrence and the log-sum-exp merge of
  split partials, whose only use is to be pinned against the definition.

Every function is pinned by ``tests/test_oracle_*.py`` against something other
than itself: the block-size-4 worked example printed in the "Batching and
memory management" tutorial, brute-force contiguous attention, closed forms,
permutation invariance, the online == two-pass identity, and the format tables.
No function here is "parity unpinned".
"""
from . import codecs, paged  # noqa: F401
