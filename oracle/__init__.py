"""fp64 CPU oracle of the gated delta-rule forward (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP path
in ``recurrent_state_memory_amd``.

* ``oracle.seq``   -- the definition: a token-by-token recurrence in float64.
* ``oracle.chunk`` -- the chunk-parallel WY algebra in float64, pinned to
  ``oracle.seq`` by brute force.
* ``oracle.errors`` -- the error measure used for parity.
"""
