"""fp64 CPU oracle for packed shared-prefix attention (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The HIP library shares no code with it.
"""
