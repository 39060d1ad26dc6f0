"""Float64 CPU reference for the Gated DeltaNet prefill -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  It shares no code with the HIP library.
"""
