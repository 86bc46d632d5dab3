"""fp64 CPU oracle for FFD sparse decode attention -- TEST INFRASTRUCTURE ONLY.

Follows "Faster Than Flash: Exploiting Attention Sparsity for Efficient
Long-Context Decoding" (gist.science technical summary of arXiv 2609.00097),
Method sections 1 (2-bit thumbnail + 8-bit residual K cache), 2 (Top-delta
selection, pseudo-max) and 3 (the three kernel stages).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything under ``oracle/``.  It shares no code, table
or constant generator with the HIP library and imports nothing from it; the
product path never calls it.

Modules
-------
``ffd_oracle``  vectorised numpy float64 implementation (pack, scores,
                pseudo-max, block selection, exact attention, LSE merge,
                dense attention).
``bruteforce``  deliberately naive pure-Python version for tiny inputs
                (``fractions.Fraction`` for every quantizer decision, exact
                rational dot products); it pins ``ffd_oracle``.

Every function is pinned by a ``-m "not gpu"`` test against something other
than itself (brute force, closed forms, invariants, textbook softmax);
nothing here is "parity unpinned".
"""
