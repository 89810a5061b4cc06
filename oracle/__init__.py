"""CPU oracle for the chunked-prefill / decode paged-attention step.

THIS PACKAGE IS TEST INFRASTRUCTURE. Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it.
The product path (the HIP library and its Python binding) never imports,
calls or links anything here, and nothing here imports the product path.

Modules
-------
attention  plain fp64 causal softmax attention over a contiguous KV history
paging     host model of the paged KV cache (append through a slot mapping,
           gather through a block table), exact byte-for-byte copies
scheduler  plain-Python FIFO batch builder (token budget, request cap, page
           budget, safety margin; decodes, then active prefills, then waiting)

Every function states the passage of the source pages it follows; the pages
are cited by title and section.  Points the pages leave open are read the
plainest way and listed in each module's docstring.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
to facts that do not come from the oracle itself (the pages' worked example,
a library routine, closed forms, brute force, invariants).
"""
