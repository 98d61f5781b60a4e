"""CPU oracle of the CSA / HCA hot path (fp64, numpy).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may use it; the library and its Python binding never import
it, and it imports nothing from them.

Parity status: every function is pinned by CPU tests against closed forms,
invariants, library special cases and brute force, except the readings that
no pin can distinguish (entry 0 without a previous window, the RoPE position
of an entry, empty rows, the value being the non-RoPE part, the softmax
scale, and indexer keys coming from a second compressor instance).  Those
are "parity unpinned": both sides follow the stated reading.
"""
from . import formats, csa, brute  # noqa: F401
