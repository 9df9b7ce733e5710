"""CPU oracle of the block-sparse attention forward (fp64, numpy / pure Python).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the bench's
CPU-baseline leg, never by the library or its Python binding.  It shares no code
with the HIP path.  Modules:
  solattn  the pass step by step (pool, score, select, extra tokens, attend)
  dense    textbook dense softmax attention (the all-kept limit)
  brute    a pure-Python per-token twin for tiny inputs
"""
from . import solattn, dense, brute  # noqa: F401
