"""The oracle: a plain, slow, obviously-correct CPU implementation of what the
tiled GEMM + epilogue, the transpose and the layout algebra compute.

TEST INFRASTRUCTURE ONLY.  It exists to check the HIP library, and nothing in
the product path may import, call, link or execute anything in this package.
The only users are the test-suite (``tests/``), the smoke check in
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``.  It
shares no code with the HIP library and imports nothing from it.

Parts:
  * ``gemm``      -- binary64 naive-loop GEMM with the scalar epilogue, the
                     storage-format decoders and the bit-copy transpose (C,
                     via ctypes; ``oracle.c``).
  * ``layout``    -- scalar layout evaluator: shape/stride layouts, crd2idx,
                     colexicographic idx2crd, pointwise composition,
                     logical/tiled divide, local_partition, the strip-mined
                     thread map with its predicate, and the ldmatrix /
                     SM80 operand tables the pages print.

Every public function names the passage of the pages it follows.  Functions
with no independent pin say "parity unpinned" in their docstring.
"""
from . import layout  # noqa: F401
