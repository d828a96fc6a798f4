"""MI355X-native FwPKM chunked read-then-write step (HIP kernels behind a C ABI).

The package holds the HIP sources (csrc/), their in-tree build (build.py) and
a thin ctypes binding (memory.py).  Importing it does not load the library;
creating a ``Memory`` does, and fails loudly if the library is not built.
"""

from .memory import Config, FwPKMError, Memory, State, empty_state  # noqa: F401
