"""OneLA large-beam Gated DeltaNet decode step for AMD MI355X (gfx950).

The compute path is the C-ABI library libonela.so (hand-written HIP kernels);
`Onela` is its thin Python binding. Importing this package does not load the
library; constructing `Onela` does, and fails if it has not been built.
"""
from .onela import EXPORTED, LIB_PATH, FullState, Onela, OnelaError, ReplayState, load_library, prefill  # noqa: F401
