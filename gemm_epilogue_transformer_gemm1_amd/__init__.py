"""MI355X (gfx950) GEMM-epilogue transformer hot path.

The compute lives in libcoda.so (hand-written HIP, C ABI declared in
include/coda.h).  `ops` wraps each C entry point for torch device tensors;
`inputs` builds the seeded synthetic workloads.  Importing the package loads
nothing native; the first call into `ops` loads the library and raises if it
has not been built.
"""

__all__ = ["inputs", "ops", "build"]
