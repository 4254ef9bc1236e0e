"""Support-aware paged alpha-entmax decode for AMD Instinct MI355X (gfx950).

The computation lives in libentmaxkv.so (hand-written HIP kernels behind the C
ABI of include/entmaxkv.h); `binding` marshals torch tensors into it and
`engine` sequences one decode step.  `workloads` draws seeded synthetic
inputs.  Importing the package does not load the library; the first call does,
and raises if it is not built.
"""
from .binding import (CacheShape, EkvError, build_page_meta, decode_step,  # noqa: F401
                      decode_workspace_bytes, entmax_decode, load_library, score_pages,
                      select_pages, status_string, step_workspace_bytes)
from .engine import PagedEntmaxDecoder  # noqa: F401
