"""MI355X (gfx950) attention over a paged KV cache: decode and prefill.

The compute lives in libpa.so (hand-written HIP kernels behind a C ABI,
declared in include/pa.h).  This package is a thin binding: it marshals torch
tensors into the library's plain descriptors and calls it.  There is no
fallback: if libpa.so is missing, every call raises.
"""

from ._lib import (  # noqa: F401
    PA_FLAG_BLOCK_ID,
    PA_FLAG_LENGTH,
    PA_FLAG_QUERY_START,
    PA_FLAG_SLOT,
    PA_NUM_FLAGS,
    LibraryMissing,
    PaError,
    lib_path,
    load,
)
from .batch import AdmittedBatch, admit_with_shared_prompt  # noqa: F401
from .ops import (  # noqa: F401
    PATH_AUTO,
    PATH_MFMA,
    PATH_VALU,
    BlockAllocator,
    BlockManager,
    PrefixCache,
    build_info,
    copy_blocks,
    decode,
    decode_noalloc,
    decode_plan,
    decode_shared_prefix,
    decode_shared_prefix_workspace_bytes,
    decode_workspace_bytes,
    prefill,
    prefill_workspace_bytes,
    reshape_and_cache,
    swap_blocks,
)
