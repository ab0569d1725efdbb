"""Block-sparse attention over a paged KV cache for AMD Instinct MI355X.

Python binding of libmsa.so (C ABI in include/msa.h): every step of the
path (block scoring, top-k selection with init/local forcing, split-K
attention over the selected blocks, log-sum-exp combine, fp8 dequantisation,
the paged append of new tokens)
runs in the library's gfx950 kernels; this package only marshals arguments.
"""

from ._lib import MsaError, load  # noqa: F401
from .api import (  # noqa: F401
    MsaConfig,
    alloc_workspace,
    append_kv,
    block_score,
    blocks_from_tokens,
    decode_workspace_size,
    fp8_dequant,
    prefill_workspace_size,
    select_blocks,
    sparse_attend,
    sparse_decode,
    sparse_decode_noalloc,
    sparse_prefill,
    version,
)
