"""Block-sparse programmable attention for MI355X (gfx950).

The product is the C-ABI library ``libfa.so`` (include/fa.h).  This package holds
its HIP sources (csrc/), the build script and a thin ctypes binding.  Importing the
binding functions loads the library and fails loudly if it has not been built.
"""
from ._lib import FAError, load  # noqa: F401
from .api import (BlockMask, backward, compile_mask, create_block_mask, forward, forward_noalloc, forward_paged,  # noqa: F401
                  forward_args, forward_workspace_size, block_mask_sizes, block_mask_desc,
                  slice_block_mask, block_mask_from_indices)
