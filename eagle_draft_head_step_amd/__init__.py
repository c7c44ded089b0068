"""MI355X (gfx950) EAGLE-3 draft-head hot path: one draft step, a chain of
steps, and greedy chain verification, as HIP kernels behind a C ABI
(include/eagle3.h).  This package holds the kernels' sources (csrc/), the
in-tree build (build.py) and a ctypes binding (binding.py)."""
from .binding import (ATTN_MHA, ATTN_MLA, DraftHead, Eagle3Error, greedy_accept,  # noqa: F401
                      header_symbols, lib, make_config, packed_weights_size, workspace_size)
