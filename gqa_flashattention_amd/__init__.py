"""MI355X-native grouped-query attention: gfx950 HIP kernels behind a C ABI.

``decode`` and ``prefill`` call ``libgqa_attn.so`` (built in-tree by
``gqa_flashattention_amd.build``); importing the package does not load it,
the first call does, and fails loudly when it is missing.
"""

from .binding import (  # noqa: F401
    GQAError,
    decode,
    decode_split_tokens,
    decode_workspace_bytes,
    lib,
    prefill,
)

__all__ = ["decode", "prefill", "decode_split_tokens", "decode_workspace_bytes", "lib",
           "GQAError"]
