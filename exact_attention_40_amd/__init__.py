"""exact_attention_40_amd: tiled exact softmax attention for AMD Instinct MI355X (gfx950).

The computation runs in hand-written HIP kernels inside ``libexattn.so`` behind a C ABI
(``include/exattn.h``); this package is the thin Python binding over it. Importing the
package does not load the library; the first call does, and fails loudly if it is missing.
"""

from .api import (  # noqa: F401
    AttnFunction,
    attention,
    attn_bwd,
    attn_fwd,
    exattn_bwd,
    exattn_check,
    exattn_fwd,
    timing_enable,
    timing_read,
    workspace_size,
)

__version__ = "0.1.0"
