"""MI355X (gfx950) routed mixture-of-experts FFN over low-bit block-quantised experts.

The compute path is the HIP library libstrata_moe.so (built in-tree by
`quantized_moe_expert_gemv_amd.build`); `binding` marshals torch tensors
into its C ABI.  Importing `binding` fails loudly when the library is
missing; there is no fallback implementation.
"""

import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libstrata_moe.so")


def load():
    """Import and return the binding module (raises if the library is not built)."""
    from . import binding
    return binding
