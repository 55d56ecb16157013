"""MI355X-native transformer linear layer: Y = X·Wᵀ (+ bias, optional tanh-GELU).

The compute path is ``libtlgemm.so`` (hand-written HIP kernels for gfx950
behind a C ABI, declared in ``include/tlgemm.h``).  ``tlgemm`` is its thin
Python binding; ``inputs`` draws the seeded synthetic inputs.
"""

__all__ = ["inputs", "tlgemm"]
