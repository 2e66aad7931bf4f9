"""CPU oracle for the generalized gated delta-rule recurrence.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark are the only code allowed to import this package. The
product path (the HIP library and its Python binding) never imports, links or
calls it, and shares no code with it.

Two parts, written independently of each other and of the HIP path:

* ``forward`` -- the plain sequential fp64 recurrence in C (``gdr_oracle.c``),
  one token at a time, OpenMP over independent (batch, head, column block)
  chains.  Source: "Recurrent Memory: Write, Erase, Decay, Read", section 05
  (unified equation), generalised with the channel-wise erase gate ``b`` and
  write gate ``w`` of the Gated DeltaNet-2 abstract.
* ``reference`` -- NumPy fp64 twins used to pin the C oracle: the same
  recurrence in operator form, the closed forms of its special settings and
  the chunkwise (WY) algebra.
* ``backward`` -- the adjoint of the token loop in NumPy fp64: gradients of
  every input given the gradients of the outputs and of the final state.
"""
from .native import KIND_CHANNEL, KIND_NONE, KIND_SCALAR, ORDER_DECAY_THEN_ERASE, \
    ORDER_ERASE_THEN_DECAY, build, forward, library_path
from . import reference
from .backward import backward

__all__ = [
    "forward", "backward", "build", "library_path", "reference", "KIND_NONE", "KIND_SCALAR",
    "KIND_CHANNEL", "ORDER_ERASE_THEN_DECAY", "ORDER_DECAY_THEN_ERASE",
]
