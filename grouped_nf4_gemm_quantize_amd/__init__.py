"""MI355X-native grouped NF4 MoE expert GEMM.

The compute lives in a HIP shared library (``libnf4moe.so``) behind a C ABI;
:mod:`.binding` marshals PyTorch tensors into it.  :mod:`.synth` draws the
seeded synthetic layer inputs.
"""

__all__ = ["binding", "synth"]
