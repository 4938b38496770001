"""MI355X (gfx950) routed-expert MoE layer: HIP kernels behind a C ABI
(include/moe.h) and a ctypes binding with the same names.

Importing the package loads nothing; ``binding.load()`` opens the HIP library.
"""
__all__ = ["binding", "inputs", "layer"]
