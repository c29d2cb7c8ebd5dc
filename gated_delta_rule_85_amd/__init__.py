"""Gated delta-rule linear attention forward pass for MI355X (gfx950).

The compute path is the HIP library ``libgdr.so`` built from ``csrc/`` behind
the C ABI declared in ``include/gdr.h``; ``binding`` marshals arguments to it.
Importing this package loads nothing; ``binding.lib()`` loads the library and
raises if it has not been built.
"""
__all__ = ["binding", "inputs"]
