"""Tree-attention speculative verification for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libspecverify.so`` (hand-written HIP);
``binding`` is a thin ctypes layer over it with the same entry-point names.
``synth`` produces seeded synthetic inputs.  Importing the package loads
nothing; ``binding.load()`` loads the library and fails loudly if it is absent.
"""
__all__ = ["binding", "synth"]
