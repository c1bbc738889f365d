"""MI355X (gfx950) DSA prefill hot path: indexer -> top-k -> sparse MLA attention.

``binding`` wraps the HIP library's C ABI (include/dsa.h); ``synth`` draws the
seeded synthetic inputs; ``build`` compiles the library in-tree with hipcc.
"""
from . import binding, synth  # noqa: F401

__all__ = ["binding", "synth"]
