"""MI355X-native cluster attention: C-ABI HIP library and its Python binding.

``inputs`` draws seeded synthetic workloads; ``binding`` wraps the C-ABI
library (``libclusterattn.so``) built from ``csrc/`` for gfx950.
"""
__all__ = ["inputs", "binding", "build"]
