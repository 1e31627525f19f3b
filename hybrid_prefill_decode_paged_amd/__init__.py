"""Fused hybrid-batch (chunked prefill + split-KV decode) paged attention for MI355X (gfx950).

The compute path is the C-ABI library ``libpod_attn.so`` built from ``csrc/``; the Python
side is argument marshalling only (``binding``) plus the seeded synthetic input generator
(``inputs``), which holds no attention arithmetic.

Importing this package loads nothing native; ``binding.load()`` does, and raises if the
library is missing.
"""

__all__ = ["binding", "inputs"]
