"""KQV KV-cache quantisation and decode attention over the compressed cache,
for AMD Instinct MI355X (gfx950).

The product is the C-ABI library ``libkvq.so`` (header ``include/kvq.h``);
``kvq`` is its Python binding (argument marshalling only) and ``synth`` makes
seeded synthetic workloads.
"""
from . import kvq  # noqa: F401
from .kvq import KVQCache, KVQError  # noqa: F401

__all__ = ["kvq", "KVQCache", "KVQError"]
