"""libmoe: forward pass of one top-k routed Mixture-of-Experts FFN layer on one MI355X (gfx950).

The compute path is the HIP shared library built from ``csrc/`` (C ABI declared in
``include/moe.h``); ``libmoe`` is its thin ctypes binding.  Importing this package loads nothing;
``from sparse_mixture_experts_counting_amd import libmoe`` loads the library and raises if it has
not been built.
"""

__all__ = ["libmoe", "synth", "layer"]
