"""MI355X-native DyRA layer: C-ABI library libdyra (HIP, gfx950) and its Python binding.

``structured_rank_matmul_amd.dyra`` exposes the library's entry points under
their C names; ``structured_rank_matmul_amd.synth`` draws seeded synthetic
layer workloads.  Importing the package loads nothing; the library is loaded on
first use and raises if it has not been built.
"""
__all__ = ["dyra", "synth"]
