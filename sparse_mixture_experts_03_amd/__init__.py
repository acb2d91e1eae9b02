"""MI355X-native forward pass of a sparse Mixture-of-Experts FFN layer.

The layer runs in hand-written HIP kernels for gfx950 behind the C ABI
declared in ``include/moe.h`` (library ``libmoe.so``).  ``binding`` is the
thin Python layer over that ABI (argument marshalling only); ``synth``
draws seeded synthetic inputs.  Import them explicitly:

    from sparse_mixture_experts_03_amd import binding, synth
"""
