"""MI355X-native forward pass of one top-k-routed Mixture-of-Experts layer.

The hot path lives in hand-written HIP kernels for gfx950 behind the C ABI of
``include/moe.h`` (library ``libmoe.so`` built next to this file).  The
Python side only marshals arguments: :mod:`.binding` wraps the five C entry
points under their C names, :mod:`.layer` strings them into one forward pass,
:mod:`.inputs` makes seeded synthetic workloads and :mod:`.counters` holds the
algorithmic byte and FLOP counts used for roofline reporting.

Nothing is imported eagerly, so ``import mixture_experts_layer_08_amd.inputs``
works on a machine without a GPU or without a built library.
"""

__all__ = ["binding", "layer", "inputs", "counters"]
