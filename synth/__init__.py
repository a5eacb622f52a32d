"""Seeded synthetic inputs shared by the oracle tests, the device tests and the
benchmark.  Holds none of the method's arithmetic: it only draws activations,
gradients and sketches with the shapes and spectra of the workloads (see
``gen`` for the recipe)."""

from .gen import (  # noqa: F401
    LayerSpec, InputSpec, Workload, single_layer, llama_block, llama_stack,
    haar, power_law, draw_input, draw_gradient, draw_isotropic_gradient, gaussian_sketch,
    to_bf16_values,
    rotation_pair, rotate_input,
)
