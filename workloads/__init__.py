"""Seeded synthetic workloads shared by the oracle-side tests and the HIP
path's tests and benchmark.  This package draws random inputs only; it holds
none of the layer's arithmetic and imports neither ``oracle`` nor the
product package."""
from .synth import (  # noqa: F401
    round_to,
    make_projection,
    tiny_mixed,
    prefill_lora_dora,
    decoder_layer_mixed,
    vera_sweep,
    LLAMA8B_PROJECTIONS,
)
