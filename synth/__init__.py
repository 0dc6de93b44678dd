"""Seeded synthetic inputs for the MAPL boundary codec.

This package produces *inputs only*: activations, token IDs, projector and
anchor matrices, codebooks and gradients, each from its own seeded NumPy
stream.  It holds none of the codec's arithmetic.  Both the fp64 oracle (via
the tests) and the HIP path consume the exact bits it returns.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    stream,
    gaussian,
    orthonormal_columns,
    orthonormal_rows,
    zipf_tids,
    low_rank_plus_noise,
    to_dtype,
    codec_inputs,
    rvq_codebooks,
    stream_packets,
    spel_inputs,
)
