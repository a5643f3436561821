"""Seeded synthetic inputs for MLA latent-cache decode.

This module only draws and lays out inputs; it holds none of the decode
arithmetic. The same bytes feed the CPU oracle and the GPU library.
"""

from .inputs import (  # noqa: F401
    Dims,
    TINY,
    DSV2,
    WORKLOADS,
    Inputs,
    make_inputs,
    oracle_args,
    rope_rotate,
    rms_normalise,
    quantise_rows_e4m3,
    AppendInputs,
    make_append_inputs,
    make_oproj_inputs,
    QueryInputs,
    make_query_inputs,
)
