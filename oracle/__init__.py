"""CPU oracle for MLA latent-cache decode.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything in this package: only the tests, the smoke check and the
CPU-baseline leg of the benchmark use it. The GPU path (the HIP library and
its Python binding) shares no code with it.

Everything here is plain NumPy in float64, written from the DeepSeek-V2 paper
(Chinese translation), section 2.1 "Multi-Head Latent Attention": the
non-absorbed form that up-projects the latent cache to per-head keys and
values and runs textbook softmax attention over them.
"""

from .mla import (  # noqa: F401
    attend_nonabsorbed,
    attend_absorbed,
    decode,
    decode_one,
    decode_multi,
    prefill,
    decode_heads,
    gather_rows,
    lse_merge,
    attend_split,
    cache_elements_per_token,
    mha_elements_per_token,
    gqa_equivalent_groups,
    kv_reduction_vs_gqa_model,
)
from .e4m3 import decode_e4m3, encode_e4m3, e4m3_table  # noqa: F401
from .append import append_entry, quantise_entry, rms_norm, rope, rope_with  # noqa: F401
from .query import query_path, rope_frequencies  # noqa: F401
from .output import output_projection  # noqa: F401
