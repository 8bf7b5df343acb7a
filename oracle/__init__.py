"""fp64 CPU oracle for SGMV.  Test infrastructure only: the GPU library never uses it."""
from .sgmv_oracle import (  # noqa: F401
    decode, round_io, segments, ptr_table, shrink, expand, lora_add, lora_add_problem,
    segments_ranked, lora_add_ranked, DecodedPool, shrink_f64, expand_f64, lora_add_f64,
)
