"""Plain fp64 CPU oracle for the MiTA forward pass (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library never does, and this package never
imports the GPU library.  See ``mita_oracle.h`` for what each step computes
and which passage of the pages it follows.
"""
from .oracle import (  # noqa: F401
    ROUND_NONE,
    ROUND_F32,
    ROUND_BF16,
    build,
    lib,
    use_library,
    threads,
    round_bf16,
    window,
    pool,
    topk,
    landmark_values,
    route,
    bucket,
    output,
    route_s,
    bucket_s,
    output_s,
    forward,
    dense,
    backward,
)
