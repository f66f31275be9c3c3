"""Seeded synthetic inputs for the per-shard ZeRO optimizer step.

This module is shared by the tests, the smoke check and the benchmark.  It
draws random numbers and describes workload shapes; it holds none of the
method's arithmetic (no shard plan, no reduction, no Adam, no rounding of
results).  Shard bounds that a generator needs are passed in by the caller.

Every tensor is produced by torch's generators from a seed derived with
splitmix64 from (workload seed, rank, step, stream), so a given call gives
the same values on every run.  Generation on a CUDA device uses torch's
device generator; the values differ from the CPU generator's, so a caller
that needs the same inputs on both sides generates once and copies.
"""

from .gen import (  # noqa: F401
    WORKLOAD_SEED,
    seed_for,
    normal,
    log_uniform_signed,
    shared_mask,
    fill_pattern,
)
from .workloads import (  # noqa: F401
    Workload,
    gpt2_small_tensors,
    llama3_8b_tensors,
    WORKLOADS,
)
