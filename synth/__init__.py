"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This package only draws and lays out inputs (random values, block tables, cache lengths, the
sinusoidal positional tables that feed the attention, linear-layer weights and activations). It
contains none of the path's arithmetic and imports neither the oracle nor the HIP path.
"""

from .cohorts import (  # noqa: F401
    WORKLOADS,
    ChunkCohort,
    VarlenCohort,
    make_chunk_cohort,
    make_varlen_cohort,
    make_config,
    sinusoidal_embedding,
    relpos_projection,
    embed_distances,
    descending_table,
    column_blocked,
    column_blocked_table,
    add_blocked_table,
    key_position_tables,
    use_key_position_tables,
    linear_weights,
    activations,
)
