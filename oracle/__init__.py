"""CPU oracle for paged chunk attention with a Transformer-XL relative-position term.

TEST INFRASTRUCTURE ONLY. This package is the slow, obviously correct definition that the
HIP path is checked against. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The product path (the C-ABI library and
its Python binding in ``paged_kv_chunk_amd``) never imports, links or calls anything here,
and nothing here imports the product path.

Every function is plain numpy in float64 on host copies of the stored inputs. Converting a
stored bf16 or fp32 value to float64 is exact, so the oracle sees exactly what the kernels see.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``.
"""

from .relpos_attn import (  # noqa: F401
    DEFAULT_LAYOUT,
    paged_kv_append,
    commit_chunk,
    gather_stream,
    table_row,
    chunk_relpos_attn,
    chunked_limited_keep,
    varlen_relpos_attn,
)
from .projections import (  # noqa: F401
    linear,
    sinusoid,
    table_positions,
    rel_pos_projection,
    qkv_project,
    qkv_append,
)
