"""fp64 CPU oracle for the shared-KV cross-attention path.

TEST INFRASTRUCTURE ONLY: imported by the tests, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py``; never by the product package.
"""
from .xattn import (  # noqa: F401
    attend_rows,
    decode_ref,
    kv_append_ref,
    kv_head_of,
    prefill_ref,
    scores,
    softmax_weights,
    visible_rows,
)
from .producer import (  # noqa: F401
    YOCOPP_LAMBDA,
    kv_combine_ref,
    kv_project_ref,
    project_append_ref,
    rmsnorm_ref,
)
from .gret import (  # noqa: F401
    GRET_CHUNK,
    gret_chunkwise_ref,
    gret_decay_matrix,
    gret_decode_ref,
    gret_parallel_ref,
    gret_prefill_ref,
    gret_recurrent_ref,
)
