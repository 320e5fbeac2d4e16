"""Plain, slow fp64 CPU oracle for attention-based prompt-token importance.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the bench's
CPU-baseline leg may import this package.  The product library never calls it
and shares no code with it.

Parity pins for every function are listed in the ``kvs`` module docstring.
``score_ref.c`` (built by ``build_ref``) is a second, independent fp64
implementation of the window score, in plain C, that the NumPy oracle is
checked against.
"""
from .kvs import (  # noqa: F401
    bf16_to_f64,
    score,
    score_raw,
    aggregate_raw,
    head_reduce,
    pool,
    pages,
    pool_pages,
    aggregate_layers,
    delta_pages,
    gather_kv,
    cluster_priority,
    topk,
    block_select,
    block_union_pagetable,
    token_pagetable,
    HEADS_NONE,
    HEADS_GROUP_SUM,
    HEADS_GROUP_MAX,
    HEADS_ALL_SUM,
    RED_NONE,
    RED_SUM,
    RED_MAX,
    RED_MEAN,
    RED_SUM_L1,
)
