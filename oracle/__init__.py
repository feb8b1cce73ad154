"""CPU oracle for the Prism Attention decode hot path.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg.  The product package never imports it.
"""
from .oracle import (  # noqa: F401
    AGG_MAX,
    AGG_SUM,
    attend_unit,
    dense,
    dense_unit,
    load,
    max_threads,
    propose,
    propose_unit,
    quantize_query,
    quantize_rows,
    quantize_rows_int2,
    refine,
    refine_unit,
)
