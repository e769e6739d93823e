"""Seeded synthetic inputs for the decode-step token-selection path.

This package only draws inputs and lays them out in memory (queries, keys,
values, planted critical tokens, page permutations, a paged pool). It holds
none of the method's arithmetic, so both the HIP path and the fp64 oracle can
take their inputs from it without sharing any computation.
"""
from .workloads import (  # noqa: F401
    CONFIGS,
    Geometry,
    Request,
    PagedBatch,
    make_request,
    make_batch,
    page_requests,
    ar1_queries,
    workload,
    request_lengths,
)
