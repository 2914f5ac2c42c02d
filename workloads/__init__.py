"""Seeded synthetic workloads shared by the CPU oracle tests, the GPU tests and the benchmark.

This package only *generates inputs*: random tables, weights, hidden states, target logits,
uniform variates, the Zipf ranking that picks the kept vocabulary.  It contains none of the
method's arithmetic (no softmax of its outputs, no sampling, no acceptance test), so the
oracle and the HIP path can both consume it without sharing any of the computation under test.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    Config,
    ToyTables,
    Workload,
    article_toy,
    article_toy_counts,
    bf16_round,
    counter_uniforms,
    make_workload,
    token_stream,
    toy_tables,
    zipf_ranking,
)
