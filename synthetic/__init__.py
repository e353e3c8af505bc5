"""Seeded synthetic inputs for the group-shared fixed fan-in layer.

This package only draws random inputs (index sets, features, weights,
upstream gradients, sparse 0/1 labels) and rounds them to bf16.  It holds
none of the layer's arithmetic, so both the CPU oracle's tests and the HIP
path's tests and benchmark can use it without sharing method code.
"""

from .configs import WORKLOADS, Workload, get_workload  # noqa: F401
from .gen import (  # noqa: F401
    bf16_bits,
    bf16_value,
    head_tail_labels,
    kmeans_draws,
    label_embeddings,
    make_inputs,
    normal_bf16,
    sorted_subsets,
    zipf_labels,
)
