"""Seeded synthetic inputs for the Spense linear layer.

This package only *draws* inputs: Gaussian weights and activations, their
storage encodings (fp32 / bf16 / OCP e4m3fn with a per-output-channel scale)
and seeded dense-column sets.  It contains none of the layer's own arithmetic
(no 2:4 selection, no packing, no products), so both the CPU oracle and the
HIP path can be fed from it without sharing method code.
"""

from .gen import (  # noqa: F401
    DT_F32,
    DT_BF16,
    DT_FP8,
    bf16_encode,
    e4m3_encode,
    make_weight,
    make_x,
    random_dense_set,
    tail_dense_set,
)
from .workloads import WORKLOADS, LayerSpec, Workload, layer_inputs  # noqa: F401
