"""Seeded synthetic workloads for the KV-cache compression path.

This package only draws inputs (keys, values, queries, hidden states, a vocab
projection) with the shapes and planted structure of the workloads the pages
describe. It holds none of the compression method's arithmetic, so both the
CPU oracle and the GPU library can consume its tensors without sharing code.
"""
from .configs import Config, CONFIGS, get_config, small_config  # noqa: F401
from .gen import make_inputs, make_policy  # noqa: F401
