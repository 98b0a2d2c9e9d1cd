"""Seeded synthetic inputs for the DSpark loss: the five named workloads.

This package is the only code shared by the oracle's tests and the HIP path's
tests: it draws random tensors and holds none of the loss arithmetic.
"""
from .configs import WORKLOADS, Workload, get_workload
from .synth import make_inputs, subset_blocks, to_numpy_f64
