"""Seeded synthetic inputs shared by the oracle, the tests and the bench.

This package holds shapes and random draws only: no step of the decoder's
arithmetic lives here.  Both the CPU oracle and the HIP path receive the
same arrays from it and compute from them independently.
"""
from .shapes import ModelShape, Workload, WORKLOADS, shape_for, workload
from .gen import (tensor_names, tensor_shapes, make_weights, make_prompt,
                  lane_slice_weights, lane_from_full, workload_weights, N_TENSORS_PER_LAYER,
                  layer_tensors)

__all__ = ["ModelShape", "Workload", "WORKLOADS", "shape_for", "workload",
           "tensor_names", "tensor_shapes", "make_weights", "make_prompt",
           "lane_slice_weights", "lane_from_full", "workload_weights", "N_TENSORS_PER_LAYER",
           "layer_tensors"]
