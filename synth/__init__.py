"""Seeded synthetic inputs for the DSA indexer + Top-K + Sparse Flash Attention path.

This package only draws random numbers and stores them in the cache formats the path
reads (fp32, bf16 bits, fp8-e4m3 codes with one fp32 scale per token, paged pools and a
block table).  It holds none of the path's arithmetic: no scoring, no selection and no
attention.  Both the CPU oracle and the HIP path consume what it produces.
"""
from .configs import Spec, WORKLOADS, workload, scaled_spec
from .generate import Inputs, make_inputs, PrologInputs, make_prolog_inputs

__all__ = ["Spec", "WORKLOADS", "workload", "scaled_spec", "Inputs", "make_inputs",
           "PrologInputs", "make_prolog_inputs"]
