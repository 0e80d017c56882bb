"""Seeded synthetic inputs for the quantized-attention forward path.

This package only draws random data with the shapes, dtypes, value
distributions and structure (varlen mixes, permuted page pools, sparse index
sets) of the workloads described on the pages.  It holds none of the
method's arithmetic: no quantizer, no rotation, no attention.  The same bytes
feed the CPU oracle (``oracle/``) and the HIP library (``paged_kv_amd``).

Dtype conventions of every array returned here (numpy):
  bf16 -> np.uint16 bit patterns, fp16 -> np.float16, fp8 e4m3fn -> np.uint8
  codes, int8 -> np.int8, fp32 -> np.float32, indices -> np.int32.
"""
from .configs import *  # noqa: F401,F403
