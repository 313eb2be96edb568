"""Seeded synthetic inputs, shared by the CPU oracle's tests and the GPU path.

This package holds no step of what the quantized linear layer computes: it
draws random numbers and stores them in the layer's storage formats, using
torch's CPU casts for bfloat16 and float8_e4m3fn.  Weight quantisation here is
the offline preparation that precedes every kernel on the pages (the
checkpoint's FP8 weights, the NVFP4 packing, "B is pre-quantized at weight
load" on the int8_matmul page); no kernel and no oracle function repeats it.
"""

from .gen import *  # noqa: F401,F403
