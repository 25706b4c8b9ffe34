"""CPU oracle for the TurboQuant packed-KV path (quantize-on-append and paged decode attention).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library, its C ABI and the
Python binding) may import, call, link or execute anything in this package.  Only the tests,
the smoke check and the CPU-baseline leg of the benchmark use it.

The oracle is plain, slow and written to be checked by eye against the pages it follows:
fp64 NumPy/SciPy, dense matrices instead of fast transforms, explicit loops where the
definition is a loop.  It shares no code with the GPU path.

Modules
-------
codebook   Lloyd-Max codebooks for one rotated coordinate (Beta-sphere and Gaussian families).
rotation   SplitMix64 sign vector and the dense randomized-Hadamard rotation matrix.
quantize   fp32 norm, nearest-centroid index, LSB-first bit packing, TQ4 page slots, dequantization.
attention  Dense decode attention over dequantized K/V with GQA, block tables and fp16 sinks.
qjl        1-bit QJL residual sketch of keys (SRHT signs + residual norm) and its estimator.

Parity pins: every function here is pinned by the CPU tests against closed forms, textbook
values, printed byte counts on the pages, or brute force.  None is left unpinned.
"""

from . import codebook, rotation, quantize, qjl, attention  # noqa: F401
