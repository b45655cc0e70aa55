"""CPU oracle for the mixed-precision quantized linear of 6Bit-Diffusion.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously-correct
numpy implementation of what the quantized-linear hot path computes.  It
exists to check the HIP library and is imported, called or executed only by
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py``.  The product path (the ``mixed_precision_quantized_act_amd``
package and its HIP library) never imports it and shares no code with it:
no kernels, headers, helpers, tables or constant generators.

Sources: the 6Bit-Diffusion pages (arXiv 2603.18742): the abstract (an
inference-time NVFP4/INT8 mixed-precision framework; a linear predictor from
a block's input-output difference; the Temporal Delta Cache), and the
captions of Figures 1-4 (relative L2 quantization error per linear; the
relative L1 distance Gamma of a block at the preceding timestep; the fit
y = alpha*x + beta per internal linear; the block updates Delta of the two
preceding timesteps).

Modules
  formats  E2M1, E4M3 and bfloat16 encode/decode from their definitions
  quant    NVFP4 and per-token INT8 activation/weight quantization, dequant
  gemm     dequantize-then-fp64 GEMM, GELU-tanh, the exact INT8 accumulators
  tdc      Gamma, the DMPQ precision rule, the Temporal Delta Cache machine

Every function states the passage it follows.  Where the pages are silent,
the reading taken is written in the function's docstring.
"""
