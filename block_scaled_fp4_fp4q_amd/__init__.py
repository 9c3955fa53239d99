"""Block-scaled 4-bit quantization (NVFP4 / MXFP4 / IF4, ScaleSweep) for MI355X.

The quantizer itself lives in the HIP library ``libfp4q.so`` behind the C ABI
declared in ``include/fp4q.h``; :mod:`.binding` marshals torch tensors onto it.
"""
