"""dsq: group-quantized fused-dequant GEMV/GEMM and routed MoE FFN for MI355X.

The compute lives in the HIP library ``libdsq.so`` (C ABI declared in
``include/dsq.h``); ``group_quantized_moe_dsq_amd.dsq`` is its thin ctypes
binding.  Importing this package loads nothing: the library is opened on the
first call and its absence is an error, never a fallback.
"""
