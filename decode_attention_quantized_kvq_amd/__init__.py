"""libkvq: single-query decode attention over a low-bit KV cache on MI355X.

Modules: ``kvq`` (ctypes binding of the C ABI in include/kvq.h; imports torch),
``synth`` (seeded synthetic inputs, numpy only), ``build`` (hipcc build of
libkvq.so).  Nothing is imported here so that ``synth`` stays torch-free.
"""
