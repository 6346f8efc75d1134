"""CPU oracle for paged, varlen, relative-bias attention.

TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the HIP library and its Python
binding never do.  ``attention`` is the fp64 vectorised oracle, ``brute`` a
scalar pure-Python transcription used to pin it on tiny inputs, ``kv_cache``
the paged KV write, ``fp8`` the E4M3 KV cache (quantise at store, attention
over dequantised pages).
"""
from . import attention, brute  # noqa: F401
