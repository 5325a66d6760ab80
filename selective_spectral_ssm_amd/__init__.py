"""MI355X-native selective spectral mixer core (ESSH): chunked prefill scan and fused decode.

The compute path is the HIP library ``libessh.so`` (C ABI declared in
``include/essh.h``); ``selective_spectral_ssm_amd.essh`` is its thin Python
binding.  Importing the package does not load the library; the first call
through the binding does, and fails loudly if it has not been built.
"""
__all__ = ["essh", "inputs", "sizes"]
