"""MI355X-native MLA decode over a paged latent KV cache.

The compute path is the HIP library ``libmla_decode.so`` (C ABI declared in
``include/mla_decode.h``); ``binding`` is its thin ctypes front end and
``workloads`` draws seeded synthetic inputs.  Importing the package loads
nothing; the library is opened on first use of ``binding``.
"""
__all__ = ["binding", "workloads"]
