"""MI355X-native window step of WeDLM's Streaming Parallel Decoding.

The compute lives in a C-ABI HIP library (``libwedlm.so``, built for gfx950);
``causal_streaming_decoding_amd.wedlm`` is a thin ctypes binding over it with
the same function names. Importing this package does not load the library:
the first call does, and it raises if the library is missing.
"""

from .workloads import ALL as WORKLOADS, BY_NAME as WORKLOADS_BY_NAME, Workload  # noqa: F401
