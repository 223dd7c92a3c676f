"""MI355X-native paged grouped-query decode attention.

The kernels live in ``libpa.so`` (HIP, gfx950) behind the C ABI declared in
``include/pa.h``; this package is its thin Python binding plus the seeded
synthetic workload generators used by the tests and the benchmark.
"""
from ._lib import (PAError, decode, decode_append, decode_append_quant,  # noqa: F401
                   default_split_tokens, prefill,
                   reshape_and_cache, reshape_and_cache_quant, verify, verify_varlen,
                   version, workspace_size)
