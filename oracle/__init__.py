"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .attention import (attend, decode, gather_context, reshape_and_cache, verify,  # noqa: F401
                        verify_varlen, widen)
from .requant import requantize_block, reshape_and_cache_int8  # noqa: F401
