"""CPU reference (oracle) for paged MLA decode attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call, link or
execute anything in this package: only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.  It
shares no code with the HIP library (no kernels, headers, helpers, tables or
pre/post-processing); the only thing both sides consume is the seeded input
generator, which holds none of the method's arithmetic.

Modules
-------
decode    exact attention over the paged latent KV cache, fp64 (NumPy), plus a
          pure-Python brute force for tiny shapes and a merge-by-LSE of partial
          results.
metadata  integer re-derivation of the split-KV tile schedule.
fp8       exact values of an fp8 e4m3 latent cache with per-page scales.
mha       paged multi-head / grouped-query decode over separate K and V caches
          (any head sizes, h_kv dividing h_q), fp64, with its split schedule.
"""

from .decode import (  # noqa: F401
    oracle_decode,
    oracle_decode_rows,
    brute_force_decode,
    oracle_partial,
    oracle_merge,
    visible_keys,
    D_K,
    D_V,
    PAGE,
)
from .metadata import oracle_metadata, schedule_chunks  # noqa: F401
from .fp8 import decode_e4m3fn, dequantize_cache, dequantize_heads, e4m3fn_value  # noqa: F401
from .mha import brute_force_mha, oracle_mha_decode, oracle_mha_metadata, oracle_mha_rows  # noqa: F401
