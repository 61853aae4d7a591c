"""CPU fp64 oracle for attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  This package is the checker of the HIP path, not part of
it: only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import it.  It shares no code with the HIP library or its Python binding (no common
kernels, headers, helpers, tables or constant generators) and imports neither.

What it computes is *exact* attention: paging only changes where a token's K/V row is
stored, online softmax and split-KV partitions are exact rewrites of the softmax, so
the oracle is the plain definition written out in float64 over NumPy arrays:

  append   write each new token's K/V row into the slot its block table names
  gather   read token t of a sequence from page table[t // P], slot t % P
  logits   z_t = scale * sum_d q_d K_t,d
  softmax  w_t = exp(z_t - max z) / sum_u exp(z_u - max z)
  output   o = sum_t w_t V_t ;  lse = max z + ln sum_t exp(z_t - max z)

The FP8 codec (fp8_e4m3) is written from the OCP 8-bit floating point definition of
E4M3, and the 4-bit codec (mxfp4) from the OCP Microscaling (MX) definition of MXFP4,
not from the pages, which only name FP8 and 4-bit KV caches.

Every function here is pinned against facts fixed outside itself by the tests in
tests/test_oracle_*.py (closed forms, invariants, a library attention routine on
small inputs, the pages' worked block-table example, torch's float8_e4m3fn cast).
"""
from .fp8_e4m3 import decode_table, encode_e4m3, decode_e4m3  # noqa: F401
from .mxfp4 import mx_encode, mx_decode, decode_fp4, scale_value  # noqa: F401
from .paged_attention import (  # noqa: F401
    new_pool, encode_rows, append, copy_pages, slot_of, gather, decode, prefill_chunk,
    attend_rows, partition_stats, lse_merge,
)
