"""CPU oracle of the Quant VideoGen KV-cache codec.

TEST INFRASTRUCTURE: a plain, slow reference written from the pages' description
of the method.  Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import it.  It shares no code with the HIP library, and the library
never calls it.

Every public function here is pinned by a ``-m "not gpu"`` test against
something other than itself (closed forms, library routines, brute force,
hand-derived fixtures under tests/golden/); no function is "parity unpinned".
"""
from .formats import bf16_round, e4m3_decode, e4m3_encode, e4m3_values, E4M3_MAX
from .rng import forgy_indices, forgy_key, shuffle_prefix, splitmix64_next
from .qvg import (CodecConfig, Encoded, assign, update, lloyd, group_quant, pack2, unpack2,
                  dequant, encode_chunk, decode_chunk, decode, rope_rotate, rtn_reconstruct, mse,
                  kv_cache_bytes, chunk_bytes, compression_ratio, bits_per_value_ratio,
                  E4M3_TABLE_HEADER, e4m3_table_exponent, store_e4m3, attention,
                  attention_tolerance, two_level_exponent)
