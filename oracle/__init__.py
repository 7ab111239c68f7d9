"""CPU oracle for compressed-KV decode attention (TEST INFRASTRUCTURE ONLY).

A plain, slow, float64 restatement of what the method computes, written from
the AttentionPack summaries ("Attention-aware Inference Optimizations for Large
Vision-Language Models with Memory-efficient Decoding", gist.science pages in
Spanish [es], French [fr] and German [de]; cited below as e.g. [fr §2.B]).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never calls it and shares no code with it: the two meet
only through the seeded input generators in
``rank_compressed_kv_ap_amd.workloads``, which hold none of the method's
arithmetic.

Modules
  jacobi      one-sided Jacobi SVD                        [es §2.A] [fr §2.A] [de §2.A]
  factorize   randomized range-finding + Jacobi core      (compression, [fr §2.A])
  decode      explicit mixed-rank decompression + softmax ([es §2.B] [fr §2.B] [de §2.B]),
              the moving-average importance selector over several steps, and
              decode over several separately factored segments plus dense tokens
  brute       the same decode in pure-Python loops        (tiny inputs only)
  quant       4-bit token factors: codes and block scales  [es §3] [fr §4] [de §3] [de §4]
  accounting  storage / FLOP bookkeeping                  [fr §2.A] [es §4] [de §4]

Every function here is pinned by ``tests/test_oracle_pins.py`` to something
other than itself (a library routine, a closed form, an exact special case,
brute force, or a number printed on the pages).  Items with no such pin are
listed as "parity unpinned" in the module that holds them.
"""
from .jacobi import jacobi_svd
from .factorize import orth_mgs2, rsvd, round_to_storage
from .decode import decode_ref, decode_ema_steps, decode_segments, select_top, band_mask, recon_error
from .accounting import factored_bytes, dense_bytes, decompression_flop_fraction
from .quant import quantize_u4, dequant_u4, quantize_dequant_u4

__all__ = [
    "jacobi_svd", "orth_mgs2", "rsvd", "round_to_storage", "decode_ref", "decode_ema_steps",
    "decode_segments",
    "select_top", "band_mask", "recon_error", "factored_bytes", "dense_bytes",
    "decompression_flop_fraction", "quantize_u4", "dequant_u4", "quantize_dequant_u4",
]
