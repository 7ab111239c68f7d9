"""Storage and FLOP bookkeeping of the compressed cache — oracle only.

[fr §2.A "Gain"]: a factored cache stores T x R + R x H x D values per matrix
instead of T x H x D.  [es §4 "Reducción de Memoria"] / [de §4
"Speichereffizienz"]: for LLaVA-1.5-7B the per-instance cache falls from about
328 MB to about 64 MB (64.5 MB on the German page).  [es §4 "Análisis de
Sensibilidad"]: rank 64 is the best trade-off, and decompressing only 25% of
the tokens at full rank cuts decompression FLOPs by 67.5%.

The 67.5% figure is *parity unpinned*: with the reduced rank R/4 that the
French page gives as its example, 25% of tokens at full rank costs
0.25 + 0.75/4 = 43.75% of full decompression, i.e. a 56.25% cut, and no
reading of the pages found here reproduces 67.5%.
"""
from __future__ import annotations


def factored_bytes(n_tokens: int, rank: int, width: int, bytes_per: int) -> int:
    """Bytes of one factored matrix: N*r + r*W values."""
    return bytes_per * (n_tokens * rank + rank * width)


def dense_bytes(n_tokens: int, width: int, bytes_per: int) -> int:
    """Bytes of one dense N x W matrix."""
    return bytes_per * n_tokens * width


def decompression_flop_fraction(frac_full: float, r_lo: int, r: int) -> float:
    """Decompression FLOPs with frac_full of the tokens at rank r and the rest
    at r_lo, as a fraction of decompressing every token at rank r."""
    return frac_full + (1.0 - frac_full) * (r_lo / r)
