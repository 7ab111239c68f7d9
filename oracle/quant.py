"""4-bit token factors — oracle only (test infrastructure).

The pages say the method composes with 4-bit quantization of the cache, for a
further memory saving and about twice the decode speed ([es §3 "Integración
Modular"], [fr §4 "Compatibilité"], [de §3 "Kombinierbarkeit"], [de §4
"Kombination mit anderen Techniken"]).  They also note that plain quantization
struggles with outlier values ([fr §1 "Limites des solutions existantes"],
[de §1 "Ineffizienz bestehender Lösungen"]).  They give no format, so this module
states one; these are readings, not the pages' format:

  * only the token factor U (N x r, singular values folded in) is quantized;
    the r x W factor B stays at the storage precision;
  * symmetric codes in [-7, 7] with one scale per (block of 32 consecutive tokens,
    column).  A column of large values (a leading singular direction) then never
    coarsens the small ones: the outlier concern above;
  * scale = bf16 round-to-nearest-even of the float32 product
    float32(max |x|) * float32(1/7), the maximum taken over the block's tokens of
    that column; a zero maximum gives scale 0 and codes 0;
  * code = x / scale rounded to the nearest integer, ties to even.  x is a
    float32 value and the scale has 8 significant bits, so every midpoint
    (k + 1/2) * scale is exact in float32; the quotient below is formed in
    float64, whose rounding cannot move it across a midpoint it does not sit
    on (the exact quotient lies at least 2^-25 from any midpoint it does not
    equal), so the decision is the exact one;
  * the stored value is code * scale, exact in float32.

Everything here is float64 NumPy on values that are exactly float32.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32          # tokens per scale group
QMAX = 7            # codes are in [-QMAX, QMAX]


def _bf16_rne(x32: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float32 values."""
    bits = np.asarray(x32, np.float32).view(np.uint32).astype(np.int64)
    lsb = (bits >> 16) & 1
    bits = ((bits + 0x7FFF + lsb) >> 16) << 16
    return bits.astype(np.uint32).view(np.float32)


def quantize_u4(U) -> tuple[np.ndarray, np.ndarray]:
    """Codes int8 [N][r] and scales float32 [ceil(N/32)][r] of a float32 factor U."""
    U32 = np.asarray(U, dtype=np.float32)
    N, r = U32.shape
    nblk = (N + BLOCK - 1) // BLOCK
    codes = np.zeros((N, r), dtype=np.int8)
    scales = np.zeros((nblk, r), dtype=np.float32)
    inv7 = np.float32(1.0) / np.float32(QMAX)
    for j in range(nblk):
        rows = U32[j * BLOCK:(j + 1) * BLOCK]
        m = np.max(np.abs(rows), axis=0)                     # float32, exact
        s = _bf16_rne(m * inv7)                              # float32 product, then bf16
        scales[j] = s
        with np.errstate(divide="ignore", invalid="ignore"):
            t = rows.astype(np.float64) / s.astype(np.float64)
        c = np.where(s > 0, np.rint(t), 0.0)                 # rint: ties to even
        codes[j * BLOCK:(j + 1) * BLOCK] = np.clip(c, -QMAX, QMAX).astype(np.int8)
    return codes, scales


def dequant_u4(codes, scales) -> np.ndarray:
    """The stored values code * scale, float64 [N][r]."""
    codes = np.asarray(codes)
    N = codes.shape[0]
    s = np.repeat(np.asarray(scales, np.float64), BLOCK, axis=0)[:N]
    return codes.astype(np.float64) * s


def quantize_dequant_u4(U) -> np.ndarray:
    """Round-trip: the values a 4-bit cache stores for U."""
    return dequant_u4(*quantize_u4(U))
