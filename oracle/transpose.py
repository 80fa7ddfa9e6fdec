"""Oracle for the tied-embedding transposes (test infrastructure only).

"Unified zero-copy optimizer and transposed LM head" page, section 2.2: with
the LM head stored transposed, (768, 50304), and the input embedding as
(50304, 768), tying them needs two element-wise transposed operations in the
optimizer step: the LM head's gradient is added into the embedding's
gradient (transpose_add), and the embedding's updated weights are copied into
the LM head (transpose_copy).  Plain definitions:

    transpose_copy:  dst[j][i] = src[i][j]                    (a bit copy)
    transpose_add:   dst[j][i] = RN_fmt(dst[j][i] + src[i][j])  (one rounding)

for src [rows, cols] and dst [cols, rows], row-major, fmt fp32 or bf16.
"""

import numpy as np

from .muon import BF16, F32, bf16_bits_to_f64, f64_to_bf16_bits, round_to_bf16, round_to_f32


def transpose_copy(src) -> np.ndarray:
    """dst = src^T, every element's bits unchanged (section 2.2)."""
    src = np.asarray(src)
    rows, cols = src.shape
    out = np.empty((cols, rows), dtype=src.dtype)
    for i in range(rows):
        out[:, i] = src[i, :]
    return out


def transpose_add(dst, src, fmt: str) -> np.ndarray:
    """dst + src^T, each sum rounded once to fmt (section 2.2).

    fmt F32: float32 arrays.  fmt BF16: uint16 bf16 bit patterns.  The sum of
    two values of either format is formed in float64: exact unless the
    exponents differ by more than 29 (fp32) or 45 (bf16), and then the
    smaller term is below 1/32 of an ulp of the larger and the rounded result
    is the larger term either way, so rounding the float64 sum once gives the
    correctly rounded sum."""
    dst = np.asarray(dst)
    src_t = transpose_copy(src)
    if fmt == F32:
        s = dst.astype(np.float64) + src_t.astype(np.float64)
        return round_to_f32(s).astype(np.float32)
    if fmt == BF16:
        s = bf16_bits_to_f64(dst) + bf16_bits_to_f64(src_t)
        return f64_to_bf16_bits(round_to_bf16(s))
    raise ValueError(fmt)
