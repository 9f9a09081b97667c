"""Affine group quantization of K/V rows (oracle; test infrastructure only).

Pages: "@mlx-bun/inference 0.0.0-stage -> 1.0.0", diff page 134, src/state/paged/cache.ts,
class BlockPool (constructor and ``writeBlock``): affine pages hold packed codes plus one
scale and one bias per group of ``groupSize`` elements along the head dimension, and every
appended row is quantized before it is written.  The quantizer itself is MLX's
``ops.quantize``, which the pages call but do not show, so its formula is the reading
this build adopts (plain min/max affine quantization, as the workload definitions state
for 4 bits: scale = (max - min) / 15, bias = min):

1. mx, mn = max and min of the group's bf16 values (exact);
2. s32 = f32(mx - mn) / f32(2**bits - 1), IEEE f32 subtraction and division;
3. scale = s32 rounded *up* to bf16 (so that no code exceeds 2**bits - 1 after rounding);
4. bias = mn (already a bf16 value, exact; a zero minimum is stored as +0);
5. code = clamp(rint((x - bias) / scale), 0, 2**bits - 1) in f32, rint = half to even;
   a degenerate group (scale == 0) stores code 0 everywhere.

Packing: "@mlx-bun/inference 0.0.0-stage -> 1.0.0", diff page 50, paged.ts
(``paged_attention_affine_partial``) and kvq4-decode.ts (the partial kernel): element i of
a row is code ``(word[i / PACK] >> (BITS * (i % PACK))) & (2**BITS - 1)`` with
PACK = 32 / BITS, i.e. the lowest bits of a word hold its first element.  The same pages
(diff page 134, paged.ts ``directReadable``) accept widths that do not divide 32 (3, 5 and
6 bits), whose codes straddle words, but read them only through the library's dequantize and
never show their layout; the reading here is the plain extension of the rule above: a row's
codes form one little-endian bit stream, code i in bits [BITS * i, BITS * i + BITS) of the row
and bit k of the stream in bit k % 32 of word k / 32.  For widths dividing 32 this is the PACK
rule itself.

Dequantization: value = scale * code + bias, evaluated exactly here in f64 (the
product of a bf16 and an integer below 256 plus a bf16 is exact in f64); the pages'
vector kernel keeps this product in f32 without re-rounding to bf16, and so does this
build.
"""
from __future__ import annotations

import numpy as np

from . import bf16

GROUP = 64


def levels(bits: int) -> int:
    """Largest code, 2**bits - 1."""
    return (1 << bits) - 1


def quantize_codes(x_bits: np.ndarray, bits: int, group: int = GROUP):
    """Quantize bf16 rows along the last axis.

    x_bits: uint16 [..., D] bf16 patterns.
    Returns (codes uint32 [..., D] (unpacked), scale_bits uint16 [..., D/group],
    bias_bits uint16 [..., D/group]).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    D = x_bits.shape[-1]
    assert D % group == 0
    G = D // group
    x = bf16.to_f32(x_bits).reshape(x_bits.shape[:-1] + (G, group))
    mx = x.max(axis=-1)
    mn = x.min(axis=-1)
    n = np.float32(levels(bits))
    s32 = (mx - mn).astype(np.float32) / n                      # f32 sub, f32 RN division
    scale_bits = bf16.roundup(s32)
    scale = bf16.to_f32(scale_bits)
    # bias = min; a zero minimum is stored as +0 (mn + 0 in f32 turns -0 into +0), so the
    # stored bias does not depend on which of several equal minima a reduction returns
    bias = (mn + np.float32(0.0)).astype(np.float32)
    bias_bits = (bias.view(np.uint32) >> 16).astype(np.uint16)   # exact: mn is a bf16 value
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (x - bias[..., None]).astype(np.float32) / scale[..., None]
    t = np.rint(t)
    t = np.where(scale[..., None] > 0, t, np.float32(0.0))
    codes = np.clip(t, 0, n).astype(np.uint32)
    return codes.reshape(x_bits.shape), scale_bits, bias_bits


def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    """Codes uint32 [..., D] -> words uint32 [..., D * bits / 32]: the row's codes as one
    little-endian bit stream (code i in stream bits [bits * i, bits * i + bits), stream bit k
    in bit k % 32 of word k / 32)."""
    codes = np.asarray(codes, dtype=np.uint32)
    D = codes.shape[-1]
    assert (D * bits) % 32 == 0
    lead = codes.shape[:-1]
    # the stream, bit by bit: [..., D, bits], least significant bit of each code first
    stream = (codes[..., None] >> np.arange(bits, dtype=np.uint32)) & np.uint32(1)
    stream = stream.reshape(lead + (D * bits // 32, 32))
    return np.bitwise_or.reduce(stream << np.arange(32, dtype=np.uint32), axis=-1).astype(np.uint32)


def unpack(words: np.ndarray, bits: int) -> np.ndarray:
    """Words uint32 [..., W] -> codes uint32 [..., W * 32 / bits] (the inverse of pack)."""
    words = np.asarray(words, dtype=np.uint32)
    W = words.shape[-1]
    assert (W * 32) % bits == 0
    lead = words.shape[:-1]
    stream = (words[..., None] >> np.arange(32, dtype=np.uint32)) & np.uint32(1)
    stream = stream.reshape(lead + (W * 32 // bits, bits))
    return np.bitwise_or.reduce(stream << np.arange(bits, dtype=np.uint32), axis=-1).astype(np.uint32)


def quantize(x_bits: np.ndarray, bits: int, group: int = GROUP):
    """Quantize and pack: returns (words uint32 [..., W], scale_bits, bias_bits)."""
    codes, s, b = quantize_codes(x_bits, bits, group)
    return pack(codes, bits), s, b


def dequantize(words: np.ndarray, scale_bits: np.ndarray, bias_bits: np.ndarray, bits: int,
               group: int = GROUP) -> np.ndarray:
    """Exact f64 values scale * code + bias, [..., D]."""
    c = unpack(words, bits).astype(np.float64)
    D = c.shape[-1]
    G = D // group
    c = c.reshape(c.shape[:-1] + (G, group))
    s = bf16.to_f64(scale_bits)[..., None]
    b = bf16.to_f64(bias_bits)[..., None]
    return (s * c + b).reshape(c.shape[:-2] + (D,))


def bytes_per_token_head(bits: int, D: int, group: int = GROUP) -> int:
    """K + V bytes one token row of one KV head occupies (codes + bf16 scale + bf16 bias,
    or bf16 values for bits == 16): the unit of the effective-bandwidth figure."""
    if bits == 16:
        return 2 * 2 * D
    return 2 * (D * bits // 8 + 2 * 2 * (D // group))
