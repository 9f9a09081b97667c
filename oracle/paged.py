"""Paged KV pool model of the oracle (test infrastructure only).

Pages: "@mlx-bun/inference 0.0.0-stage -> 1.0.0", diff page 134, src/state/paged/cache.ts:

* class BlockPool -- every plane is shaped [numBlocks, H, blockSize, width]; bf16 pages
  keep ``keys``/``values`` of width D; affine pages keep packed codes (uint32, width
  D * bits / 32) plus key/value scales and biases (bf16, width D / groupSize).  The value
  planes take the pool's ``vHeadDim`` (DV) in place of D, which defaults to D.
* ``writeBlock`` -- an appended row lands at [physical block, head, row within block].
* ``pickBlocks`` / ``gather`` -- the fetch copy: the table's blocks in logical order,
  transposed to [H, blocks * blockSize, width], then cut to the cached length.

and "@mlx-bun/inference 0.0.0-stage -> 1.0.0", diff page 50, paged.ts
(``paged_attention_partial``): token t of a sequence lives in physical block
``table[t / BS]`` at row ``t % BS``.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

from . import quant

PLANES_AFFINE = ("k", "v", "k_scale", "k_bias", "v_scale", "v_bias")
PLANES_BF16 = ("k", "v")


class Pool:
    """Planes of one layer's block pool, zero-initialised like the pages' ``ops.zeros`` pool."""

    def __init__(self, num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int,
                 bits: int, group: int = quant.GROUP, v_head_dim: Optional[int] = None):
        self.NB, self.HK, self.BS, self.D = num_blocks, num_kv_heads, block_size, head_dim
        self.DV = head_dim if v_head_dim is None else v_head_dim
        self.bits, self.group = bits, group
        shape = lambda w: (num_blocks, num_kv_heads, block_size, w)  # noqa: E731
        if bits == 16:
            self.planes: Dict[str, np.ndarray] = {
                "k": np.zeros(shape(head_dim), np.uint16), "v": np.zeros(shape(self.DV), np.uint16)}
        else:
            # the codes' bit stream of a row fills whole words for every width read here
            assert (head_dim * bits) % 32 == 0 and (self.DV * bits) % 32 == 0, "rows of whole words"
            W, G = head_dim * bits // 32, head_dim // group
            WV, GV = self.DV * bits // 32, self.DV // group
            self.planes = {
                "k": np.zeros(shape(W), np.uint32), "v": np.zeros(shape(WV), np.uint32),
                "k_scale": np.zeros(shape(G), np.uint16), "k_bias": np.zeros(shape(G), np.uint16),
                "v_scale": np.zeros(shape(GV), np.uint16), "v_bias": np.zeros(shape(GV), np.uint16)}

    @property
    def names(self):
        return PLANES_BF16 if self.bits == 16 else PLANES_AFFINE

    def write(self, k_bits: np.ndarray, v_bits: np.ndarray, slots: np.ndarray) -> None:
        """Quantize (affine pages) and store rows, K [T, HK, D] and V [T, HK, DV], at slots
        phys * BS + offset.

        Negative slots are skipped.
        """
        slots = np.asarray(slots, dtype=np.int64)
        keep = slots >= 0
        slots, k_bits, v_bits = slots[keep], k_bits[keep], v_bits[keep]
        phys, off = slots // self.BS, slots % self.BS
        if self.bits == 16:
            self.planes["k"][phys, :, off] = k_bits
            self.planes["v"][phys, :, off] = v_bits
            return
        for name, x in (("k", k_bits), ("v", v_bits)):
            words, s, b = quant.quantize(x, self.bits, self.group)
            self.planes[name][phys, :, off] = words
            self.planes[name + "_scale"][phys, :, off] = s
            self.planes[name + "_bias"][phys, :, off] = b

    def gather(self, table_row: np.ndarray, length: int) -> Dict[str, np.ndarray]:
        """The fetch copy: every plane's rows of one sequence, [HK, length, width], in token order."""
        nblk = (length + self.BS - 1) // self.BS
        idx = np.asarray(table_row[:nblk], dtype=np.int64)
        out = {}
        for name in self.names:
            took = self.planes[name][idx]                       # [nb, HK, BS, w]
            t = np.transpose(took, (1, 0, 2, 3))                # [HK, nb, BS, w]
            out[name] = t.reshape(self.HK, nblk * self.BS, -1)[:, :length]
        return out

    def dequantized(self, table_row: np.ndarray, length: int):
        """Gathered K [length, HK, D] and V [length, HK, DV] of one sequence, exact f64 values."""
        g = self.gather(table_row, length)
        if self.bits == 16:
            from . import bf16
            k = bf16.to_f64(g["k"])
            v = bf16.to_f64(g["v"])
        else:
            k = quant.dequantize(g["k"], g["k_scale"], g["k_bias"], self.bits, self.group)
            v = quant.dequantize(g["v"], g["v_scale"], g["v_bias"], self.bits, self.group)
        return np.transpose(k, (1, 0, 2)), np.transpose(v, (1, 0, 2))


def rows_dequantized(k_bits: np.ndarray, v_bits: np.ndarray, bits: int, group: int = quant.GROUP):
    """Contiguous path: quantize and dequantize one sequence's rows (K [len, HK, D], V
    [len, HK, DV]) directly (no pool), exact f64.  Equal to the paged gather of the same rows."""
    from . import bf16
    if bits == 16:
        return bf16.to_f64(k_bits), bf16.to_f64(v_bits)
    out: List[np.ndarray] = []
    for x in (k_bits, v_bits):
        w, s, b = quant.quantize(x, bits, group)
        out.append(quant.dequantize(w, s, b, bits, group))
    return out[0], out[1]
