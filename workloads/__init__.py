"""Seeded synthetic inputs for paged decode attention.

This module only draws inputs: lengths, a shuffled block table, q, and per-sequence
K/V rows rounded to bf16.  It holds none of the method's arithmetic (no quantizer,
no attention), so the CPU oracle and the HIP path can both take their inputs from it
without sharing any of the computation they are compared on.

Recipe (numpy PCG64; every stream keyed by a SeedSequence):

* ``default_rng(SeedSequence([seed, c]))`` draws, in order: lengths
  (``integers(lo, hi + 1, B)``, inclusive bounds), the block permutation over
  ``NB = sum(ceil(len_b / BS))`` physical blocks, and for the outlier workload the
  outlier channels of each KV head (``choice(D, 3, replace=False)``, head 0 first).
* sequence ``b`` takes ``perm[cum_b : cum_b + nblk_b]`` in logical order; table rows
  are padded with -1.
* q: ``default_rng(SeedSequence([seed, c, 0])).standard_normal((B, HQ, N, D), f32)``.
* sequence b: ``r = default_rng(SeedSequence([seed, c, 1 + b]))``;
  K = ``r.standard_normal((len_b, HK, D), f32)``, then V likewise (``(len_b, HK, DV)``; DV = D
  unless a V head dim of its own is asked for, and the outlier channels below DV); for the
  per-token-norm workload K factors then V factors
  ``exp(r.uniform(ln 0.5, ln 4, (len_b, HK)))`` scale each row.
* K, V and q are rounded to bf16 (round to nearest even on the f32 bit pattern).

The named workloads follow the decode shapes the pages discuss: one-row GQA decode
over a contiguous 4-bit cache with head dim 256 (also at 32k-token contexts in shuffled
pages), and paged decode over bf16 or affine-quantized pages with a shuffled block table;
``WORKLOADS`` below gives each one's shape.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import numpy as np

__all__ = ["WORKLOADS", "Workload", "make_workload", "bf16_bits_from_f32"]


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round finite f32 values to bf16 (nearest, ties to even); returns uint16 bit patterns.

    Input preparation only: the generated K/V/q are "bf16 draws".
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape of one named workload."""

    key: int            # stream key c
    bits: int           # 16 = bf16 pages; 8/4/2 = affine codes
    B: int
    HQ: int
    HK: int
    D: int
    N: int              # query rows per sequence
    BS: int             # block size (tokens)
    len_lo: int
    len_hi: int
    scale: float
    contiguous: bool = False     # one block per sequence holding the whole context
    q_prescale: float = 1.0      # exact power-of-two factor applied to the bf16 q
    outliers: int = 0            # outlier channels per KV head, scaled x8
    token_norm: bool = False     # per-(token, head) log-uniform [0.5, 4] row factor
    group: int = 64
    DV: int = 0                  # V head dim; 0 = D


WORKLOADS = {
    # contiguous 4-bit cache, 1 x 2048 tokens, GQA 8/2, D 256; q pre-scaled by 1/sqrt(256)
    "c1": Spec(1, 4, 1, 8, 2, 256, 1, 2048, 2048, 2048, 1.0, contiguous=True, q_prescale=1.0 / 16.0),
    # bf16 pages, 8 sequences of 1024..8192 tokens, block 16, GQA 32/8, D 128
    "c2": Spec(2, 16, 8, 32, 8, 128, 1, 16, 1024, 8192, 1.0 / math.sqrt(128.0)),
    # 4-bit pages, 32 sequences of 4096..32768 tokens, block 32, GQA 16/2, D 256, 3 outlier dims x8
    "c3": Spec(3, 4, 32, 16, 2, 256, 1, 32, 4096, 32768, 1.0 / 16.0, outliers=3),
    # 8-bit pages, 4 x 131072 tokens, block 16, GQA 32/8, D 128
    "c4_8": Spec(4, 8, 4, 32, 8, 128, 1, 16, 131072, 131072, 1.0 / math.sqrt(128.0)),
    # 2-bit pages, same shapes
    "c4_2": Spec(4, 2, 4, 32, 8, 128, 1, 16, 131072, 131072, 1.0 / math.sqrt(128.0)),
    # 4-bit pages, 64 sequences of 8192..32768 tokens, block 32, GQA 32/4, D 256, 4 query rows
    "c5": Spec(5, 4, 64, 32, 4, 256, 4, 32, 8192, 32768, 1.0 / 16.0, token_norm=True),
    # the one-row GQA decode shape of the contiguous 4-bit cache (GQA 8/2, D 256) at 32k-token
    # contexts: 32 sequences of 32768 tokens in shuffled 4-bit pages of 32 tokens (q unscaled,
    # softmax scale 1/16); K/V N(0,1)
    "diag": Spec(6, 4, 32, 8, 2, 256, 1, 32, 32768, 32768, 1.0 / 16.0),
}


@dataclasses.dataclass
class Workload:
    """Concrete seeded inputs.  K/V are drawn lazily per sequence (``kv(b)``)."""

    name: str
    spec: Spec
    seed: int
    bits: int
    B: int
    HQ: int
    HK: int
    D: int
    N: int
    BS: int
    group: int
    scale: float
    DV: int                      # V head dim (D unless asked otherwise)
    lengths: np.ndarray          # int64 [B]
    table: np.ndarray            # int32 [B, max_blocks], -1 padded
    num_blocks: int
    outlier_dims: Optional[np.ndarray]   # int64 [HK, k] or None
    q_bits: np.ndarray           # uint16 [B, HQ, N, D] bf16 bit patterns

    @property
    def REP(self) -> int:
        return self.HQ // self.HK

    @property
    def max_len(self) -> int:
        return int(self.lengths.max())

    @property
    def max_blocks(self) -> int:
        return int(self.table.shape[1])

    def kv_f32(self, b: int) -> Tuple[np.ndarray, np.ndarray]:
        """Unrounded f32 draws of sequence b's K [len_b, HK, D] and V [len_b, HK, DV] rows."""
        s = self.spec
        L = int(self.lengths[b])
        r = np.random.default_rng(np.random.SeedSequence([self.seed, s.key, 1 + b]))
        k = r.standard_normal((L, self.HK, self.D), dtype=np.float32)
        v = r.standard_normal((L, self.HK, self.DV), dtype=np.float32)
        if self.outlier_dims is not None:
            for h in range(self.HK):
                k[:, h, self.outlier_dims[h]] *= np.float32(8.0)
                od = self.outlier_dims[h]
                v[:, h, od[od < self.DV]] *= np.float32(8.0)
        if s.token_norm:
            lo, hi = math.log(0.5), math.log(4.0)
            kf = np.exp(r.uniform(lo, hi, (L, self.HK))).astype(np.float32)
            vf = np.exp(r.uniform(lo, hi, (L, self.HK))).astype(np.float32)
            k *= kf[:, :, None]
            v *= vf[:, :, None]
        return k, v

    def kv(self, b: int) -> Tuple[np.ndarray, np.ndarray]:
        """Sequence b's K and V rows as bf16 bit patterns, uint16 [len_b, HK, D] and [len_b, HK, DV]."""
        k, v = self.kv_f32(b)
        return bf16_bits_from_f32(k), bf16_bits_from_f32(v)

    def slots(self, b: int, start: int = 0, stop: Optional[int] = None) -> np.ndarray:
        """Pool slot (phys * BS + offset) of tokens [start, stop) of sequence b, int64."""
        stop = int(self.lengths[b]) if stop is None else stop
        t = np.arange(start, stop, dtype=np.int64)
        return self.table[b, t // self.BS].astype(np.int64) * self.BS + t % self.BS

    def attention_flops(self) -> int:
        """Multiply-add flops of one decode step's attention: 2 * (q.k + p.v) MACs, i.e.
        sum(len) * HK * 2 * REP * N * (D + DV) (every cached token meets every query vector of its
        KV head; causal masking of the last N - 1 tokens is not discounted)."""
        return int(self.lengths.sum()) * self.HK * 2 * self.REP * self.N * (self.D + self.DV)

    def effective_bytes(self) -> int:
        """K/V bytes one decode step must read: sum(len) * HK * (K + V bytes per token row)."""
        def row(d):
            return 2 * d if self.bits == 16 else d * self.bits // 8 + 2 * 2 * (d // self.group)
        per = row(self.D) + row(self.DV)
        return int(self.lengths.sum()) * self.HK * per


def make_workload(name: str, *, B: Optional[int] = None, len_lo: Optional[int] = None,
                  len_hi: Optional[int] = None, BS: Optional[int] = None, seed: int = 0,
                  bits: Optional[int] = None, N: Optional[int] = None,
                  HQ: Optional[int] = None, HK: Optional[int] = None,
                  D: Optional[int] = None, group: Optional[int] = None,
                  DV: Optional[int] = None) -> Workload:
    """Build a named workload, optionally shrunk (fewer / shorter sequences) or reshaped for
    tests (the draws depend only on the seed, the workload's key and the shapes)."""
    s = WORKLOADS[name]
    over = {k: v for k, v in dict(B=B, len_lo=len_lo, len_hi=len_hi, BS=BS, bits=bits, N=N,
                                   HQ=HQ, HK=HK, D=D, group=group, DV=DV).items() if v is not None}
    s = dataclasses.replace(s, **over)
    rng = np.random.default_rng(np.random.SeedSequence([seed, s.key]))
    lengths = rng.integers(s.len_lo, s.len_hi + 1, size=s.B).astype(np.int64)
    if s.contiguous:
        bs = int(lengths.max())
        nblk = np.ones(s.B, dtype=np.int64)
    else:
        bs = s.BS
        nblk = (lengths + bs - 1) // bs
    NB = int(nblk.sum())
    perm = rng.permutation(NB)
    max_blocks = int(nblk.max())
    table = np.full((s.B, max_blocks), -1, dtype=np.int32)
    cum = 0
    for b in range(s.B):
        table[b, : nblk[b]] = perm[cum: cum + nblk[b]]
        cum += int(nblk[b])
    outl = None
    if s.outliers:
        outl = np.stack([rng.choice(s.D, s.outliers, replace=False) for _ in range(s.HK)])
    qr = np.random.default_rng(np.random.SeedSequence([seed, s.key, 0]))
    q = qr.standard_normal((s.B, s.HQ, s.N, s.D), dtype=np.float32)
    q_bits = bf16_bits_from_f32(q)
    if s.q_prescale != 1.0:
        # exact: a power-of-two factor only moves the bf16 exponent
        q_bits = bf16_bits_from_f32(
            (q_bits.astype(np.uint32) << 16).view(np.float32) * np.float32(s.q_prescale))
    return Workload(name=name, spec=s, seed=seed, bits=s.bits, B=s.B, HQ=s.HQ, HK=s.HK, D=s.D,
                    N=s.N, BS=bs, group=s.group, scale=s.scale, DV=s.DV or s.D, lengths=lengths,
                    table=table, num_blocks=NB, outlier_dims=outl, q_bits=q_bits)
