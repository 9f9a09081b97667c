"""Decode attention, plain definition, f64 (oracle; test infrastructure only).

Pages: "@mlx-bun/inference 0.0.0-stage -> 1.0.0", diff page 50, src/kernels/attention/paged.ts.
``pagedAttentionView.attend`` names the gather -> dequantize -> stock SDPA route as the
established result the direct kernels stand in for; this module is that route written out:

* GQA: query head hq reads KV head floor(hq / (HQ / HK)) (``paged_attention_partial``:
  ``hk = hq / (HQ / HK)``).
* Several query rows: row i of N sees tokens t < length - N + i + 1, where ``length``
  already counts the N new rows (the same kernel's loop bound, and page 134's
  ``appendDecode``/``appendWindow``, which append before they build the view).
* score z_t = scale * (q . k_t); out = sum_t exp(z_t - M) v_t / sum_t exp(z_t - M) with
  M = max_t z_t: a plain two-pass softmax (first the max, then the weighted sums).

``split_merge`` is the split-K form of the same quantity, used only to pin the merge
algebra: per partition an unnormalised output o_p, its max m_p and normaliser l_p, then
out = sum_p e^(m_p - M) o_p / sum_p e^(m_p - M) l_p with M = max_p m_p, skipping empty
partitions (m_p = -inf) -- the pages' ``paged_attention_merge`` and the kvq4 merge.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

from . import bf16
from .paged import Pool, rows_dequantized


def attend_one(qv: np.ndarray, K: np.ndarray, V: np.ndarray, T: int, scale: float) -> np.ndarray:
    """One query vector against the first T rows of K [len, D] and V [len, DV] (f64); two-pass
    softmax."""
    z = scale * (K[:T] @ qv)
    M = z.max()
    p = np.exp(z - M)
    return (p @ V[:T]) / p.sum()


def decode_attention(q: np.ndarray, K: Sequence[np.ndarray], V: Sequence[np.ndarray],
                     lengths: np.ndarray, scale: float) -> np.ndarray:
    """q [B, HQ, N, D] f64; K[b] [len_b, HK, D], V[b] [len_b, HK, DV] f64 -> out [B, HQ, N, DV] f64
    (the value head dim may differ from the key's: paged.ts's DK and DV).

    One (sequence, KV head) at a time, with its REP * N query vectors as one matrix.
    """
    B, HQ, N, D = q.shape
    DV = V[0].shape[2] if len(V) else D
    out = np.zeros((B, HQ, N, DV), dtype=np.float64)
    for b in range(B):
        L = int(lengths[b])
        HK = K[b].shape[1]
        REP = HQ // HK
        for g in range(HK):
            Kg, Vg = K[b][:L, g, :], V[b][:L, g, :]
            Qg = q[b, g * REP:(g + 1) * REP].reshape(REP * N, D)
            Z = scale * (Qg @ Kg.T)                              # [REP*N, L]
            rows = np.tile(np.arange(N), REP)                    # query row of each vector
            T = (L - N + rows + 1)[:, None]
            mask = np.arange(L)[None, :] < T
            Z = np.where(mask, Z, -np.inf)
            M = Z.max(axis=1, keepdims=True)
            P = np.where(mask, np.exp(Z - M), 0.0)
            O = (P @ Vg) / P.sum(axis=1, keepdims=True)
            out[b, g * REP:(g + 1) * REP] = O.reshape(REP, N, DV)
    return out


def split_merge(qv: np.ndarray, K: np.ndarray, V: np.ndarray, T: int, scale: float,
                part: int) -> np.ndarray:
    """Split-K form of ``attend_one``: partitions of ``part`` tokens, each an online-softmax
    triple (o, m, l), merged by log-sum-exp.  f64 throughout."""
    nparts = max(1, -(-T // part))
    os_, ms, ls = [], [], []
    for p in range(nparts):
        lo, hi = p * part, min(T, (p + 1) * part)
        m, l, o = -np.inf, 0.0, np.zeros(V.shape[1])
        for t in range(lo, hi):                                  # online softmax over the partition
            z = scale * float(K[t] @ qv)
            m_new = max(m, z)
            a = np.exp(m - m_new) if m != -np.inf else 0.0
            e = np.exp(z - m_new)
            l = l * a + e
            o = o * a + e * V[t]
            m = m_new
        os_.append(o), ms.append(m), ls.append(l)
    M = max(ms)
    num, den = np.zeros(V.shape[1]), 0.0
    for o, m, l in zip(os_, ms, ls):
        if m == -np.inf:
            continue
        w = np.exp(m - M)
        num += w * o
        den += w * l
    return num / den


def q_f64(q_bits: np.ndarray) -> np.ndarray:
    return bf16.to_f64(q_bits)


def workload_kv(w, b: int):
    """Dequantized K [len, HK, D] and V [len, HK, DV] of sequence b of a workload (contiguous
    path), f64."""
    k, v = w.kv(b)
    return rows_dequantized(k, v, w.bits, w.group)


def workload_pool(w, seqs=None) -> Pool:
    """A pool filled with the rows of the chosen sequences of a workload (all by default)."""
    pool = Pool(w.num_blocks, w.HK, w.BS, w.D, w.bits, w.group, v_head_dim=w.DV)
    for b in (range(w.B) if seqs is None else seqs):
        k, v = w.kv(b)
        pool.write(k, v, w.slots(b))
    return pool


def workload_output(w, seqs=None) -> np.ndarray:
    """The decode output of a workload (or of some of its sequences), f64 [len(seqs), HQ, N, DV]."""
    seqs = list(range(w.B)) if seqs is None else list(seqs)
    q = q_f64(w.q_bits[seqs])
    K, V = [], []
    for b in seqs:
        kb, vb = workload_kv(w, b)
        K.append(kb), V.append(vb)
    return decode_attention(q, K, V, w.lengths[seqs], w.scale)
