"""GPU: a balanced stream of more than 2^31 tokens, on periodic pages.

The stream's positions, the ranges' bounds and the merge's slot arithmetic run in 64 bits.  To
exercise them past 2^31 without 2^31 distinct rows, every sequence's block table cycles through
the few pages of one period: sequence b's logical block k maps to its period's block k mod P.
The K and V rows then repeat with period P * BS tokens, and single-row attention over m whole
periods equals attention over one period exactly (each period adds the same terms to the
softmax's numerator and normaliser).  64 sequences of 2^25 + P * BS tokens each (2^31 + 2^16 in
all; 4-bit group-64 pages, head dim 64, GQA 4) are checked against the oracle on one period (f32
output, max abs and rel L2 2e-3).  The pool holds 4.2 MB, so the pass reads its rows from the
caches and takes a few tens of milliseconds.  Every output comes from libkvq through the C ABI."""
import numpy as np
import pytest
import torch

import decode_attention_paged_split_amd as kvq
from oracle import attention
from tests import gpu_util as G
from workloads import make_workload

pytestmark = pytest.mark.gpu

BS, P = 256, 4                                   # page size, pages per period


def test_stream_past_2_31_tokens():
    period = P * BS
    w = make_workload("c3", B=64, len_lo=period, len_hi=period, BS=BS, HQ=4, HK=1, D=64)
    assert np.all(w.lengths == period) and w.table.shape[1] == P
    m = (1 << 25) // period + 1                  # periods per sequence
    L = m * period
    print(f"64 x {L} tokens = {64 * L} (2^31 + {64 * L - 2 ** 31}), {m} periods of {period}", flush=True)
    assert 64 * L > 2 ** 31
    nblk = L // BS
    table = w.table[:, np.arange(nblk) % P].astype(np.int32)     # [64, nblk]: period pages, cyclic
    ref = attention.workload_output(w)                           # one period of each sequence
    pool = G.new_pool(w)
    try:
        G.fill_pool(w, pool)
        out = kvq.decode(G.u16_dev(w.q_bits), pool, G.i32_dev(table), G.i32_dev(np.full(64, L, np.int32)),
                         w.scale, L, partition_tokens=kvq.PARTITION_STREAM, out_f32=True,
                         engine=kvq.ENGINE_VECTOR)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
    finally:
        pool.close()
    err, rl2 = G.check_f32(got, ref, tag="2^31 + tokens")
    print(f"  max abs {err:.2e} rel L2 {rl2:.2e}", flush=True)
