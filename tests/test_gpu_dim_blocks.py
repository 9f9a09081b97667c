"""GPU: every 8-dim block of the head dim reaches the scores.

K is zero except in one block of 8 consecutive head dims (random there), so each token's score
comes from that block alone, and V is one-hot over the first 64 dims per token, so the output
lists the softmax weight of every token.  A block whose codes or q values met the wrong partner
(a wrong dim order, a scale group mixed up, an operand read before it was written) gives wrong
weights here even where a full random K averages the error away.  Both engines; for the matrix
engine at head dim 256 both kernels: GQA 8 (8 query vectors, two token blocks per MFMA) and GQA
16 (16 vectors, one block per MFMA)."""
import numpy as np
import pytest

import decode_attention_paged_split_amd as kvq
from oracle import attention
from tests import gpu_util as G
from workloads import bf16_bits_from_f32, make_workload

pytestmark = pytest.mark.gpu

L = 64 + 37                                   # a full tile and a ragged one


def _case(blk, hq, seed):
    w = make_workload("c3", B=1, len_lo=L, len_hi=L, HQ=hq)
    rng = np.random.default_rng(seed)
    K = np.zeros((L, w.HK, w.D), np.float32)
    K[:, :, 8 * blk:8 * blk + 8] = rng.standard_normal((L, w.HK, 8)) * 3.0
    V = np.zeros((L, w.HK, w.D), np.float32)
    for t in range(min(L, 64)):
        V[t, :, t] = 1.0
    V[64:, :, 64] = 1.0                       # the ragged tile's tokens share one marker dim
    k, v = bf16_bits_from_f32(K), bf16_bits_from_f32(V)
    w.kv = lambda b: (k, v)
    return w


@pytest.mark.parametrize("blk", [0, 3, 7, 8, 12, 15, 16, 23, 24, 31])
@pytest.mark.parametrize("hq,engine", [(16, kvq.ENGINE_VECTOR), (16, kvq.ENGINE_MATRIX), (32, kvq.ENGINE_MATRIX)])
def test_one_dim_block_at_a_time(blk, hq, engine):
    print(f"dim block {blk} HQ={hq} engine={engine}", flush=True)
    w = _case(blk, hq, seed=100 + blk)
    pool = G.new_pool(w)
    G.fill_pool(w, pool)
    ref = attention.workload_output(w)
    got = G.run_decode(w, pool, out_f32=True, engine=engine)
    pool.close()
    G.check_f32(got, ref, tag=f"dim block {blk} HQ={hq} engine={engine}")
