"""GPU: the vector engine's balanced stream at several set costs.

Each set with tokens takes the set cost C (positions standing for a wave's change of set) ahead of
its tokens in the stream, so ranges holding a set change get fewer tokens; the kernel drops the
cost where equal lengths already give every range as many set changes.  The partial kernel and the
merge must place and find the partials alike at any C.  Checked against the oracle (f32 output, max
abs and rel L2 2e-3), with the cost forced through KVQ_SET_COST:
- ragged 4-bit GQA-8 sequences with one empty sequence, C = 0, 512 (the default) and 4096 (more
  than a range: some ranges hold only charged positions and write nothing);
- four query groups side by side (4 rows x GQA 8, 32 vectors per KV head), C = 0 and 4096, and
  with 130 short sequences (three of them empty: the stream's prefix sums cross 64-lane chunks),
  C = 0 and 512;
- equal lengths, where the cost is dropped, C = 512 and 4096;
- bf16 pages with ragged lengths, C = 0 and 4096.
Every output comes from libkvq through the C ABI."""
import os

import numpy as np
import pytest

import decode_attention_paged_split_amd as kvq
from oracle import attention
from tests import gpu_util as G
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _run(w, cost, lengths=None):
    pool = G.new_pool(w)
    G.fill_pool(w, pool)
    old = os.environ.get("KVQ_SET_COST")
    try:
        os.environ["KVQ_SET_COST"] = str(cost)
        return G.run_decode(w, pool, partition_tokens=kvq.PARTITION_STREAM, engine=kvq.ENGINE_VECTOR,
                            lengths=None if lengths is None else G.i32_dev(lengths))
    finally:
        if old is None:
            os.environ.pop("KVQ_SET_COST", None)
        else:
            os.environ["KVQ_SET_COST"] = old
        pool.close()


@pytest.mark.parametrize("cost", [0, 512, 4096])
def test_ragged_with_an_empty_sequence(cost):
    print(f"c3 heads, ragged, set cost {cost}", flush=True)
    w = make_workload("c3", B=6, len_lo=100, len_hi=3000)
    ref = attention.workload_output(w)
    lengths = w.lengths.astype(np.int32).copy()
    lengths[2] = 0
    got = _run(w, cost, lengths)
    keep = [0, 1, 3, 4, 5]
    err, rl2 = G.check_f32(got[keep], ref[keep], tag=f"set cost {cost}")
    assert np.all(got[2] == 0.0)
    print(f"  max abs {err:.2e} rel L2 {rl2:.2e}", flush=True)


@pytest.mark.parametrize("cost", [0, 4096])
def test_groups_side_by_side(cost):
    print(f"c5 shape (4 groups side by side), set cost {cost}", flush=True)
    w = make_workload("c5", B=3, len_lo=300, len_hi=2500)
    ref = attention.workload_output(w)
    err, rl2 = G.check_f32(_run(w, cost), ref, tag=f"c5 set cost {cost}")
    print(f"  max abs {err:.2e} rel L2 {rl2:.2e}", flush=True)


@pytest.mark.parametrize("cost", [0, 512])
def test_many_sequences_groups_side_by_side(cost):
    # 130 short sequences (the stream's prefix sums cross two 64-lane chunks), four query groups
    # side by side, a few sequences empty
    print(f"130 sequences, 4 groups side by side, set cost {cost}", flush=True)
    w = make_workload("c5", B=130, len_lo=40, len_hi=400, N=4, HQ=8, HK=1)
    ref = attention.workload_output(w)
    lengths = w.lengths.astype(np.int32).copy()
    empty = [0, 64, 127]
    lengths[empty] = 0
    got = _run(w, cost, lengths)
    keep = [b for b in range(w.B) if b not in empty]
    err, rl2 = G.check_f32(got[keep], ref[keep], tag=f"130 sequences, set cost {cost}")
    assert np.all(got[empty] == 0.0)
    print(f"  max abs {err:.2e} rel L2 {rl2:.2e}", flush=True)


@pytest.mark.parametrize("cost", [512, 4096])
def test_equal_lengths(cost):
    print(f"equal lengths, set cost {cost}", flush=True)
    w = make_workload("c3", B=8, len_lo=1024, len_hi=1024)
    ref = attention.workload_output(w)
    err, rl2 = G.check_f32(_run(w, cost), ref, tag=f"equal lengths, set cost {cost}")
    print(f"  max abs {err:.2e} rel L2 {rl2:.2e}", flush=True)


@pytest.mark.parametrize("cost", [0, 4096])
def test_bf16_pages(cost):
    print(f"bf16 pages, set cost {cost}", flush=True)
    w = make_workload("c2", B=5, len_lo=50, len_hi=2000)
    ref = attention.workload_output(w)
    err, rl2 = G.check_f32(_run(w, cost), ref, tag=f"bf16 set cost {cost}")
    print(f"  max abs {err:.2e} rel L2 {rl2:.2e}", flush=True)
