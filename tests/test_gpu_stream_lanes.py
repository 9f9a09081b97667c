"""GPU: the vector engine's stream with query groups worked side by side (lanes).

When a KV head's query vectors make several groups (REP * N above the engine's group size), the
balanced stream runs L of them side by side on one range (L = 4 when the groups come in fours, 2 in
pairs, else 1), one workgroup per group, so that each K/V row is fetched once for the set.  The
lanes' partial slots interleave per range and the merge reads them back by lane.
Checked against the oracle (f32 output, max abs and rel L2 2e-3):
- the c5 shape (4-bit, 32 query vectors per KV head: 4 groups) with the lane count forced to
  1, 2 and 4 (KVQ_STREAM_LANES), ragged lengths, one sequence given length 0 (its output zero, the others unchanged);
- group counts 2, 3 and 6 (automatic lanes 2, 1, 2) on a bf16 and a 4-bit pool;
- the matrix engine's head-dim-256 kernel (groups of 16 vectors) at 2 and 4 groups per KV head,
  lanes forced to 1, 2 and 4.
Every output comes from libkvq through the C ABI."""
import os

import numpy as np
import pytest

import decode_attention_paged_split_amd as kvq
from oracle import attention
from tests import gpu_util as G
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _run(w, lanes=None, lengths=None, engine=kvq.ENGINE_VECTOR):
    pool = G.new_pool(w)
    G.fill_pool(w, pool)
    old = os.environ.get("KVQ_STREAM_LANES")
    try:
        if lanes is not None:
            os.environ["KVQ_STREAM_LANES"] = str(lanes)
        return G.run_decode(w, pool, partition_tokens=kvq.PARTITION_STREAM, engine=engine,
                            lengths=None if lengths is None else G.i32_dev(lengths))
    finally:
        if old is None:
            os.environ.pop("KVQ_STREAM_LANES", None)
        else:
            os.environ["KVQ_STREAM_LANES"] = old
        pool.close()


@pytest.mark.parametrize("lanes", [1, 2, 4])
def test_four_groups_any_lane_count(lanes):
    print(f"c5 shape, lanes {lanes}", flush=True)
    w = make_workload("c5", B=4, len_lo=300, len_hi=2500)
    ref = attention.workload_output(w)
    lengths = w.lengths.astype(np.int32).copy()
    lengths[1] = 0                                        # an empty sequence between others
    got = _run(w, lanes, lengths)
    keep = [0, 2, 3]
    err, rl2 = G.check_f32(got[keep], ref[keep], tag=f"c5 lanes {lanes}")
    assert np.all(got[1] == 0.0)
    print(f"  max abs {err:.2e} rel L2 {rl2:.2e}", flush=True)


@pytest.mark.parametrize("name,N", [("c3", 2), ("c3", 3), ("c3", 6), ("c2", 4), ("c2", 6)])
def test_group_counts(name, N):
    # c3: REP 8, 8 vectors per group -> N groups; c2: REP 4 -> N / 2 groups
    print(f"{name} N={N}", flush=True)
    w = make_workload(name, B=3, len_lo=200, len_hi=1800, N=N)
    ref = attention.workload_output(w)
    got = _run(w)
    err, rl2 = G.check_f32(got, ref, tag=f"{name} N={N}")
    print(f"  max abs {err:.2e} rel L2 {rl2:.2e}", flush=True)


@pytest.mark.parametrize("N,lanes", [(4, 1), (4, 2), (8, 2), (8, 4)])
def test_matrix_engine_groups_side_by_side(N, lanes):
    # the matrix engine's head-dim-256 kernel takes 16 vectors per group: 4 rows x GQA 8 = 2 groups,
    # 8 rows = 4 groups
    print(f"matrix engine c5 N={N} lanes {lanes}", flush=True)
    w = make_workload("c5", B=3, len_lo=300, len_hi=2000, N=N, HQ=16, HK=2)
    ref = attention.workload_output(w)
    lengths = w.lengths.astype(np.int32).copy()
    lengths[1] = 0
    got = _run(w, lanes, lengths, engine=kvq.ENGINE_MATRIX)
    err, rl2 = G.check_f32(got[[0, 2]], ref[[0, 2]], tag=f"matrix N={N} lanes {lanes}")
    assert np.all(got[1] == 0.0)
    print(f"  max abs {err:.2e} rel L2 {rl2:.2e}", flush=True)
