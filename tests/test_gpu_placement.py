"""GPU: where a sequence's blocks sit in the pool does not change its output.

The same logical sequences are appended to two pools: the workload's own block placement, and
a second pool with more blocks (the extra ones never written) whose block table maps every
logical block to another physical block through a seeded permutation.  The kernels meet tokens
in logical order and only their load addresses differ, so fixed partitions and the matrix
engine (both repeat bit for bit) give bit-identical outputs, and the balanced stream agrees to
f32 rounding (its waves take tiles as they come free, so the order of its sums varies).  The pools' rows, read back through kv_gather_debug, are identical as well."""
import numpy as np
import pytest
import torch

import decode_attention_paged_split_amd as kvq
from tests import gpu_util as G
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _relocated(w, extra, seed):
    r = np.random.default_rng(seed)
    nb2 = w.num_blocks + extra
    dest = r.permutation(nb2)[: w.num_blocks]                     # old physical -> new physical
    table2 = np.where(w.table >= 0, dest[np.maximum(w.table, 0)], -1).astype(np.int32)
    pool = kvq.Pool(nb2, w.HK, w.BS, w.D, w.bits, w.group, v_head_dim=w.DV)
    for b in range(w.B):
        k, v = w.kv(b)
        t = np.arange(int(w.lengths[b]), dtype=np.int64)
        slots = table2[b, t // w.BS].astype(np.int64) * w.BS + t % w.BS
        pool.append(G.u16_dev(k), G.u16_dev(v), G.i64_dev(slots))
    torch.cuda.synchronize()
    return pool, table2


@pytest.mark.parametrize("name,bits,BS", [("c3", 4, 32), ("c3", 16, 16), ("c5", 8, 64), ("c2", 2, 32)])
def test_block_placement_does_not_change_output(name, bits, BS):
    print(f"placement {name} bits={bits} BS={BS}", flush=True)
    w = make_workload(name, B=3, len_lo=300, len_hi=1500, bits=bits, BS=BS)
    pa = G.new_pool(w)
    G.fill_pool(w, pa)
    pb, table2 = _relocated(w, extra=37, seed=11)
    try:
        t2 = G.i32_dev(table2)
        ga = kvq.gather(pa, G.i32_dev(w.table), G.i32_dev(w.lengths), w.max_len)
        gb = kvq.gather(pb, t2, G.i32_dev(w.lengths), w.max_len)
        torch.cuda.synchronize()
        assert ga.keys() == gb.keys() and len(ga) > 0
        for plane in ga:
            assert torch.equal(ga[plane], gb[plane]), f"plane {plane}"
        a = G.run_decode(w, pa, partition_tokens=96)
        b = G.run_decode(w, pb, partition_tokens=96, table=t2)
        assert np.array_equal(a, b)
        a = G.run_decode(w, pa, partition_tokens=kvq.PARTITION_STREAM)
        b = G.run_decode(w, pb, partition_tokens=kvq.PARTITION_STREAM, table=t2)
        # the stream's waves take tiles as they come free, so the two runs sum in different orders
        # and rescale at different points: f32 rounding of sums over up to max_len tokens, a few
        # ulps per sqrt(token)
        assert np.abs(a - b).max() <= 4 * 2.0 ** -24 * np.sqrt(w.max_len) * np.abs(a).max()
        if bits == 4 and w.group == 64 and w.D in (128, 256):
            a = G.run_decode(w, pa, engine=kvq.ENGINE_MATRIX)
            b = G.run_decode(w, pb, engine=kvq.ENGINE_MATRIX, table=t2)
            assert np.array_equal(a, b)
    finally:
        pa.close()
        pb.close()
