"""GPU: affine pages with scale groups of 32 and 128 head dims (the pages' PagedQuantization
carries any groupSize; 64 is the workloads' default).  Append bit-exact against the oracle,
decode against the f64 oracle on both schedules, and the decode step."""
import numpy as np
import pytest
import torch

import decode_attention_paged_split_amd as kvq
from oracle import attention, paged
from tests import gpu_util as G
from workloads import make_workload

pytestmark = pytest.mark.gpu

COMBOS = [(bits, D, group) for bits in (4, 2, 8) for D in (64, 128, 256) for group in (32, 128)
          if D % group == 0]


@pytest.mark.parametrize("bits,D,group", COMBOS)
def test_append_bit_exact_groups(bits, D, group):
    print(f"append bits={bits} D={D} group={group}", flush=True)
    w = make_workload("c3", B=3, len_lo=30, len_hi=90, BS=16, bits=bits, D=D, HK=2, HQ=4, N=1, group=group)
    pool = G.new_pool(w)
    G.fill_pool(w, pool)
    op = paged.Pool(w.num_blocks, w.HK, w.BS, w.D, w.bits, w.group)
    for b in range(w.B):
        k, v = w.kv(b)
        op.write(k, v, w.slots(b))
    got = G.pool_planes_np(pool)
    for n in op.names:
        assert np.array_equal(got[n], op.planes[n]), f"plane {n}"
    pool.close()


@pytest.mark.parametrize("bits,D,group", COMBOS)
def test_decode_groups(bits, D, group):
    print(f"decode bits={bits} D={D} group={group}", flush=True)
    w = make_workload("c5", B=2, len_lo=200, len_hi=700, bits=bits, D=D, HQ=16, HK=2, N=2, group=group)
    ref = attention.workload_output(w)
    pool = G.new_pool(w)
    G.fill_pool(w, pool)
    for pt in (kvq.PARTITION_STREAM, 96):
        got = G.run_decode(w, pool, partition_tokens=pt)
        G.check_f32(got, ref, tag=f"bits={bits} D={D} group={group} pt={pt}")
    pool.close()


def test_decode_step_group32():
    w = make_workload("c3", B=3, len_lo=300, len_hi=900, group=32)
    ref = attention.workload_output(w)
    pool = G.new_pool(w)
    kn, vn = [], []
    for b in range(w.B):
        k, v = w.kv(b)
        L = int(w.lengths[b])
        pool.append(G.u16_dev(k[: L - w.N]), G.u16_dev(v[: L - w.N]), G.i64_dev(w.slots(b, 0, L - w.N)))
        kn.append(k[L - w.N:]), vn.append(v[L - w.N:])
    out = kvq.decode_step(G.u16_dev(w.q_bits), G.u16_dev(np.stack(kn)), G.u16_dev(np.stack(vn)), pool,
                          G.i32_dev(w.table), G.i32_dev(w.lengths), w.scale, w.max_len, out_f32=True)
    torch.cuda.synchronize()
    G.check_f32(out.cpu().numpy().astype(np.float64), ref, tag="step group 32")
    pool.close()
