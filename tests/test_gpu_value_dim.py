"""GPU: V rows of a head dim of their own (the pages' vHeadDim: paged.ts reads DK and DV, the
pool's value planes take vHeadDim).  DV = D / 2 and 2 D on bf16, 8-, 4- and 2-bit pages:
append bit-exact against the oracle's quantizer (K and V planes of different widths), decode
against the f64 oracle on both schedules with several query rows, bf16 output, and the decode
step with its pool rows read back through kv_gather_debug."""
import numpy as np
import pytest
import torch

import decode_attention_paged_split_amd as kvq
from oracle import attention, paged
from tests import gpu_util as G
from workloads import make_workload

pytestmark = pytest.mark.gpu

PAIRS = [(128, 64), (256, 128), (64, 128), (128, 256)]
COMBOS = [(bits, D, DV) for bits in (16, 8, 4, 2) for D, DV in PAIRS]


@pytest.mark.parametrize("bits,D,DV", COMBOS)
def test_append_bit_exact_value_dim(bits, D, DV):
    print(f"append bits={bits} D={D} DV={DV}", flush=True)
    w = make_workload("c3", B=3, len_lo=30, len_hi=90, BS=16, bits=bits, D=D, DV=DV, HK=2, HQ=4, N=1)
    pool = G.new_pool(w)
    G.fill_pool(w, pool)
    op = paged.Pool(w.num_blocks, w.HK, w.BS, w.D, w.bits, w.group, v_head_dim=DV)
    for b in range(w.B):
        k, v = w.kv(b)
        op.write(k, v, w.slots(b))
    got = G.pool_planes_np(pool)
    for n in op.names:
        assert got[n].shape == op.planes[n].shape, f"plane {n}"
        assert np.array_equal(got[n], op.planes[n]), f"plane {n}"
    pool.close()


@pytest.mark.parametrize("bits,D,DV", COMBOS)
def test_decode_value_dim(bits, D, DV):
    """16 query vectors per KV head (GQA 8 x 2 rows), ragged lengths of several 64-token tiles."""
    print(f"decode bits={bits} D={D} DV={DV}", flush=True)
    w = make_workload("c5", B=2, len_lo=200, len_hi=700, bits=bits, D=D, DV=DV, HQ=16, HK=2, N=2)
    ref = attention.workload_output(w)
    assert ref.shape[-1] == DV
    pool = G.new_pool(w)
    G.fill_pool(w, pool)
    for pt in (kvq.PARTITION_STREAM, 96):
        got = G.run_decode(w, pool, partition_tokens=pt)
        G.check_f32(got, ref, tag=f"bits={bits} D={D} DV={DV} pt={pt}")
    G.check_bf16(G.run_decode(w, pool, out_f32=False), ref, tag=f"bits={bits} D={D} DV={DV} bf16")
    pool.close()


@pytest.mark.parametrize("HQ,HK,N", [(4, 4, 1), (4, 2, 1), (8, 2, 1)])
@pytest.mark.parametrize("bits,D,DV", [(4, 256, 128), (16, 64, 128)])
def test_decode_value_dim_group_widths(HQ, HK, N, bits, D, DV):
    """1, 2 and 4 query vectors per KV head (query groups of every width the engine carries)."""
    print(f"decode widths HQ={HQ} HK={HK} bits={bits} D={D} DV={DV}", flush=True)
    w = make_workload("c3", B=3, len_lo=100, len_hi=400, bits=bits, D=D, DV=DV, HQ=HQ, HK=HK, N=N)
    ref = attention.workload_output(w)
    pool = G.new_pool(w)
    G.fill_pool(w, pool)
    for pt in (kvq.PARTITION_STREAM, 64):
        G.check_f32(G.run_decode(w, pool, partition_tokens=pt), ref, tag=f"HQ={HQ} HK={HK} pt={pt}")
    pool.close()


@pytest.mark.parametrize("bits,D,DV", [(4, 256, 128), (8, 128, 256), (16, 128, 64), (2, 64, 128)])
def test_decode_step_value_dim(bits, D, DV):
    """The decode step appends the new rows (K of D dims, V of DV) at their block-table slots,
    then attends; output and pool rows against the oracle."""
    print(f"step bits={bits} D={D} DV={DV}", flush=True)
    w = make_workload("c5", B=3, len_lo=150, len_hi=500, bits=bits, D=D, DV=DV, HQ=8, HK=2, N=3)
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
    G.check_f32(out.cpu().numpy().astype(np.float64), ref, tag=f"step bits={bits} D={D} DV={DV}")
    op = attention.workload_pool(w)
    gat = kvq.gather(pool, G.i32_dev(w.table), G.i32_dev(w.lengths), w.max_len)
    torch.cuda.synchronize()
    for b in range(w.B):
        L = int(w.lengths[b])
        want = op.gather(w.table[b], L)
        for n in op.names:
            a = gat[n][b].cpu().numpy()
            a = a.view(np.uint32) if a.dtype == np.int32 else a.view(np.uint16)
            assert np.array_equal(a[:, :L], want[n]), f"seq {b} plane {n}"
    pool.close()


def test_matrix_engine_rejects_value_dim():
    w = make_workload("c3", B=2, len_lo=100, len_hi=200, D=256, DV=128)
    pool = G.new_pool(w)
    with pytest.raises(kvq.KvqError, match="matrix-core"):
        G.run_decode(w, pool, engine=kvq.ENGINE_MATRIX)
    pool.close()


@pytest.mark.parametrize("bits,D,DV", [(4, 256, 128), (16, 64, 128)])
def test_window_value_dim(bits, D, DV):
    """A window of 12 rows per sequence (more than a decode step's 8) with V rows of their own
    head dim: every block of query vectors of a KV head is one more unit of the partial pass."""
    print(f"window bits={bits} D={D} DV={DV}", flush=True)
    w = make_workload("c3", B=2, len_lo=150, len_hi=400, bits=bits, D=D, DV=DV, HQ=8, HK=2, N=12)
    ref = attention.workload_output(w)
    pool = G.new_pool(w)
    G.fill_pool(w, pool)
    for pt in (kvq.PARTITION_STREAM, 128):
        G.check_f32(G.run_decode(w, pool, partition_tokens=pt), ref, tag=f"window DV={DV} pt={pt}")
    pool.close()
