"""GPU: many short sequences in one call (the stream walks hundreds of units per range boundary
set; the merge sees thousands of rows), against the f64 oracle on sampled sequences, both
schedules and both engines, plus the decode step."""
import numpy as np
import pytest
import torch

import decode_attention_paged_split_amd as kvq
from oracle import attention
from tests import gpu_util as G
from workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bits,D", [(4, 128), (4, 256), (16, 64), (2, 128)])
def test_many_short_sequences(bits, D):
    print(f"many sequences bits={bits} D={D}", flush=True)
    w = make_workload("c3", B=700, len_lo=1, len_hi=200, BS=16, bits=bits, D=D, HQ=8, HK=2, N=1)
    pool = G.new_pool(w)
    G.fill_pool(w, pool)
    seqs = sorted({0, 1, 2, int(np.argmin(w.lengths)), int(np.argmax(w.lengths)), 350, 698, 699})
    ref = attention.workload_output(w, seqs=seqs)
    for pt in (kvq.PARTITION_STREAM, kvq.PARTITION_AUTO, 32):
        got = G.run_decode(w, pool, partition_tokens=pt)
        G.check_f32(got[seqs], ref, tag=f"bits={bits} D={D} pt={pt}")
    if bits == 4:
        got = G.run_decode(w, pool, engine=kvq.ENGINE_MATRIX)
        G.check_f32(got[seqs], ref, tag=f"bits={bits} D={D} matrix engine")
    pool.close()


def test_many_short_sequences_decode_step():
    w = make_workload("c5", B=500, len_lo=4, len_hi=120, BS=16, D=128, HQ=16, HK=4, N=4)
    pool = G.new_pool(w)
    kn, vn = [], []
    for b in range(w.B):
        k, v = w.kv(b)
        L = int(w.lengths[b])
        if L > w.N:
            pool.append(G.u16_dev(k[: L - w.N]), G.u16_dev(v[: L - w.N]), G.i64_dev(w.slots(b, 0, L - w.N)))
        kn.append(k[L - w.N:]), vn.append(v[L - w.N:])
    seqs = sorted({0, 1, int(np.argmin(w.lengths)), int(np.argmax(w.lengths)), 250, 499})
    ref = attention.workload_output(w, seqs=seqs)
    for engine in (kvq.ENGINE_VECTOR, kvq.ENGINE_MATRIX):
        out = kvq.decode_step(G.u16_dev(w.q_bits), G.u16_dev(np.stack(kn)), G.u16_dev(np.stack(vn)), pool,
                              G.i32_dev(w.table), G.i32_dev(w.lengths), w.scale, w.max_len, out_f32=True,
                              engine=engine)
        torch.cuda.synchronize()
        G.check_f32(out.cpu().numpy().astype(np.float64)[seqs], ref, tag=f"step engine={engine}")
    pool.close()
