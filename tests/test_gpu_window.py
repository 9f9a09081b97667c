"""GPU: windows of more than 8 query rows per sequence (prefill chunks, speculative-verify
windows) read straight from the pages, against the f64 oracle.  Row i of N sees
t < length - N + i + 1; every block of query vectors of a KV head is one more unit of the
partial pass.  Both engines, to the decode tolerances."""
import numpy as np
import pytest
import torch

import decode_attention_paged_split_amd as kvq
from oracle import attention
from tests import gpu_util as G
from workloads import make_workload

pytestmark = pytest.mark.gpu

CASES = [
    ("c5", dict(B=2, len_lo=300, len_hi=900, N=16), kvq.ENGINE_MATRIX),     # 128 vectors per KV head
    ("c5", dict(B=2, len_lo=300, len_hi=900, N=64), kvq.ENGINE_MATRIX),     # 512 vectors per KV head
    ("c3", dict(B=2, len_lo=200, len_hi=700, N=33), kvq.ENGINE_MATRIX),     # 264 vectors: a ragged group
    ("c3", dict(B=2, len_lo=150, len_hi=500, N=24, D=128, HQ=16, HK=4), kvq.ENGINE_MATRIX),
    ("c5", dict(B=2, len_lo=300, len_hi=900, N=16), kvq.ENGINE_VECTOR),
    ("c2", dict(B=2, len_lo=100, len_hi=400, N=12), kvq.ENGINE_VECTOR),     # bf16 pages
    ("c4_2", dict(B=1, len_lo=600, len_hi=600, N=20), kvq.ENGINE_VECTOR),   # 2-bit pages
]


@pytest.mark.parametrize("name,kw,engine", CASES)
def test_window_parity(name, kw, engine):
    print(f"window {name} {kw} engine={engine}", flush=True)
    w = make_workload(name, **kw)
    ref = attention.workload_output(w)
    pool = G.new_pool(w)
    G.fill_pool(w, pool)
    got = G.run_decode(w, pool, engine=engine)
    G.check_f32(got, ref, tag=f"window {name} {kw}")
    if engine == kvq.ENGINE_VECTOR:
        got = G.run_decode(w, pool, partition_tokens=96, engine=engine)
        G.check_f32(got, ref, tag=f"window {name} {kw} pt=96")
    pool.close()


def test_window_step_appends_the_rows():
    """paged_decode_step with a 16-row window: the 16 new rows are appended at their table slots
    and attended causally."""
    w = make_workload("c5", B=2, len_lo=400, len_hi=800, N=16)
    ref = attention.workload_output(w)
    pool = G.new_pool(w)
    kn, vn = [], []
    for b in range(w.B):
        k, v = w.kv(b)
        L = int(w.lengths[b])
        pool.append(G.u16_dev(k[: L - w.N]), G.u16_dev(v[: L - w.N]), G.i64_dev(w.slots(b, 0, L - w.N)))
        kn.append(k[L - w.N:]), vn.append(v[L - w.N:])
    out = kvq.decode_step(G.u16_dev(w.q_bits), G.u16_dev(np.stack(kn)), G.u16_dev(np.stack(vn)), pool,
                          G.i32_dev(w.table), G.i32_dev(w.lengths), w.scale, w.max_len, out_f32=True,
                          engine=kvq.ENGINE_MATRIX)
    torch.cuda.synchronize()
    G.check_f32(out.cpu().numpy().astype(np.float64), ref, tag="window step")
    pool.close()
