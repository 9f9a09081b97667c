"""GPU: the allocation-free decode step captured in a HIP graph and replayed.

paged_decode_step_noalloc exists for callers that cannot allocate, such as code under stream capture:
its workspace is the library's own device scratch and a call enqueues kernels only (no allocation,
no memset, no host synchronisation).  Here one call is captured (torch.cuda.graph, after an eager
call has taken the scratch's address) and the graph is replayed three times, with eager work of the
program's own and synchronisations between the replays; every replay's output is compared with the
eager call's (fixed partitions: bit-identical; the balanced stream: to 1e-5 relative L2) and with
the oracle (max abs / rel L2 2e-3), and the pool rows the step appends are the same after every
replay.  Both engines, through the C ABI."""
import numpy as np
import pytest
import torch

import decode_attention_paged_split_amd as kvq
from oracle import attention
from tests import gpu_util as G
from workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,over,pt,engine", [
    ("c3", dict(B=4, len_lo=400, len_hi=2500), 256, kvq.ENGINE_VECTOR),
    ("c3", dict(B=4, len_lo=400, len_hi=2500), kvq.PARTITION_STREAM, kvq.ENGINE_VECTOR),
    ("c5", dict(B=3, len_lo=500, len_hi=2000), kvq.PARTITION_AUTO, kvq.ENGINE_AUTO),
])
def test_noalloc_step_in_a_graph(name, over, pt, engine):
    print(f"graph replay {name} {over} pt={pt} engine={engine}", flush=True)
    w = make_workload(name, **over)
    ref = attention.workload_output(w)
    pool = G.new_pool(w)
    kn = np.zeros((w.B, w.N, w.HK, w.D), np.uint16)
    vn = np.zeros((w.B, w.N, w.HK, w.DV), np.uint16)
    for b in range(w.B):
        k, v = w.kv(b)
        L = int(w.lengths[b])
        pool.append(G.u16_dev(k[: L - w.N]), G.u16_dev(v[: L - w.N]), G.i64_dev(w.slots(b, 0, L - w.N)))
        kn[b], vn[b] = k[L - w.N:], v[L - w.N:]
    q, t, lens = G.u16_dev(w.q_bits), G.i32_dev(w.table), G.i32_dev(w.lengths)
    k_new, v_new = G.u16_dev(kn), G.u16_dev(vn)
    shape = kvq.make_shape(pool, w.B, w.HQ, w.N, w.table.shape[1], w.max_len, pt, True, engine)
    out = torch.empty((w.B, w.HQ, w.N, w.DV), dtype=torch.float32, device=G.DEV)
    try:
        s = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):                       # eager call: takes the scratch's address
            kvq.paged_decode_step_noalloc(q, k_new, v_new, pool, t, lens, w.scale, shape, out, stream=s)
        torch.cuda.synchronize()
        eager = out.cpu().numpy().astype(np.float64)
        planes0 = G.pool_planes_np(pool)
        G.check_f32(eager, ref, tag=f"{name} eager")

        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            kvq.paged_decode_step_noalloc(q, k_new, v_new, pool, t, lens, w.scale, shape, out, stream=s)
        torch.cuda.synchronize()
        for rep in range(3):
            out.fill_(float("nan"))
            junk = torch.randn(1 << 20, device=G.DEV) * 2.0 + 1.0     # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = out.cpu().numpy().astype(np.float64)
            del junk
            if pt > 0:
                assert np.array_equal(got, eager), f"replay {rep}: fixed partitions must repeat bit for bit"
            else:
                rl2 = np.linalg.norm(got - eager) / np.linalg.norm(eager)
                assert rl2 <= 1e-5, f"replay {rep}: rel L2 {rl2:.2e} against the eager call"
            G.check_f32(got, ref, tag=f"{name} replay {rep}")
            planes = G.pool_planes_np(pool)
            for n in planes0:
                assert np.array_equal(planes[n], planes0[n]), f"replay {rep}: pool plane {n} changed"
        del g
    finally:
        torch.cuda.synchronize()
        pool.close()
