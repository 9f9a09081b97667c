"""GPU: paged_decode_step_noalloc (the decode step whose workspace is the library's own device
scratch) against paged_decode_step with a caller workspace, through the C ABI.

Each case runs two calls in a row on one device, the second on a smaller input (fewer, shorter
sequences), so the second call finds the first one's partials left in the scratch.  Per call, two
pools are filled alike (every cached row but each sequence's last N); the allocating step runs on
one, the allocation-free step on the other.  Then:
  * the pool planes after the step (the N new rows quantized on append) are bit-identical;
  * fixed partitions: the f32 and bf16 outputs are bit-identical (same kernels, same order);
  * automatic schedule (the balanced stream, whose f32 sums group differently from call to call):
    the two outputs agree to 1e-5 relative L2, and both meet the oracle at max abs / rel L2 2e-3.
"""
import numpy as np
import pytest
import torch

import decode_attention_paged_split_amd as kvq
from oracle import attention
from tests import gpu_util as G
from workloads import make_workload

pytestmark = pytest.mark.gpu

# (workload, first call's shape, second call's smaller shape, engine)
CASES = [
    ("c3", dict(B=6, len_lo=500, len_hi=3000), dict(B=3, len_lo=100, len_hi=900), kvq.ENGINE_AUTO),
    ("c2", dict(B=5, len_lo=300, len_hi=2000), dict(B=2, len_lo=40, len_hi=300), kvq.ENGINE_AUTO),
    ("c5", dict(B=4, len_lo=600, len_hi=2500), dict(B=2, len_lo=50, len_hi=400), kvq.ENGINE_AUTO),
    ("c3", dict(B=6, len_lo=500, len_hi=3000), dict(B=3, len_lo=100, len_hi=900), kvq.ENGINE_MATRIX),
]


def _filled(w):
    pool = G.new_pool(w)
    kn = np.zeros((w.B, w.N, w.HK, w.D), np.uint16)
    vn = np.zeros((w.B, w.N, w.HK, w.DV), np.uint16)
    for b in range(w.B):
        k, v = w.kv(b)
        L = int(w.lengths[b])
        pool.append(G.u16_dev(k[: L - w.N]), G.u16_dev(v[: L - w.N]), G.i64_dev(w.slots(b, 0, L - w.N)))
        kn[b], vn[b] = k[L - w.N:], v[L - w.N:]
    torch.cuda.synchronize()
    return pool, kn, vn


def _both(w, partition_tokens, out_f32, engine):
    """(allocating step's output, allocation-free step's output, their pools' planes)"""
    pa, kn, vn = _filled(w)
    pb, _, _ = _filled(w)
    q, t, lens = G.u16_dev(w.q_bits), G.i32_dev(w.table), G.i32_dev(w.lengths)
    k_new, v_new = G.u16_dev(kn), G.u16_dev(vn)
    shape = kvq.make_shape(pa, w.B, w.HQ, w.N, w.table.shape[1], w.max_len, partition_tokens, out_f32, engine)
    dt = torch.float32 if out_f32 else torch.bfloat16
    out_a = torch.empty((w.B, w.HQ, w.N, w.DV), dtype=dt, device=G.DEV)
    out_b = torch.full((w.B, w.HQ, w.N, w.DV), float("nan"), dtype=dt, device=G.DEV)
    ws = torch.empty(kvq.paged_decode_workspace_bytes(pa, shape), dtype=torch.uint8, device=G.DEV)
    kvq.paged_decode_step(q, k_new, v_new, pa, t, lens, w.scale, shape, ws, out_a)
    kvq.paged_decode_step_noalloc(q, k_new, v_new, pb, t, lens, w.scale, shape, out_b)
    torch.cuda.synchronize()
    planes = (G.pool_planes_np(pa), G.pool_planes_np(pb))
    pa.close(), pb.close()
    conv = (lambda o: o.cpu().numpy().astype(np.float64)) if out_f32 else \
        (lambda o: o.view(torch.int16).cpu().numpy().view(np.uint16))
    return conv(out_a), conv(out_b), planes


@pytest.mark.parametrize("name,first,second,engine", CASES)
def test_noalloc_step_matches_the_allocating_step(name, first, second, engine):
    for call, over in (("first", first), ("second", second)):
        w = make_workload(name, **over)
        print(f"noalloc {name} engine {engine} {call} call: B={w.B} max_len={w.max_len}", flush=True)
        ref = attention.workload_output(w)
        pts = [0] if engine == kvq.ENGINE_MATRIX else [0, 64]
        for pt in pts:
            a, b, (pla, plb) = _both(w, pt, True, engine)
            for n in pla:
                assert np.array_equal(pla[n], plb[n]), f"{name} {call} pt={pt}: plane {n} differs"
            if pt > 0:
                assert np.array_equal(a, b), f"{name} {call} pt={pt}: f32 outputs differ"
                a16, b16, _ = _both(w, pt, False, engine)
                assert np.array_equal(a16, b16), f"{name} {call} pt={pt}: bf16 outputs differ"
            else:
                assert np.all(np.isfinite(b))
                rel = np.linalg.norm(a - b) / np.linalg.norm(a)
                assert rel <= 1e-5, f"{name} {call}: rel L2 {rel:.2e} between the two steps"
            G.check_f32(a, ref, tag=f"{name} {call} pt={pt} allocating step")
            G.check_f32(b, ref, tag=f"{name} {call} pt={pt} allocation-free step")
