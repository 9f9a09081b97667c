"""GPU: seeded random shapes against the f64 oracle.

Each case draws a page format (bf16, 2-8 bits), head dims (K 64/128/256; V the same or, where
the library reads it, half or double), a scale group, a block size (powers of two and others, so
both the shift and the division paths of the table lookup run), GQA shapes with REP 1-8, 1-8
query rows, 1-3 sequences of ragged lengths (at least N tokens each), and a partition size; it
checks the decode output (f32) on the stream schedule and on fixed partitions, and the matrix
engine where it reads the format; and, with draws of their own, the decode step (append of the N
new rows at their block-table slots, then attend): f32 and bf16 outputs and every pool row read
back against the oracle.  The draws are fixed by the case number, so a failure names a
reproducible case."""
import numpy as np
import pytest
import torch

import decode_attention_paged_split_amd as kvq
from oracle import attention
from tests import gpu_util as G
from workloads import make_workload

pytestmark = pytest.mark.gpu

NCASES = 128


def _draw(case: int, base: int = 2026):
    r = np.random.default_rng(np.random.SeedSequence([base, case]))
    while True:
        bits = int(r.choice([16, 8, 6, 5, 4, 3, 2]))
        D = int(r.choice([64, 128, 256]))
        if (D * bits // 8) % 16:
            continue
        group = 64 if bits == 16 else int(r.choice([g for g in (32, 64, 128) if D % g == 0]))
        DV = D
        if bits in (16, 8, 4, 2) and group == 64 and r.random() < 0.3:
            DV = int(r.choice([d for d in (D // 2, 2 * D) if 64 <= d <= 256]))
        HK = int(r.integers(1, 4))
        REP = int(r.choice([1, 2, 3, 4, 5, 8]))
        N = int(r.integers(1, 9))
        BS = int(r.choice([8, 16, 24, 32, 48, 64]))
        B = int(r.integers(1, 4))
        lo = int(r.integers(N, 200))
        hi = int(r.integers(lo, 700))
        pt = int(r.choice([32, 64, 100, 256]))
        return dict(bits=bits, D=D, DV=DV, group=group, HK=HK, HQ=HK * REP, N=N, BS=BS, B=B,
                    len_lo=lo, len_hi=hi), pt


@pytest.mark.parametrize("case", range(NCASES))
def test_random_shape(case):
    shape, pt = _draw(case)
    print(f"random case {case}: {shape} pt={pt}", flush=True)
    w = make_workload("c3", **shape)
    ref = attention.workload_output(w)
    pool = G.new_pool(w)
    G.fill_pool(w, pool)
    for p in (kvq.PARTITION_STREAM, pt):
        G.check_f32(G.run_decode(w, pool, partition_tokens=p), ref, tag=f"case {case} {shape} pt={p}")
    if _matrix_ok(shape):
        G.check_f32(G.run_decode(w, pool, engine=kvq.ENGINE_MATRIX), ref, tag=f"case {case} matrix engine")
    pool.close()


NSTEP = 64


def _matrix_ok(shape):
    return shape["bits"] == 4 and shape["group"] == 64 and shape["D"] in (128, 256) and shape["DV"] == shape["D"]


@pytest.mark.parametrize("case", range(NSTEP))
def test_random_decode_step(case):
    shape, pt = _draw(case, base=31337)
    engine = kvq.ENGINE_MATRIX if (_matrix_ok(shape) and case % 2) else kvq.ENGINE_VECTOR
    part = pt if (engine == kvq.ENGINE_VECTOR and case % 3 == 0) else kvq.PARTITION_AUTO
    print(f"random step case {case}: {shape} engine={engine} pt={part}", flush=True)
    w = make_workload("c3", **shape)
    ref = attention.workload_output(w)
    pool = G.new_pool(w)
    kn, vn = [], []
    for b in range(w.B):
        k, v = w.kv(b)
        L = int(w.lengths[b])
        if L > w.N:
            pool.append(G.u16_dev(k[: L - w.N]), G.u16_dev(v[: L - w.N]), G.i64_dev(w.slots(b, 0, L - w.N)))
        kn.append(k[L - w.N:]), vn.append(v[L - w.N:])
    out = kvq.decode_step(G.u16_dev(w.q_bits), G.u16_dev(np.stack(kn)), G.u16_dev(np.stack(vn)), pool,
                          G.i32_dev(w.table), G.i32_dev(w.lengths), w.scale, w.max_len, out_f32=True,
                          engine=engine, partition_tokens=part)
    torch.cuda.synchronize()
    G.check_f32(out.cpu().numpy().astype(np.float64), ref, tag=f"step case {case} {shape}")
    G.check_bf16(G.run_decode(w, pool, out_f32=False), ref, tag=f"step case {case} bf16")
    op = attention.workload_pool(w)
    gat = kvq.gather(pool, G.i32_dev(w.table), G.i32_dev(w.lengths), w.max_len)
    torch.cuda.synchronize()
    for b in range(w.B):
        L = int(w.lengths[b])
        want = op.gather(w.table[b], L)
        for n in op.names:
            a = gat[n][b].cpu().numpy()
            a = a.view(np.uint32) if a.dtype == np.int32 else a.view(np.uint16)
            assert np.array_equal(a[:, :L], want[n]), f"step case {case} seq {b} plane {n}"
    pool.close()
