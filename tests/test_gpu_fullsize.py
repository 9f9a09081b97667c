"""GPU: the full-size workloads, in the launch configuration bench.py times.

Each workload is built at its full size (every sequence, every cached token), the pool filled through
the append kernel with every row but each sequence's last N, and one decode step run as the bench
runs it (paged_decode_step: the step's new rows appended at the slots the block table gives them,
the partial pass with the automatic schedule and engine, the merge; for the 4-bit head-dim-256
workloads also each engine explicitly, for the c4 shapes also 1, 16 and 256 fixed partitions per
131072-token sequence).  The oracle cannot take the whole batch in seconds, so the
check is on sampled sequences (the shortest, the longest and one seeded other; two of the four
where all four hold 131072 tokens; the first, the last and one seeded other where all hold 32768): all their outputs against the oracle (f32 output to max abs /
rel L2 2e-3, bf16 output within one bf16 ulp or 2e-3), and their pool rows -- codes, scales and
biases, read back through kv_gather_debug -- against the oracle's quantizer bit for bit."""
import concurrent.futures

import numpy as np
import pytest
import torch

import decode_attention_paged_split_amd as kvq
from oracle import attention, paged
from tests import gpu_util as G
from workloads import make_workload

pytestmark = pytest.mark.gpu

FULL = ["c2", "c3", "c4_8", "c4_2", "c5", "diag"]


def _sample(w):
    order = np.argsort(w.lengths, kind="stable")
    if w.B <= 4:                                     # 131072-token sequences: the oracle's minutes
        return sorted({int(order[0]), int(order[-1])})
    if w.lengths.min() == w.lengths.max():           # equal lengths: first, last and one seeded other
        return sorted({0, w.B - 1, int(np.random.default_rng(7).integers(1, w.B - 1))})
    rng = np.random.default_rng(7)
    picks = {int(order[0]), int(order[-1]), int(rng.integers(0, w.B))}
    return sorted(picks)


@pytest.fixture(scope="module")
def full():
    cache = {}

    def get(name):
        if name in cache:
            return cache[name]
        for old in list(cache):                     # one full pool on the device at a time
            cache.pop(old)[1].close()
        w = make_workload(name)
        pool = G.new_pool(w)
        kn = np.zeros((w.B, w.N, w.HK, w.D), np.uint16)
        vn = np.zeros_like(kn)
        with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
            for b, (k, v) in enumerate(ex.map(w.kv, range(w.B))):
                L = int(w.lengths[b])
                pool.append(G.u16_dev(k[: L - w.N]), G.u16_dev(v[: L - w.N]), G.i64_dev(w.slots(b, 0, L - w.N)))
                kn[b], vn[b] = k[L - w.N:], v[L - w.N:]
        torch.cuda.synchronize()
        cache[name] = (w, pool, kn, vn)
        print(f"  filled {name}: B={w.B} sum(len)={int(w.lengths.sum())}", flush=True)
        return cache[name]
    yield get
    for w, pool, _, _ in cache.values():
        pool.close()


def _step(w, pool, kn, vn, out_f32, engine=kvq.ENGINE_AUTO, partition_tokens=kvq.PARTITION_AUTO):
    out = kvq.decode_step(G.u16_dev(w.q_bits), G.u16_dev(kn), G.u16_dev(vn), pool, G.i32_dev(w.table),
                          G.i32_dev(w.lengths), w.scale, w.max_len, out_f32=out_f32, engine=engine,
                          partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    if out_f32:
        return out.cpu().numpy().astype(np.float64)
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("name", FULL)
def test_full_size_step_on_sampled_sequences(full, name):
    print(f"full size {name}", flush=True)
    w, pool, kn, vn = full(name)
    got = _step(w, pool, kn, vn, out_f32=True)
    bits = _step(w, pool, kn, vn, out_f32=False)      # appends the same rows again: same pool
    seqs = _sample(w)
    print(f"  steps done; oracle on sequences {seqs}", flush=True)
    ref = attention.workload_output(w, seqs=seqs)
    G.check_f32(got[seqs], ref, tag=f"{name} seqs {seqs}")
    G.check_bf16(bits[seqs], ref, tag=f"{name} seqs {seqs}")
    if w.bits == 4 and w.D == 256:
        # both engines explicitly (the automatic choice is the matrix cores for c5's 32 query
        # vectors per KV head, the vector ALU for the single-row shapes)
        for engine, label in ((kvq.ENGINE_MATRIX, "matrix"), (kvq.ENGINE_VECTOR, "vector")):
            got_e = _step(w, pool, kn, vn, out_f32=True, engine=engine)
            G.check_f32(got_e[seqs], ref, tag=f"{name} {label} engine seqs {seqs}")
    if name.startswith("c4"):
        # the c4 shapes' stated partition counts: 1, 16 and 256 partitions of a 131072-token sequence
        for pt in (131072, 8192, 512):
            got_p = _step(w, pool, kn, vn, out_f32=True, partition_tokens=pt)
            G.check_f32(got_p[seqs], ref, tag=f"{name} partitions of {pt} seqs {seqs}")

    print("  outputs match; pool rows", flush=True)
    # integer parts: the sampled sequences' rows (the N the step appended included) against the
    # oracle's quantizer, read back through kv_gather_debug
    gat = kvq.gather(pool, G.i32_dev(w.table), G.i32_dev(w.lengths), w.max_len)
    torch.cuda.synchronize()
    for b in seqs:
        L = int(w.lengths[b])
        op = paged.Pool(w.num_blocks, w.HK, w.BS, w.D, w.bits, w.group)
        k, v = w.kv(b)
        op.write(k, v, w.slots(b))
        ref_rows = op.gather(w.table[b], L)
        for n in op.names:
            a = gat[n][b].cpu().numpy()
            a = a.view(np.uint32) if a.dtype == np.int32 else a.view(np.uint16)
            bad = np.argwhere(a[:, :L] != ref_rows[n])
            assert bad.size == 0, f"{name} seq {b} plane {n}: {bad.shape[0]} entries differ, first {bad[:3].tolist()}"
        del op
    del gat
