"""GPU: paged decode attention (partial + merge) against the f64 oracle.

Tolerances: the f32 output (out_f32=1) is within max abs 2e-3 and relative L2 2e-3 of the
oracle; the bf16 output is the round-to-nearest-even of the f32 output, and within rel L2 2e-3 /
max abs max(2e-3, one bf16 ulp of the reference) of the oracle.  The shapes below are the
workloads' own shapes at reduced batch and length (several partitions and a ragged tail), plus
edge cases.

Fixed partitions (partition_tokens > 0) and the matrix engine are bit-for-bit deterministic.
The vector engine's stream schedule shares each range's tiles among its waves at run time, so
which wave sums which tiles varies from call to call: its results agree to f32 rounding
(checked below), and a bf16 output may differ by one unit in the last place from the rounding
of another call's f32 output."""
import numpy as np
import pytest
import torch

import decode_attention_paged_split_amd as kvq
from oracle import attention
from tests import gpu_util as G
from workloads import make_workload

pytestmark = pytest.mark.gpu

SMALL = {
    "c1": dict(),                                                    # full size: 1 x 2048
    "c2": dict(B=3, len_lo=100, len_hi=900),
    "c3": dict(B=4, len_lo=300, len_hi=2100),
    "c4_8": dict(B=2, len_lo=3000, len_hi=3000),
    "c4_2": dict(B=2, len_lo=3000, len_hi=3000),
    "c5": dict(B=3, len_lo=500, len_hi=1500),
}


@pytest.fixture(scope="module")
def filled():
    cache = {}

    def get(name, **kw):
        key = (name, tuple(sorted(kw.items())))
        if key not in cache:
            w = make_workload(name, **kw)
            pool = G.new_pool(w)
            G.fill_pool(w, pool)
            cache[key] = (w, pool, attention.workload_output(w))
        return cache[key]
    yield get
    for w, pool, _ in cache.values():
        pool.close()


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("pt", [kvq.PARTITION_STREAM, kvq.PARTITION_AUTO, 64, 333, 512])
def test_decode_parity(filled, name, pt):
    print(f"decode {name} pt={pt}", flush=True)
    w, pool, ref = filled(name, **SMALL[name])
    got = G.run_decode(w, pool, partition_tokens=pt, out_f32=True)
    G.check_f32(got, ref, tag=f"{name} pt={pt}")
    bits = G.run_decode(w, pool, partition_tokens=pt, out_f32=False)
    rne = G.rne_f32_to_bf16(got)
    if pt > 0:
        assert np.array_equal(bits, rne), "bf16 output must be RNE of the f32 output"
    else:                           # one bf16 ulp (2^-7 relative at most), or a sign flip at ~0
        b, r = G.bf16_to_f64(bits), G.bf16_to_f64(rne)
        assert np.all(np.abs(b - r) <= 2.0 ** -7 * np.abs(r) + 1e-6)
    G.check_bf16(bits, ref, tag=f"{name} pt={pt}")


def test_partition_count_invariance(filled):
    """c4 shapes: 1, 16 and 256 partitions of one 3072-token sequence agree to rel L2 1e-5."""
    w, pool, ref = filled("c4_2", B=1, len_lo=3072, len_hi=3072)
    outs = [G.run_decode(w, pool, partition_tokens=pt) for pt in (3072, 192, 12)]
    for o in outs[1:]:
        assert np.linalg.norm(o - outs[0]) / np.linalg.norm(outs[0]) <= 1e-5
    G.check_f32(outs[0], ref)


def test_deterministic(filled):
    """Fixed partitions repeat bit for bit; the stream schedule repeats to f32 rounding."""
    w, pool, _ = filled("c3", **SMALL["c3"])
    a = G.run_decode(w, pool, partition_tokens=64)
    b = G.run_decode(w, pool, partition_tokens=64)
    assert np.array_equal(a, b)
    a = G.run_decode(w, pool, partition_tokens=kvq.PARTITION_STREAM)
    b = G.run_decode(w, pool, partition_tokens=kvq.PARTITION_STREAM)
    assert np.abs(a - b).max() <= 1e-6 * np.abs(a).max()


@pytest.mark.parametrize("case", [
    dict(name="c5", B=2, len_lo=4, len_hi=4),            # only the N new rows are cached
    dict(name="c3", B=3, len_lo=1, len_hi=3),            # one to three tokens
    dict(name="c3", B=2, len_lo=32, len_hi=32),          # exactly one block
    dict(name="c2", B=2, len_lo=15, len_hi=17),          # around one block of 16
    dict(name="c3", B=1, len_lo=5000, len_hi=5000, HQ=2, HK=2),      # REP 1
    dict(name="c5", B=2, len_lo=300, len_hi=700, N=8, HQ=16, HK=2),  # 8 rows x REP 8 = 64 vectors
    dict(name="c5", B=2, len_lo=300, len_hi=700, N=3, HQ=6, HK=2),   # 3 rows x REP 3
    dict(name="c2", B=2, len_lo=200, len_hi=900, D=64, HQ=8, HK=4),  # head dim 64, bf16 pages
    dict(name="c4_2", B=2, len_lo=200, len_hi=900, D=64),            # head dim 64, 2-bit
    dict(name="c4_8", B=2, len_lo=200, len_hi=900, D=256, HQ=4, HK=1),
])
def test_decode_edge_cases(filled, case):
    case = dict(case)
    name = case.pop("name")
    print(f"edge {name} {case}", flush=True)
    w, pool, ref = filled(name, **case)
    # the automatic engine (the matrix cores for 16+ query vectors per KV head on 4-bit pages), and
    # the vector engine's stream explicitly
    for pt, engine in ((kvq.PARTITION_STREAM, kvq.ENGINE_AUTO), (kvq.PARTITION_AUTO, kvq.ENGINE_AUTO),
                       (7, kvq.ENGINE_AUTO), (kvq.PARTITION_STREAM, kvq.ENGINE_VECTOR)):
        got = G.run_decode(w, pool, partition_tokens=pt, engine=engine)
        G.check_f32(got, ref, tag=f"{name} {case} pt={pt} engine={engine}")


@pytest.mark.parametrize("name", ["c2", "c3", "c4_8"])
def test_poisoned_tail_and_free_blocks_are_not_read(filled, name):
    """Rows past each length in its last block, and every block no sequence owns, are set to NaN
    (bf16 pages) or given NaN scales and biases (affine pages): the output must not change."""
    w, pool, ref = filled(name, **SMALL[name])
    clean = G.run_decode(w, pool)
    used = np.zeros((w.num_blocks, w.BS), bool)
    for b in range(w.B):
        t = np.arange(int(w.lengths[b]))
        used[w.table[b, t // w.BS], t % w.BS] = True
    extra = 3
    pp = kvq.Pool(w.num_blocks + extra, w.HK, w.BS, w.D, w.bits)
    for n, t in pool.planes.items():
        pp.planes[n][: w.num_blocks].copy_(t)
    mask = torch.from_numpy(np.concatenate([~used, np.ones((extra, w.BS), bool)])).to("cuda")
    mask = mask[:, None, :].expand(-1, w.HK, -1)
    nan_bf16 = torch.tensor(0x7FC0, dtype=torch.int16, device="cuda")
    names = ["k", "v"] if w.bits == 16 else ["k_scale", "k_bias", "v_scale", "v_bias"]
    for n in names:
        pp.planes[n].masked_fill_(mask[..., None].expand_as(pp.planes[n]), nan_bf16)
    got = G.run_decode(w, pp)
    assert np.all(np.isfinite(got))
    assert np.abs(got - clean).max() <= 1e-6 * np.abs(clean).max()
    pp.close()


def test_bad_table_entry_does_not_fault(filled):
    """A table entry out of range is clamped on the device (the result is unspecified, the
    kernel must not read outside the pool)."""
    w, pool, _ = filled("c3", **SMALL["c3"])
    table = w.table.copy()
    table[0, 0] = w.num_blocks + 1000
    table[1, 1] = -7
    got = G.run_decode(w, pool, table=G.i32_dev(table))
    assert got.shape == (w.B, w.HQ, w.N, w.D)


def test_precondition_violations_do_not_fault_or_leak(filled):
    """A zero length and a length above max_len break the documented preconditions: the kernels
    must still stay in bounds, and every other sequence's output must be unchanged."""
    w, pool, ref = filled("c3", **SMALL["c3"])
    lengths = w.lengths.astype(np.int32).copy()
    lengths[1] = 0
    lengths[2] = w.max_len + 500
    for pt in (kvq.PARTITION_STREAM, 64):
        got = G.run_decode(w, pool, partition_tokens=pt, lengths=G.i32_dev(lengths))
        keep = [0] + list(range(3, w.B))
        G.check_f32(got[keep], ref[keep], tag=f"pt={pt}")
        assert np.all(got[1] == 0)


MATRIX = {
    "c1": dict(),
    "c3": dict(B=4, len_lo=300, len_hi=2100),
    "c5": dict(B=3, len_lo=500, len_hi=1500),
    "c3_d128": dict(B=3, len_lo=100, len_hi=900, D=128, HQ=16, HK=4),
}


@pytest.mark.parametrize("name", list(MATRIX))
def test_matrix_engine_parity(filled, name):
    """The matrix-core engine (4-bit pages) against the oracle, to the same tolerances."""
    kw = dict(MATRIX[name])
    base = "c3" if name.startswith("c3") else name
    print(f"matrix {name}", flush=True)
    w, pool, ref = filled(base, **kw)
    got = G.run_decode(w, pool, out_f32=True, engine=kvq.ENGINE_MATRIX)
    G.check_f32(got, ref, tag=f"matrix {name}")
    bits = G.run_decode(w, pool, out_f32=False, engine=kvq.ENGINE_MATRIX)
    assert np.array_equal(bits, G.rne_f32_to_bf16(got))
    G.check_bf16(bits, ref, tag=f"matrix {name}")


@pytest.mark.parametrize("case", [
    dict(name="c5", B=2, len_lo=4, len_hi=4),            # only the N new rows
    dict(name="c3", B=3, len_lo=1, len_hi=3),            # one to three tokens
    dict(name="c3", B=2, len_lo=64, len_hi=64),          # exactly one tile
    dict(name="c3", B=1, len_lo=5000, len_hi=5000, HQ=2, HK=2),        # REP 1
    dict(name="c5", B=2, len_lo=300, len_hi=700, N=8, HQ=16, HK=2),    # 64 vectors: 4 waves' worth
    dict(name="c5", B=2, len_lo=300, len_hi=700, N=3, HQ=6, HK=2),     # 9 vectors, padded to 16
    dict(name="c3", B=3, len_lo=100, len_hi=300, BS=16),              # blocks of 16: tiles span blocks
])
def test_matrix_engine_edge_cases(filled, case):
    case = dict(case)
    name = case.pop("name")
    print(f"matrix edge {name} {case}", flush=True)
    w, pool, ref = filled(name, **case)
    got = G.run_decode(w, pool, engine=kvq.ENGINE_MATRIX)
    G.check_f32(got, ref, tag=f"matrix {name} {case}")


def test_matrix_engine_poison_and_bad_inputs(filled):
    w, pool, ref = filled("c3", **SMALL["c3"])
    clean = G.run_decode(w, pool, engine=kvq.ENGINE_MATRIX)
    table = w.table.copy()
    table[0, 0] = w.num_blocks + 1000
    G.run_decode(w, pool, table=G.i32_dev(table), engine=kvq.ENGINE_MATRIX)
    lengths = w.lengths.astype(np.int32).copy()
    lengths[1] = 0
    lengths[2] = w.max_len + 500
    got = G.run_decode(w, pool, lengths=G.i32_dev(lengths), engine=kvq.ENGINE_MATRIX)
    keep = [0] + list(range(3, w.B))
    assert np.array_equal(got[keep], clean[keep]) or G.check_f32(got[keep], ref[keep]) is not None
    assert np.all(got[1] == 0)
