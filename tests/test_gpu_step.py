"""GPU: paged_decode_step (append of the step's rows with slots from the block table, then
attention) against the explicit two-call path and the f64 oracle.

For each shape the pool is filled with every cached row but the last N of each sequence; the
step then appends those N rows itself.  The pool planes must equal those written by
kv_append_quantize with host-computed slots bit for bit (the integer part), and the output must
match the oracle to the decode tolerances and paged_decode_attention on the explicitly appended
pool (bit for bit on fixed partitions and the matrix engine, to f32 rounding on the stream
schedule)."""
import numpy as np
import pytest
import torch

import decode_attention_paged_split_amd as kvq
from oracle import attention
from tests import gpu_util as G
from workloads import make_workload

pytestmark = pytest.mark.gpu

CASES = {
    "c3": dict(B=4, len_lo=300, len_hi=2100),
    "c5": dict(B=3, len_lo=500, len_hi=1500),            # N = 4 new rows per sequence
    "c2": dict(B=3, len_lo=100, len_hi=900),             # bf16 pages, blocks of 16
    "c4_2": dict(B=2, len_lo=1000, len_hi=1000),
    "c4_8": dict(B=2, len_lo=700, len_hi=900),
    "c1": dict(),
}


def _fill_all_but_new(w, pool):
    for b in range(w.B):
        k, v = w.kv(b)
        L = int(w.lengths[b])
        pool.append(G.u16_dev(k[: L - w.N]), G.u16_dev(v[: L - w.N]), G.i64_dev(w.slots(b, 0, L - w.N)))
    torch.cuda.synchronize()


def _new_rows(w):
    ks, vs = [], []
    for b in range(w.B):
        k, v = w.kv(b)
        L = int(w.lengths[b])
        ks.append(k[L - w.N: L]), vs.append(v[L - w.N: L])
    return np.stack(ks), np.stack(vs)                  # [B, N, HK, D] bf16 bits


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("pt", [kvq.PARTITION_STREAM, kvq.PARTITION_AUTO, 64])
def test_step_matches_two_call_path_and_oracle(name, pt):
    print(f"step {name} pt={pt}", flush=True)
    w = make_workload(name, **CASES[name])
    ref = attention.workload_output(w)
    kn, vn = _new_rows(w)
    a, b = G.new_pool(w), G.new_pool(w)
    _fill_all_but_new(w, a)
    _fill_all_but_new(w, b)
    # a: explicit host slots, then attention
    for s in range(w.B):
        L = int(w.lengths[s])
        a.append(G.u16_dev(kn[s]), G.u16_dev(vn[s]), G.i64_dev(w.slots(s, L - w.N, L)))
    q, table, lengths = G.u16_dev(w.q_bits), G.i32_dev(w.table), G.i32_dev(w.lengths)
    out_a = kvq.decode(q, a, table, lengths, w.scale, w.max_len, partition_tokens=pt, out_f32=True)
    # b: the fused step
    out_b = kvq.decode_step(q, G.u16_dev(kn), G.u16_dev(vn), b, table, lengths, w.scale, w.max_len,
                            partition_tokens=pt, out_f32=True)
    torch.cuda.synchronize()
    for n in a.planes:
        assert torch.equal(a.planes[n], b.planes[n]), f"plane {n} differs"
    ga, gb = out_a.cpu().numpy().astype(np.float64), out_b.cpu().numpy().astype(np.float64)
    if pt > 0:
        assert np.array_equal(ga, gb)
    else:
        assert np.abs(ga - gb).max() <= 1e-6 * np.abs(ga).max()
    G.check_f32(gb, ref, tag=f"step {name} pt={pt}")
    a.close(), b.close()


def test_step_matrix_engine():
    w = make_workload("c3", B=3, len_lo=200, len_hi=1200)
    ref = attention.workload_output(w)
    kn, vn = _new_rows(w)
    pool = G.new_pool(w)
    _fill_all_but_new(w, pool)
    out = kvq.decode_step(G.u16_dev(w.q_bits), G.u16_dev(kn), G.u16_dev(vn), pool, G.i32_dev(w.table),
                          G.i32_dev(w.lengths), w.scale, w.max_len, out_f32=True, engine=kvq.ENGINE_MATRIX)
    torch.cuda.synchronize()
    G.check_f32(out.cpu().numpy().astype(np.float64), ref, tag="step matrix")
    pool.close()


def test_step_skips_positions_outside_the_table():
    """A length above the table's capacity puts new rows past every block: they are not written,
    and the other sequences are unaffected."""
    w = make_workload("c3", B=3, len_lo=300, len_hi=900)
    ref = attention.workload_output(w)
    kn, vn = _new_rows(w)
    pool = G.new_pool(w)
    _fill_all_but_new(w, pool)
    before = {n: t.clone() for n, t in pool.planes.items()}
    lengths = w.lengths.astype(np.int32).copy()
    lengths[1] = w.max_blocks * w.BS + 50                 # beyond the table: rows skipped
    out = kvq.decode_step(G.u16_dev(w.q_bits), G.u16_dev(kn), G.u16_dev(vn), pool, G.i32_dev(w.table),
                          G.i32_dev(lengths), w.scale, w.max_len, partition_tokens=64, out_f32=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    keep = [0, 2]
    G.check_f32(got[keep], ref[keep])
    # sequence 1's new rows were not written: its blocks hold what they held before
    t = np.arange(int(w.lengths[1]) - w.N, int(w.lengths[1]))
    blk = w.table[1, t // w.BS]
    for n in pool.planes:
        assert torch.equal(pool.planes[n][blk, :, t % w.BS], before[n][blk, :, t % w.BS])
    pool.close()
