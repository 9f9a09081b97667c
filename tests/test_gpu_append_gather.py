"""GPU: quantize-on-append codes, scales and biases, and the block-table gather, bit-exact
against the oracle (integer results: one correct answer)."""
import numpy as np
import pytest
import torch

import decode_attention_paged_split_amd as kvq
from oracle import bf16, paged
from tests import gpu_util as G
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _oracle_pool(w, seqs=None):
    pool = paged.Pool(w.num_blocks, w.HK, w.BS, w.D, w.bits, w.group)
    for b in (range(w.B) if seqs is None else seqs):
        k, v = w.kv(b)
        pool.write(k, v, w.slots(b))
    return pool


def _assert_planes_equal(gpu_pool, opool, tag):
    got = G.pool_planes_np(gpu_pool)
    for n in opool.names:
        a, e = got[n], opool.planes[n]
        assert a.shape == e.shape, (tag, n)
        bad = np.argwhere(a != e)
        assert bad.size == 0, f"{tag}: plane {n} differs at {bad[:5].tolist()} ({bad.shape[0]} entries)"


@pytest.mark.parametrize("bits", [4, 8, 2, 16])
@pytest.mark.parametrize("D", [256, 128, 64])
def test_append_bit_exact(bits, D):
    print(f"append bits={bits} D={D}", flush=True)
    for wl in ("c3", "c5"):          # outlier channels; per-token norms
        w = make_workload(wl, B=3, len_lo=30, len_hi=90, BS=16, bits=bits, D=D, HK=2, HQ=4, N=1)
        pool = G.new_pool(w)
        G.fill_pool(w, pool)
        _assert_planes_equal(pool, _oracle_pool(w), f"{wl} bits={bits} D={D}")
        pool.close()


def _special_rows(D, HK=2):
    """Hand-made groups: constant (scale 0), integer ramps (exact scales), half-integer ties,
    a -0 minimum, huge and tiny magnitudes."""
    rows = []
    G_ = D // 64
    d = np.arange(64, dtype=np.float32)
    groups = [np.full(64, 0.3125, np.float32), d % 16, (d % 16) + 0.5 * (d % 2), d % 4,
              np.where(d % 2 == 0, -1.0, 1.0).astype(np.float32), np.full(64, -0.0, np.float32),
              np.concatenate([[-0.0], np.abs(np.linspace(0, 3, 63))]).astype(np.float32),
              (d - 32) * 1e4, (d - 32) * 1e-6, np.linspace(-7, 9, 64, dtype=np.float32)]
    for i in range(len(groups)):
        row = np.stack([np.concatenate([groups[(i + h + g) % len(groups)] for g in range(G_)])
                        for h in range(HK)])
        rows.append(row)
    return bf16.rne(np.stack(rows))          # [T, HK, D]


@pytest.mark.parametrize("bits", [4, 8, 2])
def test_append_special_groups_and_skipped_slots(bits):
    D, HK, BS, NB = 128, 2, 4, 8
    k = _special_rows(D, HK)
    v = k[::-1].copy()
    T = k.shape[0]
    slots = np.arange(T, dtype=np.int64) * 3 % (NB * BS)
    slots[2] = -1                                   # skipped
    slots[5] = NB * BS + 7                          # beyond the pool: skipped
    pool = kvq.Pool(NB, HK, BS, D, bits)
    pool.append(G.u16_dev(k), G.u16_dev(v), G.i64_dev(slots))
    torch.cuda.synchronize()
    op = paged.Pool(NB, HK, BS, D, bits)
    keep = (slots >= 0) & (slots < NB * BS)
    op.write(k[keep], v[keep], slots[keep])
    _assert_planes_equal(pool, op, f"special bits={bits}")
    # a second append over the same slots replaces the rows
    pool.append(G.u16_dev(v), G.u16_dev(k), G.i64_dev(slots))
    torch.cuda.synchronize()
    op.write(v[keep], k[keep], slots[keep])
    _assert_planes_equal(pool, op, f"overwrite bits={bits}")
    pool.close()


@pytest.mark.parametrize("wl,bits", [("c3", 4), ("c2", 16), ("c4_2", 2), ("c4_8", 8)])
def test_gather_bit_exact(wl, bits):
    w = make_workload(wl, B=4, len_lo=20, len_hi=150, BS=16, bits=bits, D=128, HK=2, HQ=4, N=1)
    pool = G.new_pool(w)
    G.fill_pool(w, pool)
    op = _oracle_pool(w)
    max_len = w.max_len + 5
    got = kvq.gather(pool, G.i32_dev(w.table), G.i32_dev(w.lengths), max_len)
    torch.cuda.synchronize()
    for b in range(w.B):
        L = int(w.lengths[b])
        ref = op.gather(w.table[b], L)
        for n in op.names:
            a = got[n][b].cpu().numpy()
            a = a.view(np.uint32) if a.dtype == np.int32 else a.view(np.uint16)
            assert np.array_equal(a[:, :L], ref[n]), (wl, b, n)
            assert not a[:, L:].any(), (wl, b, n, "rows past the length must be zero")
    pool.close()
