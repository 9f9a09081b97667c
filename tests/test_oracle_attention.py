"""Pins of the oracle's attention, paging and merge (CPU only).

* a library routine: torch's scaled_dot_product_attention in f64 on the CPU, GQA expanded
  by repeat_interleave and an explicit bottom-right causal mask for several query rows;
* brute force with pure-Python loops on tiny inputs;
* closed forms (one visible token, equal keys, zero query);
* the split-K + log-sum-exp merge form equals the two-pass definition;
* paged == contiguous (shuffled small blocks vs one block);
* the quantized result approaches the unquantized one within a closed-form bound.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention, bf16, paged, quant
from workloads import make_workload


def _sdpa_ref(q, K, V, lengths, scale):
    """torch SDPA per sequence, f64 CPU; q [B,HQ,N,D]; K[b], V[b] [len,HK,D]."""
    B, HQ, N, D = q.shape
    outs = []
    for b in range(B):
        L = int(lengths[b])
        HK = K[b].shape[1]
        kk = torch.from_numpy(np.ascontiguousarray(K[b][:L].transpose(1, 0, 2)))[None]
        vv = torch.from_numpy(np.ascontiguousarray(V[b][:L].transpose(1, 0, 2)))[None]
        kk = kk.repeat_interleave(HQ // HK, dim=1)
        vv = vv.repeat_interleave(HQ // HK, dim=1)
        mask = torch.arange(L)[None, :] < (L - N + torch.arange(N)[:, None] + 1)
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[b:b + 1]), kk, vv, attn_mask=mask, scale=scale)
        outs.append(o[0].numpy())
    return np.stack(outs)


def _tiny(bits, B=2, HQ=4, HK=2, D=64, N=1, lens=(37, 64), seed=3, DV=None):
    rng = np.random.default_rng(seed)
    DV = D if DV is None else DV
    q = bf16.to_f64(bf16.rne(rng.standard_normal((B, HQ, N, D)).astype(np.float32)))
    K, V = [], []
    for b in range(B):
        kb = bf16.rne(rng.standard_normal((lens[b], HK, D)).astype(np.float32))
        vb = bf16.rne(rng.standard_normal((lens[b], HK, DV)).astype(np.float32))
        k, v = paged.rows_dequantized(kb, vb, bits)
        K.append(k), V.append(v)
    return q, K, V, np.array(lens)


@pytest.mark.parametrize("bits", [16, 8, 4, 2])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("N", [1, 3])
def test_matches_torch_sdpa(bits, D, N):
    q, K, V, lens = _tiny(bits, D=D, N=N, HQ=6, HK=2)
    scale = 1.0 / math.sqrt(D)
    got = attention.decode_attention(q, K, V, lens, scale)
    ref = _sdpa_ref(q, K, V, lens, scale)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("bits", [16, 4, 2])
@pytest.mark.parametrize("D,DV", [(128, 64), (64, 128), (256, 128), (128, 256)])
def test_value_head_dim_of_its_own_matches_torch_sdpa(bits, D, DV):
    """V rows narrower or wider than K's (the pages' DK != DV): torch's SDPA takes a value dim
    of its own, and the oracle's output has the value rows' width."""
    q, K, V, lens = _tiny(bits, D=D, DV=DV, N=2, HQ=6, HK=3)
    scale = 1.0 / math.sqrt(D)
    got = attention.decode_attention(q, K, V, lens, scale)
    assert got.shape == (2, 6, 2, DV)
    np.testing.assert_allclose(got, _sdpa_ref(q, K, V, lens, scale), rtol=1e-12, atol=1e-12)


def test_value_head_dim_of_its_own_brute_force():
    """Pure-Python loops, K rows of 64 dims and V rows of 32: out[d] for d < DV only."""
    q, K, V, lens = _tiny(16, B=1, HQ=2, HK=1, D=64, DV=32, N=1, lens=(7,))
    got = attention.decode_attention(q, K, V, lens, 0.2)
    for h in range(2):
        z = [0.2 * sum(q[0, h, 0, d] * K[0][t, 0, d] for d in range(64)) for t in range(7)]
        e = [math.exp(zz - max(z)) for zz in z]
        for d in range(32):
            want = sum(e[t] * V[0][t, 0, d] for t in range(7)) / sum(e)
            assert abs(got[0, h, 0, d] - want) <= 1e-12 * max(1.0, abs(want))


def test_brute_force_python_loops():
    q, K, V, lens = _tiny(4, B=1, HQ=4, HK=2, D=64, N=2, lens=(9,))
    scale = 0.125
    got = attention.decode_attention(q, K, V, lens, scale)
    L = int(lens[0])
    for h in range(4):
        g = h // 2
        for i in range(2):
            T = L - 2 + i + 1
            z = [scale * sum(q[0, h, i, d] * K[0][t, g, d] for d in range(64)) for t in range(T)]
            M = max(z)
            e = [math.exp(zz - M) for zz in z]
            for d in range(64):
                want = sum(e[t] * V[0][t, g, d] for t in range(T)) / sum(e)
                assert abs(got[0, h, i, d] - want) <= 1e-12 * max(1.0, abs(want))


def test_closed_forms():
    q, K, V, lens = _tiny(4, B=1, HQ=2, HK=1, D=128, N=1, lens=(50,))
    # one visible token -> out = V_0
    one = attention.decode_attention(q, [K[0][:1]], [V[0][:1]], np.array([1]), 0.1)
    assert np.array_equal(one[0, :, 0], np.repeat(V[0][0:1, 0], 2, axis=0))
    # all keys equal -> uniform weights -> mean of the visible values
    Keq = np.repeat(K[0][:1], 50, axis=0)
    o = attention.decode_attention(q, [Keq], V, lens, 0.3)
    np.testing.assert_allclose(o[0, 0, 0], V[0][:, 0].mean(axis=0), rtol=0, atol=1e-13)
    # q = 0 -> mean as well
    o = attention.decode_attention(np.zeros_like(q), K, V, lens, 0.3)
    np.testing.assert_allclose(o[0, 1, 0], V[0][:, 0].mean(axis=0), rtol=0, atol=1e-13)
    # multi-row: row i of N sees len - N + i + 1 tokens
    o = attention.decode_attention(np.zeros((1, 2, 3, 128)), K, V, lens, 0.3)
    for i in range(3):
        np.testing.assert_allclose(o[0, 0, i], V[0][: 50 - 3 + i + 1, 0].mean(axis=0), atol=1e-13)


@pytest.mark.parametrize("part", [1, 7, 64, 512, 300])
def test_split_merge_equals_two_pass(part):
    q, K, V, lens = _tiny(4, B=1, HQ=1, HK=1, D=64, N=1, lens=(300,))
    ref = attention.attend_one(q[0, 0, 0], K[0][:, 0], V[0][:, 0], 300, 0.2)
    got = attention.split_merge(q[0, 0, 0], K[0][:, 0], V[0][:, 0], 300, 0.2, part)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("wl,bs,dv", [("c3", 16, None), ("c3", 32, None), ("c2", 16, None), ("c4_2", 16, None),
                                      ("c3", 16, 64), ("c2", 16, 256), ("c4_8", 16, 256)])
def test_paged_equals_contiguous(wl, bs, dv):
    """The same rows in a shuffled pool of small blocks and in one contiguous block per
    sequence give identical planes after the gather, hence identical attention, bit for bit
    (also with V rows of a head dim of their own)."""
    w = make_workload(wl, B=3, len_lo=40, len_hi=100, BS=bs, HK=2, D=128, DV=dv)
    pool = attention.workload_pool(w)
    q = attention.q_f64(w.q_bits)
    Kp, Vp, Kc, Vc = [], [], [], []
    for b in range(w.B):
        g = pool.gather(w.table[b], int(w.lengths[b]))
        k, v = w.kv(b)
        if w.bits == 16:
            assert np.array_equal(g["k"], k.transpose(1, 0, 2))
            assert np.array_equal(g["v"], v.transpose(1, 0, 2))
        else:
            for name, x in (("k", k), ("v", v)):
                words, s, bb = quant.quantize(x, w.bits)
                assert np.array_equal(g[name], words.transpose(1, 0, 2))
                assert np.array_equal(g[name + "_scale"], s.transpose(1, 0, 2))
                assert np.array_equal(g[name + "_bias"], bb.transpose(1, 0, 2))
        assert vc_width(g, w) == w.DV
        kp, vp = pool.dequantized(w.table[b], int(w.lengths[b]))
        kc, vc = paged.rows_dequantized(k, v, w.bits)
        Kp.append(kp), Vp.append(vp), Kc.append(kc), Vc.append(vc)
    a = attention.decode_attention(q, Kp, Vp, w.lengths, w.scale)
    c = attention.decode_attention(q, Kc, Vc, w.lengths, w.scale)
    assert a.shape[-1] == w.DV
    assert np.array_equal(a, c)


def vc_width(g, w):
    """Head dims of the gathered V rows (codes of bits each, or bf16 values)."""
    return g["v"].shape[-1] * (1 if w.bits == 16 else 32) // (1 if w.bits == 16 else w.bits)


def test_unwritten_slots_stay_zero_and_tail_is_not_read():
    w = make_workload("c3", B=2, len_lo=40, len_hi=50, BS=32, HK=2, D=128)
    pool = attention.workload_pool(w)
    used = set()
    for b in range(w.B):
        for t in range(int(w.lengths[b])):
            used.add((int(w.table[b, t // 32]), t % 32))
    for phys in range(w.num_blocks):
        for off in range(32):
            if (phys, off) not in used:
                assert not pool.planes["k"][phys, :, off].any()
                assert not pool.planes["v_scale"][phys, :, off].any()
    # poison the rows past each length: the gather must not see them
    ref = [pool.dequantized(w.table[b], int(w.lengths[b])) for b in range(w.B)]
    for b in range(w.B):
        L = int(w.lengths[b])
        last = int(w.table[b, (L - 1) // 32])
        pool.planes["k_scale"][last, :, (L % 32 or 32):] = 0x7FC0
        pool.planes["v_bias"][last, :, (L % 32 or 32):] = 0x7FC0
    for b in range(w.B):
        k, v = pool.dequantized(w.table[b], int(w.lengths[b]))
        assert np.array_equal(k, ref[b][0]) and np.array_equal(v, ref[b][1])


def test_quantized_attention_converges_to_bf16_within_bound():
    """bits -> 8: with eps = max_t |dz_t| and dv = max |V_hat - V|, every output element obeys
    |out_q - out| <= (e^(2 eps) - 1) * max_t |V_t - c| + dv for c the mid-range of V (weights
    move by at most a factor e^(+-2 eps)); the mean error falls from 2 to 4 to 8 bits."""
    w = make_workload("c3", B=1, len_lo=200, len_hi=200, HK=1, HQ=4, D=128)
    k, v = w.kv(0)
    q = attention.q_f64(w.q_bits)
    K0, V0 = paged.rows_dequantized(k, v, 16)
    ref = attention.decode_attention(q, [K0], [V0], w.lengths, w.scale)
    errs = []
    for bits in (2, 4, 8):
        Kq, Vq = paged.rows_dequantized(k, v, bits)
        got = attention.decode_attention(q, [Kq], [Vq], w.lengths, w.scale)
        for h in range(4):
            dz = w.scale * np.abs((Kq[:, 0] - K0[:, 0]) @ q[0, h, 0])
            eps = dz.max()
            c = (V0[:, 0].max(0) + V0[:, 0].min(0)) / 2
            spread = np.abs(V0[:, 0] - c).max(0)
            dv = np.abs(Vq[:, 0] - V0[:, 0]).max(0)
            bound = (math.exp(2 * eps) - 1) * spread + dv
            assert np.all(np.abs(got[0, h, 0] - ref[0, h, 0]) <= bound + 1e-12)
        errs.append(np.abs(got - ref).mean())
    assert errs[0] > errs[1] > errs[2]


def test_generator_self_check_values():
    """Seeded generator: the sizes each workload is quoted with."""
    expect = {"c2": (34121, 1603, 8045, 2136, [1373, 1949, 1578]),
              "c3": (598835, 5933, 32197, 18726, [13748, 174, 12444]),
              "c5": (1320185, 8353, 32378, 41291, [2451, 11797, 23420])}
    for name, (tot, lo, hi, nb, first) in expect.items():
        w = make_workload(name)
        assert int(w.lengths.sum()) == tot and int(w.lengths.min()) == lo
        assert int(w.lengths.max()) == hi and w.num_blocks == nb
        assert list(w.table[0, :3]) == first
    w = make_workload("c3")
    assert w.effective_bytes() == 344928960
    assert make_workload("c1").effective_bytes() == 1179648
