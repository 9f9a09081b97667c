"""GPU: the matrix-core engine over the whole range of V scales.

The matrix engine splits each P.V weight w = p * s_v into two f16 halves.  Without a prescale, large
V scales overflow the high half (p * s_v above 65504: V scale above 2^8 with p up to 2^8) and small
ones push both halves below f16's normal range, where they keep a fixed absolute step instead of
~22 bits.  The engine prescales the weights by a power of two per V group, taken from the group's
largest scale, and takes the factor back exactly at the end.  So:
- its output on V scaled by 2^e is exactly 2^e times its output on V (the stream schedule of the
  matrix engine repeats bit for bit: each wave owns its range), for e = 10 (scales near 2^8, where
  the unscaled split overflowed) and e = -5;
- with V scaled by 2^-5 and a dominant first token in every sequence (an attention sink: its score
  about 12 above the rest, which still hold a few per cent of the mass), the output meets the
  oracle's tolerance (max abs and rel L2 2e-3, the absolute bound taken on outputs scaled back by
  2^5), both engines.
The pool is filled by kv_append_quantize; every output comes from libkvq through the C ABI."""
import numpy as np
import pytest
import torch

import decode_attention_paged_split_amd as kvq
from oracle import attention
from tests import gpu_util as G
from tests.test_gpu_value_scale import _scale_bits
from workloads import bf16_bits_from_f32, make_workload

pytestmark = pytest.mark.gpu


def _with_v_scale_and_sink(w, e, sink):
    """w with its V rows scaled by 2^e and (sink) token 0's K row of each KV head replaced by
    0.75 times the sum of that head's query vectors (score ~12 against ~N(0, 1) for the rest)."""
    base_kv = w.kv
    q = G.bf16_to_f64(w.q_bits)                                    # [B, HQ, N, D]

    def kv(b):
        k, v = base_kv(b)
        v = _scale_bits(v, e) if e else v
        if sink:
            k = k.copy()
            for hk in range(w.HK):
                s = q[b, hk * w.REP:(hk + 1) * w.REP].reshape(-1, w.D).sum(axis=0) * 0.75
                k[0, hk] = bf16_bits_from_f32(s.astype(np.float32))
        return k, v
    w.kv = kv
    return w


def _fill(w):
    pool = G.new_pool(w)
    G.fill_pool(w, pool)
    return pool


@pytest.mark.parametrize("name,over", [("c3", dict(B=3, len_lo=900, len_hi=3000)),
                                       ("c5", dict(B=2, len_lo=700, len_hi=2000)),
                                       ("c3", dict(B=2, len_lo=600, len_hi=1800, D=128, HQ=16, HK=4))])
@pytest.mark.parametrize("e", [10, -5])
def test_matrix_engine_is_exact_under_v_scaling(name, over, e):
    print(f"matrix engine V x 2^{e}: {name} {over}", flush=True)
    w0 = make_workload(name, **over)
    w1 = _with_v_scale_and_sink(make_workload(name, **over), e, sink=False)
    p0, p1 = _fill(w0), _fill(w1)
    try:
        o0 = G.run_decode(w0, p0, engine=kvq.ENGINE_MATRIX)
        o1 = G.run_decode(w1, p1, engine=kvq.ENGINE_MATRIX)
        assert np.all(np.isfinite(o1)), f"V x 2^{e}: non-finite output"
        f = np.float64(2.0) ** e
        bad = np.argwhere(o0 * f != o1)
        assert bad.size == 0, f"V x 2^{e}: {bad.shape[0]} outputs not exactly 2^{e} times, first {bad[:3].tolist()}"
    finally:
        p0.close()
        p1.close()


@pytest.mark.parametrize("name,over", [("c3", dict(B=3, len_lo=1500, len_hi=4000)),
                                       ("c5", dict(B=2, len_lo=1000, len_hi=3000))])
def test_small_values_with_an_attention_sink(name, over):
    print(f"V x 2^-5 with a sink token: {name} {over}", flush=True)
    e = -5
    w = _with_v_scale_and_sink(make_workload(name, **over), e, sink=True)
    pool = _fill(w)
    try:
        ref = attention.workload_output(w)
        f = np.float64(2.0) ** -e                   # compare at the unscaled magnitude
        for engine in (kvq.ENGINE_VECTOR, kvq.ENGINE_MATRIX):
            got = G.run_decode(w, pool, engine=engine)
            err, rl2 = G.check_f32(got * f, ref * f, tag=f"{name} sink engine={engine}")
            print(f"  engine {engine}: max abs {err:.2e} (x 2^5) rel L2 {rl2:.2e}", flush=True)
    finally:
        pool.close()
