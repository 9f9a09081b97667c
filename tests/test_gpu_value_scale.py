"""GPU: the path is exactly equivariant under a power-of-two scaling of V.

Multiplying every V element by 2^e (with e small enough that no value, scale, weight or sum
leaves f32's and bf16's normal range) multiplies each bf16 value exactly by 2^e.  For affine
pages it multiplies each group's max - min, its rounded-up scale and its bias (the group minimum)
exactly by 2^e and leaves every code unchanged.  Every later step then scales exactly too:
- the weights p * s and the bias terms p * b;
- their f32 sums and the lazy rescales by 2^(m_old - m_new);
- the merge's weighted sums and its division;
- the round-to-nearest-even to bf16.
So, with no oracle and at any size:
- the scaled pool's V codes equal the unscaled pool's, and its V scale and bias planes (or bf16 V
  values) are exactly 2^e times theirs;
- fixed partitions (bit-for-bit repeatable) give an f32 output exactly 2^e times the unscaled
  one, and a bf16 output as well;
- the balanced stream, whose waves share tiles at run time, agrees to f32 rounding.
The pool is filled by kv_append_quantize and every output comes from libkvq through the C ABI.
The matrix engine passes its weights through f16 halves, whose lower half can be subnormal, so
its exactness does not hold; its tolerance is checked elsewhere against the oracle."""
import numpy as np
import pytest
import torch

import decode_attention_paged_split_amd as kvq
from tests import gpu_util as G
from workloads import make_workload

pytestmark = pytest.mark.gpu

FORMATS = [(16, 64), (8, 64), (6, 64), (5, 32), (4, 64), (4, 32), (4, 128), (3, 64), (2, 64)]


def _scale_bits(v: np.ndarray, e: int) -> np.ndarray:
    """bf16 patterns times 2^e, exactly: e added to the exponent field of every normal value."""
    x = v.astype(np.int32)
    ex = (x >> 7) & 0xFF
    mant = x & 0x7F
    assert np.all((ex > 0) | (mant == 0)), "no subnormal inputs"
    assert np.all((ex == 0) | ((ex + e > 0) & (ex + e < 255))), "scaled values stay normal"
    return np.where(ex == 0, x, x + (e << 7)).astype(np.uint16)


def _filled(w, e):
    pool = G.new_pool(w)
    for b in range(w.B):
        k, v = w.kv(b)
        pool.append(G.u16_dev(k), G.u16_dev(_scale_bits(v, e)), G.i64_dev(w.slots(b)))
    torch.cuda.synchronize()
    return pool


@pytest.mark.parametrize("e", [-8, 9])
@pytest.mark.parametrize("bits,group", FORMATS)
def test_value_scale_equivariance(bits, group, e):
    print(f"value scale bits={bits} group={group} e={e}", flush=True)
    w = make_workload("c3", B=3, len_lo=200, len_hi=1300, bits=bits, group=group)
    base, scaled = _filled(w, 0), _filled(w, e)
    try:
        pa, pb = G.pool_planes_np(base), G.pool_planes_np(scaled)
        assert np.array_equal(pa["k"], pb["k"])
        if bits == 16:
            assert np.array_equal(_scale_bits(pa["v"], e), pb["v"])
        else:
            assert np.array_equal(pa["v"], pb["v"])                 # codes unchanged
            assert np.array_equal(_scale_bits(pa["v_scale"], e), pb["v_scale"])
            assert np.array_equal(_scale_bits(pa["v_bias"], e), pb["v_bias"])
            assert np.array_equal(pa["k_scale"], pb["k_scale"])
            assert np.array_equal(pa["k_bias"], pb["k_bias"])
        f = np.float64(2.0) ** e
        for pt in (64, 192):
            o0 = G.run_decode(w, base, partition_tokens=pt)
            o1 = G.run_decode(w, scaled, partition_tokens=pt)
            assert np.array_equal(o0 * f, o1), f"fixed partitions of {pt}: not exactly 2^{e} times"
            b0 = G.run_decode(w, base, partition_tokens=pt, out_f32=False)
            b1 = G.run_decode(w, scaled, partition_tokens=pt, out_f32=False)
            assert np.array_equal(_scale_bits(b0, e), b1), f"bf16 output, partitions of {pt}"
        s0 = G.run_decode(w, base, partition_tokens=kvq.PARTITION_STREAM)
        s1 = G.run_decode(w, scaled, partition_tokens=kvq.PARTITION_STREAM)
        assert np.abs(s0 * f - s1).max() <= 1e-6 * np.abs(s1).max()
    finally:
        base.close()
        scaled.close()


@pytest.mark.parametrize("e", [-6, 7])
@pytest.mark.parametrize("bits,group", [(16, 64), (8, 64), (4, 64), (3, 64), (2, 64)])
def test_query_scale_cancels_softmax_scale(bits, group, e):
    """q times 2^e with the softmax scale times 2^-e leaves every score, and so the output,
    bit-identical: the q copy, the dot products and the group sums of q scale exactly, and
    scale * log2(e) is scaled by 2^-e exactly.  Fixed partitions, and the matrix engine where
    it applies (both repeat bit for bit)."""
    print(f"query scale bits={bits} group={group} e={e}", flush=True)
    w = make_workload("c3", B=3, len_lo=200, len_hi=1300, bits=bits, group=group)
    pool = _filled(w, 0)
    try:
        q0, q1 = G.u16_dev(w.q_bits), G.u16_dev(_scale_bits(w.q_bits, e))
        tbl, lens = G.i32_dev(w.table), G.i32_dev(w.lengths)
        runs = [dict(partition_tokens=128, engine=kvq.ENGINE_VECTOR)]
        if bits == 4 and group == 64:
            runs.append(dict(partition_tokens=kvq.PARTITION_STREAM, engine=kvq.ENGINE_MATRIX))
        for kw in runs:
            a = kvq.decode(q0, pool, tbl, lens, w.scale, w.max_len, out_f32=True, **kw)
            b = kvq.decode(q1, pool, tbl, lens, w.scale * 2.0 ** -e, w.max_len, out_f32=True, **kw)
            torch.cuda.synchronize()
            assert torch.equal(a, b), f"{kw}: scores changed"
    finally:
        pool.close()
