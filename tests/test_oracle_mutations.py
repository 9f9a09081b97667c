"""Planted mistakes in the oracle (on the CPU) must each fail at least one pin.

Every mutation below is a plausible slip -- a reversed packing order, a scale rounded the
wrong way, truncation instead of round-half-even, a dropped bias, an off-by-one causal
end, a wrong GQA head map, a transposed gather, a merge without its weights -- and the
test asserts that some pin of tests/test_oracle_*.py catches it.  Nothing here touches
the HIP path.
"""
import numpy as np
import pytest

import oracle.attention as A
import oracle.bf16 as BF
import oracle.paged as P
import oracle.quant as Q
import tests.test_oracle_attention as TA
import tests.test_oracle_quant as TQ


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def _unpack_high_first(words, bits):
    words = np.asarray(words, dtype=np.uint32)
    Pk = 32 // bits
    shifts = (np.arange(Pk, dtype=np.uint32)[::-1] * np.uint32(bits))
    c = (words[..., None] >> shifts) & np.uint32((1 << bits) - 1)
    return c.reshape(words.shape[:-1] + (words.shape[-1] * Pk,))


def _dequant_no_bias(words, s, b, bits, group=64):
    c = Q.unpack(words, bits).astype(np.float64)
    D = c.shape[-1]
    c = c.reshape(c.shape[:-1] + (D // group, group))
    return (BF.to_f64(s)[..., None] * c).reshape(c.shape[:-2] + (D,))


def _decode_wrong_gqa(q, K, V, lengths, scale):
    B, HQ, N, D = q.shape
    out = np.zeros((B, HQ, N, V[0].shape[2]))
    for b in range(B):
        L = int(lengths[b])
        HK = K[b].shape[1]
        for h in range(HQ):
            g = h % HK                       # mistake: interleaved instead of grouped heads
            for i in range(N):
                T = L - N + i + 1
                out[b, h, i] = A.attend_one(q[b, h, i], K[b][:, g], V[b][:, g], T, scale)
    return out


def _decode_off_by_one(q, K, V, lengths, scale):
    B, HQ, N, D = q.shape
    out = np.zeros((B, HQ, N, V[0].shape[2]))
    for b in range(B):
        L = int(lengths[b])
        HK = K[b].shape[1]
        for h in range(HQ):
            g = h // (HQ // HK)
            for i in range(N):
                T = L - N + i                 # mistake: the row's own token is not visible
                out[b, h, i] = A.attend_one(q[b, h, i], K[b][:, g], V[b][:, g], max(T, 1), scale)
    return out


def _split_merge_unweighted(qv, K, V, T, scale, part):
    nparts = max(1, -(-T // part))
    num, den = np.zeros(V.shape[1]), 0.0
    for p in range(nparts):
        lo, hi = p * part, min(T, (p + 1) * part)
        z = scale * (K[lo:hi] @ qv)
        m = z.max()
        e = np.exp(z - m)
        num += e @ V[lo:hi]                   # mistake: partitions merged without e^(m_p - M)
        den += e.sum()
    return num / den


def _gather_transposed(self, table_row, length):
    nblk = (length + self.BS - 1) // self.BS
    idx = np.asarray(table_row[:nblk], dtype=np.int64)
    out = {}
    for name in self.names:
        took = self.planes[name][idx]                           # [nb, HK, BS, w]
        out[name] = took.reshape(self.HK, nblk * self.BS, -1)[:, :length]   # mistake: no transpose
    return out


def _quantize_codes_variant(mode):
    orig = Q.quantize_codes

    def f(x_bits, bits, group=64):
        x = BF.to_f32(x_bits).reshape(x_bits.shape[:-1] + (x_bits.shape[-1] // group, group))
        mx, mn = x.max(-1), x.min(-1)
        n = np.float32((1 << bits) - 1)
        s32 = (mx - mn).astype(np.float32) / n
        sb = BF.rne(s32) if mode == "rne_scale" else BF.roundup(s32)
        sc = BF.to_f32(sb)
        bias = (mn + np.float32(0)).astype(np.float32)
        with np.errstate(divide="ignore", invalid="ignore"):
            t = (x - bias[..., None]) / sc[..., None]
        t = np.floor(t) if mode == "trunc" else np.rint(t)
        t = np.where(sc[..., None] > 0, t, 0)
        codes = np.clip(t, 0, n).astype(np.uint32)
        return codes.reshape(x_bits.shape), sb, (bias.view(np.uint32) >> 16).astype(np.uint16)
    return f, orig


MUTATIONS = {
    "packing high-first": (Q, "unpack", _unpack_high_first),
    "dequant drops bias": (Q, "dequantize", _dequant_no_bias),
    "scale rounded to nearest": (Q, "quantize_codes", _quantize_codes_variant("rne_scale")[0]),
    "codes truncated": (Q, "quantize_codes", _quantize_codes_variant("trunc")[0]),
    "GQA heads interleaved": (A, "decode_attention", _decode_wrong_gqa),
    "causal end off by one": (A, "decode_attention", _decode_off_by_one),
    "merge without weights": (A, "split_merge", _split_merge_unweighted),
    "gather not transposed": (P.Pool, "gather", _gather_transposed),
}

PINS = [
    (TQ.test_packing_worked_words, ()),
    (TQ.test_quantizer_worked_groups, ()),
    (TQ.test_quantize_error_bound, (8, "c3", 64)),
    (TQ.test_quantize_error_bound, (4, "c3", 32)),
    (TA.test_matches_torch_sdpa, (4, 64, 3)),
    (TA.test_closed_forms, ()),
    (TA.test_split_merge_equals_two_pass, (64,)),
    (TA.test_paged_equals_contiguous, ("c3", 16, None)),
    (TA.test_paged_equals_contiguous, ("c3", 16, 64)),
    (TA.test_value_head_dim_of_its_own_matches_torch_sdpa, (4, 128, 64)),
]


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    owner, attr, repl = MUTATIONS[name]
    monkeypatch.setattr(owner, attr, repl)
    caught = [fn.__name__ for fn, args in PINS if _fails(fn, *args)]
    assert caught, f"no pin caught the planted mistake: {name}"


def test_unmutated_oracle_passes_every_pin():
    for fn, args in PINS:
        fn(*args)
