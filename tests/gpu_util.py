"""Helpers of the GPU tests: move seeded inputs to the device, fill a pool through the HIP
append kernel, and compare results with the oracle.  Imports the oracle only for expected
values; every device-side result comes from libkvq through the C ABI."""
from __future__ import annotations

import numpy as np
import torch

import decode_attention_paged_split_amd as kvq
from oracle import bf16 as obf16

DEV = "cuda"


def u16_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def i32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def i64_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).to(DEV)


def new_pool(w, num_blocks=None) -> kvq.Pool:
    return kvq.Pool(num_blocks or w.num_blocks, w.HK, w.BS, w.D, w.bits, w.group, v_head_dim=w.DV)


def fill_pool(w, pool: kvq.Pool, seqs=None) -> None:
    """Append every token of the chosen sequences through kv_append_quantize."""
    for b in (range(w.B) if seqs is None else seqs):
        k, v = w.kv(b)
        pool.append(u16_dev(k), u16_dev(v), i64_dev(w.slots(b)))
    torch.cuda.synchronize()


def pool_planes_np(pool: kvq.Pool):
    """Pool planes as numpy arrays with the oracle's dtypes (uint32 codes, uint16 bf16)."""
    out = {}
    for n, t in pool.planes.items():
        a = t.cpu().numpy()
        out[n] = a.view(np.uint32) if a.dtype == np.int32 else a.view(np.uint16)
    return out


def run_decode(w, pool, partition_tokens=0, out_f32=True, q=None, lengths=None, table=None, engine=0):
    q = u16_dev(w.q_bits) if q is None else q
    table = i32_dev(w.table) if table is None else table
    lengths = i32_dev(w.lengths) if lengths is None else lengths
    out = kvq.decode(q, pool, table, lengths, w.scale, w.max_len, partition_tokens=partition_tokens,
                     out_f32=out_f32, engine=engine)
    torch.cuda.synchronize()
    if out_f32:
        return out.cpu().numpy().astype(np.float64)
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


bf16_to_f64 = obf16.to_f64
rne_f32_to_bf16 = obf16.rne


def check_f32(got: np.ndarray, ref: np.ndarray, atol=2e-3, rel_l2=2e-3, tag=""):
    """f32 output vs f64 oracle: max abs and relative L2 over the whole tensor."""
    assert np.all(np.isfinite(got)), f"{tag}: non-finite output"
    err = np.abs(got - ref)
    rl2 = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert err.max() <= atol, f"{tag}: max abs {err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}"
    assert rl2 <= rel_l2, f"{tag}: rel L2 {rl2:.3e}"
    return float(err.max()), float(rl2)


def check_bf16(got_bits: np.ndarray, ref: np.ndarray, tag=""):
    """bf16 output vs the oracle rounded to bf16 (RNE of its f32 value): rel L2 <= 2e-3 and max abs
    <= max(2e-3, one bf16 ulp of the reference value).  The comparison is with the rounded oracle:
    the rounding alone moves a small output tensor by up to ~2e-3 in rel L2 (bf16 keeps 8
    significant bits), so against the unrounded f64 values even the correctly rounded answer
    could fail the bound."""
    got = bf16_to_f64(got_bits)
    ref32 = ref.astype(np.float32)
    ref16 = bf16_to_f64(rne_f32_to_bf16(ref32))
    u = ref32.view(np.uint32)
    exp = ((u >> 23) & 0xFF).astype(np.int64) - 127
    ulp = np.ldexp(1.0, np.maximum(exp, -126) - 7)
    err = np.abs(got - ref16)
    assert np.all(err <= np.maximum(2e-3, ulp)), f"{tag}: bf16 max abs {err.max():.3e}"
    rl2 = np.linalg.norm(got - ref16) / max(np.linalg.norm(ref16), 1e-30)
    assert rl2 <= 2e-3, f"{tag}: bf16 rel L2 {rl2:.3e}"

