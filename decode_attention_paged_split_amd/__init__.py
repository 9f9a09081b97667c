"""Paged split-K decode attention over bf16 / affine-quantized KV pages, for MI355X (gfx950).

A thin ctypes binding over ``libkvq.so`` (the C ABI in ``include/kvq.h``).  Every step of
the path runs in the library's HIP kernels; this module only marshals arguments.  PyTorch
supplies device memory (``torch.empty`` / ``torch.zeros`` on a ROCm device) and the
current stream.  There is no CPU fallback: importing works without a GPU, but every
compute call needs the built library and a GPU, and raises otherwise.

Functions with the C ABI's names:

* ``kv_pool_create(desc)`` / ``kv_pool_wrap(desc, planes)`` / ``kv_pool_destroy(handle)``
* ``kv_append_quantize(pool, k, v, slots)``
* ``paged_decode_workspace_bytes(pool, shape)``
* ``paged_decode_attention(q, pool, block_table, lengths, scale, shape, workspace, out)``
* ``kv_gather_debug(pool, block_table, lengths, batch, max_blocks, max_len, out_planes)``

plus ``Pool`` (planes held as torch tensors, wrapped by the library) and ``decode``
(allocates workspace and output, then calls ``paged_decode_attention``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

__all__ = [
    "KvqError", "PoolDesc", "DecodeShape", "Pool", "decode", "lib", "kv_pool_create", "kv_pool_wrap",
    "kv_pool_destroy", "kv_pool_plane_bytes", "kv_append_quantize", "paged_decode_workspace_bytes",
    "paged_decode_partition_tokens", "paged_decode_engine", "paged_decode_attention", "paged_decode_partial",
    "paged_decode_merge", "paged_decode_step", "paged_decode_step_partial", "paged_decode_step_noalloc",
    "NOALLOC_WORKSPACE_BYTES", "kv_gather_debug", "make_shape", "gather", "decode_step",
    "kvq_timing_enable", "kvq_timing_read", "kvq_probe_read", "kvq_probe_read_ex", "kvq_probe_pool_read", "TIMING_PREP", "TIMING_PARTIAL", "TIMING_MERGE", "PARTITION_AUTO", "PARTITION_STREAM",
    "PLANES", "LIB_PATH",
]

# the in-tree build; KVQ_LIB names another build of the same library (e.g. to compare two builds)
LIB_PATH = os.environ.get("KVQ_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq.so")

PLANE_K, PLANE_V, PLANE_K_SCALE, PLANE_K_BIAS, PLANE_V_SCALE, PLANE_V_BIAS = range(6)
PLANES = ("k", "v", "k_scale", "k_bias", "v_scale", "v_bias")
STATUS = {0: "KVQ_OK", -1: "KVQ_ERR_INVALID", -2: "KVQ_ERR_UNSUPPORTED", -3: "KVQ_ERR_OOM",
          -4: "KVQ_ERR_HIP", -5: "KVQ_ERR_WORKSPACE", -6: "KVQ_ERR_RANGE"}


class KvqError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class PoolDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("v_head_dim", ctypes.c_int32)]


class DecodeShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("q_rows", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("max_len", ctypes.c_int32),
                ("partition_tokens", ctypes.c_int32), ("out_f32", ctypes.c_int32),
                ("engine", ctypes.c_int32)]


ENGINE_AUTO, ENGINE_VECTOR, ENGINE_MATRIX = 0, 1, 2
TIMING_PREP, TIMING_PARTIAL, TIMING_MERGE = 0, 1, 2
PARTITION_AUTO, PARTITION_STREAM = 0, -1
NOALLOC_WORKSPACE_BYTES = 64 * 1024 * 1024     # KVQ_NOALLOC_WORKSPACE_BYTES


_lib: Optional[ctypes.CDLL] = None
_P = ctypes.c_void_p
_PP = ctypes.POINTER(ctypes.c_void_p)


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m decode_attention_paged_split_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "kvq_last_error": (ctypes.c_char_p, []),
            "kvq_version": (ctypes.c_char_p, []),
            "kv_pool_plane_bytes": (ctypes.c_size_t, [ctypes.POINTER(PoolDesc), ctypes.c_int32]),
            "kv_pool_create": (ctypes.c_int, [ctypes.POINTER(PoolDesc), _PP]),
            "kv_pool_wrap": (ctypes.c_int, [ctypes.POINTER(PoolDesc), _P * 6, _PP]),
            "kv_pool_destroy": (ctypes.c_int, [_P]),
            "kv_pool_plane": (ctypes.c_int, [_P, ctypes.c_int32, _PP, ctypes.POINTER(ctypes.c_size_t)]),
            "kv_pool_describe": (ctypes.c_int, [_P, ctypes.POINTER(PoolDesc)]),
            "kv_append_quantize": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int32, _P]),
            "paged_decode_workspace_bytes": (ctypes.c_size_t, [_P, ctypes.POINTER(DecodeShape)]),
            "paged_decode_partition_tokens": (ctypes.c_int32, [_P, ctypes.POINTER(DecodeShape)]),
            "paged_decode_engine": (ctypes.c_int32, [_P, ctypes.POINTER(DecodeShape)]),
            "paged_decode_attention": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_float,
                                                      ctypes.POINTER(DecodeShape), _P, ctypes.c_size_t,
                                                      _P, _P]),
            "paged_decode_partial": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_float, ctypes.POINTER(DecodeShape),
                                                    _P, ctypes.c_size_t, _P]),
            "paged_decode_merge": (ctypes.c_int, [_P, _P, ctypes.POINTER(DecodeShape), _P, ctypes.c_size_t,
                                                  _P, _P]),
            "paged_decode_step": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_float,
                                                 ctypes.POINTER(DecodeShape), _P, ctypes.c_size_t, _P, _P]),
            "paged_decode_step_partial": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_float,
                                                         ctypes.POINTER(DecodeShape), _P, ctypes.c_size_t, _P]),
            "paged_decode_step_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_float,
                                                         ctypes.POINTER(DecodeShape), _P, _P]),
            "kv_gather_debug": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                               _P * 6, _P]),
            "kvq_probe_read": (ctypes.c_int, [_P, ctypes.c_size_t, _P, _P]),
            "kvq_probe_read_ex": (ctypes.c_int, [_P, ctypes.c_size_t, _P, ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.c_int32, _P]),
            "kvq_probe_pool_read": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                   ctypes.c_int32, _P, _P]),
            "kvq_timing_enable": (ctypes.c_int, [ctypes.c_int32]),
            "kvq_timing_read": (ctypes.c_int, [ctypes.c_int32, ctypes.POINTER(ctypes.c_double),
                                               ctypes.POINTER(ctypes.c_int32)]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(code: int) -> None:
    if code != 0:
        raise KvqError(code, lib().kvq_last_error().decode())


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need_cuda(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("kvq kernels take device tensors; got a CPU tensor")
        if t is not None and not t.is_contiguous():
            raise ValueError("kvq kernels take contiguous tensors")


# ------------------------------------------------------------------ C ABI, same names

def kvq_timing_enable(on: bool) -> None:
    """Start (True) or stop (False) bracketing the library's kernel launches with events."""
    _check(lib().kvq_timing_enable(1 if on else 0))


def kvq_probe_read(buf, sink, stream=None) -> None:
    """Enqueue the streaming-read probe over the device tensor buf (sink: a device int32 tensor)."""
    _need_cuda(buf, sink)
    _check(lib().kvq_probe_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)))


def kvq_probe_pool_read(pool, block_table, lengths, max_len, coalesced=False, sink=None, stream=None) -> None:
    """Enqueue the pool-read probe over every cached row of the batch (block_table [B, max_blocks]
    and lengths [B] int32 device tensors; sink a device int32 tensor)."""
    _need_cuda(block_table, lengths, sink)
    B, mb = block_table.shape
    _check(lib().kvq_probe_pool_read(pool.handle, _ptr(block_table), _ptr(lengths), int(B), int(mb), int(max_len),
                                     1 if coalesced else 0, _ptr(sink), _stream(stream)))


def kvq_probe_read_ex(buf, sink, loads_in_flight=4, nontemporal=False, blocks_per_cu=32, stream=None) -> None:
    """The streaming-read probe with its launch shape chosen (loads in flight per thread,
    non-temporal loads, workgroups per compute unit)."""
    _need_cuda(buf, sink)
    _check(lib().kvq_probe_read_ex(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), int(loads_in_flight),
                                   1 if nontemporal else 0, int(blocks_per_cu), _stream(stream)))


def kvq_timing_read(kind: int):
    """(mean ms, count) of the launches of `kind` (TIMING_PREP / _PARTIAL / _MERGE) recorded since
    the last read; waits for their events."""
    avg, n = ctypes.c_double(0.0), ctypes.c_int32(0)
    _check(lib().kvq_timing_read(kind, ctypes.byref(avg), ctypes.byref(n)))
    return float(avg.value), int(n.value)


def kv_pool_plane_bytes(desc: PoolDesc, plane: int) -> int:
    return int(lib().kv_pool_plane_bytes(ctypes.byref(desc), plane))


def kv_pool_create(desc: PoolDesc) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(lib().kv_pool_create(ctypes.byref(desc), ctypes.byref(h)))
    return h


def kv_pool_wrap(desc: PoolDesc, planes: Sequence[int]) -> ctypes.c_void_p:
    arr = (_P * 6)(*[ctypes.c_void_p(p) for p in planes])
    h = ctypes.c_void_p()
    _check(lib().kv_pool_wrap(ctypes.byref(desc), arr, ctypes.byref(h)))
    return h


def kv_pool_destroy(handle) -> None:
    _check(lib().kv_pool_destroy(handle))


def kv_append_quantize(pool: "Pool", k, v, slots, stream=None) -> None:
    _need_cuda(k, v, slots)
    T = int(slots.shape[0])
    _check(lib().kv_append_quantize(pool.handle, _ptr(k), _ptr(v), _ptr(slots), T, _stream(stream)))


def paged_decode_workspace_bytes(pool: "Pool", shape: DecodeShape) -> int:
    n = int(lib().paged_decode_workspace_bytes(pool.handle, ctypes.byref(shape)))
    if n == 0:
        raise KvqError(-1, lib().kvq_last_error().decode())
    return n


def paged_decode_partition_tokens(pool: "Pool", shape: DecodeShape) -> int:
    return int(lib().paged_decode_partition_tokens(pool.handle, ctypes.byref(shape)))


def paged_decode_engine(pool: "Pool", shape: DecodeShape) -> int:
    """ENGINE_VECTOR or ENGINE_MATRIX: the engine this shape runs on (the automatic choice resolved)."""
    r = int(lib().paged_decode_engine(pool.handle, ctypes.byref(shape)))
    if r < 0:
        _check(r)
    return r


def paged_decode_attention(q, pool: "Pool", block_table, lengths, scale: float, shape: DecodeShape,
                           workspace, out, stream=None) -> None:
    _need_cuda(q, block_table, lengths, workspace, out)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().paged_decode_attention(_ptr(q), pool.handle, _ptr(block_table), _ptr(lengths),
                                        float(scale), ctypes.byref(shape), _ptr(workspace), ws_bytes,
                                        _ptr(out), _stream(stream)))


def paged_decode_step(q, k_new, v_new, pool: "Pool", block_table, lengths, scale: float, shape: DecodeShape,
                      workspace, out, stream=None) -> None:
    _need_cuda(q, k_new, v_new, block_table, lengths, workspace, out)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().paged_decode_step(_ptr(q), _ptr(k_new), _ptr(v_new), pool.handle, _ptr(block_table),
                                   _ptr(lengths), float(scale), ctypes.byref(shape), _ptr(workspace), ws_bytes,
                                   _ptr(out), _stream(stream)))


def paged_decode_step_partial(q, k_new, v_new, pool: "Pool", block_table, lengths, scale: float,
                              shape: DecodeShape, workspace, stream=None) -> None:
    _need_cuda(q, k_new, v_new, block_table, lengths, workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().paged_decode_step_partial(_ptr(q), _ptr(k_new), _ptr(v_new), pool.handle, _ptr(block_table),
                                           _ptr(lengths), float(scale), ctypes.byref(shape), _ptr(workspace),
                                           ws_bytes, _stream(stream)))


def paged_decode_step_noalloc(q, k_new, v_new, pool: "Pool", block_table, lengths, scale: float,
                              shape: DecodeShape, out, stream=None) -> None:
    """paged_decode_step with the library's own device scratch as workspace (no allocation in the
    call; at most NOALLOC_WORKSPACE_BYTES of workspace; overlapping calls on one device race)."""
    _need_cuda(q, k_new, v_new, block_table, lengths, out)
    _check(lib().paged_decode_step_noalloc(_ptr(q), _ptr(k_new), _ptr(v_new), pool.handle, _ptr(block_table),
                                           _ptr(lengths), float(scale), ctypes.byref(shape), _ptr(out),
                                           _stream(stream)))


def paged_decode_partial(q, pool: "Pool", block_table, lengths, scale: float, shape: DecodeShape,
                         workspace, stream=None) -> None:
    _need_cuda(q, block_table, lengths, workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().paged_decode_partial(_ptr(q), pool.handle, _ptr(block_table), _ptr(lengths), float(scale),
                                      ctypes.byref(shape), _ptr(workspace), ws_bytes, _stream(stream)))


def paged_decode_merge(pool: "Pool", lengths, shape: DecodeShape, workspace, out, stream=None) -> None:
    _need_cuda(lengths, workspace, out)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().paged_decode_merge(pool.handle, _ptr(lengths), ctypes.byref(shape), _ptr(workspace), ws_bytes,
                                    _ptr(out), _stream(stream)))


def kv_gather_debug(pool: "Pool", block_table, lengths, batch: int, max_blocks: int, max_len: int,
                    out_planes: Sequence, stream=None) -> None:
    _need_cuda(block_table, lengths, *[o for o in out_planes if o is not None])
    arr = (_P * 6)(*[_ptr(o) if o is not None else ctypes.c_void_p(0) for o in out_planes])
    _check(lib().kv_gather_debug(pool.handle, _ptr(block_table), _ptr(lengths), batch, max_blocks,
                                 max_len, arr, _stream(stream)))


# ------------------------------------------------------------------ convenience

class Pool:
    """A block pool whose planes are torch device tensors wrapped by the library.

    planes["k"], planes["v"]: uint32 codes [NB, HK, BS, D*bits/32] (affine; a row's codes are one
    little-endian bit stream, so 3/5/6-bit codes straddle words) or bf16 bit
    patterns as int16 [NB, HK, BS, D] (bits == 16); planes["{k,v}_{scale,bias}"]: bf16
    bit patterns as int16 [NB, HK, BS, D/group_size].  The V planes take v_head_dim (DV,
    default head_dim) in place of D.
    """

    def __init__(self, num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int,
                 bits: int, group_size: int = 64, device=None, v_head_dim: Optional[int] = None):
        import torch
        dv = head_dim if v_head_dim is None else v_head_dim
        self.desc = PoolDesc(num_blocks, num_kv_heads, block_size, head_dim, bits, group_size, dv)
        dev = torch.device(device) if device is not None else torch.device("cuda")
        shape = lambda w: (num_blocks, num_kv_heads, block_size, w)  # noqa: E731
        if bits == 16:
            self.planes = {"k": torch.zeros(shape(head_dim), dtype=torch.int16, device=dev),
                           "v": torch.zeros(shape(dv), dtype=torch.int16, device=dev)}
        else:
            W, G = head_dim * bits // 32, head_dim // group_size
            WV, GV = dv * bits // 32, dv // group_size
            # uint32 codes held as int32 storage (torch has no uint32 arithmetic on every backend)
            self.planes = {"k": torch.zeros(shape(W), dtype=torch.int32, device=dev),
                           "v": torch.zeros(shape(WV), dtype=torch.int32, device=dev)}
            for n in PLANES[2:]:
                self.planes[n] = torch.zeros(shape(GV if n.startswith("v") else G), dtype=torch.int16,
                                             device=dev)
        ptrs = [self.planes[n].data_ptr() if n in self.planes else 0 for n in PLANES]
        for i, n in enumerate(PLANES):
            if n in self.planes:
                want = kv_pool_plane_bytes(self.desc, i)
                t = self.planes[n]
                assert t.numel() * t.element_size() == want, (n, want)
        self.handle = kv_pool_wrap(self.desc, ptrs)

    @property
    def bits(self) -> int:
        return self.desc.bits

    @property
    def v_head_dim(self) -> int:
        return self.desc.v_head_dim

    def append(self, k, v, slots, stream=None) -> None:
        kv_append_quantize(self, k, v, slots, stream)

    def close(self) -> None:
        if getattr(self, "handle", None):
            kv_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def make_shape(pool: Pool, batch: int, num_q_heads: int, q_rows: int, max_blocks: int, max_len: int,
               partition_tokens: int = 0, out_f32: bool = False, engine: int = ENGINE_AUTO) -> DecodeShape:
    return DecodeShape(batch, num_q_heads, q_rows, max_blocks, max_len, partition_tokens, int(out_f32), engine)


def decode(q, pool: Pool, block_table, lengths, scale: float, max_len: int, partition_tokens: int = 0,
           out_f32: bool = False, workspace=None, out=None, stream=None, engine: int = ENGINE_AUTO):
    """Allocate (if not given) workspace and output, then run paged_decode_attention.

    q: bf16 [B, HQ, N, D] (torch.bfloat16 or int16 bit patterns); block_table int32 [B, M];
    lengths int32 [B].  Returns out [B, HQ, N, DV] (bfloat16, or float32 if out_f32; DV the pool's
    V head dim).
    """
    import torch
    B, HQ, N, _ = q.shape
    D = pool.v_head_dim
    shape = make_shape(pool, B, HQ, N, block_table.shape[1], max_len, partition_tokens, out_f32, engine)
    if workspace is None:
        workspace = torch.empty(paged_decode_workspace_bytes(pool, shape), dtype=torch.uint8,
                                device=q.device)
    if out is None:
        out = torch.empty((B, HQ, N, D), dtype=torch.float32 if out_f32 else torch.bfloat16,
                          device=q.device)
    paged_decode_attention(q, pool, block_table, lengths, scale, shape, workspace, out, stream)
    return out


def decode_step(q, k_new, v_new, pool: Pool, block_table, lengths, scale: float, max_len: int,
                partition_tokens: int = 0, out_f32: bool = False, workspace=None, out=None, stream=None,
                engine: int = ENGINE_AUTO):
    """paged_decode_step with freshly allocated workspace and output (if not given): append the
    step's new rows k_new ([B, N, HK, D] bf16) and v_new ([B, N, HK, DV]) at the slots their
    positions take in the block table, then attend.  Returns out [B, HQ, N, DV]."""
    import torch
    B, HQ, N, _ = q.shape
    D = pool.v_head_dim
    shape = make_shape(pool, B, HQ, N, block_table.shape[1], max_len, partition_tokens, out_f32, engine)
    if workspace is None:
        workspace = torch.empty(paged_decode_workspace_bytes(pool, shape), dtype=torch.uint8,
                                device=q.device)
    if out is None:
        out = torch.empty((B, HQ, N, D), dtype=torch.float32 if out_f32 else torch.bfloat16,
                          device=q.device)
    paged_decode_step(q, k_new, v_new, pool, block_table, lengths, scale, shape, workspace, out, stream)
    return out


def gather(pool: Pool, block_table, lengths, max_len: int, stream=None) -> Dict[str, object]:
    """kv_gather_debug into fresh tensors: {plane: [B, HK, max_len, width]}."""
    import torch
    B, M = block_table.shape
    outs = {}
    for n, t in pool.planes.items():
        outs[n] = torch.empty((B, pool.desc.num_kv_heads, max_len, t.shape[-1]), dtype=t.dtype,
                              device=t.device)
    kv_gather_debug(pool, block_table, lengths, B, M, max_len, [outs.get(n) for n in PLANES], stream)
    return outs
