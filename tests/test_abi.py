"""The C-ABI library loads, exports every entry point include/kvq.h declares, and rejects bad
arguments on the host (CPU only: no call here launches a kernel)."""
import ctypes
import os
import re
import subprocess

import pytest

import decode_attention_paged_split_amd as kvq
from workloads import make_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|int32_t|size_t|char\s*\*|void)\s*\**\s*(\w+)\s*\(", src, re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kvq.LIB_PATH):
        pytest.skip("libkvq.so not built (python -m decode_attention_paged_split_amd.build)")
    return kvq.lib()


def test_header_declares_the_boundary():
    names = _declared()
    for must in ["kv_pool_create", "kv_pool_destroy", "kv_append_quantize", "paged_decode_attention",
                 "paged_decode_step", "paged_decode_workspace_bytes", "kv_gather_debug", "kvq_last_error"]:
        assert must in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", kvq.LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in _declared():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_timing_without_launches(lib):
    """Launch timing: nothing recorded reads as (0 ms, 0 launches); a bad kind is rejected."""
    kvq.kvq_timing_enable(True)
    for kind in (kvq.TIMING_PREP, kvq.TIMING_PARTIAL, kvq.TIMING_MERGE):
        assert kvq.kvq_timing_read(kind) == (0.0, 0)
    kvq.kvq_timing_enable(False)
    with pytest.raises(kvq.KvqError, match="KVQ_ERR_INVALID"):
        kvq.kvq_timing_read(7)


def test_probe_read_rejects_bad_arguments(lib):
    assert lib.kvq_probe_read(None, 1024, None, None) == -1
    assert lib.kvq_probe_read(ctypes.c_void_p(256), 1000, ctypes.c_void_p(512), None) == -1   # not x16
    assert lib.kvq_probe_read(ctypes.c_void_p(255), 1024, ctypes.c_void_p(512), None) == -1   # misaligned
    P = ctypes.c_void_p(256)
    for u, bpc in ((3, 32), (0, 32), (32, 32), (4, 0), (4, 65)):
        assert lib.kvq_probe_read_ex(P, 1024, P, u, 0, bpc, None) == -1, (u, bpc)
        assert lib.kvq_last_error().decode()
    assert lib.kvq_probe_pool_read(None, P, P, 1, 1, 1, 0, P, None) == -1


def test_struct_layouts():
    assert ctypes.sizeof(kvq.PoolDesc) == 28
    assert ctypes.sizeof(kvq.DecodeShape) == 32


@pytest.mark.parametrize("name,expect", [("c3", 345157632), ("c2", 139984896), ("c1", 1179648),
                                         ("c5", 1522151424), ("c4_8", 1140850688), ("c4_2", 335544320),
                                         ("diag", 603979776)])
def test_pool_bytes_match_the_layout(lib, name, expect):
    """Pool sizes [NB, HK, BS, width] per plane for the seeded workloads."""
    w = make_workload(name)
    d = kvq.PoolDesc(w.num_blocks, w.HK, w.BS, w.D, w.bits, 64)
    total = sum(kvq.kv_pool_plane_bytes(d, p) for p in range(6))
    assert total == expect
    rows = w.num_blocks * w.HK * w.BS
    if w.bits == 16:
        assert kvq.kv_pool_plane_bytes(d, 0) == rows * w.D * 2
        assert kvq.kv_pool_plane_bytes(d, 2) == 0
    else:
        assert kvq.kv_pool_plane_bytes(d, 0) == rows * w.D * w.bits // 8
        assert kvq.kv_pool_plane_bytes(d, 5) == rows * (w.D // 64) * 2


@pytest.mark.parametrize("field,value,code", [("bits", 7, -2), ("bits", 1, -2), ("bits", 32, -2), ("group_size", 48, -2),
                                              ("group_size", 256, -2), ("group_size", 16, -2),
                                              ("head_dim", 96, -2), ("head_dim", 512, -2),
                                              ("num_blocks", 0, -1), ("block_size", 0, -1)])
def test_pool_descriptor_rejected(lib, field, value, code):
    d = kvq.PoolDesc(4, 2, 16, 128, 4, 64)
    setattr(d, field, value)
    with pytest.raises(kvq.KvqError) as e:
        kvq.kv_pool_wrap(d, [16] * 6)
    assert e.value.code == code
    assert lib.kvq_last_error().decode()


@pytest.mark.parametrize("group,D,ok", [(32, 256, True), (128, 256, True), (128, 128, True), (128, 64, False),
                                         (32, 64, True)])
def test_group_sizes(lib, group, D, ok):
    d = kvq.PoolDesc(4, 2, 16, D, 4, group)
    if ok:
        h = kvq.kv_pool_wrap(d, [16] * 6)
        assert kvq.kv_pool_plane_bytes(d, 3) == 4 * 2 * 16 * (D // group) * 2
        kvq.kv_pool_destroy(h)
    else:
        with pytest.raises(kvq.KvqError) as e:
            kvq.kv_pool_wrap(d, [16] * 6)
        assert e.value.code == -2


@pytest.mark.parametrize("bits,D,ok", [(3, 128, True), (3, 256, True), (5, 128, True), (5, 256, True),
                                        (6, 64, True), (6, 256, True), (3, 64, False), (5, 64, False)])
def test_straddling_widths(lib, bits, D, ok):
    """3/5/6-bit pages: the codes plane holds D * bits / 8 bytes per row (one bit stream); a row
    must be whole 16-byte chunks (head dim 64 at 3 or 5 bits is not: 24 or 40 bytes)."""
    d = kvq.PoolDesc(4, 2, 16, D, bits, 32)
    if ok:
        h = kvq.kv_pool_wrap(d, [16] * 6)
        assert kvq.kv_pool_plane_bytes(d, 0) == 4 * 2 * 16 * D * bits // 8
        assert kvq.kv_pool_plane_bytes(d, 5) == 4 * 2 * 16 * (D // 32) * 2
        kvq.kv_pool_destroy(h)
    else:
        with pytest.raises(kvq.KvqError) as e:
            kvq.kv_pool_wrap(d, [16] * 6)
        assert e.value.code == -2


@pytest.mark.parametrize("bits,D,DV,group,ok", [
    (16, 128, 64, 64, True), (16, 128, 256, 64, True), (16, 256, 128, 64, True), (16, 64, 128, 64, True),
    (8, 256, 128, 64, True), (4, 128, 64, 64, True), (4, 64, 128, 64, True), (2, 128, 256, 64, True),
    (4, 256, 64, 64, False),        # a quarter: not read
    (4, 128, 64, 32, False),        # group 32 with a V head dim of its own
    (5, 256, 128, 32, False),       # straddling width
    (16, 128, 512, 64, False), (16, 128, 96, 64, False)])
def test_value_head_dim(lib, bits, D, DV, group, ok):
    """A V head dim of its own (the pages' vHeadDim): the V planes take DV in place of D; 0 stands
    for D and the pool reports DV explicitly."""
    d = kvq.PoolDesc(4, 2, 16, D, bits, group, DV)
    rows = 4 * 2 * 16
    if not ok:
        with pytest.raises(kvq.KvqError) as e:
            kvq.kv_pool_wrap(d, [16] * 6)
        assert e.value.code == -2
        return
    h = kvq.kv_pool_wrap(d, [16] * 6)
    if bits == 16:
        assert kvq.kv_pool_plane_bytes(d, 0) == rows * D * 2
        assert kvq.kv_pool_plane_bytes(d, 1) == rows * DV * 2
    else:
        assert kvq.kv_pool_plane_bytes(d, 0) == rows * D * bits // 8
        assert kvq.kv_pool_plane_bytes(d, 1) == rows * DV * bits // 8
        assert kvq.kv_pool_plane_bytes(d, 2) == rows * (D // group) * 2
        assert kvq.kv_pool_plane_bytes(d, 4) == rows * (DV // group) * 2
        assert kvq.kv_pool_plane_bytes(d, 5) == rows * (DV // group) * 2
    out = kvq.PoolDesc()
    assert lib.kv_pool_describe(h, ctypes.byref(out)) == 0 and out.v_head_dim == DV
    kvq.kv_pool_destroy(h)
    # a decode shape over such a pool has a workspace; the matrix engine reads DV == D only
    h = kvq.kv_pool_wrap(d, [256] * 6)
    s = kvq.DecodeShape(2, 8, 1, 64, 1024, 0, 0, 1)
    assert lib.paged_decode_workspace_bytes(h, ctypes.byref(s)) > 0
    s.engine = 2
    assert lib.paged_decode_workspace_bytes(h, ctypes.byref(s)) == 0
    kvq.kv_pool_destroy(h)


def test_value_head_dim_zero_means_head_dim(lib):
    d = kvq.PoolDesc(4, 2, 16, 128, 4, 64)                  # v_head_dim left 0
    h = kvq.kv_pool_wrap(d, [16] * 6)
    out = kvq.PoolDesc()
    assert lib.kv_pool_describe(h, ctypes.byref(out)) == 0 and out.v_head_dim == 128
    kvq.kv_pool_destroy(h)
    d.v_head_dim = -64
    with pytest.raises(kvq.KvqError) as e:
        kvq.kv_pool_wrap(d, [16] * 6)
    assert e.value.code == -1


class _FakePool:
    def __init__(self, bits=4, HK=2, BS=32, D=256, NB=64):
        self.desc = kvq.PoolDesc(NB, HK, BS, D, bits, 64)
        self.handle = kvq.kv_pool_wrap(self.desc, [256] * 6)   # host-side handle only

    def close(self):
        kvq.kv_pool_destroy(self.handle)


@pytest.mark.parametrize("mut,code", [(dict(q_rows=129), -2), (dict(q_rows=0), -2), (dict(num_q_heads=5), -2),
                                      (dict(batch=0), -1), (dict(max_len=0), -1),
                                      (dict(max_blocks_per_seq=1, max_len=1000), -6),
                                      (dict(partition_tokens=-2), -1), (dict(engine=3), -1),
                                      (dict(engine=2, partition_tokens=64), -2)])
def test_decode_shape_rejected(lib, mut, code):
    p = _FakePool()
    s = kvq.DecodeShape(2, 16, 1, 40, 1000, 0, 0, 0)
    for k, v in mut.items():
        setattr(s, k, v)
    assert lib.paged_decode_workspace_bytes(p.handle, ctypes.byref(s)) == 0
    rc = lib.paged_decode_attention(ctypes.c_void_p(256), p.handle, ctypes.c_void_p(256), ctypes.c_void_p(256),
                                    1.0, ctypes.byref(s), ctypes.c_void_p(256), 1 << 30, ctypes.c_void_p(256),
                                    None)
    assert rc == code, lib.kvq_last_error()
    p.close()


def _up(x):
    return (x + 255) // 256 * 256


def _ws_bytes(rows, D, qvecs=0, affine=True):
    """partials: rows of D floats (padded to 256 B) + rows of (max, normaliser); then the vector
    engine's q copy (per query vector D/32 blocks of 20 words) and 512 bytes the partial kernel may
    read past it"""
    total = _up(rows * D * 4) + rows * 2 * 4
    if qvecs:
        total = _up(total) + qvecs * (D // 32) * 20 * 4 + 512    # + the q copy's 512-byte tail
    return total


def test_decode_step_rejects_missing_rows(lib):
    p = _FakePool()
    s = kvq.DecodeShape(2, 16, 1, 40, 1000, 0, 0, 0)
    need = lib.paged_decode_workspace_bytes(p.handle, ctypes.byref(s))
    P = ctypes.c_void_p(256)
    assert lib.paged_decode_step(P, None, P, p.handle, P, P, 1.0, ctypes.byref(s), P, need, P, None) == -1
    assert lib.paged_decode_step(P, ctypes.c_void_p(258), P, p.handle, P, P, 1.0, ctypes.byref(s), P, need, P,
                                 None) == -1           # misaligned
    s.q_rows = 129
    assert lib.paged_decode_step(P, P, P, p.handle, P, P, 1.0, ctypes.byref(s), P, need, P, None) == -2
    p.close()


def test_workspace_too_small_and_null_pointers(lib):
    p = _FakePool()
    s = kvq.DecodeShape(2, 16, 1, 40, 1000, 256, 0, 0)
    need = lib.paged_decode_workspace_bytes(p.handle, ctypes.byref(s))
    # partials: B*HQ*N*ceil(1000/256) rows; q copy: B*HQ*N query vectors
    parts = 4
    assert need == _ws_bytes(2 * 16 * parts, 256, qvecs=2 * 16)
    rc = lib.paged_decode_attention(ctypes.c_void_p(256), p.handle, ctypes.c_void_p(256), ctypes.c_void_p(256),
                                    1.0, ctypes.byref(s), ctypes.c_void_p(256), need - 1, ctypes.c_void_p(256),
                                    None)
    assert rc == -5
    rc = lib.paged_decode_attention(None, p.handle, ctypes.c_void_p(256), ctypes.c_void_p(256), 1.0,
                                    ctypes.byref(s), ctypes.c_void_p(256), need, ctypes.c_void_p(256), None)
    assert rc == -1
    rc = lib.kv_append_quantize(p.handle, None, ctypes.c_void_p(256), ctypes.c_void_p(256), 4, None)
    assert rc == -1
    assert lib.kv_append_quantize(p.handle, None, None, None, 0, None) == 0     # T == 0 is a no-op
    p.close()


def test_automatic_schedule_is_the_balanced_stream(lib, monkeypatch):
    """partition_tokens == 0 selects the balanced stream schedule (reported as 0 tokens); its
    workspace holds (ranges + units) * 8 partial slots of a wave's query vectors (one range per
    workgroup of 8 waves)."""
    monkeypatch.delenv("KVQ_PARTITION_TOKENS", raising=False)
    p = _FakePool()
    s = kvq.DecodeShape(32, 16, 1, 1100, 32197, 0, 0, 0)
    assert lib.paged_decode_partition_tokens(p.handle, ctypes.byref(s)) == 0
    need = lib.paged_decode_workspace_bytes(p.handle, ctypes.byref(s))
    ranges = 256                                      # no device here: 256 compute units assumed
    slots = (ranges + 32 * 2) * 8 * 8                 # units = B * HK (one query group of 8),
    assert need == _ws_bytes(slots, 256, qvecs=32 * 16)   # 8 waves per range, 8 vectors
    s.partition_tokens = 300
    assert lib.paged_decode_partition_tokens(p.handle, ctypes.byref(s)) == 300
    s.partition_tokens = kvq.PARTITION_STREAM
    assert lib.paged_decode_partition_tokens(p.handle, ctypes.byref(s)) == 0
    p.close()


@pytest.mark.parametrize("batch,max_len,expect", [(1, 2048, 64), (3, 16384, 384), (4, 16384, 0), (32, 32197, 0)])
def test_automatic_schedule_for_short_streams(lib, monkeypatch, batch, max_len, expect):
    """Automatic choice: fixed partitions of about one per compute unit (a multiple of 64 tokens)
    while B * max_len * HK * query groups is below 256 compute units x 8 tiles of 64 tokens, the
    balanced stream from there on; the matrix engine always runs the stream."""
    monkeypatch.delenv("KVQ_PARTITION_TOKENS", raising=False)
    p = _FakePool()
    s = kvq.DecodeShape(batch, 16, 1, 1100, max_len, kvq.PARTITION_AUTO, 0, 0)
    assert lib.paged_decode_partition_tokens(p.handle, ctypes.byref(s)) == expect
    s.engine = kvq.ENGINE_MATRIX
    assert lib.paged_decode_partition_tokens(p.handle, ctypes.byref(s)) == 0
    p.close()


def test_matrix_engine_limits(lib):
    """The matrix-core engine reads 4-bit pages at head dim 128/256 on the stream schedule (4
    ranges per compute unit at head dim 256, a two-wave workgroup each; 8 at 128, a wave each);
    its workspace holds 16 query vectors per slot, or 8 at head dim 256 when a KV head has at
    most 8 (the pair kernel)."""
    for hq in (16, 32):                                   # 8 or 16 query vectors per KV head
        s = kvq.DecodeShape(32, hq, 1, 1100, 32197, 0, 0, 2)
        for bits, D, ok in [(4, 256, True), (4, 128, True), (8, 256, False), (16, 128, False), (4, 64, False)]:
            p = _FakePool(bits=bits, D=D)
            need = lib.paged_decode_workspace_bytes(p.handle, ctypes.byref(s))
            if ok:
                qvw = 8 if (D == 256 and hq == 16) else 16
                slots = ((4 if D == 256 else 8) * 256 + 32 * 2) * qvw
                assert need == _ws_bytes(slots, D)
            else:
                assert need == 0
            p.close()
    s = kvq.DecodeShape(32, 16, 1, 1100, 32197, 0, 0, 2)
    d = kvq.PoolDesc(64, 2, 32, 256, 4, 32)
    h = kvq.kv_pool_wrap(d, [256] * 6)
    assert lib.paged_decode_workspace_bytes(h, ctypes.byref(s)) == 0      # matrix engine: group 64 only
    kvq.kv_pool_destroy(h)


def test_noalloc_step_refuses_shapes_beyond_its_scratch(lib):
    """paged_decode_step_noalloc checks the shape's workspace against its built-in scratch before it
    touches the device: too large is KVQ_ERR_WORKSPACE, an invalid shape the allocating entry
    point's own code, a NULL pointer KVQ_ERR_INVALID."""
    src = open(HEADER).read()
    m = re.search(r"#define KVQ_NOALLOC_WORKSPACE_BYTES \((\d+)u \* 1024u \* 1024u\)", src)
    assert m and int(m.group(1)) << 20 == kvq.NOALLOC_WORKSPACE_BYTES
    p = _FakePool(NB=4096)
    P = ctypes.c_void_p(256)
    big = kvq.DecodeShape(4096, 16, 4, 1100, 32768, 0, 0, 0)
    need = lib.paged_decode_workspace_bytes(p.handle, ctypes.byref(big))
    assert need > kvq.NOALLOC_WORKSPACE_BYTES
    assert lib.paged_decode_step_noalloc(P, P, P, p.handle, P, P, 1.0, ctypes.byref(big), P, None) == -5
    assert "KVQ_NOALLOC_WORKSPACE_BYTES" in lib.kvq_last_error().decode()
    bad = kvq.DecodeShape(2, 16, 129, 40, 1000, 0, 0, 0)
    assert lib.paged_decode_step_noalloc(P, P, P, p.handle, P, P, 1.0, ctypes.byref(bad), P, None) == -2
    ok = kvq.DecodeShape(2, 16, 1, 40, 1000, 0, 0, 0)
    assert 0 < lib.paged_decode_workspace_bytes(p.handle, ctypes.byref(ok)) <= kvq.NOALLOC_WORKSPACE_BYTES
    assert lib.paged_decode_step_noalloc(P, None, P, p.handle, P, P, 1.0, ctypes.byref(ok), P, None) == -1
    p.close()


@pytest.mark.parametrize("bits,D,HQ,HK,N,pt,engine,expect", [
    (4, 256, 16, 2, 1, 0, 0, 1),      # single-row GQA 8: a matrix-vector product per KV head -> vector ALU
    (4, 256, 8, 2, 1, 0, 0, 1),       # GQA 4, one row
    (4, 256, 16, 2, 2, 0, 0, 2),      # 16 query vectors per KV head -> matrix cores
    (4, 256, 32, 4, 4, 0, 0, 2),      # 4 rows x GQA 8 (32 vectors)
    (4, 256, 32, 4, 4, -1, 0, 2),     # the stream asked for explicitly
    (4, 256, 32, 4, 4, 64, 0, 1),     # fixed partitions: the vector engine
    (4, 256, 32, 4, 4, 0, 1, 1),      # vector asked for
    (4, 256, 16, 2, 1, 0, 2, 2),      # matrix asked for
    (4, 128, 32, 4, 4, 0, 0, 2),      # head dim 128
    (8, 128, 32, 4, 4, 0, 0, 1),      # 8-bit pages: the matrix engine does not read them
    (16, 128, 32, 4, 4, 0, 0, 1),     # bf16 pages
])
def test_engine_choice(lib, bits, D, HQ, HK, N, pt, engine, expect):
    """paged_decode_engine resolves the automatic choice: the matrix cores for 16+ query vectors
    per KV head on 4-bit group-64 pages with the stream schedule, the vector ALU otherwise."""
    p = _FakePool(bits=bits, HK=HK, D=D)
    s = kvq.DecodeShape(2, HQ, N, 40, 1000, pt, 0, engine)
    assert lib.paged_decode_engine(p.handle, ctypes.byref(s)) == expect, lib.kvq_last_error()
    s.engine = 3
    assert lib.paged_decode_engine(p.handle, ctypes.byref(s)) == -1
    p.close()
