"""GPU: calls on two streams at once (two pools of different formats, each call with its own
workspace, no synchronisation between them) give the same results as one at a time -- the
library keeps no device state of its own between calls."""
import numpy as np
import pytest
import torch

import decode_attention_paged_split_amd as kvq
from oracle import attention
from tests import gpu_util as G
from workloads import make_workload

pytestmark = pytest.mark.gpu


def test_two_streams_at_once():
    wa = make_workload("c3", B=4, len_lo=500, len_hi=3000)                    # 4-bit, D 256
    wb = make_workload("c2", B=4, len_lo=500, len_hi=3000)                    # bf16, D 128
    refs = [attention.workload_output(w) for w in (wa, wb)]
    pools = [G.new_pool(w) for w in (wa, wb)]
    for w, p in zip((wa, wb), pools):
        G.fill_pool(w, p)
    args = []
    for w, p in zip((wa, wb), pools):
        q, t, l = G.u16_dev(w.q_bits), G.i32_dev(w.table), G.i32_dev(w.lengths)
        shape = kvq.make_shape(p, w.B, w.HQ, w.N, w.max_blocks, w.max_len, 0, True)
        ws = torch.empty(kvq.paged_decode_workspace_bytes(p, shape), dtype=torch.uint8, device="cuda")
        out = torch.empty((w.B, w.HQ, w.N, w.DV), dtype=torch.float32, device="cuda")
        args.append((q, p, t, l, w.scale, shape, ws, out))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for rep in range(3):
        for a, s in zip(args, streams):
            with torch.cuda.stream(s):
                kvq.paged_decode_attention(*a[:7], a[7], s)
        torch.cuda.synchronize()
        for i, a in enumerate(args):
            G.check_f32(a[7].cpu().numpy().astype(np.float64), refs[i], tag=f"stream {i} rep {rep}")
    for p in pools:
        p.close()
