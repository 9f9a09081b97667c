"""CPU oracle for paged split-K decode attention over bf16 / affine-quantized KV pages.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links this
package: only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg use it.  It shares no code with the HIP library (``decode_attention_paged_split_amd``):
the two meet only at the seeded input generator in ``workloads/``, which holds none of
the method's arithmetic.

What it computes, and from which passage of the pages (each function cites its own):

* ``bf16``      -- bf16 <-> f64, round-to-nearest-even and round-up to bf16.
* ``quant``     -- affine group quantization along the head dim (codes, bf16 scale and
                   bias per 64 elements), low-code-first packing into uint32 words,
                   unpacking and exact f64 dequantization.
* ``paged``     -- pool planes [numBlocks, HK, blockSize, width], slot writes and the
                   gather through a block table.
* ``attention`` -- the plain definition of decode attention (two-pass softmax in f64 over
                   the gathered, dequantized rows, GQA head mapping, multi-row causal
                   visibility), the split-into-partitions + log-sum-exp merge variant, and
                   the whole decode step of a workload.

Pages cited (the text of four npm-diff web pages):

* "@mlx-bun/inference 0.0.0-stage -> 1.0.0", diff page 50: src/kernels/attention/
  kvq4-decode.ts, masks.ts, multi-query.ts, paged.ts.
* "mlx-bun 0.4.0 -> 0.5.0", diff page 24: src/lab/paged-kv/*.
* "@mlx-bun/inference 0.0.0-stage -> 1.0.0", diff page 134: src/state/paged/cache.ts.
* "mlx-bun 0.2.0 -> 0.4.0", diff page 47: model/batched-quantized-kv.ts and friends.

Every public function here is pinned by ``tests/test_oracle_*.py`` (worked words, closed
forms, brute force, a library routine); the helpers (``bf16.next_up``,
``quant.levels``, ``attention.workload_kv``) are reached only through a pinned function that
calls them, so a mistake in one fails that function's pins.  None is "parity unpinned".
"""
from . import bf16, quant, paged, attention  # noqa: F401
