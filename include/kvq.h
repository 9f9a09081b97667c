/*
 * kvq.h -- paged, split-K decode attention over bf16 or affine-quantized KV pages,
 * for AMD Instinct MI355X (gfx950).  Plain C ABI: pointers, sizes and status codes; no
 * HIP or PyTorch types appear in any signature (the stream is an opaque `void*` that
 * holds a hipStream_t; NULL means the default stream).
 *
 * Pages this interface follows (the text of four npm-diff web pages):
 *   [P50]  "@mlx-bun/inference 0.0.0-stage -> 1.0.0", diff page 50:
 *          src/kernels/attention/kvq4-decode.ts, paged.ts, multi-query.ts
 *   [P134] "@mlx-bun/inference 0.0.0-stage -> 1.0.0", diff page 134:
 *          src/state/paged/cache.ts
 *   [P47]  "mlx-bun 0.2.0 -> 0.4.0", diff page 47: model/batched-quantized-kv.ts
 *
 * Environment (tuning sweeps only; unset in normal use):
 *   KVQ_PARTITION_TOKENS=n  (n > 0) replaces the automatic partition choice of
 *                           partition_tokens == 0 by fixed partitions of n tokens.
 *   KVQ_MFMA_RANGES_PER_CU=n  ranges per compute unit of the matrix-core engine's stream
 *                           (2..16; default 4 at head dim 256, 8 at 128).
 *   KVQ_STREAM_LANES=n      query groups of a KV head worked side by side on the balanced
 *                           stream (1, 2 or 4, dividing the group count; default 4, 2 or 1 by
 *                           divisibility).
 *   KVQ_SET_COST=n          vector engine, balanced stream: positions charged per (sequence, KV
 *                           head) set ahead of its tokens, so that ranges that change sets get
 *                           fewer tokens (0..4096; default 512).
 * Each call reads these when it is made; they decide where the partials lie, so a partial call
 * and the merge call that reads its partials must run under the same values.
 *
 * Conventions shared by every entry point
 *   - Return value: KVQ_OK (0) or a negative kvq_status.  A failing call enqueues
 *     nothing; kvq_last_error() then returns a message for the calling thread.
 *   - Device pointers are borrowed for the stream-ordered duration of the call; the
 *     library never frees caller memory.  All tensors are dense, row-major, in the
 *     layouts stated below.
 *   - Calls enqueue work on `stream` and return without synchronising.  The only
 *     synchronous errors are argument checks; a device fault surfaces at the caller's
 *     next synchronisation.
 *   - bf16 values travel as their 16-bit patterns (uint16_t).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_INVALID = -1,      /* bad argument: null pointer, shape, size */
  KVQ_ERR_UNSUPPORTED = -2,  /* a format or shape this library does not read directly */
  KVQ_ERR_OOM = -3,          /* device allocation failed */
  KVQ_ERR_HIP = -4,          /* a HIP runtime call failed (message has the HIP error) */
  KVQ_ERR_WORKSPACE = -5,    /* workspace smaller than paged_decode_workspace_bytes() */
  KVQ_ERR_RANGE = -6         /* a size beyond the pool (the pages' PagedPoolExhausted) */
} kvq_status;

/* Pool planes, each shaped [num_blocks, num_kv_heads, block_size, width] ([P134]
 * cache.ts, class BlockPool).  bf16 pages (bits == 16) have only K and V (uint16, width
 * head_dim).  Affine pages have packed codes K and V (uint32, width head_dim*bits/32) and
 * bf16 scale and bias planes of width head_dim/group_size.  The V planes take v_head_dim in
 * place of head_dim (the pool's vHeadDim, which defaults to headDim).  A row's codes are one
 * little-endian bit stream: element i in stream bits [bits*i, bits*i + bits), stream bit k in
 * bit k%32 of word k/32.  For widths dividing 32 that is bits [bits*(i%P), bits*(i%P+1)) of
 * word i/P, P = 32/bits ([P50] paged.ts, paged_attention_affine_partial); 3-, 5- and 6-bit
 * codes straddle words ([P134] paged.ts, directReadable, names such widths but reads them
 * only through the library's dequantize, so their layout is this build's reading). */
typedef enum kvq_plane {
  KVQ_PLANE_K = 0,
  KVQ_PLANE_V = 1,
  KVQ_PLANE_K_SCALE = 2,
  KVQ_PLANE_K_BIAS = 3,
  KVQ_PLANE_V_SCALE = 4,
  KVQ_PLANE_V_BIAS = 5
} kvq_plane;
#define KVQ_NUM_PLANES 6

typedef struct kvq_pool_desc {
  int32_t num_blocks;    /* physical blocks NB >= 1 */
  int32_t num_kv_heads;  /* HK >= 1 */
  int32_t block_size;    /* tokens per block BS >= 1 */
  int32_t head_dim;      /* D, a multiple of group_size, at most 256 */
  int32_t bits;          /* 16 = bf16 pages; 8, 6, 5, 4, 3 or 2 = affine codes; a row of codes
                            (head_dim*bits/8 bytes) must be whole 16-byte chunks */
  int32_t group_size;    /* elements per scale/bias group along the head dim: 32, 64 or 128 */
  int32_t v_head_dim;    /* DV, the V rows' head dim ([P50] paged.ts reads DK and DV); 0 = head_dim.
                            A DV other than head_dim is read by the vector engine for bf16, 8-,
                            4- and 2-bit pages with group_size 64 (affine) and DV = head_dim / 2
                            or 2 * head_dim within 64..256; other pairs are KVQ_ERR_UNSUPPORTED */
} kvq_pool_desc;

typedef struct kvq_pool kvq_pool;  /* opaque */

/* Bytes of one plane of a pool with this descriptor (0 for a plane the format lacks or
 * an invalid descriptor). */
size_t kv_pool_plane_bytes(const kvq_pool_desc* desc, int32_t plane);

/* Create a pool whose planes the library allocates on the current device and fills with
 * zeros (the pages' pool starts as ops.zeros: [P134] BlockPool constructor).  The library
 * owns the planes until kv_pool_destroy.  Errors: KVQ_ERR_INVALID (descriptor),
 * KVQ_ERR_UNSUPPORTED (bits/group), KVQ_ERR_OOM. */
int kv_pool_create(const kvq_pool_desc* desc, kvq_pool** out);

/* Create a pool over planes the caller allocated (planes[p] for every plane the format
 * has, each at least kv_pool_plane_bytes(desc, p) bytes, 16-byte aligned; entries for
 * absent planes are ignored).  The caller keeps ownership; kv_pool_destroy frees only the
 * handle.  Errors: KVQ_ERR_INVALID, KVQ_ERR_UNSUPPORTED. */
int kv_pool_wrap(const kvq_pool_desc* desc, void* const planes[KVQ_NUM_PLANES], kvq_pool** out);

/* Release a pool handle (and its planes if the library allocated them).  NULL is a no-op.
 * Work still queued on a stream that reads the pool must finish first.  The pages' pool
 * releases its planes the same way ([P134] cache.ts, BlockPool.dispose: scales, biases, keys
 * and values disposed, the free list emptied), while a view over it releases only what it
 * holds itself ([P50] paged.ts, pagedAttentionView's dispose) -- here a wrapped pool
 * (kv_pool_wrap) is such a borrower: only the handle is freed. */
int kv_pool_destroy(kvq_pool* pool);

/* Device address and size of one plane, as the pages' pool lists its arrays ([P134] cache.ts,
 * BlockPool.arrays: keys, values, then keyScales, keyBiases, valueScales, valueBiases where the
 * format has them).  The pointer is the library's (kv_pool_create) or the caller's (kv_pool_wrap);
 * it stays valid until kv_pool_destroy.  Errors: KVQ_ERR_INVALID for a NULL argument or a plane
 * the format lacks (bf16 pages have no scale or bias planes). */
int kv_pool_plane(const kvq_pool* pool, int32_t plane, void** dev_ptr, size_t* bytes);

/* Copy a pool's descriptor out. */
int kv_pool_describe(const kvq_pool* pool, kvq_pool_desc* out);

/* Quantize-on-append ([P134] cache.ts, BlockPool.writeBlock and PagedKVCache.append):
 * write T new K/V rows into the pool, quantizing affine pages per (token, head, group of
 * group_size elements):  mn, mx = min, max; scale = (mx - mn) / (2^bits - 1) in f32,
 * rounded up to bf16; bias = mn; code = clamp(rint((x - bias) / scale), 0, 2^bits - 1)
 * (round half to even; a group with scale 0 stores code 0); codes packed low-first.
 *   k, v   device bf16 [T, num_kv_heads, head_dim] and [T, num_kv_heads, v_head_dim]
 *   slots  device int64 [T]: physical slot = block * block_size + row; a negative slot
 *          skips its row; a slot >= num_blocks * block_size is skipped as well.
 * Rows of one call must target distinct slots.  T == 0 is a no-op. */
int kv_append_quantize(kvq_pool* pool, const uint16_t* k, const uint16_t* v,
                       const int64_t* slots, int32_t num_tokens, void* stream);

/* Most query rows per sequence one call reads straight from the pages.  N <= 8 is the decode
 * case ([P50] kvq4-decode.ts reads up to 8 rows per sequence directly); larger N is a window of
 * new rows -- a prefill chunk or a speculative-verify window -- that the pages send through
 * gather + SDPA ([P50] paged.ts, the gathered route) and this library reads from the pages with the
 * same kernels: every block of query vectors of a KV head is one more unit of the partial pass,
 * row i seeing t < lengths[b] - N + i + 1.  The matrix engine suits such windows: its 16-vector
 * groups put all of a KV head's rows on the matrix cores. */
#define KVQ_MAX_Q_ROWS 128

enum { KVQ_PARTITION_AUTO = 0, KVQ_PARTITION_STREAM = -1 };

typedef struct kvq_decode_shape {
  int32_t batch;               /* B sequences */
  int32_t num_q_heads;         /* HQ, a multiple of the pool's HK */
  int32_t q_rows;              /* N query rows per sequence, 1..KVQ_MAX_Q_ROWS */
  int32_t max_blocks_per_seq;  /* columns of block_table */
  int32_t max_len;             /* host upper bound on every lengths[b] (sizes the grid) */
  int32_t partition_tokens;    /* > 0: fixed split-K partitions of this many tokens;
                                  KVQ_PARTITION_AUTO (0): the balanced stream, or, when B * max_len *
                                  HK * query groups is too few tokens to give every compute unit
                                  8 tiles of 64, fixed partitions of about one per compute unit;
                                  KVQ_PARTITION_STREAM (-1): the balanced stream */
  int32_t out_f32;             /* 0: out is bf16; 1: out is f32 (unrounded merge result) */
  int32_t engine;              /* kvq_engine: which units compute q.k and P.V */
} kvq_decode_shape;

/* Engines of the partial pass.  Both compute the same quantity to the tolerances stated for
 * paged_decode_attention.
 *   KVQ_ENGINE_VECTOR: vector ALU -- v_dot2_f32_bf16 for q.k, f32 FMA for P.V; every format.
 *   KVQ_ENGINE_MATRIX: matrix cores -- q.k with exact bf16 products, P.V with exact f16 codes
 *     against the weight split into two f16 halves (~2^-22 relative, at any V scale: the weights
 *     are prescaled by a power of two per scale group and the factor taken back exactly, so the
 *     output on V times 2^e is exactly 2^e times the output on V); 4-bit pages, head_dim
 *     128 or 256 (v_head_dim the same), the balanced stream only (partition_tokens <= 0).  It serves the GQA groups where the vector ALU
 *     rather than HBM bounds the pass ([P50] multi-query.ts puts a KV head's query rows on the
 *     matrix unit for the same reason).
 *   KVQ_ENGINE_AUTO: the matrix engine where it applies and a KV head carries at least 16 query
 *     vectors (HQ / HK * q_rows >= 16: several query rows per sequence make the per-head work a
 *     matrix-matrix product, which [P50] multi-query.ts also gives to the matrix unit) and
 *     partition_tokens <= 0; else the vector engine (single-row decode, a matrix-vector product
 *     bound by memory or the vector ALU).  paged_decode_engine reports the choice. */
enum kvq_engine { KVQ_ENGINE_AUTO = 0, KVQ_ENGINE_VECTOR = 1, KVQ_ENGINE_MATRIX = 2 };

/* Bytes of workspace paged_decode_attention needs for this shape (0 if the shape is invalid;
 * kvq_last_error() then says why).  The workspace holds what the pages' direct route allocates
 * per call and releases after the merge ([P50] paged.ts, pagedAttentionView.attend: the partial
 * outputs `out` [hq, n, parts, dv] f32 and `normal` [hq, n, parts, 2] f32 -- running max and
 * normaliser -- disposed in its finally): f32 partial rows (o, m, l) per partition or per
 * stream slot, and the vector engine's copy of q.  Here the caller owns that memory (e.g. one
 * torch.empty reused across steps); its content between calls is scratch. */
size_t paged_decode_workspace_bytes(const kvq_pool* pool, const kvq_decode_shape* shape);

/* Partition size the library uses for this shape: the fixed partition's tokens, or 0 for the
 * balanced stream (for reporting). */
int32_t paged_decode_partition_tokens(const kvq_pool* pool, const kvq_decode_shape* shape);

/* Engine the library uses for this shape: KVQ_ENGINE_VECTOR or KVQ_ENGINE_MATRIX (the automatic
 * choice resolved; for reporting), or a negative kvq_status if the shape is invalid for the pool. */
int32_t paged_decode_engine(const kvq_pool* pool, const kvq_decode_shape* shape);

/* Decode attention for N <= KVQ_MAX_Q_ROWS query rows per sequence read straight from the pages
 * ([P50] paged.ts pagedAttentionView.attend, direct route; kvq4-decode.ts):
 *   out[b, h, i, :] = sum_t softmax_t(scale * q[b,h,i,:] . K[b,t,g,:]) V[b,t,g,:]
 * (K rows of head_dim, V rows and out rows of v_head_dim)
 * over t < lengths[b] - N + i + 1, with g = h / (HQ / HK) (GQA), K and V the dequantized
 * page rows (scale * code + bias in f32) or the bf16 rows.  Token t of sequence b sits in
 * block block_table[b, t / BS], row t % BS.  Computed as a split-K partial pass (online
 * softmax in f32 per partition, every K/V row read once for all HQ/HK heads of its
 * group) followed by a log-sum-exp merge.
 *   q            device bf16 [B, HQ, N, head_dim]
 *   block_table  device int32 [B, max_blocks_per_seq]; entries past ceil(len/BS) unread
 *   lengths      device int32 [B]; each in [N, max_len] (tokens cached, counting the N
 *                new rows); not checked on the device
 *   workspace    device, >= paged_decode_workspace_bytes(pool, shape) bytes
 *   out          device [B, HQ, N, v_head_dim], bf16 (round to nearest even) or f32
 * Errors: KVQ_ERR_INVALID, KVQ_ERR_UNSUPPORTED (N > KVQ_MAX_Q_ROWS, HQ % HK != 0),
 * KVQ_ERR_WORKSPACE. */
int paged_decode_attention(const uint16_t* q, const kvq_pool* pool, const int32_t* block_table,
                           const int32_t* lengths, float scale, const kvq_decode_shape* shape,
                           void* workspace, size_t workspace_bytes, void* out, void* stream);

/* The two halves of paged_decode_attention, for callers that time or exchange partials
 * (e.g. a context-parallel split that merges partials gathered from several devices):
 * paged_decode_partial writes the per-partition (o, m, l) partials into the workspace;
 * paged_decode_merge combines them into out ([P50] paged.ts paged_attention_merge).  Same
 * arguments, layouts and errors as paged_decode_attention; the merge must be given the
 * same shape (and partition size) the partial pass used. */
int paged_decode_partial(const uint16_t* q, const kvq_pool* pool, const int32_t* block_table,
                         const int32_t* lengths, float scale, const kvq_decode_shape* shape,
                         void* workspace, size_t workspace_bytes, void* stream);
int paged_decode_merge(const kvq_pool* pool, const int32_t* lengths, const kvq_decode_shape* shape,
                       const void* workspace, size_t workspace_bytes, void* out, void* stream);

/* One decode step on the device ([P134] cache.ts PagedKVCache.appendDecode: append the step's
 * rows, then attend over the view that includes them; [P50] paged.ts direct route): the N new
 * K/V rows of every sequence are quantized on append (same quantizer as kv_append_quantize) into
 * the slots their positions take in the block table -- row i of sequence b at position
 * lengths[b] - N + i, block block_table[b, pos / BS], row pos % BS -- and then
 * paged_decode_attention runs over the updated pool, all on the given stream with no host-side
 * slot mapping.
 *   k_new, v_new  device bf16 [B, N, num_kv_heads, head_dim] and [B, N, num_kv_heads, v_head_dim],
 *                 16-byte aligned
 *   other arguments as paged_decode_attention; lengths count the new rows, and the blocks of
 *   the new positions must already be in the table (allocation is the caller's).
 * A new row whose position is outside [0, min(max_len, max_blocks_per_seq * BS)) or whose
 * table entry is outside [0, num_blocks) is not written.
 * Errors: as paged_decode_attention, and KVQ_ERR_INVALID for NULL or misaligned k_new/v_new. */
int paged_decode_step(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new, kvq_pool* pool,
                      const int32_t* block_table, const int32_t* lengths, float scale,
                      const kvq_decode_shape* shape, void* workspace, size_t workspace_bytes, void* out,
                      void* stream);

/* The first half of paged_decode_step (append of the new rows and the partial pass, partials
 * left in the workspace); paged_decode_merge with the same shape completes it.  Same arguments
 * and errors as paged_decode_step without out. */
int paged_decode_step_partial(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new, kvq_pool* pool,
                              const int32_t* block_table, const int32_t* lengths, float scale,
                              const kvq_decode_shape* shape, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Bytes of the scratch array paged_decode_step_noalloc uses as its workspace (64 MiB). */
#define KVQ_NOALLOC_WORKSPACE_BYTES (64u * 1024u * 1024u)

/* paged_decode_step for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments, layouts, results
 * and errors as paged_decode_step, without workspace: the partials and the q copy live in a
 * library-owned device array of KVQ_NOALLOC_WORKSPACE_BYTES bytes, one per device, which that
 * device holds from the first call on it until the process ends (its address is looked up once
 * per device, on that first call).  The call itself allocates nothing (no hipMalloc or hipFree, no
 * allocating library routine; the launch-timing aid, when switched on, creates its events on
 * first use).  A shape whose paged_decode_workspace_bytes() exceeds KVQ_NOALLOC_WORKSPACE_BYTES is
 * refused with KVQ_ERR_WORKSPACE before the device is touched.  Every call on a device shares that
 * device's array and leaves its content behind (no kernel relies on it being zero): calls that
 * overlap on one device -- on two streams, or from two threads without ordering -- race, and the
 * caller must serialise them. */
int paged_decode_step_noalloc(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new, kvq_pool* pool,
                              const int32_t* block_table, const int32_t* lengths, float scale,
                              const kvq_decode_shape* shape, void* out, void* stream);

/* The fetch copy, for indexing tests ([P134] cache.ts pickBlocks / BlockPool.gather):
 * every plane's rows of each sequence in token order.  out_planes[p] (device) receives
 * plane p as [B, num_kv_heads, max_len, width_p] in the plane's element type; rows at
 * t >= lengths[b] are written as zero.  Entries for absent planes are ignored. */
int kv_gather_debug(const kvq_pool* pool, const int32_t* block_table, const int32_t* lengths,
                    int32_t batch, int32_t max_blocks_per_seq, int32_t max_len,
                    void* const out_planes[KVQ_NUM_PLANES], void* stream);

/* Launch timing, a measurement aid.  While on, every launch of the kinds below records one
 * hipEvent on its stream right before it and one right after it, so an event pair brackets the
 * kernel alone (events on the kernel's own stream, not the caller's view of it):
 *   KVQ_TIMING_PREP    the decode step's first kernel (append of the new rows + q copy)
 *   KVQ_TIMING_PARTIAL the partial kernel (outside the decode step it also brackets the q copy
 *                      the vector engine launches right before it)
 *   KVQ_TIMING_MERGE   the merge kernel
 * kvq_timing_enable(1) starts recording, (0) stops it; both forget what was recorded.
 * kvq_timing_read(kind, &avg_ms, &count) waits for the kind's recorded events, returns the mean
 * duration of its launches since the last read (0 and count 0 if none) and forgets them.
 * Process-wide state behind a lock; the events are the library's, created on first use.  At most
 * 32768 launches are recorded between reads (later ones run unrecorded). */
typedef enum kvq_timing_kind { KVQ_TIMING_PREP = 0, KVQ_TIMING_PARTIAL = 1, KVQ_TIMING_MERGE = 2 } kvq_timing_kind;
int kvq_timing_enable(int32_t on);
int kvq_timing_read(int32_t kind, double* avg_ms, int32_t* count);

/* Streaming-read probe, a measurement aid: enqueues one kernel that reads every byte of buf
 * (device, 16-byte aligned, bytes a positive multiple of 16) once with 16-byte loads, from 32
 * workgroups of 256 threads per compute unit, four loads in flight per thread.  It writes
 * nothing but, in the unlikely case that the folded words hit one fixed constant, sink (a device
 * uint32 whose content is then undefined); the fold keeps the loads alive.  The caller times it
 * (events around the call).  Errors: KVQ_ERR_INVALID for NULL or misaligned pointers or a bad
 * size. */
int kvq_probe_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);
/* The same probe with its launch shape chosen: loads_in_flight 16-byte loads per thread at a time
 * (1, 2, 4, 8 or 16), non-temporal loads when nontemporal != 0, blocks_per_cu workgroups of 256
 * threads per compute unit (1..64); kvq_probe_read is (4, 0, 32).  For finding the device's
 * streaming-read ceiling.  Errors: as kvq_probe_read, and KVQ_ERR_INVALID for a value outside
 * those sets. */
int kvq_probe_read_ex(const void* buf, size_t bytes, uint32_t* sink, int32_t loads_in_flight, int32_t nontemporal,
                      int32_t blocks_per_cu, void* stream);

/* Pool-read probe, a measurement aid: enqueues one kernel that reads every cached row of every
 * (sequence, KV head) of the pool -- K and V codes or values and, for affine pages, the four
 * scale and bias planes -- reached through block_table ([batch, max_blocks_per_seq] int32,
 * device) for the tokens t < min(lengths[b], max_len, max_blocks_per_seq * block_size) (lengths:
 * [batch] int32, device), with no arithmetic.  coalesced = 0: one token per lane, each lane
 * loading its row in 16-byte pieces (the partial kernel's pattern); coalesced != 0: consecutive
 * lanes load consecutive 16-byte pieces of the rows a block holds contiguously for one KV head.
 * Either way one wave takes 64 tokens and issues all its K/V loads before using any.  Table
 * entries outside the pool are clamped into it.  sink as for kvq_probe_read.  The caller times
 * it.  Errors: KVQ_ERR_INVALID for NULL or misaligned pointers or non-positive sizes,
 * KVQ_ERR_UNSUPPORTED unless K and V rows are equal and 32, 64, 96, 128, 256 or 512 bytes. */
int kvq_probe_pool_read(const kvq_pool* pool, const int32_t* block_table, const int32_t* lengths, int32_t batch,
                        int32_t max_blocks_per_seq, int32_t max_len, int32_t coalesced, uint32_t* sink,
                        void* stream);

/* Message for the calling thread's last failing call ("" if none).  The pages fail with a typed
 * error that carries a message, never a silent truncation ([P134] cache.ts, PagedPoolExhausted:
 * the pool's block count in the message; [P50] multi-query.ts throws with the offending size);
 * here the kvq_status code is the type and this string the message.  Thread-local; valid until
 * the thread's next failing call. */
const char* kvq_last_error(void);

/* Library version string. */
const char* kvq_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
