// kvq C ABI: argument validation, pool management, launch configuration.
// Declarations and the contract of every entry point are in include/kvq.h.
#include "../../include/kvq.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.hpp"

struct kvq_pool {
  kvq_pool_desc desc;
  void* planes[KVQ_NUM_PLANES];
  size_t bytes[KVQ_NUM_PLANES];
  bool owned;
};

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(KVQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int plane_count(int bits) { return bits == 16 ? 2 : 6; }

// the V rows' head dim (0 in a descriptor stands for head_dim)
int v_dim(const kvq_pool_desc* d) { return d->v_head_dim ? d->v_head_dim : d->head_dim; }

int validate_desc(const kvq_pool_desc* d) {
  if (!d) return fail(KVQ_ERR_INVALID, "pool descriptor is NULL");
  if (d->num_blocks < 1 || d->num_kv_heads < 1 || d->block_size < 1 || d->head_dim < 1)
    return fail(KVQ_ERR_INVALID, "pool sizes must be positive (NB=%d HK=%d BS=%d D=%d)",
                d->num_blocks, d->num_kv_heads, d->block_size, d->head_dim);
  if (!(d->bits == 16 || d->bits == 8 || d->bits == 6 || d->bits == 5 || d->bits == 4 || d->bits == 3 ||
        d->bits == 2))
    return fail(KVQ_ERR_UNSUPPORTED, "bits must be 16 (bf16 pages) or 8, 6, 5, 4, 3, 2 (affine), got %d", d->bits);
  if (d->head_dim % 64 != 0 || d->head_dim > 256)
    return fail(KVQ_ERR_UNSUPPORTED, "head_dim must be 64, 128 or 256, got %d", d->head_dim);
  if (!kvq::valu_row_ok(d->bits, d->head_dim))
    return fail(KVQ_ERR_UNSUPPORTED, "a %d-bit row of %d dims is %d bytes; rows must be whole 16-byte chunks",
                d->bits, d->head_dim, d->head_dim * d->bits / 8);
  if (!(d->group_size == 32 || d->group_size == 64 || d->group_size == 128) || d->head_dim % d->group_size != 0)
    return fail(KVQ_ERR_UNSUPPORTED, "group_size must be 32, 64 or 128 and divide head_dim, got %d", d->group_size);
  const int dv = v_dim(d);
  if (d->v_head_dim < 0) return fail(KVQ_ERR_INVALID, "v_head_dim must be >= 0 (0: head_dim), got %d", d->v_head_dim);
  if (dv != d->head_dim && !kvq::valu_dv_ok(d->bits, d->head_dim, dv, d->group_size))
    return fail(KVQ_ERR_UNSUPPORTED,
                "v_head_dim %d with head_dim %d: a V head dim of its own must be head_dim / 2 or 2 * head_dim "
                "within 64..256, on bf16, 8-, 4- or 2-bit pages with group_size 64", dv, d->head_dim);
  const size_t rows = (size_t)d->num_blocks * d->num_kv_heads * d->block_size;
  if (rows >= (size_t)1 << 31)
    return fail(KVQ_ERR_UNSUPPORTED, "num_blocks * num_kv_heads * block_size must stay below 2^31 rows");
  return KVQ_OK;
}

size_t plane_row_bytes(const kvq_pool_desc* d, int plane) {
  const bool vp = plane == KVQ_PLANE_V || plane == KVQ_PLANE_V_SCALE || plane == KVQ_PLANE_V_BIAS;
  const size_t dim = (size_t)(vp ? v_dim(d) : d->head_dim);
  if (d->bits == 16) return (plane <= KVQ_PLANE_V) ? dim * 2 : 0;
  if (plane <= KVQ_PLANE_V) return dim * d->bits / 8;
  if (plane < KVQ_NUM_PLANES) return (dim / d->group_size) * 2;
  return 0;
}

int device_cus() {
  static int cus = 0;
  static std::once_flag once;
  std::call_once(once, [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  });
  return cus;
}

constexpr int MAX_PARTS = 8192;

// query vectors per workgroup: the largest power of two <= kvq::valu_max_qvw dividing REP * N
int qvw_for(int qv, int bits, int D, int DV, int gs) {
  for (int w = kvq::valu_max_qvw(bits, D, DV, gs); w >= 1; w /= 2)
    if (qv % w == 0) return w;
  return 1;
}

// The engine of the partial pass: the matrix cores when asked for, or (automatic choice) when a
// KV head carries at least one full MFMA column block of query vectors (REP * N >= 16: several
// query rows per sequence, a matrix-matrix product per KV head, which the pages' multi-row
// kernel also gives to the matrix unit), the format is one the matrix engine reads and the
// schedule is the stream; else the vector ALU (single-row decode: a matrix-vector product).
bool use_mfma(const kvq_pool* pool, const kvq_decode_shape* s) {
  if (s->engine == KVQ_ENGINE_MATRIX) return true;
  if (s->engine != KVQ_ENGINE_AUTO || s->partition_tokens > 0) return false;
  const kvq_pool_desc& d = pool->desc;
  if (d.num_kv_heads < 1 || s->num_q_heads % d.num_kv_heads != 0) return false;
  const int qv = (s->num_q_heads / d.num_kv_heads) * s->q_rows;
  return qv >= kvq::MFMA_QVW && kvq::mfma_supported(d.bits, d.head_dim, d.group_size) &&
         d.v_head_dim == d.head_dim;
}
int qgroups_of(const kvq_pool* pool, const kvq_decode_shape* s);

// Tokens per split-K partition for the fixed-partition schedule; 0 selects the balanced
// stream schedule (every wave gets an equal share of all cached tokens).  KVQ_PARTITION_TOKENS
// (> 0) overrides an automatic choice of the vector engine, for sweeps.
int choose_partition(const kvq_pool* pool, const kvq_decode_shape* s) {
  if (s->partition_tokens > 0) return s->partition_tokens;
  if (s->partition_tokens == KVQ_PARTITION_STREAM) return 0;
  if (use_mfma(pool, s)) return 0;
  if (const char* e = std::getenv("KVQ_PARTITION_TOKENS")) {
    const int v = std::atoi(e);
    if (v > 0) return v;
  }
  // A stream too short to give every compute unit a full range of 8 tiles (at most
  // B * max_len * HK * query groups tokens: the lengths themselves are on the device) runs as
  // fixed partitions instead, sized so that there are about as many partitions as compute
  // units: then every tile has a compute unit of its own and each output row has few partials
  // to merge, where the stream would pile a range's tiles on one unit.
  const double bound = (double)s->batch * s->max_len * pool->desc.num_kv_heads * qgroups_of(pool, s);
  const double full = (double)device_cus() * kvq::VALU_STREAM_WAVES * kvq::VALU_TILE;
  if (bound >= full) return 0;
  const double per = bound / device_cus();
  return kvq::VALU_TILE * std::max(1, (int)std::ceil(per / kvq::VALU_TILE));
}

// Stream schedule: the most ranges the stream is cut into and the partial slots per (unit, range).
// Every range's waves are resident at once.  The vector engine launches one workgroup of 8 waves
// (two per SIMD) per compute unit, whose waves share its range's tiles: a slot per (unit, range,
// wave), of which the range's last unit uses only the first (its waves combine in LDS).  The matrix engine runs two
// waves per SIMD: at head dim 256 a workgroup of two waves (one per half of the head dim) works one
// range, 4 workgroups per compute unit; at head dim 128 each of 8 waves per compute unit works a
// range of its own.  KVQ_MFMA_RANGES_PER_CU overrides the 4 / 8, for sweeps.
struct StreamGeom {
  int ranges, sub, min_tokens;
};

StreamGeom stream_geom(const kvq_pool* pool, const kvq_decode_shape* s) {
  if (use_mfma(pool, s)) {
    const bool split = pool->desc.head_dim == 256;
    int per_cu = split ? 4 : 8;
    if (const char* e = std::getenv("KVQ_MFMA_RANGES_PER_CU")) per_cu = std::max(2, std::min(16, std::atoi(e)));
    if (!split) per_cu &= ~1;                     // whole workgroups of two independent waves
    return {per_cu * device_cus(), 1, kvq::MFMA_TILE};
  }
  return {device_cus(), kvq::VALU_STREAM_WAVES, kvq::VALU_STREAM_WAVES * kvq::VALU_TILE};
}

// Stream schedule: the query groups of one KV head worked side by side on one range, by L
// workgroups on one XCD (one group each), so that each K/V row is fetched from memory once for
// all of them: 4 when the groups come in fours, 2 when in pairs, else 1 (the vector engine, and
// the matrix engine's head-dim-256 kernel for 16-vector groups).  KVQ_STREAM_LANES (1, 2 or 4,
// dividing the group count) overrides, for measurements.
int stream_lanes(int qgroups, int pt, bool mfma, int qvw, int head_dim) {
  if (pt != 0) return 1;
  // the matrix engine runs side-by-side groups in its head-dim-256 kernel for more than 8 vectors
  // per KV head (the split kernel, one 16-vector group per workgroup)
  if (mfma && !(head_dim == 256 && qvw == kvq::MFMA_QVW)) return 1;
  int L = qgroups % 4 == 0 ? 4 : (qgroups % 2 == 0 ? 2 : 1);
  if (const char* e = std::getenv("KVQ_STREAM_LANES")) {
    const int v = std::atoi(e);
    if ((v == 1 || v == 2 || v == 4) && qgroups % v == 0) L = v;
  }
  return L;
}

// Vector engine, stream schedule: positions charged per set that has tokens, ahead of its tokens.
// A wave that changes sets inside its range writes its partial of the old set and waits for the
// new set's q copy and first rows (about 9 us per wave on the 4-bit GQA-8 workload with ragged
// lengths, measured with per-wave timestamps); ranges holding a set change finished 6.5 us later
// than the others, and the slowest of them set the kernel's end.  The charge gives such a range
// that many fewer tokens (the kernel drops it where no range holds a set change: equal lengths
// whose sets divide the ranges evenly).  512 measured best (partial kernel on that workload
// 172 -> 162 us; 4-row 4-bit 2,157 -> 2,137 us; bf16 GQA-4 35.8 -> 34.9 us).  KVQ_SET_COST
// (0 .. 4096 tokens) overrides, for measurements.
int stream_set_cost() {
  int c = kvq::VALU_SET_COST;
  if (const char* e = std::getenv("KVQ_SET_COST")) c = std::max(0, std::min(4096, std::atoi(e)));
  return c;
}

// query vectors per workgroup (vector ALU) or per wave (matrix cores, padded to 16)
int qvw_of(const kvq_pool* pool, const kvq_decode_shape* s) {
  const int qv = (s->num_q_heads / pool->desc.num_kv_heads) * s->q_rows;
  if (use_mfma(pool, s))
    return (pool->desc.head_dim == 256 && qv <= kvq::MFMA_PAIR_QVW) ? kvq::MFMA_PAIR_QVW : kvq::MFMA_QVW;
  return qvw_for(qv, pool->desc.bits, pool->desc.head_dim, pool->desc.v_head_dim, pool->desc.group_size);
}

int qgroups_of(const kvq_pool* pool, const kvq_decode_shape* s) {
  const int qv = (s->num_q_heads / pool->desc.num_kv_heads) * s->q_rows;
  const int w = qvw_of(pool, s);
  return (qv + w - 1) / w;
}

int validate_shape(const kvq_pool* pool, const kvq_decode_shape* s) {
  if (!pool) return fail(KVQ_ERR_INVALID, "pool is NULL");
  if (!s) return fail(KVQ_ERR_INVALID, "decode shape is NULL");
  if (s->batch < 1 || s->num_q_heads < 1 || s->max_blocks_per_seq < 1 || s->max_len < 1)
    return fail(KVQ_ERR_INVALID, "batch, num_q_heads, max_blocks_per_seq and max_len must be positive");
  if (s->q_rows < 1 || s->q_rows > KVQ_MAX_Q_ROWS)
    return fail(KVQ_ERR_UNSUPPORTED, "q_rows must be 1..%d, got %d", KVQ_MAX_Q_ROWS, s->q_rows);
  if (s->num_q_heads % pool->desc.num_kv_heads != 0)
    return fail(KVQ_ERR_UNSUPPORTED, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)",
                s->num_q_heads, pool->desc.num_kv_heads);
  if (s->q_rows > s->max_len) return fail(KVQ_ERR_INVALID, "q_rows exceeds max_len");
  if (s->batch > 65535 || (long)pool->desc.num_kv_heads * s->num_q_heads > 65535)
    return fail(KVQ_ERR_UNSUPPORTED, "batch and num_q_heads * num_kv_heads must stay below 65536");
  if ((long)s->max_blocks_per_seq * pool->desc.block_size < s->max_len)
    return fail(KVQ_ERR_RANGE, "max_len %d exceeds the block table's capacity %ld tokens", s->max_len,
                (long)s->max_blocks_per_seq * pool->desc.block_size);
  if (s->partition_tokens < KVQ_PARTITION_STREAM)
    return fail(KVQ_ERR_INVALID, "partition_tokens must be > 0, 0 (automatic) or -1 (balanced stream)");
  const int pt = choose_partition(pool, s);
  if (pt > 0 && (s->max_len + pt - 1) / pt > MAX_PARTS)
    return fail(KVQ_ERR_UNSUPPORTED, "more than %d partitions (max_len %d, partition %d)", MAX_PARTS,
                s->max_len, pt);
  // (stream positions: up to 4096 set-cost positions per set ride on top of the tokens)
  if ((double)s->batch * (s->max_len + 4096.0) * pool->desc.num_kv_heads * qgroups_of(pool, s) >= 1099511627776.0)
    return fail(KVQ_ERR_UNSUPPORTED, "batch * (max_len + 4096) * num_kv_heads * query groups must stay below 2^40");
  const int qv = (s->num_q_heads / pool->desc.num_kv_heads) * s->q_rows;
  if (s->engine < KVQ_ENGINE_AUTO || s->engine > KVQ_ENGINE_MATRIX)
    return fail(KVQ_ERR_INVALID, "engine must be 0 (automatic), 1 (vector ALU) or 2 (matrix cores)");
  const kvq_pool_desc& pd = pool->desc;
  if (use_mfma(pool, s)) {
    if (!kvq::mfma_supported(pd.bits, pd.head_dim, pd.group_size) || pd.v_head_dim != pd.head_dim)
      return fail(KVQ_ERR_UNSUPPORTED, "the matrix-core engine reads 4-bit pages with head_dim 128 or 256 "
                                       "(v_head_dim the same) and group_size 64");
    if (pt > 0)
      return fail(KVQ_ERR_UNSUPPORTED, "the matrix-core engine runs the balanced stream schedule only "
                                       "(partition_tokens 0 or -1)");
  } else if (!kvq::partial_supported(pd.bits, pd.head_dim, pd.v_head_dim, pd.group_size,
                                     qvw_for(qv, pd.bits, pd.head_dim, pd.v_head_dim, pd.group_size))) {
    return fail(KVQ_ERR_UNSUPPORTED, "no kernel for bits=%d D=%d DV=%d", pd.bits, pd.head_dim, pd.v_head_dim);
  }
  return KVQ_OK;
}

// Partials: fixed partitions hold [B, HQ, N, parts] rows; the stream schedule holds
// (ranges + units) * sub slots of QVW vectors (slot = (unit + range) * sub + wave in range).  Each partial row is DV
// floats of unnormalised output (DV: the V head dim) plus (max, normaliser).  The vector engine adds its copy of q in the
// codes' pair order, D/32 blocks of Q_BLOCK_WORDS words per query vector.
struct WsLayout {
  size_t ml_off, qp_off, total;
};

WsLayout workspace_layout(const kvq_pool* pool, const kvq_decode_shape* s, int pt) {
  size_t rows;
  if (pt > 0) {
    const size_t parts = (size_t)(s->max_len + pt - 1) / pt;
    rows = (size_t)s->batch * s->num_q_heads * s->q_rows * parts;
  } else {
    const size_t units = (size_t)s->batch * pool->desc.num_kv_heads * qgroups_of(pool, s);
    const StreamGeom sg = stream_geom(pool, s);
    rows = ((size_t)sg.ranges + units) * sg.sub * qvw_of(pool, s);
  }
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  WsLayout L{};
  L.ml_off = up(rows * pool->desc.v_head_dim * sizeof(float));
  L.qp_off = L.total = L.ml_off + rows * 2 * sizeof(float);
  if (!use_mfma(pool, s)) {
    // the q copy, then kvq::Q_COPY_TAIL bytes the partial kernel's scalar-cache warm-up may read
    // past the last unit's copy (it requests whole groups of 64-byte lines)
    const size_t qv = (size_t)s->batch * pool->desc.num_kv_heads * qgroups_of(pool, s) * qvw_of(pool, s);
    L.qp_off = up(L.total);
    L.total = L.qp_off + qv * (pool->desc.head_dim / 32) * kvq::Q_BLOCK_WORDS * 4 + kvq::Q_COPY_TAIL;
  }
  return L;
}

// Launch timing: event pairs around the launches of each kind, kept until read.
struct Timing {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;                 // created events, reused
  size_t next = 0;                              // first unused event of the pool
  std::vector<std::pair<hipEvent_t, hipEvent_t>> rec[3];
};
Timing g_timing;

constexpr size_t TIMING_MAX_EVENTS = 65536;     // 32768 launches between two reads

hipEvent_t timing_event() {                     // under g_timing.mu
  if (g_timing.next >= TIMING_MAX_EVENTS) return nullptr;   // full: later launches go unrecorded
  if (g_timing.next == g_timing.pool.size()) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    g_timing.pool.push_back(e);
  }
  return g_timing.pool[g_timing.next++];
}

void timing_forget() {                          // under g_timing.mu
  for (auto& r : g_timing.rec) r.clear();
  g_timing.next = 0;
}

// runs launch() (returns hipError_t), bracketed by two events on st when timing is on
template <class F>
hipError_t timed(int kind, hipStream_t st, F launch) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  {
    std::lock_guard<std::mutex> g(g_timing.mu);
    if (g_timing.on && g_timing.next + 2 <= TIMING_MAX_EVENTS) {
      e0 = timing_event();
      e1 = timing_event();
    }
  }
  if (e0 && e1) (void)hipEventRecord(e0, st);
  const hipError_t r = launch();
  if (e0 && e1) {
    (void)hipEventRecord(e1, st);
    std::lock_guard<std::mutex> g(g_timing.mu);
    g_timing.rec[kind].push_back({e0, e1});
  }
  return r;
}

}  // namespace

namespace kvq {

int set_error(int code, const char* msg) {
  g_err = msg;
  return code;
}

}  // namespace kvq

extern "C" {

int kvq_timing_enable(int32_t on) {
  std::lock_guard<std::mutex> g(g_timing.mu);
  g_timing.on = on != 0;
  timing_forget();
  return KVQ_OK;
}

int kvq_timing_read(int32_t kind, double* avg_ms, int32_t* count) {
  if (kind < KVQ_TIMING_PREP || kind > KVQ_TIMING_MERGE || !avg_ms || !count)
    return fail(KVQ_ERR_INVALID, "kvq_timing_read: bad kind or NULL output");
  std::lock_guard<std::mutex> g(g_timing.mu);
  double sum = 0.0;
  int n = 0;
  for (auto& pr : g_timing.rec[kind]) {
    hipError_t e = hipEventSynchronize(pr.second);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, pr.first, pr.second);
    if (e != hipSuccess) return hip_fail(e, "kvq_timing_read");
    sum += ms;
    ++n;
  }
  g_timing.rec[kind].clear();
  bool any = false;
  for (auto& r : g_timing.rec) any |= !r.empty();
  if (!any) g_timing.next = 0;                  // every event is free again
  *avg_ms = n ? sum / n : 0.0;
  *count = n;
  return KVQ_OK;
}

int kvq_probe_read_ex(const void* buf, size_t bytes, uint32_t* sink, int32_t loads_in_flight, int32_t nontemporal,
                      int32_t blocks_per_cu, void* stream) {
  if (!buf || !sink || !aligned(buf, 16) || !aligned(sink, 4))
    return fail(KVQ_ERR_INVALID, "kvq_probe_read: buf (16-byte aligned) and sink must be device pointers");
  if (bytes == 0 || bytes % 16 != 0) return fail(KVQ_ERR_INVALID, "kvq_probe_read: bytes must be a positive multiple of 16");
  const int u = loads_in_flight;
  if (!(u == 1 || u == 2 || u == 4 || u == 8 || u == 16))
    return fail(KVQ_ERR_INVALID, "kvq_probe_read_ex: loads_in_flight must be 1, 2, 4, 8 or 16, got %d", u);
  if (blocks_per_cu < 1 || blocks_per_cu > 64)
    return fail(KVQ_ERR_INVALID, "kvq_probe_read_ex: blocks_per_cu must be 1..64, got %d", blocks_per_cu);
  hipError_t e = kvq::launch_probe_read(buf, bytes, sink, blocks_per_cu * device_cus(), u, nontemporal != 0,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "probe launch");
  return KVQ_OK;
}

int kvq_probe_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  return kvq_probe_read_ex(buf, bytes, sink, 4, 0, 32, stream);
}

int kvq_probe_pool_read(const kvq_pool* pool, const int32_t* block_table, const int32_t* lengths, int32_t batch,
                        int32_t max_blocks_per_seq, int32_t max_len, int32_t coalesced, uint32_t* sink,
                        void* stream) {
  if (!pool) return fail(KVQ_ERR_INVALID, "pool is NULL");
  if (!block_table || !lengths || !sink || !aligned(block_table, 4) || !aligned(lengths, 4) || !aligned(sink, 4))
    return fail(KVQ_ERR_INVALID, "kvq_probe_pool_read: block_table, lengths and sink must be device pointers");
  if (batch < 1 || max_blocks_per_seq < 1 || max_len < 1 || batch > 65535)
    return fail(KVQ_ERR_INVALID, "kvq_probe_pool_read: batch (1..65535), max_blocks_per_seq and max_len must be positive");
  const kvq_pool_desc& d = pool->desc;
  kvq::PoolProbeArgs a{};
  a.krow = (int)plane_row_bytes(&d, KVQ_PLANE_K);
  a.vrow = (int)plane_row_bytes(&d, KVQ_PLANE_V);
  {
    const int kc = a.krow / 16;
    if (a.krow != a.vrow || a.krow % 16 != 0 || !(kc == 2 || kc == 4 || kc == 6 || kc == 8 || kc == 16 || kc == 32))
      return fail(KVQ_ERR_UNSUPPORTED,
                  "kvq_probe_pool_read: K and V rows must be equal and 32, 64, 96, 128, 256 or 512 bytes (%d, %d)",
                  a.krow, a.vrow);
  }
  a.k = static_cast<const uint8_t*>(pool->planes[KVQ_PLANE_K]);
  a.v = static_cast<const uint8_t*>(pool->planes[KVQ_PLANE_V]);
  const int sp[4] = {KVQ_PLANE_K_SCALE, KVQ_PLANE_K_BIAS, KVQ_PLANE_V_SCALE, KVQ_PLANE_V_BIAS};
  for (int p = 0; p < 4; ++p) {
    a.sp[p] = static_cast<const uint8_t*>(pool->planes[sp[p]]);
    a.srow[p] = a.sp[p] ? (int)plane_row_bytes(&d, sp[p]) : 0;
  }
  a.table = block_table; a.lengths = lengths; a.sink = sink;
  a.HK = d.num_kv_heads; a.BS = d.block_size; a.max_blocks = max_blocks_per_seq; a.num_blocks = d.num_blocks;
  a.len_cap = (int)std::min<long>(max_len, (long)max_blocks_per_seq * d.block_size);
  hipError_t e = kvq::launch_probe_pool(a, batch, coalesced != 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pool probe launch");
  return KVQ_OK;
}

const char* kvq_last_error(void) { return g_err.c_str(); }

const char* kvq_version(void) { return "kvq 0.1 (gfx950)"; }

size_t kv_pool_plane_bytes(const kvq_pool_desc* desc, int32_t plane) {
  if (!desc || plane < 0 || plane >= KVQ_NUM_PLANES) return 0;
  if (validate_desc(desc) != KVQ_OK) return 0;
  return plane_row_bytes(desc, plane) * desc->num_blocks * desc->num_kv_heads * desc->block_size;
}

int kv_pool_create(const kvq_pool_desc* desc, kvq_pool** out) {
  if (!out) return fail(KVQ_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (int r = validate_desc(desc)) return r;
  kvq_pool* p = new kvq_pool();
  p->desc = *desc;
  p->desc.v_head_dim = v_dim(desc);
  p->owned = true;
  for (int i = 0; i < KVQ_NUM_PLANES; ++i) {
    p->planes[i] = nullptr;
    p->bytes[i] = kv_pool_plane_bytes(desc, i);
    if (p->bytes[i] == 0) continue;
    hipError_t e = hipMalloc(&p->planes[i], p->bytes[i]);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      kv_pool_destroy(p);
      return fail(KVQ_ERR_OOM, "hipMalloc of %zu bytes for plane %d failed: %s", p->bytes[i], i,
                  hipGetErrorString(e));
    }
    e = hipMemset(p->planes[i], 0, p->bytes[i]);
    if (e != hipSuccess) {
      kv_pool_destroy(p);
      return hip_fail(e, "hipMemset");
    }
  }
  *out = p;
  return KVQ_OK;
}

int kv_pool_wrap(const kvq_pool_desc* desc, void* const planes[KVQ_NUM_PLANES], kvq_pool** out) {
  if (!out) return fail(KVQ_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (int r = validate_desc(desc)) return r;
  if (!planes) return fail(KVQ_ERR_INVALID, "planes is NULL");
  kvq_pool* p = new kvq_pool();
  p->desc = *desc;
  p->desc.v_head_dim = v_dim(desc);
  p->owned = false;
  for (int i = 0; i < KVQ_NUM_PLANES; ++i) {
    p->bytes[i] = kv_pool_plane_bytes(desc, i);
    p->planes[i] = p->bytes[i] ? planes[i] : nullptr;
    if (p->bytes[i] && (!planes[i] || !aligned(planes[i], 16))) {
      delete p;
      return fail(KVQ_ERR_INVALID, "plane %d is NULL or not 16-byte aligned", i);
    }
  }
  *out = p;
  return KVQ_OK;
}

int kv_pool_destroy(kvq_pool* pool) {
  if (!pool) return KVQ_OK;
  if (pool->owned)
    for (int i = 0; i < KVQ_NUM_PLANES; ++i)
      if (pool->planes[i]) (void)hipFree(pool->planes[i]);
  delete pool;
  return KVQ_OK;
}

int kv_pool_plane(const kvq_pool* pool, int32_t plane, void** dev_ptr, size_t* bytes) {
  if (!pool || !dev_ptr || !bytes) return fail(KVQ_ERR_INVALID, "NULL argument");
  if (plane < 0 || plane >= KVQ_NUM_PLANES || pool->bytes[plane] == 0)
    return fail(KVQ_ERR_INVALID, "pool has no plane %d", plane);
  *dev_ptr = pool->planes[plane];
  *bytes = pool->bytes[plane];
  return KVQ_OK;
}

int kv_pool_describe(const kvq_pool* pool, kvq_pool_desc* out) {
  if (!pool || !out) return fail(KVQ_ERR_INVALID, "NULL argument");
  *out = pool->desc;
  return KVQ_OK;
}

int kv_append_quantize(kvq_pool* pool, const uint16_t* k, const uint16_t* v, const int64_t* slots,
                       int32_t num_tokens, void* stream) {
  if (!pool) return fail(KVQ_ERR_INVALID, "pool is NULL");
  if (num_tokens < 0) return fail(KVQ_ERR_INVALID, "num_tokens < 0");
  if (num_tokens == 0) return KVQ_OK;
  if (!k || !v || !slots) return fail(KVQ_ERR_INVALID, "k, v and slots must be device pointers");
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(slots, 8))
    return fail(KVQ_ERR_INVALID, "k and v must be 16-byte aligned, slots 8-byte aligned");
  const kvq_pool_desc& d = pool->desc;
  kvq::AppendArgs a{};
  a.k = k; a.v = v; a.slots = slots;
  a.k_plane = pool->planes[KVQ_PLANE_K]; a.v_plane = pool->planes[KVQ_PLANE_V];
  a.k_scale = pool->planes[KVQ_PLANE_K_SCALE]; a.k_bias = pool->planes[KVQ_PLANE_K_BIAS];
  a.v_scale = pool->planes[KVQ_PLANE_V_SCALE]; a.v_bias = pool->planes[KVQ_PLANE_V_BIAS];
  a.T = num_tokens; a.HK = d.num_kv_heads; a.D = d.head_dim; a.Dv = d.v_head_dim; a.BS = d.block_size;
  a.group = d.group_size;
  a.num_slots = (int64_t)d.num_blocks * d.block_size;
  hipError_t e = kvq::launch_append(a, d.bits, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return KVQ_OK;
}

size_t paged_decode_workspace_bytes(const kvq_pool* pool, const kvq_decode_shape* shape) {
  if (validate_shape(pool, shape) != KVQ_OK) return 0;
  return workspace_layout(pool, shape, choose_partition(pool, shape)).total;
}

int32_t paged_decode_partition_tokens(const kvq_pool* pool, const kvq_decode_shape* shape) {
  if (validate_shape(pool, shape) != KVQ_OK) return 0;
  return choose_partition(pool, shape);
}

int32_t paged_decode_engine(const kvq_pool* pool, const kvq_decode_shape* shape) {
  if (int r = validate_shape(pool, shape)) return r;
  return use_mfma(pool, shape) ? KVQ_ENGINE_MATRIX : KVQ_ENGINE_VECTOR;
}

namespace {

struct Plan {
  kvq::PartialArgs a;
  kvq::MergeArgs m;
  int qvw;
  bool mfma;
  int merge_threads;
};

// Merge workgroup size: one output row per workgroup, D/4 threads per stream of partials, 64 to
// 256 threads.  Few rows (under 8 per compute unit) leave the merge latency-bound: streams of about
// four partials each; many rows keep every compute unit busy anyway, and then streams of about
// eight partials waste fewer waves on the row's set-up (measured: 512 rows of 17-40 partials run
// fastest at 4-10 per stream, 8192 rows of 3-10 partials at one stream).  Partials per row: the
// fixed partitions' count, or the stream's slots for a unit, sub in every range it meets (each of
// its rows reads them all).  The vector engine's stream combines a unit's slots in all but the
// last range it meets, so its rows read fewer than this counts (the 4-bit GQA-8 decode at 32
// sequences: 2-15, against 40 counted); the sizes it gives measured best there as well (256
// threads: 9.4 us against 9.8 at 128 and 10.5 at 64).
int merge_threads_for(int dv, int pt, int parts, const StreamGeom& sg, double units, double rows) {
  const double per_row = pt > 0 ? (double)parts : (double)sg.sub * (sg.ranges + units) / units;
  const double per_stream = rows >= 8.0 * device_cus() ? 8.0 : 4.0;
  int streams = 1;
  while (streams * 2 <= per_row / per_stream) streams *= 2;
  return std::max(64, std::min(256, (dv / 4) * streams));
}

hipError_t launch_plan_partial(const Plan& P, const kvq_pool* pool, int B, hipStream_t st, bool q_ready = false) {
  return timed(KVQ_TIMING_PARTIAL, st, [&] {
    if (P.mfma) return kvq::launch_partial_mfma(P.a, pool->desc.head_dim, st);
    return kvq::launch_partial(P.a, pool->desc.bits, pool->desc.head_dim, pool->desc.v_head_dim,
                               pool->desc.group_size, P.qvw, B, q_ready, st);
  });
}

hipError_t launch_plan_merge(const Plan& P, int B, hipStream_t st) {
  return timed(KVQ_TIMING_MERGE, st, [&] { return kvq::launch_merge(P.m, B, P.merge_threads, st); });
}

int plan(const uint16_t* q, const kvq_pool* pool, const int32_t* block_table, const int32_t* lengths, float scale,
         const kvq_decode_shape* shape, void* workspace, size_t workspace_bytes, void* out, bool need_q,
         bool need_out, Plan* P) {
  if (int r = validate_shape(pool, shape)) return r;
  if ((need_q && (!q || !block_table)) || !lengths || !workspace || (need_out && !out))
    return fail(KVQ_ERR_INVALID, "q, block_table, lengths, workspace and out must be device pointers");
  if ((need_q && (!aligned(q, 16) || !aligned(block_table, 4))) || !aligned(lengths, 4) ||
      !aligned(workspace, 16) || (need_out && !aligned(out, shape->out_f32 ? 4 : 2)))
    return fail(KVQ_ERR_INVALID, "misaligned pointer (q and workspace need 16 bytes)");
  const int pt = choose_partition(pool, shape);
  const WsLayout L = workspace_layout(pool, shape, pt);
  const size_t need = L.total;
  if (workspace_bytes < need)
    return fail(KVQ_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
  const kvq_pool_desc& d = pool->desc;
  const int parts = pt > 0 ? (shape->max_len + pt - 1) / pt : 0;
  P->qvw = qvw_of(pool, shape);
  P->mfma = use_mfma(pool, shape);

  kvq::PartialArgs& a = P->a;
  a = kvq::PartialArgs{};
  a.q = q;
  a.k = pool->planes[KVQ_PLANE_K]; a.v = pool->planes[KVQ_PLANE_V];
  a.ks = static_cast<const uint16_t*>(pool->planes[KVQ_PLANE_K_SCALE]);
  a.kb = static_cast<const uint16_t*>(pool->planes[KVQ_PLANE_K_BIAS]);
  a.vs = static_cast<const uint16_t*>(pool->planes[KVQ_PLANE_V_SCALE]);
  a.vb = static_cast<const uint16_t*>(pool->planes[KVQ_PLANE_V_BIAS]);
  a.table = block_table; a.lengths = lengths;
  a.opart = static_cast<float*>(workspace);
  a.ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.ml_off);
  a.qp = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + L.qp_off);
  a.scale_log2e = scale * 1.4426950408889634f;
  a.HQ = shape->num_q_heads; a.HK = d.num_kv_heads; a.N = shape->q_rows; a.BS = d.block_size;
  a.bs_shift = -1;
  for (int s = 0; s < 31; ++s)
    if ((1 << s) == d.block_size) a.bs_shift = s;
  a.max_blocks = shape->max_blocks_per_seq; a.num_blocks = d.num_blocks; a.max_len = shape->max_len;
  a.part_tokens = pt; a.num_parts = parts; a.qgroups = qgroups_of(pool, shape);
  a.len_cap = (int)std::min<long>(shape->max_len, (long)shape->max_blocks_per_seq * d.block_size);
  const StreamGeom sg = stream_geom(pool, shape);
  a.batch = shape->batch; a.num_ranges = sg.ranges; a.range_sub = sg.sub; a.min_tokens = sg.min_tokens;
  a.lanes = stream_lanes(a.qgroups, pt, P->mfma, P->qvw, d.head_dim);
  if (a.lanes > 1) a.num_ranges = std::max(1, a.num_ranges / a.lanes);   // L workgroups per range
  a.set_cost = (pt == 0 && !P->mfma) ? stream_set_cost() : 0;

  P->merge_threads = merge_threads_for(d.v_head_dim, pt, parts, sg,
                                       (double)shape->batch * d.num_kv_heads * a.qgroups,
                                       (double)shape->batch * shape->num_q_heads * shape->q_rows);
  kvq::MergeArgs& m = P->m;
  m = kvq::MergeArgs{};
  m.opart = a.opart; m.ml = a.ml; m.lengths = lengths; m.out = out;
  m.HQ = shape->num_q_heads; m.N = shape->q_rows; m.D = d.v_head_dim; m.part_tokens = pt;
  m.num_parts = parts; m.out_f32 = shape->out_f32 ? 1 : 0; m.max_len = shape->max_len;
  m.len_cap = a.len_cap;
  m.batch = shape->batch; m.HK = d.num_kv_heads; m.qgroups = a.qgroups; m.qvw = P->qvw;
  m.num_ranges = a.num_ranges; m.range_sub = a.range_sub; m.min_tokens = a.min_tokens;
  m.stream_combined = (pt == 0 && !P->mfma) ? 1 : 0;
  m.lanes = a.lanes;
  m.set_cost = a.set_cost;
  return KVQ_OK;
}

}  // namespace

int paged_decode_partial(const uint16_t* q, const kvq_pool* pool, const int32_t* block_table,
                         const int32_t* lengths, float scale, const kvq_decode_shape* shape, void* workspace,
                         size_t workspace_bytes, void* stream) {
  Plan P;
  if (int r = plan(q, pool, block_table, lengths, scale, shape, workspace, workspace_bytes, nullptr, true, false, &P))
    return r;
  hipError_t e = launch_plan_partial(P, pool, shape->batch, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "partial launch");
  return KVQ_OK;
}

int paged_decode_merge(const kvq_pool* pool, const int32_t* lengths, const kvq_decode_shape* shape,
                       const void* workspace, size_t workspace_bytes, void* out, void* stream) {
  Plan P;
  if (int r = plan(nullptr, pool, nullptr, lengths, 0.0f, shape, const_cast<void*>(workspace), workspace_bytes, out,
                   false, true, &P))
    return r;
  hipError_t e = launch_plan_merge(P, shape->batch, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return KVQ_OK;
}

int paged_decode_attention(const uint16_t* q, const kvq_pool* pool, const int32_t* block_table,
                           const int32_t* lengths, float scale, const kvq_decode_shape* shape,
                           void* workspace, size_t workspace_bytes, void* out, void* stream) {
  Plan P;
  if (int r = plan(q, pool, block_table, lengths, scale, shape, workspace, workspace_bytes, out, true, true, &P))
    return r;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = launch_plan_partial(P, pool, shape->batch, st);
  if (e != hipSuccess) return hip_fail(e, "partial launch");
  e = launch_plan_merge(P, shape->batch, st);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return KVQ_OK;
}

namespace {

int step_partial(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new, kvq_pool* pool,
                 const int32_t* block_table, const int32_t* lengths, float scale, const kvq_decode_shape* shape,
                 void* workspace, size_t workspace_bytes, void* out, bool need_out, void* stream, Plan* Pout) {
  Plan& P = *Pout;
  if (int r = plan(q, pool, block_table, lengths, scale, shape, workspace, workspace_bytes, out, true, need_out, &P))
    return r;
  if (!k_new || !v_new) return fail(KVQ_ERR_INVALID, "k_new and v_new must be device pointers");
  if (!aligned(k_new, 16) || !aligned(v_new, 16)) return fail(KVQ_ERR_INVALID, "k_new and v_new must be 16-byte aligned");
  const kvq_pool_desc& d = pool->desc;
  kvq::AppendArgs ap{};
  ap.k = k_new; ap.v = v_new; ap.slots = nullptr;
  ap.table = block_table; ap.lengths = lengths;
  ap.N = shape->q_rows; ap.max_blocks = shape->max_blocks_per_seq; ap.len_cap = P.a.len_cap;
  ap.k_plane = pool->planes[KVQ_PLANE_K]; ap.v_plane = pool->planes[KVQ_PLANE_V];
  ap.k_scale = pool->planes[KVQ_PLANE_K_SCALE]; ap.k_bias = pool->planes[KVQ_PLANE_K_BIAS];
  ap.v_scale = pool->planes[KVQ_PLANE_V_SCALE]; ap.v_bias = pool->planes[KVQ_PLANE_V_BIAS];
  ap.T = shape->batch * shape->q_rows; ap.HK = d.num_kv_heads; ap.D = d.head_dim; ap.Dv = d.v_head_dim;
  ap.BS = d.block_size; ap.group = d.group_size;
  ap.num_slots = (int64_t)d.num_blocks * d.block_size;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = timed(KVQ_TIMING_PREP, st, [&] {
    return kvq::launch_step_prep(ap, P.a, d.bits, d.head_dim, d.v_head_dim, d.group_size, P.qvw, !P.mfma,
                                 shape->batch, st);
  });
  if (e != hipSuccess) return hip_fail(e, "step launch");
  e = launch_plan_partial(P, pool, shape->batch, st, true);
  if (e != hipSuccess) return hip_fail(e, "partial launch");
  return KVQ_OK;
}

}  // namespace

int paged_decode_step(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new, kvq_pool* pool,
                      const int32_t* block_table, const int32_t* lengths, float scale,
                      const kvq_decode_shape* shape, void* workspace, size_t workspace_bytes, void* out,
                      void* stream) {
  Plan P;
  if (int r = step_partial(q, k_new, v_new, pool, block_table, lengths, scale, shape, workspace, workspace_bytes,
                           out, true, stream, &P))
    return r;
  hipError_t e = launch_plan_merge(P, shape->batch, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return KVQ_OK;
}

int paged_decode_step_partial(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new, kvq_pool* pool,
                              const int32_t* block_table, const int32_t* lengths, float scale,
                              const kvq_decode_shape* shape, void* workspace, size_t workspace_bytes,
                              void* stream) {
  Plan P;
  return step_partial(q, k_new, v_new, pool, block_table, lengths, scale, shape, workspace, workspace_bytes,
                      nullptr, false, stream, &P);
}

int kv_gather_debug(const kvq_pool* pool, const int32_t* block_table, const int32_t* lengths, int32_t batch,
                    int32_t max_blocks_per_seq, int32_t max_len, void* const out_planes[KVQ_NUM_PLANES],
                    void* stream) {
  if (!pool || !block_table || !lengths || !out_planes) return fail(KVQ_ERR_INVALID, "NULL argument");
  if (batch < 1 || max_blocks_per_seq < 1 || max_len < 1) return fail(KVQ_ERR_INVALID, "sizes must be positive");
  const kvq_pool_desc& d = pool->desc;
  for (int p = 0; p < plane_count(d.bits); ++p) {
    if (!out_planes[p]) return fail(KVQ_ERR_INVALID, "out plane %d is NULL", p);
    kvq::GatherArgs g{};
    g.plane = static_cast<const uint8_t*>(pool->planes[p]);
    g.out = static_cast<uint8_t*>(out_planes[p]);
    g.table = block_table; g.lengths = lengths;
    g.B = batch; g.HK = d.num_kv_heads; g.BS = d.block_size; g.max_blocks = max_blocks_per_seq;
    g.max_len = max_len; g.num_blocks = d.num_blocks;
    g.row_bytes = (int)plane_row_bytes(&d, p);
    hipError_t e = kvq::launch_gather(g, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "gather launch");
  }
  return KVQ_OK;
}

}  // extern "C"
