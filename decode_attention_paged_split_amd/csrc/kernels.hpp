// Kernel argument blocks and launchers of the kvq library (host and device visible).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

struct AppendArgs {
  const uint16_t* k;      // [T, HK, D] bf16
  const uint16_t* v;      // [T, HK, Dv] bf16
  const int64_t* slots;   // [T]; NULL: a decode step's new rows, slots from the block table
  const int32_t* table;   // decode step: [B, max_blocks] block table
  const int32_t* lengths; // decode step: [B], counting the N new rows
  int32_t N, max_blocks, len_cap;   // decode step: rows per sequence (token = b * N + i), ...
  void* k_plane;          // codes (uint32) or bf16 values
  void* v_plane;
  void* k_scale;          // bf16 planes (affine only)
  void* k_bias;
  void* v_scale;
  void* v_bias;
  int32_t T, HK, D, BS;
  int32_t Dv;             // V head dim
  int32_t group;          // scale-group size (affine pages)
  int64_t num_slots;      // num_blocks * BS
};

struct GatherArgs {
  const uint8_t* plane;   // one pool plane
  uint8_t* out;           // [B, HK, max_len, row_bytes]
  const int32_t* table;
  const int32_t* lengths;
  int32_t B, HK, BS, max_blocks, max_len, num_blocks;
  int32_t row_bytes;      // bytes of one row of this plane (a multiple of 2)
};

struct PartialArgs {
  const uint16_t* q;        // [B, HQ, N, D] bf16
  const void* k;            // code plane (uint32) or bf16 values
  const void* v;
  const uint16_t* ks;       // [NB, HK, BS, G] bf16 (affine only)
  const uint16_t* kb;
  const uint16_t* vs;
  const uint16_t* vb;
  const int32_t* table;     // [B, max_blocks]
  const int32_t* lengths;   // [B]
  float* opart;             // [B, HQ, N, P, DV] f32, unnormalised (DV: the V head dim)
  float* ml;                // [B, HQ, N, P, 2] f32: running max (log2 units), normaliser
  uint32_t* qp;             // vector engine: [units, D/32 blocks x QVW, Q_BLOCK_WORDS] q in the codes' order
  float scale_log2e;        // softmax scale * log2(e)
  int32_t HQ, HK, N, BS, bs_shift, max_blocks, num_blocks, max_len;
  int32_t part_tokens;      // > 0: fixed partitions of this many tokens; 0: balanced stream
  int32_t num_parts;        // fixed partitions: partitions per sequence (grid x)
  int32_t qgroups;          // query groups of QVW vectors per KV head
  int32_t batch;
  int32_t num_ranges;       // stream: most ranges the stream is cut into (one per workgroup or wave)
  int32_t range_sub;        // stream: partial slots per (unit, range): the waves sharing a range
  int32_t min_tokens;       // stream: fewest tokens per working range
  int32_t len_cap;          // min(max_len, max_blocks * BS): lengths are clamped to [0, len_cap]
  int32_t lanes;            // vector stream: query groups of a KV head worked side by side (1, 2, 4)
  int32_t set_cost;         // vector stream: positions charged per set that has tokens, ahead of them
};

struct MergeArgs {
  const float* opart;
  const float* ml;
  const int32_t* lengths;
  void* out;                // [B, HQ, N, D] bf16 or f32 (D: the V head dim)
  int32_t HQ, N, D, part_tokens, num_parts, out_f32, max_len;
  int32_t len_cap;          // min(max_len, max_blocks * BS): lengths are clamped to [0, len_cap]
  int32_t batch, HK, qgroups, qvw, num_ranges, range_sub, min_tokens;   // stream (part_tokens == 0)
  int32_t stream_combined;  // stream: a range's waves combined their partials of its last unit
  int32_t lanes;            // stream: query groups side by side per set (partial slots interleave)
  int32_t set_cost;         // stream: positions charged per set that has tokens, ahead of them
};

// words per block of the vector engine's q copy: 16 bf16 pairs of one query vector, then (last
// block of a scale group, affine pages) the f32 sum of q over the group, then padding; a query
// vector takes head_dim / 32 blocks
constexpr int Q_BLOCK_WORDS = 20;
// bytes of workspace after the q copy: the partial kernel warms the scalar cache with a unit's copy
// in groups of eight 64-byte lines, which may reach up to seven lines past the last unit's copy
constexpr int Q_COPY_TAIL = 512;

// records msg as the calling thread's kvq_last_error() and returns code (host side)
int set_error(int code, const char* msg);

hipError_t launch_append(const AppendArgs& a, int bits, hipStream_t stream);
// streaming-read probe over bytes (a multiple of 16) of buf with `blocks` workgroups of 256,
// loads_in_flight (1, 2, 4, 8 or 16) 16-byte loads per thread at a time, optionally non-temporal
hipError_t launch_probe_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, int loads_in_flight,
                             bool nontemporal, hipStream_t stream);
hipError_t launch_gather(const GatherArgs& a, hipStream_t stream);

// pool-read probe: every cached row (K, V, and the four scale planes where sp[p] is set) of every
// (sequence, KV head), through the block table; krow and vrow multiples of 16
struct PoolProbeArgs {
  const uint8_t* k;
  const uint8_t* v;
  const uint8_t* sp[4];     // k scale, k bias, v scale, v bias planes (nullptr: none)
  const int32_t* table;
  const int32_t* lengths;
  uint32_t* sink;
  int32_t HK, BS, max_blocks, num_blocks, len_cap;
  int32_t krow, vrow, srow[4];
};
hipError_t launch_probe_pool(const PoolProbeArgs& a, int B, bool coalesced, hipStream_t stream);

// qvw: query vectors per workgroup (REP * N split into qgroups groups of qvw)
// q_ready: the vector engine's q copy is already in the workspace (decode step); gs: the pool's
// scale-group size (affine pages); D, DV: the K and V head dims
hipError_t launch_partial(const PartialArgs& a, int bits, int D, int DV, int gs, int qvw, int B, bool q_ready,
                          hipStream_t stream);
// threads: 64, 128 or 256 per output row (at least D / 4)
hipError_t launch_merge(const MergeArgs& a, int B, int threads, hipStream_t stream);
// decode step: the new rows' append (slots from the block table) and, for the vector engine, the
// q copy, in one launch
hipError_t launch_step_prep(const AppendArgs& ap, const PartialArgs& a, int bits, int D, int DV, int gs, int qvw,
                            bool vector_q, int B, hipStream_t stream);
bool partial_supported(int bits, int D, int DV, int gs, int qvw);
// a V head dim other than K's: the vector engine reads DV = D / 2 or 2 D (within 64..256) for
// bf16, 8-, 4- and 2-bit pages with 64-element scale groups
constexpr bool valu_dv_ok(int bits, int D, int DV, int gs) {
  return DV == D || ((bits == 16 || ((bits == 8 || bits == 4 || bits == 2) && gs == 64)) &&
                     (2 * DV == D || DV == 2 * D) && DV >= 64 && DV <= 256 && D >= 64 && D <= 256);
}
// most query vectors one wave of the vector engine carries: 8, or 4 where a V lane owns 16 head
// dims (2-bit pages; bf16, 8-, 6- and 5-bit pages at head dim 256, whose rows take two parts) or
// a row has 8 scale groups (the per-lane bias sums, vectors x groups, stay within 32 registers)
constexpr int valu_max_qvw(int bits, int D, int gs) {
  return (bits == 2 || (D == 256 && bits >= 5) || (bits != 16 && D / gs > 4)) ? 4 : 8;
}
// the same for K rows of D and V rows of DV dims: the smaller of the two
constexpr int valu_max_qvw(int bits, int D, int DV, int gs) {
  return valu_max_qvw(bits, D, gs) < valu_max_qvw(bits, DV, gs) ? valu_max_qvw(bits, D, gs)
                                                                : valu_max_qvw(bits, DV, gs);
}
// a row layout the vector engine reads: whole 16-byte chunks
constexpr bool valu_row_ok(int bits, int D) { return (D * bits / 8) % 16 == 0; }

// matrix-core engine (4-bit pages, head dim 128/256, stream schedule, 16 query vectors per wave,
// 64-token tiles)
bool mfma_supported(int bits, int D, int gs);
hipError_t launch_partial_mfma(const PartialArgs& a, int D, hipStream_t s);
constexpr int MFMA_QVW = 16;
// head dim 256 with at most this many query vectors per KV head: 8 vectors per unit, two token
// blocks per MFMA (the pair kernel)
constexpr int MFMA_PAIR_QVW = 8;
constexpr int MFMA_TILE = 64;
// vector engine, stream schedule: one workgroup of VALU_STREAM_WAVES waves per compute unit owns
// a range and shares its 64-token tiles among its waves
constexpr int VALU_STREAM_WAVES = 8;
constexpr int VALU_TILE = 64;
// vector engine, stream schedule: positions charged per set ahead of its tokens (the cost of a
// wave's change of set, in tokens; measured best at 512 on the workloads with ragged lengths)
constexpr int VALU_SET_COST = 512;

}  // namespace kvq
