// Split-K partial kernel of paged decode attention (vector ALU engine): the kernels, their
// launchers by bit width (instantiated once per width in partial_valu_b{16,8,6,5,4,3,2}.hip).
// Template parameters: BITS (page format), D (K head dim: the K phase, the q copy, K's scale
// groups), DV (V head dim: the V rows, weights, bias sums, accumulators and partial rows; the
// pages' vHeadDim), QVW (query vectors per wave), GS (scale-group size).
//
// What is computed follows "@mlx-bun/inference 0.0.0-stage -> 1.0.0", diff page 50:
//  * paged.ts, paged_attention_partial / paged_attention_affine_partial: token t of a
//    sequence is read straight from physical block table[t / BS], row t % BS; affine pages
//    are dequantized on load (scale * code + bias, codes low-first in uint32 words); each
//    partition keeps an online softmax (running max m, normaliser l, unnormalised output o)
//    in f32; row i of N sees t < length - N + i + 1.
//  * kvq4-decode.ts, the partial kernel: one read of a K/V row serves every query head of
//    its GQA group, and the token sub-chunks of a workgroup combine in on-chip memory with
//    the log-sum-exp algebra before one partial per partition is written.
//
// gfx950 layout (not the pages' Metal one).  A unit is (sequence, KV head, query group of QVW
// vectors); a wave walks tiles of 64 consecutive tokens of a unit.  Per tile:
//  1. K phase, one token per lane.  The tile's rows arrive with 16-byte loads (rows of 64 to 128
//     bytes, and affine rows of two 128-byte parts at scale groups of 64 or more, coalesced:
//     consecutive lanes read consecutive pieces in token order, and each piece reaches its
//     token's lane through LDS; other rows one token per lane).  The lane turns its token's
//     codes into bf16 pairs (4/2-bit codes c as bf16(128 + c) with one v_and_or, 8-bit codes
//     through an exact f32 conversion, bf16 rows as they are) and meets q in v_dot2_f32_bf16
//     with the q pair in a scalar register: q sits in the workspace in the codes' pair order
//     (qprep_kernel), every lane needs the same q pair at the same time, so it is read with
//     scalar loads, and no cross-lane sum is needed.  Products are exact (q and codes are
//     exact in bf16) and sums are f32.  The group's scale and bias apply once per (token,
//     vector, group): q.k = s * sum(q c') + (b - 128 s) * sum(q), sum(q) also prepared.
//  2. Softmax in the same layout.  Per vector the running max m is wave-uniform and only
//     moves when some score exceeds it by more than 2^8 (one ballot per tile; the exact tile
//     max and the rescale of o, l and the bias sums run only then), so p = 2^(z - m) <= 2^8.
//     Each lane keeps its share of the normaliser l and of the bias sum sum_t p b_v per scale
//     group; the weights p * s_v (per vector and scale group) go to LDS.
//  3. V phase.  The tile's V rows are loaded like its K rows and staged in LDS, and the tile is
//     read back transposed: VLPR lanes per row,
//     each owning VDPL head dims.  Codes become f32 with v_cvt_f32_ubyteN and accumulate as
//     o[vector][dim] += (p s)[vector] * code in f32.
// At the end of a wave's range the lanes' shares are summed and o += sum_t p b_v, so the
// unnormalised output is sum_t p (s c + b) as the pages define it.
// Loads run one tile ahead: the next tile's block-table entries are fetched while the current
// tile's q.k runs; its K and V rows and scales while the current softmax and P.V run.  Rows
// longer than 128 bytes (bf16 head dim >= 128, 8-bit head dim 256) are walked in parts of
// 128 bytes per lane.
//
// Two schedules share this tile engine:
//  * fixed partitions (partition_tokens > 0): workgroup = (partition, KV head x query group,
//    sequence); its 4 waves interleave tiles and combine in LDS; one partial per partition.
//  * balanced stream (partition_tokens == 0): a set is L consecutive query groups of one KV
//    head of one sequence (L = 4 when a KV head's groups come in fours, 2 in pairs, else 1).
//    Every set with tokens is laid end to end in one stream, taking a set cost of C positions (a
//    wave's change of set, in tokens) and then one per token, T positions in all, cut into R
//    equal ranges (R = min(compute units / L, ceil(T / 512))); each range is worked by L
//    workgroups of 8 waves, one per group of the set (one workgroup per compute unit), placed on
//    one XCD so that the K/V rows one of them fetches are found in that XCD's L2 by the others,
//    which walk the same tiles at about the same pace.  A workgroup's waves share its range's
//    64-token tiles through an LDS counter, each claiming its next tile as the current one
//    starts: the two waves on a SIMD do not progress at the same rate (the older one has issue
//    priority), and a static split would leave the slower one running alone at the end.  Each wave writes one partial per set that ends inside its range,
//    at slot ((set + r) * L + lane) * 8 + wave (distinct for every (set, range, lane, wave)
//    because ranges are contiguous and ordered); for the range's last set the 8 waves' partials
//    are combined in LDS first and written once, at slot ((set + r) * L + lane) * 8.  (A combine
//    at every set's end would need a barrier there, and the waves that took one tile fewer of the
//    set would wait a whole tile.)
#pragma once

#include "append_rows.hpp"
#include "device_common.hpp"
#include "kernels.hpp"

namespace kvq {

constexpr int PV_WAVES = 4;
constexpr int PV_TILE = VALU_TILE;              // tokens per tile: one per lane in the K phase
constexpr float LAZY_LOG2 = 8.0f;               // the running max moves when exceeded by this
constexpr float M_EMPTY = -1.0e30f;             // running max before any visible token

typedef __attribute__((address_space(4))) const uint32_t scalar_u32;   // read by s_load

template <int BITS, int D, int GS>
struct Geo {
  static constexpr int ROWB = D * BITS / 8;                 // bytes per pool row
  static constexpr bool AFF = BITS != 16;
  static constexpr bool STR = AFF && (32 % BITS != 0);      // codes straddle words (3, 5, 6 bits)
  static constexpr int GSZ = AFF ? GS : 64;                 // dims per scale group (bf16: 64-dim blocks)
  static constexpr int G = D / GSZ;                         // scale groups per row
  static constexpr int NP = (ROWB + 127) / 128;             // parts per row (<= 128 bytes each)
  static constexpr int KPB = ROWB / NP;                     // bytes of a row per part
  static constexpr int KCP = KPB / 16;                      // 16-byte chunks per part
  static constexpr int GPP = G / NP;                        // scale groups per part
  static constexpr int NHB = GSZ / 32;                      // 16-pair blocks per group
  static constexpr int WPH = BITS;                          // words per 16-pair block (32 dims)
  static constexpr int PPW = STR ? 0 : (BITS == 16 ? 1 : 16 / BITS);  // bf16 pairs per word
  static constexpr int DPP_ = KPB * 8 / BITS;               // head dims per part
  // V bytes per lane per row: 8 dims (straddling widths: 8 codes = BITS bytes, read as two
  // dwords and shifted into place), 4 dims (bf16) or one dword of codes
  static constexpr int VW = STR ? BITS : (BITS == 16 ? 8 : 4);
  static constexpr int VLPR = KPB / VW;                     // V lanes per row (one part)
  static constexpr int VRPL = 64 / VLPR;                    // rows per V read
  static constexpr int VDPL = VW * 8 / BITS;                // dims per V lane per part
  static constexpr int NBV = PV_TILE / VRPL;                // V reads per part
  static constexpr int VPITCH = KPB + 16;                   // LDS pitch of a staged V row
  static constexpr int WG = AFF ? G : 1;                    // weights per (token, vector)
  static constexpr float OFFS = (AFF && BITS <= 6) ? 128.0f : 0.0f;   // K codes as bf16(128 + c)
  static_assert(ROWB % NP == 0 && KPB % 16 == 0, "rows of whole 16-byte chunks per part");
  static_assert(G % NP == 0 && GPP * NHB * WPH * 4 == KPB, "whole groups per part");
  static_assert(VLPR >= 1 && VLPR <= 64 && 64 % VLPR == 0 && KPB % VW == 0 && GSZ % VDPL == 0, "V layout");
};

// dims (lo, hi) of bf16 pair P in the codes' order (natural word order; inside a word the
// pairing the unpack below produces)
template <int BITS>
__device__ __forceinline__ void pair_dims(int P, int& lo, int& hi) {
  if constexpr (BITS == 4) {
    const int w = P >> 2, k = P & 3; lo = 8 * w + k; hi = lo + 4;
  } else if constexpr (BITS == 2) {
    const int w = P >> 3, k = P & 7; lo = 16 * w + k; hi = lo + 8;
  } else {
    lo = 2 * P; hi = lo + 1;
  }
}

// (x & m) | o in one v_and_or_b32 (gfx9 VOP3 takes no literal, so the mask rides in an SGPR
// and the OR constant in a VGPR)
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(o));
  return r;
}

// one 32-bit word of a K row -> PPW bf16 pairs (affine codes c as bf16(OFFS + c), exact);
// magic holds 0x43004300 (bf16 128 in both halves)
template <int BITS>
__device__ __forceinline__ void word_pairs(uint32_t w, uint32_t* out, uint32_t magic) {
  if constexpr (BITS == 16) {
    out[0] = w;
  } else if constexpr (BITS == 8) {
    // an integer below 256 is exact in bf16: the low half of its f32 pattern is zero
    const float c0 = (float)(w & 0xFFu), c1 = (float)((w >> 8) & 0xFFu);
    const float c2 = (float)((w >> 16) & 0xFFu), c3 = (float)(w >> 24);
    out[0] = __builtin_amdgcn_perm(__float_as_uint(c1), __float_as_uint(c0), 0x07060302u);
    out[1] = __builtin_amdgcn_perm(__float_as_uint(c3), __float_as_uint(c2), 0x07060302u);
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) out[k] = and_or(w >> (4 * k), 0x000F000Fu, magic);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) out[k] = and_or(w >> (2 * k), 0x00030003u, magic);
  }
}

// the 32 codes of a 16-pair block of a straddling-width row (BITS words, one little-endian bit
// stream) -> 16 bf16 pairs (dims 2p, 2p + 1) as bf16(128 + c), exact: the pair's 2 * BITS bits are
// funnel-shifted down (v_alignbit_b32 where they cross a word), the low code masked into the
// low half and the high code shifted and masked into the high half
template <int BITS>
__device__ __forceinline__ void block_pairs(const uint32_t* w, uint32_t* out, uint32_t magic) {
  constexpr uint32_t M = (1u << BITS) - 1u;
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    constexpr int F = 2 * BITS;
    const int o = F * p, wj = o >> 5, sh = o & 31;
    uint32_t x;
    if (sh + F <= 32) x = sh ? (w[wj] >> sh) : w[wj];
    else x = __builtin_amdgcn_alignbit(w[wj + 1], w[wj], sh);
    out[p] = and_or(x << (16 - BITS), M << 16, and_or(x, M, magic));
  }
}

// the 8 codes of a straddling-width V lane -> f32: (w0, w1) are the two dwords from the lane's
// first byte rounded down to a dword, s = 8 * (that byte offset % 4); the codes sit at bits
// BITS * d of the 64-bit value (w1:w0) >> s (8 * BITS + s <= 64 for every lane of a row)
template <int BITS>
__device__ __forceinline__ void value8_str(uint32_t w0, uint32_t w1, uint32_t s, float* v) {
  const uint32_t lo = __builtin_amdgcn_alignbit(w1, w0, s);
  const uint32_t hi = w1 >> s;
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    const int o = BITS * d;
    uint32_t c;
    if (o + BITS <= 32) c = __builtin_amdgcn_ubfe(lo, o, BITS);
    else if (o >= 32) c = __builtin_amdgcn_ubfe(hi, o - 32, BITS);
    else c = __builtin_amdgcn_ubfe(__builtin_amdgcn_alignbit(hi, lo, o), 0, BITS);
    v[d] = (float)c;
  }
}

// byte N of x as f32 (v_cvt_f32_ubyteN: one instruction per code once codes sit in bytes)
template <int N>
__device__ __forceinline__ float ubyte_f32(uint32_t x) {
  float r;
  if constexpr (N == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(x));
  else if constexpr (N == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(x));
  else if constexpr (N == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(x));
  else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

// VW bytes of a V row -> VDPL f32 values in natural dim order: the codes themselves (affine
// pages; scale and bias are applied through the weights and the bias sums) or the bf16 values
template <int BITS, int VDPL>
__device__ __forceinline__ void value_f32(const uint32_t* w, float* v) {
  if constexpr (BITS == 16) {
#pragma unroll
    for (int k = 0; k < VDPL / 2; ++k) { v[2 * k] = bf16_lo(w[k]); v[2 * k + 1] = bf16_hi(w[k]); }
  } else if constexpr (BITS == 8) {
    v[0] = ubyte_f32<0>(w[0]); v[1] = ubyte_f32<1>(w[0]);
    v[2] = ubyte_f32<2>(w[0]); v[3] = ubyte_f32<3>(w[0]);
  } else {
    // mask the codes into bytes, then v_cvt_f32_ubyte{0..3} converts one code each
    constexpr int PER = 8 / BITS;                                   // codes per byte
    constexpr uint32_t M = (BITS == 4) ? 0x0F0F0F0Fu : 0x03030303u;
#pragma unroll
    for (int sh = 0; sh < PER; ++sh) {
      const uint32_t x = (w[0] >> (BITS * sh)) & M;
      v[0 * PER + sh] = ubyte_f32<0>(x);
      v[1 * PER + sh] = ubyte_f32<1>(x);
      v[2 * PER + sh] = ubyte_f32<2>(x);
      v[3 * PER + sh] = ubyte_f32<3>(x);
    }
  }
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, a), __builtin_bit_cast(bf2, b), c, false);
}

// order LDS writes of this wave before its following LDS reads (a wave's LDS ops execute in
// order; this keeps the compiler from moving them across each other)
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float uni_f(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uni64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// lane sum over an exact xor distance (values differ across lanes)
template <int OFF>
__device__ __forceinline__ float xor_sum(float x) {
  if constexpr (OFF == 32) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else if constexpr (OFF == 16) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    return x + __shfl_xor(x, OFF, 64);
  }
}

template <int OFF>
__device__ __forceinline__ float rows_sum(float x) {
  if constexpr (OFF < 64) return rows_sum<OFF * 2>(xor_sum<OFF>(x));
  else return x;
}

// per-wave LDS of the tile engine: the tile's weights p * s_v, [token][group][vector] (each
// token's row padded by 4 words, so the 64 lanes' row writes spread over all banks), and one
// part of the tile's V rows (V rows of DV head dims)
template <int BITS, int DV, int QVW, int GS>
struct WaveScratch {
  static constexpr int WPITCH = Geo<BITS, DV, GS>::WG * QVW + 4;
  float w[PV_TILE][WPITCH];
  uint8_t v[PV_TILE][Geo<BITS, DV, GS>::VPITCH];
  __device__ float* wrow(int t, int g) { return &w[t][g * QVW]; }
};

// running state of one wave over one range of one unit (V rows of DV head dims)
template <int BITS, int DV, int QVW, int GS>
struct Acc {
  float o[QVW][Geo<BITS, DV, GS>::NP][Geo<BITS, DV, GS>::VDPL];  // V lanes: sum_t p * code (or value)
  float pb[QVW][Geo<BITS, DV, GS>::G];        // token lanes: this lane's share of sum_t p * b_v
  float l[QVW];                           // token lanes: this lane's share of sum_t p
  float m[QVW];                           // wave-uniform running max (log2 units)
};

struct Unit {
  int b, hk, qg, len;
  int64_t u;                              // unit index (b * HK + hk) * qgroups + qg
};

template <int BITS, int DV, int QVW, int GS>
__device__ __forceinline__ void acc_init(Acc<BITS, DV, QVW, GS>& st) {
  using Gm = Geo<BITS, DV, GS>;
#pragma unroll
  for (int j = 0; j < QVW; ++j) {
#pragma unroll
    for (int h = 0; h < Gm::NP; ++h)
#pragma unroll
      for (int d = 0; d < Gm::VDPL; ++d) st.o[j][h][d] = 0.0f;
#pragma unroll
    for (int g = 0; g < Gm::G; ++g) st.pb[j][g] = 0.0f;
    st.l[j] = 0.0f;
    st.m[j] = M_EMPTY;
  }
}

// the tile's per-token scale-plane entries: G bf16 each of k scale and k bias, GV each of v
// scale and v bias
template <int G, int GV>
struct Scales {
  uint32_t ks[(G + 1) / 2], kb[(G + 1) / 2], vs[(GV + 1) / 2], vb[(GV + 1) / 2];
};

template <int G>
__device__ __forceinline__ void load_plane_row(const uint16_t* p, int64_t row, uint32_t* out) {
  if constexpr (G == 8) {
    const uint4 x = *reinterpret_cast<const uint4*>(p + row * 8);
    out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
  } else if constexpr (G == 4) {
    const uint2 x = *reinterpret_cast<const uint2*>(p + row * 4);
    out[0] = x.x; out[1] = x.y;
  } else if constexpr (G == 2) {
    out[0] = *reinterpret_cast<const uint32_t*>(p + row * 2);
  } else {
    out[0] = p[row];
  }
}

template <int G>
__device__ __forceinline__ float plane_val(const uint32_t* x, int g) {
  return (g & 1) ? bf16_hi(x[g >> 1]) : bf16_lo(x[g >> 1]);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// one part (<= 128 bytes) of a pool row, held by the lane of its token
template <int KCP>
struct RowPart {
  u32x4 c[KCP];
};

template <int KCP>
__device__ __forceinline__ RowPart<KCP> load_row_part(const char* plane, int row, int rowb, int offs) {
  RowPart<KCP> r;
  const u32x4* src = reinterpret_cast<const u32x4*>(plane + (int64_t)row * rowb + offs);
#pragma unroll
  for (int c = 0; c < KCP; ++c) r.c[c] = src[c];
  return r;
}

// The same part (rows of one part only) of the rows of a tile's 64 tokens, loaded coalesced: lane
// l takes 16-byte piece l % KCP of the row of token l / KCP + c * (64 / KCP), c < KCP, so that
// consecutive lanes read consecutive bytes of a block (a block holds its rows of one KV head
// contiguously); row is each lane's own token's pool row.
template <int KCP>
__device__ __forceinline__ RowPart<KCP> load_rows_coalesced(const char* plane, int row, int rowb, int lane) {
  static_assert(64 % KCP == 0, "whole tokens per wave load");
  RowPart<KCP> r;
  const int piece = lane % KCP, tok0 = lane / KCP;
#pragma unroll
  for (int c = 0; c < KCP; ++c) {
    const int rr = __shfl(row, tok0 + c * (64 / KCP), 64);
    r.c[c] = *reinterpret_cast<const u32x4*>(plane + (int64_t)rr * rowb + piece * 16);
  }
  return r;
}

// Tiles of unit un (tokens < t1), accumulated into st by one wave.  grab() returns the first
// token of the next tile this wave takes (>= t1: none left), valid in lane 0 at least; it is
// called one tile ahead and read (made uniform) only a tile later, so an atomic behind it has a
// whole tile to return and its wait does not hold up the loads issued after it.
template <int BITS, int D, int DV, int QVW, int GS, class Grab>
__device__ __forceinline__ void run_tiles(const PartialArgs& a, const Unit& un, int t1, Grab grab,
                                          WaveScratch<BITS, DV, QVW, GS>& ws, Acc<BITS, DV, QVW, GS>& st, int lane) {
  using Gm = Geo<BITS, D, GS>;                                    // K rows
  using Gv = Geo<BITS, DV, GS>;                                   // V rows
  constexpr int ROWB = Gm::ROWB, G = Gm::G, NP = Gm::NP, KCP = Gm::KCP, GPP = Gm::GPP, NHB = Gm::NHB;
  constexpr int PPW = Gm::PPW, WPH = Gm::WPH, KPB = Gm::KPB;
  constexpr int VW = Gv::VW, VLPR = Gv::VLPR, VRPL = Gv::VRPL, VDPL = Gv::VDPL, NBV = Gv::NBV;
  constexpr int GV = Gv::G, NPV = Gv::NP, KCPV = Gv::KCP, ROWBV = Gv::ROWB, KPBV = Gv::KPB;
  constexpr bool AFF = Gm::AFF;
  constexpr int QBS = Q_BLOCK_WORDS;                              // words per q block
  // Row parts of 64 to 128 bytes (K's no wider than V's) are loaded coalesced, a part of a tile's
  // 64 rows as 64 * KCP pieces in token order, and reach their token's lane through LDS: V's by
  // the staging the V phase does anyway, K's by a round trip before the part is used.  Rows of one
  // part, and affine rows of two parts at scale groups of 64 or more (8-bit at head dim 256: 7 %
  // faster); wider rows and 8-bit head-dim-256 rows at group 32 would spill registers, and bf16
  // rows of two parts measured 2.5 % slower (c2: a few tiles per wave, the K round trip adds
  // latency that nothing hides).  Parts of 48, 80 or
  // 96 bytes (3-, 5- and 6-bit codes) and parts under 64 bytes (where the K round trip costs more
  // than it saves: 2-bit codes at head dim 128 measured 1.4 % slower) are loaded one token per lane.
  constexpr bool COAL = ((NP == 1 && NPV == 1) || (NP == 2 && NPV == 2 && GS >= 64 && AFF)) &&
                        KPB <= KPBV && KCP >= 4 && 64 % KCP == 0 && 64 % KCPV == 0;
  int tt = uni(grab());
  if (tt >= t1) return;

  const int vsl = lane % VLPR, vrg = lane / VLPR;                // V: dim slot, row in read
  const int N = a.N;
  int vend[QVW];                                                  // row i of vector j sees t < vend
#pragma unroll
  for (int j = 0; j < QVW; ++j) {
    const int jj = un.qg * QVW + j;
    vend[j] = un.len - N + (jj - (jj / N) * N) + 1;
  }
  const scalar_u32* qu = (const scalar_u32*)(a.qp) + un.u * (G * NHB * QVW * QBS);
  const char* kplane = static_cast<const char*>(a.k);
  const char* vplane = static_cast<const char*>(a.v);
  const int32_t* trow = a.table + (int64_t)un.b * a.max_blocks;
  const int hk = un.hk;
  const uint32_t magic = 0x43004300u;

  auto table_entry = [&](int t) -> int {                          // block-table entry of token t
    const int blk = (a.bs_shift >= 0) ? (t >> a.bs_shift) : (t / a.BS);
    return trow[blk];
  };
  auto row_of = [&](int t, int phys) -> int {                    // pool row of token t
    const int blk = (a.bs_shift >= 0) ? (t >> a.bs_shift) : (t / a.BS);
    phys = min(max(phys, 0), a.num_blocks - 1);                   // a bad entry cannot fault
    return (phys * a.HK + hk) * a.BS + (t - blk * a.BS);
  };
  auto load_scales = [&](int row, Scales<G, GV>& sc) {
    if constexpr (AFF) {
      load_plane_row<G>(a.ks, row, sc.ks);
      load_plane_row<G>(a.kb, row, sc.kb);
      load_plane_row<GV>(a.vs, row, sc.vs);
      load_plane_row<GV>(a.vb, row, sc.vb);
    }
  };
  auto stage_v = [&](const RowPart<KCPV>& src) {                 // V row part(s) -> LDS rows
    if constexpr (COAL) {
      const int piece = lane % KCPV, tok0 = lane / KCPV;
#pragma unroll
      for (int c = 0; c < KCPV; ++c)
        *reinterpret_cast<u32x4*>(&ws.v[tok0 + c * (64 / KCPV)][16 * piece]) = src.c[c];
    } else {
#pragma unroll
      for (int c = 0; c < KCPV; ++c) *reinterpret_cast<u32x4*>(&ws.v[lane][16 * c]) = src.c[c];
    }
  };
  auto own_k_row = [&](const RowPart<KCP>& src) {                // coalesced K pieces -> own row
    RowPart<KCP> r;
    const int piece = lane % KCP, tok0 = lane / KCP;
#pragma unroll
    for (int c = 0; c < KCP; ++c)
      *reinterpret_cast<u32x4*>(&ws.v[tok0 + c * (64 / KCP)][16 * piece]) = src.c[c];
    wave_lds_sync();
#pragma unroll
    for (int c = 0; c < KCP; ++c) r.c[c] = *reinterpret_cast<const u32x4*>(&ws.v[lane][16 * c]);
    return r;
  };

  // ---- prologue: the first tile's block-table entries are requested, then the unit's q copy is
  // pulled into the scalar cache while they arrive (eight 64-byte lines requested per wait: the K
  // phase asks for its blocks one after the other and would wait for every line's first miss in
  // turn; the last group may reach past the copy, into the next unit's or the workspace's
  // Q_COPY_TAIL bytes), then rows, K and V part 0 and scales of the first tile
  const int t_first = min(tt + lane, t1 - 1);
  const int tbl_first = table_entry(t_first);
  {
    constexpr int QL = (G * NHB * QVW * QBS + 15) / 16;           // 64-byte lines of the q copy
#pragma unroll
    for (int c = 0; c < QL; c += 8) {
      const scalar_u32* base = qu + 16 * c;
      typedef int i32x16 __attribute__((ext_vector_type(16)));
      i32x16 sink;
      // the loads land in the same 16 registers (values unused) and are waited for in this block
      asm volatile(
          "s_load_dwordx16 %0, %1, 0x0\n\t"
          "s_load_dwordx16 %0, %1, 0x40\n\t"
          "s_load_dwordx16 %0, %1, 0x80\n\t"
          "s_load_dwordx16 %0, %1, 0xc0\n\t"
          "s_load_dwordx16 %0, %1, 0x100\n\t"
          "s_load_dwordx16 %0, %1, 0x140\n\t"
          "s_load_dwordx16 %0, %1, 0x180\n\t"
          "s_load_dwordx16 %0, %1, 0x1c0\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&s"(sink) : "s"(base) : "memory");
    }
  }
  int row = row_of(t_first, tbl_first);
  RowPart<KCP> kcur;
  if constexpr (COAL) kcur = load_rows_coalesced<KCP>(kplane, row, ROWB, lane);
  else kcur = load_row_part<KCP>(kplane, row, ROWB, 0);
  Scales<G, GV> sc, scn;
  load_scales(row, sc);
  RowPart<KCPV> vcur;
  if constexpr (COAL) vcur = load_rows_coalesced<KCPV>(vplane, row, ROWBV, lane);
  else vcur = load_row_part<KCPV>(vplane, row, ROWBV, 0);

  while (true) {
    // the next tile is claimed only as this one starts, so that a wave holds no more than the
    // tile it works and the one it prefetches: near the end of a range the last tiles go to the
    // waves that are free
    const int tn = uni(grab());
    const bool has_next = tn < t1;                                // uniform
    const int t_next = min(tn + lane, t1 - 1);
    const int tbl_next = has_next ? table_entry(t_next) : 0;

    // ---- K phase: z[j] = q_j . k_t for this lane's token.
    // q block b = ((g * NHB + hb) * QVW + j): the 16 q pairs of 16-pair block hb of scale group g
    // for vector j, then (last block of the group) the group's q sum.  Block b + 1's base address
    // passes through an asm that depends on the dot products of block b - 1, so its scalar loads
    // are issued one block ahead of their use and no earlier (loads of invariant memory would
    // otherwise be hoisted, all of q at once, into too few scalar registers).
    float z[QVW];
#pragma unroll
    for (int j = 0; j < QVW; ++j) z[j] = 0.0f;
    constexpr int NQB = G * NHB * QVW;
    uint32_t qb[2][17];
    float last = 0.0f;                                            // result of the latest block
    auto q_fetch = [&](int b, uint32_t* dst) {
      const scalar_u32* qt;
      asm volatile("s_mov_b64 %0, %1" : "=s"(qt) : "s"(qu), "v"(last));
#pragma unroll
      for (int p = 0; p < 17; ++p) dst[p] = qt[b * QBS + p];
    };
    q_fetch(0, qb[0]);
    RowPart<KCP> kpart;
    if constexpr (COAL) kpart = own_k_row(kcur);
    else kpart = kcur;
#pragma unroll
    for (int h = 0; h < NP; ++h) {
      RowPart<KCP> knext;
      if (h + 1 < NP) {
        if constexpr (COAL) knext = load_rows_coalesced<KCP>(kplane + (h + 1) * KPB, row, ROWB, lane);
        else knext = load_row_part<KCP>(kplane, row, ROWB, (h + 1) * KPB);
      }
#pragma unroll
      for (int gp = 0; gp < GPP; ++gp) {
        const int g = h * GPP + gp;                               // scale group
        float s = 1.0f, bb = 0.0f;
        if constexpr (AFF) {
          s = plane_val<G>(sc.ks, g);
          bb = fmaf(-Gm::OFFS, s, plane_val<G>(sc.kb, g));
        }
        float acc[QVW];
#pragma unroll
        for (int j = 0; j < QVW; ++j) acc[j] = 0.0f;
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          uint32_t kp[16];
          if constexpr (Gm::STR) {
            uint32_t bw[WPH];
#pragma unroll
            for (int wi = 0; wi < WPH; ++wi) {
              const int word = (gp * NHB + hb) * WPH + wi;        // word of the part
              bw[wi] = kpart.c[word >> 2][word & 3];
            }
            block_pairs<BITS>(bw, kp, magic);
          } else {
#pragma unroll
            for (int wi = 0; wi < WPH; ++wi) {
              const int word = (gp * NHB + hb) * WPH + wi;        // word of the part
              word_pairs<BITS>(kpart.c[word >> 2][word & 3], &kp[wi * PPW], magic);
            }
          }
#pragma unroll
          for (int j = 0; j < QVW; ++j) {
            const int b = (g * NHB + hb) * QVW + j;
            if (b + 1 < NQB) q_fetch(b + 1, qb[(b + 1) & 1]);
            const uint32_t* qq = qb[b & 1];
#pragma unroll
            for (int p = 0; p < 16; ++p) acc[j] = dot2_bf16(qq[p], kp[p], acc[j]);
            last = acc[j];
            if (hb == NHB - 1) {
              if constexpr (AFF) z[j] = fmaf(s, acc[j], fmaf(bb, __uint_as_float(qq[16]), z[j]));
              else z[j] += acc[j];
            }
          }
        }
      }
      if (h + 1 < NP) {
        if constexpr (COAL) kpart = own_k_row(knext);
        else kpart = knext;
      }
    }

    // ---- stage V part 0 of this tile, then start the next tile's loads.  After a wave's last
    // tile of a unit there is no next tile: the loads are skipped (a uniform branch), except in
    // the 4-bit, head-dim-256, 8-vector instance, whose live registers the branch pushes past 256
    // (spills, 7 % slower); it reloads the current rows instead (valid addresses, never used).
    stage_v(vcur);
    const int row_next = has_next ? row_of(t_next, tbl_next) : row;
    constexpr bool RELOAD = BITS == 4 && D == 256 && DV == 256 && QVW == 8;
    if (RELOAD || has_next) {
      if constexpr (COAL) kcur = load_rows_coalesced<KCP>(kplane, row_next, ROWB, lane);
      else kcur = load_row_part<KCP>(kplane, row_next, ROWB, 0);
      load_scales(row_next, scn);
      if constexpr (COAL) vcur = load_rows_coalesced<KCPV>(vplane, row_next, ROWBV, lane);
      else vcur = load_row_part<KCPV>(vplane, row_next, ROWBV, 0);
    }

    // ---- softmax, one token per lane
    const int tok = tt + lane;
    float zs[QVW];
    bool exceed = false;
#pragma unroll
    for (int j = 0; j < QVW; ++j) {
      zs[j] = (tok < t1 && tok < vend[j]) ? z[j] * a.scale_log2e : -INFINITY;
      exceed |= zs[j] > st.m[j] + LAZY_LOG2;
    }
    if (__ballot(exceed)) {                                       // uniform; rare after the start
      asm volatile("; running max moves");                        // keeps this a real branch
#pragma unroll
      for (int j = 0; j < QVW; ++j) {
        const float mt = uni_f(block_reduce<OpMax, 1, 64>(zs[j]));
        const float mn = (mt > st.m[j] + LAZY_LOG2) ? mt : st.m[j];
        const float al = fast_exp2(st.m[j] - mn);
        st.m[j] = mn;
        st.l[j] *= al;
#pragma unroll
        for (int g = 0; g < GV; ++g) st.pb[j][g] *= al;
#pragma unroll
        for (int h = 0; h < NPV; ++h)
#pragma unroll
          for (int d = 0; d < VDPL; ++d) st.o[j][h][d] *= al;
      }
    }
#pragma unroll
    for (int j = 0; j < QVW; ++j) {
      const float p = fast_exp2(zs[j] - st.m[j]);
      st.l[j] += p;
      if constexpr (AFF) {
#pragma unroll
        for (int g = 0; g < GV; ++g) {
          ws.wrow(lane, g)[j] = p * plane_val<GV>(sc.vs, g);
          st.pb[j][g] = fmaf(p, plane_val<GV>(sc.vb, g), st.pb[j][g]);
        }
      } else {
        ws.wrow(lane, 0)[j] = p;
      }
    }
    wave_lds_sync();

    // ---- V phase: o[j][d] += w[row][group][j] * value[row][d], one part of the row at a time
    RowPart<KCPV> vpart;
#pragma unroll
    for (int h = 0; h < NPV; ++h) {
      RowPart<KCPV> vnext;
      if (h + 1 < NPV) {
        if constexpr (COAL) vnext = load_rows_coalesced<KCPV>(vplane + (h + 1) * KPBV, row, ROWBV, lane);
        else vnext = load_row_part<KCPV>(vplane, row, ROWBV, (h + 1) * KPBV);
      }
      if (h > 0) {
        stage_v(vpart);
        wave_lds_sync();
      }
      const int vgrp = AFF ? (h * Gv::DPP_ + vsl * VDPL) / Gv::GSZ : 0;
#pragma unroll
      for (int i = 0; i < NBV; ++i) {
        const int r = vrg + VRPL * i;
        float wv[QVW];
        if constexpr (QVW % 4 == 0) {
#pragma unroll
          for (int j4 = 0; j4 < QVW / 4; ++j4) {
            const float4 x = *reinterpret_cast<const float4*>(ws.wrow(r, vgrp) + 4 * j4);
            wv[4 * j4] = x.x; wv[4 * j4 + 1] = x.y; wv[4 * j4 + 2] = x.z; wv[4 * j4 + 3] = x.w;
          }
        } else {
#pragma unroll
          for (int j = 0; j < QVW; ++j) wv[j] = ws.wrow(r, vgrp)[j];
        }
        float vv[VDPL];
        if constexpr (Gv::STR) {
          const int ob = vsl * VW;                                // the lane's first byte
          const uint32_t* src = reinterpret_cast<const uint32_t*>(&ws.v[r][ob & ~3]);
          value8_str<BITS>(src[0], src[1], 8u * (uint32_t)(ob & 3), vv);
        } else {
          uint32_t cw[VW / 4];
          if constexpr (VW == 8) {
            const uint2 x = *reinterpret_cast<const uint2*>(&ws.v[r][vsl * VW]);
            cw[0] = x.x; cw[1] = x.y;
          } else {
            cw[0] = *reinterpret_cast<const uint32_t*>(&ws.v[r][vsl * VW]);
          }
          value_f32<BITS, VDPL>(cw, vv);
        }
#pragma unroll
        for (int j = 0; j < QVW; ++j)
#pragma unroll
          for (int d = 0; d < VDPL; ++d) st.o[j][h][d] = fmaf(wv[j], vv[d], st.o[j][h][d]);
      }
      wave_lds_sync();                                            // ws.v is rewritten next
      if (h + 1 < NPV) vpart = vnext;
    }

    if (!has_next) break;
    tt = tn;
    row = row_next;
    sc = scn;
  }
}

// Sum the lanes' shares and write one partial (o, m, l) of QVW vectors: o to orow(j) + dim,
// (m, l) through set_ml(j, m, l) on lane 0.  m is reported as -inf when no token of the range
// was visible to a vector.
template <int BITS, int DV, int QVW, int GS, class ORow, class SetML>
__device__ __forceinline__ void acc_write(Acc<BITS, DV, QVW, GS>& st, int lane, ORow orow, SetML set_ml) {
  using Gm = Geo<BITS, DV, GS>;
  constexpr int VDPL = Gm::VDPL, VLPR = Gm::VLPR, G = Gm::G, NP = Gm::NP;
  const int vsl = lane % VLPR, vrg = lane / VLPR;
#pragma unroll
  for (int j = 0; j < QVW; ++j) {
    float pbt[G];
#pragma unroll
    for (int g = 0; g < G; ++g) pbt[g] = Gm::AFF ? block_reduce<OpAdd, 1, 64>(st.pb[j][g]) : 0.0f;
    const float l = block_reduce<OpAdd, 1, 64>(st.l[j]);
#pragma unroll
    for (int h = 0; h < NP; ++h) {
      const int d0 = h * Gm::DPP_ + vsl * VDPL;                   // first head dim of the lane
      float bias = 0.0f;
#pragma unroll
      for (int g = 0; g < G; ++g)
        if (g == d0 / Gm::GSZ) bias = pbt[g];
      float ov[VDPL];
#pragma unroll
      for (int d = 0; d < VDPL; ++d) ov[d] = rows_sum<VLPR>(st.o[j][h][d]) + bias;
      float* dst = orow(j) + d0;
      if (vrg == 0) {
        if constexpr (VDPL % 4 == 0) {
#pragma unroll
          for (int d = 0; d < VDPL; d += 4)
            *reinterpret_cast<float4*>(dst + d) = make_float4(ov[d], ov[d + 1], ov[d + 2], ov[d + 3]);
        } else {
#pragma unroll
          for (int d = 0; d < VDPL; ++d) dst[d] = ov[d];
        }
      }
    }
    if (lane == 0) set_ml(j, (st.m[j] == M_EMPTY) ? -INFINITY : st.m[j], l);
  }
}

__device__ __forceinline__ int clamp_len(const PartialArgs& a, int b) {
  return max(0, min(a.lengths[b], a.len_cap));
}

// ------------------------------------------------------------------- q in the codes' pair order

// One workgroup (PREP_THREADS threads) per unit.  Block b = ((g * NHB + hb) * QVW + j) of
// Q_BLOCK_WORDS words holds the 16 q pairs of 16-pair block hb of scale group g for vector j, in
// the order the K phase meets the codes; the last block of each group then holds (affine pages)
// the f32 sum of q over the group's dims, the bias term's factor (one wave per (group, vector),
// each lane adding GSZ / 64 dims).  Every load is issued before the first store (the stores may
// alias q as far as the compiler knows, so a load after a store would wait for it): the kernel
// takes about one memory round trip instead of one per element.
constexpr int PREP_THREADS = 256;

template <int BITS, int D, int QVW, int GS>
__device__ __forceinline__ void prep_q(const PartialArgs& a, int64_t u) {
  using Gm = Geo<BITS, D, GS>;
  constexpr int G = Gm::G, NHB = Gm::NHB, GSZ = Gm::GSZ, QBS = Q_BLOCK_WORDS;
  constexpr int NE = G * NHB * QVW * 16;                       // q pairs of the unit
  constexpr int PER = (NE + PREP_THREADS - 1) / PREP_THREADS;  // pairs per thread
  constexpr int NW = PREP_THREADS / 64;
  constexpr int NGJ = G * QVW, PERW = (NGJ + NW - 1) / NW;      // (group, vector) sums per wave
  constexpr int KS = GSZ / 64 + (GSZ < 64);                     // q elements per lane and sum
  const int qg = (int)(u % a.qgroups);
  const int hk = (int)((u / a.qgroups) % a.HK);
  const int b = (int)(u / ((int64_t)a.qgroups * a.HK));
  const int REP = a.HQ / a.HK, N = a.N;
  auto qrow = [&](int j) -> const uint16_t* {
    const int jj = qg * QVW + j, h = hk * REP + jj / N, i = jj - (jj / N) * N;
    return a.q + (((int64_t)b * a.HQ + h) * N + i) * D;
  };
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t pr[PER];
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int e = tid + PREP_THREADS * r;
    pr[r] = 0;
    if (e < NE) {
      const int blk = e / 16, p = e - blk * 16;
      const int j = blk % QVW, ghb = blk / QVW;                 // ghb = g * NHB + hb
      int lo, hi;
      pair_dims<BITS>(ghb * 16 + p, lo, hi);
      const uint16_t* q = qrow(j);
      pr[r] = (uint32_t)q[lo] | ((uint32_t)q[hi] << 16);
    }
  }
  float xs[PERW][KS];
  if constexpr (Gm::AFF) {
#pragma unroll
    for (int it = 0; it < PERW; ++it) {
      const int gj = wave + NW * it;
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        xs[it][k] = 0.0f;
        if (gj < NGJ && k * 64 + lane < GSZ) {
          const int g = gj / QVW, j = gj - g * QVW;
          xs[it][k] = bf16_to_f32(qrow(j)[g * GSZ + k * 64 + lane]);
        }
      }
    }
  }
  uint32_t* out = a.qp + u * (G * NHB * QVW * QBS);
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int e = tid + PREP_THREADS * r;
    if (e < NE) out[(e / 16) * QBS + (e % 16)] = pr[r];
  }
  if constexpr (Gm::AFF) {
#pragma unroll
    for (int it = 0; it < PERW; ++it) {
      const int gj = wave + NW * it;
      float x = 0.0f;
#pragma unroll
      for (int k = 0; k < KS; ++k) x += xs[it][k];
      const float s = block_reduce<OpAdd, 1, 64>(x);
      if (gj < NGJ && lane == 0) {
        const int g = gj / QVW, j = gj - g * QVW;
        out[((g * NHB + NHB - 1) * QVW + j) * QBS + 16] = __float_as_uint(s);
      }
    }
  }
}

template <int BITS, int D, int QVW, int GS>
__global__ void __launch_bounds__(PREP_THREADS) qprep_kernel(PartialArgs a) {
  prep_q<BITS, D, QVW, GS>(a, blockIdx.x);
}

// Decode step, first launch: blocks [0, na) append the step's new rows (slots from the block
// table), blocks [na, na + units) prepare q for the vector engine.
template <int BITS, int D, int QVW, int GS, bool VQ>
__global__ void __launch_bounds__(PREP_THREADS) step_prep_kernel(AppendArgs ap, PartialArgs a, int na) {
  if ((int)blockIdx.x < na) {
    append_rows<BITS, Geo<BITS, D, GS>::GSZ>(ap, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
  } else if constexpr (VQ) {
    prep_q<BITS, D, QVW, GS>(a, (int64_t)blockIdx.x - na);
  }
}

// ------------------------------------------------------------------- fixed partitions

template <int BITS, int D, int DV, int QVW, int GS>
__global__ void __launch_bounds__(PV_WAVES * 64, 2)
partial_part_kernel(PartialArgs a) {
  // the waves' tile scratch, then (after a barrier) their partials for the combine
  __shared__ __align__(16) union {
    WaveScratch<BITS, DV, QVW, GS> ws[PV_WAVES];
    struct {
      float o[PV_WAVES][QVW][DV];
      float m[PV_WAVES][QVW], l[PV_WAVES][QVW];
    } comb;
  } sh;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int p = blockIdx.x;
  Unit un;
  un.b = blockIdx.z;
  un.hk = blockIdx.y / a.qgroups;
  un.qg = blockIdx.y - un.hk * a.qgroups;
  un.len = clamp_len(a, un.b);
  un.u = ((int64_t)un.b * a.HK + un.hk) * a.qgroups + un.qg;
  const int t0 = p * a.part_tokens;
  if (t0 >= un.len) return;                                      // uniform over the workgroup
  const int t1 = min(un.len, t0 + a.part_tokens);

  Acc<BITS, DV, QVW, GS> st;
  acc_init(st);
  int cur = t0 + wave * PV_TILE;
  run_tiles<BITS, D, DV, QVW, GS>(
      a, un, t1, [&]() { const int t = cur; cur += PV_WAVES * PV_TILE; return t; }, sh.ws[wave], st, lane);
  __syncthreads();
  acc_write<BITS, DV, QVW, GS>(
      st, lane, [&](int j) { return &sh.comb.o[wave][j][0]; },
      [&](int j, float m, float l) { sh.comb.m[wave][j] = m; sh.comb.l[wave][j] = l; });
  __syncthreads();

  // combine the waves (log-sum-exp), write this partition's partial
  const int REP = a.HQ / a.HK, N = a.N;
  for (int e = tid; e < QVW * DV; e += PV_WAVES * 64) {
    const int j = e / DV, d = e - j * DV;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < PV_WAVES; ++w) M = fmaxf(M, sh.comb.m[w][j]);
    float num = 0.0f, den = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < PV_WAVES; ++w) {
        const float mw = sh.comb.m[w][j];
        if (mw == -INFINITY) continue;
        const float f = fast_exp2(mw - M);
        num = fmaf(f, sh.comb.o[w][j][d], num);
        den = fmaf(f, sh.comb.l[w][j], den);
      }
    }
    const int jj = un.qg * QVW + j;
    const int h = un.hk * REP + jj / N, i = jj - (jj / N) * N;
    const int64_t idx = (((int64_t)un.b * a.HQ + h) * N + i) * a.num_parts + p;
    a.opart[idx * DV + d] = num;
    if (d == 0) { a.ml[idx * 2] = M; a.ml[idx * 2 + 1] = den; }
  }
}

// ------------------------------------------------------------------- balanced stream

template <int BITS, int D, int DV, int QVW, int GS>
__global__ void __launch_bounds__(VALU_STREAM_WAVES * 64, 1)
partial_stream_kernel(PartialArgs a) {
  constexpr int NW = VALU_STREAM_WAVES;
  // the waves' tile scratch; a wave done with the range's last set puts its partial of it in its
  // own scratch for the combine: [QVW][DV] o, then [QVW] m, then [QVW] l
  __shared__ __align__(16) WaveScratch<BITS, DV, QVW, GS> ws[NW];
  static_assert(sizeof(WaveScratch<BITS, DV, QVW, GS>) >= (QVW * DV + 2 * QVW + NW * QVW) * sizeof(float),
                "a wave's partial, and after wave 0's the combine's factor table, fit its scratch");
  __shared__ int tile_ctr;                                       // next tile of the range

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int B = a.batch;
  // Lanes: the L query groups of a set (KV head, L consecutive groups) run side by side on L
  // workgroups of one XCD, one group each, over the same range of the set stream, so each K/V row
  // comes from memory once for the set and the other lanes find it in that XCD's L2 cache.
  // L = 1: one workgroup per range, every group in turn.
  const int L = a.lanes;
  int g, ln;                                                     // this workgroup's range, lane
  stream_range_lane(L, blockIdx.x, gridDim.x, g, ln);
  g = uni(g);
  ln = uni(ln);
  const int QGB = a.qgroups / L, HS = a.HK * QGB;                // sets per KV head, per sequence

  // The stream: every set that has tokens takes C positions (the set cost: what changing sets costs
  // a wave -- its partial written, the next set's q copy and first rows fetched -- counted in
  // tokens) followed by one position per token; sequences of length 0 take none.  Ranges cut the
  // stream into equal parts, so a range whose tokens span two sets holds C fewer tokens.
  // Total length T and the number of working ranges (every wave computes the same):
  const StreamSpan sp = stream_span(a.lengths, B, a.len_cap, HS, a.num_ranges, a.min_tokens, a.set_cost, lane);
  const int C = sp.C;
  const int64_t T = sp.T;
  const int R = sp.R;
  if (g >= R) return;                                            // whole workgroup
  const int64_t x0 = ((int64_t)g * T + R - 1) / R;
  const int64_t x1 = ((int64_t)(g + 1) * T + R - 1) / R;
  if (x0 >= x1) return;                                          // whole workgroup

  // locate the sequence holding stream position x0 (the first with prefix end > x0)
  int b = -1;
  int64_t pb = 0;                                                // positions of sequences before b
  {
    int64_t base = 0;
    for (int c = 0; c < B; c += 64) {
      const int bb = c + lane;
      const int l = bb < B ? clamp_len(a, bb) : 0;
      const uint32_t lv = l > 0 ? (uint32_t)l + (uint32_t)C : 0u;   // < 2^31 + 4097
      const int64_t incl = (int64_t)wave_scan_u64(lv);
      const uint64_t hit = __ballot((base + incl) * HS > x0 && lv > 0);
      if (hit) {
        const int k = __builtin_ctzll(hit);
        b = uni(c + k);
        pb = base + (int64_t)lane_u64((uint64_t)incl, k) - (int64_t)lane_u64(lv, k);
        break;
      }
      base += (int64_t)lane_u64((uint64_t)incl, 63);
    }
  }
  if (b < 0) return;                                             // x0 < T: not reached
  int len = uni(clamp_len(a, b));
  int64_t lp = (int64_t)len + C;                                 // positions of one set of b
  int uu = uni((int)((x0 - pb * HS) / lp));                      // set within the sequence
  int64_t start = pb * HS + (int64_t)uu * lp;                    // the set's first position
  // the range's tokens of this set: [t_lo, t_hi); none if the range lies within its C positions
  int t_lo = uni((int)max<int64_t>(0, x0 - start - C));
  int t_hi = uni((int)min<int64_t>(len, x1 - start - C));
  if (t_hi <= t_lo) return;                                      // whole workgroup
  if (threadIdx.x == 0) tile_ctr = 0;
  __syncthreads();

  // The range is a list of tiles: set by set, the set's part of the range cut into 64-token
  // tiles.  The workgroup's waves take tiles from one LDS counter, so faster waves take more of
  // them; every wave walks every set of the range.  For a set that ends inside the range each
  // wave writes its own partial (possibly empty) at slot ((set + range) * L + lane) * NW + wave;
  // the range's last set, whose tiles end with the range, has its waves' partials combined in LDS
  // and written once, at slot ((set + range) * L + lane) * NW (a barrier there costs nothing:
  // every wave is done).
  auto take = [&]() {
    int k = 0;
    if (lane == 0) k = atomicAdd(&tile_ctr, 1);
    return uni(k);
  };
  int kq = -1;                          // a tile this wave claimed for a later set (-1: none)
  int kbase = 0;                                                 // first tile of the current set
  float* const opart = a.opart;
  float* const ml = a.ml;
  while (true) {
    const int seg = t_hi - t_lo;                                 // > 0
    const int t_end = t_hi, ntiles = (seg + PV_TILE - 1) / PV_TILE;
    Unit un;
    un.b = b; un.hk = uu / QGB; un.qg = (uu - un.hk * QGB) * L + ln; un.len = len;
    un.u = ((int64_t)b * a.HK + un.hk) * a.qgroups + un.qg;
    Acc<BITS, DV, QVW, GS> st;
    acc_init(st);
    const int t0u = t_lo, kb = kbase;
    run_tiles<BITS, D, DV, QVW, GS>(
        a, un, t_end,
        [&]() {
          // claim a tile as it is needed; one that lies in a later set is kept for it
          if (kq < 0) kq = take();
          const int k = kq;
          if (k - kb >= ntiles) return t_end;                    // the set's tiles are all taken
          kq = -1;
          return t0u + (k - kb) * PV_TILE;
        },
        ws[wave], st, lane);
    const int64_t slot = (((int64_t)b * HS + uu + g) * L + ln) * NW;
    // the next set starts at position start + lp; it has a token in the range if its first token,
    // C positions on, comes before x1 (a later set then too, and the next one has tokens: empty
    // sequences take no positions)
    const int64_t next = start + lp;
    if (next + C < x1) {
      // a set that ends inside the range: one partial per wave (no barrier: the waves that are
      // done with its tiles go on to the next set)
      acc_write<BITS, DV, QVW, GS>(
          st, lane, [&](int j) { return opart + ((slot + wave) * QVW + j) * DV; },
          [&](int j, float m, float l) {
            ml[((slot + wave) * QVW + j) * 2] = m; ml[((slot + wave) * QVW + j) * 2 + 1] = l;
          });
      kbase += ntiles;
      if (++uu == HS) {
        uu = 0;
        do { ++b; } while (b < B && clamp_len(a, b) == 0);
        if (b >= B) break;                                       // (next < T: not reached)
        len = uni(clamp_len(a, b));
        lp = (int64_t)len + C;
      }
      start = next;
      t_lo = 0;
      t_hi = uni((int)min<int64_t>(len, x1 - start - C));        // >= 1
      continue;
    }
    // the range's last set: each wave, done with its tiles, puts its partial in its own scratch;
    // once all are there they combine (log-sum-exp) into one, written at the set's first slot of
    // the range
    {
      float* mine = reinterpret_cast<float*>(&ws[wave]);
      acc_write<BITS, DV, QVW, GS>(
          st, lane, [&](int j) { return mine + j * DV; },
          [&](int j, float m, float l) { mine[QVW * DV + j] = m; mine[QVW * DV + QVW + j] = l; });
    }
    __syncthreads();
    // one lane per vector: the running max M over the waves, each wave's factor 2^(m_w - M) (0 for
    // a wave that saw no token) and the combined normaliser, into a table after wave 0's partial;
    // then every thread of the workgroup sums the waves' o for its elements with those factors
    auto part = [&](int w) { return reinterpret_cast<const float*>(&ws[w]); };
    float* tab = reinterpret_cast<float*>(&ws[0]) + QVW * DV + 2 * QVW;   // [NW][QVW] factors
    if (threadIdx.x < QVW) {
      const int j = threadIdx.x;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, part(w)[QVW * DV + j]);
      float den = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = part(w)[QVW * DV + j];
        const float f = (M == -INFINITY || mw == -INFINITY) ? 0.0f : fast_exp2(mw - M);
        tab[w * QVW + j] = f;
        den = fmaf(f, part(w)[QVW * DV + QVW + j], den);
      }
      ml[(slot * QVW + j) * 2] = M;
      ml[(slot * QVW + j) * 2 + 1] = den;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < QVW * DV; e += NW * 64) {
      const int j = e / DV, d = e - j * DV;
      float num = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) num = fmaf(tab[w * QVW + j], part(w)[j * DV + d], num);
      opart[(slot * QVW + j) * DV + d] = num;
    }
    break;
  }
}

// ------------------------------------------------------------------- launch

template <int BITS, int D, int DV, int QVW, int GS>
static hipError_t launch_valu(const PartialArgs& a, int B, bool q_ready, hipStream_t s) {
  const unsigned units = (unsigned)((int64_t)B * a.HK * a.qgroups);
  if (!q_ready) hipLaunchKernelGGL((qprep_kernel<BITS, D, QVW, GS>), dim3(units), dim3(PREP_THREADS), 0, s, a);
  if (a.part_tokens > 0) {
    dim3 grid((unsigned)a.num_parts, (unsigned)(a.HK * a.qgroups), (unsigned)B);
    hipLaunchKernelGGL((partial_part_kernel<BITS, D, DV, QVW, GS>), grid, dim3(PV_WAVES * 64), 0, s, a);
  } else {
    hipLaunchKernelGGL((partial_stream_kernel<BITS, D, DV, QVW, GS>), dim3((unsigned)(a.num_ranges * a.lanes)),
                       dim3(VALU_STREAM_WAVES * 64), 0, s, a);
  }
  return hipGetLastError();
}

template <int BITS, int D, int QVW, int GS>
static hipError_t launch_step(const AppendArgs& ap, const PartialArgs& a, bool vq, int B, hipStream_t s) {
  // (the V head dim enters only through ap.Dv)
  const int64_t total = (int64_t)ap.T * ap.HK * (max(ap.D, ap.Dv) / append_ept(BITS));
  const int na = (int)((total + PREP_THREADS - 1) / PREP_THREADS);
  const int nq = vq ? (int)((int64_t)B * a.HK * a.qgroups) : 0;
  if (na + nq == 0) return hipSuccess;
  if (vq)
    hipLaunchKernelGGL((step_prep_kernel<BITS, D, QVW, GS, true>), dim3((unsigned)(na + nq)), dim3(PREP_THREADS), 0, s, ap, a,
                       na);
  else
    hipLaunchKernelGGL((step_prep_kernel<BITS, D, QVW, GS, false>), dim3((unsigned)na), dim3(PREP_THREADS), 0, s, ap, a, na);
  return hipGetLastError();
}

// one call of F<BITS, D, DV, QVW, GS> for the runtime qvw, or hipErrorInvalidValue
template <int BITS, int D, int DV, int GS, class F>
static hipError_t with_qvw(int qvw, F f) {
  switch (qvw) {
    case 1: return f.template run<BITS, D, DV, 1, GS>();
    case 2: return f.template run<BITS, D, DV, 2, GS>();
    case 4: return f.template run<BITS, D, DV, 4, GS>();
    case 8:
      if constexpr (valu_max_qvw(BITS, D, DV, GS) >= 8) return f.template run<BITS, D, DV, 8, GS>();
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <int BITS, int D, class F>
static hipError_t with_group(int gs, int qvw, F f) {
  if constexpr (BITS == 16) {
    return with_qvw<BITS, D, D, 64>(qvw, f);                 // bf16 pages have no scale groups
  } else {
    switch (gs) {
      case 32: return with_qvw<BITS, D, D, 32>(qvw, f);
      case 64: return with_qvw<BITS, D, D, 64>(qvw, f);
      case 128:
        if constexpr (D >= 128) return with_qvw<BITS, D, D, 128>(qvw, f);
        return hipErrorInvalidValue;
      default: return hipErrorInvalidValue;
    }
  }
}

// V rows of a head dim of their own: DV = D / 2 or 2 D, 64-element scale groups (bf16 pages
// have none), bf16, 8-, 4- and 2-bit pages (valu_dv_ok)
template <int BITS, int D, class F>
static hipError_t with_dv(int DV, int gs, int qvw, F f) {
  if constexpr (BITS == 16 || BITS == 8 || BITS == 4 || BITS == 2) {
    if (BITS != 16 && gs != 64) return hipErrorInvalidValue;
    if constexpr (D >= 128) {
      if (2 * DV == D) return with_qvw<BITS, D, D / 2, 64>(qvw, f);
    }
    if constexpr (D <= 128) {
      if (DV == 2 * D) return with_qvw<BITS, D, 2 * D, 64>(qvw, f);
    }
  }
  return hipErrorInvalidValue;
}

template <int BITS, class F>
static hipError_t with_shape(int D, int DV, int gs, int qvw, F f) {
  switch (D) {
    case 64:
      if constexpr (valu_row_ok(BITS, 64)) return DV == D ? with_group<BITS, 64>(gs, qvw, f) : with_dv<BITS, 64>(DV, gs, qvw, f);
      return hipErrorInvalidValue;
    case 128: return DV == D ? with_group<BITS, 128>(gs, qvw, f) : with_dv<BITS, 128>(DV, gs, qvw, f);
    case 256: return DV == D ? with_group<BITS, 256>(gs, qvw, f) : with_dv<BITS, 256>(DV, gs, qvw, f);
    default: return hipErrorInvalidValue;
  }
}

struct PartialLaunch {
  const PartialArgs& a; int B; bool q_ready; hipStream_t s;
  template <int BITS, int D, int DV, int QVW, int GS>
  hipError_t run() const { return launch_valu<BITS, D, DV, QVW, GS>(a, B, q_ready, s); }
};

struct StepLaunch {
  const AppendArgs& ap; const PartialArgs& a; bool vq; int B; hipStream_t s;
  template <int BITS, int D, int DV, int QVW, int GS>
  hipError_t run() const { return launch_step<BITS, D, QVW, GS>(ap, a, vq, B, s); }
};

template <int BITS>
hipError_t launch_valu_bits(const PartialArgs& a, int D, int DV, int gs, int qvw, int B, bool q_ready, hipStream_t s) {
  return with_shape<BITS>(D, DV, gs, qvw, PartialLaunch{a, B, q_ready, s});
}

template <int BITS>
hipError_t launch_step_bits(const AppendArgs& ap, const PartialArgs& a, int D, int gs, int qvw, bool vq, int B,
                            hipStream_t s) {
  // without the q copy the step kernel is only the append: one instance per (D, group); it reads
  // the V head dim from ap, so every V head dim shares the K head dim's instance
  return with_shape<BITS>(D, D, gs, vq ? qvw : 1, StepLaunch{ap, a, vq, B, s});
}

}  // namespace kvq
