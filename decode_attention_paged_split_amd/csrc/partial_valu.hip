// Split-K partial kernel of paged decode attention (vector ALU engine).
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
// gfx950 layout (not the pages' Metal one).  A workgroup is (partition, KV head [x query
// group], sequence) with 4 waves; each wave walks tiles of TILE consecutive tokens of the
// partition.  Per tile:
//  1. K phase -- 16-byte coalesced loads, KLPR lanes per row, each lane owning KDPL
//     consecutive head dims.  Codes become bf16 pairs with one v_and_or (4/2-bit codes c
//     as bf16(128 + c), exact; 8-bit codes through an exact f32 conversion) and meet q in
//     v_dot2_f32_bf16 (q is exact in bf16, products are exact, sums are f32).  q pairs come
//     from LDS, each 16-byte q read serving every row the lane holds.  The group's scale and
//     bias are applied once per lane: q.k = s * sum(q c) + (b - 128 s) * sum(q).  Partial
//     dots reduce across the KLPR lanes of a row with DPP.
//  2. Softmax pass -- one lane per (row, head group) reads the tile's scores from LDS:
//     tile max across rows (DPP / permlane), one exp2 per (token, head), running max and
//     normaliser per head; probabilities go back to LDS.
//  3. V phase -- 4/8-byte loads, VLPR lanes per row, each lane owning VDPL dims of one row
//     per load; V is dequantized in f32 registers (fma(scale, code, bias)) and accumulated
//     as o[head][dim] += p[head] * v[dim] in f32 after one rescale of o per tile.
// The affine scales and biases of a tile are staged once in LDS as f32 (scale, bias).
// When a full tile lies inside one block its rows sit at one base address; otherwise lane r
// looks up token r of the tile in the block table and the others fetch it by lane shuffle.
//
// Two schedules share this tile engine:
//  * fixed partitions (partition_tokens > 0): workgroup = (partition, KV head x query group,
//    sequence); its 4 waves interleave tiles and combine in LDS; one partial per partition.
//  * balanced stream (partition_tokens == 0): every cached token of every (sequence, KV
//    head, query group) unit is laid end to end in one stream of T tokens, cut into W_eff
//    equal ranges, one per wave (W_eff = min(waves launched, ceil(T / TILE))).  A wave walks
//    its range unit by unit and writes one partial per unit it touches, at slot unit + wave
//    (distinct for every (unit, wave) pair because ranges are contiguous and ordered).  All
//    waves get the same number of tokens whatever the length mix, and partials stay few.
#include "device_common.hpp"
#include "kernels.hpp"

namespace kvq {

constexpr int PV_WAVES = 4;

template <int BITS, int D>
struct Geo {
  static constexpr int ROWB = D * BITS / 8;                          // bytes per pool row
  static constexpr int KLPR0 = ROWB / 16;
  static constexpr int KLPR = KLPR0 < 8 ? KLPR0 : 8;                 // lanes per row (K)
  static constexpr int KCH = ROWB / 16 / KLPR;                       // 16-byte chunks per lane
  static constexpr int KRPL = 64 / KLPR;                             // rows per K load
  static constexpr int KDPL = KCH * 16 * 8 / BITS;                   // dims per lane (K)
  static constexpr int KNP = KDPL / 2;                               // bf16 pairs per lane
  static constexpr int TILE = KRPL > 32 ? KRPL : 32;                 // tokens per tile
  static constexpr int NBK = TILE / KRPL;                            // K loads per tile
  static constexpr int VW = (BITS == 16) ? 8 : 4;                    // bytes per lane per row (V)
  static constexpr int VLPR = ROWB / VW;                             // lanes per row (V)
  static constexpr int VRPL = 64 / VLPR;                             // rows per V load
  static constexpr int VDPL = VW * 8 / BITS;                         // dims per lane (V)
  static constexpr int NBV = TILE / VRPL;                            // V loads per tile
  static constexpr int G = D / 64;
  static constexpr int PPW = (BITS == 16) ? 1 : 16 / BITS;           // bf16 pairs per 32-bit word
  static constexpr float OFFS = (BITS == 4 || BITS == 2) ? 128.0f : 0.0f;
  static_assert(KLPR >= 1 && KRPL <= 64 && VLPR >= 1 && VLPR <= 64, "row layout");
  static_assert(TILE % VRPL == 0 && TILE <= 64, "tile");
};

// dims (lo, hi) of bf16 pair P in the K lanes' order (natural word order; inside a word the
// pairing the unpack below produces)
template <int BITS>
__device__ __forceinline__ void pair_dims(int P, int& lo, int& hi) {
  if constexpr (BITS == 4) {
    const int w = P >> 2, k = P & 3; lo = 8 * w + k; hi = lo + 4;
  } else if constexpr (BITS == 2) {
    const int w = P >> 3, k = P & 7; lo = 16 * w + k; hi = lo + 8;
  } else if constexpr (BITS == 8) {
    lo = 2 * P; hi = lo + 1;
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

// VW bytes of a V row -> VDPL f32 values (natural dim order)
template <int BITS, int VDPL>
__device__ __forceinline__ void value_f32(const uint32_t* w, float s, float b, float* v) {
  if constexpr (BITS == 16) {
#pragma unroll
    for (int k = 0; k < VDPL / 2; ++k) { v[2 * k] = bf16_lo(w[k]); v[2 * k + 1] = bf16_hi(w[k]); }
  } else if constexpr (BITS == 8) {
    v[0] = fmaf(s, ubyte_f32<0>(w[0]), b); v[1] = fmaf(s, ubyte_f32<1>(w[0]), b);
    v[2] = fmaf(s, ubyte_f32<2>(w[0]), b); v[3] = fmaf(s, ubyte_f32<3>(w[0]), b);
  } else {
    // mask the codes into bytes, then v_cvt_f32_ubyte{0..3} converts one code each
    constexpr int PER = 8 / BITS;                                   // codes per byte
    constexpr uint32_t M = (BITS == 4) ? 0x0F0F0F0Fu : 0x03030303u;
#pragma unroll
    for (int sh = 0; sh < PER; ++sh) {
      const uint32_t x = (w[0] >> (BITS * sh)) & M;
      v[0 * PER + sh] = fmaf(s, ubyte_f32<0>(x), b);
      v[1 * PER + sh] = fmaf(s, ubyte_f32<1>(x), b);
      v[2 * PER + sh] = fmaf(s, ubyte_f32<2>(x), b);
      v[3 * PER + sh] = fmaf(s, ubyte_f32<3>(x), b);
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


template <int BITS, int D, int QVW>
struct Shape {
  using Gm = Geo<BITS, D>;
  static constexpr int TILE = Gm::TILE;
  static constexpr int SH = 64 / TILE;                           // softmax lanes per row
  static constexpr int QS = (QVW + SH - 1) / SH;                 // heads per softmax lane
  static constexpr bool AFF = BITS != 16;
};

// per-wave LDS scratch of the tile engine
template <int BITS, int D, int QVW>
struct WaveScratch {
  using Gm = Geo<BITS, D>;
  float z[Gm::TILE][QVW];                                        // scores, then probabilities
  float2 sb[BITS != 16 ? 2 : 1][BITS != 16 ? Gm::TILE : 1][Gm::G];  // (scale, bias) of K and V
};

// running state of one wave over one segment of one unit
template <int BITS, int D, int QVW>
struct Acc {
  float o[QVW][Geo<BITS, D>::VDPL];                              // V lanes: o[vector][dim]
  float m[Shape<BITS, D, QVW>::QS], l[Shape<BITS, D, QVW>::QS];  // softmax lanes: per vector
};

struct Unit {
  int b, hk, qg, len;
};

// q of the unit's QVW query vectors -> LDS as bf16 pairs in the K lanes' order, plus the sum
// of q over each K lane's dims (for the bias term)
template <int BITS, int D, int QVW>
__device__ __forceinline__ void load_q(const PartialArgs& a, const Unit& un, uint32_t (*q_lds)[D / 2],
                                       float (*qs_lds)[Geo<BITS, D>::KLPR], int tid, int nthr) {
  using Gm = Geo<BITS, D>;
  const int REP = a.HQ / a.HK, N = a.N;
  for (int idx = tid; idx < QVW * (D / 2); idx += nthr) {
    const int j = idx / (D / 2), P = idx - j * (D / 2);
    const int jj = un.qg * QVW + j, h = un.hk * REP + jj / N, i = jj - (jj / N) * N;
    const uint16_t* qrow = a.q + (((int64_t)un.b * a.HQ + h) * N + i) * D;
    int lo, hi;
    pair_dims<BITS>(P, lo, hi);
    q_lds[j][P] = (uint32_t)qrow[lo] | ((uint32_t)qrow[hi] << 16);
  }
  if constexpr (BITS != 16) {
    constexpr int KLPR = Gm::KLPR, KDPL = Gm::KDPL;
    for (int idx = tid; idx < QVW * KLPR; idx += nthr) {
      const int j = idx / KLPR, sl = idx - j * KLPR;
      const int jj = un.qg * QVW + j, h = un.hk * REP + jj / N, i = jj - (jj / N) * N;
      const uint16_t* qrow = a.q + (((int64_t)un.b * a.HQ + h) * N + i) * D + sl * KDPL;
      float s = 0.0f;
      for (int d = 0; d < KDPL; ++d) s += bf16_to_f32(qrow[d]);
      qs_lds[j][sl] = s;
    }
  }
}

template <int BITS, int D, int QVW>
__device__ __forceinline__ void acc_init(Acc<BITS, D, QVW>& st) {
  using Sp = Shape<BITS, D, QVW>;
#pragma unroll
  for (int j = 0; j < QVW; ++j)
#pragma unroll
    for (int d = 0; d < Geo<BITS, D>::VDPL; ++d) st.o[j][d] = 0.0f;
#pragma unroll
  for (int hh = 0; hh < Sp::QS; ++hh) { st.m[hh] = -INFINITY; st.l[hh] = 0.0f; }
}

// Tiles t_first, t_first + stride, ... (< t1) of unit un, accumulated into st by one wave.
template <int BITS, int D, int QVW>
__device__ __forceinline__ void run_tiles(const PartialArgs& a, const Unit& un, int t_first, int t1, int stride,
                                          const uint32_t (*q_lds)[D / 2], const float (*qs_lds)[Geo<BITS, D>::KLPR],
                                          WaveScratch<BITS, D, QVW>& ws, Acc<BITS, D, QVW>& st, int lane) {
  using Gm = Geo<BITS, D>;
  using Sp = Shape<BITS, D, QVW>;
  constexpr int TILE = Gm::TILE, KLPR = Gm::KLPR, KRPL = Gm::KRPL, KCH = Gm::KCH, KNP = Gm::KNP;
  constexpr int NBK = Gm::NBK, VLPR = Gm::VLPR, VRPL = Gm::VRPL, VDPL = Gm::VDPL, NBV = Gm::NBV;
  constexpr int G = Gm::G, ROWB = Gm::ROWB, VW = Gm::VW;
  constexpr bool AFF = Sp::AFF;
  constexpr int QS = Sp::QS;
  const int hk = un.hk, N = a.N;

  const int ksl = lane % KLPR, krg = lane / KLPR;                // K: dim chunk, row in load
  const int vsl = lane % VLPR, vrg = lane / VLPR;                // V: dim chunk, row in load
  const int srow = lane % TILE, spart = lane / TILE;             // softmax: row, head group
  const int kgrp = (ksl * Gm::KDPL) / 64, vgrp = (vsl * VDPL) / 64;
  (void)VLPR;
  float qlane[QVW];
#pragma unroll
  for (int j = 0; j < QVW; ++j) qlane[j] = AFF ? qs_lds[j][ksl] : 0.0f;
  int vend[QS];
#pragma unroll
  for (int hh = 0; hh < QS; ++hh) {
    const int j = spart * QS + hh;
    const int jj = un.qg * QVW + (j < QVW ? j : 0);
    const int i = jj - (jj / N) * N;
    vend[hh] = (j < QVW) ? un.len - N + i + 1 : 0;
  }
  const char* kplane = static_cast<const char*>(a.k);
  const char* vplane = static_cast<const char*>(a.v);
  const int32_t* trow = a.table + (int64_t)un.b * a.max_blocks;
  const uint32_t magic = 0x43004300u;

  auto row_of = [&](int t) -> int64_t {                          // pool row of token t
    const int blk = (a.bs_shift >= 0) ? (t >> a.bs_shift) : (t / a.BS);
    const int off = t - blk * a.BS;
    int phys = trow[blk];
    phys = min(max(phys, 0), a.num_blocks - 1);                   // a bad entry cannot fault
    return ((int64_t)phys * a.HK + hk) * a.BS + off;
  };

  for (int tt = t_first; tt < t1; tt += stride) {
    const int last = t1 - 1 - tt;                                 // rows > last are past the end
    // ---- loads of the tile.  A full tile inside one block: one base row and per-lane
    // constant offsets.  Otherwise lane r < TILE looks up token tt + min(r, last) in the block
    // table and the other lanes fetch row indices by lane shuffle.
    const bool one_block = (a.bs_shift >= 0) && ((tt & (a.BS - 1)) + TILE <= a.BS);
    const bool fast = one_block && last >= TILE - 1;
    uint4 kraw[NBK][KCH];
    uint32_t vraw[NBV][VW / 4];
    int64_t krow[NBK], vrow[NBV], srow_e[(2 * TILE + 63) / 64];
    if (fast) {
      const int64_t base = row_of(tt);
#pragma unroll
      for (int i = 0; i < NBK; ++i) krow[i] = base + (krg + KRPL * i);
#pragma unroll
      for (int i = 0; i < NBV; ++i) vrow[i] = base + (vrg + VRPL * i);
#pragma unroll
      for (int e0 = 0; e0 < 2 * TILE; e0 += 64) srow_e[e0 / 64] = base + ((e0 + lane) % TILE);
    } else {
      const int my_row = (int)row_of(tt + min(lane % TILE, last));
#pragma unroll
      for (int i = 0; i < NBK; ++i) krow[i] = __shfl(my_row, krg + KRPL * i, 64);
#pragma unroll
      for (int i = 0; i < NBV; ++i) vrow[i] = __shfl(my_row, vrg + VRPL * i, 64);
#pragma unroll
      for (int e0 = 0; e0 < 2 * TILE; e0 += 64) srow_e[e0 / 64] = __shfl(my_row, (e0 + lane) % TILE, 64);
    }
#pragma unroll
    for (int i = 0; i < NBK; ++i) {
      const char* src = kplane + krow[i] * ROWB + ksl * (KCH * 16);
#pragma unroll
      for (int c = 0; c < KCH; ++c) kraw[i][c] = *reinterpret_cast<const uint4*>(src + 16 * c);
    }
#pragma unroll
    for (int i = 0; i < NBV; ++i) {
      const char* src = vplane + vrow[i] * ROWB + vsl * VW;
      if constexpr (VW == 8) {
        const uint2 x = *reinterpret_cast<const uint2*>(src);
        vraw[i][0] = x.x; vraw[i][1] = x.y;
      } else {
        vraw[i][0] = *reinterpret_cast<const uint32_t*>(src);
      }
    }
    if constexpr (AFF) {
      // (scale, bias) of K and V for the tile's rows -> LDS as f32 pairs
#pragma unroll
      for (int e0 = 0; e0 < 2 * TILE; e0 += 64) {
        const int e = e0 + lane;
        if (e < 2 * TILE) {
          const int kv = e / TILE, r = e - kv * TILE;
          const int64_t ri = srow_e[e0 / 64] * G;
          const uint16_t* sp = kv ? a.vs : a.ks;
          const uint16_t* bp = kv ? a.vb : a.kb;
#pragma unroll
          for (int g = 0; g < G; ++g)
            ws.sb[kv][r][g] = make_float2(bf16_to_f32(sp[ri + g]), bf16_to_f32(bp[ri + g]));
        }
      }
      wave_lds_sync();
    }

    // ---- K phase: partial dots of every row held by the lane with every query vector.
    // Words are unpacked a step at a time (PPS >= 4 pairs), each 16-byte q read serving the
    // NBK rows the lane holds.
    constexpr int PPW = Gm::PPW;
    constexpr int WPS = (PPW >= 4) ? 1 : 4 / PPW;                  // words per step
    constexpr int PPS = WPS * PPW;                                 // pairs per step
    float acc[NBK][QVW];
#pragma unroll
    for (int i = 0; i < NBK; ++i)
#pragma unroll
      for (int j = 0; j < QVW; ++j) acc[i][j] = 0.0f;
#pragma unroll
    for (int st = 0; st < KNP / PPS; ++st) {
      uint32_t kp[NBK][PPS];
#pragma unroll
      for (int i = 0; i < NBK; ++i)
#pragma unroll
        for (int ws = 0; ws < WPS; ++ws) {
          const int wi = st * WPS + ws;
          const uint4 c4 = kraw[i][wi >> 2];
          const uint32_t word = (wi & 3) == 0 ? c4.x : (wi & 3) == 1 ? c4.y : (wi & 3) == 2 ? c4.z : c4.w;
          word_pairs<BITS>(word, &kp[i][ws * PPW], magic);
        }
#pragma unroll
      for (int j = 0; j < QVW; ++j) {
#pragma unroll
        for (int c4 = 0; c4 < PPS / 4; ++c4) {
          const int cc = st * (PPS / 4) + c4;
          const uint4 qq = *reinterpret_cast<const uint4*>(&q_lds[j][ksl * KNP + cc * 4]);
          const uint32_t qv[4] = {qq.x, qq.y, qq.z, qq.w};
#pragma unroll
          for (int i = 0; i < NBK; ++i)
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[i][j] = dot2_bf16(qv[k], kp[i][c4 * 4 + k], acc[i][j]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NBK; ++i) {
      float s = 1.0f, bb = 0.0f;
      if constexpr (AFF) {
        const float2 sb = ws.sb[0][krg + KRPL * i][kgrp];
        s = sb.x;
        bb = fmaf(-Gm::OFFS, sb.x, sb.y);
      }
#pragma unroll
      for (int j = 0; j < QVW; ++j) {
        float z = AFF ? fmaf(s, acc[i][j], bb * qlane[j]) : acc[i][j];
        z = block_reduce<OpAdd, 1, KLPR>(z);
        acc[i][j] = z;
      }
    }
    if (ksl == 0) {
#pragma unroll
      for (int i = 0; i < NBK; ++i)
#pragma unroll
        for (int j = 0; j < QVW; ++j) ws.z[krg + KRPL * i][j] = acc[i][j];
    }
    wave_lds_sync();

    // ---- softmax pass: one lane per (row, head group)
    const int tok = tt + srow;
    float alpha_s[QS];
#pragma unroll
    for (int hh = 0; hh < QS; ++hh) {
      const int j = spart * QS + hh;
      const bool jv = j < QVW;
      float z = jv ? ws.z[srow][j] * a.scale_log2e : -INFINITY;
      if (tok >= t1 || tok >= vend[hh]) z = -INFINITY;
      float mt = block_reduce<OpMax, 1, TILE>(z);
      const float mnew = fmaxf(st.m[hh], mt);
      const float muse = (mnew == -INFINITY) ? 0.0f : mnew;
      const float al = fast_exp2(st.m[hh] - muse);
      const float pz = fast_exp2(z - muse);
      st.l[hh] = fmaf(st.l[hh], al, pz);
      st.m[hh] = mnew;
      alpha_s[hh] = al;
      if (jv) ws.z[srow][j] = pz;
    }
    wave_lds_sync();

    // ---- V phase
#pragma unroll
    for (int j = 0; j < QVW; ++j) {
      const float al = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha_s[j % QS]), (j / QS) * TILE));
#pragma unroll
      for (int d = 0; d < VDPL; ++d) st.o[j][d] *= al;
    }
#pragma unroll
    for (int i = 0; i < NBV; ++i) {
      const int r = vrg + VRPL * i;
      float pr[QVW];
      if constexpr (QVW % 4 == 0) {
#pragma unroll
        for (int j4 = 0; j4 < QVW / 4; ++j4) {
          const float4 x = *reinterpret_cast<const float4*>(&ws.z[r][4 * j4]);
          pr[4 * j4] = x.x; pr[4 * j4 + 1] = x.y; pr[4 * j4 + 2] = x.z; pr[4 * j4 + 3] = x.w;
        }
      } else {
#pragma unroll
        for (int j = 0; j < QVW; ++j) pr[j] = ws.z[r][j];
      }
      float s = 0.0f, bb = 0.0f;
      if constexpr (AFF) {
        const float2 sb = ws.sb[1][r][vgrp];
        s = sb.x; bb = sb.y;
      }
      float vv[VDPL];
      value_f32<BITS, VDPL>(vraw[i], s, bb, vv);
#pragma unroll
      for (int j = 0; j < QVW; ++j)
#pragma unroll
        for (int d = 0; d < VDPL; ++d) st.o[j][d] = fmaf(pr[j], vv[d], st.o[j][d]);
    }
    wave_lds_sync();                      // z_lds / sb_lds are rewritten by the next tile
  }

}

// sum o over the VRPL row slots of the wave and l over the TILE softmax rows
template <int BITS, int D, int QVW>
__device__ __forceinline__ void acc_finish(Acc<BITS, D, QVW>& st) {
  using Gm = Geo<BITS, D>;
  using Sp = Shape<BITS, D, QVW>;
#pragma unroll
  for (int j = 0; j < QVW; ++j)
#pragma unroll
    for (int d = 0; d < Gm::VDPL; ++d) {
      float x = st.o[j][d];
#pragma unroll
      for (int off = Gm::VLPR; off < 64; off *= 2) x += __shfl_xor(x, off, 64);
      st.o[j][d] = x;
    }
#pragma unroll
  for (int hh = 0; hh < Sp::QS; ++hh) st.l[hh] = block_reduce<OpAdd, 1, Gm::TILE>(st.l[hh]);
}

__device__ __forceinline__ int clamp_len(const PartialArgs& a, int b) {
  return max(0, min(a.lengths[b], a.len_cap));
}

// ------------------------------------------------------------------- fixed partitions

template <int BITS, int D, int QVW>
__global__ void __launch_bounds__(PV_WAVES * 64, 2)
partial_part_kernel(PartialArgs a) {
  using Gm = Geo<BITS, D>;
  using Sp = Shape<BITS, D, QVW>;
  constexpr int TILE = Gm::TILE, VDPL = Gm::VDPL, VLPR = Gm::VLPR, QS = Sp::QS;
  __shared__ __align__(16) uint32_t q_lds[QVW][D / 2];
  __shared__ float qs_lds[QVW][Gm::KLPR];
  __shared__ __align__(16) WaveScratch<BITS, D, QVW> ws[PV_WAVES];
  __shared__ __align__(16) float comb_o[PV_WAVES][QVW][D];
  __shared__ float comb_m[PV_WAVES][QVW], comb_l[PV_WAVES][QVW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int p = blockIdx.x;
  Unit un;
  un.b = blockIdx.z;
  un.hk = blockIdx.y / a.qgroups;
  un.qg = blockIdx.y - un.hk * a.qgroups;
  un.len = clamp_len(a, un.b);
  const int t0 = p * a.part_tokens;
  if (t0 >= un.len) return;                                      // uniform over the workgroup
  const int t1 = min(un.len, t0 + a.part_tokens);
  load_q<BITS, D, QVW>(a, un, q_lds, qs_lds, tid, PV_WAVES * 64);
  __syncthreads();

  Acc<BITS, D, QVW> st;
  acc_init(st);
  run_tiles<BITS, D, QVW>(a, un, t0 + wave * TILE, t1, PV_WAVES * TILE, q_lds, qs_lds, ws[wave], st, lane);
  acc_finish(st);

  const int vsl = lane % VLPR, vrg = lane / VLPR, srow = lane % TILE, spart = lane / TILE;
  if (vrg == 0) {
#pragma unroll
    for (int j = 0; j < QVW; ++j)
#pragma unroll
      for (int d = 0; d < VDPL; ++d) comb_o[wave][j][vsl * VDPL + d] = st.o[j][d];
  }
  if (srow == 0) {
#pragma unroll
    for (int hh = 0; hh < QS; ++hh) {
      const int j = spart * QS + hh;
      if (j < QVW) { comb_m[wave][j] = st.m[hh]; comb_l[wave][j] = st.l[hh]; }
    }
  }
  __syncthreads();

  // combine the waves (log-sum-exp), write this partition's partial
  const int REP = a.HQ / a.HK, N = a.N;
  for (int e = tid; e < QVW * D; e += PV_WAVES * 64) {
    const int j = e / D, d = e - j * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < PV_WAVES; ++w) M = fmaxf(M, comb_m[w][j]);
    float num = 0.0f, den = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < PV_WAVES; ++w) {
        const float mw = comb_m[w][j];
        if (mw == -INFINITY) continue;
        const float f = fast_exp2(mw - M);
        num = fmaf(f, comb_o[w][j][d], num);
        den = fmaf(f, comb_l[w][j], den);
      }
    }
    const int jj = un.qg * QVW + j;
    const int h = un.hk * REP + jj / N, i = jj - (jj / N) * N;
    const int64_t idx = (((int64_t)un.b * a.HQ + h) * N + i) * a.num_parts + p;
    a.opart[idx * D + d] = num;
    if (d == 0) { a.ml[idx * 2] = M; a.ml[idx * 2 + 1] = den; }
  }
}

// ------------------------------------------------------------------- balanced stream

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uni64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off *= 2) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

template <int BITS, int D, int QVW>
__global__ void __launch_bounds__(PV_WAVES * 64, 2)
partial_stream_kernel(PartialArgs a) {
  using Gm = Geo<BITS, D>;
  using Sp = Shape<BITS, D, QVW>;
  constexpr int TILE = Gm::TILE, VDPL = Gm::VDPL, VLPR = Gm::VLPR, QS = Sp::QS;
  __shared__ __align__(16) uint32_t q_lds[PV_WAVES][QVW][D / 2];
  __shared__ float qs_lds[PV_WAVES][QVW][Gm::KLPR];
  __shared__ __align__(16) WaveScratch<BITS, D, QVW> ws[PV_WAVES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = blockIdx.x * PV_WAVES + wave;                    // this wave's worker index
  const int B = a.batch, HQG = a.HK * a.qgroups;

  // total stream length T and the number of working waves (every wave computes the same)
  int64_t tot = 0;
  for (int c = 0; c < B; c += 64) {
    const int bb = c + lane;
    long long s = bb < B ? clamp_len(a, bb) : 0;
#pragma unroll
    for (int off = 32; off >= 1; off /= 2) s += __shfl_xor(s, off, 64);
    tot += s;
  }
  const int64_t T = uni64(tot) * HQG;
  const int64_t weff64 = (T + a.min_tokens - 1) / a.min_tokens;
  const int W_eff = (int)min<int64_t>((int64_t)a.num_waves, weff64);
  if (w >= W_eff) return;                                        // no block-level barriers below
  const int64_t x0 = ((int64_t)w * T + W_eff - 1) / W_eff;
  const int64_t x1 = ((int64_t)(w + 1) * T + W_eff - 1) / W_eff;
  if (x0 >= x1) return;

  // locate the sequence holding stream position x0 (the first with prefix end > x0)
  int b = -1;
  int64_t pb = 0;                                                // tokens of sequences before b
  {
    int64_t base = 0;
    for (int c = 0; c < B; c += 64) {
      const int bb = c + lane;
      const int lv = bb < B ? clamp_len(a, bb) : 0;
      const int incl = wave_incl_scan(lv, lane);
      const uint64_t hit = __ballot((base + incl) * HQG > x0 && lv > 0);
      if (hit) {
        const int k = __builtin_ctzll(hit);
        b = uni(c + k);
        pb = uni64(base + __shfl(incl, k, 64) - __shfl(lv, k, 64));
        break;
      }
      base += uni(__shfl(incl, 63, 64));
    }
  }
  if (b < 0) return;                                             // x0 < T: not reached
  int len = uni(clamp_len(a, b));
  const int64_t rem = x0 - pb * HQG;
  int uu = uni((int)(rem / len));                                // unit within the sequence
  int t_lo = uni((int)(rem - (int64_t)uu * len));

  float* const opart = a.opart;
  float* const ml = a.ml;
  const int vsl = lane % VLPR, vrg = lane / VLPR, srow = lane % TILE, spart = lane / TILE;
  int64_t x = x0;
  while (x < x1) {
    const int seg = (int)min<int64_t>((int64_t)(len - t_lo), x1 - x);
    Unit un;
    un.b = b; un.hk = uu / a.qgroups; un.qg = uu - un.hk * a.qgroups; un.len = len;
    load_q<BITS, D, QVW>(a, un, q_lds[wave], qs_lds[wave], lane, 64);
    wave_lds_sync();
    Acc<BITS, D, QVW> st;
    acc_init(st);
    run_tiles<BITS, D, QVW>(a, un, t_lo, t_lo + seg, TILE, q_lds[wave], qs_lds[wave], ws[wave], st, lane);
    acc_finish(st);
    const int64_t slot = (int64_t)b * HQG + uu + w;
    if (vrg == 0) {
#pragma unroll
      for (int j = 0; j < QVW; ++j)
#pragma unroll
        for (int d = 0; d < VDPL; ++d) opart[(slot * QVW + j) * D + vsl * VDPL + d] = st.o[j][d];
    }
    if (srow == 0) {
#pragma unroll
      for (int hh = 0; hh < QS; ++hh) {
        const int j = spart * QS + hh;
        if (j < QVW) { ml[(slot * QVW + j) * 2] = st.m[hh]; ml[(slot * QVW + j) * 2 + 1] = st.l[hh]; }
      }
    }
    wave_lds_sync();                                             // q_lds is rewritten next
    x += seg;
    t_lo += seg;
    if (t_lo >= len && x < x1) {
      t_lo = 0;
      if (++uu == HQG) {
        uu = 0;
        do { ++b; } while (b < B && clamp_len(a, b) == 0);
        if (b >= B) break;                                       // (x1 <= T: not reached)
        len = uni(clamp_len(a, b));
      }
    }
  }
}

// ------------------------------------------------------------------- launch

template <int BITS, int D, int QVW>
static hipError_t launch_valu(const PartialArgs& a, int B, hipStream_t s) {
  if (a.part_tokens > 0) {
    dim3 grid((unsigned)a.num_parts, (unsigned)(a.HK * a.qgroups), (unsigned)B);
    hipLaunchKernelGGL((partial_part_kernel<BITS, D, QVW>), grid, dim3(PV_WAVES * 64), 0, s, a);
  } else {
    dim3 grid((unsigned)(a.num_waves / PV_WAVES));
    hipLaunchKernelGGL((partial_stream_kernel<BITS, D, QVW>), grid, dim3(PV_WAVES * 64), 0, s, a);
  }
  return hipGetLastError();
}

template <int BITS, int D>
static hipError_t launch_valu_d(const PartialArgs& a, int qvw, int B, hipStream_t s) {
  switch (qvw) {
    case 1: return launch_valu<BITS, D, 1>(a, B, s);
    case 2: return launch_valu<BITS, D, 2>(a, B, s);
    case 4: return launch_valu<BITS, D, 4>(a, B, s);
    case 8:
      if constexpr (BITS != 2) return launch_valu<BITS, D, 8>(a, B, s);   // 2-bit: at most 4
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <int BITS>
static hipError_t launch_valu_b(const PartialArgs& a, int D, int qvw, int B, hipStream_t s) {
  switch (D) {
    case 64: return launch_valu_d<BITS, 64>(a, qvw, B, s);
    case 128: return launch_valu_d<BITS, 128>(a, qvw, B, s);
    case 256: return launch_valu_d<BITS, 256>(a, qvw, B, s);
    default: return hipErrorInvalidValue;
  }
}

bool partial_supported(int bits, int D, int qvw) {
  const bool b = bits == 16 || bits == 8 || bits == 4 || bits == 2;
  const bool d = D == 64 || D == 128 || D == 256;
  const bool q = qvw == 1 || qvw == 2 || qvw == 4 || (qvw == 8 && bits != 2);
  return b && d && q;
}

int tile_tokens(int bits, int D) {
  switch (bits * 1000 + D) {
    case 16064: return Geo<16, 64>::TILE;
    case 16128: return Geo<16, 128>::TILE;
    case 16256: return Geo<16, 256>::TILE;
    case 8064: return Geo<8, 64>::TILE;
    case 8128: return Geo<8, 128>::TILE;
    case 8256: return Geo<8, 256>::TILE;
    case 4064: return Geo<4, 64>::TILE;
    case 4128: return Geo<4, 128>::TILE;
    case 4256: return Geo<4, 256>::TILE;
    case 2064: return Geo<2, 64>::TILE;
    case 2128: return Geo<2, 128>::TILE;
    case 2256: return Geo<2, 256>::TILE;
    default: return 32;
  }
}

hipError_t launch_partial(const PartialArgs& a, int bits, int D, int qvw, int B, hipStream_t s) {
  switch (bits) {
    case 16: return launch_valu_b<16>(a, D, qvw, B, s);
    case 8: return launch_valu_b<8>(a, D, qvw, B, s);
    case 4: return launch_valu_b<4>(a, D, qvw, B, s);
    case 2: return launch_valu_b<2>(a, D, qvw, B, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
