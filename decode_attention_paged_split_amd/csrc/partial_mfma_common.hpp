// Split-K partial kernel of paged decode attention, matrix-core engine (4-bit affine pages,
// head dim 128 or 256), on the balanced stream schedule.
//
// Same computation as the vector-ALU engine (partial_valu.hip), after
// "@mlx-bun/inference 0.0.0-stage -> 1.0.0", diff page 50: paged.ts (paged_attention_partial,
// paged_attention_affine_partial) and kvq4-decode.ts (the partial kernel: one read of a K/V row
// for every query head of its GQA group; online softmax in f32; a partial (o, m, l) per range).
// The pages' own few-row variant (multi-query.ts, mlx_bun_attn_multi_query_partial) puts the
// REP x rows query vectors of a KV head on the simdgroup matrix unit; this is that idea on
// gfx950's MFMA, for the GQA groups where the vector ALU, not HBM, bounds the partial kernel.
//
// Two kernels.  At head dim 128 a wave owns 16 query vectors (the MFMA N dimension; unused ones
// are zero) and walks 64-token tiles alone, two waves per SIMD.  At head dim 256 a workgroup of
// two waves shares each tile, one per half of the head dim (partial_mfma_split_kernel, below).
// Both:
//  * q.k: v_mfma_f32_16x16x32_bf16 with A = a 16-token block of K rows and B = q^T.  Codes
//    become bf16(128 + c) with one v_and_or (exact) and q is exact in bf16, so every product is
//    exact; each MFMA step covers 32 dims of one 64-dim scale group, so the group's scale and
//    bias apply once per (token, group): z = s * acc + (b - 128 s) * sum_g(q).  A lane loads 16
//    contiguous bytes of its row and four v_permlane{32,16}_swap turn four lanes' chunks into
//    the word each lane's k-slot needs.
//  * softmax: the MFMA result gives every lane one query vector (lane % 16) and four tokens per
//    16-token block, so the running max, normaliser and per-group sums are per-lane scalars; the
//    tile max needs two lane swaps.  The running max moves only when a score exceeds it by more
//    than 2^8, so the accumulators are rescaled only then.
//  * P.V: v_mfma_f32_16x16x32_f16 with A = V^T and B = (p * scale)^T.  V^T comes straight from
//    the raw 4-bit tile in LDS through ds_read_b64_tr_b4 (a 16 x 16 nibble transpose per 16
//    lanes); its codes enter as f16 subnormals (bits c = value c * 2^-24, exact, one AND per
//    pair) and the accumulators are scaled by 2^24 at the end.  The weight w = p * s(token, group),
//    prescaled by a power of two per group (mf_vpre_update), is split into f16 hi + lo (rounded
//    to nearest), two MFMAs per step, so the product is accurate to ~2^-22 relative whatever the
//    V scale; the bias term sum_t p * b is accumulated per (vector, group) in f32 and added at
//    the end.
//  * loads: the K rows, V rows and scales of tile i + 1 are in flight while tile i is computed.

//
// This header holds what the three kernels share (fragment helpers, the stream's range lookup,
// the two-wave layout of head dim 256); each kernel has a translation unit of its own:
// partial_mfma.hip (head dim 128, and the launcher), partial_mfma_split.hip, partial_mfma_pair.hip.
#pragma once

#include "device_common.hpp"
#include "kernels.hpp"

namespace kvq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int MF_WAVES = 2;     // independent waves per workgroup (keeps a block's LDS under 64 KB)
constexpr int MF_TILE = 64;     // tokens per tile
constexpr int MF_QV = 16;       // query vectors per wave (MFMA N)

template <int D>
struct MGeo {
  static constexpr int ROWB = D / 2;             // bytes per 4-bit row
  static constexpr int KSTEPS = D / 32;          // q.k MFMA steps (32 dims each)
  static constexpr int CPR = ROWB / 16;          // 16-byte chunks per row
  static constexpr int KSETS = KSTEPS / 4;       // 16-byte loads per lane per 16-token block
  static constexpr int G = D / 64;               // scale groups per row
  static constexpr int DT = D / 16;              // P.V dim tiles
  static constexpr int PITCH = ROWB + 16;        // LDS row pitch of the raw V tile (no bank clash)
  static constexpr int NVL = MF_TILE * CPR / 64; // V 16-byte loads per lane per tile
  static_assert(D == 128, "head dim (256 runs the split kernel)");
};

template <int D>
struct MScratch {
  using Mg = MGeo<D>;
  uint8_t v[MF_TILE][Mg::PITCH];                 // raw V codes of the tile
  uint8_t k[MF_TILE][Mg::PITCH];                 // raw K codes of the tile
  float2 ksb[MF_TILE][Mg::G];                    // K (scale, bias - 128 scale)
  float vs[Mg::G][MF_TILE];                      // V scale
  float vb[Mg::G][MF_TILE];                      // V bias
  float pt[MF_QV][MF_TILE];                      // probabilities [vector][token]
};

// The constants of the K-code unpack, (x & m) | o with m = 0x000F000F in an SGPR and
// o = bf16 128 in both halves in a VGPR.  The unpack itself is plain C, so that the compiler sees
// each VALU write that feeds an MFMA operand and keeps the wait states between them (an inline-asm
// v_and_or_b32 once let an MFMA read its operand registers before those writes had landed); the
// constants come out of asm only so that the compiler cannot fold them into an AND and an OR
// (VOP3 takes no literal on this target) and forms one v_and_or_b32 per pair.
struct KUnpack {
  uint32_t m, o;
};
__device__ __forceinline__ KUnpack k_unpack_consts() {
  KUnpack k;
  asm volatile("s_mov_b32 %0, 0x000F000F" : "=s"(k.m));
  asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(k.o));
  return k;
}

__device__ __forceinline__ void mf_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// a 4-bit word -> 8 bf16 (128 + c) in pair order (n0,n4),(n1,n5),(n2,n6),(n3,n7)
__device__ __forceinline__ bf16x8 k_frag(uint32_t w, const KUnpack& ku) {
  uint4 r;
  r.x = (w & ku.m) | ku.o;
  r.y = ((w >> 4) & ku.m) | ku.o;
  r.z = ((w >> 8) & ku.m) | ku.o;
  r.w = ((w >> 12) & ku.m) | ku.o;
  return __builtin_bit_cast(bf16x8, r);
}

// a 4-bit word -> 8 f16 subnormals (c * 2^-24) in pair order (n0,n4),(n1,n5),(n2,n6),(n3,n7)
__device__ __forceinline__ f16x8 v_frag_sub(uint32_t w) {
  uint4 r;
  r.x = w & 0x000F000Fu;
  r.y = (w >> 4) & 0x000F000Fu;
  r.z = (w >> 8) & 0x000F000Fu;
  r.w = (w >> 12) & 0x000F000Fu;
  return __builtin_bit_cast(f16x8, r);
}

// f32 pair -> packed f16 pair, each rounded to nearest (v_cvt_pk_f16_f32)
__device__ __forceinline__ f16x2 pk_f16(float a, float b) { return f16x2{(_Float16)a, (_Float16)b}; }

// The f16 hi + lo split of two weights: hi = w rounded to nearest, lo = (w - hi) rounded to nearest,
// so the pair carries ~22 bits and the rounding errors of many small weights do not pile up on
// one side.
__device__ __forceinline__ void split_f16(float w0, float w1, uint32_t& hi, uint32_t& lo) {
  const f16x2 h2 = pk_f16(w0, w1);
  hi = __builtin_bit_cast(uint32_t, h2);
  lo = __builtin_bit_cast(uint32_t, pk_f16(w0 - (float)h2[0], w1 - (float)h2[1]));
}

// Power-of-two prescale of the P.V weights before their f16 split, per V scale group: the weights
// enter as w * 2^-E, E the group's exponent, so that the largest sit near 2^14 whatever the V scale
// (hi and lo then both stay normal and keep ~22 bits, and hi never overflows: a tile's V scales stay
// below 2^(E+7) and p <= 2^8 with the lazy running max, so w * 2^-E < 2^15).  E starts unset, is
// taken from the first tile's largest scale and only grows: when a tile's scale passes 2^(E+7) the
// group's accumulators are multiplied by 2^(E_old - E_new), exactly, and E moves.  The output
// takes the factor 2^E back at the end, exactly.
constexpr int MF_VE_NONE = -1000;

__device__ __forceinline__ float mf_pow2(int k) { return __int_as_float(max(k + 127, 1) << 23); }

// whether this lane's V scale s needs the group's prescale to move (E unset, or s > 2^(E+7))
__device__ __forceinline__ bool mf_vpre_moves(float s, int e) {
  return e == MF_VE_NONE || s > mf_pow2(e + 7);
}

// the whole wave: move the group's exponent e to cover every lane's scale s; returns the factor
// (<= 1) by which the group's accumulators must be multiplied
__device__ __forceinline__ float mf_vpre_update(float s, int& e) {
  const float smax = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
      __builtin_bit_cast(int, block_reduce<OpMax, 1, 64>(s))));
  if (e != MF_VE_NONE && smax <= mf_pow2(e + 7)) return 1.0f;
  // smax < 2^f, f its frexp exponent: with E = f - 7, smax * 2^-E < 2^7
  const int en = max(__builtin_amdgcn_readfirstlane(__builtin_amdgcn_frexp_expf(smax)) - 7, -100);
  const float r = (e == MF_VE_NONE) ? 1.0f : mf_pow2(e - en);
  e = en;
  return r;
}

// 4 x 4 transpose of dwords across the four 16-lane rows of a wave: on entry register j of row
// s holds element (s, j); on return register j of row s holds element (j, s).
__device__ __forceinline__ void transpose4(uint32_t& r0, uint32_t& r1, uint32_t& r2, uint32_t& r3) {
  auto a = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);
  auto b = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  r0 = c[0]; r1 = c[1]; r2 = d[0]; r3 = d[1];
}

__device__ __forceinline__ int mf_uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t mf_uni64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int mf_len(const PartialArgs& a, int b) {
  return max(0, min(a.lengths[b], a.len_cap));
}

// The raw loads of one 64-token tile, in registers: V as 16-byte chunks (lane i of load j holds
// chunk (64 j + i) % CPR of row (64 j + i) / CPR), K for the four 16-row MFMA blocks (lane (qv, ks)
// holds chunks ks, ks + 4, ... of row 16 mt + qv), and the four scale planes of row `lane`.
template <int D>
struct MTileRegs {
  using Mg = MGeo<D>;
  u32x4 v[Mg::NVL];
  u32x4 k[4][Mg::KSETS];
  uint32_t ks[Mg::G / 2], kb[Mg::G / 2], vs[Mg::G / 2], vb[Mg::G / 2];
};

template <int NW>
__device__ __forceinline__ void mf_load_words(uint32_t (&w)[NW], const uint16_t* p) {
  if constexpr (NW == 2) {
    const uint2 t = *reinterpret_cast<const uint2*>(p);
    w[0] = t.x; w[1] = t.y;
  } else {
    static_assert(NW == 1, "scale groups per row");
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  }
}

template <int NW>
__device__ __forceinline__ float mf_bf16(const uint32_t (&w)[NW], int g) {
  return (g & 1) ? bf16_hi(w[g >> 1]) : bf16_lo(w[g >> 1]);
}

// Issue the loads of the tile whose row `lane` sits at pool row my_row (rows of other lanes come
// by lane shuffle).  Nothing waits on them here.
template <int D>
__device__ __forceinline__ void mf_issue(MTileRegs<D>& t, const PartialArgs& a, int my_row, int lane) {
  using Mg = MGeo<D>;
  const char* kplane = static_cast<const char*>(a.k);
  const char* vplane = static_cast<const char*>(a.v);
  const int qv = lane & 15, ks = lane >> 4;
  constexpr int RPL = 64 / Mg::CPR;                  // V rows per load instruction
  const int vr = lane / Mg::CPR, ch = lane % Mg::CPR; // lane's row within the load, its chunk
#pragma unroll
  for (int i = 0; i < Mg::NVL; ++i) {
    const int64_t row = __builtin_amdgcn_ds_bpermute(4 * vr + 4 * RPL * i, my_row);
    t.v[i] = *reinterpret_cast<const u32x4*>(vplane + row * Mg::ROWB + 16 * ch);
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int64_t row = __builtin_amdgcn_ds_bpermute(4 * qv + 64 * mt, my_row);
    const char* src = kplane + row * Mg::ROWB;
#pragma unroll
    for (int c = 0; c < Mg::KSETS; ++c) t.k[mt][c] = *reinterpret_cast<const u32x4*>(src + 16 * (4 * c + ks));
  }
  const int64_t ri = (int64_t)my_row * Mg::G;
  mf_load_words(t.ks, a.ks + ri);
  mf_load_words(t.kb, a.kb + ri);
  mf_load_words(t.vs, a.vs + ri);
  mf_load_words(t.vb, a.vb + ri);
}

// A range [x0, x1) of the flattened (sequence, query group unit, token) stream and where it
// starts: sequence b (length len), unit uu, token t_lo.  All values are wave-uniform.
struct MfRange {
  int64_t x0, x1;
  int b, len, uu, t_lo;
};

// Range `w` of the stream split into at most num_ranges equal ranges of at least min_tokens
// tokens; false if range w is empty.  HQG: stream units per sequence (KV heads x query groups, or
// x sets of `lanes` groups where those run side by side); r.uu is the unit (or set) index.
__device__ __forceinline__ bool mf_find_range(const PartialArgs& a, int w, int lane, MfRange& r, int HQG) {
  const int B = a.batch;
  int64_t tot = 0;
  for (int c = 0; c < B; c += 64) {
    const int bb = c + lane;
    long long s = bb < B ? mf_len(a, bb) : 0;
#pragma unroll
    for (int off = 32; off >= 1; off /= 2) s += __shfl_xor(s, off, 64);
    tot += s;
  }
  const int64_t T = mf_uni64(tot) * HQG;
  const int W_eff = (int)min<int64_t>((int64_t)a.num_ranges, (T + a.min_tokens - 1) / a.min_tokens);
  if (w >= W_eff) return false;
  r.x0 = ((int64_t)w * T + W_eff - 1) / W_eff;
  r.x1 = ((int64_t)(w + 1) * T + W_eff - 1) / W_eff;
  if (r.x0 >= r.x1) return false;
  int b = -1;
  int64_t pb = 0;
  int64_t base = 0;
  for (int c = 0; c < B; c += 64) {
    const int bb = c + lane;
    const int lv = bb < B ? mf_len(a, bb) : 0;
    int incl = lv;
#pragma unroll
    for (int off = 1; off < 64; off *= 2) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    const uint64_t hit = __ballot((base + incl) * HQG > r.x0 && lv > 0);
    if (hit) {
      const int k = __builtin_ctzll(hit);
      b = mf_uni(c + k);
      pb = mf_uni64(base + __shfl(incl, k, 64) - __shfl(lv, k, 64));
      break;
    }
    base += mf_uni(__shfl(incl, 63, 64));
  }
  if (b < 0) return false;
  r.b = b;
  r.len = mf_uni(mf_len(a, b));
  const int64_t rem = r.x0 - pb * HQG;
  r.uu = mf_uni((int)(rem / r.len));
  r.t_lo = mf_uni((int)(rem - (int64_t)r.uu * r.len));
  return true;
}

// max / sum over the four lanes that share a query vector (lane, lane ^ 16, ^ 32, ^ 48)
__device__ __forceinline__ float qv_max(float x) { return block_reduce<OpMax, 16, 64>(x); }
__device__ __forceinline__ float qv_sum(float x) { return block_reduce<OpAdd, 16, 64>(x); }

// ---------------------------------------------------------------------------------------------
// Head dim 256: a workgroup of two waves shares each tile, wave h owning dims [128 h, 128 h + 128)
// (scale groups 2h and 2h + 1) in both products, so each wave holds half of q, of the output
// accumulators and of the tile's K/V bytes, and two waves fit one SIMD.  Each wave's q.k covers
// its dims only; the two partial scores meet in LDS (one workgroup barrier per tile) and both
// waves run the same softmax on z0 + z1, so they hold identical probabilities.
//  * P.V takes its weights from registers: the tile's V rows sit in LDS in the order the score
//    layout gives each lane (token 16 mt + 4 ks + i at LDS row 16 ks + 4 mt + i), so the
//    transposing read hands k-slot ks exactly the eight tokens whose probabilities it holds.
//  * V codes enter the f16 MFMA as subnormals (bits c = value c * 2^-24, exact), one AND per
//    pair; the accumulators are scaled by 2^24 at the end.
constexpr int SP_HD = 128;                        // dims per wave
constexpr int SP_HB = SP_HD / 2;                  // bytes per half row (4-bit codes)
constexpr int SP_VPITCH = SP_HB + 16;             // LDS pitch of a V half row (no bank clash)
constexpr int SP_G = SP_HD / 64;                  // scale groups per wave
constexpr int SP_DT = SP_HD / 16;                 // P.V dim tiles per wave

struct SpWave {
  uint8_t v[MF_TILE][SP_VPITCH];                  // V half rows, permuted token order
  float ksb[MF_TILE][2 * SP_G];                   // per token: (K scale, K bias - 128 scale) x group
  float vs[SP_G][MF_TILE];                        // V scale
  float vb[SP_G][MF_TILE];                        // V bias
};

struct SpShared {
  SpWave w[2];
  float4 zx[2][2][4][64];                         // partial scores [buffer][wave][16-token block][lane]
};

// The raw loads of one tile for one wave: K half rows of the four 16-row blocks (lane (m, ks):
// chunk ks of row 16 mt + m), V half rows (load i, lane L: chunk L % 4 of row 16 i + L / 4) and
// the wave's two groups of the four scale planes for row `lane`.
struct SpTileRegs {
  u32x4 k[4];
  u32x4 v[4];
  uint32_t ks, kb, vs, vb;
};

__device__ __forceinline__ void sp_issue(SpTileRegs& t, const PartialArgs& a, int my_row, int lane, int h) {
  const char* kplane = static_cast<const char*>(a.k) + SP_HB * h;
  const char* vplane = static_cast<const char*>(a.v) + SP_HB * h;
  const int m = lane & 15, ks = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = __builtin_amdgcn_ds_bpermute(4 * (lane >> 2) + 64 * i, my_row);
    t.v[i] = *reinterpret_cast<const u32x4*>(vplane + row * (2 * SP_HB) + 16 * (lane & 3));
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int64_t row = __builtin_amdgcn_ds_bpermute(4 * m + 64 * mt, my_row);
    t.k[mt] = *reinterpret_cast<const u32x4*>(kplane + row * (2 * SP_HB) + 16 * ks);
  }
  const int64_t ri = (int64_t)my_row * (2 * SP_G) + SP_G * h;      // bf16 index of group 2h
  t.ks = *reinterpret_cast<const uint32_t*>(a.ks + ri);
  t.kb = *reinterpret_cast<const uint32_t*>(a.kb + ri);
  t.vs = *reinterpret_cast<const uint32_t*>(a.vs + ri);
  t.vb = *reinterpret_cast<const uint32_t*>(a.vb + ri);
}

// launchers of the head-dim-256 kernels (one translation unit each)
hipError_t launch_mfma_split(const PartialArgs& a, hipStream_t s);
hipError_t launch_mfma_pair(const PartialArgs& a, hipStream_t s);

}  // namespace kvq
