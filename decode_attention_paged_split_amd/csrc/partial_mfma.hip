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
//    pair) and the accumulators are scaled by 2^24 at the end.  The weight w = p * s(token, group) is split into f16 hi + lo (rounded to nearest),
//    two MFMAs per step, so the product is accurate to ~2^-22 relative; the bias term
//    sum_t p * b is accumulated per (vector, group) in f32 and added at the end.
//  * loads: the K rows, V rows and scales of tile i + 1 are in flight while tile i is computed.

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
// tokens; false if range w is empty.
__device__ __forceinline__ bool mf_find_range(const PartialArgs& a, int w, int lane, MfRange& r) {
  const int B = a.batch, HQG = a.HK * a.qgroups;
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

template <int D>
__global__ void __launch_bounds__(MF_WAVES * 64, 1)
partial_mfma_kernel(PartialArgs a) {
  const KUnpack ku = k_unpack_consts();
  using Mg = MGeo<D>;
  constexpr int G = Mg::G, KSTEPS = Mg::KSTEPS, KSETS = Mg::KSETS, DT = Mg::DT;
  constexpr int CPR = Mg::CPR, NVL = Mg::NVL;
  __shared__ __align__(16) MScratch<D> scr[MF_WAVES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = blockIdx.x * MF_WAVES + wave;
  MScratch<D>& S = scr[wave];
  const int B = a.batch, HQG = a.HK * a.qgroups;
  const int qv = lane & 15, ks = lane >> 4;       // query vector (MFMA n / m%16), k-slot (lane / 16)

  MfRange rg;
  if (!mf_find_range(a, w, lane, rg)) return;      // no block-level barriers in this kernel
  int b = rg.b, len = rg.len, uu = rg.uu, t_lo = rg.t_lo;
  const int64_t x0 = rg.x0, x1 = rg.x1;

  const int REP = a.HQ / a.HK, N = a.N;
  const int QV_total = REP * N;

  int64_t x = x0;
  while (x < x1) {
    const int seg = (int)min<int64_t>((int64_t)(len - t_lo), x1 - x);
    const int t1 = t_lo + seg;
    const int hk = uu / a.qgroups, qg = uu - hk * a.qgroups;
    const int32_t* trow = a.table + (int64_t)b * a.max_blocks;

    // ---- q^T fragments of this lane's query vector (zero for padding vectors)
    const int jj = qg * MF_QV + qv;
    const bool qreal = jj < QV_total;
    const int h = hk * REP + (qreal ? jj / N : 0), qi = qreal ? jj - (jj / N) * N : 0;
    const uint16_t* qrow = a.q + (((int64_t)b * a.HQ + h) * N + qi) * D;
    bf16x8 qf[KSTEPS];
    float qsum[G];
#pragma unroll
    for (int g = 0; g < G; ++g) qsum[g] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      // dims of word 4 kk + ks: 8 (4 kk + ks) .. + 8, in pair order (0,4),(1,5),(2,6),(3,7)
      uint4 d = qreal ? *reinterpret_cast<const uint4*>(qrow + 8 * (4 * kk + ks)) : make_uint4(0, 0, 0, 0);
      uint4 r;
      r.x = __builtin_amdgcn_perm(d.z, d.x, 0x05040100u);
      r.y = __builtin_amdgcn_perm(d.z, d.x, 0x07060302u);
      r.z = __builtin_amdgcn_perm(d.w, d.y, 0x05040100u);
      r.w = __builtin_amdgcn_perm(d.w, d.y, 0x07060302u);
      qf[kk] = __builtin_bit_cast(bf16x8, r);
      const float s8 = bf16_lo(d.x) + bf16_hi(d.x) + bf16_lo(d.y) + bf16_hi(d.y) + bf16_lo(d.z) + bf16_hi(d.z) +
                       bf16_lo(d.w) + bf16_hi(d.w);
      qsum[kk / 2] += s8;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) qsum[g] = qv_sum(qsum[g]);   // the four k-slots of the vector
    const int vend = qreal ? len - N + qi + 1 : 0;

    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m = -INFINITY, l = 0.0f, pbias[G];
#pragma unroll
    for (int g = 0; g < G; ++g) pbias[g] = 0.0f;

    // ---- tile pipeline: while tile i is computed, the K rows, V rows and scales of tile i + 1
    // are in flight, and the block-table entries of tile i + 2 one step earlier still.  Lane r
    // owns tile row r (the segment's last row stands in for rows past its end).
    auto tab_idx = [&](int tstart) -> int {          // logical block of this lane's tile row
      const int t = min(tstart + lane, t1 - 1);
      return (a.bs_shift >= 0) ? (t >> a.bs_shift) : (t / a.BS);
    };
    auto row_of = [&](int tstart, int phys) -> int {  // pool row of this lane's tile row
      const int t = min(tstart + lane, t1 - 1);
      const int blk = (a.bs_shift >= 0) ? (t >> a.bs_shift) : (t / a.BS);
      phys = min(max(phys, 0), a.num_blocks - 1);
      return (phys * a.HK + hk) * a.BS + (t - blk * a.BS);
    };
    MTileRegs<D> cur;
    int ph_next = 0;
    if (t_lo < t1) {
      mf_issue<D>(cur, a, row_of(t_lo, trow[tab_idx(t_lo)]), lane);
      if (t_lo + MF_TILE < t1) ph_next = trow[tab_idx(t_lo + MF_TILE)];
    }

    for (int tt = t_lo; tt < t1; tt += MF_TILE) {
      // ---- this tile's K and V codes and its scales into LDS (K in the lane layout of the q.k step)
#pragma unroll
      for (int i = 0; i < NVL; ++i)
        *reinterpret_cast<u32x4*>(&S.v[(64 / CPR) * i + lane / CPR][16 * (lane % CPR)]) = cur.v[i];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float ksc = mf_bf16(cur.ks, g), kbi = mf_bf16(cur.kb, g);
        S.ksb[lane][g] = make_float2(ksc, fmaf(-128.0f, ksc, kbi));
        S.vs[g][lane] = mf_bf16(cur.vs, g);
        S.vb[g][lane] = mf_bf16(cur.vb, g);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int c = 0; c < KSETS; ++c)
          *reinterpret_cast<u32x4*>(&S.k[16 * mt + qv][16 * (4 * c + ks)]) = cur.k[mt][c];
      if (tt + MF_TILE < t1) {                        // wave-uniform
        mf_issue<D>(cur, a, row_of(tt + MF_TILE, ph_next), lane);
        if (tt + 2 * MF_TILE < t1) ph_next = trow[tab_idx(tt + 2 * MF_TILE)];
      }
      mf_lds_sync();
      __builtin_amdgcn_sched_barrier(0);

      // ---- q.k on the matrix cores, then per-group scale and bias
      float z[4][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        uint32_t kw[KSTEPS];
#pragma unroll
        for (int c = 0; c < KSETS; ++c) {
          const u32x4 kq = *reinterpret_cast<const u32x4*>(&S.k[16 * mt + qv][16 * (4 * c + ks)]);
          uint32_t r0 = kq.x, r1 = kq.y, r2 = kq.z, r3 = kq.w;
          transpose4(r0, r1, r2, r3);                   // register j = word 4 (4c + j) + ks
          kw[4 * c + 0] = r0; kw[4 * c + 1] = r1; kw[4 * c + 2] = r2; kw[4 * c + 3] = r3;
        }
        f32x4 acc[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          acc[g] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_frag(kw[2 * g], ku), qf[2 * g], acc[g], 0, 0, 0);
          acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_frag(kw[2 * g + 1], ku), qf[2 * g + 1], acc[g], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * mt + 4 * ks + i;             // token row of this accumulator entry
          float zz = 0.0f;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float2 sb = S.ksb[r][g];
            zz = fmaf(sb.x, acc[g][i], fmaf(sb.y, qsum[g], zz));
          }
          z[mt][i] = zz;
        }
        __builtin_amdgcn_sched_barrier(0);
      }

      // ---- online softmax for this lane's query vector
      float mt_ = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = tt + 16 * mt + 4 * ks + i;
          float zz = z[mt][i] * a.scale_log2e;
          if (tok >= t1 || tok >= vend) zz = -INFINITY;
          z[mt][i] = zz;
          mt_ = fmaxf(mt_, zz);
        }
      mt_ = qv_max(mt_);
      // the running max moves only when a score exceeds it by more than 2^8 (p <= 256), so the
      // rescale of the accumulators runs only then (wave-uniform branch)
      if (__ballot(mt_ > m + 8.0f)) {
        asm volatile("; running max moves");                      // keeps this a real branch
        const float mnew = (mt_ > m + 8.0f) ? mt_ : m;
        const float alpha = (mnew == -INFINITY) ? 1.0f : fast_exp2(m - mnew);
        m = mnew;
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
#pragma unroll
        for (int g = 0; g < G; ++g) pbias[g] *= alpha;
      }
      const float muse = (m == -INFINITY) ? 0.0f : m;
      float ls = 0.0f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        float4 pv;
        pv.x = fast_exp2(z[mt][0] - muse); pv.y = fast_exp2(z[mt][1] - muse);
        pv.z = fast_exp2(z[mt][2] - muse); pv.w = fast_exp2(z[mt][3] - muse);
        ls += (pv.x + pv.y) + (pv.z + pv.w);
        *reinterpret_cast<float4*>(&S.pt[qv][16 * mt + 4 * ks]) = pv;
      }
      l += ls;
      mf_lds_sync();
      __builtin_amdgcn_sched_barrier(0);

      // ---- P.V on the matrix cores: per scale group, B = (p * s)^T split f16 hi + lo
#pragma unroll
      for (int g = 0; g < G; ++g) {
        f16x8 bhi[2], blo[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int t0 = 16 * ks + 8 * st;              // this k-slot's 8 tokens of step st
          const float4 p0 = *reinterpret_cast<const float4*>(&S.pt[qv][t0]);
          const float4 p1 = *reinterpret_cast<const float4*>(&S.pt[qv][t0 + 4]);
          const float4 s0 = *reinterpret_cast<const float4*>(&S.vs[g][t0]);
          const float4 s1 = *reinterpret_cast<const float4*>(&S.vs[g][t0 + 4]);
          const float4 b0 = *reinterpret_cast<const float4*>(&S.vb[g][t0]);
          const float4 b1 = *reinterpret_cast<const float4*>(&S.vb[g][t0 + 4]);
          const float pp[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
          const float ss[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
          const float bq[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
          float pbs = 0.0f;
          uint32_t hi[4], lo[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {                 // pair (token k, token k + 4)
            const float w0 = pp[k] * ss[k], w1 = pp[k + 4] * ss[k + 4];
            split_f16(w0, w1, hi[k], lo[k]);
            pbs = fmaf(pp[k], bq[k], fmaf(pp[k + 4], bq[k + 4], pbs));
          }
          pbias[g] += pbs;
          bhi[st] = __builtin_bit_cast(f16x8, make_uint4(hi[0], hi[1], hi[2], hi[3]));
          blo[st] = __builtin_bit_cast(f16x8, make_uint4(lo[0], lo[1], lo[2], lo[3]));
        }
#pragma unroll
        for (int dq = 0; dq < DT / G; ++dq) {
          const int dt = g * (DT / G) + dq;              // 16-dim tile inside group g
          // lane r of each 16-lane row points at tile row 16 * ks + r, dims 16 dt .. 16 dt + 15
          const i32x2 tw = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
              (__attribute__((address_space(3))) i32x2*)(&S.v[lane][8 * dt]));
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const f16x8 af = v_frag_sub((uint32_t)tw[st]);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bhi[st], o[dt], 0, 0, 0);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, blo[st], o[dt], 0, 0, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      mf_lds_sync();                                   // the tile's LDS is rewritten next
    }

    // ---- segment end: normaliser and bias sums over the four k-slots, write the partial
    l = qv_sum(l);
#pragma unroll
    for (int g = 0; g < G; ++g) pbias[g] = qv_sum(pbias[g]);
    const int64_t slot = (int64_t)b * HQG + uu + w;
    if (qreal) {
      float* orow = a.opart + (slot * MF_QV + qv) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const float pbv = pbias[dt / (DT / G)];
        constexpr float two24 = 16777216.0f;        // the V codes entered as c * 2^-24
        const float4 v4 = make_float4(fmaf(o[dt][0], two24, pbv), fmaf(o[dt][1], two24, pbv),
                                      fmaf(o[dt][2], two24, pbv), fmaf(o[dt][3], two24, pbv));
        *reinterpret_cast<float4*>(orow + 16 * dt + 4 * ks) = v4;
      }
      if (ks == 0) {
        a.ml[(slot * MF_QV + qv) * 2] = m;
        a.ml[(slot * MF_QV + qv) * 2 + 1] = l;
      }
    }

    x += seg;
    t_lo += seg;
    if (t_lo >= len && x < x1) {
      t_lo = 0;
      if (++uu == HQG) {
        uu = 0;
        do { ++b; } while (b < B && mf_len(a, b) == 0);
        if (b >= B) break;
        len = mf_uni(mf_len(a, b));
      }
    }
  }
}

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

__global__ void __launch_bounds__(128, 2)
partial_mfma_split_kernel(PartialArgs a) {
  const KUnpack ku = k_unpack_consts();
  constexpr int D = 256;
  __shared__ __align__(16) SpShared sh;

  const int lane = threadIdx.x & 63;
  const int h = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // dim half of this wave
  const int w = blockIdx.x;                                         // range (whole workgroup)
  SpWave& S = sh.w[h];
  const int B = a.batch, HQG = a.HK * a.qgroups;
  const int qv = lane & 15, ks = lane >> 4;

  MfRange rg;
  if (!mf_find_range(a, w, lane, rg)) return;     // the same for both waves: no barrier is left
  int b = rg.b, len = rg.len, uu = rg.uu, t_lo = rg.t_lo;
  const int64_t x1 = rg.x1;
  const int REP = a.HQ / a.HK, N = a.N;
  const int QV_total = REP * N;
  int zbuf = 0;

  int64_t x = rg.x0;
  while (x < x1) {
    const int seg = (int)min<int64_t>((int64_t)(len - t_lo), x1 - x);
    const int t1 = t_lo + seg;
    const int hk = uu / a.qgroups, qg = uu - hk * a.qgroups;
    const int32_t* trow = a.table + (int64_t)b * a.max_blocks;

    // ---- q^T fragments of this lane's query vector over the wave's dims (zero for padding)
    const int jj = qg * MF_QV + qv;
    const bool qreal = jj < QV_total;
    const int hq = hk * REP + (qreal ? jj / N : 0), qi = qreal ? jj - (jj / N) * N : 0;
    const uint16_t* qrow = a.q + (((int64_t)b * a.HQ + hq) * N + qi) * D + SP_HD * h;
    bf16x8 qf[4];
    float qsum[SP_G] = {0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint4 d = qreal ? *reinterpret_cast<const uint4*>(qrow + 8 * (4 * kk + ks)) : make_uint4(0, 0, 0, 0);
      uint4 r;
      r.x = __builtin_amdgcn_perm(d.z, d.x, 0x05040100u);
      r.y = __builtin_amdgcn_perm(d.z, d.x, 0x07060302u);
      r.z = __builtin_amdgcn_perm(d.w, d.y, 0x05040100u);
      r.w = __builtin_amdgcn_perm(d.w, d.y, 0x07060302u);
      qf[kk] = __builtin_bit_cast(bf16x8, r);
      qsum[kk / 2] += bf16_lo(d.x) + bf16_hi(d.x) + bf16_lo(d.y) + bf16_hi(d.y) + bf16_lo(d.z) + bf16_hi(d.z) +
                      bf16_lo(d.w) + bf16_hi(d.w);
    }
#pragma unroll
    for (int g = 0; g < SP_G; ++g) qsum[g] = qv_sum(qsum[g]);
    const int vend = qreal ? len - N + qi + 1 : 0;

    f32x4 o[SP_DT];
#pragma unroll
    for (int dt = 0; dt < SP_DT; ++dt) o[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m = -INFINITY, l = 0.0f, pbias[SP_G] = {0.0f, 0.0f};

    // ---- tile pipeline as in the single-wave kernel: tile i + 1's loads in flight during tile i
    auto tab_idx = [&](int tstart) -> int {
      const int t = min(tstart + lane, t1 - 1);
      return (a.bs_shift >= 0) ? (t >> a.bs_shift) : (t / a.BS);
    };
    auto row_of = [&](int tstart, int phys) -> int {
      const int t = min(tstart + lane, t1 - 1);
      const int blk = (a.bs_shift >= 0) ? (t >> a.bs_shift) : (t / a.BS);
      phys = min(max(phys, 0), a.num_blocks - 1);
      return (phys * a.HK + hk) * a.BS + (t - blk * a.BS);
    };
    SpTileRegs cur;
    int ph_next = 0;
    if (t_lo < t1) {
      sp_issue(cur, a, row_of(t_lo, trow[tab_idx(t_lo)]), lane, h);
      if (t_lo + MF_TILE < t1) ph_next = trow[tab_idx(t_lo + MF_TILE)];
    }

    for (int tt = t_lo; tt < t1; tt += MF_TILE) {
      // ---- V half rows (permuted) and the scales into this wave's LDS; K stays in registers
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * i + (lane >> 2);       // tile row: token 16 mt + 4 ks' + i' ...
        const int pr = 16 * ((r >> 2) & 3) + 4 * (r >> 4) + (r & 3);   // ... sits at row 16 ks' + 4 mt + i'
        *reinterpret_cast<u32x4*>(&S.v[pr][16 * (lane & 3)]) = cur.v[i];
      }
      {
        const float ks0 = bf16_lo(cur.ks), ks1 = bf16_hi(cur.ks);
        *reinterpret_cast<float4*>(&S.ksb[lane][0]) =
            make_float4(ks0, fmaf(-128.0f, ks0, bf16_lo(cur.kb)), ks1, fmaf(-128.0f, ks1, bf16_hi(cur.kb)));
        S.vs[0][lane] = bf16_lo(cur.vs);
        S.vs[1][lane] = bf16_hi(cur.vs);
        S.vb[0][lane] = bf16_lo(cur.vb);
        S.vb[1][lane] = bf16_hi(cur.vb);
      }
      u32x4 kc[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) kc[mt] = cur.k[mt];
      if (tt + MF_TILE < t1) {                    // the same for both waves
        sp_issue(cur, a, row_of(tt + MF_TILE, ph_next), lane, h);
        if (tt + 2 * MF_TILE < t1) ph_next = trow[tab_idx(tt + 2 * MF_TILE)];
      }
      mf_lds_sync();
      __builtin_amdgcn_sched_barrier(0);

      // ---- q.k over this wave's dims, then its groups' scale and bias
      float z[4][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        uint32_t r0 = kc[mt].x, r1 = kc[mt].y, r2 = kc[mt].z, r3 = kc[mt].w;
        transpose4(r0, r1, r2, r3);               // register j: word ks of 32-dim step j
        f32x4 acc0 = f32x4{0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0;
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_frag(r0, ku), qf[0], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_frag(r2, ku), qf[2], acc1, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_frag(r1, ku), qf[1], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_frag(r3, ku), qf[3], acc1, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 sb = *reinterpret_cast<const float4*>(&S.ksb[16 * mt + 4 * ks + i][0]);
          z[mt][i] = fmaf(sb.z, acc1[i], fmaf(sb.w, qsum[1], fmaf(sb.x, acc0[i], sb.y * qsum[0])));
        }
      }
      __builtin_amdgcn_sched_barrier(0);

      // ---- the two halves' scores meet: z = z(dims 0..127) + z(dims 128..255) in both waves
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        sh.zx[zbuf][h][mt][lane] = make_float4(z[mt][0], z[mt][1], z[mt][2], z[mt][3]);
      __syncthreads();
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const float4 zo = sh.zx[zbuf][h ^ 1][mt][lane];
        if (h == 0) {
          z[mt][0] += zo.x; z[mt][1] += zo.y; z[mt][2] += zo.z; z[mt][3] += zo.w;
        } else {
          z[mt][0] = zo.x + z[mt][0]; z[mt][1] = zo.y + z[mt][1];
          z[mt][2] = zo.z + z[mt][2]; z[mt][3] = zo.w + z[mt][3];
        }
      }
      zbuf ^= 1;

      // ---- online softmax for this lane's query vector (identical in both waves)
      float mt_ = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = tt + 16 * mt + 4 * ks + i;
          float zz = z[mt][i] * a.scale_log2e;
          if (tok >= t1 || tok >= vend) zz = -INFINITY;
          z[mt][i] = zz;
          mt_ = fmaxf(mt_, zz);
        }
      mt_ = qv_max(mt_);
      if (__ballot(mt_ > m + 8.0f)) {
        asm volatile("; running max moves");
        const float mnew = (mt_ > m + 8.0f) ? mt_ : m;
        const float alpha = (mnew == -INFINITY) ? 1.0f : fast_exp2(m - mnew);
        m = mnew;
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < SP_DT; ++dt) o[dt] *= alpha;
#pragma unroll
        for (int g = 0; g < SP_G; ++g) pbias[g] *= alpha;
      }
      const float muse = (m == -INFINITY) ? 0.0f : m;
      float ls = 0.0f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          z[mt][i] = fast_exp2(z[mt][i] - muse);  // now p
          ls += z[mt][i];
        }
      l += ls;
      __builtin_amdgcn_sched_barrier(0);

      // ---- P.V over this wave's dims; step st covers this k-slot's tokens of blocks 2 st, 2 st + 1
#pragma unroll
      for (int g = 0; g < SP_G; ++g) {
        f16x8 bhi[2], blo[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const float4 s0 = *reinterpret_cast<const float4*>(&S.vs[g][32 * st + 4 * ks]);
          const float4 s1 = *reinterpret_cast<const float4*>(&S.vs[g][32 * st + 16 + 4 * ks]);
          const float4 b0 = *reinterpret_cast<const float4*>(&S.vb[g][32 * st + 4 * ks]);
          const float4 b1 = *reinterpret_cast<const float4*>(&S.vb[g][32 * st + 16 + 4 * ks]);
          const float* p0 = z[2 * st];
          const float* p1 = z[2 * st + 1];
          const float ss0[4] = {s0.x, s0.y, s0.z, s0.w}, ss1[4] = {s1.x, s1.y, s1.z, s1.w};
          const float bb0[4] = {b0.x, b0.y, b0.z, b0.w}, bb1[4] = {b1.x, b1.y, b1.z, b1.w};
          float pbs = 0.0f;
          uint32_t hi[4], lo[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {           // pair (block 2 st token k, block 2 st + 1 token k)
            const float w0 = p0[k] * ss0[k], w1 = p1[k] * ss1[k];
            split_f16(w0, w1, hi[k], lo[k]);
            pbs = fmaf(p0[k], bb0[k], fmaf(p1[k], bb1[k], pbs));
          }
          pbias[g] += pbs;
          bhi[st] = __builtin_bit_cast(f16x8, make_uint4(hi[0], hi[1], hi[2], hi[3]));
          blo[st] = __builtin_bit_cast(f16x8, make_uint4(lo[0], lo[1], lo[2], lo[3]));
        }
#pragma unroll
        for (int dq = 0; dq < SP_DT / SP_G; ++dq) {
          const int dt = g * (SP_DT / SP_G) + dq;
          const i32x2 tw = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
              (__attribute__((address_space(3))) i32x2*)(&S.v[lane][8 * dt]));
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const f16x8 af = v_frag_sub((uint32_t)tw[st]);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bhi[st], o[dt], 0, 0, 0);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, blo[st], o[dt], 0, 0, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      mf_lds_sync();                              // this wave's LDS is rewritten next tile
    }

    // ---- segment end: normaliser and bias sums over the four k-slots, write the partial
    l = qv_sum(l);
#pragma unroll
    for (int g = 0; g < SP_G; ++g) pbias[g] = qv_sum(pbias[g]);
    const int64_t slot = (int64_t)b * HQG + uu + w;
    if (qreal) {
      float* orow = a.opart + (slot * MF_QV + qv) * D + SP_HD * h;
      constexpr float two24 = 16777216.0f;        // the V codes entered as c * 2^-24
#pragma unroll
      for (int dt = 0; dt < SP_DT; ++dt) {
        const float pbv = pbias[dt / (SP_DT / SP_G)];
        const float4 v4 = make_float4(fmaf(o[dt][0], two24, pbv), fmaf(o[dt][1], two24, pbv),
                                      fmaf(o[dt][2], two24, pbv), fmaf(o[dt][3], two24, pbv));
        *reinterpret_cast<float4*>(orow + 16 * dt + 4 * ks) = v4;
      }
      if (h == 0 && ks == 0) {
        a.ml[(slot * MF_QV + qv) * 2] = m;
        a.ml[(slot * MF_QV + qv) * 2 + 1] = l;
      }
    }

    x += seg;
    t_lo += seg;
    if (t_lo >= len && x < x1) {
      t_lo = 0;
      if (++uu == HQG) {
        uu = 0;
        do { ++b; } while (b < B && mf_len(a, b) == 0);
        if (b >= B) break;
        len = mf_uni(mf_len(a, b));
      }
    }
  }
}

// ------------------------------------------------------------------- head dim 256, <= 8 vectors
//
// partial_mfma_pair_kernel: the split kernel's layout for a KV head with at most 8 query vectors
// (GQA 8 x one row, the decode shape), where 16 MFMA columns would carry 8 padded ones.  The
// tile's four 16-token blocks are taken in pairs (X, Y) = (0, 1), (2, 3), and each MFMA works on
// both blocks of a pair at once with block-diagonal operands:
//  * q.k: columns 0-7 are the 8 vectors against block X, columns 8-15 against block Y.  The A
//    operand's k-slots 0-15 hold codes of X's tokens and 16-31 codes of Y's (lane (m, g) holds row
//    m of block X for g < 2, of block Y for g >= 2); B holds q in the slots of the column's own
//    block and zeros in the other's.  One MFMA thus covers 16 dims of 16 tokens in each of two
//    blocks, the same work as 32 dims of one block against 16 columns of which 8 were padding, and
//    every output column is a real (vector, block) pair.  Lane (m, g) takes its 8 dims from 16-byte
//    chunk (g & 1) of its row for scale group 0 and chunk 2 + (g & 1) for group 1, so each MFMA
//    stays inside one scale group and no lane shuffle is needed to place the codes.
//  * each lane then holds 4 scores (4 tokens x 1 vector) per pair instead of 8 (half of them
//    padding): the score exchange, softmax, weights and bias sums do half the work.
//  * P.V: the transposing LDS read gives lane (m, g) dim m of 8 tokens per pair, X's tokens
//    4g..4g+3 in the even k-slots and Y's in the odd ones (the permuted V rows of the split
//    kernel); B holds the lane's own 4 weights in the slots of its column's block and zeros in the
//    other's, so columns 0-7 accumulate X's tokens and 8-15 Y's, and the two halves of a vector's
//    output are added once at the end of a range.
constexpr int PQ = 8;                             // query vectors per unit

struct PairShared {
  SpWave w[2];
  float4 zx[2][2][2][64];                         // partial scores [buffer][wave][pair][lane]
};

__global__ void __launch_bounds__(128, 2)
partial_mfma_pair_kernel(PartialArgs a) {
  const KUnpack ku = k_unpack_consts();
  constexpr int D = 256;
  __shared__ __align__(16) PairShared sh;

  const int lane = threadIdx.x & 63;
  const int h = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // dim half of this wave
  const int w = blockIdx.x;                                         // range (whole workgroup)
  SpWave& S = sh.w[h];
  const int B = a.batch, HQG = a.HK * a.qgroups;
  const int n = lane & 15, g = lane >> 4;         // MFMA column / A row, lane group
  const int bx = n >> 3, v = n & 7;               // block of the pair (0: X, 1: Y), vector
  const bool mine = bx == (g >> 1);               // this lane's k-slots belong to its column's block
  // v_perm selectors: half 0 (group 0) / half 1 (group 1) of a packed f16 pair into the low half
  // (block X columns) or the high half (block Y columns), zeros elsewhere
  const uint32_t sel0 = bx ? 0x01000C0Cu : 0x0C0C0100u;
  const uint32_t sel1 = bx ? 0x03020C0Cu : 0x0C0C0302u;

  MfRange rg;
  if (!mf_find_range(a, w, lane, rg)) return;     // the same for both waves: no barrier is left
  int b = rg.b, len = rg.len, uu = rg.uu, t_lo = rg.t_lo;
  const int64_t x1 = rg.x1;
  const int REP = a.HQ / a.HK, N = a.N;
  const int QV_total = REP * N;
  int zbuf = 0;

  int64_t x = rg.x0;
  while (x < x1) {
    const int seg = (int)min<int64_t>((int64_t)(len - t_lo), x1 - x);
    const int t1 = t_lo + seg;
    const int hk = uu / a.qgroups, qg = uu - hk * a.qgroups;
    const int32_t* trow = a.table + (int64_t)b * a.max_blocks;

    // ---- q fragments: MFMA j (group j >> 2, dword j & 3) takes the 8 dims of dword j & 3 of chunk
    // (g & 1) + 2 (j >> 2) of the wave's half row, in the codes' pair order; zero where the slots
    // belong to the other block.  Every lane sums its vector's q over those dims for the bias term.
    const int jj0 = qg * PQ + v;
    const bool qreal = jj0 < QV_total;
    const int hq = hk * REP + (qreal ? jj0 / N : 0), qi = qreal ? jj0 - (jj0 / N) * N : 0;
    const uint16_t* qrow = a.q + (((int64_t)b * a.HQ + hq) * N + qi) * D + SP_HD * h;
    bf16x8 qf[8];
    float qsum[SP_G] = {0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = (g & 1) + 2 * (j >> 2);
      uint4 d = qreal ? *reinterpret_cast<const uint4*>(qrow + 32 * c + 8 * (j & 3)) : make_uint4(0, 0, 0, 0);
      qsum[j >> 2] += bf16_lo(d.x) + bf16_hi(d.x) + bf16_lo(d.y) + bf16_hi(d.y) + bf16_lo(d.z) + bf16_hi(d.z) +
                      bf16_lo(d.w) + bf16_hi(d.w);
      if (!mine) d = make_uint4(0, 0, 0, 0);
      uint4 r;
      r.x = __builtin_amdgcn_perm(d.z, d.x, 0x05040100u);
      r.y = __builtin_amdgcn_perm(d.z, d.x, 0x07060302u);
      r.z = __builtin_amdgcn_perm(d.w, d.y, 0x05040100u);
      r.w = __builtin_amdgcn_perm(d.w, d.y, 0x07060302u);
      qf[j] = __builtin_bit_cast(bf16x8, r);
    }
#pragma unroll
    for (int gg = 0; gg < SP_G; ++gg) qsum[gg] += __shfl_xor(qsum[gg], 16, 64);   // both chunks of a group
    const int vend = qreal ? len - N + qi + 1 : 0;

    f32x4 o[SP_DT];
#pragma unroll
    for (int dt = 0; dt < SP_DT; ++dt) o[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m = -INFINITY, l = 0.0f, pbias[SP_G] = {0.0f, 0.0f};

    auto tab_idx = [&](int tstart) -> int {
      const int t = min(tstart + lane, t1 - 1);
      return (a.bs_shift >= 0) ? (t >> a.bs_shift) : (t / a.BS);
    };
    auto row_of = [&](int tstart, int phys) -> int {
      const int t = min(tstart + lane, t1 - 1);
      const int blk = (a.bs_shift >= 0) ? (t >> a.bs_shift) : (t / a.BS);
      phys = min(max(phys, 0), a.num_blocks - 1);
      return (phys * a.HK + hk) * a.BS + (t - blk * a.BS);
    };
    // loads of one tile: V half rows (as the split kernel), K: for pair st and group c the chunk
    // (g & 1) + 2c of row m of block 2 st + (g >> 1), and the scale planes of row `lane`
    auto issue = [&](SpTileRegs& t, int my_row) {
      const char* kplane = static_cast<const char*>(a.k) + SP_HB * h;
      const char* vplane = static_cast<const char*>(a.v) + SP_HB * h;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = __builtin_amdgcn_ds_bpermute(4 * (lane >> 2) + 64 * i, my_row);
        t.v[i] = *reinterpret_cast<const u32x4*>(vplane + row * (2 * SP_HB) + 16 * (lane & 3));
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int64_t row = __builtin_amdgcn_ds_bpermute(4 * (16 * (2 * st + (g >> 1)) + n), my_row);
#pragma unroll
        for (int c = 0; c < 2; ++c)
          t.k[2 * st + c] = *reinterpret_cast<const u32x4*>(kplane + row * (2 * SP_HB) + 16 * ((g & 1) + 2 * c));
      }
      const int64_t ri = (int64_t)my_row * (2 * SP_G) + SP_G * h;
      t.ks = *reinterpret_cast<const uint32_t*>(a.ks + ri);
      t.kb = *reinterpret_cast<const uint32_t*>(a.kb + ri);
      t.vs = *reinterpret_cast<const uint32_t*>(a.vs + ri);
      t.vb = *reinterpret_cast<const uint32_t*>(a.vb + ri);
    };
    SpTileRegs cur;
    int ph_next = 0;
    if (t_lo < t1) {
      issue(cur, row_of(t_lo, trow[tab_idx(t_lo)]));
      if (t_lo + MF_TILE < t1) ph_next = trow[tab_idx(t_lo + MF_TILE)];
    }

    for (int tt = t_lo; tt < t1; tt += MF_TILE) {
      // ---- V half rows (permuted) and the scales into this wave's LDS; K stays in registers
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * i + (lane >> 2);
        const int pr = 16 * ((r >> 2) & 3) + 4 * (r >> 4) + (r & 3);
        *reinterpret_cast<u32x4*>(&S.v[pr][16 * (lane & 3)]) = cur.v[i];
      }
      {
        const float ks0 = bf16_lo(cur.ks), ks1 = bf16_hi(cur.ks);
        *reinterpret_cast<float4*>(&S.ksb[lane][0]) =
            make_float4(ks0, fmaf(-128.0f, ks0, bf16_lo(cur.kb)), ks1, fmaf(-128.0f, ks1, bf16_hi(cur.kb)));
        S.vs[0][lane] = bf16_lo(cur.vs);
        S.vs[1][lane] = bf16_hi(cur.vs);
        S.vb[0][lane] = bf16_lo(cur.vb);
        S.vb[1][lane] = bf16_hi(cur.vb);
      }
      u32x4 kc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) kc[i] = cur.k[i];
      if (tt + MF_TILE < t1) {                    // the same for both waves
        issue(cur, row_of(tt + MF_TILE, ph_next));
        if (tt + 2 * MF_TILE < t1) ph_next = trow[tab_idx(tt + 2 * MF_TILE)];
      }
      mf_lds_sync();

      // ---- q.k for both pairs, then each score's scale and bias: lane (n, g), pair st holds the
      // scores of tokens 16 (2 st + bx) + 4 g + i for vector v
      float z[2][4];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        f32x4 acc0 = f32x4{0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_frag(kc[2 * st][j], ku), qf[j], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_frag(kc[2 * st + 1][j], ku), qf[4 + j], acc1, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 sb = *reinterpret_cast<const float4*>(&S.ksb[16 * (2 * st + bx) + 4 * g + i][0]);
          z[st][i] = fmaf(sb.z, acc1[i], fmaf(sb.w, qsum[1], fmaf(sb.x, acc0[i], sb.y * qsum[0])));
        }
      }

      // ---- the two halves' scores meet: z = z(dims 0..127) + z(dims 128..255) in both waves
#pragma unroll
      for (int st = 0; st < 2; ++st)
        sh.zx[zbuf][h][st][lane] = make_float4(z[st][0], z[st][1], z[st][2], z[st][3]);
      __syncthreads();
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const float4 zo = sh.zx[zbuf][h ^ 1][st][lane];
        if (h == 0) {
          z[st][0] += zo.x; z[st][1] += zo.y; z[st][2] += zo.z; z[st][3] += zo.w;
        } else {
          z[st][0] = zo.x + z[st][0]; z[st][1] = zo.y + z[st][1];
          z[st][2] = zo.z + z[st][2]; z[st][3] = zo.w + z[st][3];
        }
      }
      zbuf ^= 1;

      // ---- online softmax for vector v (identical in both waves); its 64 tokens sit in the 8
      // lanes v, v + 8, ... (lane bits 3, 4, 5)
      float mt_ = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = tt + 16 * (2 * st + bx) + 4 * g + i;
          float zz = z[st][i] * a.scale_log2e;
          if (tok >= t1 || tok >= vend) zz = -INFINITY;
          z[st][i] = zz;
          mt_ = fmaxf(mt_, zz);
        }
      mt_ = xor8_reduce<OpMax>(mt_);
      if (__ballot(mt_ > m + 8.0f)) {
        asm volatile("; running max moves");
        const float mnew = (mt_ > m + 8.0f) ? mt_ : m;
        const float alpha = (mnew == -INFINITY) ? 1.0f : fast_exp2(m - mnew);
        m = mnew;
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < SP_DT; ++dt) o[dt] *= alpha;
#pragma unroll
        for (int gg = 0; gg < SP_G; ++gg) pbias[gg] *= alpha;
      }
      const float muse = (m == -INFINITY) ? 0.0f : m;
      float ls = 0.0f;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          z[st][i] = fast_exp2(z[st][i] - muse);  // now p
          ls += z[st][i];
        }
      l += ls;

      // ---- weights w = p * s_v per (pair, token, group), split into f16 hi + lo (each rounded to
      // nearest), both groups of a token packed in one f16 pair and moved by v_perm into the
      // k-slot half of the lane's block (zeros in the other block's half)
      uint32_t bh[SP_G][2][4], bl[SP_G][2][4];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int t0 = 16 * (2 * st + bx) + 4 * g;
        const float4 s0 = *reinterpret_cast<const float4*>(&S.vs[0][t0]);
        const float4 s1 = *reinterpret_cast<const float4*>(&S.vs[1][t0]);
        const float4 c0 = *reinterpret_cast<const float4*>(&S.vb[0][t0]);
        const float4 c1 = *reinterpret_cast<const float4*>(&S.vb[1][t0]);
        const float sv0[4] = {s0.x, s0.y, s0.z, s0.w}, sv1[4] = {s1.x, s1.y, s1.z, s1.w};
        const float bv0[4] = {c0.x, c0.y, c0.z, c0.w}, bv1[4] = {c1.x, c1.y, c1.z, c1.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = z[st][i];
          uint32_t hi2, lo2;
          split_f16(p * sv0[i], p * sv1[i], hi2, lo2);           // (group 0, group 1)
          bh[0][st][i] = __builtin_amdgcn_perm(hi2, hi2, sel0);
          bh[1][st][i] = __builtin_amdgcn_perm(hi2, hi2, sel1);
          bl[0][st][i] = __builtin_amdgcn_perm(lo2, lo2, sel0);
          bl[1][st][i] = __builtin_amdgcn_perm(lo2, lo2, sel1);
          pbias[0] = fmaf(p, bv0[i], pbias[0]);
          pbias[1] = fmaf(p, bv1[i], pbias[1]);
        }
      }

      // ---- P.V over this wave's dims
#pragma unroll
      for (int gg = 0; gg < SP_G; ++gg) {
        f16x8 bhi[2], blo[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          bhi[st] = __builtin_bit_cast(f16x8, make_uint4(bh[gg][st][0], bh[gg][st][1], bh[gg][st][2], bh[gg][st][3]));
          blo[st] = __builtin_bit_cast(f16x8, make_uint4(bl[gg][st][0], bl[gg][st][1], bl[gg][st][2], bl[gg][st][3]));
        }
#pragma unroll
        for (int dq = 0; dq < SP_DT / SP_G; ++dq) {
          const int dt = gg * (SP_DT / SP_G) + dq;
          const i32x2 tw = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
              (__attribute__((address_space(3))) i32x2*)(&S.v[lane][8 * dt]));
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const f16x8 af = v_frag_sub((uint32_t)tw[st]);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bhi[st], o[dt], 0, 0, 0);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, blo[st], o[dt], 0, 0, 0);
          }
        }
        }
      mf_lds_sync();                              // this wave's LDS is rewritten next tile
    }

    // ---- segment end: a vector's normaliser and bias sums over its 8 lanes, its output as the
    // sum of its block-X and block-Y columns; write the partial
    l = xor8_reduce<OpAdd>(l);
#pragma unroll
    for (int gg = 0; gg < SP_G; ++gg) pbias[gg] = xor8_reduce<OpAdd>(pbias[gg]);
#pragma unroll
    for (int dt = 0; dt < SP_DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[dt][i] += __shfl_xor(o[dt][i], 8, 64);
    const int64_t slot = (int64_t)b * HQG + uu + w;
    if (qreal && bx == 0) {
      float* orow = a.opart + (slot * PQ + v) * D + SP_HD * h;
      constexpr float two24 = 16777216.0f;        // the V codes entered as c * 2^-24
#pragma unroll
      for (int dt = 0; dt < SP_DT; ++dt) {
        const float pbv = pbias[dt / (SP_DT / SP_G)];
        const float4 v4 = make_float4(fmaf(o[dt][0], two24, pbv), fmaf(o[dt][1], two24, pbv),
                                      fmaf(o[dt][2], two24, pbv), fmaf(o[dt][3], two24, pbv));
        *reinterpret_cast<float4*>(orow + 16 * dt + 4 * g) = v4;
      }
      if (h == 0 && g == 0) {
        a.ml[(slot * PQ + v) * 2] = m;
        a.ml[(slot * PQ + v) * 2 + 1] = l;
      }
    }

    x += seg;
    t_lo += seg;
    if (t_lo >= len && x < x1) {
      t_lo = 0;
      if (++uu == HQG) {
        uu = 0;
        do { ++b; } while (b < B && mf_len(a, b) == 0);
        if (b >= B) break;
        len = mf_uni(mf_len(a, b));
      }
    }
  }
}

bool mfma_supported(int bits, int D, int gs) { return bits == 4 && gs == 64 && (D == 128 || D == 256); }

hipError_t launch_partial_mfma(const PartialArgs& a, int D, hipStream_t s) {
  switch (D) {
    case 128:
      hipLaunchKernelGGL(partial_mfma_kernel<128>, dim3((unsigned)(a.num_ranges / MF_WAVES)), dim3(MF_WAVES * 64),
                         0, s, a);
      break;
    case 256:
      if ((a.HQ / a.HK) * a.N <= MFMA_PAIR_QVW)
        hipLaunchKernelGGL(partial_mfma_pair_kernel, dim3((unsigned)a.num_ranges), dim3(2 * 64), 0, s, a);
      else
        hipLaunchKernelGGL(partial_mfma_split_kernel, dim3((unsigned)a.num_ranges), dim3(2 * 64), 0, s, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
