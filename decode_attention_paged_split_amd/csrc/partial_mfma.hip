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
// A wave owns 16 query vectors (the MFMA N dimension; unused ones are zero) and walks tiles of
// 64 tokens:
//  * q.k: v_mfma_f32_16x16x32_bf16 with A = a 16-token block of K rows and B = q^T.  Codes
//    become bf16(128 + c) with one v_and_or (exact) and q is exact in bf16, so every product is
//    exact; each MFMA step covers 32 dims of one 64-dim scale group, so the group's scale and
//    bias apply once per (token, group): z = s * acc + (b - 128 s) * sum_g(q).  A lane loads 16
//    contiguous bytes of its row and four v_permlane{32,16}_swap turn four lanes' chunks into
//    the word each lane's k-slot needs.
//  * softmax: the MFMA result gives every lane one query vector (lane % 16) and four tokens, so
//    the running max, normaliser and per-group sums are per-lane scalars; the tile max needs two
//    lane swaps.  The running max moves only when a score exceeds it by more than 2^8, so the
//    accumulators are rescaled only then.
//  * P.V: v_mfma_f32_16x16x32_f16 with A = V^T and B = (p * scale)^T.  V^T comes straight from
//    the raw 4-bit tile in LDS through ds_read_b64_tr_b4 (a 16 x 16 nibble transpose per 16
//    lanes); codes become exact f16 (1024 + c, then - 1024 with one packed add).  The weight
//    w = p * s(token, group) is split into f16 hi + lo (hi = w rounded toward zero, lo = the
//    rest), two MFMAs per step, so the product is accurate to ~2^-22 relative; the bias term
//    sum_t p * b is accumulated per (vector, group) in f32 and added at the end.
#include "device_common.hpp"
#include "kernels.hpp"

namespace kvq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

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
  static_assert(D == 128 || D == 256, "head dim");
};

template <int D>
struct MScratch {
  using Mg = MGeo<D>;
  uint8_t v[MF_TILE][Mg::PITCH];                 // raw V codes of the tile
  float2 ksb[MF_TILE][Mg::G];                    // K (scale, bias - 128 scale)
  float vs[Mg::G][MF_TILE];                      // V scale
  float vb[Mg::G][MF_TILE];                      // V bias
  float pt[MF_QV][MF_TILE];                      // probabilities [vector][token]
};

__device__ __forceinline__ uint32_t mf_and_or(uint32_t x, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(o));
  return r;
}

__device__ __forceinline__ void mf_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// a 4-bit word -> 8 bf16 (128 + c) in pair order (n0,n4),(n1,n5),(n2,n6),(n3,n7)
__device__ __forceinline__ bf16x8 k_frag(uint32_t w) {
  const uint32_t mg = 0x43004300u;
  uint4 r;
  r.x = mf_and_or(w, 0x000F000Fu, mg);
  r.y = mf_and_or(w >> 4, 0x000F000Fu, mg);
  r.z = mf_and_or(w >> 8, 0x000F000Fu, mg);
  r.w = mf_and_or(w >> 12, 0x000F000Fu, mg);
  return __builtin_bit_cast(bf16x8, r);
}

// a 4-bit word -> 8 exact f16 codes in pair order (n0,n4),(n1,n5),(n2,n6),(n3,n7)
__device__ __forceinline__ f16x8 v_frag(uint32_t w) {
  const uint32_t mg = 0x64006400u;                 // f16 1024 in both halves
  const f16x2 off = {(_Float16)-1024.0f, (_Float16)-1024.0f};
  f16x2 p0 = __builtin_bit_cast(f16x2, mf_and_or(w, 0x000F000Fu, mg)) + off;
  f16x2 p1 = __builtin_bit_cast(f16x2, mf_and_or(w >> 4, 0x000F000Fu, mg)) + off;
  f16x2 p2 = __builtin_bit_cast(f16x2, mf_and_or(w >> 8, 0x000F000Fu, mg)) + off;
  f16x2 p3 = __builtin_bit_cast(f16x2, mf_and_or(w >> 12, 0x000F000Fu, mg)) + off;
  uint4 r = make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                       __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
  return __builtin_bit_cast(f16x8, r);
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

// max / sum over the four lanes that share a query vector (lane, lane ^ 16, ^ 32, ^ 48)
__device__ __forceinline__ float qv_max(float x) { return block_reduce<OpMax, 16, 64>(x); }
__device__ __forceinline__ float qv_sum(float x) { return block_reduce<OpAdd, 16, 64>(x); }

template <int D>
__global__ void __launch_bounds__(MF_WAVES * 64, 1)
partial_mfma_kernel(PartialArgs a) {
  using Mg = MGeo<D>;
  constexpr int G = Mg::G, KSTEPS = Mg::KSTEPS, KSETS = Mg::KSETS, DT = Mg::DT, ROWB = Mg::ROWB;
  constexpr int CPR = Mg::CPR, NVL = Mg::NVL;
  __shared__ __align__(16) MScratch<D> scr[MF_WAVES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = blockIdx.x * MF_WAVES + wave;
  MScratch<D>& S = scr[wave];
  const int B = a.batch, HQG = a.HK * a.qgroups;
  const int qv = lane & 15, ks = lane >> 4;       // query vector (MFMA n / m%16), k-slot (lane / 16)

  // ---- the stream: total length, working waves, this wave's range [x0, x1)
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
  if (w >= W_eff) return;                          // no block-level barriers in this kernel
  const int64_t x0 = ((int64_t)w * T + W_eff - 1) / W_eff;
  const int64_t x1 = ((int64_t)(w + 1) * T + W_eff - 1) / W_eff;
  if (x0 >= x1) return;
  int b = -1;
  int64_t pb = 0;
  {
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
      const uint64_t hit = __ballot((base + incl) * HQG > x0 && lv > 0);
      if (hit) {
        const int k = __builtin_ctzll(hit);
        b = mf_uni(c + k);
        pb = mf_uni64(base + __shfl(incl, k, 64) - __shfl(lv, k, 64));
        break;
      }
      base += mf_uni(__shfl(incl, 63, 64));
    }
  }
  if (b < 0) return;
  int len = mf_uni(mf_len(a, b));
  const int64_t rem = x0 - pb * HQG;
  int uu = mf_uni((int)(rem / len));
  int t_lo = mf_uni((int)(rem - (int64_t)uu * len));

  const char* kplane = static_cast<const char*>(a.k);
  const char* vplane = static_cast<const char*>(a.v);
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

    for (int tt = t_lo; tt < t1; tt += MF_TILE) {
      const int last = t1 - 1 - tt;
      // pool row of tile row lane (lane < 64 == MF_TILE): one base when the tile is inside one block
      const bool one_block = (a.bs_shift >= 0) && ((tt & (a.BS - 1)) + MF_TILE <= a.BS);
      int64_t base = 0;
      int my_row = 0;
      auto row_of = [&](int t) -> int64_t {
        const int blk = (a.bs_shift >= 0) ? (t >> a.bs_shift) : (t / a.BS);
        const int off = t - blk * a.BS;
        int phys = trow[blk];
        phys = min(max(phys, 0), a.num_blocks - 1);
        return ((int64_t)phys * a.HK + hk) * a.BS + off;
      };
      if (one_block) base = row_of(tt);
      else my_row = (int)row_of(tt + min(lane, last));
      auto rowi = [&](int r) -> int64_t {
        return one_block ? base + min(r, last) : (int64_t)__shfl(my_row, r, 64);
      };

      // ---- loads: V tile (straight into LDS), scales, and K block by block (16 rows each; k-slot
      // ks takes 16-byte chunks ks, ks + 4, ...), the next block prefetched during q.k of this one
      auto load_k = [&](int mt, uint4* kr) {
        const char* src = kplane + rowi(16 * mt + qv) * ROWB;
#pragma unroll
        for (int c = 0; c < KSETS; ++c) kr[c] = *reinterpret_cast<const uint4*>(src + 16 * (4 * c + ks));
      };
      uint4 kcur[KSETS], knext[KSETS];
      {
        uint4 vraw[NVL];
#pragma unroll
        for (int i = 0; i < NVL; ++i) {
          const int e = i * 64 + lane, r = e / CPR, ch = e - r * CPR;
          vraw[i] = *reinterpret_cast<const uint4*>(vplane + rowi(r) * ROWB + 16 * ch);
        }
        load_k(0, kcur);
        const int64_t ri = rowi(lane) * G;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float ksc = bf16_to_f32(a.ks[ri + g]), kbi = bf16_to_f32(a.kb[ri + g]);
          S.ksb[lane][g] = make_float2(ksc, fmaf(-128.0f, ksc, kbi));
          S.vs[g][lane] = bf16_to_f32(a.vs[ri + g]);
          S.vb[g][lane] = bf16_to_f32(a.vb[ri + g]);
        }
#pragma unroll
        for (int i = 0; i < NVL; ++i) {
          const int e = i * 64 + lane, r = e / CPR, ch = e - r * CPR;
          *reinterpret_cast<uint4*>(&S.v[r][16 * ch]) = vraw[i];
        }
      }
      mf_lds_sync();
      __builtin_amdgcn_sched_barrier(0);

      // ---- q.k on the matrix cores, then per-group scale and bias
      float z[4][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if (mt + 1 < 4) load_k(mt + 1, knext);
        uint32_t kw[KSTEPS];
#pragma unroll
        for (int c = 0; c < KSETS; ++c) {
          uint32_t r0 = kcur[c].x, r1 = kcur[c].y, r2 = kcur[c].z, r3 = kcur[c].w;
          transpose4(r0, r1, r2, r3);                   // register j = word 4 (4c + j) + ks
          kw[4 * c + 0] = r0; kw[4 * c + 1] = r1; kw[4 * c + 2] = r2; kw[4 * c + 3] = r3;
        }
        f32x4 acc[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          acc[g] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_frag(kw[2 * g]), qf[2 * g], acc[g], 0, 0, 0);
          acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_frag(kw[2 * g + 1]), qf[2 * g + 1], acc[g], 0, 0, 0);
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
#pragma unroll
        for (int c = 0; c < KSETS; ++c) kcur[c] = knext[c];
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
            const auto h2 = __builtin_amdgcn_cvt_pkrtz(w0, w1);       // round toward zero
            const auto l2 = __builtin_amdgcn_cvt_pkrtz(w0 - (float)h2[0], w1 - (float)h2[1]);
            hi[k] = __builtin_bit_cast(uint32_t, h2);
            lo[k] = __builtin_bit_cast(uint32_t, l2);
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
            const f16x8 af = v_frag((uint32_t)tw[st]);
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
        float4 v4 = make_float4(o[dt][0] + pbv, o[dt][1] + pbv, o[dt][2] + pbv, o[dt][3] + pbv);
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

bool mfma_supported(int bits, int D, int gs) { return bits == 4 && gs == 64 && (D == 128 || D == 256); }

hipError_t launch_partial_mfma(const PartialArgs& a, int D, hipStream_t s) {
  dim3 grid((unsigned)(a.num_ranges / MF_WAVES));
  switch (D) {
    case 128: hipLaunchKernelGGL(partial_mfma_kernel<128>, grid, dim3(MF_WAVES * 64), 0, s, a); break;
    case 256: hipLaunchKernelGGL(partial_mfma_kernel<256>, grid, dim3(MF_WAVES * 64), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
