// Matrix-core engine: the head-dim-128 kernel and the launcher (the engine's design and the
// shared helpers: partial_mfma_common.hpp).
#include "partial_mfma_common.hpp"

namespace kvq {

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
  if (!mf_find_range(a, w, lane, rg, HQG)) return;      // no block-level barriers in this kernel
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
    int ve[G];                                       // V groups' prescale exponents
#pragma unroll
    for (int g = 0; g < G; ++g) { pbias[g] = 0.0f; ve[g] = MF_VE_NONE; }

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
      {
        bool moves = false;
#pragma unroll
        for (int g = 0; g < G; ++g) moves |= mf_vpre_moves(mf_bf16(cur.vs, g), ve[g]);
        if (__ballot(moves)) {                          // uniform; a segment's first tile
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float r = mf_vpre_update(mf_bf16(cur.vs, g), ve[g]);
#pragma unroll
            for (int dt = g * (DT / G); dt < (g + 1) * (DT / G); ++dt) o[dt] *= r;
          }
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float ksc = mf_bf16(cur.ks, g), kbi = mf_bf16(cur.kb, g);
        S.ksb[lane][g] = make_float2(ksc, fmaf(-128.0f, ksc, kbi));
        S.vs[g][lane] = mf_bf16(cur.vs, g) * mf_pow2(-ve[g]);
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
        const float sc = mf_pow2(ve[dt / (DT / G)]);   // the weights' prescale
        constexpr float two24 = 16777216.0f;        // the V codes entered as c * 2^-24
        const float4 v4 = make_float4(fmaf(o[dt][0] * sc, two24, pbv), fmaf(o[dt][1] * sc, two24, pbv),
                                      fmaf(o[dt][2] * sc, two24, pbv), fmaf(o[dt][3] * sc, two24, pbv));
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
  switch (D) {
    case 128:
      hipLaunchKernelGGL(partial_mfma_kernel<128>, dim3((unsigned)(a.num_ranges / MF_WAVES)), dim3(MF_WAVES * 64),
                         0, s, a);
      break;
    case 256:
      return ((a.HQ / a.HK) * a.N <= MFMA_PAIR_QVW) ? launch_mfma_pair(a, s) : launch_mfma_split(a, s);
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
