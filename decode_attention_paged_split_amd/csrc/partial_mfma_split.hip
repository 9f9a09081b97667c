// Matrix-core engine, head dim 256 with more than 8 query vectors per KV head: the split kernel
// (the layout and the shared helpers: partial_mfma_common.hpp).
#include "partial_mfma_common.hpp"

namespace kvq {

__global__ void __launch_bounds__(128, 2)
partial_mfma_split_kernel(PartialArgs a) {
  const KUnpack ku = k_unpack_consts();
  constexpr int D = 256;
  __shared__ __align__(16) SpShared sh;

  const int lane = threadIdx.x & 63;
  const int h = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // dim half of this wave
  // this workgroup's range and lane: the L = a.lanes query groups of a set (KV head, L
  // consecutive groups) run side by side on L workgroups of one XCD, one group each, over the same
  // range, so each K/V row is fetched from memory once for the set
  int w, ln;
  stream_range_lane(a.lanes, blockIdx.x, gridDim.x, w, ln);
  w = __builtin_amdgcn_readfirstlane(w);
  ln = __builtin_amdgcn_readfirstlane(ln);
  SpWave& S = sh.w[h];
  const int B = a.batch, L = a.lanes, QGB = a.qgroups / L, HS = a.HK * QGB;   // sets per sequence
  const int qv = lane & 15, ks = lane >> 4;

  MfRange rg;
  if (!mf_find_range(a, w, lane, rg, HS)) return;  // the same for both waves: no barrier is left
  int b = rg.b, len = rg.len, uu = rg.uu, t_lo = rg.t_lo;
  const int64_t x1 = rg.x1;
  const int REP = a.HQ / a.HK, N = a.N;
  const int QV_total = REP * N;
  int zbuf = 0;

  int64_t x = rg.x0;
  while (x < x1) {
    const int seg = (int)min<int64_t>((int64_t)(len - t_lo), x1 - x);
    const int t1 = t_lo + seg;
    const int hk = uu / QGB, qg = (uu - hk * QGB) * L + ln;
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
    int ve[SP_G] = {MF_VE_NONE, MF_VE_NONE};         // this wave's V groups' prescale exponents

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
        if (__ballot(mf_vpre_moves(bf16_lo(cur.vs), ve[0]) || mf_vpre_moves(bf16_hi(cur.vs), ve[1]))) {
          const float r0 = mf_vpre_update(bf16_lo(cur.vs), ve[0]);   // uniform; a segment's first tile
          const float r1 = mf_vpre_update(bf16_hi(cur.vs), ve[1]);
#pragma unroll
          for (int dt = 0; dt < SP_DT; ++dt) o[dt] *= (dt < SP_DT / SP_G) ? r0 : r1;
        }
        S.vs[0][lane] = bf16_lo(cur.vs) * mf_pow2(-ve[0]);
        S.vs[1][lane] = bf16_hi(cur.vs) * mf_pow2(-ve[1]);
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
    const int64_t slot = ((int64_t)b * HS + uu + w) * L + ln;
    if (qreal) {
      float* orow = a.opart + (slot * MF_QV + qv) * D + SP_HD * h;
      constexpr float two24 = 16777216.0f;        // the V codes entered as c * 2^-24
#pragma unroll
      for (int dt = 0; dt < SP_DT; ++dt) {
        const float pbv = pbias[dt / (SP_DT / SP_G)];
        const float sc = mf_pow2(ve[dt / (SP_DT / SP_G)]);   // the weights' prescale
        const float4 v4 = make_float4(fmaf(o[dt][0] * sc, two24, pbv), fmaf(o[dt][1] * sc, two24, pbv),
                                      fmaf(o[dt][2] * sc, two24, pbv), fmaf(o[dt][3] * sc, two24, pbv));
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
      if (++uu == HS) {
        uu = 0;
        do { ++b; } while (b < B && mf_len(a, b) == 0);
        if (b >= B) break;
        len = mf_uni(mf_len(a, b));
      }
    }
  }
}

hipError_t launch_mfma_split(const PartialArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(partial_mfma_split_kernel, dim3((unsigned)(a.num_ranges * a.lanes)), dim3(2 * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
