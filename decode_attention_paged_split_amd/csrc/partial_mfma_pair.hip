// Matrix-core engine, head dim 256 with at most 8 query vectors per KV head: the pair kernel
// (the layout and the shared helpers: partial_mfma_common.hpp).
#include "partial_mfma_common.hpp"

namespace kvq {

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
  if (!mf_find_range(a, w, lane, rg, HQG)) return;     // the same for both waves: no barrier is left
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
    int ve[SP_G] = {MF_VE_NONE, MF_VE_NONE};         // this wave's V groups' prescale exponents

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
        const float sc = mf_pow2(ve[dt / (SP_DT / SP_G)]);   // the weights' prescale
        const float4 v4 = make_float4(fmaf(o[dt][0] * sc, two24, pbv), fmaf(o[dt][1] * sc, two24, pbv),
                                      fmaf(o[dt][2] * sc, two24, pbv), fmaf(o[dt][3] * sc, two24, pbv));
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

hipError_t launch_mfma_pair(const PartialArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(partial_mfma_pair_kernel, dim3((unsigned)a.num_ranges), dim3(2 * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
