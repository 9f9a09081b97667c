// Split-K paged decode attention: partial kernel + log-sum-exp merge kernel.
//
// What is computed follows "@mlx-bun/inference 0.0.0-stage -> 1.0.0", diff page 50:
//  * paged.ts, paged_attention_partial / paged_attention_affine_partial: token t of a
//    sequence is read straight from physical block table[t / BS], row t % BS; affine
//    pages are dequantized on load (scale * code + bias, codes low-first in uint32
//    words); each partition keeps an online softmax (running max, normaliser and
//    unnormalised output) in f32; row i of N sees t < length - N + i + 1.
//  * kvq4-decode.ts, the partial kernel: one read of a K/V row serves every query head
//    of its GQA group (duplication-free GQA), and the token sub-chunks of a workgroup are
//    combined in on-chip memory with the same log-sum-exp algebra.
//  * paged_attention_merge / the kvq4 merge: out = sum_p e^(m_p - M) o_p /
//    sum_p e^(m_p - M) l_p, skipping partitions whose max is -inf.
//
// gfx950 design (not the pages' Metal layout):
//  * workgroup = (partition, KV head [x query group], sequence), 4 waves of 64 lanes;
//    lanes own DPL consecutive head dims of one token row (LPR lanes per row, RPW rows per
//    wave step), so K/V loads are coalesced 4/8/16-byte loads along a row;
//  * q.k uses v_dot2_f32_bf16 on (q pair, code pair): codes become bf16 pairs with one
//    v_and_or (the 4/2-bit codes c are packed as bf16(128 + c), exact), the scale and
//    bias are applied once per group: q.k = s * sum(q c) + b * sum(q);
//  * the dot is reduced across the LPR lanes of a row with DPP / permlane swaps;
//  * softmax is online per tile of tokens (one rescale per tile), in exp2 units;
//  * P.V dequantizes V in f32 registers (fma(scale, code, bias)) and accumulates in f32;
//  * waves combine in LDS, then one partial (o, m, l) per (sequence, head, row, partition).
#include "device_common.hpp"
#include "kernels.hpp"

namespace kvq {

constexpr int NWAVES = 4;

template <int BITS>
struct Fmt {
  static constexpr int DPL = (BITS == 2) ? 16 : 8;                          // dims per lane
  static constexpr int WPL = (BITS == 16) ? 4 : (BITS == 8 ? 2 : 1);        // words per lane-row
  static constexpr int NP = DPL / 2;                                        // bf16 pairs per lane
  static constexpr float OFFS = (BITS == 4 || BITS == 2) ? 128.0f : 0.0f;   // code bias in pairs
  // dims (relative to the lane's first dim) of pair k
  __device__ static constexpr int lo(int k) {
    return (BITS == 4) ? k : (BITS == 2) ? k : 2 * k;
  }
  __device__ static constexpr int hi(int k) {
    return (BITS == 4) ? k + 4 : (BITS == 2) ? k + 8 : 2 * k + 1;
  }
};

// K row chunk -> bf16 pairs (pair k = dims lo(k), hi(k)); affine codes as bf16(OFFS + c)
template <int BITS>
__device__ __forceinline__ void key_pairs(const uint32_t* w, uint32_t* pr) {
  if constexpr (BITS == 16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) pr[k] = w[k];
  } else if constexpr (BITS == 8) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float c0 = (float)(w[j] & 0xFFu), c1 = (float)((w[j] >> 8) & 0xFFu);
      const float c2 = (float)((w[j] >> 16) & 0xFFu), c3 = (float)(w[j] >> 24);
      // an integer below 256 is exact in bf16: its f32 pattern's low half is zero
      pr[2 * j] = (__float_as_uint(c0) >> 16) | (__float_as_uint(c1) & 0xFFFF0000u);
      pr[2 * j + 1] = (__float_as_uint(c2) >> 16) | (__float_as_uint(c3) & 0xFFFF0000u);
    }
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) pr[k] = ((w[0] >> (4 * k)) & 0x000F000Fu) | 0x43004300u;
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) pr[k] = ((w[0] >> (2 * k)) & 0x00030003u) | 0x43004300u;
  }
}

// V row chunk -> f32 values in natural dim order
template <int BITS>
__device__ __forceinline__ void value_f32(const uint32_t* w, float s, float b, float* v) {
  if constexpr (BITS == 16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) { v[2 * k] = bf16_lo(w[k]); v[2 * k + 1] = bf16_hi(w[k]); }
  } else if constexpr (BITS == 8) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[4 * j + i] = fmaf(s, (float)((w[j] >> (8 * i)) & 0xFFu), b);
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = fmaf(s, (float)((w[0] >> (4 * i)) & 0xFu), b);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = fmaf(s, (float)((w[0] >> (2 * i)) & 0x3u), b);
  }
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, a), __builtin_bit_cast(bf2, b), c, false);
}

// exact xor-partner exchange (used once per workgroup, for the slot combine)
__device__ __forceinline__ float shfl_xor_f(float x, int m) { return __shfl_xor(x, m, 64); }

template <int BITS, int D, int QVW, int U>
__global__ void __launch_bounds__(NWAVES * 64)
partial_kernel(PartialArgs a) {
  using F = Fmt<BITS>;
  constexpr int DPL = F::DPL, LPR = D / DPL, RPW = 64 / LPR, NP = F::NP, WPL = F::WPL;
  constexpr int WROW = D * BITS / 32;        // 32-bit words per pool row
  constexpr int G = D / 64;
  constexpr int TILE = RPW * U;              // tokens per wave step
  static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "lane layout");

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = lane / LPR, sl = lane - slot * LPR;
  const int p = blockIdx.x, b = blockIdx.z;
  const int hk = blockIdx.y / a.qgroups, qg = blockIdx.y - hk * a.qgroups;
  const int len = min(a.lengths[b], min(a.max_len, a.max_blocks * a.BS));
  const int t0 = p * a.part_tokens;
  if (t0 >= len) return;                     // uniform over the workgroup
  const int t1 = min(len, t0 + a.part_tokens);
  const int REP = a.HQ / a.HK;
  const int N = a.N;

  // ---- this lane's slice of the query vectors
  uint32_t qp[QVW][NP];
  float qsum[QVW];
  int vend[QVW];
#pragma unroll
  for (int j = 0; j < QVW; ++j) {
    const int jj = qg * QVW + j;
    const int h = hk * REP + jj / N, i = jj - (jj / N) * N;
    const uint16_t* qrow = a.q + (((int64_t)b * a.HQ + h) * N + i) * D + sl * DPL;
    uint16_t qv[DPL];
#pragma unroll
    for (int c = 0; c < DPL / 8; ++c) {
      const uint4 x = reinterpret_cast<const uint4*>(qrow)[c];
      const uint32_t ws[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) { qv[8 * c + 2 * e] = (uint16_t)(ws[e] & 0xFFFFu); qv[8 * c + 2 * e + 1] = (uint16_t)(ws[e] >> 16); }
    }
    float s = 0.0f;
#pragma unroll
    for (int d = 0; d < DPL; ++d) s += bf16_to_f32(qv[d]);
    qsum[j] = s;
#pragma unroll
    for (int k = 0; k < NP; ++k) qp[j][k] = (uint32_t)qv[F::lo(k)] | ((uint32_t)qv[F::hi(k)] << 16);
    vend[j] = len - N + i + 1;
  }

  float m[QVW], l[QVW], o[QVW][DPL];
#pragma unroll
  for (int j = 0; j < QVW; ++j) {
    m[j] = -INFINITY; l[j] = 0.0f;
#pragma unroll
    for (int d = 0; d < DPL; ++d) o[j][d] = 0.0f;
  }

  const int32_t* trow = a.table + (int64_t)b * a.max_blocks;
  const uint32_t* kplane = static_cast<const uint32_t*>(a.k);
  const uint32_t* vplane = static_cast<const uint32_t*>(a.v);
  const int grp = (sl * DPL) / 64;

  for (int base = t0 + wave * TILE; base < t1; base += NWAVES * TILE) {
    uint32_t kw[U][WPL], vw[U][WPL];
    float ksc[U], kbi[U], vsc[U], vbi[U];
    bool ok[U];
    int tok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = base + u * RPW + slot;
      ok[u] = t < t1;
      tok[u] = t;
      const int tq = ok[u] ? t : t0;
      const int blk = (a.bs_shift >= 0) ? (tq >> a.bs_shift) : (tq / a.BS);
      const int off = tq - blk * a.BS;
      int phys = trow[blk];
      phys = min(max(phys, 0), a.num_blocks - 1);       // a bad table entry cannot fault
      const int64_t prow = ((int64_t)phys * a.HK + hk) * a.BS + off;
      const uint32_t* kr = kplane + prow * WROW + sl * WPL;
      const uint32_t* vr = vplane + prow * WROW + sl * WPL;
      if constexpr (WPL == 4) {
        const uint4 x = *reinterpret_cast<const uint4*>(kr), y = *reinterpret_cast<const uint4*>(vr);
        kw[u][0] = x.x; kw[u][1] = x.y; kw[u][2] = x.z; kw[u][3] = x.w;
        vw[u][0] = y.x; vw[u][1] = y.y; vw[u][2] = y.z; vw[u][3] = y.w;
      } else if constexpr (WPL == 2) {
        const uint2 x = *reinterpret_cast<const uint2*>(kr), y = *reinterpret_cast<const uint2*>(vr);
        kw[u][0] = x.x; kw[u][1] = x.y; vw[u][0] = y.x; vw[u][1] = y.y;
      } else {
        kw[u][0] = kr[0]; vw[u][0] = vr[0];
      }
      if constexpr (BITS != 16) {
        const int64_t si = prow * G + grp;
        ksc[u] = bf16_to_f32(a.ks[si]); kbi[u] = bf16_to_f32(a.kb[si]);
        vsc[u] = bf16_to_f32(a.vs[si]); vbi[u] = bf16_to_f32(a.vb[si]);
      } else {
        ksc[u] = kbi[u] = vsc[u] = vbi[u] = 0.0f;
      }
    }

    // ---- scores
    float z[U][QVW];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint32_t pr[NP];
      key_pairs<BITS>(kw[u], pr);
      const float bb = (BITS == 16) ? 0.0f : fmaf(-F::OFFS, ksc[u], kbi[u]);
#pragma unroll
      for (int j = 0; j < QVW; ++j) {
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < NP; ++k) acc = dot2_bf16(qp[j][k], pr[k], acc);
        z[u][j] = (BITS == 16) ? acc : fmaf(ksc[u], acc, bb * qsum[j]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < QVW; ++j) {
        const float s = block_reduce<OpAdd, 1, LPR>(z[u][j]);
        z[u][j] = (ok[u] && tok[u] < vend[j]) ? s * a.scale_log2e : -INFINITY;
      }

    // ---- online softmax, one rescale per tile
#pragma unroll
    for (int j = 0; j < QVW; ++j) {
      float mt = z[0][j];
#pragma unroll
      for (int u = 1; u < U; ++u) mt = fmaxf(mt, z[u][j]);
      mt = block_reduce<OpMax, LPR, 64>(mt);
      const float mnew = fmaxf(m[j], mt);
      const float muse = (mnew == -INFINITY) ? 0.0f : mnew;
      const float alpha = fast_exp2(m[j] - muse);
      m[j] = mnew;
      float ls = l[j] * alpha;
#pragma unroll
      for (int d = 0; d < DPL; ++d) o[j][d] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) { const float e = fast_exp2(z[u][j] - muse); z[u][j] = e; ls += e; }
      l[j] = ls;
    }

    // ---- P.V with V dequantized in registers
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vv[DPL];
      value_f32<BITS>(vw[u], vsc[u], vbi[u], vv);
#pragma unroll
      for (int j = 0; j < QVW; ++j)
#pragma unroll
        for (int d = 0; d < DPL; ++d) o[j][d] = fmaf(z[u][j], vv[d], o[j][d]);
    }
  }

  // ---- combine the RPW token slots of the wave (same running max: plain sums)
#pragma unroll
  for (int j = 0; j < QVW; ++j) {
    l[j] = block_reduce<OpAdd, LPR, 64>(l[j]);
#pragma unroll
    for (int d = 0; d < DPL; ++d) {
      float x = o[j][d];
#pragma unroll
      for (int off = LPR; off < 64; off *= 2) x += shfl_xor_f(x, off);
      o[j][d] = x;
    }
  }

  // ---- combine the waves in LDS and write this partition's partial
  __shared__ float sm_o[NWAVES][QVW][D];
  __shared__ float sm_m[NWAVES][QVW], sm_l[NWAVES][QVW];
  if (slot == 0) {
#pragma unroll
    for (int j = 0; j < QVW; ++j)
#pragma unroll
      for (int d = 0; d < DPL; ++d) sm_o[wave][j][sl * DPL + d] = o[j][d];
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < QVW; ++j) { sm_m[wave][j] = m[j]; sm_l[wave][j] = l[j]; }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < QVW * D; e += NWAVES * 64) {
    const int j = e / D, d = e - j * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) M = fmaxf(M, sm_m[w][j]);
    float num = 0.0f, den = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NWAVES; ++w) {
        const float mw = sm_m[w][j];
        if (mw == -INFINITY) continue;
        const float f = fast_exp2(mw - M);
        num = fmaf(f, sm_o[w][j][d], num);
        den = fmaf(f, sm_l[w][j], den);
      }
    }
    const int jj = qg * QVW + j;
    const int h = hk * REP + jj / N, i = jj - (jj / N) * N;
    const int64_t idx = (((int64_t)b * a.HQ + h) * N + i) * a.num_parts + p;
    a.opart[idx * D + d] = num;
    if (d == 0) { a.ml[idx * 2] = M; a.ml[idx * 2 + 1] = den; }
  }
}

// ------------------------------------------------------------------------------ merge

__global__ void __launch_bounds__(256) merge_kernel(MergeArgs a) {
  extern __shared__ float sw[];                 // [num_parts] weights
  __shared__ float red[8];
  const int row = blockIdx.x;                   // (b, h, i)
  const int b = row / (a.HQ * a.N);
  const int len = min(a.lengths[b], a.max_len);
  const int nparts = len > 0 ? min((len + a.part_tokens - 1) / a.part_tokens, a.num_parts) : 0;
  const float* mlr = a.ml + (int64_t)row * a.num_parts * 2;
  const float* orow = a.opart + (int64_t)row * a.num_parts * a.D;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, nw = blockDim.x >> 6;

  float mx = -INFINITY;
  for (int p = tid; p < nparts; p += blockDim.x) mx = fmaxf(mx, mlr[2 * p]);
  mx = block_reduce<OpMax, 1, 64>(mx);
  if (lane == 0) red[wv] = mx;
  __syncthreads();
  float M = -INFINITY;
  for (int w = 0; w < nw; ++w) M = fmaxf(M, red[w]);
  __syncthreads();

  float den = 0.0f;
  for (int p = tid; p < nparts; p += blockDim.x) {
    const float mp = mlr[2 * p];
    const float w = (mp == -INFINITY || M == -INFINITY) ? 0.0f : fast_exp2(mp - M);
    sw[p] = w;
    den = fmaf(w, mlr[2 * p + 1], den);
  }
  den = block_reduce<OpAdd, 1, 64>(den);
  if (lane == 0) red[wv] = den;
  __syncthreads();
  float tot = 0.0f;
  for (int w = 0; w < nw; ++w) tot += red[w];

  for (int d = tid; d < a.D; d += blockDim.x) {
    float num = 0.0f;
    for (int p = 0; p < nparts; ++p) num = fmaf(sw[p], orow[(int64_t)p * a.D + d], num);
    const float r = (tot > 0.0f) ? num / tot : 0.0f;
    if (a.out_f32) static_cast<float*>(a.out)[(int64_t)row * a.D + d] = r;
    else static_cast<uint16_t*>(a.out)[(int64_t)row * a.D + d] = (uint16_t)f32_to_bf16_rne(r);
  }
}

// ------------------------------------------------------------------------------ launch

template <int BITS, int D, int QVW>
static hipError_t launch_one(const PartialArgs& a, int B, hipStream_t s) {
  constexpr int U = 4;
  dim3 grid((unsigned)a.num_parts, (unsigned)(a.HK * a.qgroups), (unsigned)B);
  hipLaunchKernelGGL((partial_kernel<BITS, D, QVW, U>), grid, dim3(NWAVES * 64), 0, s, a);
  return hipGetLastError();
}

template <int BITS, int D>
static hipError_t launch_d(const PartialArgs& a, int qvw, int B, hipStream_t s) {
  switch (qvw) {
    case 1: return launch_one<BITS, D, 1>(a, B, s);
    case 2: return launch_one<BITS, D, 2>(a, B, s);
    case 4: return launch_one<BITS, D, 4>(a, B, s);
    case 8: return launch_one<BITS, D, 8>(a, B, s);
    default: return hipErrorInvalidValue;
  }
}

template <int BITS>
static hipError_t launch_b(const PartialArgs& a, int D, int qvw, int B, hipStream_t s) {
  switch (D) {
    case 64: return launch_d<BITS, 64>(a, qvw, B, s);
    case 128: return launch_d<BITS, 128>(a, qvw, B, s);
    case 256: return launch_d<BITS, 256>(a, qvw, B, s);
    default: return hipErrorInvalidValue;
  }
}

bool partial_supported(int bits, int D, int qvw) {
  const bool b = bits == 16 || bits == 8 || bits == 4 || bits == 2;
  const bool d = D == 64 || D == 128 || D == 256;
  const bool q = qvw == 1 || qvw == 2 || qvw == 4 || qvw == 8;
  return b && d && q;
}

hipError_t launch_partial(const PartialArgs& a, int bits, int D, int qvw, int B, hipStream_t s) {
  switch (bits) {
    case 16: return launch_b<16>(a, D, qvw, B, s);
    case 8: return launch_b<8>(a, D, qvw, B, s);
    case 4: return launch_b<4>(a, D, qvw, B, s);
    case 2: return launch_b<2>(a, D, qvw, B, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_merge(const MergeArgs& a, int B, hipStream_t s) {
  const unsigned rows = (unsigned)(B * a.HQ * a.N);
  const size_t shm = (size_t)a.num_parts * sizeof(float);
  hipLaunchKernelGGL(merge_kernel, dim3(rows), dim3(256), shm, s, a);
  return hipGetLastError();
}

}  // namespace kvq
