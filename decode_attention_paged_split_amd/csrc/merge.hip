// Log-sum-exp merge of the split-K partials.
//
// "@mlx-bun/inference 0.0.0-stage -> 1.0.0", diff page 50: paged.ts paged_attention_merge and
// kvq4-decode.ts (merge kernel): for each (sequence, query head, row) with partials
// (o_p, m_p, l_p) over partitions p, out = sum_p e^(m_p - M) o_p / sum_p e^(m_p - M) l_p with
// M = max_p m_p; partitions whose max is -inf (no visible token) are skipped.  Maxima are in
// log2 units here (the partial kernel scales scores by log2(e)), so the weights are exp2.
// One workgroup per output row: the partition weights are computed once into LDS, then each
// thread accumulates four head dims over a stride of the partials (several loads in flight per
// thread) and the strides' sums are added in LDS.  Output is bf16 (round to nearest even) or f32.
// Stream schedule: the stream of T tokens is cut into R = min(num_ranges, ceil(T / min_tokens))
// ranges; a unit's partials sit in range_sub consecutive slots per range it meets, from slot
// (unit + first range) * range_sub on.
#include "device_common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace kvq {

// ------------------------------------------------------------------------------ merge

__global__ void __launch_bounds__(256) merge_kernel(MergeArgs a) {
  extern __shared__ float sw[];                 // partition weights
  __shared__ float red[8];
  __shared__ long long red64[2][8];
  const int row = blockIdx.x;                   // (b, h, i)
  const int b = row / (a.HQ * a.N);
  const int hi_ = row - b * (a.HQ * a.N);
  const int h = hi_ / a.N, i = hi_ - h * a.N;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, nw = blockDim.x >> 6;
  const int len = max(0, min(a.lengths[b], a.len_cap));

  // where partition p of this row lives
  int nparts = 0;
  int64_t mbase = 0, obase = 0, mstride = 2, ostride = a.D;
  if (a.part_tokens > 0) {
    nparts = len > 0 ? min((len + a.part_tokens - 1) / a.part_tokens, a.num_parts) : 0;
    mbase = (int64_t)row * a.num_parts * 2;
    obase = (int64_t)row * a.num_parts * a.D;
  } else {
    // stream: tokens of all sequences before b, and of all sequences
    long long pre = 0, tot = 0;
    for (int bb = tid; bb < a.batch; bb += blockDim.x) {
      const long long l = max(0, min(a.lengths[bb], a.len_cap));
      tot += l;
      if (bb < b) pre += l;
    }
#pragma unroll
    for (int off = 32; off >= 1; off /= 2) {
      pre += __shfl_xor(pre, off, 64);
      tot += __shfl_xor(tot, off, 64);
    }
    if (lane == 0) { red64[0][wv] = pre; red64[1][wv] = tot; }
    __syncthreads();
    pre = 0; tot = 0;
    for (int w = 0; w < nw; ++w) { pre += red64[0][w]; tot += red64[1][w]; }
    const int HQG = a.HK * a.qgroups;
    const int64_t T = (int64_t)tot * HQG;
    const int64_t weff = min<int64_t>((int64_t)a.num_ranges, (T + a.min_tokens - 1) / a.min_tokens);
    const int REP = a.HQ / a.HK;
    const int hk = h / REP;
    const int jj = (h - hk * REP) * a.N + i;
    const int qg = jj / a.qvw, j = jj - qg * a.qvw;
    const int64_t u = (int64_t)b * HQG + hk * a.qgroups + qg;
    if (len > 0 && weff > 0) {
      const int64_t start = (int64_t)pre * HQG + (int64_t)(hk * a.qgroups + qg) * len;
      const int64_t end = start + len;
      const int64_t w_first = start * weff / T, w_last = (end - 1) * weff / T;
      nparts = (int)(w_last - w_first + 1) * a.range_sub;
      const int64_t slot0 = (u + w_first) * a.range_sub;
      mbase = (slot0 * a.qvw + j) * 2;
      obase = (slot0 * a.qvw + j) * a.D;
      mstride = (int64_t)a.qvw * 2;
      ostride = (int64_t)a.qvw * a.D;
    }
  }

  float mx = -INFINITY;
  for (int p = tid; p < nparts; p += blockDim.x) mx = fmaxf(mx, a.ml[mbase + p * mstride]);
  mx = block_reduce<OpMax, 1, 64>(mx);
  if (lane == 0) red[wv] = mx;
  __syncthreads();
  float M = -INFINITY;
  for (int w = 0; w < nw; ++w) M = fmaxf(M, red[w]);
  __syncthreads();

  float den = 0.0f;
  for (int p = tid; p < nparts; p += blockDim.x) {
    const float mp = a.ml[mbase + p * mstride];
    const float w = (mp == -INFINITY || M == -INFINITY) ? 0.0f : fast_exp2(mp - M);
    sw[p] = w;
    den = fmaf(w, a.ml[mbase + p * mstride + 1], den);
  }
  den = block_reduce<OpAdd, 1, 64>(den);
  if (lane == 0) red[wv] = den;
  __syncthreads();
  float tot = 0.0f;
  for (int w = 0; w < nw; ++w) tot += red[w];

  // weighted sum of the partials: thread (stream s, dim lane dl) owns dims 4 dl .. 4 dl + 3 and
  // partials s, s + S, ...; the S streams' sums are added in LDS
  const int DL = a.D / 4, S = blockDim.x / DL;
  const int dl = tid % DL, sidx = tid / DL;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (sidx < S) {
    const float* ob = a.opart + obase + 4 * dl;
#pragma unroll 4
    for (int p = sidx; p < nparts; p += S) {
      const float wp = sw[p];
      if (wp != 0.0f) {                                  // (a skipped partial's o is never read)
        const float4 o = *reinterpret_cast<const float4*>(ob + p * ostride);
        acc.x = fmaf(wp, o.x, acc.x); acc.y = fmaf(wp, o.y, acc.y);
        acc.z = fmaf(wp, o.z, acc.z); acc.w = fmaf(wp, o.w, acc.w);
      }
    }
  }
  __syncthreads();                                       // sw is reused for the stream sums
  float4* part = reinterpret_cast<float4*>(sw);
  if (sidx < S) part[sidx * DL + dl] = acc;
  __syncthreads();
  if (tid < DL) {
    float4 r = part[tid];
    for (int k = 1; k < S; ++k) {
      const float4 x = part[k * DL + tid];
      r.x += x.x; r.y += x.y; r.z += x.z; r.w += x.w;
    }
    const float v[4] = {r.x, r.y, r.z, r.w};
    for (int k = 0; k < 4; ++k) {
      const float y = (tot > 0.0f) ? v[k] / tot : 0.0f;
      const int64_t oi = (int64_t)row * a.D + 4 * tid + k;
      if (a.out_f32) static_cast<float*>(a.out)[oi] = y;
      else static_cast<uint16_t*>(a.out)[oi] = (uint16_t)f32_to_bf16_rne(y);
    }
  }
}

hipError_t launch_merge(const MergeArgs& a, int B, hipStream_t s) {
  const unsigned rows = (unsigned)(B * a.HQ * a.N);
  const int most = a.part_tokens > 0 ? a.num_parts : (a.num_ranges + 1) * a.range_sub;
  // partition weights, then the 256 threads' float4 sums
  const size_t shm = (size_t)std::max(most, 256 * 4) * sizeof(float);
  hipLaunchKernelGGL(merge_kernel, dim3(rows), dim3(256), shm, s, a);
  return hipGetLastError();
}

}  // namespace kvq
