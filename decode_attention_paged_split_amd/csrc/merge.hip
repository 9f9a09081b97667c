// Log-sum-exp merge of the split-K partials.
//
// "@mlx-bun/inference 0.0.0-stage -> 1.0.0", diff page 50: paged.ts paged_attention_merge and
// kvq4-decode.ts (merge kernel): for each (sequence, query head, row) with partials
// (o_p, m_p, l_p) over partitions p, out = sum_p e^(m_p - M) o_p / sum_p e^(m_p - M) l_p with
// M = max_p m_p; partitions whose max is -inf (no visible token) are skipped.  Maxima are in
// log2 units here (the partial kernel scales scores by log2(e)), so the weights are exp2.
// One workgroup per output row, one pass over the partials: thread (stream s, dim lane dl) owns
// head dims 4 dl .. 4 dl + 3 and partials s, s + S, ... (S = threads / (D / 4); the host sizes
// the workgroup, 64 to 256 threads, for about five partials per stream); it loads each
// partial's (m, l) and o together and folds them into a running (max, sum of weights, weighted
// o) (the weights are rescaled when the max moves), and the S streams' states are combined in
// LDS the same way.
// Output is bf16 (round to nearest even) or f32.
// Stream schedule: the stream of T set positions (a set: `lanes` consecutive query groups of one KV
// head, worked side by side; each set with tokens takes set_cost positions, then one per token) is
// cut into R = min(num_ranges, ceil(T / min_tokens)) ranges; per range it meets, a group owns
// range_sub consecutive slots from ((set + range) * lanes + lane) * range_sub on -- or
// (stream_combined) the first of them only, for every range in which the set is the last with
// tokens (its waves combined their partials).
#include "device_common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace kvq {

// ------------------------------------------------------------------------------ merge

template <int NT>
__global__ void __launch_bounds__(NT) merge_kernel(MergeArgs a) {
  extern __shared__ float sw[];                 // the streams' partial states
  const int row = blockIdx.x;                   // (b, h, i)
  const int b = row / (a.HQ * a.N);
  const int hi_ = row - b * (a.HQ * a.N);
  const int h = hi_ / a.N, i = hi_ - h * a.N;
  const int tid = threadIdx.x, lane = tid & 63;
  const int len = max(0, min(a.lengths[b], a.len_cap));

  // where partition p of this row lives: fixed partitions at mbase + p * mstride (and obase +
  // p * ostride); stream slots from slot0 on, one per (range, wave), except that (combined) the
  // ranges before the last one the unit meets hold one partial each and so may the last one
  int nparts = 0, nr = 0;
  int64_t mbase = 0, obase = 0, mstride = 2, ostride = a.D, slot0 = 0, slot_last = 0;
  int64_t rstride = 0;                                          // stream: slots between ranges
  bool by_slot = false;
  if (a.part_tokens > 0) {
    nparts = len > 0 ? min((len + a.part_tokens - 1) / a.part_tokens, a.num_parts) : 0;
    mbase = (int64_t)row * a.num_parts * 2;
    obase = (int64_t)row * a.num_parts * a.D;
  } else {
    // sets: L = a.lanes consecutive query groups of one KV head, worked side by side (one
    // workgroup each) on one range
    const int L = a.lanes, QGB = a.qgroups / L, HS = a.HK * QGB;
    // the stream's length, ranges and set cost in force, as the partial kernel computes them;
    // then the positions of the sequences before b (each wave sums them itself): per set with
    // tokens, C and then its tokens
    const StreamSpan sp = stream_span(a.lengths, a.batch, a.len_cap, HS, a.num_ranges, a.min_tokens,
                                      a.set_cost, lane);
    const int C = sp.C;
    long long pre = 0;
    for (int c = 0; c < b; c += 64) {
      const int bb = c + lane;
      const int l = bb < b ? max(0, min(a.lengths[bb], a.len_cap)) : 0;
      pre += (long long)wave_sum_u64(l > 0 ? (uint32_t)l + (uint32_t)C : 0u);
    }
    const int64_t T = sp.T;
    const int64_t weff = sp.R;
    const int REP = a.HQ / a.HK;
    const int hk = h / REP;
    const int jj = (h - hk * REP) * a.N + i;
    const int qg = jj / a.qvw, j = jj - qg * a.qvw;
    const int sq = hk * QGB + qg / L;                            // set within the sequence
    const int ln = qg - (qg / L) * L;                            // the group's lane in its set
    rstride = (int64_t)L * a.range_sub;                          // slots between a lane's ranges
    const int64_t u = (int64_t)b * HS + sq;
    if (len > 0 && weff > 0) {
      // the set's tokens sit at positions [first, end), after its C positions
      const int64_t first = (int64_t)pre * HS + (int64_t)sq * ((int64_t)len + C) + C;
      const int64_t end = first + len;
      const int64_t w_first = first * weff / T, w_last = (end - 1) * weff / T;
      if (a.stream_combined) {
        // a range in which the set is the last with tokens combined each lane's partials into one:
        // every range before the last, and the last too unless the next set's first token (C
        // positions after end) lies inside it
        const int64_t x1_last = ((w_last + 1) * T + weff - 1) / weff;
        nr = (int)(w_last - w_first);
        nparts = nr + (x1_last <= end + C ? 1 : a.range_sub);
      } else {
        nparts = (int)(w_last - w_first + 1) * a.range_sub;
      }
      slot0 = ((u + w_first) * L + ln) * a.range_sub;
      slot_last = ((u + w_last) * L + ln) * a.range_sub;
      by_slot = true;
      mbase = j * 2;
      obase = (int64_t)j * a.D;
      mstride = (int64_t)a.qvw * 2;
      ostride = (int64_t)a.qvw * a.D;
    }
  }

  // one pass: running (max m, weight sum den, weighted o acc) per thread over its partials
  const int DL = a.D / 4, S = blockDim.x / DL;
  const int dl = tid % DL, sidx = tid / DL;
  float m_run = -INFINITY, den = 0.0f;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (sidx < S) {
    const float* ob = a.opart + obase + 4 * dl;
    const float* mb = a.ml + mbase;
#pragma unroll 4
    for (int p = sidx; p < nparts; p += S) {
      int64_t q = p;                                           // slot (stream) or partition
      if (by_slot) {
        if (!a.stream_combined) {
          const int r = p / a.range_sub;
          q = slot0 + r * rstride + (p - r * a.range_sub);
        } else {
          q = p < nr ? slot0 + p * rstride : slot_last + (p - nr);
        }
      }
      const float2 ml = *reinterpret_cast<const float2*>(mb + q * mstride);
      const float4 o = *reinterpret_cast<const float4*>(ob + q * ostride);
      // branch-free, so every load is issued ahead of the arithmetic; a skipped partial
      // (m = -inf) contributes through selects only, so its unwritten l and o are never used
      const bool ok = ml.x != -INFINITY;
      const float mnew = ok ? fmaxf(m_run, ml.x) : m_run;
      const float sc = (mnew == -INFINITY) ? 1.0f : fast_exp2(m_run - mnew);
      const float wp = ok ? fast_exp2(ml.x - mnew) : 0.0f;
      m_run = mnew;
      den = fmaf(den, sc, ok ? wp * ml.y : 0.0f);
      acc.x = fmaf(acc.x, sc, ok ? wp * o.x : 0.0f); acc.y = fmaf(acc.y, sc, ok ? wp * o.y : 0.0f);
      acc.z = fmaf(acc.z, sc, ok ? wp * o.z : 0.0f); acc.w = fmaf(acc.w, sc, ok ? wp * o.w : 0.0f);
    }
  }
  // the streams' states meet in LDS: [stream][dim lane] float4 acc, then (m, den) per stream
  float4* part = reinterpret_cast<float4*>(sw);
  float2* mden = reinterpret_cast<float2*>(sw + 4 * S * DL);
  if (sidx < S) {
    part[sidx * DL + dl] = acc;
    if (dl == 0) mden[sidx] = make_float2(m_run, den);
  }
  __syncthreads();
  if (tid < DL) {
    float M = -INFINITY;
    for (int k = 0; k < S; ++k) M = fmaxf(M, mden[k].x);
    float4 r = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float tot = 0.0f;
    for (int k = 0; k < S; ++k) {
      const float2 md = mden[k];
      if (md.x == -INFINITY) continue;
      const float w = fast_exp2(md.x - M);
      const float4 x = part[k * DL + tid];
      tot = fmaf(w, md.y, tot);
      r.x = fmaf(w, x.x, r.x); r.y = fmaf(w, x.y, r.y); r.z = fmaf(w, x.z, r.z); r.w = fmaf(w, x.w, r.w);
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

template <int NT>
static hipError_t launch_merge_nt(const MergeArgs& a, unsigned rows, hipStream_t s) {
  // the threads' float4 sums and each stream's (max, weight sum)
  const size_t shm = (size_t)(NT * 4 + 2 * NT) * sizeof(float);
  hipLaunchKernelGGL(merge_kernel<NT>, dim3(rows), dim3(NT), shm, s, a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, int B, int threads, hipStream_t s) {
  const unsigned rows = (unsigned)(B * a.HQ * a.N);
  switch (threads) {
    case 64: return launch_merge_nt<64>(a, rows, s);
    case 128: return launch_merge_nt<128>(a, rows, s);
    case 256: return launch_merge_nt<256>(a, rows, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
