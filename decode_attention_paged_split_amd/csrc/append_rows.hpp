// Quantize-on-append of new K/V rows into the pool planes (device part, shared by the append
// kernel and the decode-step kernel).
//
// Follows "@mlx-bun/inference 0.0.0-stage -> 1.0.0", diff page 134 (src/state/paged/
// cache.ts): BlockPool.writeBlock quantizes each appended row per group of groupSize elements
// (PagedQuantization; 32, 64 or 128 here) along the head dim and slice-updates codes, scales and biases at [block, head, row];
// PagedKVCache.append maps each new token to (physical block, row).  The slot of a token is
// either the caller's (one int64 slot = block * block_size + row per token) or, for a decode
// step, the one its position takes in the block table: the N new rows of sequence b are
// positions lengths[b] - N + i (lengths count the new rows, as appendDecode appends before it
// attends).
//
// Quantizer (the pages call MLX's ops.quantize without showing it; this is the reading
// the library implements, bit for bit):
//   mn, mx = min, max of the group;  scale = bf16_round_up(f32(mx - mn) / (2^bits - 1));
//   bias = mn (a zero minimum stored as +0);
//   code = clamp(rint(f32(x - bias) / scale), 0, 2^bits - 1), rint = half to even,
//   code 0 everywhere when scale == 0.
// Division is IEEE round-to-nearest (__fdiv_rn), never a reciprocal approximation, so
// codes match any correctly rounded f32 implementation exactly.
//
// Packing: a row's codes form one little-endian bit stream, code i in bits [bits * i, bits * i +
// bits) (the pages' low-first rule; 3-, 5- and 6-bit codes straddle words).
// Mapping: one thread per EPT consecutive elements of one (token, head) row (EPT = 8, 16 at 2
// bits and 32 at 3, 5 and 6 bits, so that a thread owns whole words); the GS/EPT threads of a
// group are adjacent lanes and reduce min/max with DPP.  Loads are 16-byte, coalesced along
// the row.
#pragma once

#include "device_common.hpp"
#include "kernels.hpp"

namespace kvq {

constexpr int append_ept(int bits) { return bits == 2 ? 16 : (32 % bits != 0 ? 32 : 8); }

// slot of new row tok = b * N + i of a decode step: position lengths[b] - N + i looked up in the
// block table; -1 (skipped) when the position is outside [0, capacity) or the entry is outside the pool
__device__ __forceinline__ int64_t decode_slot(const AppendArgs& a, int64_t tok) {
  const int b = (int)(tok / a.N), i = (int)(tok - (int64_t)b * a.N);
  const int t = a.lengths[b] - a.N + i;
  if (t < 0 || t >= a.len_cap) return -1;
  const int phys = a.table[(int64_t)b * a.max_blocks + t / a.BS];
  if (phys < 0 || (int64_t)phys * a.BS >= a.num_slots) return -1;
  return (int64_t)phys * a.BS + t % a.BS;
}

// one thread per EPT elements of one (token, head) row; gid indexes (token, head, chunk) with
// chunks over the wider of the K row (D) and the V row (Dv); GS is the scale-group size (affine
// pages; bf16 rows ignore it)
template <int BITS, int GS>
__device__ __forceinline__ void append_rows(const AppendArgs& a, int64_t gid) {
  constexpr int EPT = append_ept(BITS);         // elements per thread
  constexpr int TPG = GS / EPT;                 // threads per scale group
  const int chunks = max(a.D, a.Dv) / EPT;
  const int64_t total = (int64_t)a.T * a.HK * chunks;
  const bool live = gid < total;
  const int64_t g = live ? gid : 0;
  const int chunk = (int)(g % chunks);
  const int64_t row = g / chunks;               // token * HK + head
  const int head = (int)(row % a.HK);
  const int64_t tok = row / a.HK;

  const int64_t slot = a.slots ? a.slots[tok] : (live ? decode_slot(a, tok) : -1);
  const bool store = live && slot >= 0 && slot < a.num_slots;
  const int64_t phys = store ? slot / a.BS : 0;
  const int off = store ? (int)(slot % a.BS) : 0;
  const int64_t prow = (phys * a.HK + head) * a.BS + off;   // row index within a plane

  // the K and V chunks are loaded before anything is stored (the stores may alias the sources
  // as far as the compiler knows, so loads after a store would wait for it); a row's width is D
  // for K and Dv for V, and chunks beyond it (the narrower row's) are whole scale groups that
  // load and store nothing
  uint32_t src_w[2][EPT / 2];
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    const int dk = kv ? a.Dv : a.D;
    const bool on = live && chunk * EPT < dk;
    const uint4* s4 = reinterpret_cast<const uint4*>((kv ? a.v : a.k) + row * dk + chunk * EPT);
#pragma unroll
    for (int q = 0; q < EPT / 8; ++q) {
      const uint4 x = on ? s4[q] : make_uint4(0, 0, 0, 0);
      src_w[kv][4 * q] = x.x; src_w[kv][4 * q + 1] = x.y; src_w[kv][4 * q + 2] = x.z; src_w[kv][4 * q + 3] = x.w;
    }
  }

#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    const int dk = kv ? a.Dv : a.D;
    const bool on = live && chunk * EPT < dk;
    const bool put = store && on;
    const uint32_t* w = src_w[kv];
    if constexpr (BITS == 16) {
      if (put) {
        uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(kv ? a.v_plane : a.k_plane) +
                                              prow * dk + chunk * EPT);
        dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
      }
      continue;
    } else {
      float x[EPT];
#pragma unroll
      for (int i = 0; i < EPT / 2; ++i) { x[2 * i] = bf16_lo(w[i]); x[2 * i + 1] = bf16_hi(w[i]); }
      float mn = x[0], mx = x[0];
#pragma unroll
      for (int i = 1; i < EPT; ++i) { mn = fminf(mn, x[i]); mx = fmaxf(mx, x[i]); }
      // the TPG adjacent lanes of this group (aligned: chunks per row is a multiple of TPG)
      mn = -block_reduce<OpMax, 1, TPG>(-mn);
      mx = block_reduce<OpMax, 1, TPG>(mx);
      constexpr float NLEV = (float)((1 << BITS) - 1);
      const float s32 = __fdiv_rn(mx - mn, NLEV);
      const uint32_t sbits = f32_to_bf16_up(s32);
      const float scale = bf16_to_f32(sbits);
      const uint32_t mnbits = __float_as_uint(mn);
      const uint32_t bbits = (mnbits == 0x80000000u) ? 0u : (mnbits >> 16);   // exact (bf16 input)
      const float bias = bf16_to_f32(bbits);
      uint32_t c[EPT];
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        float q = 0.0f;
        if (scale > 0.0f) q = rintf(__fdiv_rn(x[i] - bias, scale));
        q = fminf(fmaxf(q, 0.0f), NLEV);
        c[i] = (uint32_t)q;
      }
      // the thread's codes as its stretch of the row's bit stream (EPT * BITS bits, whole words)
      constexpr int NWORDS = EPT * BITS / 32;
      uint32_t out[NWORDS];
#pragma unroll
      for (int j = 0; j < NWORDS; ++j) out[j] = 0;
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        const int o = BITS * i, wj = o >> 5, sh = o & 31;
        out[wj] |= c[i] << sh;
        if (sh + BITS > 32) out[wj + 1] |= c[i] >> (32 - sh);   // a code straddling two words
      }
      if (put) {
        const int W = dk * BITS / 32;
        uint32_t* dst = static_cast<uint32_t*>(kv ? a.v_plane : a.k_plane) + prow * W + chunk * NWORDS;
#pragma unroll
        for (int j = 0; j < NWORDS; ++j) dst[j] = out[j];
        if ((chunk % TPG) == 0) {
          const int G = dk / GS;
          const int grp = chunk / TPG;
          uint16_t* sp = static_cast<uint16_t*>(kv ? a.v_scale : a.k_scale);
          uint16_t* bp = static_cast<uint16_t*>(kv ? a.v_bias : a.k_bias);
          sp[prow * G + grp] = (uint16_t)sbits;
          bp[prow * G + grp] = (uint16_t)bbits;
        }
      }
    }
  }
}


}  // namespace kvq
