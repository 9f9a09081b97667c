// Device helpers shared by the kvq kernels (gfx950, wave64).
//
// bf16 handling, the round-up conversion used for affine scales, and cross-lane
// reductions built from DPP row controls and the gfx950 permlane swaps (no LDS traffic).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

// ---------------------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
// low / high bf16 of a packed pair, widened exactly
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// f32 -> bf16, round to nearest, ties to even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// smallest bf16 >= x (finite x >= 0 in our use; negative handled for completeness)
__device__ __forceinline__ uint32_t f32_to_bf16_up(float x) {
  uint32_t r = f32_to_bf16_rne(x);
  if (bf16_to_f32(r) < x) {
    if ((r & 0x7FFFu) == 0u) r = 1u;           // +-0 -> smallest positive subnormal
    else if (r & 0x8000u) r -= 1u;             // negative: toward zero
    else r += 1u;
  }
  return r;
}

// ---------------------------------------------------------------------------- lanes

// DPP controls (gfx9 encoding)
enum : int {
  DPP_QUAD_1032 = 0xB1,      // quad_perm [1,0,3,2]  (lane ^ 1)
  DPP_QUAD_2301 = 0x4E,      // quad_perm [2,3,0,1]  (lane ^ 2)
  DPP_ROW_MIRROR = 0x140,    // lane i <- 15 - i within a row of 16
  DPP_ROW_HALF_MIRROR = 0x141, // lane i <- 7 - i within each half row of 8
  DPP_ROW_ROR8 = 0x128       // row_ror:8: lane i <- lane (i + 8) % 16 within a row (lane ^ 8)
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

struct OpAdd { __device__ static float f(float a, float b) { return a + b; } };
struct OpMax { __device__ static float f(float a, float b) { return fmaxf(a, b); } };

// One butterfly step at lane distance OFF (a power of two <= 32), combining every lane
// with a lane of the neighbouring aligned block of OFF lanes.  Steps must be taken in
// increasing OFF starting from a block size over which the values are already uniform
// (distance 1 and 2 are exact xor swaps; 4 and 8 use the mirror controls, which pick
// some lane of the other block -- equal to the xor partner once blocks are uniform).
template <class OP, int OFF>
__device__ __forceinline__ float xstep(float x) {
  if constexpr (OFF == 1) {
    return OP::f(x, dpp<DPP_QUAD_1032>(x));
  } else if constexpr (OFF == 2) {
    return OP::f(x, dpp<DPP_QUAD_2301>(x));
  } else if constexpr (OFF == 4) {
    return OP::f(x, dpp<DPP_ROW_HALF_MIRROR>(x));
  } else if constexpr (OFF == 8) {
    return OP::f(x, dpp<DPP_ROW_MIRROR>(x));
  } else if constexpr (OFF == 16) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return OP::f(__uint_as_float(r[0]), __uint_as_float(r[1]));
  } else {
    static_assert(OFF == 32, "lane distance");
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return OP::f(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
}

// Integer forms over all 64 lanes, for the stream's lengths: an all-reduce (every lane ends with
// the result) and an inclusive prefix sum (row shifts 1, 2, 4, 8 within each row of 16, then the
// row broadcasts of lanes 15 and 31), both on DPP and the permlane swaps.  Sums of values below
// 2^32 go through two 32-bit halves (16 bits and the rest), each summing exactly over 64 lanes.
struct OpAddU { __device__ static uint32_t f(uint32_t a, uint32_t b) { return a + b; } };
struct OpMinU { __device__ static uint32_t f(uint32_t a, uint32_t b) { return a < b ? a : b; } };
struct OpMaxU { __device__ static uint32_t f(uint32_t a, uint32_t b) { return a > b ? a : b; } };
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
template <class OP>
__device__ __forceinline__ uint32_t wave_all_u32(uint32_t x) {
  x = OP::f(x, dpp_u32<DPP_QUAD_1032>(x));
  x = OP::f(x, dpp_u32<DPP_QUAD_2301>(x));
  x = OP::f(x, dpp_u32<DPP_ROW_HALF_MIRROR>(x));
  x = OP::f(x, dpp_u32<DPP_ROW_MIRROR>(x));
  {
    auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = OP::f(r[0], r[1]);
  }
  auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return OP::f(r[0], r[1]);
}
__device__ __forceinline__ uint64_t wave_sum_u64(uint32_t x) {
  const uint32_t lo = wave_all_u32<OpAddU>(x & 0xFFFFu), hi = wave_all_u32<OpAddU>(x >> 16);
  return ((uint64_t)hi << 16) + lo;
}
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);   // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}
__device__ __forceinline__ uint64_t wave_scan_u64(uint32_t x) {
  const uint32_t lo = wave_scan_u32(x & 0xFFFFu), hi = wave_scan_u32(x >> 16);
  return ((uint64_t)hi << 16) + lo;
}
// lane k's value of a 64-bit x, k uniform
__device__ __forceinline__ uint64_t lane_u64(uint64_t x, int k) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, k);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), k);
  return ((uint64_t)hi << 32) | lo;
}

// All-reduce over the 8 lanes i, i ^ 8, i ^ 16, ..., i ^ 56 (every lane's value may differ):
// exact xor steps at distances 8, 16 and 32.
template <class OP>
__device__ __forceinline__ float xor8_reduce(float x) {
  x = OP::f(x, dpp<DPP_ROW_ROR8>(x));
  x = xstep<OP, 16>(x);
  return xstep<OP, 32>(x);
}

// All-reduce over aligned blocks of HI lanes, assuming values are uniform over aligned
// blocks of LO lanes (LO, HI powers of two, 1 <= LO <= HI <= 64).  Every lane of a block
// ends with the block's result.
template <class OP, int LO, int HI>
__device__ __forceinline__ float block_reduce(float x) {
  if constexpr (LO < HI) {
    x = xstep<OP, LO>(x);
    return block_reduce<OP, LO * 2, HI>(x);
  } else {
    return x;
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Stream schedule: its length T in positions, the number R of working ranges and the set cost C in
// force.  A set (a KV head's query groups worked together) of a sequence with tokens takes C
// positions and then one per token.  C is the requested cost unless every range would hold the
// same number of set changes anyway -- all sequences with tokens equally long, and the number of
// sets S and the uncharged range count R0 dividing one another: then the set starts fall on
// range boundaries (or every range holds S / R0 whole sets) and C is 0.  Every wave computes the
// same, from the lengths clamped to [0, len_cap].
struct StreamSpan {
  int64_t T;
  int R, C;
};
__device__ __forceinline__ StreamSpan stream_span(const int32_t* lengths, int B, int len_cap, int HS,
                                                  int num_ranges, int min_tokens, int set_cost, int lane) {
  uint64_t tok = 0;
  uint32_t nz = 0, lmin = 0x7fffffffu, lmax = 0;
  for (int c = 0; c < B; c += 64) {
    const int bb = c + lane;
    const uint32_t l = bb < B ? (uint32_t)max(0, min(lengths[bb], len_cap)) : 0u;
    tok += wave_sum_u64(l);
    nz += wave_all_u32<OpAddU>(l > 0 ? 1u : 0u);
    lmin = min(lmin, wave_all_u32<OpMinU>(l > 0 ? l : 0x7fffffffu));
    lmax = max(lmax, wave_all_u32<OpMaxU>(l));
  }
  {                                     // every lane holds the results; take them as scalars
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)tok);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(tok >> 32));
    tok = ((uint64_t)hi << 32) | lo;
  }
  nz = (uint32_t)__builtin_amdgcn_readfirstlane((int)nz);
  lmin = (uint32_t)__builtin_amdgcn_readfirstlane((int)lmin);
  lmax = (uint32_t)__builtin_amdgcn_readfirstlane((int)lmax);
  const int64_t T0 = (int64_t)tok * HS, S = (int64_t)nz * HS;
  const int R0 = (int)min<int64_t>((int64_t)num_ranges, (T0 + min_tokens - 1) / min_tokens);
  int C = set_cost;
  if (S > 0 && R0 > 0 && lmin == lmax && (R0 % S == 0 || S % R0 == 0)) C = 0;
  StreamSpan r;
  r.C = C;
  r.T = T0 + S * C;
  r.R = (int)min<int64_t>((int64_t)num_ranges, (r.T + min_tokens - 1) / min_tokens);
  return r;
}

// Range w and lane ln of workgroup i of nwg on the balanced stream when the L query groups of a set
// (one KV head's L consecutive groups) run side by side, one workgroup each, over the same range:
// workgroups are handed to the 8 XCDs (each with its own L2) in turn by index, so the L workgroups
// of a range are taken 8 indices apart (one XCD) and an XCD's ranges are consecutive.  L = 1: w = i.
__device__ __forceinline__ void stream_range_lane(int L, int i, int nwg, int& w, int& ln) {
  if (L > 1 && nwg % (8 * L) == 0) {
    const int q = i >> 3;
    ln = q % L;
    w = (i & 7) * (nwg / (8 * L)) + q / L;
  } else {
    ln = i % L;
    w = i / L;
  }
}

}  // namespace kvq
