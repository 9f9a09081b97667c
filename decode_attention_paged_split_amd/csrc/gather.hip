// The fetch copy through the block table, for indexing tests.
//
// "@mlx-bun/inference 0.0.0-stage -> 1.0.0", diff page 134 (src/state/paged/cache.ts,
// pickBlocks and BlockPool.gather): a sequence's blocks taken in logical order and laid
// out as [H, blocks * blockSize, width], cut to the cached length.  Here every plane of a
// batch goes to [B, HK, max_len, width]; rows at t >= length are zero.  Copies 16-bit
// units (every plane row is a whole number of them).
#include "device_common.hpp"
#include "kernels.hpp"

namespace kvq {

__global__ void __launch_bounds__(256) gather_plane_kernel(GatherArgs a) {
  const int units = a.row_bytes / 2;
  const int64_t total = (int64_t)a.B * a.HK * a.max_len * units;
  const uint16_t* src = reinterpret_cast<const uint16_t*>(a.plane);
  uint16_t* dst = reinterpret_cast<uint16_t*>(a.out);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int u = (int)(i % units);
    int64_t r = i / units;
    const int t = (int)(r % a.max_len);
    r /= a.max_len;
    const int h = (int)(r % a.HK);
    const int b = (int)(r / a.HK);
    uint16_t val = 0;
    const int blk = t / a.BS;
    if (t < a.lengths[b] && blk < a.max_blocks) {
      const int64_t phys = a.table[(int64_t)b * a.max_blocks + blk];
      if (phys >= 0 && phys < a.num_blocks) {       // an out-of-range entry reads as zero
        const int64_t prow = (phys * a.HK + h) * a.BS + (t % a.BS);
        val = src[prow * units + u];
      }
    }
    dst[i] = val;
  }
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t stream) {
  const int64_t total = (int64_t)a.B * a.HK * a.max_len * (a.row_bytes / 2);
  if (total == 0) return hipSuccess;
  int64_t grid = (total + 255) / 256;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(gather_plane_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
