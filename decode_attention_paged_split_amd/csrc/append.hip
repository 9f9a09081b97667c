// Quantize-on-append kernel: new K/V rows at caller-given slots -> pool planes.  The row
// arithmetic (quantizer reading, packing, mapping) is in append_rows.hpp.
#include "append_rows.hpp"

#include <algorithm>

namespace kvq {

template <int BITS, int GS>
__global__ void __launch_bounds__(256) append_quantize_kernel(AppendArgs a) {
  append_rows<BITS, GS>(a, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

template <int BITS>
static hipError_t launch_append_g(const AppendArgs& a, dim3 grid, hipStream_t stream) {
  if constexpr (BITS == 16) {
    hipLaunchKernelGGL((append_quantize_kernel<16, 64>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  switch (a.group) {
    case 32: hipLaunchKernelGGL((append_quantize_kernel<BITS, 32>), grid, dim3(256), 0, stream, a); break;
    case 64: hipLaunchKernelGGL((append_quantize_kernel<BITS, 64>), grid, dim3(256), 0, stream, a); break;
    case 128: hipLaunchKernelGGL((append_quantize_kernel<BITS, 128>), grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, int bits, hipStream_t stream) {
  const int ept = append_ept(bits);
  const int64_t total = (int64_t)a.T * a.HK * (std::max(a.D, a.Dv) / ept);
  if (total == 0) return hipSuccess;
  const int block = 256;
  const int64_t grid = (total + block - 1) / block;
  const dim3 g((unsigned)grid);
  switch (bits) {
    case 16: return launch_append_g<16>(a, g, stream);
    case 8: return launch_append_g<8>(a, g, stream);
    case 6: return launch_append_g<6>(a, g, stream);
    case 5: return launch_append_g<5>(a, g, stream);
    case 4: return launch_append_g<4>(a, g, stream);
    case 3: return launch_append_g<3>(a, g, stream);
    case 2: return launch_append_g<2>(a, g, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
