// Quantize-on-append kernel: new K/V rows at caller-given slots -> pool planes.  The row
// arithmetic (quantizer reading, packing, mapping) is in append_rows.hpp.
#include "append_rows.hpp"

namespace kvq {

template <int BITS>
__global__ void __launch_bounds__(256) append_quantize_kernel(AppendArgs a) {
  append_rows<BITS>(a, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

hipError_t launch_append(const AppendArgs& a, int bits, hipStream_t stream) {
  const int ept = append_ept(bits);
  const int64_t total = (int64_t)a.T * a.HK * (a.D / ept);
  if (total == 0) return hipSuccess;
  const int block = 256;
  const int64_t grid = (total + block - 1) / block;
  switch (bits) {
    case 16: hipLaunchKernelGGL(append_quantize_kernel<16>, dim3((unsigned)grid), dim3(block), 0, stream, a); break;
    case 8:  hipLaunchKernelGGL(append_quantize_kernel<8>,  dim3((unsigned)grid), dim3(block), 0, stream, a); break;
    case 4:  hipLaunchKernelGGL(append_quantize_kernel<4>,  dim3((unsigned)grid), dim3(block), 0, stream, a); break;
    case 2:  hipLaunchKernelGGL(append_quantize_kernel<2>,  dim3((unsigned)grid), dim3(block), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
