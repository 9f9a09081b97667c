// Vector-engine kernels for 2-bit pages (one translation unit per page format keeps the build parallel).
#include "partial_valu_impl.hpp"

namespace kvq {
template hipError_t launch_valu_bits<2>(const PartialArgs&, int, int, int, int, int, bool, hipStream_t);
template hipError_t launch_step_bits<2>(const AppendArgs&, const PartialArgs&, int, int, int, bool, int, hipStream_t);
}  // namespace kvq
