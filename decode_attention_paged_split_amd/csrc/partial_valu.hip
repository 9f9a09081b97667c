// Vector-engine launch by page format (the kernels: partial_valu_impl.hpp).
#include "kernels.hpp"

namespace kvq {

template <int BITS>
hipError_t launch_valu_bits(const PartialArgs& a, int D, int DV, int gs, int qvw, int B, bool q_ready, hipStream_t s);
template <int BITS>
hipError_t launch_step_bits(const AppendArgs& ap, const PartialArgs& a, int D, int gs, int qvw, bool vq, int B,
                            hipStream_t s);
extern template hipError_t launch_valu_bits<16>(const PartialArgs&, int, int, int, int, int, bool, hipStream_t);
extern template hipError_t launch_valu_bits<8>(const PartialArgs&, int, int, int, int, int, bool, hipStream_t);
extern template hipError_t launch_valu_bits<4>(const PartialArgs&, int, int, int, int, int, bool, hipStream_t);
extern template hipError_t launch_valu_bits<2>(const PartialArgs&, int, int, int, int, int, bool, hipStream_t);
extern template hipError_t launch_valu_bits<6>(const PartialArgs&, int, int, int, int, int, bool, hipStream_t);
extern template hipError_t launch_valu_bits<5>(const PartialArgs&, int, int, int, int, int, bool, hipStream_t);
extern template hipError_t launch_valu_bits<3>(const PartialArgs&, int, int, int, int, int, bool, hipStream_t);
extern template hipError_t launch_step_bits<16>(const AppendArgs&, const PartialArgs&, int, int, int, bool, int,
                                                hipStream_t);
extern template hipError_t launch_step_bits<8>(const AppendArgs&, const PartialArgs&, int, int, int, bool, int,
                                               hipStream_t);
extern template hipError_t launch_step_bits<4>(const AppendArgs&, const PartialArgs&, int, int, int, bool, int,
                                               hipStream_t);
extern template hipError_t launch_step_bits<2>(const AppendArgs&, const PartialArgs&, int, int, int, bool, int,
                                               hipStream_t);

extern template hipError_t launch_step_bits<6>(const AppendArgs&, const PartialArgs&, int, int, int, bool, int,
                                               hipStream_t);
extern template hipError_t launch_step_bits<5>(const AppendArgs&, const PartialArgs&, int, int, int, bool, int,
                                               hipStream_t);
extern template hipError_t launch_step_bits<3>(const AppendArgs&, const PartialArgs&, int, int, int, bool, int,
                                               hipStream_t);

bool partial_supported(int bits, int D, int DV, int gs, int qvw) {
  const bool b = bits == 16 || bits == 8 || bits == 6 || bits == 5 || bits == 4 || bits == 3 || bits == 2;
  const bool d = (D == 64 || D == 128 || D == 256) && valu_row_ok(bits, D) && valu_row_ok(bits, DV) &&
                 valu_dv_ok(bits, D, DV, gs);
  const bool g = bits == 16 || ((gs == 32 || gs == 64 || gs == 128) && D % gs == 0 && DV % gs == 0);
  const bool q = (qvw == 1 || qvw == 2 || qvw == 4 || qvw == 8) && qvw <= valu_max_qvw(bits, D, DV, gs);
  return b && d && g && q;
}

hipError_t launch_partial(const PartialArgs& a, int bits, int D, int DV, int gs, int qvw, int B, bool q_ready,
                          hipStream_t s) {
  switch (bits) {
    case 16: return launch_valu_bits<16>(a, D, DV, gs, qvw, B, q_ready, s);
    case 8: return launch_valu_bits<8>(a, D, DV, gs, qvw, B, q_ready, s);
    case 6: return launch_valu_bits<6>(a, D, DV, gs, qvw, B, q_ready, s);
    case 5: return launch_valu_bits<5>(a, D, DV, gs, qvw, B, q_ready, s);
    case 4: return launch_valu_bits<4>(a, D, DV, gs, qvw, B, q_ready, s);
    case 3: return launch_valu_bits<3>(a, D, DV, gs, qvw, B, q_ready, s);
    case 2: return launch_valu_bits<2>(a, D, DV, gs, qvw, B, q_ready, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_step_prep(const AppendArgs& ap, const PartialArgs& a, int bits, int D, int DV, int gs, int qvw,
                            bool vector_q, int B, hipStream_t s) {
  (void)DV;                                       // the step kernel reads it from ap.Dv
  switch (bits) {
    case 16: return launch_step_bits<16>(ap, a, D, gs, qvw, vector_q, B, s);
    case 8: return launch_step_bits<8>(ap, a, D, gs, qvw, vector_q, B, s);
    case 6: return launch_step_bits<6>(ap, a, D, gs, qvw, vector_q, B, s);
    case 5: return launch_step_bits<5>(ap, a, D, gs, qvw, vector_q, B, s);
    case 4: return launch_step_bits<4>(ap, a, D, gs, qvw, vector_q, B, s);
    case 3: return launch_step_bits<3>(ap, a, D, gs, qvw, vector_q, B, s);
    case 2: return launch_step_bits<2>(ap, a, D, gs, qvw, vector_q, B, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
