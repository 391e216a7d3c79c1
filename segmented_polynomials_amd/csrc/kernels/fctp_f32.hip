// Fully connected tensor product kernels, float instantiations (the templates
// are in fctp.hpp; one file per dtype keeps the builds parallel).
#include "fctp.hpp"

namespace segpoly {

int launch_fctp_f32(const FcArgs& a, const FcTiles& t) {
  using namespace kern;
  return a.layout == kMulIr ? fctp_launch<float, kMulIr>(a, t) : fctp_launch<float, kIrMul>(a, t);
}

int launch_fctp_dw_f32(const FcDwArgs& a, const FcDwTiles& t) {
  using namespace kern;
  return a.layout == kMulIr ? fctp_dw_launch<float, kMulIr>(a, t) : fctp_dw_launch<float, kIrMul>(a, t);
}

int launch_fctp_transpose_f32(const FcTrArgs& a) { return kern::fctp_transpose_launch<float>(a); }

}  // namespace segpoly
