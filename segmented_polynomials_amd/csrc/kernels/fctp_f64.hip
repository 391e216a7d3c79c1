// Fully connected tensor product kernels, double instantiations (the templates
// are in fctp.hpp; one file per dtype keeps the builds parallel).
#include "fctp.hpp"

namespace segpoly {

int launch_fctp_f64(const FcArgs& a, const FcTiles& t) {
  using namespace kern;
  return a.layout == kMulIr ? fctp_launch<double, kMulIr>(a, t) : fctp_launch<double, kIrMul>(a, t);
}

int launch_fctp_dw_f64(const FcDwArgs& a, const FcDwTiles& t) {
  using namespace kern;
  return a.layout == kMulIr ? fctp_dw_launch<double, kMulIr>(a, t) : fctp_dw_launch<double, kIrMul>(a, t);
}

int launch_fctp_transpose_f64(const FcTrArgs& a) { return kern::fctp_transpose_launch<double>(a); }

}  // namespace segpoly
