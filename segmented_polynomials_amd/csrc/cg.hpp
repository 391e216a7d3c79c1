// Real-basis Clebsch-Gordan coupling tensors for the channelwise paths.
//
// The pages describe the [ijk] factor of [ijk]*a[uv]*b[iu]*c[jv] -> D[kuv]
// as the Clebsch-Gordan tensor, known at compile time and mostly zero, with
// normalisation folded into the coefficients (e3nn-course Lesson 12a,
// sections 21.1 and 21.4; cuequivariance-torch skill document,
// "SegmentedPolynomial: gather and scatter").  This is the host builder's own
// construction (long double, rounded once to double):
//   * complex Condon-Shortley coefficients by Racah's formula;
//   * change of basis to the real harmonics (index m = -l..l; l = 1 is
//     (y, z, x)) with real Y_m = sum_mu Q[m,mu] complex Y^mu,
//       m<0: (i/sqrt2)(Y^m - (-1)^m Y^-m), m=0: Y^0, m>0: (1/sqrt2)(Y^-m + (-1)^m Y^m),
//     C[m1,m2,m3] = sum conj(Q[m1,mu1]) conj(Q[m2,mu2]) Q[m3,mu3] CG[mu1,mu2,mu3],
//     keeping the real or the imaginary part, whichever is non-zero;
//   * "component" scaling: sum_ij C_ijk C_ijk' = delta_kk' (what the unitary
//     change of basis gives), so 0 x l -> l and l x 0 -> l are the identity;
//   * sign: for even l1+l2+l3 the (m1, m2, m3) = (0, 0, 0) entry is positive
//     (equivalently, coupling the harmonics of one vector with themselves
//     gives a positive multiple of its degree-l3 harmonics, by evaluating at
//     the z axis); for odd l1+l2+l3 the first non-zero entry in index order
//     is positive.
#pragma once
#include <vector>

namespace segpoly {

// Row-major [2l1+1][2l2+1][2l3+1]; all zeros if the triangle rule fails.
const std::vector<double>& real_cg(int l1, int l2, int l3);

}  // namespace segpoly
