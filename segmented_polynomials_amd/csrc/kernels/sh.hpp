// Real spherical harmonics of a vector, l = 0..LMAX, "component"
// normalisation (sum_m Y_lm^2 = 2l + 1 on the unit sphere), device code.
//
// cuequivariance-torch skill document, "Spherical harmonics and a NumPy
// reference": normalize=True evaluates on v / |v|, normalize=False the raw
// (homogeneous) polynomial.  The basis (the pages print none) is the
// textbook real one, index l^2 + l + m:
//   m > 0: sqrt2 N_lm q_l^m Re (x + i y)^m,  m = 0: N_l0 q_l^0,
//   m < 0: sqrt2 N_l|m| q_l^|m| Im (x + i y)^|m|,
// N_lm = sqrt((2l+1) (l-m)! / (l+m)!), q_l^m = r^(l-m) P_l^(m)(z / r) the
// homogeneous form of the m-th derivative of the Legendre polynomial
// (no Condon-Shortley phase), so that l = 1 is sqrt3 (y, z, x).  Recurrences:
//   q_m^m = (2m-1)!!,  q_(m+1)^m = (2m+1) z q_m^m,
//   q_l^m = ((2l-1) z q_(l-1)^m - (l+m-1) r^2 q_(l-2)^m) / (l - m),
//   (x + i y)^(m+1) = (x + i y)^m (x + i y).
// With normalisation the recurrences run on u = v / |v| with r^2 = 1 (the
// polynomial that agrees with Y on the sphere); its gradient is then
// projected tangentially, dY/dv = (I - u u^T) / |v| grad_u, which removes
// the radial part in which extensions differ.  A zero vector with
// normalisation gives Y_0 = 1, Y_l>0 = 0 and a zero gradient.
#pragma once
#include <hip/hip_runtime.h>

#include "../launch.hpp"

namespace segpoly {
namespace kern {

// value and gradient with respect to the three polynomial variables
template <typename T>
struct Dual {
  T v, dx, dy, dz;
};
template <typename T>
__device__ __forceinline__ Dual<T> operator+(Dual<T> a, Dual<T> b) { return {a.v + b.v, a.dx + b.dx, a.dy + b.dy, a.dz + b.dz}; }
template <typename T>
__device__ __forceinline__ Dual<T> operator-(Dual<T> a, Dual<T> b) { return {a.v - b.v, a.dx - b.dx, a.dy - b.dy, a.dz - b.dz}; }
template <typename T>
__device__ __forceinline__ Dual<T> operator*(Dual<T> a, Dual<T> b) {
  return {a.v * b.v, a.dx * b.v + a.v * b.dx, a.dy * b.v + a.v * b.dy, a.dz * b.v + a.v * b.dz};
}
template <typename T>
__device__ __forceinline__ Dual<T> operator*(T s, Dual<T> a) { return {s * a.v, s * a.dx, s * a.dy, s * a.dz}; }

template <typename N, typename T>
__device__ __forceinline__ N sh_const(T c);
template <>
__device__ __forceinline__ float sh_const<float, float>(float c) { return c; }
template <>
__device__ __forceinline__ double sh_const<double, double>(double c) { return c; }
template <>
__device__ __forceinline__ Dual<float> sh_const<Dual<float>, float>(float c) { return {c, 0.f, 0.f, 0.f}; }
template <>
__device__ __forceinline__ Dual<double> sh_const<Dual<double>, double>(double c) { return {c, 0.0, 0.0, 0.0}; }

// Y[l^2 + l + m] for the polynomial variables x, y, z (numbers of type N:
// T for values, Dual<T> for values with gradients); r2 = x^2 + y^2 + z^2,
// or the constant 1 on the sphere.
template <typename T, typename N, int LMAX>
__device__ __forceinline__ void sh_poly(N x, N y, N z, N r2, const ShConsts& K, N (&Y)[(LMAX + 1) * (LMAX + 1)]) {
  N cm = sh_const<N, T>(T(1)), sm = sh_const<N, T>(T(0));   // (x + i y)^m
  T dfact = T(1);                                              // (2m - 1)!!
#pragma unroll
  for (int m = 0; m <= LMAX; ++m) {
    if (m > 0) {
      const N c2 = cm * x - sm * y, s2 = sm * x + cm * y;
      cm = c2;
      sm = s2;
      dfact *= T(2 * m - 1);
    }
    N q2 = sh_const<N, T>(T(0));
    N q1 = sh_const<N, T>(dfact);  // q_m^m
#pragma unroll
    for (int l = m; l <= LMAX; ++l) {
      N q;
      if (l == m) {
        q = q1;
      } else if (l == m + 1) {
        q = T(2 * m + 1) * (z * q1);
        q2 = q1;
        q1 = q;
      } else {
        q = T(1) / T(l - m) * (T(2 * l - 1) * (z * q1) - T(l + m - 1) * (r2 * q2));
        q2 = q1;
        q1 = q;
      }
      const T nrm = static_cast<T>(K.c[l * (l + 1) / 2 + m]);
      if (m == 0) {
        Y[l * l + l] = nrm * q;
      } else {
        Y[l * l + l + m] = nrm * (q * cm);
        Y[l * l + l - m] = nrm * (q * sm);
      }
    }
  }
}

// Harmonics of the vector (vx, vy, vz).
template <typename T, int LMAX>
__device__ __forceinline__ void sh_eval(T vx, T vy, T vz, bool normalize, const ShConsts& K,
                                        T (&Y)[(LMAX + 1) * (LMAX + 1)]) {
  T x = vx, y = vy, z = vz, r2 = vx * vx + vy * vy + vz * vz;
  if (normalize) {
    const T r = sqrt(r2);
    const T inv = r > T(0) ? T(1) / r : T(0);
    x *= inv;
    y *= inv;
    z *= inv;
    r2 = r > T(0) ? T(1) : T(0);
  }
  sh_poly<T, T, LMAX>(x, y, z, r2, K, Y);
}

// sum_j g[j] dY_j / dv for the vector (vx, vy, vz).
template <typename T, int LMAX>
__device__ __forceinline__ void sh_vjp(T vx, T vy, T vz, bool normalize, const ShConsts& K,
                                       const T (&g)[(LMAX + 1) * (LMAX + 1)], T& gx, T& gy, T& gz) {
  using D = Dual<T>;
  T ux = vx, uy = vy, uz = vz, r = T(1);
  bool zero = false;
  if (normalize) {
    r = sqrt(vx * vx + vy * vy + vz * vz);
    zero = !(r > T(0));
    const T inv = zero ? T(0) : T(1) / r;
    ux *= inv;
    uy *= inv;
    uz *= inv;
  }
  const D x{ux, T(1), T(0), T(0)}, y{uy, T(0), T(1), T(0)}, z{uz, T(0), T(0), T(1)};
  const D r2 = normalize ? D{T(1), T(0), T(0), T(0)} : x * x + y * y + z * z;
  D Y[(LMAX + 1) * (LMAX + 1)];
  sh_poly<T, D, LMAX>(x, y, z, r2, K, Y);
  T ax = T(0), ay = T(0), az = T(0);
#pragma unroll
  for (int j = 0; j < (LMAX + 1) * (LMAX + 1); ++j) {
    ax += g[j] * Y[j].dx;
    ay += g[j] * Y[j].dy;
    az += g[j] * Y[j].dz;
  }
  if (normalize) {
    if (zero) {
      ax = ay = az = T(0);
    } else {
      const T radial = ux * ax + uy * ay + uz * az;
      ax = (ax - ux * radial) / r;
      ay = (ay - uy * radial) / r;
      az = (az - uz * radial) / r;
    }
  }
  gx = ax;
  gy = ay;
  gz = az;
}

}  // namespace kern
}  // namespace segpoly
