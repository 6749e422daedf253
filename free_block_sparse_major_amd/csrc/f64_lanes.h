// fp64 helpers shared by the fp64 kernels (probe fit, RCP factors): a
// refined reciprocal, cross-lane sums of fp64 values with DPP, and the Sturm
// count of a symmetric tridiagonal matrix.
#pragma once

#include "common.h"

namespace spr {

constexpr double kEps64 = 2.220446049250313e-16;
constexpr double kTiny = 1e-290;   // pivot floor of the normalised tridiagonal matrix

// 1 / y from the hardware estimate and one Newton step (a few ulp)
SPR_DEV double rcp64(double y) {
  const double r = __builtin_amdgcn_rcp(y);
  return fma(fma(-y, r, 1.0), r, r);
}

// Cross-lane moves of fp64 values with DPP (two 32-bit halves).
template <int CTRL>
SPR_DEV double dpp_f64(double v) {
  const unsigned long long u = static_cast<unsigned long long>(__double_as_longlong(v));
  const int lo = __builtin_amdgcn_update_dpp(0, int(uint32_t(u)), CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, int(uint32_t(u >> 32)), CTRL, 0xf, 0xf, false);
  return __longlong_as_double(
      static_cast<long long>((static_cast<unsigned long long>(uint32_t(hi)) << 32) | uint32_t(lo)));
}

// Sum over aligned groups of GL lanes (4, 8 or 16): lane pairs meet by quad
// permutations, then half-row and row mirrors; every lane of a group ends
// with the same bits.
template <int GL>
SPR_DEV double group_sum_f64(double v) {
  v += dpp_f64<0xB1>(v);                    // quad_perm [1,0,3,2]
  v += dpp_f64<0x4E>(v);                    // quad_perm [2,3,0,1]
  if constexpr (GL >= 8) v += dpp_f64<0x141>(v);   // row_half_mirror
  if constexpr (GL >= 16) v += dpp_f64<0x140>(v);  // row_mirror
  return v;
}

SPR_DEV double readlane_f64(double v, int l) {
  const unsigned long long u = static_cast<unsigned long long>(__double_as_longlong(v));
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(u)), l));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(u >> 32)), l));
  return __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo));
}

// Wave-wide sum, the same value in every lane.
SPR_DEV double wave_sum_f64(double v) {
  v = group_sum_f64<16>(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// Sum over aligned groups of GL lanes, GL a power of two up to 64.
template <int GL>
SPR_DEV double group_sum_any(double v) {
  if constexpr (GL <= 16) {
    return group_sum_f64<GL>(v);
  } else {
    v = group_sum_f64<16>(v);
    v += __shfl_xor(v, 16);
    if constexpr (GL == 64) v += __shfl_xor(v, 32);
    return v;
  }
}

// Sturm counts of the normalised tridiagonal matrix at two points (two
// independent recurrences interleaved): eigenvalues below x1 and below x2.
// st[i] = (d_(i+1), e_i^2), i < n - 1.
SPR_DEV void sturm_count2(double d0, const double2* st, int n, double x1, double x2, int& c1,
                          int& c2) {
  double q1 = d0 - x1, q2 = d0 - x2;
  int n1 = 0, n2 = 0;
  auto step = [&](double2 s) {
    if (fabs(q1) < kTiny) q1 = -kTiny;
    if (fabs(q2) < kTiny) q2 = -kTiny;
    n1 += q1 < 0.0 ? 1 : 0;
    n2 += q2 < 0.0 ? 1 : 0;
    q1 = (s.x - x1) - s.y * rcp64(q1);
    q2 = (s.x - x2) - s.y * rcp64(q2);
  };
  int i = 0;
  for (; i + 4 <= n - 1; i += 4) {
    const double2 s0 = st[i], s1 = st[i + 1], s2 = st[i + 2], s3 = st[i + 3];
    step(s0);
    step(s1);
    step(s2);
    step(s3);
  }
  for (; i < n - 1; ++i) step(st[i]);
  if (fabs(q1) < kTiny) q1 = -kTiny;
  if (fabs(q2) < kTiny) q2 = -kTiny;
  c1 = n1 + (q1 < 0.0 ? 1 : 0);
  c2 = n2 + (q2 < 0.0 ? 1 : 0);
}

}  // namespace spr
