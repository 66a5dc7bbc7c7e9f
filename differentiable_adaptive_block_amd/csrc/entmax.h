// Wave-level alpha-entmax threshold solve (gfx950, wave64).
//
// alpha-entmax over the candidate scores of one query row (DashAttention
// pages: "Key Concepts", alpha-entmax bullet; AdaSplash-2 abstract on the
// thelatestinai.com page: the normaliser tau is the costly part of entmax).
// With u = (alpha-1) z and m = 1/(alpha-1), tau solves
//     f(tau) = sum_b [u_b - tau]_+^m = 1.
// f is convex and decreasing, so Newton's method started left of the root
// (at max u - 1, where the largest term alone gives f >= 1) increases
// monotonically to it, one pair of wave reductions per step.  alpha = 1 is
// the softmax: tau = log-sum-exp(z).
#pragma once

#include "common.h"

struct EntmaxOut {
  float tau;
  float lognorm;
  int nsel;
};

// One row per wave.  Lane l holds u[k] = score of candidate l + 64 k for
// k < NPL, or -INFINITY where there is none.  n = number of candidates (> 0).
// The result is identical in every lane.
template <int NPL>
__device__ __forceinline__ EntmaxOut entmax_solve(const float (&u)[NPL], const CoarseArith& ca) {
  float umax = -INFINITY;
#pragma unroll
  for (int k = 0; k < NPL; ++k) umax = fmaxf(umax, u[k]);
  umax = wave_max(umax);
  EntmaxOut r;
  if (ca.softmax) {
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < NPL; ++k) s += (u[k] != -INFINITY) ? __expf(u[k] - umax) : 0.f;
    s = wave_sum(s);
    r.tau = umax + __logf(s);
    float s2 = 0.f;
    int c = 0;
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      if (u[k] != -INFINITY) { s2 += __expf(u[k] - r.tau); ++c; }
    }
    r.lognorm = __logf(wave_sum(s2));
    r.nsel = wave_sum_i(c);
    return r;
  }
  const float m = ca.m;
  float t = -1.f;  // relative to max u: f(-1) >= 1 from the largest term alone
  // Newton from the left.
  for (int it = 0; it < 64; ++it) {
    float f = 0.f, fp = 0.f;
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      float x = (u[k] - umax) - t;
      if (x > 0.f) { f += pow_m(x, m); fp += pow_m1(x, m); }
    }
    f = wave_sum(f);
    fp = wave_sum(fp);
    float step = (f - 1.f) / (m * fp);
    if (!(step > 0.f)) break;  // at (or, by rounding, just past) the root
    t += step;
    if (step <= 1e-7f) break;
  }
  r.tau = umax + t;
  float s = 0.f;
  int c = 0;
#pragma unroll
  for (int k = 0; k < NPL; ++k) {
    float x = u[k] - r.tau;
    if (x > 0.f) { s += pow_m(x, m); ++c; }
  }
  r.lognorm = __logf(wave_sum(s));
  r.nsel = wave_sum_i(c);
  return r;
}
