// Wave-level alpha-entmax threshold solve (gfx950, wave64).
//
// alpha-entmax over the candidate scores of one query row (DashAttention
// pages: "Key Concepts", alpha-entmax bullet; AdaSplash-2 abstract on the
// thelatestinai.com page: the normaliser tau is the costly part of entmax).
// With u = (alpha-1) z and m = 1/(alpha-1), tau solves
//     f(tau) = sum_b [u_b - tau]_+^m = 1.
// The iteration is Newton's method on g = f^(1/m) - 1, the m-norm of
// [u - tau]_+ minus one, rather than on f itself: g is convex and
// decreasing, so steps taken from the left of the root increase
// monotonically to it, and g is nearly linear (exactly linear while the
// support does not change and its scores are equal), so the steps are long
// for every alpha, where Newton on f crawls at small alpha (each step
// closes only a fraction 1/m of the gap far from the root).  The start is
// max u - 1, where the largest term alone gives f >= 1; at alpha = 1.5 a
// closed-form start is taken first (see entmax_newton).  alpha = 1 is the
// softmax: tau = log-sum-exp(z).
//
// A row is held by a group of G lanes (G = 16: four rows per wave; G = 64:
// one row per wave).  Group reductions use DPP within each 16-lane row of
// the wave (quad swaps, half-row and row mirrors), so every lane of the row
// ends with the same bits; G = 64 then adds the four row results read back
// with readlane, in a fixed order.
#pragma once

#include "common.h"

struct EntmaxOut {
  float tau;
  float lognorm;
  int nsel;    // selected candidates (-1 when not counted)
  int passes;  // passes over the row's scores the threshold took
};

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// DPP controls: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
#define DPP_QSWAP1 0xB1
#define DPP_QSWAP2 0x4E
#define DPP_HMIRROR 0x141
#define DPP_MIRROR 0x140

__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<DPP_QSWAP1>(v);
  v += dpp_f<DPP_QSWAP2>(v);
  v += dpp_f<DPP_HMIRROR>(v);
  v += dpp_f<DPP_MIRROR>(v);
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<DPP_QSWAP1>(v));
  v = fmaxf(v, dpp_f<DPP_QSWAP2>(v));
  v = fmaxf(v, dpp_f<DPP_HMIRROR>(v));
  v = fmaxf(v, dpp_f<DPP_MIRROR>(v));
  return v;
}
__device__ __forceinline__ int row16_sum_i(int v) {
  v += dpp_i<DPP_QSWAP1>(v);
  v += dpp_i<DPP_QSWAP2>(v);
  v += dpp_i<DPP_HMIRROR>(v);
  v += dpp_i<DPP_MIRROR>(v);
  return v;
}

template <int G>
__device__ __forceinline__ float grp_sum(float v) {
  v = row16_sum(v);
  if constexpr (G == 64) {
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    v = (r0 + r1) + (r2 + r3);
  }
  return v;
}
template <int G>
__device__ __forceinline__ float grp_max(float v) {
  v = row16_max(v);
  if constexpr (G == 64) {
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    v = fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
  }
  return v;
}
template <int G>
__device__ __forceinline__ int grp_sum_i(int v) {
  v = row16_sum_i(v);
  if constexpr (G == 64) {
    v = (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
        (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
  }
  return v;
}

// [x]_+^m and [x]_+^(m-1) for x = v - t, branch-free: PW = 1 (m = 1,
// alpha = 2), 2 (alpha = 1.5), 4 (alpha = 1.25), 0 (any other m > 1, via
// the hardware exp2 / log2; x <= 0 gives log2 = -inf and so 0).
template <int PW>
__device__ __forceinline__ void entmax_terms(float x, float m, float& fx, float& fpx) {
  x = fmaxf(x, 0.f);
  if constexpr (PW == 1) {
    fx = x;
    fpx = x > 0.f ? 1.f : 0.f;
  } else if constexpr (PW == 2) {
    fx = x * x;
    fpx = x;
  } else if constexpr (PW == 4) {
    const float x2 = x * x;
    fx = x2 * x2;
    fpx = x2 * x;
  } else {
    const float lx = __builtin_amdgcn_logf(x);
    fx = __builtin_amdgcn_exp2f(m * lx);
    fpx = __builtin_amdgcn_exp2f((m - 1.f) * lx);
  }
}

// f^((m-1)/m), the factor of the Newton step on f^(1/m).
template <int PW>
__device__ __forceinline__ float step_pow(float f, float m) {
  if constexpr (PW == 1) return 1.f;
  else if constexpr (PW == 2) return __builtin_sqrtf(f);
  else if constexpr (PW == 4) {
    const float r = __builtin_sqrtf(f);
    return r * __builtin_sqrtf(r);
  } else {
    return __builtin_amdgcn_exp2f((m - 1.f) / m * __builtin_amdgcn_logf(f));
  }
}

// alpha > 1: Newton on f^(1/m) from the left, on t = tau - max u (see the
// header).  With x = [v - t]_+ (v = u - max u), S = sum x^m and
// S1 = sum x^(m-1), the step is (S - S^((m-1)/m)) / S1.  Every pass keeps
// S, so the pass that finds the step at most 1e-7 is the last: tau =
// max u + t there and lognorm = log S(t).  `count`: also count the
// support (one more pass, compares only).
template <int NPL, int G, int PW>
__device__ __forceinline__ EntmaxOut entmax_newton(const float (&u)[NPL], int nvalid, float umax, float m,
                                                   bool count) {
  // v = u - umax, recomputed where used rather than held (NPL registers)
  auto vof = [&](int k) { return u[k] - umax; };
  float t = -1.f;  // f(-1) >= 1 from the largest term alone
  int passes = 0;
  // the closed-form start pays off on short rows, where most candidates end
  // up in the support; on long rows (measured at 1023 candidates) Newton from
  // -1 takes fewer passes than the start's two
  if constexpr (PW == 2) if (nvalid <= 512) {
    // alpha = 1.5: sum_{v > t} (v - t)^2 = 1 is a quadratic in t once the
    // support is fixed.  Its smaller root t_c on the support {v > -1} lies at
    // or right of the true root (elements of that set that fall below the
    // root still add to the left-hand side); g is convex, so one step from
    // there lands at or left of the root, where the iteration below starts.
    // A start that rounding puts anywhere else falls back to -1.
    float n = 0.f, sa = 0.f, sb = 0.f;
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      if (k * G < nvalid) {
        const float vk = vof(k);
        const bool in = vk > -1.f;
        n += in ? 1.f : 0.f;
        sa += in ? vk : 0.f;
        sb += in ? vk * vk : 0.f;
      }
    }
    n = grp_sum<G>(n);
    sa = grp_sum<G>(sa);
    sb = grp_sum<G>(sb);
    const float tc = (sa - __builtin_sqrtf(fmaxf(sa * sa - n * (sb - 1.f), 0.f))) / n;
    float f = 0.f, s1 = 0.f;
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      if (k * G < nvalid) {
        const float x = fmaxf(vof(k) - tc, 0.f);
        f += x * x;
        s1 += x;
      }
    }
    f = grp_sum<G>(f);
    s1 = grp_sum<G>(s1);
    const float t1 = tc + (f - __builtin_sqrtf(f)) / s1;
    if (t1 > -1.f && t1 <= 0.f) t = t1;  // false for NaN too
    passes = 2;
  }
  bool done = false;
  float tfin = t, lnf = 0.f;
  int npass = passes;
  // groups that have converged keep their result while the others iterate
  // (all lanes stay active for the DPP reductions)
  for (int it = 0; it < 64; ++it) {
    float f = 0.f, s1 = 0.f;
    const float tabs = umax + t;  // the trial threshold in u units
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      if (k * G < nvalid) {
        float a, b;
        entmax_terms<PW>(u[k] - tabs, m, a, b);
        f += a;
        s1 += b;
      }
    }
    f = grp_sum<G>(f);
    s1 = grp_sum<G>(s1);
    ++passes;
    const float step = (f - step_pow<PW>(f, m)) / s1;
    if (!done) {
      if (!(step > 1e-7f)) {  // converged (or, by rounding, just past the root; NaN too)
        done = true;
        tfin = t;
        lnf = __logf(f);
        npass = passes;
      } else {
        t += step;
      }
    }
    if (__ballot(!done) == 0ull) break;
  }
  if (!done) {  // not reached on finite scores; keep the outputs defined
    tfin = t;
    npass = passes;
  }
  EntmaxOut r;
  r.tau = umax + tfin;
  r.lognorm = lnf;
  r.passes = npass;
  r.nsel = -1;
  if (count) {
    int c = 0;
#pragma unroll
    for (int k = 0; k < NPL; ++k)
      if (k * G < nvalid) c += (u[k] - r.tau) > 0.f ? 1 : 0;
    r.nsel = grp_sum_i<G>(c);
  }
  return r;
}

// One row per group of G lanes.  Lane (group-local index g) holds
// u[k] = score of candidate g + G k for k < NPL, or -INFINITY where there is
// none; only k with G k < nvalid can hold a candidate (nvalid is the same on
// every lane of the wave, so the loops skip the rest with scalar branches);
// every row has at least one candidate.  All lanes of the wave call this
// together; the result is identical across each group.
template <int NPL, int G>
__device__ __forceinline__ EntmaxOut entmax_solve(const float (&u)[NPL], int nvalid, const CoarseArith& ca,
                                                  bool count = true) {
  float umax = -INFINITY;
#pragma unroll
  for (int k = 0; k < NPL; ++k)
    if (k * G < nvalid) umax = fmaxf(umax, u[k]);
  umax = grp_max<G>(umax);
  if (ca.softmax) {
    EntmaxOut r;
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < NPL; ++k)
      if (k * G < nvalid) s += __expf(u[k] - umax);  // exp(-inf) = 0 for empty slots
    s = grp_sum<G>(s);
    r.tau = umax + __logf(s);
    float s2 = 0.f;
    int c = 0;
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      if (k * G < nvalid) {
        s2 += __expf(u[k] - r.tau);
        c += u[k] != -INFINITY ? 1 : 0;
      }
    }
    r.lognorm = __logf(grp_sum<G>(s2));
    r.nsel = grp_sum_i<G>(c);
    r.passes = 2;
    return r;
  }
  const float m = ca.m;
  if (m == 2.f) return entmax_newton<NPL, G, 2>(u, nvalid, umax, m, count);
  if (m == 4.f) return entmax_newton<NPL, G, 4>(u, nvalid, umax, m, count);
  if (m == 1.f) return entmax_newton<NPL, G, 1>(u, nvalid, umax, m, count);
  return entmax_newton<NPL, G, 0>(u, nvalid, umax, m, count);
}
