// Device helpers shared by the DashAttention HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define DASH_BLOCK 64       // keys per block (Stage 0 pooling and Stage 2 key tile)
#define DASH_QTILE 128      // query rows per Stage-2 tile (4 waves x 32 rows)
#define DASH_MAX_NB 1536    // longest prefill sequence: 1536 blocks = 98304 tokens
#define DASH_LD_RANGE 128   // low-density schedule: row groups (of 64 rows) per row range of its work items

typedef uint16_t bf16_t;  // raw bfloat16 storage

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ conversions

__device__ __forceinline__ float bf2f(bf16_t x) { return __uint_as_float(((uint32_t)x) << 16); }

// float -> bfloat16, round to nearest even (inputs are finite).
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// double -> bfloat16 in one rounding step (nearest, ties to even): keep the
// top 7 fraction bits of the binary64 pattern, add the rounding increment at
// bit 44 and re-bias the exponent.  Exact zero keeps its sign; the values
// pooled here are far from the bf16 subnormal and overflow ranges.
__device__ __forceinline__ bf16_t d2bf(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  uint64_t sign = u >> 63;
  uint64_t mag = u & 0x7FFFFFFFFFFFFFFFull;
  if (mag == 0) return (bf16_t)(sign << 15);
  uint64_t lsb = (mag >> 45) & 1ull;
  mag += (1ull << 44) - 1ull + lsb;
  mag >>= 45;                     // 11-bit exponent : 7-bit fraction
  uint64_t e = mag >> 7;          // biased binary64 exponent (after rounding carry)
  uint64_t frac = mag & 0x7Full;
  uint64_t be = e - 1023 + 127;   // bf16 biased exponent
  return (bf16_t)((sign << 15) | (be << 7) | frac);
}

template <typename T> __device__ __forceinline__ float to_f(T x);
template <> __device__ __forceinline__ float to_f<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t x) { return bf2f(x); }

template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float x) { return f2bf(x); }

template <typename T> __device__ __forceinline__ double to_d(T x) { return (double)to_f<T>(x); }

// ------------------------------------------------------------------ wave reductions (wave64)

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ------------------------------------------------------------------ MFMA operands

// 8 consecutive bf16 (16 bytes) as an MFMA operand.
__device__ __forceinline__ bf16x8 load8(const bf16_t* p) {
  uint4 r = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row index of accumulator register r of a 32x32 MFMA tile held by lane l
// (the column is l % 32).
__device__ __forceinline__ int acc_row32(int r, int l) { return 8 * (r >> 2) + 4 * (l >> 5) + (r & 3); }

// ------------------------------------------------------------------ Stage-1 score arithmetic
//
// One definition of the coarse score used by every kernel, so that the
// selection seen by Stage 1, Stage 2, decode and the backward is the same
// bit pattern:  acc = q . kbar (fp32 accumulation), z = acc * coarse_scale,
// u = z * (alpha - 1)  (alpha = 1: u = z).
struct CoarseArith {
  float coarse_scale;
  float am1;       // alpha - 1
  float m;         // 1 / (alpha - 1); unused when alpha == 1
  int softmax;     // alpha == 1
  __device__ __forceinline__ float u_of(float acc) const {
    float z = acc * coarse_scale;
    return softmax ? z : z * am1;
  }
  // log p_b from u and the row's (tau, lognorm); -inf when not selected.
  __device__ __forceinline__ float logp(float u, float tau, float lognorm) const {
    if (softmax) return (u - tau) - lognorm;
    float x = u - tau;
    return x > 0.f ? m * __logf(x) - lognorm : -INFINITY;
  }
  __device__ __forceinline__ bool selected(float u, float tau) const {
    return softmax ? true : (u - tau) > 0.f;
  }
};
