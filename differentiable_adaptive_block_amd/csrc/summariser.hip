// The learned Stage-0 summariser: attention pooling with one vector w per
// head, zero at initialisation (the montana-research page, "What
// alpha-entmax changes": a small learned attention head that starts at zero,
// so training starts from mean pooling).  For block b of head h,
//   e_j = w_h . k_j,  a = softmax(e) over the block's 64 keys,
//   kbar_b = sum_j a_j k_j.
// At w = 0 every a_j is exactly 1/64 and the fp64 sums are exact, so the
// summaries equal the mean-pooling kernel's bit for bit.
//
// Backward (the summary's rounding taken as the identity), with g = dkbar_b
// and c_j = k_j . g - kbar_b . g:
//   dk_j += a_j g + a_j c_j w_h,   dw_h = sum over batch and blocks of sum_j a_j c_j k_j.
//
// Both kernels: one wave per (block, head), the block's keys staged in LDS
// as float (exact for bf16 and fp32) with padded rows, lane j owning key j
// for the scores and lane c owning feature c (and c + 64) for the sums.
// dw is reduced in a fixed order from per-block partials (deterministic).
#include "summariser.h"

namespace {

constexpr int KP = 129;  // padded LDS row (floats): lane j reading row j hits bank (j * 129) % 64 = j

__device__ __forceinline__ double wave_max_d(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmax(v, __shfl_xor(v, m, 64));
  return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

template <typename T>
__device__ __forceinline__ void stage_block(const T* src, float (*ks)[KP], int D, int l) {
  for (int r = 0; r < DASH_BLOCK; ++r)
    for (int c = l; c < D; c += 64) ks[r][c] = to_f<T>(src[(size_t)r * D + c]);
}

// Softmax weight of key l (this lane) over the block, in fp64.
__device__ __forceinline__ double block_weight(const float (*ks)[KP], const float* wh, int D, int l) {
  double e = 0.0;
  for (int c = 0; c < D; ++c) e = fma((double)wh[c], (double)ks[l][c], e);
  const double mx = wave_max_d(e);
  const double x = exp(e - mx);
  return x / wave_sum_d(x);
}

template <typename T>
__global__ __launch_bounds__(64) void pool_attn_kernel(const T* __restrict__ k, const float* __restrict__ w,
                                                       T* __restrict__ kbar, int H, int T_, int D) {
  __shared__ float ks[DASH_BLOCK][KP];
  __shared__ double as[DASH_BLOCK];
  const int b = blockIdx.x, l = threadIdx.x;
  const size_t bh = blockIdx.y;
  const int nb = T_ / DASH_BLOCK;
  stage_block<T>(k + (bh * T_ + (size_t)b * DASH_BLOCK) * D, ks, D, l);
  __syncthreads();
  as[l] = block_weight(ks, w + (bh % H) * D, D, l);
  __syncthreads();
  T* dst = kbar + (bh * nb + b) * D;
  for (int c = l; c < D; c += 64) {
    double acc = 0.0;
    for (int r = 0; r < DASH_BLOCK; ++r) acc = fma(as[r], (double)ks[r][c], acc);
    if constexpr (sizeof(T) == 2) dst[c] = d2bf(acc);
    else dst[c] = __double2float_rn(acc);
  }
}

template <typename T>
__global__ __launch_bounds__(64) void pool_attn_bwd_kernel(const T* __restrict__ k, const float* __restrict__ w,
                                                           const float* __restrict__ dkbar, T* __restrict__ dk,
                                                           float* __restrict__ dw_part, int H, int T_, int D) {
  __shared__ float ks[DASH_BLOCK][KP];
  __shared__ float gs[128], ms[128];
  __shared__ float as[DASH_BLOCK], des[DASH_BLOCK];
  const int b = blockIdx.x, l = threadIdx.x;
  const size_t bh = blockIdx.y;
  const int nb = T_ / DASH_BLOCK;
  const size_t row0 = bh * T_ + (size_t)b * DASH_BLOCK;
  const float* wh = w + (bh % H) * D;
  stage_block<T>(k + row0 * D, ks, D, l);
  for (int c = l; c < D; c += 64) gs[c] = dkbar[(bh * nb + b) * D + c];
  __syncthreads();
  const float a = (float)block_weight(ks, wh, D, l);
  as[l] = a;
  __syncthreads();
  for (int c = l; c < D; c += 64) {  // the summary before rounding
    float m = 0.f;
    for (int r = 0; r < DASH_BLOCK; ++r) m = fmaf(as[r], ks[r][c], m);
    ms[c] = m;
  }
  __syncthreads();
  float kg = 0.f, mg = 0.f;
  for (int c = 0; c < D; ++c) {
    kg = fmaf(ks[l][c], gs[c], kg);
    mg = fmaf(ms[c], gs[c], mg);
  }
  des[l] = a * (kg - mg);  // gradient of key l's score
  __syncthreads();
  T* dkb = dk + row0 * D;
  for (int r = 0; r < DASH_BLOCK; ++r) {
    for (int c = l; c < D; c += 64) {
      const float add = fmaf(as[r], gs[c], des[r] * wh[c]);
      if constexpr (sizeof(T) == 2) dkb[(size_t)r * D + c] = f2bf(bf2f(dkb[(size_t)r * D + c]) + add);
      else dkb[(size_t)r * D + c] += add;
    }
  }
  for (int c = l; c < D; c += 64) {
    float acc = 0.f;
    for (int r = 0; r < DASH_BLOCK; ++r) acc = fmaf(des[r], ks[r][c], acc);
    dw_part[(bh * nb + b) * D + c] = acc;
  }
}

// dw[h][c] = sum over (batch, block) of the partials, in a fixed order.
__global__ void reduce_dw_kernel(const float* __restrict__ dw_part, float* __restrict__ dw, int B, int H, int nb,
                                 int D) {
  const int h = blockIdx.x;
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    float acc = 0.f;
    for (int bb = 0; bb < B; ++bb) {
      const float* src = dw_part + ((size_t)(bb * H + h) * nb) * D + c;
      for (int b = 0; b < nb; ++b) acc += src[(size_t)b * D];
    }
    dw[(size_t)h * D + c] = acc;
  }
}

}  // namespace

hipError_t launch_pool_attn(const void* k, const float* w, void* kbar, int BH, int H, int T_, int D, int dtype,
                            hipStream_t st) {
  if (D > 128) return hipErrorNotSupported;
  dim3 grid(T_ / DASH_BLOCK, BH);
  if (dtype == 1)
    pool_attn_kernel<bf16_t><<<grid, 64, 0, st>>>((const bf16_t*)k, w, (bf16_t*)kbar, H, T_, D);
  else
    pool_attn_kernel<float><<<grid, 64, 0, st>>>((const float*)k, w, (float*)kbar, H, T_, D);
  return hipGetLastError();
}

hipError_t launch_pool_attn_bwd(const void* k, const float* w, const float* dkbar, void* dk, float* dw,
                                float* dw_part, int B, int H, int T_, int D, int dtype, hipStream_t st) {
  if (D > 128) return hipErrorNotSupported;
  const int nb = T_ / DASH_BLOCK;
  dim3 grid(nb, B * H);
  if (dtype == 1)
    pool_attn_bwd_kernel<bf16_t><<<grid, 64, 0, st>>>((const bf16_t*)k, w, dkbar, (bf16_t*)dk, dw_part, H, T_, D);
  else
    pool_attn_bwd_kernel<float><<<grid, 64, 0, st>>>((const float*)k, w, dkbar, (float*)dk, dw_part, H, T_, D);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  reduce_dw_kernel<<<H, 128, 0, st>>>(dw_part, dw, B, H, nb, D);
  return hipGetLastError();
}
