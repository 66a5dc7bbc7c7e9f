// Row copies for a causal prefill whose length T is not a multiple of 64:
// the library runs the whole-block kernels on copies padded to Tp = 64
// ceil(T / 64) rows per head (in the caller's workspace) and copies the
// first T rows of each result back.  Padding rows hold zeros (queries,
// keys, values, outputs, output gradients) or a given value (the
// log-sum-exp of the padded rows, +inf, so their weights are 0).  Under the
// causal mask no real query attends a padded key, and the padded block is
// no query's candidate, so the real rows are those of the unpadded problem.
#include "ragged.h"

namespace {

// dst[bh][t] = t < T ? src[bh][t] : 0, in 16-byte pieces (rb = row bytes).
__global__ void pad_rows_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int BH, int T, int Tp,
                                int rb16) {
  const size_t n = (size_t)BH * Tp * rb16;
  for (size_t x = (size_t)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += (size_t)gridDim.x * blockDim.x) {
    const size_t c = x % rb16, row = x / rb16;
    const size_t bh = row / Tp, t = row % Tp;
    dst[x] = t < (size_t)T ? src[(bh * T + t) * rb16 + c] : make_uint4(0u, 0u, 0u, 0u);
  }
}

// dst[bh][t] = src[bh][t] for t < T, from rows of Tp.
__global__ void unpad_rows_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int BH, int T, int Tp,
                                  int rb16) {
  const size_t n = (size_t)BH * T * rb16;
  for (size_t x = (size_t)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += (size_t)gridDim.x * blockDim.x) {
    const size_t c = x % rb16, row = x / rb16;
    const size_t bh = row / T, t = row % T;
    dst[x] = src[(bh * Tp + t) * rb16 + c];
  }
}

__global__ void pad_f32_kernel(const float* __restrict__ src, float* __restrict__ dst, int BH, int T, int Tp,
                               float fill) {
  const size_t n = (size_t)BH * Tp;
  for (size_t x = (size_t)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += (size_t)gridDim.x * blockDim.x) {
    const size_t bh = x / Tp, t = x % Tp;
    dst[x] = t < (size_t)T ? src[bh * T + t] : fill;
  }
}

__global__ void unpad_f32_kernel(const float* __restrict__ src, float* __restrict__ dst, int BH, int T, int Tp) {
  const size_t n = (size_t)BH * T;
  for (size_t x = (size_t)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += (size_t)gridDim.x * blockDim.x) {
    const size_t bh = x / T, t = x % T;
    dst[x] = src[bh * Tp + t];
  }
}

}  // namespace

hipError_t launch_pad_rows(const void* src, void* dst, int BH, int T, int Tp, int row_bytes, hipStream_t st) {
  if (row_bytes % 16) return hipErrorInvalidValue;
  pad_rows_kernel<<<2048, 256, 0, st>>>(static_cast<const uint4*>(src), static_cast<uint4*>(dst), BH, T, Tp,
                                        row_bytes / 16);
  return hipGetLastError();
}

hipError_t launch_unpad_rows(const void* src, void* dst, int BH, int T, int Tp, int row_bytes, hipStream_t st) {
  if (row_bytes % 16) return hipErrorInvalidValue;
  unpad_rows_kernel<<<2048, 256, 0, st>>>(static_cast<const uint4*>(src), static_cast<uint4*>(dst), BH, T, Tp,
                                          row_bytes / 16);
  return hipGetLastError();
}

hipError_t launch_pad_f32(const float* src, float* dst, int BH, int T, int Tp, float fill, hipStream_t st) {
  pad_f32_kernel<<<512, 256, 0, st>>>(src, dst, BH, T, Tp, fill);
  return hipGetLastError();
}

hipError_t launch_unpad_f32(const float* src, float* dst, int BH, int T, int Tp, hipStream_t st) {
  unpad_f32_kernel<<<512, 256, 0, st>>>(src, dst, BH, T, Tp);
  return hipGetLastError();
}
