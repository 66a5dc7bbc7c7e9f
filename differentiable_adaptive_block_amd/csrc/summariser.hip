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
// bf16, D = 128 (the fast path): one wave per (block, head), four blocks
// per workgroup; the block's 64 keys stay in registers, lane (g, c) =
// (l / 16, l % 16) holding keys 4 it + g (it = 0..15), features 8c..8c+7,
// loaded 1 KB per wave instruction.  Dot products over a key are 8-term
// partials summed across the 16 lanes of a group; sums over keys are
// per-lane partials summed across the 4 groups.  The forward works in fp64
// (scores, softmax and the weighted sum; the sum is exact at w = 0); the
// backward in fp32.
// Other shapes (fp32, D = 64): one wave per block with the keys staged in
// LDS as float with padded rows, lane j owning key j for the scores and lane
// c owning feature c (and c + 64) for the sums.
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
                                                           const float* __restrict__ dk_in, float* __restrict__ dw_part,
                                                           int H, int T_, int D) {
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
  const float* dki = dk_in ? dk_in + row0 * D : nullptr;  // unrounded fp32 terms to add to, or dk itself
  for (int r = 0; r < DASH_BLOCK; ++r) {
    for (int c = l; c < D; c += 64) {
      const float add = fmaf(as[r], gs[c], des[r] * wh[c]);
      const float base = dki ? dki[(size_t)r * D + c] : to_f<T>(dkb[(size_t)r * D + c]);
      dkb[(size_t)r * D + c] = from_f<T>(base + add);
    }
  }
  for (int c = l; c < D; c += 64) {
    float acc = 0.f;
    for (int r = 0; r < DASH_BLOCK; ++r) acc = fmaf(des[r], ks[r][c], acc);
    dw_part[(bh * nb + b) * D + c] = acc;
  }
}

// dw[h][c] = sum over (batch, block) of the partials, in a fixed order:
// grid (H, ceil(D / 16)), 256 threads = 16 columns x 16 row groups; thread
// (c, r) sums the partials r, r + 16, ... of its column, then the 16 sums
// are added in row-group order.
__global__ __launch_bounds__(256) void reduce_dw_kernel(const float* __restrict__ dw_part, float* __restrict__ dw,
                                                        int B, int H, int nb, int D) {
  __shared__ float red[16][17];
  const int h = blockIdx.x;
  const int cl = threadIdx.x & 15, rg = threadIdx.x >> 4;
  const int c = blockIdx.y * 16 + cl;
  float acc = 0.f;
  if (c < D) {
    const int n = B * nb;  // partial rows of head h: (batch bb, block b) -> bb * nb + b
    for (int x = rg; x < n; x += 16) {
      const int bb = x / nb, b = x % nb;
      acc += dw_part[((size_t)(bb * H + h) * nb + b) * D + c];
    }
  }
  red[rg][cl] = acc;
  __syncthreads();
  if (rg == 0 && c < D) {
    float sum = 0.f;
    for (int r = 0; r < 16; ++r) sum += red[r][cl];
    dw[(size_t)h * D + c] = sum;
  }
}

__device__ __forceinline__ void unpack8(const uint4& r, float (&f)[8]) {
  const uint32_t u[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = __uint_as_float(u[e] << 16);
    f[2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  uint32_t u[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) u[e] = (uint32_t)f2bf(f[2 * e]) | ((uint32_t)f2bf(f[2 * e + 1]) << 16);
  return make_uint4(u[0], u[1], u[2], u[3]);
}

template <typename V>
__device__ __forceinline__ V sum16_of(V v) {  // over the 16 lanes of a group
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

template <typename V>
__device__ __forceinline__ V sum_groups(V v) {  // over the 4 groups (lanes l, l^16, l^32, l^48)
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// Hides the key registers' contents from the optimiser between the two
// passes over them, so it unpacks them again instead of keeping all 128
// unpacked values live (which halves the waves that fit on a SIMD).
__device__ __forceinline__ void launder(uint4 (&r)[16]) {
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    uint32_t x = r[it].x, y = r[it].y, z = r[it].z, u = r[it].w;
    asm volatile("" : "+v"(x), "+v"(y), "+v"(z), "+v"(u));
    r[it] = make_uint4(x, y, z, u);
  }
}

// Lane layout and block index shared by the two bf16 kernels.  `total` =
// BH * nb blocks; waves past it do no loads or stores but reach the barriers.
struct Bf16Block {
  int wv, l, g, c, gb;
  bool valid;
  size_t bh;
  __device__ Bf16Block(int H, int T_, int total) {
    wv = threadIdx.x >> 6;
    l = threadIdx.x & 63;
    g = l >> 4;
    c = l & 15;
    gb = blockIdx.x * 4 + wv;  // bh * nb + b
    valid = gb < total;
    const int nb = T_ / DASH_BLOCK;
    bh = valid ? (size_t)(gb / nb) : 0;
    (void)H;
  }
  // row (it * 4 + g) of the block, this lane's 16-byte chunk
  __device__ const bf16_t* row(const bf16_t* base, int T_, int it) const {
    const int nb = T_ / DASH_BLOCK;
    const size_t key0 = bh * T_ + (size_t)(gb % nb) * DASH_BLOCK;
    return base + (key0 + it * 4 + g) * 128 + c * 8;
  }
};

__global__ __launch_bounds__(256) void pool_attn_bf16_kernel(const bf16_t* __restrict__ k, const float* __restrict__ w,
                                                            bf16_t* __restrict__ kbar, int H, int T_, int total) {
  __shared__ double es[4][DASH_BLOCK];
  const Bf16Block t(H, T_, total);
  uint4 kr[16];
#pragma unroll
  for (int it = 0; it < 16; ++it)
    kr[it] = t.valid ? *reinterpret_cast<const uint4*>(t.row(k, T_, it)) : make_uint4(0u, 0u, 0u, 0u);
  double wd[8];
  const float* wh = w + (t.bh % H) * 128 + t.c * 8;
#pragma unroll
  for (int e = 0; e < 8; ++e) wd[e] = t.valid ? (double)wh[e] : 0.0;
  double ek[16];
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    float kf[8];
    unpack8(kr[it], kf);
    double part = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) part = fma(wd[e], (double)kf[e], part);
    ek[it] = sum16_of(part);  // score of key 4 it + g
  }
  if (t.c == 0) {
#pragma unroll
    for (int it = 0; it < 16; ++it) es[t.wv][it * 4 + t.g] = ek[it];
  }
  launder(kr);
  __syncthreads();
  const double e = es[t.wv][t.l];  // lane l: key l
  const double x = exp(e - wave_max_d(e));
  const double a = x / wave_sum_d(x);
  __syncthreads();
  es[t.wv][t.l] = a;
  __syncthreads();
  double acc[8];
#pragma unroll
  for (int e2 = 0; e2 < 8; ++e2) acc[e2] = 0.0;
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const double aj = es[t.wv][it * 4 + t.g];
    float kf[8];
    unpack8(kr[it], kf);
#pragma unroll
    for (int e2 = 0; e2 < 8; ++e2) acc[e2] = fma(aj, (double)kf[e2], acc[e2]);
  }
#pragma unroll
  for (int e2 = 0; e2 < 8; ++e2) acc[e2] = sum_groups(acc[e2]);
  if (t.valid && t.g == 0) {
    uint32_t u[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2)
      u[e2] = (uint32_t)d2bf(acc[2 * e2]) | ((uint32_t)d2bf(acc[2 * e2 + 1]) << 16);
    *reinterpret_cast<uint4*>(kbar + (size_t)t.gb * 128 + t.c * 8) = make_uint4(u[0], u[1], u[2], u[3]);
  }
}

// F32IN: the other dK terms come unrounded from dk_in (fp32, same layout)
// and dk is written once; otherwise dk holds them (bf16) and is updated.
template <bool F32IN>
__global__ __launch_bounds__(256) void pool_attn_bwd_bf16_kernel(const bf16_t* __restrict__ k,
                                                                const float* __restrict__ w,
                                                                const float* __restrict__ dkbar,
                                                                bf16_t* __restrict__ dk,
                                                                const float* __restrict__ dk_in,
                                                                float* __restrict__ dw_part, int H, int T_,
                                                                int total) {
  const Bf16Block t(H, T_, total);
  if (!t.valid) return;  // no barriers in this kernel
  uint4 kr[16], dr[16];
#pragma unroll
  for (int it = 0; it < 16; ++it) kr[it] = *reinterpret_cast<const uint4*>(t.row(k, T_, it));
  if constexpr (!F32IN) {
#pragma unroll
    for (int it = 0; it < 16; ++it) dr[it] = *reinterpret_cast<const uint4*>(t.row(dk, T_, it));
  }
  float wf[8], gf[8];
  const float* wh = w + (t.bh % H) * 128 + t.c * 8;
  const float* gh = dkbar + (size_t)t.gb * 128 + t.c * 8;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    wf[e] = wh[e];
    gf[e] = gh[e];
  }
  float ek[16], kg[16];
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    float kf[8];
    unpack8(kr[it], kf);
    float pe = 0.f, pg = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pe = fmaf(wf[e], kf[e], pe);
      pg = fmaf(gf[e], kf[e], pg);
    }
    ek[it] = sum16_of(pe);  // score of key 4 it + g
    kg[it] = sum16_of(pg);  // k . dkbar of that key
  }
  launder(kr);
  float mx = ek[0];
#pragma unroll
  for (int it = 1; it < 16; ++it) mx = fmaxf(mx, ek[it]);
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  float a[16], s = 0.f;
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    a[it] = __expf(ek[it] - mx);
    s += a[it];
  }
  const float inv = 1.f / sum_groups(s);
  float mg = 0.f;  // kbar . dkbar = sum_j a_j (k_j . dkbar)
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    a[it] *= inv;
    mg = fmaf(a[it], kg[it], mg);
  }
  mg = sum_groups(mg);
  float dwp[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) dwp[e] = 0.f;
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const float de = a[it] * (kg[it] - mg);  // gradient of the key's score
    float kf[8], df[8];
    unpack8(kr[it], kf);
    if constexpr (F32IN) {
      // the same element of the fp32 buffer: dk_in has dk's layout
      const size_t off = t.row(dk, T_, it) - dk;
      const float4 x0 = *reinterpret_cast<const float4*>(dk_in + off);
      const float4 x1 = *reinterpret_cast<const float4*>(dk_in + off + 4);
      df[0] = x0.x; df[1] = x0.y; df[2] = x0.z; df[3] = x0.w;
      df[4] = x1.x; df[5] = x1.y; df[6] = x1.z; df[7] = x1.w;
    } else {
      unpack8(dr[it], df);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      df[e] += fmaf(a[it], gf[e], de * wf[e]);
      dwp[e] = fmaf(de, kf[e], dwp[e]);
    }
    *reinterpret_cast<uint4*>(const_cast<bf16_t*>(t.row(dk, T_, it))) = pack8(df);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) dwp[e] = sum_groups(dwp[e]);
  if (t.g == 0) {
    float* dst = dw_part + (size_t)t.gb * 128 + t.c * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[e] = dwp[e];
  }
}

}  // namespace

hipError_t launch_pool_attn(const void* k, const float* w, void* kbar, int BH, int H, int T_, int D, int dtype,
                            hipStream_t st) {
  if (D > 128) return hipErrorNotSupported;
  dim3 grid(T_ / DASH_BLOCK, BH);
  const int total = BH * (T_ / DASH_BLOCK);
  if (dtype == 1 && D == 128)
    pool_attn_bf16_kernel<<<(total + 3) / 4, 256, 0, st>>>((const bf16_t*)k, w, (bf16_t*)kbar, H, T_, total);
  else if (dtype == 1)
    pool_attn_kernel<bf16_t><<<grid, 64, 0, st>>>((const bf16_t*)k, w, (bf16_t*)kbar, H, T_, D);
  else
    pool_attn_kernel<float><<<grid, 64, 0, st>>>((const float*)k, w, (float*)kbar, H, T_, D);
  return hipGetLastError();
}

hipError_t launch_pool_attn_bwd(const void* k, const float* w, const float* dkbar, void* dk, float* dw,
                                float* dw_part, int B, int H, int T_, int D, int dtype, hipStream_t st,
                                const float* dk_in) {
  if (D > 128) return hipErrorNotSupported;
  const int nb = T_ / DASH_BLOCK;
  dim3 grid(nb, B * H);
  const int total = B * H * nb;
  if (dtype == 1 && D == 128) {
    if (dk_in)
      pool_attn_bwd_bf16_kernel<true><<<(total + 3) / 4, 256, 0, st>>>((const bf16_t*)k, w, dkbar, (bf16_t*)dk, dk_in,
                                                                       dw_part, H, T_, total);
    else
      pool_attn_bwd_bf16_kernel<false><<<(total + 3) / 4, 256, 0, st>>>((const bf16_t*)k, w, dkbar, (bf16_t*)dk,
                                                                        nullptr, dw_part, H, T_, total);
  } else if (dtype == 1)
    pool_attn_bwd_kernel<bf16_t><<<grid, 64, 0, st>>>((const bf16_t*)k, w, dkbar, (bf16_t*)dk, dk_in, dw_part, H, T_,
                                                      D);
  else
    pool_attn_bwd_kernel<float><<<grid, 64, 0, st>>>((const float*)k, w, dkbar, (float*)dk, dk_in, dw_part, H, T_,
                                                     D);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  reduce_dw_kernel<<<dim3(H, (D + 15) / 16), 256, 0, st>>>(dw_part, dw, B, H, nb, D);
  return hipGetLastError();
}
