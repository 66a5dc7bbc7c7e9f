// Stage 0 (block pooling) and Stage 1 (block scores + alpha-entmax + tile lists).
//
// Stage 0: the pages' summariser starts from mean pooling ("What
// alpha-entmax changes", montana-research page).  Stage 1: coarse scores
// q . kbar and alpha-entmax over them ("Core Mechanism", alanhou.org page).
#include "kernels.h"
#include "entmax.h"

// ---------------------------------------------------------------------------- Stage 0

// kbar[bh][b][d] = mean of k[bh][64 b + r][d] over r, summed in fp64 (exact for
// bf16 keys and for fp32 keys of ordinary magnitude), divided by 64 (exact)
// and rounded once to the storage type.  grid (nb, BH), 64 threads.  k has
// Tr rows per head (the row stride); rows at or past Tr (the missing rows
// of a partial last block) count as zeros.
template <typename T>
__global__ __launch_bounds__(64) void pool_kernel(const T* __restrict__ k, T* __restrict__ kbar, int T_, int Tr,
                                                  int D) {
  const int b = blockIdx.x;
  const size_t bh = blockIdx.y;
  const int nb = T_ / DASH_BLOCK;
  const T* src = k + (bh * Tr + (size_t)b * DASH_BLOCK) * D;
  const int nrow = min(DASH_BLOCK, Tr - b * DASH_BLOCK);
  T* dst = kbar + (bh * nb + b) * D;
  for (int c = threadIdx.x; c < D; c += 64) {
    double acc = 0.0;
    for (int r = 0; r < nrow; ++r) acc += to_d<T>(src[(size_t)r * D + c]);
    double mean = acc * (1.0 / DASH_BLOCK);
    if constexpr (sizeof(T) == 2) dst[c] = d2bf(mean);
    else dst[c] = __double2float_rn(mean);
  }
}

// bf16 keys, D in {64, 128}: the same exact fp64 sums with 16-byte loads.
// D/8 lanes cover a key row, so one wave load instruction reads 64/(D/8)
// consecutive rows (1 KB); lane l sums the rows l/(D/8) + (64/(D/8)) x of
// its 8 columns, then the row groups are added across lanes (xor
// shuffles).  A bf16 value carries 8 significant bits and 64 of them add at
// most 6 bits of carry, so every partial sum fits a double's 53 bits exactly
// while a block's non-zero magnitudes lie within 2^39 of each other (any
// realistic key block): then the order does not change the result, and it
// equals the sequential sum.  Beyond that range the lane-split order here and
// the position order of other summers may round differently.
// grid (nb, BH), 64 threads.
template <int D>
__global__ __launch_bounds__(64) void pool_bf16_kernel(const bf16_t* __restrict__ k, bf16_t* __restrict__ kbar,
                                                       int T_, int Tr) {
  constexpr int CPL = D / 8;            // lanes per key row
  constexpr int RPI = 64 / CPL;         // rows per load instruction
  constexpr int NL = DASH_BLOCK / RPI;  // loads per lane
  const int b = blockIdx.x;
  const size_t bh = blockIdx.y;
  const int nb = T_ / DASH_BLOCK;
  const int l = threadIdx.x;
  const int c = l % CPL, r0 = l / CPL;
  const bf16_t* src = k + (bh * Tr + (size_t)b * DASH_BLOCK + r0) * D + 8 * c;
  const int nrow = Tr - b * DASH_BLOCK;  // rows of the block in the tensor (rows past it count as zeros)
  uint4 raw[NL];
#pragma unroll
  for (int x = 0; x < NL; ++x)
    raw[x] = r0 + RPI * x < nrow ? *reinterpret_cast<const uint4*>(src + (size_t)RPI * x * D) : make_uint4(0, 0, 0, 0);
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
#pragma unroll
  for (int x = 0; x < NL; ++x) {
    const uint32_t wv[4] = {raw[x].x, raw[x].y, raw[x].z, raw[x].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += (double)__uint_as_float(wv[e] << 16);
      acc[2 * e + 1] += (double)__uint_as_float(wv[e] & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int o = CPL; o < 64; o <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
  if (l < CPL) {
    uint32_t pk[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      pk[e] = (uint32_t)d2bf(acc[2 * e] * (1.0 / DASH_BLOCK)) | ((uint32_t)d2bf(acc[2 * e + 1] * (1.0 / DASH_BLOCK)) << 16);
    *reinterpret_cast<uint4*>(kbar + (bh * nb + b) * D + 8 * c) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  }
}

__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

// ---------------------------------------------------------------------------- Stage 1 outputs

// Writes tau / lognorm / nsel / mask for one row (lane 0 writes the scalars)
// and returns nothing; `uni` receives the row's selected bits (OR).
template <int NPL>
__device__ __forceinline__ void write_row_selection(const SelectArgs& a, size_t row_g, const float (&u)[NPL],
                                                    int nc, const EntmaxOut& e, const CoarseArith& ca,
                                                    uint32_t* uni_lds, uint32_t* tile_bits_g) {
  const int l = lane_id();
  const int nbw = (a.T / DASH_BLOCK + 31) / 32;
  if (l == 0) {
    a.tau[row_g] = e.tau;
    a.lognorm[row_g] = e.lognorm;
    if (a.nsel) a.nsel[row_g] = e.nsel;
    if (a.passes) a.passes[row_g] = e.passes;
  }
#pragma unroll
  for (int k = 0; k < NPL; ++k) {
    const int idx = l + 64 * k;
    unsigned long long bal = __ballot(idx < nc && ca.selected(u[k], e.tau));
    const uint32_t lo = (uint32_t)bal, hi = (uint32_t)(bal >> 32);
    if (l == 0) {
      if (2 * k < nbw) {
        if (a.mask) a.mask[row_g * nbw + 2 * k] = lo;
        if (lo) {
          if (uni_lds) atomicOr(&uni_lds[2 * k], lo);
          else atomicOr(&tile_bits_g[2 * k], lo);
        }
      }
      if (2 * k + 1 < nbw) {
        if (a.mask) a.mask[row_g * nbw + 2 * k + 1] = hi;
        if (hi) {
          if (uni_lds) atomicOr(&uni_lds[2 * k + 1], hi);
          else atomicOr(&tile_bits_g[2 * k + 1], hi);
        }
      }
    }
  }
}

__device__ __forceinline__ void write_empty_row(const SelectArgs& a, size_t row_g) {
  const int l = lane_id();
  const int nbw = (a.T / DASH_BLOCK + 31) / 32;
  if (l == 0) {
    a.tau[row_g] = __uint_as_float(0x7fc00000u);
    a.lognorm[row_g] = 0.f;
    if (a.nsel) a.nsel[row_g] = 0;
    if (a.passes) a.passes[row_g] = 0;
  }
  if (a.mask)
    for (int w = l; w < nbw; w += 64) a.mask[row_g * nbw + w] = 0u;
}

// Four rows per wave, 16 lanes per row: lane g of the group holds
// candidates g + 16 k.  Word w of a row's mask takes its low 16 bits from
// k = 2w and its high 16 bits from k = 2w + 1; lane g writes words g + 16 j
// and ORs them into the tile's union in LDS.
template <int NPL>
__device__ __forceinline__ void write_rows16(const SelectArgs& a, size_t row_g, const float (&u)[NPL], int nc,
                                             const EntmaxOut& e, const CoarseArith& ca, uint32_t* uni_lds) {
  const int l = lane_id(), g = l & 15, sh = l & 48;
  const int nbw = (a.T / DASH_BLOCK + 31) / 32;
  if (g == 0) {
    a.tau[row_g] = e.tau;
    a.lognorm[row_g] = e.lognorm;
    if (a.nsel) a.nsel[row_g] = e.nsel;
    if (a.passes) a.passes[row_g] = e.passes;
  }
  constexpr int NW = (NPL + 1) / 2;
  constexpr int NJ = (NW + 15) / 16;
  uint32_t mine[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) mine[j] = 0u;
#pragma unroll
  for (int wd = 0; wd < NW; ++wd) {
    if (32 * wd < nc) {  // nc is the same on every lane
      const int k0 = 2 * wd, k1 = 2 * wd + 1;
      const unsigned long long b0 = __ballot(g + 16 * k0 < nc && ca.selected(u[k0], e.tau));
      unsigned long long b1 = 0ull;
      if (k1 < NPL) b1 = __ballot(g + 16 * k1 < nc && ca.selected(u[k1], e.tau));
      const uint32_t word = (uint32_t)((b0 >> sh) & 0xFFFFull) | ((uint32_t)((b1 >> sh) & 0xFFFFull) << 16);
      if (g == (wd & 15)) mine[wd >> 4] = word;
    }
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int idx = g + 16 * j;
    if (idx < nbw) {
      if (a.mask) a.mask[row_g * nbw + idx] = mine[j];
      if (mine[j]) atomicOr(&uni_lds[idx], mine[j]);
    }
  }
}

// ---------------------------------------------------------------------------- Stage 1, bf16 MFMA

// One workgroup (4 or 8 waves) per 32 query rows.  The block scores of the 32
// rows (all inside one 64-block, so they share their causal candidates) are
// computed 32 blocks at a time on the 32x32x16 bf16 MFMA as
//     Z^T[block][query] = kbar[block] . q[query]
// (operand A = summary rows, B = the queries, fp32 accumulation) and kept in
// LDS as u = (alpha-1) * coarse_scale * acc; then each wave solves tau for
// its rows (8 with 4 waves, 4 with 8), four at a time (16 lanes per row, see
// entmax_solve).
// coarse_acc_chunk() is the one definition of the score arithmetic; the
// Stage-2 and backward kernels call it too, so they see the same bits.
template <int D, int NPL, int NW>
__global__ __launch_bounds__(64 * NW) void select_mfma_kernel(SelectArgs a) {
  constexpr int RPW = 32 / NW;   // rows per wave, solved 4 at a time
  extern __shared__ float zs[];  // [32][nb + 1] followed by nbw union words
  const int nb = a.T / DASH_BLOCK;
  const int nbp = nb + 1;
  const int nbw = (nb + 31) / 32;
  uint32_t* uni = reinterpret_cast<uint32_t*>(zs + 32 * nbp);
  const size_t bh = blockIdx.y;
  const int row0 = (gridDim.x - 1 - blockIdx.x) * 32;  // last rows (most causal candidates) first
  const int w = threadIdx.x >> 6, l = lane_id(), j = l & 31, h = l >> 5;
  const int nc = a.causal ? row0 / DASH_BLOCK : nb;
  const CoarseArith ca = a.ca;
  for (int x = threadIdx.x; x < nbw; x += 64 * NW) uni[x] = 0u;

  const bf16_t* qh = reinterpret_cast<const bf16_t*>(a.q) + bh * a.Tr * D;
  const bf16_t* kb = reinterpret_cast<const bf16_t*>(a.kbar) + (bh / a.grp) * nb * D;
  if (nc > 0) {
    bf16x8 qb[D / 16];
    const bool qin = row0 + j < a.Tr;  // rows past the tensor (a partial last block) are zero queries
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      qb[s] = qin ? load8(qh + (size_t)(row0 + j) * D + 16 * s + 8 * h) : bf16x8{};
    // the next sub-chunk's summaries are requested once this one's
    // products have read theirs
    bf16x8 ka[D / 16];
    coarse_load_kbar<D>(kb, w * 32 + j < nc ? w * 32 + j : 0, ka);
    for (int c = w; c * 32 < nc; c += NW) {
      f32x16 acc = coarse_acc_q<D>(ka, qb);
      const int cn = c + NW;
      if (cn * 32 < nc) coarse_load_kbar<D>(kb, cn * 32 + j < nc ? cn * 32 + j : 0, ka);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int b = c * 32 + acc_row32(r, l);
        if (b < nc) zs[j * nbp + b] = ca.u_of(acc[r]);
      }
    }
  }
  __syncthreads();
  const int g = l & 15;
  for (int pass = 0; pass < RPW / 4; ++pass) {
    const int row = RPW * w + 4 * pass + (l >> 4);
    const size_t row_g = bh * a.T + row0 + row;
    if (nc == 0) {
      if (g == 0) {
        a.tau[row_g] = __uint_as_float(0x7fc00000u);
        a.lognorm[row_g] = 0.f;
        if (a.nsel) a.nsel[row_g] = 0;
        if (a.passes) a.passes[row_g] = 0;
      }
      if (a.mask)
        for (int x = g; x < nbw; x += 16) a.mask[row_g * nbw + x] = 0u;
      continue;
    }
    float u[NPL];
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      const int idx = g + 16 * k;
      u[k] = idx < nc ? zs[row * nbp + idx] : -INFINITY;
    }
    const EntmaxOut e = entmax_solve<NPL, 16>(u, nc, ca, a.nsel != nullptr);
    write_rows16<NPL>(a, row_g, u, nc, e, ca, uni);
  }
  __syncthreads();
  const int ntile = (a.T + DASH_QTILE - 1) / DASH_QTILE;
  uint32_t* tb = a.tile_bits + (bh * ntile + row0 / DASH_QTILE) * nbw;
  for (int x = threadIdx.x; x < nbw; x += 64 * NW)
    if (uni[x]) atomicOr(&tb[x], uni[x]);
}

// Long sequences (more than 256 blocks): the same computation with the score
// tile staged 256 blocks at a time (32 rows x 257 floats of LDS), the query
// operands read from LDS and each wave keeping its 4 rows' scores in
// registers, so that two 8-wave workgroups fit on a CU.  Lane g of a row's 16 holds candidates g + 16 k,
// chunk ch filling k = 16 ch .. 16 ch + 15.
template <int D, int NPL>
__global__ __launch_bounds__(512, NPL > 64 ? 2 : 4) void select_chunked_kernel(SelectArgs a) {
  constexpr int CB = 256;
  constexpr int NCH = NPL / 16;
  constexpr int QP = D + 8;
  __shared__ float zs[32 * (CB + 1)];
  __shared__ __attribute__((aligned(16))) bf16_t qs[32 * QP];  // the 32 query rows
  __shared__ uint32_t uni[DASH_MAX_NB / 32];
  const int nb = a.T / DASH_BLOCK;
  const int nbw = (nb + 31) / 32;
  const size_t bh = blockIdx.y;
  const int row0 = (gridDim.x - 1 - blockIdx.x) * 32;  // last rows (most causal candidates) first
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = lane_id(), j = l & 31, g = l & 15;
  const int nc = a.causal ? row0 / DASH_BLOCK : nb;
  const CoarseArith ca = a.ca;
  for (int x = tid; x < nbw; x += 512) uni[x] = 0u;
  const int row = 4 * w + (l >> 4);
  const size_t row_g = bh * a.T + row0 + row;

  const bf16_t* qh = reinterpret_cast<const bf16_t*>(a.q) + bh * a.Tr * D;
  const bf16_t* kb = reinterpret_cast<const bf16_t*>(a.kbar) + (bh / a.grp) * nb * D;
  float u[NPL];
  if (nc > 0) {
    // this wave's summaries of chunk ch: sub-chunk 8 ch + w of 32 blocks;
    // those of the next chunk are requested as soon as this chunk's products
    // have read theirs, so their latency overlaps the score tile's hand-over
    auto brow_of = [&](int ch) { const int b = (ch * CB / 32 + w) * 32 + j; return b < nc ? b : 0; };
    bf16x8 ka[D / 16];
    coarse_load_kbar<D>(kb, brow_of(0), ka);
    for (int x = tid; x < 32 * (D / 8); x += 512) {
      const int r = x / (D / 8), c8 = x % (D / 8);
      *reinterpret_cast<uint4*>(&qs[r * QP + 8 * c8]) =
          row0 + r < a.Tr ? *reinterpret_cast<const uint4*>(qh + (size_t)(row0 + r) * D + 8 * c8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      const int c0 = ch * CB;
      if (c0 < nc) {  // the same on every thread
        __syncthreads();  // the previous chunk's reads are done (first chunk: the queries are staged)
        const int c = c0 / 32 + w;  // 8 sub-chunks of 32 blocks, one per wave
        if (c * 32 < nc) {
          const f32x16 acc = coarse_acc_lds<D>(ka, qs, QP);
          if (ch + 1 < NCH && c0 + CB < nc) coarse_load_kbar<D>(kb, brow_of(ch + 1), ka);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int b = c * 32 + acc_row32(r, l);
            if (b < nc) zs[j * (CB + 1) + (b - c0)] = ca.u_of(acc[r]);
          }
        } else if (ch + 1 < NCH && c0 + CB < nc) {
          coarse_load_kbar<D>(kb, brow_of(ch + 1), ka);
        }
        __syncthreads();
      }
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) {
        const int idx = c0 + g + 16 * kk;
        u[16 * ch + kk] = idx < nc ? zs[row * (CB + 1) + g + 16 * kk] : -INFINITY;
      }
    }
  }
  if (nc == 0) {
    if (g == 0) {
      a.tau[row_g] = __uint_as_float(0x7fc00000u);
      a.lognorm[row_g] = 0.f;
      if (a.nsel) a.nsel[row_g] = 0;
      if (a.passes) a.passes[row_g] = 0;
    }
    if (a.mask)
      for (int x = g; x < nbw; x += 16) a.mask[row_g * nbw + x] = 0u;
  } else {
    const EntmaxOut e = entmax_solve<NPL, 16>(u, nc, ca, a.nsel != nullptr);
    write_rows16<NPL>(a, row_g, u, nc, e, ca, uni);
  }
  __syncthreads();
  const int ntile = (a.T + DASH_QTILE - 1) / DASH_QTILE;
  uint32_t* tb = a.tile_bits + (bh * ntile + row0 / DASH_QTILE) * nbw;
  for (int x = tid; x < nbw; x += 512)
    if (uni[x]) atomicOr(&tb[x], uni[x]);
}

// ---------------------------------------------------------------------------- Stage 1, generic

// One wave per query row; scores by a sequential fp32 dot product
// (dot_row), the same function the generic Stage-2 kernel uses.
template <typename T, int NPL>
__global__ __launch_bounds__(64) void select_generic_kernel(SelectArgs a) {
  __shared__ float qs[128];
  const int D = a.D;
  const int nb = a.T / DASH_BLOCK;
  const int nbw = (nb + 31) / 32;
  const size_t bh = blockIdx.y;
  const int i = blockIdx.x;
  const int l = lane_id();
  const T* q = reinterpret_cast<const T*>(a.q) + (bh * a.Tr + i) * D;
  const T* kb = reinterpret_cast<const T*>(a.kbar) + (bh / a.grp) * nb * D;
  for (int d = l; d < D; d += 64) qs[d] = i < a.Tr ? to_f<T>(q[d]) : 0.f;
  __syncthreads();
  const int nc = a.causal ? i / DASH_BLOCK : nb;
  const size_t row_g = bh * a.T + i;
  if (nc == 0) {
    write_empty_row(a, row_g);
    return;
  }
  const CoarseArith ca = a.ca;
  float u[NPL];
#pragma unroll
  for (int k = 0; k < NPL; ++k) {
    const int b = l + 64 * k;
    u[k] = b < nc ? ca.u_of(dot_row<T>(qs, kb + (size_t)b * D, D)) : -INFINITY;
  }
  const EntmaxOut e = entmax_solve<NPL, 64>(u, nc, ca, a.nsel != nullptr);
  const int ntile = (a.T + DASH_QTILE - 1) / DASH_QTILE;
  uint32_t* tb = a.tile_bits + (bh * ntile + i / DASH_QTILE) * nbw;
  write_row_selection<NPL>(a, row_g, u, nc, e, ca, nullptr, tb);
}

// ---------------------------------------------------------------------------- tile lists

// Per query tile: add the tile's own blocks (causal), write the bit set back
// and compact it into an ascending block list.  grid (ntile, BH), 64 threads;
// nbw <= 32.
__global__ __launch_bounds__(64) void tile_list_kernel(uint32_t* tile_bits, int* tile_cnt, int* tile_blk, int T_,
                                                       int causal) {
  const int nb = T_ / DASH_BLOCK;
  const int nbw = (nb + 31) / 32;
  const int ntile = (T_ + DASH_QTILE - 1) / DASH_QTILE;
  const size_t t = (size_t)blockIdx.y * ntile + blockIdx.x;
  const int l = lane_id();
  uint32_t word = l < nbw ? tile_bits[t * nbw + l] : 0u;
  if (causal) {
    const int r0 = blockIdx.x * DASH_QTILE;
    const int r1 = min(T_, r0 + DASH_QTILE) - 1;
    for (int b = r0 / DASH_BLOCK; b <= r1 / DASH_BLOCK; ++b)
      if ((b >> 5) == l) word |= 1u << (b & 31);
  }
  if (l < nbw) tile_bits[t * nbw + l] = word;
  const int c = __popc(word);
  int incl = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(incl, o, 64);
    if (l >= o) incl += y;
  }
  int pos = incl - c;
  int* dst = tile_blk + t * nb;
  while (word) {
    const int bit = __ffs(word) - 1;
    word &= word - 1;
    dst[pos++] = l * 32 + bit;
  }
  if (l == 63) tile_cnt[t] = incl;
}

// ---------------------------------------------------------------------------- launchers

hipError_t launch_pool(const void* k, void* kbar, int BH, int T_, int D, int dtype, hipStream_t st, int Tr) {
  if (Tr < 0) Tr = T_;
  dim3 grid(T_ / DASH_BLOCK, BH);
  if (dtype == 1 && D == 128)
    pool_bf16_kernel<128><<<grid, 64, 0, st>>>((const bf16_t*)k, (bf16_t*)kbar, T_, Tr);
  else if (dtype == 1 && D == 64)
    pool_bf16_kernel<64><<<grid, 64, 0, st>>>((const bf16_t*)k, (bf16_t*)kbar, T_, Tr);
  else if (dtype == 1)
    pool_kernel<bf16_t><<<grid, 64, 0, st>>>((const bf16_t*)k, (bf16_t*)kbar, T_, Tr, D);
  else
    pool_kernel<float><<<grid, 64, 0, st>>>((const float*)k, (float*)kbar, T_, Tr, D);
  return hipGetLastError();
}

// Grouped-query heads share one block list per tile: OR the tile bit sets
// of the grp heads of each group and give every head of the group the union.
__global__ void group_union_kernel(uint32_t* bits, int ngroups, int grp, size_t words) {
  const size_t n = (size_t)ngroups * words;
  for (size_t x = (size_t)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += (size_t)gridDim.x * blockDim.x) {
    const size_t g = x / words, wi = x % words;
    uint32_t* base = bits + g * grp * words + wi;
    uint32_t u = 0;
    for (int h = 0; h < grp; ++h) u |= base[(size_t)h * words];
    for (int h = 0; h < grp; ++h) base[(size_t)h * words] = u;
  }
}

hipError_t launch_group_union(uint32_t* tile_bits, int BH, int grp, size_t words_per_head, hipStream_t st) {
  if (grp <= 1) return hipSuccess;
  group_union_kernel<<<1024, 256, 0, st>>>(tile_bits, BH / grp, grp, words_per_head);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t st) {
  if (n == 0) return hipSuccess;
  int blocks = (int)((n + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  fill_u32_kernel<<<blocks, 256, 0, st>>>(p, n, v);
  return hipGetLastError();
}

template <int D, int NPL>
static hipError_t launch_select_mfma_t(const SelectArgs& a, int BH, hipStream_t st) {
  const int nb = a.T / DASH_BLOCK;
  const size_t lds = (size_t)32 * (nb + 1) * sizeof(float) + ((nb + 31) / 32) * sizeof(uint32_t);
  // long sequences: the score tile fills most of the LDS, so one workgroup
  // per CU; give it 8 waves (4 rows each) instead of 4
  constexpr int NW = NPL >= 32 ? 8 : 4;
  auto kfn = select_mfma_kernel<D, NPL, NW>;
  hipError_t e = hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  kfn<<<dim3(a.T / 32, BH), 64 * NW, lds, st>>>(a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_select_mfma_d(const SelectArgs& a, int BH, hipStream_t st) {
  const int nb = a.T / DASH_BLOCK;
  // candidates per lane at 16 lanes per row
  if (nb <= 64) return launch_select_mfma_t<D, 4>(a, BH, st);
  if (nb <= 128) return launch_select_mfma_t<D, 8>(a, BH, st);
  if (nb <= 256) return launch_select_mfma_t<D, 16>(a, BH, st);
  // longer: score tile staged in 256-block chunks
  if (nb <= 512) {
    select_chunked_kernel<D, 32><<<dim3(a.T / 32, BH), 512, 0, st>>>(a);
    return hipGetLastError();
  }
  if (nb <= 1024) {
    select_chunked_kernel<D, 64><<<dim3(a.T / 32, BH), 512, 0, st>>>(a);
    return hipGetLastError();
  }
  // beyond 64K tokens: 96 scores per lane, one 8-wave workgroup per CU
  select_chunked_kernel<D, 96><<<dim3(a.T / 32, BH), 512, 0, st>>>(a);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_select_generic_t(const SelectArgs& a, int BH, hipStream_t st) {
  const int nb = a.T / DASH_BLOCK;
  dim3 grid(a.T, BH);
  if (nb <= 64) select_generic_kernel<T, 1><<<grid, 64, 0, st>>>(a);
  else if (nb <= 128) select_generic_kernel<T, 2><<<grid, 64, 0, st>>>(a);
  else if (nb <= 256) select_generic_kernel<T, 4><<<grid, 64, 0, st>>>(a);
  else if (nb <= 512) select_generic_kernel<T, 8><<<grid, 64, 0, st>>>(a);
  else if (nb <= 1024) select_generic_kernel<T, 16><<<grid, 64, 0, st>>>(a);
  else select_generic_kernel<T, 24><<<grid, 64, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, int BH, int dtype, hipStream_t st) {
  if (dtype == 1) return a.D == 128 ? launch_select_mfma_d<128>(a, BH, st) : launch_select_mfma_d<64>(a, BH, st);
  return launch_select_generic_t<float>(a, BH, st);
}

hipError_t launch_tile_lists(uint32_t* tile_bits, int* tile_cnt, int* tile_blk, int BH, int T_, int causal,
                             hipStream_t st) {
  const int ntile = (T_ + DASH_QTILE - 1) / DASH_QTILE;
  tile_list_kernel<<<dim3(ntile, BH), 64, 0, st>>>(tile_bits, tile_cnt, tile_blk, T_, causal);
  return hipGetLastError();
}
