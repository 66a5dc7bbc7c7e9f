// Argument block and launcher of the backward kernels (attn_bwd.hip).
#pragma once

#include "common.h"

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  const void* kbar;
  const float* tau;
  const float* lognorm;
  const int* tile_cnt;
  const int* tile_blk;
  const uint32_t* tile_bits;
  void* dq;
  void* dk;
  void* dv;
  float* dkbar;
  // workspace
  float* delta;    // [BH, T]      dout . o
  float* dq_acc;   // [BH, T, D]   fp32
  float* gbuf;     // [BH, entries, QTILE]  G_ib for listed blocks (entries: bwd_entries_per_head)
  float* pbuf;     // [BH, entries, QTILE]  log2 prior used for (row, listed block)
  float* gsum;     // [BH / grp, entries, QTILE]  G summed over a group's heads (grp > 1)
  float* phbuf;    // [BH, entries, QTILE]  the row's own log2 p (grp > 1)
  int BH, T, D, causal;
  int grp;  // query heads per key/value head: k, v, kbar are indexed by bh / grp
  float fine_scale;
  float pool_scale;  // dK += pool_scale * dkbar of the key's block: 1/64 (mean pooling) or 0
  int dk_f32;        // bf16 path: write dK unrounded, as fp32 [BH, T, D] (another Stage-0 term follows)
  CoarseArith ca;
};

// Entries of the per-(query tile, listed block, row) buffers G and prior: a
// causal tile t lists at most its candidates and its own blocks,
// min(nb, 2t + 2) (a 128-row tile spans two 64-key blocks), so its entries
// start at sum over t' < t of 2t' + 2 = t (t + 1); a non-causal tile lists
// at most nb.
__host__ __device__ inline size_t bwd_tile_base(int causal, int nb, int tile) {
  return causal ? (size_t)tile * (tile + 1) : (size_t)tile * nb;
}
__host__ __device__ inline size_t bwd_entries_per_head(int causal, int nb, int ntile) {
  return causal ? (size_t)(ntile - 1) * ntile + (size_t)(nb < 2 * ntile ? nb : 2 * ntile) : (size_t)ntile * nb;
}

hipError_t launch_bwd(const BwdArgs& a, int dtype, hipStream_t st);
// Grouped-query heads: a.dk, a.dv, a.dkbar receive per-query-head partials
// ([BH, T, D] dtype, [BH, nb, D] f32), summed over each group into dk, dv,
// dkbar ([BH / grp, ...]).
hipError_t launch_bwd_gqa(const BwdArgs& a, void* dk, void* dv, float* dkbar, hipStream_t st);
