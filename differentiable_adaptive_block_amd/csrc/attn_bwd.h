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
  float* gbuf;     // [BH, ntile, nb, QTILE]  G_ib for listed blocks
  float* pbuf;     // [BH, ntile, nb, QTILE]  log2 prior used for (row, listed block)
  float* gsum;     // [BH / grp, ntile, nb, QTILE]  G summed over a group's heads (grp > 1)
  float* phbuf;    // [BH, ntile, nb, QTILE]  the row's own log2 p (grp > 1)
  int BH, T, D, causal;
  int grp;  // query heads per key/value head: k, v, kbar are indexed by bh / grp
  float fine_scale;
  float pool_scale;  // dK += pool_scale * dkbar of the key's block: 1/64 (mean pooling) or 0
  CoarseArith ca;
};

hipError_t launch_bwd(const BwdArgs& a, int dtype, hipStream_t st);
// Grouped-query heads: a.dk, a.dv, a.dkbar receive per-query-head partials
// ([BH, T, D] dtype, [BH, nb, D] f32), summed over each group into dk, dv,
// dkbar ([BH / grp, ...]).
hipError_t launch_bwd_gqa(const BwdArgs& a, void* dk, void* dv, float* dkbar, hipStream_t st);
