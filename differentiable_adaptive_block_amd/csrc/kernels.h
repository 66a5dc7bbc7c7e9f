// Kernel argument blocks and launchers of the DashAttention HIP library.
#pragma once

#include "common.h"


struct SelectArgs {
  const void* q;      // [BH, T, D]
  const void* kbar;   // [BH / grp, nb, D]
  int T, D, causal;
  int grp;            // query heads per key/value head (1: one each)
  CoarseArith ca;
  float* tau;         // [BH, T]
  float* lognorm;     // [BH, T]
  int* nsel;          // [BH, T] or null
  uint32_t* mask;     // [BH, T, nbw] or null
  uint32_t* tile_bits;  // [BH, ntile, nbw], zeroed before the launch
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* kbar;
  void* o;
  float* lse;
  const float* tau;
  const float* lognorm;
  const int* tile_cnt;
  const int* tile_blk;
  int BH, T, D, causal;
  int grp;  // query heads per key/value head: k, v, kbar are indexed by bh / grp
  float fine_scale;
  CoarseArith ca;
};

// The one Stage-1 score accumulation (see select_mfma_kernel): 32 summaries
// (operand A, row = lane % 32 is summary `brow`) against the 32 queries in
// qb (operand B), bf16 MFMA with fp32 accumulation, k-steps in order.
template <int D>
__device__ __forceinline__ f32x16 coarse_acc_chunk(const bf16_t* kb, int brow, const bf16x8 (&qb)[D / 16]) {
  const int h = lane_id() >> 5;
  // all operand loads first, so that they are in flight together
  bf16x8 ka[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) ka[s] = load8(kb + (size_t)brow * D + 16 * s + 8 * h);
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) acc = mfma32(ka[s], qb[s], acc);
  return acc;
}

// The same accumulation with the query operands read from LDS (q_lds: 32
// query rows, row pitch `pitch` bf16) instead of registers: identical MFMA
// sequence and operands, so identical bits.
template <int D>
__device__ __forceinline__ f32x16 coarse_acc_chunk_lds(const bf16_t* kb, int brow, const bf16_t* q_lds, int pitch) {
  const int l = lane_id(), h = l >> 5, j = l & 31;
  bf16x8 ka[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) ka[s] = load8(kb + (size_t)brow * D + 16 * s + 8 * h);
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) acc = mfma32(ka[s], load8(q_lds + j * pitch + 16 * s + 8 * h), acc);
  return acc;
}

// log2 priors of one wave's 32 query rows (lane column j) for the listed
// blocks e0 .. e0+31 of a tile list: lane (j, h) gets slots 8(r/4) + 4h +
// r%4 of row j in register r.  -inf for slots past the list, blocks the
// row did not select, and (causal) the row's own block and later ones.
// The summary loads are issued together, ahead of the MFMAs.
template <int D>
__device__ __forceinline__ f32x16 prior_chunk32(const bf16_t* KB, const int* list, int cnt, int e0,
                                                const bf16x8 (&qb)[D / 16], const CoarseArith& ca, float tau_i,
                                                float ln_i, int causal, int wblk) {
  const int l = lane_id(), j = l & 31;
  const int ent = e0 + j;
  f32x16 pacc = coarse_acc_chunk<D>(KB, ent < cnt ? list[ent] : 0, qb);
  __builtin_amdgcn_sched_group_barrier(0x020, D / 16, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, D / 16, 0);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int en = e0 + acc_row32(r, l);
    float p2 = -INFINITY;
    if (en < cnt) {
      const int bb = list[en];
      if (!causal || bb < wblk) p2 = ca.logp(ca.u_of(pacc[r]), tau_i, ln_i) * 1.4426950408889634f;
    }
    pacc[r] = p2;
  }
  return pacc;
}

// prior_chunk32 for G query heads sharing one key/value head (grouped-query
// heads with entmax head aggregation): the prior of a listed block for this
// lane's row is log2 of pbar = (1/G) sum over the group's heads g of p_g,
// each head's p_g from its own query row at the same position (q0 + g
// head_stride), its own tau and log-normaliser, and the same summaries;
// -inf where no head of the group selected the block (and, causal, for the
// row's own block and later ones).  The list must be the group's union.
template <int D>
__device__ __forceinline__ f32x16 prior_chunk32_group(const bf16_t* KB, const int* list, int cnt, int e0,
                                                      const bf16_t* q0, size_t head_stride, const float* tau0,
                                                      const float* ln0, size_t stat_stride, int G,
                                                      const CoarseArith& ca, int causal, int wblk) {
  const int l = lane_id(), j = l & 31, h = l >> 5;
  const int ent = e0 + j;
  const int brow = ent < cnt ? list[ent] : 0;
  f32x16 psum;
#pragma unroll
  for (int r = 0; r < 16; ++r) psum[r] = 0.f;
  for (int g = 0; g < G; ++g) {
    bf16x8 qb[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qb[s] = load8(q0 + g * head_stride + 16 * s + 8 * h);
    const float tg = tau0[g * stat_stride], lg = ln0[g * stat_stride];
    const f32x16 z = coarse_acc_chunk<D>(KB, brow, qb);
#pragma unroll
    for (int r = 0; r < 16; ++r) psum[r] += __expf(ca.logp(ca.u_of(z[r]), tg, lg));
  }
  const float lg2G = __log2f((float)G);
  f32x16 pacc;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int en = e0 + acc_row32(r, l);
    float p2 = -INFINITY;
    if (en < cnt && psum[r] > 0.f) {
      const int bb = list[en];
      if (!causal || bb < wblk) p2 = __log2f(psum[r]) - lg2G;
    }
    pacc[r] = p2;
  }
  return pacc;
}

// The prior of list entry e for this lane's row from prior_chunk32's
// registers: slot e%32 sits in register 4(slot/8) + slot%4 of the half
// (slot/4)%2; the other half's value comes across with permlane32_swap.
__device__ __forceinline__ float prior_pick(const f32x16& pacc, int e) {
  const int slot = e & 31;
  const int rr = 4 * (slot >> 3) + (slot & 3);
  float v = pacc[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) v = (r == rr) ? pacc[r] : v;
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  // sw[0]: lanes 0-31 keep their value, lanes 32-63 get lanes 0-31's;
  // sw[1]: lanes 0-31 get lanes 32-63's, lanes 32-63 keep theirs
  return __uint_as_float(((slot >> 2) & 1) ? sw[1] : sw[0]);
}

// The generic-path score: sequential fp32 dot product of a query held in
// LDS (as float) with one summary row.
template <typename T>
__device__ __forceinline__ float dot_row(const float* qs, const T* kr, int D) {
  float acc = 0.f;
  for (int d = 0; d < D; ++d) acc = fmaf(qs[d], to_f<T>(kr[d]), acc);
  return acc;
}

hipError_t launch_pool(const void* k, void* kbar, int BH, int T, int D, int dtype, hipStream_t st);
hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t st);
hipError_t launch_select(const SelectArgs& a, int BH, int dtype, hipStream_t st);
hipError_t launch_group_union(uint32_t* tile_bits, int BH, int grp, size_t words_per_head, hipStream_t st);
hipError_t launch_tile_lists(uint32_t* tile_bits, int* tile_cnt, int* tile_blk, int BH, int T, int causal,
                             hipStream_t st);
hipError_t launch_fwd(const FwdArgs& a, int dtype, hipStream_t st);
