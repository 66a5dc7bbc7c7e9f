// Kernel argument blocks and launchers of the DashAttention HIP library.
#pragma once

#include "common.h"

#define DASH_DEC_SPLIT 16  // split-KV workgroups per decode row

struct SelectArgs {
  const void* q;      // [BH, T, D]
  const void* kbar;   // [BH, nb, D]
  int T, D, causal;
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
  float fine_scale;
  CoarseArith ca;
};

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
  int BH, T, D, causal;
  float fine_scale;
  CoarseArith ca;
};

struct DecodeArgs {
  const void* q;     // [SH, D]
  const void* kc;    // [SH, N, D]
  const void* vc;
  const void* kbar;  // [SH, nb, D]
  void* o;           // [SH, D]
  float* lse;        // [SH] or null
  int* nsel;         // [SH] or null
  float* tau_out;    // [SH] or null
  // workspace
  float* zrow;       // [SH, nb]       coarse u scores
  float* rowstat;    // [SH, 2]        tau, lognorm
  int* sel_cnt;      // [SH]
  int* sel_blk;      // [SH, nb]       selected candidate blocks, ascending, then the last block
  float* sel_lp;     // [SH, nb]       log2 prior of each listed block
  float* part;       // [SH, nsplit, D + 2] partial (m, l, o)
  int SH, N, D, nsplit, chunk;
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
hipError_t launch_tile_lists(uint32_t* tile_bits, int* tile_cnt, int* tile_blk, int BH, int T, int causal,
                             hipStream_t st);
hipError_t launch_fwd(const FwdArgs& a, int dtype, hipStream_t st);
hipError_t launch_bwd(const BwdArgs& a, int dtype, hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t st);
