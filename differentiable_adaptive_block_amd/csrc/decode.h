// Argument blocks and launchers of the decode kernels (decode.hip).
#pragma once

#include "common.h"

#define DASH_DEC_SPLIT 16      // split-KV workgroups per decode row
#define DASH_DEC_SPLIT_GQA 64  // split-KV workgroups per group of grouped-query decode rows

struct DecodeArgs {
  const void* q;     // [SH, D]
  const void* kc;    // [SH, N, D], N the capacity
  const void* vc;
  const void* kbar;  // [SH, N / 64, D]
  void* o;           // [SH, D]
  float* lse;        // [SH] or null
  int* nsel;         // [SH] or null
  float* tau_out;    // [SH] or null
  uint32_t* mask;    // [SH, ceil(N / 64 / 32)] or null: bit b set iff candidate block b is selected
  // workspace
  float* rowstat;    // [SH, 2]        tau, lognorm
  int* sel_cnt;      // [SH]           list length (0: length out of range)
  int* sel_blk;      // [SH, N / 64]   selected candidate blocks, ascending, then the query's own block
  float* sel_lp;     // [SH, N / 64]   log2 prior of each listed block
  float* part;       // [SH, nsplit, D + 2] partial (m, l, o)
  const int* len;    // [SH / H] tokens per sequence (+ len_add), or null: every row holds N
  int SH, H, N, D, nsplit, chunk, len_add;  // N: cache capacity (row stride in tokens)
  int grp;           // query heads per key/value head (1: one each); kc, vc, kbar rows are row / grp
  float fine_scale;
  CoarseArith ca;
};

// Tokens the decode row holds: len[sequence] + len_add, or the capacity.
__device__ __forceinline__ int decode_row_len(const DecodeArgs& a, int row) {
  return a.len ? a.len[row / a.H] + a.len_add : a.N;
}

struct AppendArgs {
  const void* k_new;  // [SH, D]
  const void* v_new;
  const int* len;     // [SH / H] tokens already cached
  void* kc;           // [SH, N, D]
  void* vc;
  void* kbar;         // [SH, N / 64, D]
  int SH, H, N, D;
};

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t st);
hipError_t launch_append(const AppendArgs& a, int dtype, hipStream_t st);
