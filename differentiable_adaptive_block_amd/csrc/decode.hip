// Decode: one new query per (sequence, head) against a long KV cache
// (the pages' decoding path; their speed claim is at 96K context with
// 93.75% block sparsity, "The numbers" on the montana-research page).
// The new token is the last cached token.  A row whose cache holds n tokens
// (n = the capacity N, or a length per sequence) has its query at n-1: its
// candidates are the complete blocks 0..own-1, own = (n-1)/64, and its own
// block is attended over its cached tokens with prior 0.
//
// Cache maintenance, decode_append: one wave per row writes the new key and
// value at position len and, when that completes a block, the block's
// summary (the decoding path keeps one summary per 64-token chunk of the
// cache; chunk-summarise stage of the code samples listed by the
// codewithpapers.app entry for the DashAttention paper).
//
// Three decode kernels, HBM-bound:
//   decode_select   one 4-wave workgroup per row: u = (alpha-1) * coarse_scale
//                   * q.kbar_b for every candidate (a coalesced GEMV over the
//                   row's summaries, two rounds of loads in flight) into LDS,
//                   then on one wave the entmax threshold, mask words and the
//                   compacted ascending list of the selected blocks with their
//                   log2 prior, then the last block;
//   decode_attend   split-KV: workgroup (split s, row) and its 4 waves take list
//                   entries s*4 + w, stepping by 4*nsplit; each wave streams a
//                   block's 64 keys and values (16 KB each, contiguous) with
//                   16-byte loads, 1 KB per wave instruction, online softmax,
//                   the next entry's K requested once the scores are formed
//                   and its V once the weighted sum is done;
//                   the 4 waves merge in LDS and write one partial (m, l, o);
//   decode_combine  merges the nsplit partials of a row (one wave per row).
#include "kernels.h"
#include "decode.h"
#include "entmax.h"
#include "tiles.h"

#define LOG2E_F 1.4426950408889634f
#define LN2_F 0.6931471805599453f

// 16 lanes share one 256-byte row (D = 128): lane l holds 8 elements at
// chunk (l % 16).  Returns the sum over the 16 lanes (a DPP row).
__device__ __forceinline__ float sum16(float v) { return row16_sum(v); }

__device__ __forceinline__ void unpack8(const uint4& r, float (&f)[8]) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = __uint_as_float(w[e] << 16);
    f[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
  }
}

// ---------------------------------------------------------------------------- selection

// Block scores of one decode row: u_b = (alpha-1) coarse_scale q . kbar_b
// for the candidates b < nc, into LDS.  The workgroup's 4 waves read 16
// summary rows per instruction round (16 lanes per 256-byte row, 8
// elements each); a lane keeps two rounds of DEC_UN 16-byte loads in
// flight, so one 4-wave workgroup per row streams the row's summaries at
// full rate.
#define DEC_UN 8                    // 16-byte loads per lane per round
#define DEC_SPR (4 * 4 * DEC_UN)    // summary rows per round of the workgroup
__device__ __forceinline__ void decode_row_scores(const DecodeArgs& a, int row, int nc, float* zs) {
  constexpr int D = 128;
  const int nbc = a.N / DASH_BLOCK;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const bf16_t* q = reinterpret_cast<const bf16_t*>(a.q) + (size_t)row * D;
  const bf16_t* kb = reinterpret_cast<const bf16_t*>(a.kbar) + (size_t)(row / a.grp) * nbc * D + (l & 15) * 8;
  const CoarseArith ca = a.ca;
  float qf[8];
  unpack8(*reinterpret_cast<const uint4*>(q + (l & 15) * 8), qf);
  auto bof = [&](int b0, int x) { return b0 + (x * 4 + w) * 4 + (l >> 4); };
  uint4 R[2][DEC_UN];
  auto load = [&](int b0, uint4 (&r)[DEC_UN]) {
#pragma unroll
    for (int x = 0; x < DEC_UN; ++x) {
      const int b = bof(b0, x);
      r[x] = b < nc ? *reinterpret_cast<const uint4*>(kb + (size_t)b * D) : make_uint4(0, 0, 0, 0);
    }
  };
  auto score = [&](int b0, const uint4 (&r)[DEC_UN]) {
#pragma unroll
    for (int x = 0; x < DEC_UN; ++x) {
      const int b = bof(b0, x);
      float kf[8];
      unpack8(r[x], kf);
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) part = fmaf(qf[e], kf[e], part);
      part = sum16(part);
      if (b < nc && (l & 15) == 0) zs[b] = ca.u_of(part);
    }
  };
  // rounds alternate between the two register sets (unrolled by two so
  // that each set keeps fixed registers)
  load(0, R[0]);
  for (int b0 = 0; b0 < nc; b0 += 2 * DEC_SPR) {
    if (b0 + DEC_SPR < nc) load(b0 + DEC_SPR, R[1]);
    score(b0, R[0]);
    if (b0 + DEC_SPR >= nc) break;
    if (b0 + 2 * DEC_SPR < nc) load(b0 + 2 * DEC_SPR, R[0]);
    score(b0 + DEC_SPR, R[1]);
  }
}

// The scores of the G query heads of a group (rows row0 .. row0 + G - 1)
// over their shared KV head's summaries, into zs[h * zst + b]: one read of
// the summaries for the G heads, each head's score formed exactly as in
// decode_row_scores.
template <int G>
__device__ __forceinline__ void decode_group_scores(const DecodeArgs& a, int row0, int nc, float* zs, int zst) {
  constexpr int D = 128;
  const int nbc = a.N / DASH_BLOCK;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const bf16_t* kb = reinterpret_cast<const bf16_t*>(a.kbar) + (size_t)(row0 / a.grp) * nbc * D + (l & 15) * 8;
  const CoarseArith ca = a.ca;
  float qf[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
    unpack8(*reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(a.q) + (size_t)(row0 + h) * D + (l & 15) * 8),
            qf[h]);
  auto bof = [&](int b0, int x) { return b0 + (x * 4 + w) * 4 + (l >> 4); };
  uint4 R[2][DEC_UN];
  auto load = [&](int b0, uint4 (&r)[DEC_UN]) {
#pragma unroll
    for (int x = 0; x < DEC_UN; ++x) {
      const int b = bof(b0, x);
      r[x] = b < nc ? *reinterpret_cast<const uint4*>(kb + (size_t)b * D) : make_uint4(0, 0, 0, 0);
    }
  };
  auto score = [&](int b0, const uint4 (&r)[DEC_UN]) {
#pragma unroll
    for (int x = 0; x < DEC_UN; ++x) {
      const int b = bof(b0, x);
      float kf[8];
      unpack8(r[x], kf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) part = fmaf(qf[h][e], kf[e], part);
        part = sum16(part);
        if (b < nc && (l & 15) == 0) zs[h * zst + b] = ca.u_of(part);
      }
    }
  };
  load(0, R[0]);
  for (int b0 = 0; b0 < nc; b0 += 2 * DEC_SPR) {
    if (b0 + DEC_SPR < nc) load(b0 + DEC_SPR, R[1]);
    score(b0, R[0]);
    if (b0 + DEC_SPR >= nc) break;
    if (b0 + 2 * DEC_SPR < nc) load(b0 + 2 * DEC_SPR, R[0]);
    score(b0 + DEC_SPR, R[1]);
  }
}

// Grouped-query heads (entmax head aggregation): one 4-wave workgroup per
// group of G query heads sharing a KV head.  Every head's scores from one
// read of the summaries; each head's own threshold, mask words and count
// (wave h, and h + 4 when G = 8); then the group's list: the blocks where
// pbar = (1/G) sum_h p_h > 0, with log2 pbar as prior, then the own block
// (prior 0), in the group's first row, and the count in every row of the
// group.  A length out of range gives every row of the group an empty list.
template <int NPL, int G>
__global__ __launch_bounds__(256) void decode_select_group_kernel(DecodeArgs a) {
  constexpr int ZST = DASH_BLOCK * 32;  // up to 2048 candidates per head
  __shared__ float zs[G * ZST];         // per head: scores, then p
  __shared__ int wcnt[4];
  const int row0 = blockIdx.x * G;
  const int nbc = a.N / DASH_BLOCK;
  const int n = decode_row_len(a, row0);  // the group's rows are one sequence's heads
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int nbw = (nbc + 31) / 32;
  if (n < 1 || n > a.N) {
    for (int h = w; h < G; h += 4) {
      const int row = row0 + h;
      if (l == 0) {
        a.sel_cnt[row] = 0;
        if (a.nsel) a.nsel[row] = -1;
        if (a.tau_out) a.tau_out[row] = __uint_as_float(0x7fc00000u);
      }
      if (a.mask)
        for (int x = l; x < nbw; x += 64) a.mask[(size_t)row * nbw + x] = 0u;
    }
    return;
  }
  const int own = (n - 1) / DASH_BLOCK;
  const int nc = own;
  decode_group_scores<G>(a, row0, nc, zs, ZST);
  __syncthreads();
  const CoarseArith ca = a.ca;
  for (int h = w; h < G; h += 4) {
    const int row = row0 + h;
    float* zh = zs + h * ZST;
    float u[NPL];
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      const int idx = l + 64 * k;
      u[k] = idx < nc ? zh[idx] : -INFINITY;
    }
    EntmaxOut e;
    if (nc > 0) e = entmax_solve<NPL, 64>(u, nc, ca);
    else { e.tau = __uint_as_float(0x7fc00000u); e.lognorm = 0.f; e.nsel = 0; e.passes = 0; }
    if (a.mask) {
      uint32_t* mw = a.mask + (size_t)row * nbw;
#pragma unroll
      for (int k = 0; k < NPL; ++k) {
        const int idx = l + 64 * k;
        const unsigned long long bal = __ballot(idx < nc && ca.selected(u[k], e.tau));
        if (l == 0 && 2 * k < nbw) mw[2 * k] = (uint32_t)bal;
        if (l == 0 && 2 * k + 1 < nbw) mw[2 * k + 1] = (uint32_t)(bal >> 32);
      }
    }
    // this head's p over the candidates (its own LDS row, this wave only)
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      const int idx = l + 64 * k;
      if (idx < nc) zh[idx] = ca.selected(u[k], e.tau) ? __expf(ca.logp(u[k], e.tau, e.lognorm)) : 0.f;
    }
    if (l == 0) {
      a.rowstat[2 * row] = e.tau;
      a.rowstat[2 * row + 1] = e.lognorm;
      if (a.nsel) a.nsel[row] = e.nsel;
      if (a.tau_out) a.tau_out[row] = e.tau;
    }
  }
  __syncthreads();
  // the group's list, 256 candidates per step (a ballot per wave, the
  // waves' counts added in LDS)
  int* list = a.sel_blk + (size_t)row0 * nbc;
  float* lp = a.sel_lp + (size_t)row0 * nbc;
  const float inv = 1.f / (float)G;
  int base = 0;
  for (int c0 = 0; c0 < own; c0 += 256) {
    const int idx = c0 + tid;
    float ps = 0.f;
    if (idx < own)
#pragma unroll
      for (int h = 0; h < G; ++h) ps += zs[h * ZST + idx];
    const bool sl = ps > 0.f;
    const unsigned long long bal = __ballot(sl);
    if (l == 0) wcnt[w] = __popcll(bal);
    __syncthreads();
    int before = base, total = 0;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      before += x < w ? wcnt[x] : 0;
      total += wcnt[x];
    }
    if (sl) {
      const int pos = before + __popcll(bal & ((1ull << l) - 1ull));
      list[pos] = idx;
      lp[pos] = __log2f(ps * inv);
    }
    base += total;
    __syncthreads();  // the counts are read before the next step overwrites them
  }
  if (tid == 0) {
    list[base] = own;
    lp[base] = 0.f;
  }
  if (tid < G) a.sel_cnt[row0 + tid] = base + 1;
}

// Per row (one 4-wave workgroup): the row's scores (decode_row_scores, all
// waves), then on wave 0 the entmax threshold over them, the mask words,
// and the compacted ascending list of the selected blocks with their log2
// priors, then the query's own block (prior 0).
template <int NPL>
__global__ __launch_bounds__(256) void decode_select_kernel(DecodeArgs a) {
  __shared__ float zs[DASH_BLOCK * 32];  // scores of up to 2048 candidates
  const int row = blockIdx.x;
  const int nbc = a.N / DASH_BLOCK;  // capacity in blocks: row stride of the summaries and the lists
  const int n = decode_row_len(a, row);
  const int l = threadIdx.x;
  const int nbw = (nbc + 31) / 32;   // mask words per row
  if (n < 1 || n > a.N) {  // length out of range: empty list and mask; the combine writes NaN
    if (l >= 64) return;
    if (l == 0) {
      a.sel_cnt[row] = 0;
      if (a.nsel) a.nsel[row] = -1;
      if (a.tau_out) a.tau_out[row] = __uint_as_float(0x7fc00000u);
    }
    if (a.mask)
      for (int x = l; x < nbw; x += 64) a.mask[(size_t)row * nbw + x] = 0u;
    return;
  }
  const int own = (n - 1) / DASH_BLOCK;  // the query's block
  const int nc = own;                    // the complete blocks before it are the candidates
  decode_row_scores(a, row, nc, zs);
  __syncthreads();
  if (l >= 64) return;
  const CoarseArith ca = a.ca;
  const float* us = zs;
  float u[NPL];
#pragma unroll
  for (int k = 0; k < NPL; ++k) {
    const int idx = l + 64 * k;
    u[k] = idx < nc ? us[idx] : -INFINITY;
  }
  EntmaxOut e;
  if (nc > 0) e = entmax_solve<NPL, 64>(u, nc, ca);
  else { e.tau = __uint_as_float(0x7fc00000u); e.lognorm = 0.f; e.nsel = 0; e.passes = 0; }
  if (a.mask) {
    // the row's selected candidates as bits: word 2k + x from ballot k
    uint32_t* mw = a.mask + (size_t)row * nbw;
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      const int idx = l + 64 * k;
      const unsigned long long bal = __ballot(idx < nc && ca.selected(u[k], e.tau));
      if (l == 0 && 2 * k < nbw) mw[2 * k] = (uint32_t)bal;
      if (l == 0 && 2 * k + 1 < nbw) mw[2 * k + 1] = (uint32_t)(bal >> 32);
    }
  }
  int* list = a.sel_blk + (size_t)row * nbc;
  float* lp = a.sel_lp + (size_t)row * nbc;
  int base = 0;
#pragma unroll
  for (int k = 0; k < NPL; ++k) {
    const int idx = l + 64 * k;
    const bool s = idx < nc && ca.selected(u[k], e.tau);
    const unsigned long long bal = __ballot(s);
    if (s) {
      const int pos = base + __popcll(bal & ((1ull << l) - 1ull));
      list[pos] = idx;
      lp[pos] = ca.logp(u[k], e.tau, e.lognorm) * LOG2E_F;
    }
    base += __popcll(bal);
  }
  if (l == 0) {
    list[base] = own;  // the query's own block, prior 0
    lp[base] = 0.f;
    a.sel_cnt[row] = base + 1;
    a.rowstat[2 * row] = e.tau;
    a.rowstat[2 * row + 1] = e.lognorm;
    if (a.nsel) a.nsel[row] = e.nsel;
    if (a.tau_out) a.tau_out[row] = e.tau;
  }
}

// ---------------------------------------------------------------------------- split-KV attention

__global__ __launch_bounds__(256) void decode_attend_kernel(DecodeArgs a) {
  constexpr int D = 128;
  __shared__ float red_m[4], red_l[4];
  __shared__ float red_o[4][D];
  // grid (row, split): every row's split 0 is dispatched first, then split 1,
  // ...; low splits hold the most list entries, so the launch ends on light
  // workgroups
  const int row = blockIdx.x, split = blockIdx.y;
  const int nbc = a.N / DASH_BLOCK;
  const int n = decode_row_len(a, row);  // in range whenever the list is not empty
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int g = l >> 4, c = l & 15;  // key group within a 1 KB load, 16-byte chunk
  const int cnt = a.sel_cnt[row];
  const int* list = a.sel_blk + (size_t)row * nbc;
  const float* lpl = a.sel_lp + (size_t)row * nbc;
  const bf16_t* K = reinterpret_cast<const bf16_t*>(a.kc) + (size_t)row * a.N * D;
  const bf16_t* V = reinterpret_cast<const bf16_t*>(a.vc) + (size_t)row * a.N * D;
  const float sl2 = a.fine_scale * LOG2E_F;
  float qf[8];
  unpack8(*reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(a.q) + (size_t)row * D + c * 8), qf);
  float m = -INFINITY, lsum = 0.f;
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  const int stride = 4 * a.nsplit;
  const int first = split * 4 + w;
  // this wave's list entries, one per lane, loaded once (at most 64: the list
  // holds <= 2048 blocks and the stride is 64)
  int myb = 0;
  float mylp = 0.f;
  {
    const int en = first + l * stride;
    if (en < cnt) { myb = list[en]; mylp = lpl[en]; }
  }
  const int nmine = cnt > first ? (cnt - first + stride - 1) / stride : 0;
  // K and V of the next entry are requested as soon as this entry's
  // registers are consumed: K(k+1) after the scores of k, V(k+1) after its
  // weighted sum, so each load overlaps the other half's arithmetic
  uint4 kr[16], vr[16];
  auto load_k = [&](int b) {
    const bf16_t* kb = K + (size_t)b * DASH_BLOCK * D;
#pragma unroll
    for (int it = 0; it < 16; ++it) kr[it] = *reinterpret_cast<const uint4*>(kb + (size_t)(it * 4 + g) * D + c * 8);
  };
  auto load_v = [&](int b) {
    const bf16_t* vb = V + (size_t)b * DASH_BLOCK * D;
#pragma unroll
    for (int it = 0; it < 16; ++it) vr[it] = *reinterpret_cast<const uint4*>(vb + (size_t)(it * 4 + g) * D + c * 8);
  };
  if (nmine > 0) {
    const int b0 = __shfl(myb, 0, 64);
    load_k(b0);
    load_v(b0);
  }
  for (int k = 0; k < nmine; ++k) {
    const int b = __shfl(myb, k, 64);
    const float pr = __shfl(mylp, k, 64);
    const int bn = __shfl(myb, k + 1 < nmine ? k + 1 : k, 64);
    float s[16];
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      float kf[8];
      unpack8(kr[it], kf);
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) part = fmaf(qf[e], kf[e], part);
      s[it] = sum16(part) * sl2 + pr;  // key it*4 + g, identical in the 16 lanes of group g
    }
    if (k + 1 < nmine) load_k(bn);
    if ((b + 1) * DASH_BLOCK > n) {
      // the query's own block, partly filled: positions from n on hold no
      // token (whatever their bits), so they get weight 0 and value 0
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        if (b * DASH_BLOCK + it * 4 + g >= n) {
          s[it] = -INFINITY;
          vr[it] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
    }
    float mx = s[0];
#pragma unroll
    for (int it = 1; it < 16; ++it) mx = fmaxf(mx, s[it]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m, mx);
    const float rs = (mn == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m - mn);
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= rs;
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const float p = __builtin_amdgcn_exp2f(s[it] - mn);
      ps += p;
      float vf[8];
      unpack8(vr[it], vf);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = fmaf(p, vf[e], o[e]);
    }
    if (k + 1 < nmine) load_v(bn);
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    lsum = lsum * rs + ps;
    m = mn;
  }
  // merge the 4 key groups of the wave (same m in every lane)
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    o[e] += __shfl_xor(o[e], 16, 64);
    o[e] += __shfl_xor(o[e], 32, 64);
  }
  if (l == 0) { red_m[w] = m; red_l[w] = lsum; }
  if (g == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red_o[w][c * 8 + e] = o[e];
  }
  __syncthreads();
  if (w == 0) {
    const float M = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
    const float Mr = M == -INFINITY ? 0.f : M;
    float L = 0.f;
    float sc[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) { sc[x] = exp2f(red_m[x] - Mr); L += red_l[x] * sc[x]; }
    float* part = a.part + ((size_t)row * a.nsplit + split) * (D + 2);
    for (int d = l; d < D; d += 64)
      part[d] = red_o[0][d] * sc[0] + red_o[1][d] * sc[1] + red_o[2][d] * sc[2] + red_o[3][d] * sc[3];
    if (l == 0) { part[D] = M; part[D + 1] = L; }
  }
}

// One wave per row, 4 rows per workgroup: lane s < nsplit holds split s's
// (m, l); the output sums run over the splits with their scales read back
// lane by lane.
template <int NS>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  constexpr int D = 128;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.SH) return;
  const int l = threadIdx.x & 63;
  bf16_t* O = reinterpret_cast<bf16_t*>(a.o) + (size_t)row * D;
  if (a.sel_cnt[row] <= 0) {  // length out of range (a valid row lists its own block)
    const bf16_t qnan = 0x7FC0u;
    O[l] = qnan;
    O[l + 64] = qnan;
    if (l == 0 && a.lse) a.lse[row] = __uint_as_float(0x7fc00000u);
    return;
  }
  const float* part = a.part + (size_t)row * NS * (D + 2);
  const float ms = l < NS ? part[l * (D + 2) + D] : -INFINITY;
  const float ls = l < NS ? part[l * (D + 2) + D + 1] : 0.f;
  const float M = grp_max<64>(ms);
  const float Mr = M == -INFINITY ? 0.f : M;
  const float sc = (l < NS && ms != -INFINITY) ? __builtin_amdgcn_exp2f(ms - Mr) : 0.f;
  const float L = grp_sum<64>(ls * sc);
  float o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float scs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc), s));
    o0 = fmaf(part[s * (D + 2) + l], scs, o0);
    o1 = fmaf(part[s * (D + 2) + l + 64], scs, o1);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  O[l] = f2bf(o0 * inv);
  O[l + 64] = f2bf(o1 * inv);
  if (l == 0 && a.lse) a.lse[row] = (M + __log2f(L)) * LN2_F;
}

// ---------------------------------------------------------------------------- grouped heads

// Split-KV attention for a group: workgroup (split, group), wave w = the
// group's head w; the workgroup walks list entries split, split + nsplit, ...
// Each block's K and V (32 KB) are read from HBM once: the waves copy a
// share each straight into LDS (buffer loads to LDS, double-buffered, the
// next block's copy in flight while this one is used), then every wave
// computes its head from LDS with the same lane layout as the per-head
// kernel (16 lanes read one 256-byte row: no bank conflicts, no permutation
// needed).  Each wave writes its row's partial.  NW = 2, 4 or 8 heads.
__device__ constexpr int tile_swz_none(int) { return 0; }

template <int NW>
__global__ __launch_bounds__(64 * NW) void decode_attend_group_kernel(DecodeArgs a) {
  constexpr int D = 128;
  constexpr int CH = D / 8;  // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) bf16_t kt0[DASH_BLOCK * D];
  __shared__ __attribute__((aligned(16))) bf16_t kt1[DASH_BLOCK * D];
  __shared__ __attribute__((aligned(16))) bf16_t vt0[DASH_BLOCK * D];
  __shared__ __attribute__((aligned(16))) bf16_t vt1[DASH_BLOCK * D];
  const int split = blockIdx.x, grp_id = blockIdx.y;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int row = grp_id * a.grp + w;
  const int row0 = grp_id * a.grp;
  const int nbc = a.N / DASH_BLOCK;
  const int n = decode_row_len(a, row0);
  const int g = l >> 4, c = l & 15;
  const int cnt = a.sel_cnt[row0];
  const int* list = a.sel_blk + (size_t)row0 * nbc;
  const float* lpl = a.sel_lp + (size_t)row0 * nbc;
  const bf16_t* K = reinterpret_cast<const bf16_t*>(a.kc) + (size_t)grp_id * a.N * D;
  const bf16_t* V = reinterpret_cast<const bf16_t*>(a.vc) + (size_t)grp_id * a.N * D;
  const float sl2 = a.fine_scale * LOG2E_F;
  // the query's 8 features of this lane as bf16 pairs (scores by v_dot2)
  const uint4 qraw = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(a.q) + (size_t)row * D + c * 8);
  const bf16x2 q0 = __builtin_bit_cast(bf16x2, qraw.x), q1 = __builtin_bit_cast(bf16x2, qraw.y);
  const bf16x2 q2 = __builtin_bit_cast(bf16x2, qraw.z), q3 = __builtin_bit_cast(bf16x2, qraw.w);
  const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
  float m = -INFINITY, lsum = 0.f;
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  const int stride = a.nsplit;
  const int nmine = cnt > split ? (cnt - split + stride - 1) / stride : 0;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  TileCopy<D, tile_swz_none, NW> kcp, vcp;
  kcp.init(wu, l);
  vcp.init(wu, l);
  auto copy_block = [&](int b, bf16_t* kd, bf16_t* vd) {
    const size_t off = (size_t)__builtin_amdgcn_readfirstlane(b) * DASH_BLOCK * D;
    kcp.copy(K + off, kd, wu);
    vcp.copy(V + off, vd, wu);
  };
  int b = 0;
  float pr = 0.f;
  if (nmine > 0) {
    b = list[split];
    pr = lpl[split];
    copy_block(b, kt0, vt0);
  }
  for (int k = 0; k < nmine; ++k) {
    // the next entry's block and prior, loaded before the wait below so that
    // the wait covers them too
    int bn = 0;
    float prn = 0.f;
    if (k + 1 < nmine) {
      bn = list[split + (k + 1) * stride];
      prn = lpl[split + (k + 1) * stride];
    }
    tile_copies_done();
    __syncthreads();  // block k is in LDS; every wave is done with the other buffers
    const bf16_t* kt = (k & 1) ? kt1 : kt0;
    const bf16_t* vt = (k & 1) ? vt1 : vt0;
    if (k + 1 < nmine) copy_block(bn, (k & 1) ? kt0 : kt1, (k & 1) ? vt0 : vt1);
    float s[16];
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const uint4 kr = *reinterpret_cast<const uint4*>(kt + (it * 4 + g) * D + c * 8);
      float part = __builtin_amdgcn_fdot2_f32_bf16(q0, __builtin_bit_cast(bf16x2, kr.x), 0.f, false);
      part = __builtin_amdgcn_fdot2_f32_bf16(q1, __builtin_bit_cast(bf16x2, kr.y), part, false);
      part = __builtin_amdgcn_fdot2_f32_bf16(q2, __builtin_bit_cast(bf16x2, kr.z), part, false);
      part = __builtin_amdgcn_fdot2_f32_bf16(q3, __builtin_bit_cast(bf16x2, kr.w), part, false);
      s[it] = sum16(part) * sl2 + pr;
    }
    const bool partial = (b + 1) * DASH_BLOCK > n;  // the own block, partly filled
    if (partial) {
#pragma unroll
      for (int it = 0; it < 16; ++it)
        if (b * DASH_BLOCK + it * 4 + g >= n) s[it] = -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int it = 1; it < 16; ++it) mx = fmaxf(mx, s[it]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m, mx);
    const float rs = (mn == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m - mn);
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= rs;
    // weights rounded to bf16 two keys at a time; each v_dot2 adds both keys'
    // products for one feature (the two keys' values paired by v_perm), and
    // the normaliser sums the same rounded weights
#pragma unroll
    for (int it = 0; it < 16; it += 2) {
      uint4 va = *reinterpret_cast<const uint4*>(vt + (it * 4 + g) * D + c * 8);
      uint4 vb = *reinterpret_cast<const uint4*>(vt + ((it + 1) * 4 + g) * D + c * 8);
      if (partial) {
        if (b * DASH_BLOCK + it * 4 + g >= n) va = make_uint4(0u, 0u, 0u, 0u);
        if (b * DASH_BLOCK + (it + 1) * 4 + g >= n) vb = make_uint4(0u, 0u, 0u, 0u);
      }
      bf16x2 pp;
      pp[0] = (__bf16)__builtin_amdgcn_exp2f(s[it] - mn);
      pp[1] = (__bf16)__builtin_amdgcn_exp2f(s[it + 1] - mn);
      ps = __builtin_amdgcn_fdot2_f32_bf16(pp, one2, ps, false);
      const uint32_t wa[4] = {va.x, va.y, va.z, va.w}, wb[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const bf16x2 lo = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(wb[d], wa[d], 0x05040100u));
        const bf16x2 hi = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(wb[d], wa[d], 0x07060302u));
        o[2 * d] = __builtin_amdgcn_fdot2_f32_bf16(pp, lo, o[2 * d], false);
        o[2 * d + 1] = __builtin_amdgcn_fdot2_f32_bf16(pp, hi, o[2 * d + 1], false);
      }
    }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    lsum = lsum * rs + ps;
    m = mn;
    b = bn;
    pr = prn;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    o[e] += __shfl_xor(o[e], 16, 64);
    o[e] += __shfl_xor(o[e], 32, 64);
  }
  float* part = a.part + ((size_t)row * a.nsplit + split) * (D + 2);
  if (g == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) part[c * 8 + e] = o[e];
  }
  if (l == 0) {
    part[D] = m;
    part[D + 1] = lsum;
  }
}

// Split-KV attention for a group of G = 2 or 4 heads, streamed through
// registers: workgroup (split s, group), its 4 waves take list entries
// s * 4 + w stepping by 4 * nsplit, as in the per-head kernel; a wave loads
// a block's 64 keys and values once (16-byte loads, 16 lanes per 256-byte
// row) and computes every head of the group from those registers, so each
// block is read from HBM once per group with a whole block in flight per
// wave.  The waves' per-head partials are merged in LDS and wave h writes
// head h's partial of this split.
template <int G>
__global__ __launch_bounds__(256) void decode_attend_group_reg_kernel(DecodeArgs a) {
  constexpr int D = 128;
  __shared__ float red_m[4][G], red_l[4][G];
  __shared__ float red_o[4][G][D];
  const int split = blockIdx.x, grp_id = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int g = l >> 4, c = l & 15;
  const int row0 = grp_id * G;
  const int nbc = a.N / DASH_BLOCK;
  const int n = decode_row_len(a, row0);  // in range whenever the list is not empty
  const int cnt = a.sel_cnt[row0];
  const int* list = a.sel_blk + (size_t)row0 * nbc;
  const float* lpl = a.sel_lp + (size_t)row0 * nbc;
  const bf16_t* K = reinterpret_cast<const bf16_t*>(a.kc) + (size_t)grp_id * a.N * D;
  const bf16_t* V = reinterpret_cast<const bf16_t*>(a.vc) + (size_t)grp_id * a.N * D;
  const float sl2 = a.fine_scale * LOG2E_F;
  const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
  // each head's query: this lane's 8 features as bf16 pairs
  bf16x2 qh[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 r = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(a.q) + (size_t)(row0 + h) * D + c * 8);
    qh[h][0] = __builtin_bit_cast(bf16x2, r.x);
    qh[h][1] = __builtin_bit_cast(bf16x2, r.y);
    qh[h][2] = __builtin_bit_cast(bf16x2, r.z);
    qh[h][3] = __builtin_bit_cast(bf16x2, r.w);
  }
  float m[G], lsum[G], o[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
  }
  const int stride = 4 * a.nsplit;
  for (int en = split * 4 + w; en < cnt; en += stride) {
    const int b = list[en];
    const float pr = lpl[en];
    const bool partial = (b + 1) * DASH_BLOCK > n;  // the own block, partly filled
    // keys first: every head's scores, running max and bf16 weights (so the
    // key registers are free before the values are loaded into them)
    uint4 r[16];
    {
      const bf16_t* kb = K + (size_t)b * DASH_BLOCK * D;
#pragma unroll
      for (int it = 0; it < 16; ++it) r[it] = *reinterpret_cast<const uint4*>(kb + (size_t)(it * 4 + g) * D + c * 8);
    }
    bf16x2 pw[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float sc[16];
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        float part = __builtin_amdgcn_fdot2_f32_bf16(qh[h][0], __builtin_bit_cast(bf16x2, r[it].x), 0.f, false);
        part = __builtin_amdgcn_fdot2_f32_bf16(qh[h][1], __builtin_bit_cast(bf16x2, r[it].y), part, false);
        part = __builtin_amdgcn_fdot2_f32_bf16(qh[h][2], __builtin_bit_cast(bf16x2, r[it].z), part, false);
        part = __builtin_amdgcn_fdot2_f32_bf16(qh[h][3], __builtin_bit_cast(bf16x2, r[it].w), part, false);
        sc[it] = sum16(part) * sl2 + pr;
      }
      if (partial) {
#pragma unroll
        for (int it = 0; it < 16; ++it)
          if (b * DASH_BLOCK + it * 4 + g >= n) sc[it] = -INFINITY;
      }
      float mx = sc[0];
#pragma unroll
      for (int it = 1; it < 16; ++it) mx = fmaxf(mx, sc[it]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mn = fmaxf(m[h], mx);
      const float rs = (mn == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m[h] - mn);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] *= rs;
      // weights rounded to bf16 two keys at a time; the normaliser sums the
      // same rounded weights
      float ps = 0.f;
#pragma unroll
      for (int it = 0; it < 16; it += 2) {
        bf16x2 pp;
        pp[0] = (__bf16)__builtin_amdgcn_exp2f(sc[it] - mn);
        pp[1] = (__bf16)__builtin_amdgcn_exp2f(sc[it + 1] - mn);
        ps = __builtin_amdgcn_fdot2_f32_bf16(pp, one2, ps, false);
        pw[h][it >> 1] = pp;
      }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      lsum[h] = lsum[h] * rs + ps;
      m[h] = mn;
    }
    // then the values: each v_dot2 adds two keys' products for one feature
    // (the two keys' values paired by v_perm).  The lane offset passes
    // through an empty asm that reads the last head's max, so the value
    // loads are not moved above the scores (which would keep both blocks
    // in registers at once)
    {
      int voff = g * D + c * 8;
      asm volatile("" : "+v"(voff) : "v"(m[G - 1]));
      const bf16_t* vb = V + (size_t)b * DASH_BLOCK * D + voff;
#pragma unroll
      for (int it = 0; it < 16; ++it) r[it] = *reinterpret_cast<const uint4*>(vb + (size_t)(it * 4) * D);
    }
    if (partial) {
#pragma unroll
      for (int it = 0; it < 16; ++it)
        if (b * DASH_BLOCK + it * 4 + g >= n) r[it] = make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int it = 0; it < 16; it += 2) {
      const uint32_t wa[4] = {r[it].x, r[it].y, r[it].z, r[it].w};
      const uint32_t wb[4] = {r[it + 1].x, r[it + 1].y, r[it + 1].z, r[it + 1].w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const bf16x2 lo = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(wb[d], wa[d], 0x05040100u));
        const bf16x2 hi = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(wb[d], wa[d], 0x07060302u));
#pragma unroll
        for (int h = 0; h < G; ++h) {
          o[h][2 * d] = __builtin_amdgcn_fdot2_f32_bf16(pw[h][it >> 1], lo, o[h][2 * d], false);
          o[h][2 * d + 1] = __builtin_amdgcn_fdot2_f32_bf16(pw[h][it >> 1], hi, o[h][2 * d + 1], false);
        }
      }
    }
  }
  // merge the 4 waves' partials of each head in LDS
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[h][e] += __shfl_xor(o[h][e], 16, 64);
      o[h][e] += __shfl_xor(o[h][e], 32, 64);
    }
    if (g == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) red_o[w][h][c * 8 + e] = o[h][e];
    }
    if (l == 0) {
      red_m[w][h] = m[h];
      red_l[w][h] = lsum[h];
    }
  }
  __syncthreads();
  if (w >= G) return;
  const int h = w;
  float M = -INFINITY;
#pragma unroll
  for (int x = 0; x < 4; ++x) M = fmaxf(M, red_m[x][h]);
  float sc4[4], L = 0.f;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    sc4[x] = (red_m[x][h] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(red_m[x][h] - M);
    L += red_l[x][h] * sc4[x];
  }
  float* part = a.part + ((size_t)(row0 + h) * a.nsplit + split) * (D + 2);
#pragma unroll
  for (int d2 = 0; d2 < 2; ++d2) {
    const int d = l + 64 * d2;
    float acc = 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x) acc = fmaf(red_o[x][h][d], sc4[x], acc);
    part[d] = acc;
  }
  if (l == 0) {
    part[D] = M;
    part[D + 1] = L;
  }
}

// ---------------------------------------------------------------------------- cache maintenance

// One wave per row, 4 rows per workgroup; lane l moves elements 2l and 2l+1
// (one 4-byte bf16 pair) of the new key and value to position len.  When the
// token completes its block, the same lane also forms the block's summary
// for its two elements: the 63 cached keys and the new one summed in fp64
// in position order, times 1/64, rounded once, which is the arithmetic of
// the Stage-0 pool kernel.
__global__ __launch_bounds__(256) void decode_append_kernel(AppendArgs a) {
  constexpr int D = 128, W = D / 2;  // 32-bit words per row
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.SH) return;
  const int l = threadIdx.x & 63;
  const int n = a.len[row / a.H];
  if (n < 0 || n >= a.N) return;  // full cache or length out of range: nothing written
  const uint32_t kw = reinterpret_cast<const uint32_t*>(a.k_new)[(size_t)row * W + l];
  const uint32_t vw = reinterpret_cast<const uint32_t*>(a.v_new)[(size_t)row * W + l];
  uint32_t* kc = reinterpret_cast<uint32_t*>(a.kc) + (size_t)row * a.N * W;
  uint32_t* vc = reinterpret_cast<uint32_t*>(a.vc) + (size_t)row * a.N * W;
  kc[(size_t)n * W + l] = kw;
  vc[(size_t)n * W + l] = vw;
  if (n % DASH_BLOCK != DASH_BLOCK - 1) return;
  const int b = n / DASH_BLOCK;
  const uint32_t* blk = kc + (size_t)b * DASH_BLOCK * W;
  double s0 = 0.0, s1 = 0.0;
  for (int r = 0; r < DASH_BLOCK - 1; ++r) {
    const uint32_t x = blk[(size_t)r * W + l];
    s0 += (double)bf2f((bf16_t)(x & 0xFFFFu));
    s1 += (double)bf2f((bf16_t)(x >> 16));
  }
  s0 += (double)bf2f((bf16_t)(kw & 0xFFFFu));
  s1 += (double)bf2f((bf16_t)(kw >> 16));
  const uint32_t m0 = d2bf(s0 * (1.0 / DASH_BLOCK)), m1 = d2bf(s1 * (1.0 / DASH_BLOCK));
  reinterpret_cast<uint32_t*>(a.kbar)[((size_t)row * (a.N / DASH_BLOCK) + b) * W + l] = m0 | (m1 << 16);
}

hipError_t launch_append(const AppendArgs& a, int dtype, hipStream_t st) {
  if (dtype != 1 || a.D != 128) return hipErrorNotSupported;
  decode_append_kernel<<<(a.SH + 3) / 4, 256, 0, st>>>(a);
  return hipGetLastError();
}

template <int G>
static hipError_t launch_select_group(const DecodeArgs& a, int nb, hipStream_t st) {
  const int ng = a.SH / G;
  if (nb <= 128) decode_select_group_kernel<2, G><<<ng, 256, 0, st>>>(a);
  else if (nb <= 256) decode_select_group_kernel<4, G><<<ng, 256, 0, st>>>(a);
  else if (nb <= 512) decode_select_group_kernel<8, G><<<ng, 256, 0, st>>>(a);
  else if (nb <= 1024) decode_select_group_kernel<16, G><<<ng, 256, 0, st>>>(a);
  else if (nb <= 1536) decode_select_group_kernel<24, G><<<ng, 256, 0, st>>>(a);
  else decode_select_group_kernel<32, G><<<ng, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a0, int dtype, hipStream_t st) {
  if (dtype != 1 || a0.D != 128) return hipErrorNotSupported;
  DecodeArgs a = a0;
  a.nsplit = DASH_DEC_SPLIT;
  const int nb = a.N / DASH_BLOCK;
  hipError_t e;
  if (a.grp == 1) {
    if (nb <= 128) decode_select_kernel<2><<<a.SH, 256, 0, st>>>(a);
    else if (nb <= 256) decode_select_kernel<4><<<a.SH, 256, 0, st>>>(a);
    else if (nb <= 512) decode_select_kernel<8><<<a.SH, 256, 0, st>>>(a);
    else if (nb <= 1024) decode_select_kernel<16><<<a.SH, 256, 0, st>>>(a);
    else if (nb <= 1536) decode_select_kernel<24><<<a.SH, 256, 0, st>>>(a);
    else decode_select_kernel<32><<<a.SH, 256, 0, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    decode_attend_kernel<<<dim3(a.SH, a.nsplit), 256, 0, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    decode_combine_kernel<DASH_DEC_SPLIT><<<(a.SH + 3) / 4, 256, 0, st>>>(a);
    return hipGetLastError();
  }
  {
    if (a.SH % a.grp) return hipErrorInvalidValue;
    if (a.grp == 2) e = launch_select_group<2>(a, nb, st);
    else if (a.grp == 4) e = launch_select_group<4>(a, nb, st);
    else if (a.grp == 8) e = launch_select_group<8>(a, nb, st);
    else return hipErrorNotSupported;
    if (e != hipSuccess) return e;
    if (a.grp == 2 || a.grp == 4) {
      // blocks streamed through registers, all the group's heads per wave
      a.nsplit = DASH_DEC_SPLIT;
      const dim3 grid(a.nsplit, a.SH / a.grp);
      if (a.grp == 2) decode_attend_group_reg_kernel<2><<<grid, 256, 0, st>>>(a);
      else decode_attend_group_reg_kernel<4><<<grid, 256, 0, st>>>(a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      decode_combine_kernel<DASH_DEC_SPLIT><<<(a.SH + 3) / 4, 256, 0, st>>>(a);
      return hipGetLastError();
    }
    a.nsplit = DASH_DEC_SPLIT_GQA;  // a group walks G times the blocks of a row: more splits
    const dim3 grid(a.nsplit, a.SH / a.grp);
    if (a.grp == 8) decode_attend_group_kernel<8><<<grid, 512, 0, st>>>(a);
    else return hipErrorNotSupported;
    if ((e = hipGetLastError()) != hipSuccess) return e;
    decode_combine_kernel<DASH_DEC_SPLIT_GQA><<<(a.SH + 3) / 4, 256, 0, st>>>(a);
    return hipGetLastError();
  }
}
