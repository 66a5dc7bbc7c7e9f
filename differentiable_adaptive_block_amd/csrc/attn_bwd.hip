// Backward of the DashAttention hot path: gradients of <dO, O> through
// Stage 2, log p, the alpha-entmax Jacobian, the block scores and mean
// pooling ("Core Mechanism" of the alanhou.org page: gradients flow from
// Stage 2 back through the log into Stage 1's entmax; "What alpha-entmax
// changes" of the montana-research page: they reach the summariser).
//
// With a_ij the Stage-2 weights, l_ij = fine_scale q_i.k_j + log p_{i,blk(j)}:
//   delta_i = dO_i . O_i,   dS_ij = a_ij (dO_i . v_j - delta_i)
//   dQ_i  = fine_scale sum_j dS_ij k_j      dK_j = fine_scale sum_i dS_ij q_i
//   dV_j  = sum_i a_ij dO_i                 G_ib = sum_{j in b} dS_ij   (= dL/dlog p_ib)
//   s = p^(2-alpha), s.g = G p^(1-alpha),   dz_ib = s_b g_b - s_b <s,g>/sum s
//   dQ_i += coarse_scale sum_b dz_ib kbar_b,  dkbar_b = coarse_scale sum_i dz_ib q_i,
//   dK_j += dkbar_{blk(j)} / 64 (mean pooling; left out when the summaries come
//   from another summariser, whose own backward then adds its term).
//
// bf16 path (deterministic, no floating-point atomics):
//   bwd_delta     delta
//   bwd_dq        query-tile-major, walks the tile's block list like the forward;
//                 MFMA for S^T, dP^T and dQ^T; writes G and the log2 prior of
//                 every (row, listed block) to the workspace
//   bwd_coarse    per row: dz over its listed candidate blocks (overwrites G),
//                 then dQ = fine part + coarse part, to bf16
//   bwd_dkdv      key-block-major over the query tiles whose list holds the
//                 block; MFMA for S, dP, dV^T and dK^T; also dkbar and the
//                 pooling term
// fp32 path: a row pass (dQ, G, dz), an ordered dkbar reduction and a
// key-block pass (dK, dV); no atomics either.
#include "kernels.h"
#include "attn_bwd.h"
#include "entmax.h"
#include "tiles.h"

#define LOG2E_F 1.4426950408889634f

// ---------------------------------------------------------------------------- delta

// delta = rowsum(dO o O) of the bf16 rows (the fp32 path forms it in its
// row kernel), with 16-byte loads: D/8 lanes per row, 64/(D/8) rows per
// wave.  Each lane adds its 8 products in order, then the lanes of a row add
// theirs by a butterfly (the same order in every row).
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_bf16_kernel(const bf16_t* __restrict__ o, const bf16_t* __restrict__ dout,
                                                             float* __restrict__ delta, size_t rows) {
  constexpr int LPR = D / 8, RPW = 64 / LPR;
  const int l = threadIdx.x & 63, c = l % LPR;
  const size_t r = ((size_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + l / LPR;
  float acc = 0.f;
  if (r < rows) {
    const uint4 a = *reinterpret_cast<const uint4*>(o + r * D + 8 * c);
    const uint4 b = *reinterpret_cast<const uint4*>(dout + r * D + 8 * c);
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      acc = fmaf(__uint_as_float(aw[x] << 16), __uint_as_float(bw[x] << 16), acc);
      acc = fmaf(__uint_as_float(aw[x] & 0xFFFF0000u), __uint_as_float(bw[x] & 0xFFFF0000u), acc);
    }
  }
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) acc += __shfl_xor(acc, m, 64);
  if (r < rows && c == 0) delta[r] = acc;
}
static hipError_t launch_delta_bf16(const BwdArgs& a, size_t rows, hipStream_t st) {
  const bf16_t* o = reinterpret_cast<const bf16_t*>(a.o);
  const bf16_t* g = reinterpret_cast<const bf16_t*>(a.dout);
  if (a.D == 128) bwd_delta_bf16_kernel<128><<<(unsigned)((rows + 15) / 16), 256, 0, st>>>(o, g, a.delta, rows);
  else if (a.D == 64) bwd_delta_bf16_kernel<64><<<(unsigned)((rows + 31) / 32), 256, 0, st>>>(o, g, a.delta, rows);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- dQ (fine), G, priors

// Slot of (query tile, listed entry e, row of the tile) in the per-entry
// buffers (G, prior): each head stores its tiles' entries one after the
// other, tile t taking room for the most entries its list can hold
// (bwd_tile_base in attn_bwd.h: the lower triangle when causal).
__device__ __forceinline__ size_t gidx(size_t bh, int ntile, int tile, int nb, int e, int row_in_tile, int causal) {
  return ((bh * bwd_entries_per_head(causal, nb, ntile) + bwd_tile_base(causal, nb, tile) + e) * DASH_QTILE) +
         row_in_tile;
}

// Query-tile-major like the forward: workgroup = 4 waves = 128 query rows,
// wave w rows 32w..32w+31; the tile's listed blocks are walked in order with
// the K and V tiles copied straight into LDS, double-buffered, one barrier
// per block.  Per wave, block and 32-key half:
//   S^T = K Q^T, dP^T = V dO^T       D/16 MFMA each (row reads of K, V)
//   dS^T = P^T (dP^T - delta),  G += sum over the keys of dS
//   dQ^T += K^T dS^T                 (D/32) x 2 MFMA (transposing reads of K)
// The K tile uses the permutation that serves both read kinds.
template <int D, bool GQA>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a) {
  constexpr int KS = D / 16;
  constexpr int NDT = D / 32;
  __shared__ __attribute__((aligned(16))) bf16_t kt0[64 * D];
  __shared__ __attribute__((aligned(16))) bf16_t kt1[64 * D];
  __shared__ __attribute__((aligned(16))) bf16_t vt0[64 * D];
  __shared__ __attribute__((aligned(16))) bf16_t vt1[64 * D];
  __shared__ float prs[4][32][32];  // per wave: log2 prior [list slot % 32][row]

  const int nb = a.T / DASH_BLOCK;
  const int ntile = (a.T + DASH_QTILE - 1) / DASH_QTILE;
  const int nwg = gridDim.x, wg = blockIdx.x;
  const int logical = (nwg % 8 == 0) ? (wg % 8) * (nwg / 8) + wg / 8 : wg;
  const size_t bh = logical / ntile;
  const int tile = ntile - 1 - (logical % ntile);
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, j = l & 31, h = l >> 5;
  const int qrow0 = tile * DASH_QTILE + w * 32;
  const bool active = qrow0 < a.T;
  const int wblk = qrow0 / DASH_BLOCK;
  const int i = qrow0 + j;

  const size_t bkv = GQA ? bh / a.grp : bh;  // the key/value head
  const bf16_t* Q = reinterpret_cast<const bf16_t*>(a.q) + bh * a.T * D;
  const bf16_t* K = reinterpret_cast<const bf16_t*>(a.k) + bkv * a.T * D;
  const bf16_t* V = reinterpret_cast<const bf16_t*>(a.v) + bkv * a.T * D;
  const bf16_t* dO = reinterpret_cast<const bf16_t*>(a.dout) + bh * a.T * D;
  const bf16_t* KB = reinterpret_cast<const bf16_t*>(a.kbar) + bkv * nb * D;
  const int* list = a.tile_blk + (bh * ntile + tile) * nb;
  const int cnt = a.tile_cnt[bh * ntile + tile];
  const CoarseArith ca = a.ca;
  const float sl2 = a.fine_scale * LOG2E_F;
  // list entries at a wave-uniform index go through the scalar cache: a
  // vector-memory load inside the loop would wait for the tile copies in
  // flight, which retire on the same counter
  const __attribute__((address_space(4))) int* slist =
      (const __attribute__((address_space(4))) int*)(uintptr_t)list;

  bf16x8 qb[KS], dob[KS];
  float tau_i = 0.f, ln_i = 0.f, lse2 = 0.f, dlt = 0.f;
  if (active) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qb[s] = load8(Q + (size_t)i * D + 16 * s + 8 * h);
      dob[s] = load8(dO + (size_t)i * D + 16 * s + 8 * h);
    }
    tau_i = a.tau[bh * a.T + i];
    ln_i = a.lognorm[bh * a.T + i];
    lse2 = a.lse[bh * a.T + i] * LOG2E_F;
    dlt = a.delta[bh * a.T + i];
  }
  f32x16 dqa[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqa[dt][r] = 0.f;

  const int wu = __builtin_amdgcn_readfirstlane(w);
  TileCopy<D, TileSwz<D>::kv> kcp;
  TileCopy<D, TileSwz<D>::k> vcp;
  kcp.init(wu, l);
  vcp.init(wu, l);
  auto copy_block = [&](int e, bf16_t* kd, bf16_t* vd) {
    const size_t o = (size_t)slist[e] * DASH_BLOCK * D;
    kcp.copy(K + o, kd, wu);
    vcp.copy(V + o, vd, wu);
  };
  // priors of list entries e0..e0+31 into this wave's LDS table
  auto prior_chunk = [&](int e0) {
    f32x16 pacc;
    if constexpr (GQA) {
      const size_t bh0 = bkv * a.grp;  // the group's first query head
      if (active) {
        {
          // the row's own log2 p (its own entmax, whose Jacobian the coarse
          // kernel applies), from the same score MFMAs as the forward's
          const f32x16 own = prior_chunk32<D>(KB, list, cnt, e0, qb, ca, tau_i, ln_i, a.causal, wblk);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int en = e0 + acc_row32(r, l);
            if (en < cnt) a.phbuf[gidx(bh, ntile, tile, nb, en, w * 32 + j, a.causal)] = own[r];
          }
        }
        pacc = prior_chunk32_group<D>(KB, list, cnt, e0, reinterpret_cast<const bf16_t*>(a.q) + (bh0 * a.T + i) * D,
                                      (size_t)a.T * D, a.tau + bh0 * a.T + i, a.lognorm + bh0 * a.T + i, a.T,
                                      a.grp, ca, a.causal, wblk);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) pacc[r] = -INFINITY;
      }
    } else {
      pacc = prior_chunk32<D>(KB, list, cnt, e0, qb, ca, tau_i, ln_i, a.causal, wblk);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) prs[w][acc_row32(r, l)][j] = pacc[r];
  };
  auto put_g = [&](int e, float g, float p2) {
    if (h == 0) {
      const size_t gi = gidx(bh, ntile, tile, nb, e, w * 32 + j, a.causal);
      a.gbuf[gi] = g;
      a.pbuf[gi] = p2;
    }
  };

  auto block_step = [&](int e, const bf16_t* kt, const bf16_t* vt) {
    const int b = slist[e];
    if (a.causal && b > wblk) {
      put_g(e, 0.f, -INFINITY);
      return;
    }
    const bool diag = a.causal && b == wblk;
    const float pr = diag ? 0.f : prs[w][e & 31][j];
    if (!diag && __ballot(pr != -INFINITY) == 0ull) {
      put_g(e, 0.f, -INFINITY);
      return;
    }
    // operand addresses recomputed per block (see bwd_dkdv_kernel)
    int lx = l;
    asm volatile("" : "+v"(lx));
    const int jx = lx & 31, hx = lx >> 5;
    const float off = (pr == -INFINITY) ? -INFINITY : pr - lse2;
    // row reads of keys jx and 32 + jx (same permutation: it depends on row
    // bits 0-3 only): chunk (2 s + h) ^ swz = 2 s ^ (h ^ swz), so k-step s
    // XORs 32 s into a per-lane byte offset
    const char* krb = reinterpret_cast<const char*>(kt + jx * D);
    const char* vrb = reinterpret_cast<const char*>(vt + jx * D);
    const uint32_t ky = 16u * (uint32_t)(hx ^ TileSwz<D>::kv(jx));
    const uint32_t vy = 16u * (uint32_t)(hx ^ TileSwz<D>::k(jx));
    // transposing reads of K (bytes): A + ((64 dt) ^ B) + 32 D k-step
    uint32_t A1, B1, A2, B2;
    col8_parts<D, TileSwz<D>::kv>(lx, A1, B1, A2, B2);
    float gsum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x16 sc, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) { sc[r] = 0.f; dp[r] = 0.f; }
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        sc = mfma32(load8(reinterpret_cast<const bf16_t*>(krb + 64 * D * t + ((32u * s) ^ ky))), qb[s], sc);
        dp = mfma32(load8(reinterpret_cast<const bf16_t*>(vrb + 64 * D * t + ((32u * s) ^ vy))), dob[s], dp);
      }
      if (diag) {  // the wave's own block: keys after the row are masked (wave-uniform branch)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * t + acc_row32(r, lx) > (qrow0 - b * DASH_BLOCK) + jx) sc[r] = -INFINITY;
      }
      // dS^T of this half, as the B operand of the dQ product (k-steps of
      // 16 keys: registers 8 s2 .. 8 s2 + 7)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8 db;
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) {
          const int r = 8 * s2 + e8;
          const float p = __builtin_amdgcn_exp2f(fmaf(sc[r], sl2, off));
          const float dsv = p * (dp[r] - dlt);
          gsum += dsv;
          db[e8] = (__bf16)dsv;
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          dqa[dt] = mfma32(tile_col8_b(reinterpret_cast<const char*>(kt) + 32 * D * (2 * t + s2),
                                       A1 + ((64u * dt) ^ B1), A2 + ((64u * dt) ^ B2)),
                           db, dqa[dt]);
      }
    }
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(gsum), __float_as_uint(gsum), false, false);
    gsum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    put_g(e, diag ? 0.f : gsum, pr);
  };

  if (cnt > 0) {
    copy_block(0, kt0, vt0);
    for (int e = 0; e < cnt; e += 2) {
      if ((e & 31) == 0 && active) prior_chunk(e);
      tile_copies_done();
      __syncthreads();  // block e in buffers 0; everyone is done with buffers 1
      if (e + 1 < cnt) copy_block(e + 1, kt1, vt1);
      if (active) block_step(e, kt0, vt0);
      if (e + 1 >= cnt) break;
      tile_copies_done();
      __syncthreads();  // block e+1 in buffers 1; everyone is done with buffers 0
      if (e + 2 < cnt) copy_block(e + 2, kt0, vt0);
      if (active) block_step(e + 1, kt1, vt1);
    }
  }
  if (active) {
    float* dq = a.dq_acc + (bh * a.T + i) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * dt + 8 * r4 + 4 * h;
        float4 v4 = make_float4(dqa[dt][4 * r4] * a.fine_scale, dqa[dt][4 * r4 + 1] * a.fine_scale,
                                dqa[dt][4 * r4 + 2] * a.fine_scale, dqa[dt][4 * r4 + 3] * a.fine_scale);
        *reinterpret_cast<float4*>(dq + d) = v4;
      }
  }
}

// ---------------------------------------------------------------------------- dK, dV, dkbar

// Position of block b in a tile's ascending list (from the tile's bit set),
// or -1 when the tile does not list it.
__device__ __forceinline__ int list_slot(const uint32_t* bits, int b) {
  const uint32_t word = bits[b >> 5];
  if (!((word >> (b & 31)) & 1u)) return -1;
  int slot = __popc(word & ((1u << (b & 31)) - 1u));
  for (int x = 0; x < (b >> 5); ++x) slot += __popc(bits[x]);
  return slot;
}

// Key-block-major: a workgroup of 8 waves owns 128 keys (blocks b0, b0+1)
// and walks the items: 64-query chunks (tile t, half c) that see either
// block, in ascending (t, c); the item list is built once in LDS.  Wave w:
// block kb = w/4, key half kh = (w/2)&1, query half qh = w&1.  Per item and
// wave (32 queries x 32 keys), with keys as MFMA columns:
//   S = Q K^T, dP = dO V^T               D/16 MFMA each
//   dV^T += dO^T P, dK^T += Q^T dS        (D/32) x 2 MFMA each
// K and V stay in LDS for the whole walk; each item's Q and dO chunks are
// copied straight into LDS, double-buffered (one barrier per item), in the
// permutation that serves both the row reads (S, dP) and the transposing
// reads (dV, dK).  dkbar_b = coarse_scale sum_q dz_qb q_q accumulates from
// the same Q chunks.
template <int D>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int KS = D / 16;
  constexpr int NDT = D / 32;
  constexpr int CH = D / 8;
  constexpr int NITEM = 32 * CH;       // (row pair, chunk) dkbar items per query chunk
  constexpr int MAXIT = 2 * (DASH_MAX_NB / 2);  // 64-query chunks of the longest sequence
  constexpr int KP = D + 8;  // row pitch of the K and V tiles (padded: conflict-free 16-byte row reads)
  // per-item tiles, one object per buffer (reads of one are not ordered
  // behind the copy into the other); the Q tile, then the dO tile 64 D
  // elements on, so both take one address and an immediate offset
  __shared__ __attribute__((aligned(16))) bf16_t qo0[2 * 64 * D];
  __shared__ __attribute__((aligned(16))) bf16_t qo1[2 * 64 * D];
  bf16_t* const qc0 = qo0;
  bf16_t* const oc0 = qo0 + 64 * D;
  bf16_t* const qc1 = qo1;
  bf16_t* const oc1 = qo1 + 64 * D;
  __shared__ __attribute__((aligned(16))) bf16_t ks[128 * KP];
  __shared__ __attribute__((aligned(16))) bf16_t vs[128 * KP];
  __shared__ float prq[2][2][64], dzq[2][2][64], dlq[2][64];  // [buffer][block][row], [buffer][row]
  __shared__ int itm[MAXIT][3];                                // (t * 2 + c, slot0, slot1)
  __shared__ int nit_s, wsum[8];
  __shared__ float kbg[2][D];
  static_assert(2 * 32 * D * 4 <= 128 * KP * 2, "dkbar reduction space in the K tile");
  static_assert(NDT * 16 * 64 * 4 <= 64 * D * 2, "merge space: one partial per 64-row tile buffer");

  const int nb = a.T / DASH_BLOCK;
  const int nbw = (nb + 31) / 32;
  const int ntile = (a.T + DASH_QTILE - 1) / DASH_QTILE;
  const int ngrp = (nb + 1) / 2;
  const int nwg = gridDim.x, wg = blockIdx.x;
  const int logical = (nwg % 8 == 0) ? (wg % 8) * (nwg / 8) + wg / 8 : wg;
  const size_t bh = logical / ngrp;
  const int b0 = 2 * (logical % ngrp);  // early blocks (most query tiles when causal) first
  const int nblk = min(2, nb - b0);
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, j = l & 31, h = l >> 5;
  const int kb = w >> 2, kh = (w >> 1) & 1, qh = w & 1;
  const int wb = b0 + kb;  // this wave's key block

  const bf16_t* Q = reinterpret_cast<const bf16_t*>(a.q) + bh * a.T * D;
  const bf16_t* K = reinterpret_cast<const bf16_t*>(a.k) + (bh / a.grp) * a.T * D;
  const bf16_t* V = reinterpret_cast<const bf16_t*>(a.v) + (bh / a.grp) * a.T * D;
  const bf16_t* dO = reinterpret_cast<const bf16_t*>(a.dout) + bh * a.T * D;
  const float sl2 = a.fine_scale * LOG2E_F;

  // K and V of the two blocks, rows 0-63 block b0, 64-127 block b0 + 1:
  // loaded once per workgroup, into row-padded tiles
  const int wu = __builtin_amdgcn_readfirstlane(w);
  for (int x = tid; x < 64 * nblk * CH; x += 512) {
    const int row = x / CH, ch = x % CH;
    const size_t g = ((size_t)b0 * DASH_BLOCK + row) * D + 8 * ch;
    *reinterpret_cast<uint4*>(ks + row * KP + 8 * ch) = *reinterpret_cast<const uint4*>(K + g);
    *reinterpret_cast<uint4*>(vs + row * KP + 8 * ch) = *reinterpret_cast<const uint4*>(V + g);
  }

  // item list: thread x looks at tile x (then x + 512, ...), keeps its 0-2
  // items, and a workgroup prefix sum places them in ascending order
  if (tid == 0) nit_s = 0;
  __syncthreads();
  for (int t0 = 0; t0 < ntile; t0 += 512) {
    const int t = t0 + tid;
    int my[2][3];
    int n = 0;
    if (t < ntile) {
      const uint32_t* bits = a.tile_bits + (bh * ntile + t) * nbw;
      const int s0 = list_slot(bits, b0);
      const int s1 = nblk > 1 ? list_slot(bits, b0 + 1) : -1;
      if (s0 >= 0 || s1 >= 0) {
        for (int c = 0; c < DASH_QTILE / 64; ++c) {
          const int q0 = t * DASH_QTILE + c * 64;
          if (q0 >= a.T) break;
          const int ob = q0 / DASH_BLOCK;
          const int sl0 = (a.causal && ob < b0) ? -1 : s0;
          const int sl1 = (a.causal && ob < b0 + 1) ? -1 : s1;
          if (sl0 >= 0 || sl1 >= 0) {
            my[n][0] = 2 * t + c;
            my[n][1] = sl0;
            my[n][2] = sl1;
            ++n;
          }
        }
      }
    }
    // exclusive prefix sum of n over the workgroup
    int incl = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (l >= o) incl += y;
    }
    if (l == 63) wsum[w] = incl;
    __syncthreads();
    int base = nit_s;
    for (int x = 0; x < w; ++x) base += wsum[x];
    const int pos = base + incl - n;
    for (int x = 0; x < n; ++x) {
      itm[pos + x][0] = my[x][0];
      itm[pos + x][1] = my[x][1];
      itm[pos + x][2] = my[x][2];
    }
    __syncthreads();
    if (tid == 0) {
      int tot = 0;
      for (int x = 0; x < 8; ++x) tot += wsum[x];
      nit_s += tot;
    }
    __syncthreads();
  }
  const int nit = nit_s;

  f32x16 dva[NDT], dka[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dva[dt][r] = 0.f; dka[dt][r] = 0.f; }
  float kbp[2][8];  // dkbar partials of this thread's (row pair, chunk)
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
    for (int e = 0; e < 8; ++e) kbp[k2][e] = 0.f;
  const bool kbthr = tid < NITEM;
  const int spr = tid / CH, sch = tid % CH;

  // per-row data of an item: threads 0-63 issue the loads into registers
  // (no arithmetic on the loaded values, so nothing waits for them here and
  // the wave goes on to its share of the next copy), then, after the item in
  // flight is computed, combine them and store them into LDS buffer `buf`
  float s_pr0 = 0.f, s_pr1 = 0.f, s_dz0 = 0.f, s_dz1 = 0.f, s_dl = 0.f, s_ls = 0.f;
  auto load_rows = [&](int n) {
    if (tid < 64) {
      const int t = itm[n][0] >> 1, c = itm[n][0] & 1;
      const int q0 = t * DASH_QTILE + c * 64;
      const int row = c * 64 + tid;
      s_ls = a.lse[bh * a.T + q0 + tid];
      s_dl = a.delta[bh * a.T + q0 + tid];
      s_pr0 = -INFINITY; s_dz0 = 0.f;
      s_pr1 = -INFINITY; s_dz1 = 0.f;
      if (itm[n][1] >= 0) {
        const size_t gi = gidx(bh, ntile, t, nb, itm[n][1], row, a.causal);
        s_pr0 = a.pbuf[gi];
        s_dz0 = a.gbuf[gi];
      }
      if (itm[n][2] >= 0) {
        const size_t gi = gidx(bh, ntile, t, nb, itm[n][2], row, a.causal);
        s_pr1 = a.pbuf[gi];
        s_dz1 = a.gbuf[gi];
      }
    }
  };
  auto store_rows = [&](int buf) {
#pragma clang fp contract(off)  // lse * log2e rounded, then subtracted
    if (tid < 64) {
      const float ls = s_ls * LOG2E_F;
      prq[buf][0][tid] = s_pr0 - ls;  // -inf stays -inf
      prq[buf][1][tid] = s_pr1 - ls;
      dzq[buf][0][tid] = s_dz0;
      dzq[buf][1][tid] = s_dz1;
      dlq[buf][tid] = s_dl;
    }
  };
  TileCopy<D, TileSwz<D>::kv> qocp;  // waves 0-3 copy the Q chunk, waves 4-7 the dO chunk
  qocp.init(wu & 3, l);
  auto copy_item = [&](int n, bf16_t* qd, bf16_t* od) {
    const int t = itm[n][0] >> 1, c = itm[n][0] & 1;
    const size_t r0 = (size_t)(t * DASH_QTILE + c * 64) * D;
    if (wu < 4) qocp.copy(Q + r0, qd, wu);
    else qocp.copy(dO + r0, od, wu - 4);
  };

  auto item_step = [&](int n, int buf, const bf16_t* qc, const bf16_t* oc) {
    const int t = itm[n][0] >> 1, c = itm[n][0] & 1;
    const int q0 = t * DASH_QTILE + c * 64;
    // dkbar partials from the chunk's rows 2 spr, 2 spr + 1, chunk sch
    if (kbthr) {
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int row = 2 * spr + rr;
        const uint4 qv = *reinterpret_cast<const uint4*>(qc + row * D + 8 * (sch ^ TileSwz<D>::kv(row)));
        const uint32_t wv[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const float z = dzq[buf][k2][row];
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            kbp[k2][2 * x] = fmaf(z, __uint_as_float(wv[x] << 16), kbp[k2][2 * x]);
            kbp[k2][2 * x + 1] = fmaf(z, __uint_as_float(wv[x] & 0xFFFF0000u), kbp[k2][2 * x + 1]);
          }
        }
      }
    }
    const int wslot = itm[n][1 + kb];
    if (wslot < 0) return;
    const bool diag = a.causal && q0 / DASH_BLOCK == wb;
    // The operand addresses below depend on the lane only; recomputing them
    // per item (from a lane index the compiler cannot see through) keeps
    // them out of the registers held across the item loop.
    int lx = l;
    asm volatile("" : "+v"(lx));
    const int jx = lx & 31, hx = lx >> 5;
    f32x16 sc, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) { sc[r] = 0.f; dp[r] = 0.f; }
    const int krow = 64 * kb + 32 * kh + jx;
    // Q / dO row reads: chunk (2 st + h) ^ swz(row) = 2 st ^ (h ^ swz(row)),
    // so k-step st XORs 32 st into a per-lane byte offset
    const int qrow = 32 * qh + jx;
    const char* qrb = reinterpret_cast<const char*>(qc + qrow * D);
    const uint32_t qy = 16u * (uint32_t)(hx ^ TileSwz<D>::kv(qrow));
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      const bf16x8 bk = load8(ks + krow * KP + 16 * st + 8 * hx);
      const bf16x8 bv = load8(vs + krow * KP + 16 * st + 8 * hx);
      const char* qa = qrb + ((32u * st) ^ qy);
      sc = mfma32(load8(reinterpret_cast<const bf16_t*>(qa)), bk, sc);
      dp = mfma32(load8(reinterpret_cast<const bf16_t*>(qa + 2 * 64 * D)), bv, dp);
    }
    // transposing-read offsets (bytes) of this wave's k-steps 2 qh + s2
    uint32_t A1, B1, A2, B2;
    col8_parts<D, TileSwz<D>::kv>(lx, A1, B1, A2, B2);
    const char* qcb = reinterpret_cast<const char*>(qc) + 64 * D * qh;  // k-step 2 qh
    if (diag) {  // the wave's own block: keys after the row are masked (wave-uniform branch)
      const int kx = wb * DASH_BLOCK + 32 * kh + jx - q0;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kx > 32 * qh + acc_row32(r, lx)) sc[r] = -INFINITY;
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      bf16x8 pb, db;
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        const int r = 8 * s2 + e8;
        const int ql = 32 * qh + acc_row32(r, l);
        const float p = __builtin_amdgcn_exp2f(fmaf(sc[r], sl2, prq[buf][kb][ql]));  // prior2 - lse2
        pb[e8] = (__bf16)p;
        db[e8] = (__bf16)(p * (dp[r] - dlq[buf][ql]));
      }
      // queries 16 (2 qh + s2) .. +15 of the chunk are this k-step
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const uint32_t o1 = A1 + ((64u * dt) ^ B1), o2 = A2 + ((64u * dt) ^ B2);
        dva[dt] = mfma32(tile_col8_b(qcb + 2 * 64 * D + 32 * D * s2, o1, o2), pb, dva[dt]);
        dka[dt] = mfma32(tile_col8_b(qcb + 32 * D * s2, o1, o2), db, dka[dt]);
      }
    }
  };

  if (nit > 0) {
    load_rows(0);
    copy_item(0, qc0, oc0);
    store_rows(0);
    for (int n = 0; n < nit; n += 2) {
      tile_copies_done();
      __syncthreads();  // item n in buffers 0; everyone is done with buffers 1
      if (n + 1 < nit) {
        load_rows(n + 1);  // before the copy: waiting on these loads does not wait on it
        copy_item(n + 1, qc1, oc1);
      }
      item_step(n, 0, qc0, oc0);
      if (n + 1 < nit) store_rows(1);
      if (n + 1 >= nit) break;
      tile_copies_done();
      __syncthreads();  // item n+1 in buffers 1; everyone is done with buffers 0
      if (n + 2 < nit) {
        load_rows(n + 2);
        copy_item(n + 2, qc0, oc0);
      }
      item_step(n + 1, 1, qc1, oc1);
      if (n + 2 < nit) store_rows(0);
    }
  }

  // dkbar: sum the 32 row-pair partials of each column in a fixed order
  __syncthreads();
  float* red = reinterpret_cast<float*>(ks);
  if (kbthr) {
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[(k2 * 32 + spr) * D + sch * 8 + e] = kbp[k2][e];
  }
  __syncthreads();
  if (tid < 2 * D) {
    const int k2 = tid / D, d = tid % D;
    float g = 0.f;
    for (int pr = 0; pr < 32; ++pr) g += red[(k2 * 32 + pr) * D + d];
    g *= a.ca.coarse_scale;
    kbg[k2][d] = g;
    if (k2 < nblk) a.dkbar[(bh * nb + b0 + k2) * D + d] = g;
  }
  __syncthreads();
  // merge the two query halves, add the pooling term, write bf16 rows; the
  // query-half-1 wave of key pair (kb, kh) leaves its dV and dK partials
  // ([NDT][16][64] floats each) in two of the eight 64-row tile buffers
  const int pairw = w >> 1;  // (kb, kh) index 0..3
  float* red1 = reinterpret_cast<float*>(pairw < 2 ? ks + pairw * 64 * D : vs + (pairw - 2) * 64 * D);
  float* red2 = reinterpret_cast<float*>(pairw == 0 ? qc0 : pairw == 1 ? qc1 : pairw == 2 ? oc0 : oc1);
  if (qh == 1) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        red1[(dt * 16 + r) * 64 + l] = dva[dt][r];
        red2[(dt * 16 + r) * 64 + l] = dka[dt][r];
      }
  }
  __syncthreads();
  if (qh == 0 && kb < nblk) {
    bf16_t* dV = reinterpret_cast<bf16_t*>(a.dv) + bh * a.T * D;
    bf16_t* dK = reinterpret_cast<bf16_t*>(a.dk) + bh * a.T * D;
    const int key = wb * DASH_BLOCK + 32 * kh + j;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * dt + 8 * r4 + 4 * h;
        uint32_t pv2[2], pk2[2];
        float kf4[4];
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          float v0[2], k0[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int r = 4 * r4 + 2 * e2 + e;
            const int ri = (dt * 16 + r) * 64 + l;
            v0[e] = dva[dt][r] + red1[ri];
            // the Stage-2 and Stage-1 terms rounded to fp32 first, then the
            // pooling share added (exact: a power-of-two multiple of dkbar), so
            // a later Stage-0 term added to the unrounded fp32 value
            // (dk_f32) takes the same rounding steps as this one
            k0[e] = fmaf(kbg[kb][d + 2 * e2 + e], a.pool_scale, __fmul_rn(dka[dt][r] + red2[ri], a.fine_scale));
            kf4[2 * e2 + e] = k0[e];
          }
          pv2[e2] = (uint32_t)f2bf(v0[0]) | ((uint32_t)f2bf(v0[1]) << 16);
          pk2[e2] = (uint32_t)f2bf(k0[0]) | ((uint32_t)f2bf(k0[1]) << 16);
        }
        *reinterpret_cast<uint2*>(dV + (size_t)key * D + d) = make_uint2(pv2[0], pv2[1]);
        if (a.dk_f32)
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.dk) + (bh * a.T + key) * D + d) =
              make_float4(kf4[0], kf4[1], kf4[2], kf4[3]);
        else
          *reinterpret_cast<uint2*>(dK + (size_t)key * D + d) = make_uint2(pk2[0], pk2[1]);
      }
  }
}

// ---------------------------------------------------------------------------- entmax backward + coarse dQ

// Sum over the 8 consecutive lanes of a row group (DPP: quad swaps, then
// the half-row mirror), identical in the 8 lanes.
__device__ __forceinline__ float sum8(float v) {
  v += dpp_f<DPP_QSWAP1>(v);
  v += dpp_f<DPP_QSWAP2>(v);
  v += dpp_f<DPP_HMIRROR>(v);
  return v;
}

// Per query row i and the tile's listed candidate blocks b (the entmax
// Jacobian-vector product): s_b = p_b^(2-alpha) on the support,
// dz_b = s_b g_b - s_b <s, g> / sum s with g_b = G_ib / p_ib, computed as
// G_ib p^(1-alpha) from the log2 prior; dz overwrites G (the dK kernel
// reads it for dkbar).  Then dQ_i = dq_acc_i + coarse_scale sum_b dz_b kbar_b.
// Grouped-query heads (GQA): the prior in pbuf is the group's log2 pbar,
// gsum holds G summed over the group and phbuf the row's own log2 p (whose
// Jacobian applies), written by the dQ kernel; with g_b = Gsum_b /
// (grp pbar_b):  s_b g_b = p_b^(2-alpha) Gsum_b pbar_b^-1 / grp.
//
// Workgroup = one 128-row query tile, 4 waves of 32 rows; lane (j, h) of
// wave w holds row 32 w + j.  A first pass over the list gives each row
// <s, g> / sum s (half h takes the entries of parity h, so a half-wave reads
// 32 consecutive rows of one entry, 128 bytes); the second pass, 16 entries
// per k-step, forms the row's dz for the 8 entries its MFMA operand needs,
// stores them, and adds coarse_scale dz kbar to dQ as a matrix product
//   dQc^T (D x 32 rows) += Kbar^T (D x 16 entries) dz^T (16 entries x 32 rows)
// on bf16 MFMA 32x32x16, the summaries of 64 listed entries at a time staged
// in LDS (rows permuted as the forward's V tiles) and read transposed, as
// the forward's PV product reads V.
template <int D, bool GQA>
__global__ __launch_bounds__(256, 2) void bwd_coarse_kernel(BwdArgs a) {
  constexpr int NDT = D / 32;
  constexpr int CH = D / 8;  // 16-byte chunks per summary row
  __shared__ __attribute__((aligned(16))) bf16_t kbt[64 * D];
  __shared__ int lst[DASH_MAX_NB];
  const int nb = a.T / DASH_BLOCK;
  const int ntile = (a.T + DASH_QTILE - 1) / DASH_QTILE;
  const size_t bh = blockIdx.y;
  const int tile = gridDim.x - 1 - blockIdx.x;  // longest lists (last tiles, causal) first
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, j = l & 31, h = l >> 5;
  const int rt = 32 * w + j;
  const int i = tile * DASH_QTILE + rt;
  const bool valid = i < a.T;
  const int own = i / DASH_BLOCK;
  const int* glist = a.tile_blk + (bh * ntile + tile) * nb;
  const int cnt = a.tile_cnt[bh * ntile + tile];
  for (int x = tid; x < cnt; x += 256) lst[x] = glist[x];
  __syncthreads();
  const float am2 = 2.f - (a.ca.softmax ? 1.f : 1.f + a.ca.am1);  // 2 - alpha
  const float am1n = am2 - 1.f;                                    // 1 - alpha
  const size_t bkv = GQA ? bh / a.grp : bh;
  const float inv_grp = GQA ? 1.f / (float)a.grp : 1.f;
  const size_t g0 = gidx(bh, ntile, tile, nb, 0, rt, a.causal);   // entry e at g0 + 128 e
  const size_t s0 = gidx(bkv, ntile, tile, nb, 0, rt, a.causal);  // the group's G sum (GQA)
  // The per-entry values of 8 entries are loaded together before any of
  // them is used, the next 8's while they are summed (entries past the list
  // read as unselected).  s_b and s_b g_b of (this row, entry e) follow;
  // an entry the row does not select (at or after its own block, or p = 0)
  // gives none.
  struct Ent {
    float lp2, g, lpb2;  // log2 p (own), G or G summed over the group, log2 pbar (GQA)
  };
  auto load_ent = [&](int e) -> Ent {
    Ent x{-INFINITY, 0.f, -INFINITY};
    if (e < cnt) {
      const size_t gi = g0 + (size_t)e * DASH_QTILE;
      if constexpr (GQA) {
        x.lpb2 = a.pbuf[gi];
        x.lp2 = a.phbuf[gi];
        x.g = a.gsum[s0 + (size_t)e * DASH_QTILE];
      } else {
        x.lp2 = a.pbuf[gi];
        x.g = a.gbuf[gi];
      }
    }
    return x;
  };
  auto terms = [&](int e, const Ent& x, float& sv, float& sg) -> bool {
    if (e >= cnt || (a.causal && lst[e] >= own)) return false;
    if constexpr (GQA) {
      if (x.lpb2 == -INFINITY || x.lp2 == -INFINITY) return false;
      sv = __builtin_amdgcn_exp2f(am2 * x.lp2);
      sg = sv * (x.g * __builtin_amdgcn_exp2f(-x.lpb2) * inv_grp);
    } else {
      if (x.lp2 == -INFINITY) return false;
      sv = __builtin_amdgcn_exp2f(am2 * x.lp2);
      sg = x.g * __builtin_amdgcn_exp2f(am1n * x.lp2);
    }
    return true;
  };
  float ss = 0.f, ssg = 0.f;
  if (valid) {
    // the next 8 entries' loads go out before this 8's terms are summed
    Ent xn[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) xn[u] = load_ent(h + 2 * u);
    for (int e0 = h; e0 < cnt; e0 += 16) {
      Ent x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = xn[u];
      if (e0 + 16 < cnt) {
#pragma unroll
        for (int u = 0; u < 8; ++u) xn[u] = load_ent(e0 + 16 + 2 * u);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        float sv, sg;
        if (terms(e0 + 2 * u, x[u], sv, sg)) {
          ss += sv;
          ssg += sg;
        }
      }
    }
  }
  ss += __shfl_xor(ss, 32, 64);
  ssg += __shfl_xor(ssg, 32, 64);
  const float ratio = ss > 0.f ? ssg / ss : 0.f;

  // transposing-read offsets (k-step s, d tile dt): A1 + ((64 dt) ^ B1) + 32 D s
  uint32_t A1, B1, A2, B2;
  col8_parts<D, TileSwz<D>::v>(l, A1, B1, A2, B2);
  const char* kbb = reinterpret_cast<const char*>(kbt);
  const bf16_t* KB = reinterpret_cast<const bf16_t*>(a.kbar) + bkv * nb * D;
  f32x16 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  // k-step ks covers entries 16 ks .. 16 ks + 15; this lane's operand
  // entries are 16 ks + 4 h + {0..3} and 16 ks + 8 + 4 h + {0..3}, loaded one
  // k-step ahead
  auto ent_of = [&](int ks, int x) { return 16 * ks + 4 * h + (x < 4 ? x : x + 4); };
  const int nks = (cnt + 15) / 16;
  Ent nx[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) nx[x] = (valid && nks > 0) ? load_ent(ent_of(0, x)) : Ent{-INFINITY, 0.f, -INFINITY};
  for (int ks = 0; ks < nks; ++ks) {
    if ((ks & 3) == 0) {
      const int c0 = 16 * ks;
      __syncthreads();  // the previous chunk's summaries are read
      for (int x = tid; x < 64 * CH; x += 256) {
        const int r = x / CH, c = x % CH;
        const int e = c0 + r;
        const uint4 v = e < cnt ? *reinterpret_cast<const uint4*>(KB + (size_t)lst[e] * D + 8 * c) : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(kbt + r * D + 8 * (c ^ TileSwz<D>::v(r))) = v;
      }
      __syncthreads();
    }
    Ent xe[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) xe[x] = nx[x];
    if (ks + 1 < nks) {
#pragma unroll
      for (int x = 0; x < 8; ++x) nx[x] = valid ? load_ent(ent_of(ks + 1, x)) : Ent{-INFINITY, 0.f, -INFINITY};
    }
    bf16x8 pb;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int e = ent_of(ks, x);
      float dz = 0.f;
      if (valid && e < cnt) {
        float sv, sg;
        if (terms(e, xe[x], sv, sg)) dz = sg - sv * ratio;
        a.gbuf[g0 + (size_t)e * DASH_QTILE] = dz;
      }
      pb[x] = (__bf16)dz;
    }
    const uint32_t so = 32u * D * (ks & 3);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const bf16x8 ka = tile_col8_b(kbb, A1 + ((64u * dt) ^ B1) + so, A2 + ((64u * dt) ^ B2) + so);
      acc[dt] = mfma32(ka, pb, acc[dt]);
    }
  }
  if (!valid) return;
  const float cs = a.ca.coarse_scale;
  const float* dqa = a.dq_acc + (bh * a.T + i) * D;
  bf16_t* dq = reinterpret_cast<bf16_t*>(a.dq) + (bh * a.T + i) * D;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = 32 * dt + 8 * r4 + 4 * h;  // registers 4 r4 .. 4 r4 + 3 hold d .. d + 3
      const float4 f = *reinterpret_cast<const float4*>(dqa + d);
      bf16x4 o4;
      o4[0] = (__bf16)(f.x + cs * acc[dt][4 * r4 + 0]);
      o4[1] = (__bf16)(f.y + cs * acc[dt][4 * r4 + 1]);
      o4[2] = (__bf16)(f.z + cs * acc[dt][4 * r4 + 2]);
      o4[3] = (__bf16)(f.w + cs * acc[dt][4 * r4 + 3]);
      *reinterpret_cast<bf16x4*>(dq + d) = o4;
    }
}

// ---------------------------------------------------------------------------- fp32 path
//
// Three kernels, each output written by one thread in a fixed order (no
// atomics, so reruns give the same bits):
//   bwd_rows_generic   one wave per query row: delta, the row's Stage-2
//                      gradient terms, G per candidate block, the entmax JVP
//                      dz and dQ (fine + coarse); stores delta, the log prior
//                      lp[row][b] of every candidate (-inf when not selected)
//                      and coarse_scale * dz[row][b] in the workspace
//   bwd_dkbar_generic  dkbar_b = sum over rows, ascending, of
//                      coarse_scale dz[row][b] q_row
//   bwd_keys_generic   one wave per key block, lane = key: walks the rows
//                      that attend the block (its own rows when causal, then
//                      the rows whose lp is finite) in ascending order and
//                      accumulates dK, dV; adds the pooling term.
// Scores use dot_row, the generic forward's arithmetic, so both passes see
// the forward's logits bit for bit.

template <typename T>
__global__ __launch_bounds__(64) void bwd_rows_generic_kernel(BwdArgs a) {
  __shared__ float qs[128], gs[128], dsv[64];
  __shared__ float gb[DASH_MAX_NB], lpb[DASH_MAX_NB];
  const int D = a.D;
  const int nb = a.T / DASH_BLOCK;
  const size_t bh = blockIdx.y;
  const int i = blockIdx.x;
  const int l = lane_id();
  const T* q = reinterpret_cast<const T*>(a.q) + (bh * a.T + i) * D;
  const T* go = reinterpret_cast<const T*>(a.dout) + (bh * a.T + i) * D;
  const T* o = reinterpret_cast<const T*>(a.o) + (bh * a.T + i) * D;
  const T* K = reinterpret_cast<const T*>(a.k) + bh * a.T * D;
  const T* V = reinterpret_cast<const T*>(a.v) + bh * a.T * D;
  const T* KB = reinterpret_cast<const T*>(a.kbar) + bh * nb * D;
  float* lp_row = a.pbuf + (bh * a.T + i) * (size_t)nb;
  float* dz_row = a.gbuf + (bh * a.T + i) * (size_t)nb;
  float dl = 0.f;
  for (int d = l; d < D; d += 64) {
    qs[d] = to_f<T>(q[d]);
    gs[d] = to_f<T>(go[d]);
    dl = fmaf(to_f<T>(o[d]), gs[d], dl);
  }
  dl = wave_sum(dl);
  if (l == 0) a.delta[bh * a.T + i] = dl;
  __syncthreads();
  const CoarseArith ca = a.ca;
  const float tau_i = a.tau[bh * a.T + i], ln_i = a.lognorm[bh * a.T + i];
  const float lse = a.lse[bh * a.T + i];
  const int own = i / DASH_BLOCK;
  const int last = a.causal ? own : nb - 1;
  const int nc = a.causal ? own : nb;
  for (int b = l; b < nb; b += 64) lp_row[b] = -INFINITY;  // overwritten below for candidates
  __syncthreads();
  float dq0 = 0.f, dq1 = 0.f;
  for (int b = 0; b <= last; ++b) {
    float pr;
    const bool cand = b < nc;
    if (!cand) pr = 0.f;
    else {
      pr = ca.logp(ca.u_of(dot_row<T>(qs, KB + (size_t)b * D, D)), tau_i, ln_i);
      if (l == 0) { lpb[b] = pr; gb[b] = 0.f; lp_row[b] = pr; }
      if (pr == -INFINITY) continue;
    }
    const int key = b * DASH_BLOCK + l;
    float s = dot_row<T>(qs, K + (size_t)key * D, D) * a.fine_scale + pr;
    if (a.causal && key > i) s = -INFINITY;
    const float p = expf(s - lse);
    const float dp = dot_row<T>(gs, V + (size_t)key * D, D);
    const float ds = p * (dp - dl);
    const float g = wave_sum(ds);
    if (cand && l == 0) gb[b] = g;
    dsv[l] = ds;
    __syncthreads();
    for (int kk = 0; kk < DASH_BLOCK; ++kk) {
      const T* kr = K + (size_t)(b * DASH_BLOCK + kk) * D;
      dq0 = fmaf(dsv[kk], to_f<T>(kr[l]), dq0);
      if (l + 64 < D) dq1 = fmaf(dsv[kk], to_f<T>(kr[l + 64]), dq1);
    }
    __syncthreads();
  }
  dq0 *= a.fine_scale;
  dq1 *= a.fine_scale;
  // entmax backward over the candidates
  __syncthreads();
  const float am2 = ca.softmax ? 1.f : 1.f - ca.am1;  // 2 - alpha
  float ss = 0.f, ssg = 0.f;
  for (int b = l; b < nc; b += 64) {
    const float lpv = lpb[b];
    if (lpv == -INFINITY) continue;
    ss += expf(am2 * lpv);
    ssg += gb[b] * expf((am2 - 1.f) * lpv);
  }
  ss = wave_sum(ss);
  ssg = wave_sum(ssg);
  const float ratio = ss > 0.f ? ssg / ss : 0.f;
  for (int b = l; b < nb; b += 64) dz_row[b] = 0.f;
  __syncthreads();
  for (int b = 0; b < nc; ++b) {
    const float lpv = lpb[b];
    if (lpv == -INFINITY) continue;
    const float dz = (gb[b] * expf((am2 - 1.f) * lpv) - expf(am2 * lpv) * ratio) * ca.coarse_scale;
    const T* kb = KB + (size_t)b * D;
    dq0 = fmaf(dz, to_f<T>(kb[l]), dq0);
    if (l + 64 < D) dq1 = fmaf(dz, to_f<T>(kb[l + 64]), dq1);
    if (l == 0) dz_row[b] = dz;
  }
  float* dQ = reinterpret_cast<float*>(a.dq) + (bh * a.T + i) * D;
  dQ[l] = dq0;
  if (l + 64 < D) dQ[l + 64] = dq1;
}

// dkbar[b][d] = sum over rows r ascending of dz[r][b] q_r[d] (dz carries the
// coarse scale).  grid (nb, BH), 64 threads over d.
template <typename T>
__global__ __launch_bounds__(64) void bwd_dkbar_generic_kernel(BwdArgs a) {
  const int D = a.D;
  const int nb = a.T / DASH_BLOCK;
  const int b = blockIdx.x;
  const size_t bh = blockIdx.y;
  const int l = lane_id();
  const T* Q = reinterpret_cast<const T*>(a.q) + bh * a.T * D;
  const float* dz = a.gbuf + bh * a.T * (size_t)nb + b;
  float acc0 = 0.f, acc1 = 0.f;
  for (int r = a.causal ? (b + 1) * DASH_BLOCK : 0; r < a.T; ++r) {
    const float z = dz[(size_t)r * nb];
    if (z == 0.f) continue;
    acc0 = fmaf(z, to_f<T>(Q[(size_t)r * D + l]), acc0);
    if (l + 64 < D) acc1 = fmaf(z, to_f<T>(Q[(size_t)r * D + l + 64]), acc1);
  }
  float* out = a.dkbar + (bh * nb + b) * D;
  out[l] = acc0;
  if (l + 64 < D) out[l + 64] = acc1;
}

// dK, dV of one key block, lane = key.  DM: the head dim (64 or 128).
template <typename T, int DM>
__global__ __launch_bounds__(64) void bwd_keys_generic_kernel(BwdArgs a) {
  __shared__ float qs[DM], gs[DM];
  const int nb = a.T / DASH_BLOCK;
  const int b = blockIdx.x;
  const size_t bh = blockIdx.y;
  const int l = lane_id();
  const int key = b * DASH_BLOCK + l;
  const T* Q = reinterpret_cast<const T*>(a.q) + bh * a.T * DM;
  const T* dO = reinterpret_cast<const T*>(a.dout) + bh * a.T * DM;
  const T* kr = reinterpret_cast<const T*>(a.k) + (bh * a.T + key) * DM;
  const T* vr = reinterpret_cast<const T*>(a.v) + (bh * a.T + key) * DM;
  const float* lp = a.pbuf + bh * a.T * (size_t)nb + b;
  float dk[DM], dv[DM];
#pragma unroll
  for (int d = 0; d < DM; ++d) { dk[d] = 0.f; dv[d] = 0.f; }
  for (int r = a.causal ? b * DASH_BLOCK : 0; r < a.T; ++r) {
    const bool diag = a.causal && r / DASH_BLOCK == b;
    const float pr = diag ? 0.f : lp[(size_t)r * nb];  // the same for every lane
    if (pr == -INFINITY) continue;
    __syncthreads();  // the previous row's operands are no longer read
    for (int d = l; d < DM; d += 64) {
      qs[d] = to_f<T>(Q[(size_t)r * DM + d]);
      gs[d] = to_f<T>(dO[(size_t)r * DM + d]);
    }
    __syncthreads();
    float s = dot_row<T>(qs, kr, DM) * a.fine_scale + pr;
    if (diag && key > r) s = -INFINITY;
    const float p = expf(s - a.lse[bh * a.T + r]);
    const float dp = dot_row<T>(gs, vr, DM);
    const float ds = p * (dp - a.delta[bh * a.T + r]);
#pragma unroll
    for (int d = 0; d < DM; ++d) {
      dk[d] = fmaf(ds, qs[d], dk[d]);
      dv[d] = fmaf(p, gs[d], dv[d]);
    }
  }
  const float* kbg = a.dkbar + (bh * nb + b) * DM;
  float* dK = reinterpret_cast<float*>(a.dk) + (bh * a.T + key) * DM;
  float* dV = reinterpret_cast<float*>(a.dv) + (bh * a.T + key) * DM;
#pragma unroll
  for (int d = 0; d < DM; ++d) {
    dK[d] = dk[d] * a.fine_scale + a.pool_scale * kbg[d];
    dV[d] = dv[d];
  }
}

// Grouped-query heads: G of the group's heads summed per (tile, listed
// block, row) into gsum, in head order.  grid (ntile, BH / grp), 256
// threads; a thread takes 4 consecutive rows of an entry (16-byte loads) and
// has the grp heads' loads in flight together.
template <int GRP>
__global__ __launch_bounds__(256) void bwd_gqa_gsum_kernel(BwdArgs a) {
  const int ntile = (a.T + DASH_QTILE - 1) / DASH_QTILE;
  const int nb = a.T / DASH_BLOCK;
  const int tile = gridDim.x - 1 - blockIdx.x;  // longest lists first
  const size_t bkv = blockIdx.y, bh0 = bkv * GRP;
  const int cnt = a.tile_cnt[bh0 * ntile + tile];  // the group's heads share the list
  const size_t hstride = bwd_entries_per_head(a.causal, nb, ntile) * DASH_QTILE;  // floats per head
  const float* g0 = a.gbuf + gidx(bh0, ntile, tile, nb, 0, 0, a.causal);
  float* gs = a.gsum + gidx(bkv, ntile, tile, nb, 0, 0, a.causal);
  for (int x = threadIdx.x; x < cnt * (DASH_QTILE / 4); x += blockDim.x) {
    float4 v[GRP];
#pragma unroll
    for (int h = 0; h < GRP; ++h) v[h] = *reinterpret_cast<const float4*>(g0 + h * hstride + 4 * (size_t)x);
    float4 g = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      g.x += v[h].x;
      g.y += v[h].y;
      g.z += v[h].z;
      g.w += v[h].w;
    }
    *reinterpret_cast<float4*>(gs + 4 * (size_t)x) = g;
  }
}

// dK, dV (bf16, 8 per thread, fp32 sums) and dkbar of each KV head = the sum
// of its query heads' partials, in head order.
__global__ void bwd_gqa_reduce_kernel(const bf16_t* __restrict__ dkp, const bf16_t* __restrict__ dvp,
                                      const float* __restrict__ dkbp, bf16_t* __restrict__ dk,
                                      bf16_t* __restrict__ dv, float* __restrict__ dkbar, int BHkv, int grp,
                                      size_t TD, size_t nbD) {
  const size_t n8 = (size_t)BHkv * TD / 8;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t x = (size_t)blockIdx.x * blockDim.x + threadIdx.x; x < n8; x += stride) {
    const size_t g = (x * 8) / TD, r = (x * 8) % TD;
    float sk[8], sv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sk[e] = sv[e] = 0.f;
    for (int h = 0; h < grp; ++h) {
      const size_t src = ((size_t)g * grp + h) * TD + r;
      const uint4 kw = *reinterpret_cast<const uint4*>(dkp + src);
      const uint4 vw = *reinterpret_cast<const uint4*>(dvp + src);
      const uint32_t ku[4] = {kw.x, kw.y, kw.z, kw.w}, vu[4] = {vw.x, vw.y, vw.z, vw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sk[2 * e] += __uint_as_float(ku[e] << 16);
        sk[2 * e + 1] += __uint_as_float(ku[e] & 0xFFFF0000u);
        sv[2 * e] += __uint_as_float(vu[e] << 16);
        sv[2 * e + 1] += __uint_as_float(vu[e] & 0xFFFF0000u);
      }
    }
    uint32_t ko[4], vo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ko[e] = (uint32_t)f2bf(sk[2 * e]) | ((uint32_t)f2bf(sk[2 * e + 1]) << 16);
      vo[e] = (uint32_t)f2bf(sv[2 * e]) | ((uint32_t)f2bf(sv[2 * e + 1]) << 16);
    }
    *reinterpret_cast<uint4*>(dk + x * 8) = make_uint4(ko[0], ko[1], ko[2], ko[3]);
    *reinterpret_cast<uint4*>(dv + x * 8) = make_uint4(vo[0], vo[1], vo[2], vo[3]);
  }
  const size_t nkb = (size_t)BHkv * nbD;
  for (size_t x = (size_t)blockIdx.x * blockDim.x + threadIdx.x; x < nkb; x += stride) {
    const size_t g = x / nbD, r = x % nbD;
    float sum = 0.f;
    for (int h = 0; h < grp; ++h) sum += dkbp[((size_t)g * grp + h) * nbD + r];
    dkbar[x] = sum;
  }
}

hipError_t launch_bwd_gqa(const BwdArgs& a, void* dk, void* dv, float* dkbar, hipStream_t st) {
  if (a.grp <= 1 || a.BH % a.grp) return hipErrorInvalidValue;
  const size_t rows = (size_t)a.BH * a.T;
  const int ntile = (a.T + DASH_QTILE - 1) / DASH_QTILE;
  const int nb = a.T / DASH_BLOCK;
  hipError_t e;
  if ((e = launch_delta_bf16(a, rows, st)) != hipSuccess) return e;
  if (a.D == 128) bwd_dq_kernel<128, true><<<ntile * a.BH, 256, 0, st>>>(a);
  else bwd_dq_kernel<64, true><<<ntile * a.BH, 256, 0, st>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  {
    const dim3 grid(ntile, a.BH / a.grp);
    if (a.grp == 2) bwd_gqa_gsum_kernel<2><<<grid, 256, 0, st>>>(a);
    else if (a.grp == 4) bwd_gqa_gsum_kernel<4><<<grid, 256, 0, st>>>(a);
    else if (a.grp == 8) bwd_gqa_gsum_kernel<8><<<grid, 256, 0, st>>>(a);
    else return hipErrorNotSupported;
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.D == 128) bwd_coarse_kernel<128, true><<<dim3(ntile, a.BH), 256, 0, st>>>(a);
  else bwd_coarse_kernel<64, true><<<dim3(ntile, a.BH), 256, 0, st>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int ngrp = (nb + 1) / 2;
  if (a.D == 128) bwd_dkdv_kernel<128><<<ngrp * a.BH, 512, 0, st>>>(a);
  else bwd_dkdv_kernel<64><<<ngrp * a.BH, 512, 0, st>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  bwd_gqa_reduce_kernel<<<2048, 256, 0, st>>>(reinterpret_cast<const bf16_t*>(a.dk), reinterpret_cast<const bf16_t*>(a.dv),
                                              a.dkbar, reinterpret_cast<bf16_t*>(dk), reinterpret_cast<bf16_t*>(dv), dkbar,
                                              a.BH / a.grp, a.grp, (size_t)a.T * a.D, (size_t)nb * a.D);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, int dtype, hipStream_t st) {
  const size_t rows = (size_t)a.BH * a.T;
  const int ntile = (a.T + DASH_QTILE - 1) / DASH_QTILE;
  const int nb = a.T / DASH_BLOCK;
  hipError_t e;
  if (dtype == 1) {
    if ((e = launch_delta_bf16(a, rows, st)) != hipSuccess) return e;
    if (a.D == 128) bwd_dq_kernel<128, false><<<ntile * a.BH, 256, 0, st>>>(a);
    else bwd_dq_kernel<64, false><<<ntile * a.BH, 256, 0, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.D == 128) bwd_coarse_kernel<128, false><<<dim3(ntile, a.BH), 256, 0, st>>>(a);
    else bwd_coarse_kernel<64, false><<<dim3(ntile, a.BH), 256, 0, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int ngrp = (nb + 1) / 2;
    if (a.D == 128) bwd_dkdv_kernel<128><<<ngrp * a.BH, 512, 0, st>>>(a);
    else bwd_dkdv_kernel<64><<<ngrp * a.BH, 512, 0, st>>>(a);
    return hipGetLastError();
  }
  bwd_rows_generic_kernel<float><<<dim3(a.T, a.BH), 64, 0, st>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  bwd_dkbar_generic_kernel<float><<<dim3(nb, a.BH), 64, 0, st>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.D == 128) bwd_keys_generic_kernel<float, 128><<<dim3(nb, a.BH), 64, 0, st>>>(a);
  else bwd_keys_generic_kernel<float, 64><<<dim3(nb, a.BH), 64, 0, st>>>(a);
  return hipGetLastError();
}
