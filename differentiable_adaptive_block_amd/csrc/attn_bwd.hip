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
//   dK_j += dkbar_{blk(j)} / 64.
//
// bf16 path (deterministic, no floating-point atomics):
//   bwd_delta     delta
//   bwd_dq        query-tile-major, walks the tile's block list like the forward;
//                 MFMA for S^T, dP^T and dQ^T; writes G and the log2 prior of
//                 every (row, listed block) to the workspace
//   bwd_entmax    per row: dz over its listed candidate blocks (overwrites G)
//   bwd_dkdv      key-block-major over the query tiles whose list holds the
//                 block; MFMA for S, dP, dV^T and dK^T; also dkbar and the
//                 pooling term
//   bwd_dq_final  dQ = fine part + coarse part, to bf16
// fp32 path: one wave per query row, dK / dV / dkbar by float atomics.
#include "kernels.h"

#define LOG2E_F 1.4426950408889634f

// ---------------------------------------------------------------------------- delta

template <typename T>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const T* __restrict__ o, const T* __restrict__ dout,
                                                        float* __restrict__ delta, size_t rows, int D) {
  const size_t r = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (r >= rows) return;
  float acc = 0.f;
  for (int d = l; d < D; d += 64) acc = fmaf(to_f<T>(o[r * D + d]), to_f<T>(dout[r * D + d]), acc);
  acc = wave_sum(acc);
  if (l == 0) delta[r] = acc;
}

// ---------------------------------------------------------------------------- dQ (fine), G, priors

__device__ __forceinline__ size_t gidx(size_t bh, int ntile, int tile, int nb, int e, int row_in_tile) {
  return (((bh * ntile + tile) * (size_t)nb + e) * DASH_QTILE) + row_in_tile;
}

template <int D>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a) {
  constexpr int KP = D + 8;
  constexpr int VP = 64 + 4;
  constexpr int CH = D / 8;
  constexpr int NVL = 64 * CH / 256;   // V uint4 per thread
  constexpr int NKP = 32 * CH / 256;   // K row pairs per thread
  __shared__ __attribute__((aligned(16))) bf16_t ks[64 * KP];
  __shared__ __attribute__((aligned(16))) bf16_t vs[64 * KP];
  __shared__ __attribute__((aligned(16))) bf16_t kt[D * VP];
  __shared__ float pri[4][32 * 32];

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

  const bf16_t* Q = reinterpret_cast<const bf16_t*>(a.q) + bh * a.T * D;
  const bf16_t* K = reinterpret_cast<const bf16_t*>(a.k) + bh * a.T * D;
  const bf16_t* V = reinterpret_cast<const bf16_t*>(a.v) + bh * a.T * D;
  const bf16_t* dO = reinterpret_cast<const bf16_t*>(a.dout) + bh * a.T * D;
  const bf16_t* KB = reinterpret_cast<const bf16_t*>(a.kbar) + bh * nb * D;
  const int* list = a.tile_blk + (bh * ntile + tile) * nb;
  const int cnt = a.tile_cnt[bh * ntile + tile];
  const CoarseArith ca = a.ca;
  const float sl2 = a.fine_scale * LOG2E_F;

  bf16x8 qb[D / 16], dob[D / 16];
  float tau_i = 0.f, ln_i = 0.f, lse2 = 0.f, dlt = 0.f;
  if (active) {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      qb[s] = load8(Q + (size_t)i * D + 16 * s + 8 * h);
      dob[s] = load8(dO + (size_t)i * D + 16 * s + 8 * h);
    }
    tau_i = a.tau[bh * a.T + i];
    ln_i = a.lognorm[bh * a.T + i];
    lse2 = a.lse[bh * a.T + i] * LOG2E_F;
    dlt = a.delta[bh * a.T + i];
  }
  f32x16 dqa[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqa[dt][r] = 0.f;

  uint4 kr[2 * NKP], vr[NVL];
  auto gload = [&](int b) {
    const bf16_t* kb0 = K + (size_t)b * DASH_BLOCK * D;
    const bf16_t* vb0 = V + (size_t)b * DASH_BLOCK * D;
#pragma unroll
    for (int x = 0; x < NKP; ++x) {
      const int idx = tid + 256 * x;
      const int pr = idx / CH, ch = idx % CH;
      kr[2 * x] = *reinterpret_cast<const uint4*>(kb0 + (size_t)(2 * pr) * D + ch * 8);
      kr[2 * x + 1] = *reinterpret_cast<const uint4*>(kb0 + (size_t)(2 * pr + 1) * D + ch * 8);
    }
#pragma unroll
    for (int x = 0; x < NVL; ++x) {
      const int idx = tid + 256 * x;
      vr[x] = *reinterpret_cast<const uint4*>(vb0 + (size_t)(idx / CH) * D + (idx % CH) * 8);
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int x = 0; x < NKP; ++x) {
      const int idx = tid + 256 * x;
      const int pr = idx / CH, ch = idx % CH;
      *reinterpret_cast<uint4*>(&ks[(2 * pr) * KP + ch * 8]) = kr[2 * x];
      *reinterpret_cast<uint4*>(&ks[(2 * pr + 1) * KP + ch * 8]) = kr[2 * x + 1];
      const uint32_t* k0 = reinterpret_cast<const uint32_t*>(&kr[2 * x]);
      const uint32_t* k1 = reinterpret_cast<const uint32_t*>(&kr[2 * x + 1]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = (e & 1) ? (k0[e >> 1] >> 16) : (k0[e >> 1] & 0xFFFFu);
        const uint32_t hi = (e & 1) ? (k1[e >> 1] >> 16) : (k1[e >> 1] & 0xFFFFu);
        *reinterpret_cast<uint32_t*>(&kt[(ch * 8 + e) * VP + 2 * pr]) = lo | (hi << 16);
      }
    }
#pragma unroll
    for (int x = 0; x < NVL; ++x) {
      const int idx = tid + 256 * x;
      *reinterpret_cast<uint4*>(&vs[(idx / CH) * KP + (idx % CH) * 8]) = vr[x];
    }
  };
  auto put_g = [&](int e, float g, float p2) {
    if (h == 0) {
      const size_t gi = gidx(bh, ntile, tile, nb, e, w * 32 + j);
      a.gbuf[gi] = g;
      a.pbuf[gi] = p2;
    }
  };

  if (cnt > 0) gload(list[0]);
  for (int e = 0; e < cnt; ++e) {
    const int b = list[e];
    __syncthreads();
    sstore();
    if ((e & 31) == 0 && active) {
      const int ent = e + j;
      f32x16 acc = coarse_acc_chunk<D>(KB, ent < cnt ? list[ent] : 0, qb);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int slot = acc_row32(r, l);
        const int en = e + slot;
        float p2 = -INFINITY;
        if (en < cnt) {
          const int bb = list[en];
          if (!a.causal || bb < wblk) p2 = ca.logp(ca.u_of(acc[r]), tau_i, ln_i) * LOG2E_F;
        }
        pri[w][slot * 32 + j] = p2;
      }
    }
    __syncthreads();
    if (e + 1 < cnt) gload(list[e + 1]);
    if (!active) continue;
    if (a.causal && b > wblk) {
      put_g(e, 0.f, -INFINITY);
      continue;
    }
    const bool diag = a.causal && b == wblk;
    const float pr = diag ? 0.f : pri[w][(e & 31) * 32 + j];
    if (!diag && __ballot(pr != -INFINITY) == 0ull) {
      put_g(e, 0.f, -INFINITY);
      continue;
    }
    float gsum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) { s[r] = 0.f; dp[r] = 0.f; }
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        const bf16x8 ak = *reinterpret_cast<const bf16x8*>(&ks[(32 * t + j) * KP + 16 * st + 8 * h]);
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(&vs[(32 * t + j) * KP + 16 * st + 8 * h]);
        s = mfma32(ak, qb[st], s);
        dp = mfma32(av, dob[st], dp);
      }
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[r] * sl2 + pr;
        if (diag && b * DASH_BLOCK + 32 * t + acc_row32(r, l) > i) x = -INFINITY;
        const float p = exp2f(x - lse2);
        ds[r] = p * (dp[r] - dlt);
        gsum += ds[r];
      }
      // dQ^T += K^T dS^T over this half's 32 keys (2 k-steps of 16)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8 pb;
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) pb[e8] = (__bf16)ds[8 * s2 + e8];
        const int key0 = 32 * t + 16 * s2 + 4 * h;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const bf16_t* krow = &kt[(32 * dt + j) * VP + key0];
          const uint2 lo = *reinterpret_cast<const uint2*>(krow);
          const uint2 hi = *reinterpret_cast<const uint2*>(krow + 8);
          const uint4 pk = make_uint4(lo.x, lo.y, hi.x, hi.y);
          dqa[dt] = mfma32(__builtin_bit_cast(bf16x8, pk), pb, dqa[dt]);
        }
      }
    }
    gsum += __shfl_xor(gsum, 32, 64);
    put_g(e, diag ? 0.f : gsum, pr);
  }
  if (active) {
    float* dq = a.dq_acc + (bh * a.T + i) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * dt + 8 * r4 + 4 * h;
        float4 v4 = make_float4(dqa[dt][4 * r4] * a.fine_scale, dqa[dt][4 * r4 + 1] * a.fine_scale,
                                dqa[dt][4 * r4 + 2] * a.fine_scale, dqa[dt][4 * r4 + 3] * a.fine_scale);
        *reinterpret_cast<float4*>(dq + d) = v4;
      }
  }
}

// ---------------------------------------------------------------------------- entmax backward

// One thread per query row: dz over the row's listed candidate blocks,
// written over G; zero for every other slot.
__global__ __launch_bounds__(128) void bwd_entmax_kernel(BwdArgs a) {
  const int nb = a.T / DASH_BLOCK;
  const int ntile = (a.T + DASH_QTILE - 1) / DASH_QTILE;
  const size_t bh = blockIdx.y;
  const int tile = blockIdx.x;
  const int rt = threadIdx.x;
  const int i = tile * DASH_QTILE + rt;
  if (i >= a.T) return;
  const int own = i / DASH_BLOCK;
  const int* list = a.tile_blk + (bh * ntile + tile) * nb;
  const int cnt = a.tile_cnt[bh * ntile + tile];
  const float am2 = 2.f - (a.ca.softmax ? 1.f : 1.f + a.ca.am1);  // 2 - alpha
  const float am1n = am2 - 1.f;                                    // 1 - alpha
  float ss = 0.f, ssg = 0.f;
  for (int e = 0; e < cnt; ++e) {
    const int b = list[e];
    if (a.causal && b >= own) continue;
    const size_t gi = gidx(bh, ntile, tile, nb, e, rt);
    const float lp2 = a.pbuf[gi];
    if (lp2 == -INFINITY) continue;
    ss += exp2f(am2 * lp2);
    ssg += a.gbuf[gi] * exp2f(am1n * lp2);
  }
  const float ratio = ss > 0.f ? ssg / ss : 0.f;
  for (int e = 0; e < cnt; ++e) {
    const int b = list[e];
    const size_t gi = gidx(bh, ntile, tile, nb, e, rt);
    float dz = 0.f;
    if (!(a.causal && b >= own)) {
      const float lp2 = a.pbuf[gi];
      if (lp2 != -INFINITY) dz = a.gbuf[gi] * exp2f(am1n * lp2) - exp2f(am2 * lp2) * ratio;
    }
    a.gbuf[gi] = dz;
  }
}

// ---------------------------------------------------------------------------- dK, dV, dkbar

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int KP = D + 8;
  constexpr int QP = 64 + 4;
  constexpr int CH = D / 8;
  constexpr int NL = 64 * CH / 256;  // uint4 per thread for a 64-row tile
  constexpr int NP = 32 * CH / 256;  // row pairs per thread
  // one LDS buffer: [ks | vs | qs | qt | os | ot]; after the main loop the
  // qs..ot part (>= 2 x 2 x (D/32) x 16 x 64 floats) holds the cross-wave sums
  constexpr int ROWT = 64 * KP;  // bf16 elements of a 64-row tile
  constexpr int COLT = D * QP;   // bf16 elements of a transposed tile
  __shared__ __attribute__((aligned(16))) bf16_t smem[4 * ROWT + 2 * COLT];
  static_assert((2 * ROWT + 2 * COLT) * 2 >= 2 * 2 * (D / 32) * 16 * 64 * 4, "reduction space");
  bf16_t* ks = smem;
  bf16_t* vs = ks + ROWT;
  bf16_t* qs = vs + ROWT;
  bf16_t* qt = qs + ROWT;
  bf16_t* os_ = qt + COLT;
  bf16_t* ot = os_ + ROWT;
  __shared__ float prq[64], lsq[64], dlq[64], dzq[64];
  __shared__ float kbg[D];

  const int nb = a.T / DASH_BLOCK;
  const int nbw = (nb + 31) / 32;
  const int ntile = (a.T + DASH_QTILE - 1) / DASH_QTILE;
  const int nwg = gridDim.x, wg = blockIdx.x;
  const int logical = (nwg % 8 == 0) ? (wg % 8) * (nwg / 8) + wg / 8 : wg;
  const size_t bh = logical / nb;
  const int b = logical % nb;  // early blocks (most query tiles when causal) first
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, j = l & 31, h = l >> 5;
  const int kh = w & 1, qh = w >> 1;

  const bf16_t* Q = reinterpret_cast<const bf16_t*>(a.q) + bh * a.T * D;
  const bf16_t* K = reinterpret_cast<const bf16_t*>(a.k) + bh * a.T * D;
  const bf16_t* V = reinterpret_cast<const bf16_t*>(a.v) + bh * a.T * D;
  const bf16_t* dO = reinterpret_cast<const bf16_t*>(a.dout) + bh * a.T * D;
  const float sl2 = a.fine_scale * LOG2E_F;

  // the key block, row-major
  {
    const bf16_t* kb0 = K + (size_t)b * DASH_BLOCK * D;
    const bf16_t* vb0 = V + (size_t)b * DASH_BLOCK * D;
#pragma unroll
    for (int x = 0; x < NL; ++x) {
      const int idx = tid + 256 * x;
      const int row = idx / CH, ch = idx % CH;
      *reinterpret_cast<uint4*>(&ks[row * KP + ch * 8]) = *reinterpret_cast<const uint4*>(kb0 + (size_t)row * D + ch * 8);
      *reinterpret_cast<uint4*>(&vs[row * KP + ch * 8]) = *reinterpret_cast<const uint4*>(vb0 + (size_t)row * D + ch * 8);
    }
  }
  f32x16 dva[D / 32], dka[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dva[dt][r] = 0.f; dka[dt][r] = 0.f; }
  float kbacc = 0.f;  // dkbar_b[tid] for tid < D

  const int t0 = a.causal ? (b * DASH_BLOCK) / DASH_QTILE : 0;
  for (int t = t0; t < ntile; ++t) {
    const uint32_t* bits = a.tile_bits + (bh * ntile + t) * nbw;
    const uint32_t word = bits[b >> 5];
    if (!((word >> (b & 31)) & 1u)) continue;
    int slot = __popc(word & ((1u << (b & 31)) - 1u));
    for (int x = 0; x < (b >> 5); ++x) slot += __popc(bits[x]);
    for (int c = 0; c < DASH_QTILE / 64; ++c) {
      const int q0 = t * DASH_QTILE + c * 64;
      if (q0 >= a.T) break;
      if (a.causal && q0 / DASH_BLOCK < b) continue;  // queries before the block never see it
      const bool diag = a.causal && q0 / DASH_BLOCK == b;
      __syncthreads();
      // stage Q and dO rows q0..q0+63 (row-major and transposed) and per-row scalars
#pragma unroll
      for (int x = 0; x < NP; ++x) {
        const int idx = tid + 256 * x;
        const int pr = idx / CH, ch = idx % CH;
        const size_t r0 = (size_t)(q0 + 2 * pr) * D + ch * 8;
        const uint4 q0v = *reinterpret_cast<const uint4*>(Q + r0);
        const uint4 q1v = *reinterpret_cast<const uint4*>(Q + r0 + D);
        const uint4 o0v = *reinterpret_cast<const uint4*>(dO + r0);
        const uint4 o1v = *reinterpret_cast<const uint4*>(dO + r0 + D);
        *reinterpret_cast<uint4*>(&qs[(2 * pr) * KP + ch * 8]) = q0v;
        *reinterpret_cast<uint4*>(&qs[(2 * pr + 1) * KP + ch * 8]) = q1v;
        *reinterpret_cast<uint4*>(&os_[(2 * pr) * KP + ch * 8]) = o0v;
        *reinterpret_cast<uint4*>(&os_[(2 * pr + 1) * KP + ch * 8]) = o1v;
        const uint32_t* a0 = reinterpret_cast<const uint32_t*>(&q0v);
        const uint32_t* a1 = reinterpret_cast<const uint32_t*>(&q1v);
        const uint32_t* b0 = reinterpret_cast<const uint32_t*>(&o0v);
        const uint32_t* b1 = reinterpret_cast<const uint32_t*>(&o1v);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int sh = (e & 1) * 16;
          *reinterpret_cast<uint32_t*>(&qt[(ch * 8 + e) * QP + 2 * pr]) =
              ((a0[e >> 1] >> sh) & 0xFFFFu) | (((a1[e >> 1] >> sh) & 0xFFFFu) << 16);
          *reinterpret_cast<uint32_t*>(&ot[(ch * 8 + e) * QP + 2 * pr]) =
              ((b0[e >> 1] >> sh) & 0xFFFFu) | (((b1[e >> 1] >> sh) & 0xFFFFu) << 16);
        }
      }
      if (tid < 64) {
        const size_t gi = gidx(bh, ntile, t, nb, slot, c * 64 + tid);
        prq[tid] = a.pbuf[gi];
        dzq[tid] = a.gbuf[gi];
        lsq[tid] = a.lse[bh * a.T + q0 + tid] * LOG2E_F;
        dlq[tid] = a.delta[bh * a.T + q0 + tid];
      }
      __syncthreads();
      // S = Q K^T and dP = dO V^T for this wave's 32 queries x 32 keys
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) { s[r] = 0.f; dp[r] = 0.f; }
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        const bf16x8 aq = *reinterpret_cast<const bf16x8*>(&qs[(32 * qh + j) * KP + 16 * st + 8 * h]);
        const bf16x8 ao = *reinterpret_cast<const bf16x8*>(&os_[(32 * qh + j) * KP + 16 * st + 8 * h]);
        const bf16x8 bk = *reinterpret_cast<const bf16x8*>(&ks[(32 * kh + j) * KP + 16 * st + 8 * h]);
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&vs[(32 * kh + j) * KP + 16 * st + 8 * h]);
        s = mfma32(aq, bk, s);
        dp = mfma32(ao, bv, dp);
      }
      float pv[16], dsv[16];
      const int key = b * DASH_BLOCK + 32 * kh + j;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = 32 * qh + acc_row32(r, l);
        float x = s[r] * sl2 + prq[ql];
        if (diag && key > q0 + ql) x = -INFINITY;
        const float p = exp2f(x - lsq[ql]);
        pv[r] = p;
        dsv[r] = p * (dp[r] - dlq[ql]);
      }
      // dV^T += dO^T P and dK^T += Q^T dS over the 32 queries (2 k-steps)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8 pb, db;
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) {
          pb[e8] = (__bf16)pv[8 * s2 + e8];
          db[e8] = (__bf16)dsv[8 * s2 + e8];
        }
        const int qk0 = 32 * qh + 16 * s2 + 4 * h;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const bf16_t* orow = &ot[(32 * dt + j) * QP + qk0];
          const bf16_t* qrow = &qt[(32 * dt + j) * QP + qk0];
          const uint2 olo = *reinterpret_cast<const uint2*>(orow);
          const uint2 ohi = *reinterpret_cast<const uint2*>(orow + 8);
          const uint2 qlo = *reinterpret_cast<const uint2*>(qrow);
          const uint2 qhi = *reinterpret_cast<const uint2*>(qrow + 8);
          dva[dt] = mfma32(__builtin_bit_cast(bf16x8, make_uint4(olo.x, olo.y, ohi.x, ohi.y)), pb, dva[dt]);
          dka[dt] = mfma32(__builtin_bit_cast(bf16x8, make_uint4(qlo.x, qlo.y, qhi.x, qhi.y)), db, dka[dt]);
        }
      }
      // dkbar_b += sum_q dz_qb q_q  (the coarse scale is applied at the end)
      if (tid < D) {
        float acc = 0.f;
        for (int q = 0; q < 64; ++q) acc = fmaf(dzq[q], bf2f(qs[q * KP + tid]), acc);
        kbacc += acc;
      }
    }
  }
  // merge the two query halves, add the pooling term, write bf16 rows
  __syncthreads();
  float* red = reinterpret_cast<float*>(qs);  // qs, qt, os_, ot are free now
  float* red2 = red + 2 * (D / 32) * 16 * 64;
  if (tid < D) {
    const float g = kbacc * a.ca.coarse_scale;
    kbg[tid] = g;
    a.dkbar[(bh * nb + b) * D + tid] = g;
  }
  if (qh == 1) {
    // [kh][dt][r][lane] layout, 2 x (D/32) x 16 x 64 floats = 16 KB per array for D = 128
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        red[((kh * (D / 32) + dt) * 16 + r) * 64 + l] = dva[dt][r];
        red2[((kh * (D / 32) + dt) * 16 + r) * 64 + l] = dka[dt][r];
      }
  }
  __syncthreads();
  if (qh == 0) {
    bf16_t* dV = reinterpret_cast<bf16_t*>(a.dv) + bh * a.T * D;
    bf16_t* dK = reinterpret_cast<bf16_t*>(a.dk) + bh * a.T * D;
    const int key = b * DASH_BLOCK + 32 * kh + j;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * dt + 8 * r4 + 4 * h;
        uint32_t pv2[2], pk2[2];
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          float v0[2], k0[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int r = 4 * r4 + 2 * e2 + e;
            const size_t ri = ((kh * (D / 32) + dt) * 16 + r) * 64 + l;
            v0[e] = dva[dt][r] + red[ri];
            k0[e] = (dka[dt][r] + red2[ri]) * a.fine_scale + kbg[d + 2 * e2 + e] * (1.f / DASH_BLOCK);
          }
          pv2[e2] = (uint32_t)f2bf(v0[0]) | ((uint32_t)f2bf(v0[1]) << 16);
          pk2[e2] = (uint32_t)f2bf(k0[0]) | ((uint32_t)f2bf(k0[1]) << 16);
        }
        *reinterpret_cast<uint2*>(dV + (size_t)key * D + d) = make_uint2(pv2[0], pv2[1]);
        *reinterpret_cast<uint2*>(dK + (size_t)key * D + d) = make_uint2(pk2[0], pk2[1]);
      }
  }
}

// ---------------------------------------------------------------------------- dQ finalize

// dQ_i = fine part (dq_acc) + coarse_scale * sum_slots dz_i,slot kbar_{list[slot]}.
// grid (ntile * 4, BH), 256 threads = 32 rows x 8 groups of 16 columns (D = 128)
// or 32 rows x 8 groups of 8 columns (D = 64).
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_final_kernel(BwdArgs a) {
  constexpr int G = D / 8;  // columns per thread
  const int nb = a.T / DASH_BLOCK;
  const int ntile = (a.T + DASH_QTILE - 1) / DASH_QTILE;
  const size_t bh = blockIdx.y;
  const int tile = blockIdx.x >> 2;
  const int sub = blockIdx.x & 3;
  const int rt = sub * 32 + (threadIdx.x >> 3);
  const int cg = threadIdx.x & 7;
  const int i = tile * DASH_QTILE + rt;
  if (i >= a.T) return;
  const int* list = a.tile_blk + (bh * ntile + tile) * nb;
  const int cnt = a.tile_cnt[bh * ntile + tile];
  const bf16_t* KB = reinterpret_cast<const bf16_t*>(a.kbar) + bh * nb * D;
  float acc[G];
#pragma unroll
  for (int x = 0; x < G; ++x) acc[x] = 0.f;
  for (int e = 0; e < cnt; ++e) {
    const float dz = a.gbuf[gidx(bh, ntile, tile, nb, e, rt)];
    if (dz == 0.f) continue;
    const bf16_t* kr = KB + (size_t)list[e] * D + cg * G;
#pragma unroll
    for (int x = 0; x < G; ++x) acc[x] = fmaf(dz, bf2f(kr[x]), acc[x]);
  }
  const float* dqa = a.dq_acc + (bh * a.T + i) * D + cg * G;
  bf16_t* dq = reinterpret_cast<bf16_t*>(a.dq) + (bh * a.T + i) * D + cg * G;
#pragma unroll
  for (int x = 0; x < G; ++x) dq[x] = f2bf(dqa[x] + a.ca.coarse_scale * acc[x]);
}

// ---------------------------------------------------------------------------- fp32 path

// One wave per query row; dK, dV and dkbar accumulate with float atomics
// (zeroed first), dQ is owned by the row.  Blocks in ascending order, the
// prior from the same dot_row score as the generic forward.
template <typename T>
__global__ __launch_bounds__(64) void bwd_generic_kernel(BwdArgs a) {
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
  float* dK = reinterpret_cast<float*>(a.dk) + bh * a.T * D;
  float* dV = reinterpret_cast<float*>(a.dv) + bh * a.T * D;
  float* dKB = a.dkbar + bh * nb * D;
  float dl = 0.f;
  for (int d = l; d < D; d += 64) {
    qs[d] = to_f<T>(q[d]);
    gs[d] = to_f<T>(go[d]);
    dl = fmaf(to_f<T>(o[d]), gs[d], dl);
  }
  dl = wave_sum(dl);
  __syncthreads();
  const CoarseArith ca = a.ca;
  const float tau_i = a.tau[bh * a.T + i], ln_i = a.lognorm[bh * a.T + i];
  const float lse = a.lse[bh * a.T + i];
  const int own = i / DASH_BLOCK;
  const int last = a.causal ? own : nb - 1;
  const int nc = a.causal ? own : nb;
  float dq0 = 0.f, dq1 = 0.f;
  for (int b = 0; b <= last; ++b) {
    float pr;
    const bool cand = b < nc;
    if (!cand) pr = 0.f;
    else {
      pr = ca.logp(ca.u_of(dot_row<T>(qs, KB + (size_t)b * D, D)), tau_i, ln_i);
      if (l == 0) { lpb[b] = pr; gb[b] = 0.f; }
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
    for (int d = 0; d < D; ++d) {
      atomicAdd(&dK[(size_t)key * D + d], a.fine_scale * ds * qs[d]);
      atomicAdd(&dV[(size_t)key * D + d], p * gs[d]);
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
    const float lp = lpb[b];
    if (lp == -INFINITY) continue;
    ss += expf(am2 * lp);
    ssg += gb[b] * expf((am2 - 1.f) * lp);
  }
  ss = wave_sum(ss);
  ssg = wave_sum(ssg);
  const float ratio = ss > 0.f ? ssg / ss : 0.f;
  for (int b = 0; b < nc; ++b) {
    const float lp = lpb[b];
    if (lp == -INFINITY) continue;
    const float dz = (gb[b] * expf((am2 - 1.f) * lp) - expf(am2 * lp) * ratio) * ca.coarse_scale;
    const T* kb = KB + (size_t)b * D;
    dq0 = fmaf(dz, to_f<T>(kb[l]), dq0);
    if (l + 64 < D) dq1 = fmaf(dz, to_f<T>(kb[l + 64]), dq1);
    atomicAdd(&dKB[(size_t)b * D + l], dz * qs[l]);
    if (l + 64 < D) atomicAdd(&dKB[(size_t)b * D + l + 64], dz * qs[l + 64]);
  }
  float* dQ = reinterpret_cast<float*>(a.dq) + (bh * a.T + i) * D;
  dQ[l] = dq0;
  if (l + 64 < D) dQ[l + 64] = dq1;
}

// dk += dkbar / 64 on every key of the block (fp32 path)
__global__ void bwd_pool_grad_kernel(float* dk, const float* dkbar, int T_, int D, size_t n) {
  for (size_t x = (size_t)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += (size_t)gridDim.x * blockDim.x) {
    const size_t d = x % D;
    const size_t row = x / D;  // bh * T + t
    const size_t bh = row / T_;
    const size_t t = row % T_;
    const int nb = T_ / DASH_BLOCK;
    dk[x] += dkbar[(bh * nb + t / DASH_BLOCK) * D + d] * (1.f / DASH_BLOCK);
  }
}

__global__ void zero_f32_kernel(float* p, size_t n) {
  for (size_t x = (size_t)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += (size_t)gridDim.x * blockDim.x) p[x] = 0.f;
}

hipError_t launch_bwd(const BwdArgs& a, int dtype, hipStream_t st) {
  const size_t rows = (size_t)a.BH * a.T;
  const int ntile = (a.T + DASH_QTILE - 1) / DASH_QTILE;
  const int nb = a.T / DASH_BLOCK;
  hipError_t e;
  if (dtype == 1) {
    bwd_delta_kernel<bf16_t><<<(unsigned)((rows + 3) / 4), 256, 0, st>>>(
        reinterpret_cast<const bf16_t*>(a.o), reinterpret_cast<const bf16_t*>(a.dout), a.delta, rows, a.D);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.D == 128) bwd_dq_kernel<128><<<ntile * a.BH, 256, 0, st>>>(a);
    else bwd_dq_kernel<64><<<ntile * a.BH, 256, 0, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    bwd_entmax_kernel<<<dim3(ntile, a.BH), 128, 0, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.D == 128) bwd_dkdv_kernel<128><<<nb * a.BH, 256, 0, st>>>(a);
    else bwd_dkdv_kernel<64><<<nb * a.BH, 256, 0, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.D == 128) bwd_dq_final_kernel<128><<<dim3(ntile * 4, a.BH), 256, 0, st>>>(a);
    else bwd_dq_final_kernel<64><<<dim3(ntile * 4, a.BH), 256, 0, st>>>(a);
    return hipGetLastError();
  }
  const size_t n = rows * a.D;
  zero_f32_kernel<<<2048, 256, 0, st>>>(reinterpret_cast<float*>(a.dk), n);
  zero_f32_kernel<<<2048, 256, 0, st>>>(reinterpret_cast<float*>(a.dv), n);
  zero_f32_kernel<<<256, 256, 0, st>>>(a.dkbar, (size_t)a.BH * nb * a.D);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  bwd_generic_kernel<float><<<dim3(a.T, a.BH), 64, 0, st>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  bwd_pool_grad_kernel<<<2048, 256, 0, st>>>(reinterpret_cast<float*>(a.dk), a.dkbar, a.T, a.D, n);
  return hipGetLastError();
}
