// Stage 2 forward: softmax attention over the selected blocks with log p
// added to every logit of block b ("Core Mechanism" of the alanhou.org page:
// fine logits plus log of the coarse scores, softmax, weighted sum of V).
#include <type_traits>

#include "kernels.h"

#define LOG2E_F 1.4426950408889634f
#define LN2_F 0.6931471805599453f

// ---------------------------------------------------------------------------- bf16 MFMA kernel
//
// Workgroup = 4 waves = one query tile of 128 rows; wave w owns rows
// 32w..32w+31 of the tile.  The workgroup walks the tile's block list
// (ascending); per block the 64 keys and values are staged once in LDS and
// shared by the 4 waves.  Per wave and block:
//   S^T (64 keys x 32 queries) = K_b Q^T    2 x (D/16) MFMA 32x32x16
//   online softmax in log2 units, the prior log2 p_ib added per row
//   O^T (D x 32)  += V_b^T P^T              (D/32) x 4 MFMA 32x32x16
// Computing S^T (keys as MFMA rows) puts one query per lane column, so the
// row max / sum need one cross-half exchange, and the result of S^T feeds
// the B operand of the PV product directly (keys are the contraction index,
// so the order in which a lane holds them only has to match V's).
// The per-(row, block) prior is recomputed from the Stage-1 score
// arithmetic (coarse_acc_chunk) for 32 listed blocks at a time.
template <int D>
__global__ __launch_bounds__(256, 2) void fwd_mfma_kernel(FwdArgs a) {
  constexpr int KP = D + 8;   // K row pitch in LDS (bf16)
  constexpr int VP = VT_PITCH;  // V^T row pitch in LDS (bf16)
  constexpr int CH = D / 8;   // 16-byte chunks per key row
  constexpr int NKL = 64 * CH / 256;       // K uint4 per thread
  constexpr int NVP = 32 * CH / 256;       // V key pairs per thread
  __shared__ __attribute__((aligned(16))) bf16_t ks[64 * KP];
  __shared__ __attribute__((aligned(16))) bf16_t vt[D * VP];
  __shared__ __attribute__((aligned(16))) float pri[4][32 * 32];
  __shared__ int lst[DASH_MAX_NB];  // the tile's block list
  static_assert(D != 128 || D * VP >= 2 * 32 * KP, "epilogue space in vt");
  static_assert(D == 128 || 4 * 32 * 32 * 2 >= 2 * 32 * KP, "epilogue space in pri");

  const int nb = a.T / DASH_BLOCK;
  const int ntile = (a.T + DASH_QTILE - 1) / DASH_QTILE;
  const int nwg = gridDim.x;
  const int wg = blockIdx.x;
  // XCD-aware order: consecutive workgroup ids go round-robin over the 8
  // XCDs; give each XCD a contiguous range of heads so their K/V stay in
  // that XCD's L2, and start every head with its longest (last) tile.
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
  const bf16_t* KB = reinterpret_cast<const bf16_t*>(a.kbar) + bh * nb * D;
  const int* glist = a.tile_blk + (bh * ntile + tile) * nb;
  const int cnt = a.tile_cnt[bh * ntile + tile];
  const CoarseArith ca = a.ca;
  const float sl2 = a.fine_scale * LOG2E_F;
  // Stage the block list in LDS once: every later block index is an LDS
  // read instead of a dependent global load in front of each K/V fetch.
  for (int x = threadIdx.x; x < cnt; x += 256) lst[x] = glist[x];
  __syncthreads();
  const int* list = lst;

  bf16x8 qb[D / 16];
  float tau_i = 0.f, ln_i = 0.f;
  if (active) {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qb[s] = load8(Q + (size_t)i * D + 16 * s + 8 * h);
    tau_i = a.tau[bh * a.T + i];
    ln_i = a.lognorm[bh * a.T + i];
  }
  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float mrow = -INFINITY, lrow = 0.f;

  uint4 kr[NKL], vr[2 * NVP];
  auto gload = [&](int b) {
    const bf16_t* kb0 = K + (size_t)b * DASH_BLOCK * D;
    const bf16_t* vb0 = V + (size_t)b * DASH_BLOCK * D;
#pragma unroll
    for (int x = 0; x < NKL; ++x) {
      const int idx = tid + 256 * x;
      kr[x] = *reinterpret_cast<const uint4*>(kb0 + (size_t)(idx / CH) * D + (idx % CH) * 8);
    }
#pragma unroll
    for (int x = 0; x < NVP; ++x) {
      const int idx = tid + 256 * x;
      const int pr = vt_pos(idx / CH), ch = idx % CH;  // thread item = pair position idx / CH
      vr[2 * x] = *reinterpret_cast<const uint4*>(vb0 + (size_t)(2 * pr) * D + ch * 8);
      vr[2 * x + 1] = *reinterpret_cast<const uint4*>(vb0 + (size_t)(2 * pr + 1) * D + ch * 8);
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int x = 0; x < NKL; ++x) {
      const int idx = tid + 256 * x;
      *reinterpret_cast<uint4*>(&ks[(idx / CH) * KP + (idx % CH) * 8]) = kr[x];
    }
#pragma unroll
    for (int x = 0; x < NVP; ++x) {
      const int idx = tid + 256 * x;
      const int pos = idx / CH, ch = idx % CH;
      const uint32_t* v0 = reinterpret_cast<const uint32_t*>(&vr[2 * x]);
      const uint32_t* v1 = reinterpret_cast<const uint32_t*>(&vr[2 * x + 1]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // element e of key 2 pr (low half) and of key 2 pr + 1 (high half)
        const uint32_t pk = __builtin_amdgcn_perm(v1[e >> 1], v0[e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
        const int d = ch * 8 + e;
        *reinterpret_cast<uint32_t*>(&vt[d * VP + 2 * vt_slot(d, pos)]) = pk;
      }
    }
  };

  // One listed block.  OWN: the block may be this wave's own (diagonal)
  // block or lie after it; only the tile's own blocks, walked last, take
  // that path, so the off-diagonal loop carries no causal-mask code.
  auto block_step = [&](int e, auto own_tag) {
    constexpr bool OWN = decltype(own_tag)::value;
    const int b = list[e];
    __syncthreads();  // every wave is done with the previous block's LDS
    sstore();
    if ((e & 31) == 0 && active) {
      // log2 prior for this wave's 32 rows and listed blocks e .. e+31
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
    __syncthreads();  // LDS tile and priors visible
    if (e + 1 < cnt) gload(list[e + 1]);
    if (!active) return;
    bool diag = false;
    if constexpr (OWN) {
      if (b > wblk) return;  // after this wave's rows
      diag = b == wblk;
    }
    const float pr = diag ? 0.f : pri[w][(e & 31) * 32 + j];
    if (!diag && __ballot(pr != -INFINITY) == 0ull) return;

    // S^T = K_b Q^T
    f32x16 s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&ks[j * KP + 16 * s + 8 * h]);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&ks[(32 + j) * KP + 16 * s + 8 * h]);
      s0 = mfma32(a0, qb[s], s0);
      s1 = mfma32(a1, qb[s], s1);
    }
    if constexpr (OWN) {
      if (diag) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = b * DASH_BLOCK + acc_row32(r, l);
          if (key > i) s0[r] = -INFINITY;
          if (key + 32 > i) s1[r] = -INFINITY;
        }
      }
    }
    // The prior is constant over a row's keys in this block, so the block
    // max is taken on the raw scores and every weight is one FMA + exp2:
    // p = 2^(s * scale * log2e + prior2 - m).
    float mb = s0[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mb = fmaxf(mb, s0[r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mb = fmaxf(mb, s1[r]);
    mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
    const float mx = (mb == -INFINITY || pr == -INFINITY) ? -INFINITY : mb * sl2 + pr;
    // Rows keep a reference max and rescale O only when a block's max
    // exceeds it by more than 2^8, so weights stay <= 256 and most blocks
    // skip the rescale (wave-uniform branch).
    if (__builtin_expect(__ballot(mx > mrow + 8.f) != 0ull, 0)) {
      const float mnew = fmaxf(mrow, mx);
      const float resc = (mnew == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(mrow - mnew);
      mrow = mnew;
      lrow *= resc;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= resc;
    }
    const float off = (pr == -INFINITY || mrow == -INFINITY) ? -INFINITY : pr - mrow;
    float x[32];
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      x[r] = __builtin_amdgcn_exp2f(fmaf(s0[r], sl2, off));
      x[16 + r] = __builtin_amdgcn_exp2f(fmaf(s1[r], sl2, off));
      ps += x[r] + x[16 + r];
    }
    lrow += ps;
    // O^T += V_b^T P^T, 4 k-steps of 16 keys
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 pb;
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) pb[e8] = (__bf16)x[16 * (s >> 1) + 8 * (s & 1) + e8];
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const int d = 32 * dt + j;
        const bf16x8 va = load8(&vt[d * VP + 2 * vt_slot(d, 8 * s + 4 * h)]);
        oacc[dt] = mfma32(va, pb, oacc[dt]);
      }
    }
  };

  // With a causal mask the list ends with the tile's own blocks (every other
  // listed block precedes them): walk the rest first without mask code.
  const int nown = a.causal ? (min(a.T, (tile + 1) * DASH_QTILE) - tile * DASH_QTILE) / DASH_BLOCK : 0;
  const int nmain = cnt - nown;
  if (cnt > 0) gload(list[0]);
  int e = 0;
  for (; e < nmain; ++e) block_step(e, std::false_type{});
  for (; e < cnt; ++e) block_step(e, std::true_type{});

  // epilogue: O = O^T / l, staged through LDS for 16-byte row stores
  __syncthreads();
  const float ltot = lrow + __shfl_xor(lrow, 32, 64);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  // 32 rows x D per wave, row pitch KP: waves 0-1 in ks, waves 2-3 in vt
  // (D = 128) or in the prior buffer (D = 64), all free after the main loop
  bf16_t* ost = (w < 2) ? ks + w * 32 * KP
                        : (D == 128 ? vt : reinterpret_cast<bf16_t*>(&pri[0][0])) + (w - 2) * 32 * KP;
  if (active) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * dt + 8 * r4 + 4 * h;  // registers 4 r4 .. 4 r4 + 3 hold d .. d + 3
        bf16x4 o4;
#pragma unroll
        for (int x = 0; x < 4; ++x) o4[x] = (__bf16)(oacc[dt][4 * r4 + x] * inv);
        *reinterpret_cast<bf16x4*>(&ost[j * KP + d]) = o4;
      }
    if (h == 0) a.lse[bh * a.T + i] = (mrow + __builtin_amdgcn_logf(ltot)) * LN2_F;
  }
  __syncthreads();
  if (active) {
    bf16_t* O = reinterpret_cast<bf16_t*>(a.o) + bh * a.T * D;
#pragma unroll
    for (int it = 0; it < 32 * CH / 64; ++it) {
      const int idx = it * 64 + l;
      const int row = idx / CH, ch = idx % CH;
      *reinterpret_cast<uint4*>(O + (size_t)(qrow0 + row) * D + ch * 8) =
          *reinterpret_cast<const uint4*>(ost + row * KP + ch * 8);
    }
  }
}

// ---------------------------------------------------------------------------- generic kernel
//
// One wave per query row, blocks in ascending order, natural-exp online
// softmax in fp32.  Used for fp32 tensors.  The block prior comes from the
// same dot_row score as the generic Stage-1 kernel.
template <typename T>
__global__ __launch_bounds__(64) void fwd_generic_kernel(FwdArgs a) {
  __shared__ float qs[128];
  __shared__ float pv[64];
  const int D = a.D;
  const int nb = a.T / DASH_BLOCK;
  const size_t bh = blockIdx.y;
  const int i = blockIdx.x;
  const int l = lane_id();
  const T* q = reinterpret_cast<const T*>(a.q) + (bh * a.T + i) * D;
  const T* K = reinterpret_cast<const T*>(a.k) + bh * a.T * D;
  const T* V = reinterpret_cast<const T*>(a.v) + bh * a.T * D;
  const T* KB = reinterpret_cast<const T*>(a.kbar) + bh * nb * D;
  for (int d = l; d < D; d += 64) qs[d] = to_f<T>(q[d]);
  __syncthreads();
  const CoarseArith ca = a.ca;
  const float tau_i = a.tau[bh * a.T + i], ln_i = a.lognorm[bh * a.T + i];
  const int own = i / DASH_BLOCK;
  const int last = a.causal ? own : nb - 1;
  float m = -INFINITY, lsum = 0.f;
  float o0 = 0.f, o1 = 0.f;
  for (int b = 0; b <= last; ++b) {
    float pr;
    if (a.causal && b == own) pr = 0.f;
    else {
      pr = ca.logp(ca.u_of(dot_row<T>(qs, KB + (size_t)b * D, D)), tau_i, ln_i);
      if (pr == -INFINITY) continue;
    }
    const int key = b * DASH_BLOCK + l;
    float s = dot_row<T>(qs, K + (size_t)key * D, D) * a.fine_scale + pr;
    if (a.causal && key > i) s = -INFINITY;
    const float mx = wave_max(s);
    const float mn = fmaxf(m, mx);
    const float rs = expf(m - mn);
    const float p = expf(s - mn);
    lsum = lsum * rs + wave_sum(p);
    m = mn;
    pv[l] = p;
    __syncthreads();
    o0 *= rs;
    o1 *= rs;
    for (int kk = 0; kk < DASH_BLOCK; ++kk) {
      const T* vr = V + (size_t)(b * DASH_BLOCK + kk) * D;
      o0 = fmaf(pv[kk], to_f<T>(vr[l]), o0);
      if (l + 64 < D) o1 = fmaf(pv[kk], to_f<T>(vr[l + 64]), o1);
    }
    __syncthreads();
  }
  T* O = reinterpret_cast<T*>(a.o) + (bh * a.T + i) * D;
  O[l] = from_f<T>(o0 / lsum);
  if (l + 64 < D) O[l + 64] = from_f<T>(o1 / lsum);
  if (l == 0) a.lse[bh * a.T + i] = m + logf(lsum);
}

hipError_t launch_fwd(const FwdArgs& a, int dtype, hipStream_t st) {
  if (dtype == 1) {
    const int ntile = (a.T + DASH_QTILE - 1) / DASH_QTILE;
    dim3 grid(ntile * a.BH);
    if (a.D == 128) fwd_mfma_kernel<128><<<grid, 256, 0, st>>>(a);
    else fwd_mfma_kernel<64><<<grid, 256, 0, st>>>(a);
  } else {
    fwd_generic_kernel<float><<<dim3(a.T, a.BH), 64, 0, st>>>(a);
  }
  return hipGetLastError();
}
