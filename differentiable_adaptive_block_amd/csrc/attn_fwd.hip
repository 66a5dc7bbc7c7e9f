// Stage 2 forward: softmax attention over the selected blocks with log p
// added to every logit of block b ("Core Mechanism" of the alanhou.org page:
// fine logits plus log of the coarse scores, softmax, weighted sum of V).
#include "kernels.h"
#include "tiles.h"

#define LOG2E_F 1.4426950408889634f
#define LN2_F 0.6931471805599453f

// ---------------------------------------------------------------------------- bf16 MFMA kernel
//
// Workgroup = 4 waves = one query tile of 128 rows; wave w owns rows
// 32w..32w+31 of the tile (grouped-query heads: 4 x 32 / HG rows of the
// group's HG heads, see below).  The workgroup walks the tile's block list
// (ascending).  Per wave and block:
//   S^T (64 keys x 32 queries) = K_b Q^T    2 x (D/16) MFMA 32x32x16
//   online softmax in log2 units, the prior log2 p_ib added per row
//   O^T (D x 32)  += V_b^T P^T              (D/32) x 4 MFMA 32x32x16
// Computing S^T (keys as MFMA rows) puts one query per lane column, so the
// row max / sum need one cross-half exchange, and the result of S^T feeds
// the B operand of the PV product directly (keys are the contraction index,
// so the order in which a lane holds them only has to match V's).
//
// Staging: the K and V tiles of a block (64 rows of D bf16 each) are copied
// from global memory straight into LDS by the load unit (16 bytes per
// lane, 1 KB per wave instruction), double-buffered: while the waves
// compute block e from one buffer pair, the copy of block e+1 fills the
// other, and one barrier per block hands the buffers over.  The tiles keep
// K's and V's row-major layout with the 16-byte chunks of each row
// permuted (XOR with a function of the row), which makes the K operand
// reads (16 bytes per lane) and the transposing V operand reads
// (ds_read_b64_tr_b16, 8 bytes per lane) free of bank conflicts.
//
// The per-(row, block) prior is recomputed from the Stage-1 score
// arithmetic (coarse_acc_chunk) for 32 listed blocks at a time and kept in
// registers.
//
// Grouped-query heads (HG = a.grp > 1 query heads per key/value head): a
// wave's 32 query columns are the HG heads of the group at 32 / HG
// consecutive rows (column j: head j / (32 / HG), row j % (32 / HG)), so
// the group's heads share every K/V tile copy and operand read.  Keys,
// values and summaries are the KV head's; the prior is the group's
// aggregated one, log pbar with pbar the mean of the heads' p: each column
// computes its own head's p from one score MFMA chain (the Stage-1
// arithmetic) and the columns of a row add theirs across lanes
// (prior_chunk32_heads).
// One query tile (row group `logical` in the launch's order) of the walk;
// the body of fwd_mfma_kernel and fwd_mfma_list_kernel.
template <int D, int HG>
__device__ __forceinline__ void fwd_mfma_tile(const FwdArgs& a, const int logical) {
  constexpr int CH = D / 8;          // 16-byte chunks per row
  constexpr int KS = D / 16;         // k-steps of the S product
  constexpr int NDT = D / 32;        // 32-row d tiles of O^T
  constexpr int RPW = 32 / HG;       // rows per wave
  constexpr int RPG = 4 * RPW;       // rows per workgroup
  // one object per buffer, so that reads of one buffer are not ordered
  // behind the copy into the other
  __shared__ __attribute__((aligned(16))) bf16_t kt0[64 * D];
  __shared__ __attribute__((aligned(16))) bf16_t kt1[64 * D];
  __shared__ __attribute__((aligned(16))) bf16_t vt0[64 * D];
  __shared__ __attribute__((aligned(16))) bf16_t vt1[64 * D];
  __shared__ int lst[DASH_MAX_NB];  // the tile's block list
  static_assert(32 * (D + 8) <= 64 * D, "epilogue staging space");

  const int nb = a.T / DASH_BLOCK;
  const int ntile = (a.T + DASH_QTILE - 1) / DASH_QTILE;
  const int nrg = (a.T + RPG - 1) / RPG;  // row groups per head group
  const size_t bkv = logical / nrg;  // the key/value head (the query head when HG = 1)
  const int rg = nrg - 1 - (logical % nrg);

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, j = l & 31, h = l >> 5;
  const int qrow0 = rg * RPG + w * RPW;  // the wave's first row (all its rows lie in one block)
  const bool active = qrow0 < a.T;
  const int wblk = qrow0 / DASH_BLOCK;
  const int i = qrow0 + j % RPW;                    // this column's row
  const size_t bh = bkv * HG + j / RPW;             // and query head
  const int tile = (rg * RPG) / DASH_QTILE;         // the tile whose block list the group walks

  const bf16_t* Q = reinterpret_cast<const bf16_t*>(a.q) + bh * a.Tr * D;
  const bf16_t* K = reinterpret_cast<const bf16_t*>(a.k) + bkv * a.Tr * D;
  const bf16_t* V = reinterpret_cast<const bf16_t*>(a.v) + bkv * a.Tr * D;
  const bf16_t* KB = reinterpret_cast<const bf16_t*>(a.kbar) + bkv * nb * D;
  // a partial last block (a.Tr < a.T): its rows past the tensor are zero in
  // the LDS tiles, zero queries, and never written out
  const int part_blk = a.Tr < a.T ? nb - 1 : -1;
  const int part_rows = a.Tr - (nb - 1) * DASH_BLOCK;
  // the heads of a group share their tile lists (the union of their supports)
  const int* glist = a.tile_blk + (bkv * HG * ntile + tile) * nb;
  const int cnt = a.tile_cnt[bkv * HG * ntile + tile];
  const CoarseArith ca = a.ca;
  const float sl2 = a.fine_scale * LOG2E_F;
  // The block list is staged in LDS: a global (vector-memory) load inside
  // the loop would wait for the tile copies in flight, which retire on the
  // same counter.
  for (int x = tid; x < cnt; x += 256) lst[x] = glist[x];
  __syncthreads();
  const int* list = lst;

  bf16x8 qb[KS];
  float tau_i = 0.f, ln_i = 0.f;
  if (active) {
#pragma unroll
    for (int s = 0; s < KS; ++s) qb[s] = i < a.Tr ? load8(Q + (size_t)i * D + 16 * s + 8 * h) : bf16x8{};
    tau_i = a.tau[bh * a.T + i];
    ln_i = a.lognorm[bh * a.T + i];
  }
  f32x16 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float mrow = -INFINITY, lrow = 0.f;

  // copy block b's K and V tiles into LDS: this wave fills a quarter of
  // the rows of each, chunk slot s of row r from source chunk s ^ swz(r)
  const int wu = __builtin_amdgcn_readfirstlane(w);
  TileCopy<D, TileSwz<D>::k> kcp;
  TileCopy<D, TileSwz<D>::v> vcp;
  kcp.init(wu, l);
  vcp.init(wu, l);
  auto copy_block = [&](int b, bf16_t* kd, bf16_t* vd) {
    const int bu = __builtin_amdgcn_readfirstlane(b);
    const size_t o = (size_t)bu * DASH_BLOCK * D;
    const int rows = bu == part_blk ? part_rows : DASH_BLOCK;
    kcp.copy(K + o, kd, wu, rows);
    vcp.copy(V + o, vd, wu, rows);
  };
  // After the copy of a partial block has landed (and a barrier): its rows
  // past the tensor are set to zero (the descriptor kept the copy from
  // reading them); the caller's next barrier publishes the zeros.
  auto zero_tail = [&](bf16_t* kd, bf16_t* vd) {
    for (int x = tid; x < (DASH_BLOCK - part_rows) * CH; x += 256) {
      *reinterpret_cast<uint4*>(kd + part_rows * D + 8 * x) = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(vd + part_rows * D + 8 * x) = make_uint4(0, 0, 0, 0);
    }
  };

  f32x16 pacc;
  auto prior_chunk = [&](int e0) {
    if (!active) return;
    if constexpr (HG > 1) pacc = prior_chunk32_heads<D, HG>(KB, list, cnt, e0, qb, ca, tau_i, ln_i, a.causal, wblk);
    else pacc = prior_chunk32<D>(KB, list, cnt, e0, qb, ca, tau_i, ln_i, a.causal, wblk);
  };
  auto prior_of = [&](int e) -> float { return prior_pick(pacc, e); };

  auto block_step = [&](int e, const bf16_t* kt, const bf16_t* vt) {
    const int b = list[e];
    const bool diag = a.causal && b == wblk;
    if (a.causal && b > wblk) return;  // after this wave's rows
    const float pr = diag ? 0.f : prior_of(e);
    if (!diag && __ballot(pr != -INFINITY) == 0ull) return;

    // S^T = K_b Q^T
    f32x16 s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int c = 2 * s + h;
      const bf16x8 a0 = load8(kt + j * D + 8 * (c ^ TileSwz<D>::k(j)));
      const bf16x8 a1 = load8(kt + (32 + j) * D + 8 * (c ^ TileSwz<D>::k(32 + j)));
      s0 = mfma32(a0, qb[s], s0);
      s1 = mfma32(a1, qb[s], s1);
    }
    // issue order: operand reads run 4 ahead of the MFMAs that use them
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int s = 0; s < 2 * KS; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if (diag) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = b * DASH_BLOCK + acc_row32(r, l);
        if (key > i) s0[r] = -INFINITY;
        if (key + 32 > i) s1[r] = -INFINITY;
      }
    }
    // The prior is constant over a row's keys in this block, so the block
    // max is taken on the raw scores and every weight is one FMA + exp2:
    // p = 2^(s * scale * log2e + prior2 - m).
    float mb = fmaxf(s0[0], s0[1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mb = fmaxf(mb, s0[r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mb = fmaxf(mb, s1[r]);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mb), __float_as_uint(mb), false, false);
      mb = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
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
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= resc;
    }
    const float off = (pr == -INFINITY || mrow == -INFINITY) ? -INFINITY : pr - mrow;
    // O^T += V_b^T P^T, 4 k-steps of 16 keys.  At k-step s a lane of half h
    // needs keys 16s+4h+{0..3} and 16s+8+4h+{0..3} of its column d; its
    // weights are registers 8(s%2)..8(s%2)+7 of s0 (s < 2) or s1.  Each
    // transposing read hands lane 4a+b of a 16-lane group element b of the
    // 8-byte pieces addressed by lanes a, a+4, a+8, a+12 of the group, so
    // lane t of the group addresses row key0 + t/4, columns
    // 32 dt + 16 (group % 2) + 4 (t % 4) .. +3.
    const int tg = l & 15, grp = l >> 4;
    const int dof = 16 * (grp & 1) + 4 * (tg & 3);  // column offset within a 32-wide d tile
    // the row sum adds the weights as rounded for the MFMA, two per
    // instruction (bf16 pair dot (1, 1))
    float ps0 = 0.f, ps1 = 0.f;
    bf16x2 one2;
    one2[0] = (__bf16)1.f;
    one2[1] = (__bf16)1.f;
    // V operand of k-step s, d tile dt
    auto vread = [&](int s, int dt) -> bf16x8 {
      const int r1 = 16 * s + 4 * h + (tg >> 2), r2 = r1 + 8;
      const int col = 32 * dt + dof;
      const int c = col >> 3, half = (col >> 2) & 1;
      const bf16x4 lo = ds_read_tr4(vt + r1 * D + 8 * (c ^ TileSwz<D>::v(r1)) + 4 * half);
      const bf16x4 hi = ds_read_tr4(vt + r2 * D + 8 * (c ^ TileSwz<D>::v(r2)) + 4 * half);
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    // operands are read one k-step ahead of the MFMAs that use them, in
    // source order, so each read has NDT MFMAs to land
    bf16x8 vnext[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) vnext[dt] = vread(0, dt);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 pb;
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        const float sv = (s < 2) ? s0[8 * (s & 1) + e8] : s1[8 * (s & 1) + e8];
        pb[e8] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sv, sl2, off));
      }
      ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 0, 1), one2, ps0, false);
      ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 2, 3), one2, ps1, false);
      ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 4, 5), one2, ps0, false);
      ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 6, 7), one2, ps1, false);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const bf16x8 va = vnext[dt];
        if (s + 1 < 4) vnext[dt] = vread(s + 1, dt);
        oacc[dt] = mfma32(va, pb, oacc[dt]);
      }
    }
    lrow += ps0 + ps1;
  };

  if (cnt > 0) {
    copy_block(list[0], kt0, vt0);
    int e = 0;
    for (; e < cnt; e += 2) {
      if ((e & 31) == 0) prior_chunk(e);
      tile_copies_done();
      __syncthreads();  // block e in buffers 0; everyone is done with buffers 1
      if (list[e] == part_blk) {  // the partial last block: the last entry of the list
        zero_tail(kt0, vt0);
        __syncthreads();
      }
      if (e + 1 < cnt) copy_block(list[e + 1], kt1, vt1);
      if (active) block_step(e, kt0, vt0);
      if (e + 1 >= cnt) break;
      tile_copies_done();
      __syncthreads();  // block e+1 in buffers 1; everyone is done with buffers 0
      if (list[e + 1] == part_blk) {
        zero_tail(kt1, vt1);
        __syncthreads();
      }
      if (e + 2 < cnt) copy_block(list[e + 2], kt0, vt0);
      if (active) block_step(e + 1, kt1, vt1);
    }
  }

  // epilogue: O = O^T / l, staged through LDS (32 rows x D per wave, row
  // pitch D + 8, one tile buffer per wave) for 16-byte row stores
  __syncthreads();
  constexpr int OP = D + 8;
  const float ltot = lrow + __shfl_xor(lrow, 32, 64);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  bf16_t* ost = w == 0 ? kt0 : w == 1 ? kt1 : w == 2 ? vt0 : vt1;
  if (active) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * dt + 8 * r4 + 4 * h;  // registers 4 r4 .. 4 r4 + 3 hold d .. d + 3
        bf16x4 o4;
#pragma unroll
        for (int x = 0; x < 4; ++x) o4[x] = (__bf16)(oacc[dt][4 * r4 + x] * inv);
        *reinterpret_cast<bf16x4*>(&ost[j * OP + d]) = o4;
      }
    if (h == 0 && i < a.Tr) a.lse[bh * a.Tr + i] = (mrow + __builtin_amdgcn_logf(ltot)) * LN2_F;
  }
  __syncthreads();
  if (active) {
#pragma unroll
    for (int it = 0; it < 32 * CH / 64; ++it) {
      const int idx = it * 64 + l;
      const int col = idx / CH, ch = idx % CH;  // staged column: head col / RPW, row col % RPW
      const int row = qrow0 + col % RPW;
      bf16_t* O = reinterpret_cast<bf16_t*>(a.o) + ((bkv * HG + col / RPW) * a.Tr + row) * D;
      if (row < a.Tr) *reinterpret_cast<uint4*>(O + ch * 8) = *reinterpret_cast<const uint4*>(ost + col * OP + ch * 8);
    }
  }
}

template <int D, int HG>
__global__ __launch_bounds__(256, 2) void fwd_mfma_kernel(FwdArgs a) {
  // XCD-aware order: consecutive workgroup ids go round-robin over the 8
  // XCDs; give each XCD a contiguous range of heads so their K/V stay in
  // that XCD's L2, and start every head with its longest (last) rows.
  const int nwg = gridDim.x;
  const int wg = blockIdx.x;
  fwd_mfma_tile<D, HG>(a, (nwg % 8 == 0) ? (wg % 8) * (nwg / 8) + wg / 8 : wg);
}

// The same walk over a device-side list of row groups (the tiles a
// low-density call leaves to the dense walk): persistent workgroups take
// list entries g, g + grid, ...; a call whose tiles all take the other
// schedule launches only these few workgroups.
template <int D, int HG>
__global__ __launch_bounds__(256, 2) void fwd_mfma_list_kernel(FwdArgs a) {
  const int n = a.dense_n[0];
  for (int k = blockIdx.x; k < n; k += gridDim.x) {
    fwd_mfma_tile<D, HG>(a, a.dense_list[k]);
    __syncthreads();  // the tile's LDS is reused by the next
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
  if (i >= a.Tr) return;  // a row past the tensor (partial last block): nothing to write
  const int l = lane_id();
  const T* q = reinterpret_cast<const T*>(a.q) + (bh * a.Tr + i) * D;
  const T* K = reinterpret_cast<const T*>(a.k) + bh * a.Tr * D;
  const T* V = reinterpret_cast<const T*>(a.v) + bh * a.Tr * D;
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
    // keys after the row (causal) include every key past the tensor
    float s = (a.causal && key > i) ? -INFINITY : dot_row<T>(qs, K + (size_t)key * D, D) * a.fine_scale + pr;
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
    const int nk = min(DASH_BLOCK, a.Tr - b * DASH_BLOCK);  // keys of the block in the tensor
    for (int kk = 0; kk < nk; ++kk) {
      const T* vr = V + (size_t)(b * DASH_BLOCK + kk) * D;
      o0 = fmaf(pv[kk], to_f<T>(vr[l]), o0);
      if (l + 64 < D) o1 = fmaf(pv[kk], to_f<T>(vr[l + 64]), o1);
    }
    __syncthreads();
  }
  T* O = reinterpret_cast<T*>(a.o) + (bh * a.Tr + i) * D;
  O[l] = from_f<T>(o0 / lsum);
  if (l + 64 < D) O[l + 64] = from_f<T>(o1 / lsum);
  if (l == 0) a.lse[bh * a.Tr + i] = m + logf(lsum);
}

template <int HG>
static void launch_fwd_hg(const FwdArgs& a, hipStream_t st) {
  const int rpg = 4 * (32 / HG);
  if (a.dense_list != nullptr) {
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    const dim3 grid(2 * ncu);  // two workgroups per CU are resident
    if (a.D == 128) fwd_mfma_list_kernel<128, HG><<<grid, 256, 0, st>>>(a);
    else fwd_mfma_list_kernel<64, HG><<<grid, 256, 0, st>>>(a);
    return;
  }
  const dim3 grid(((a.T + rpg - 1) / rpg) * (a.BH / HG));
  if (a.D == 128) fwd_mfma_kernel<128, HG><<<grid, 256, 0, st>>>(a);
  else fwd_mfma_kernel<64, HG><<<grid, 256, 0, st>>>(a);
}

hipError_t launch_fwd(const FwdArgs& a, int dtype, hipStream_t st) {
  if (dtype == 1) {
    if (a.BH % a.grp) return hipErrorInvalidValue;
    switch (a.grp) {
      case 1: launch_fwd_hg<1>(a, st); break;
      case 2: launch_fwd_hg<2>(a, st); break;
      case 4: launch_fwd_hg<4>(a, st); break;
      case 8: launch_fwd_hg<8>(a, st); break;
      default: return hipErrorNotSupported;
    }
  } else {
    if (a.grp > 1) return hipErrorNotSupported;
    fwd_generic_kernel<float><<<dim3(a.T, a.BH), 64, 0, st>>>(a);
  }
  return hipGetLastError();
}
