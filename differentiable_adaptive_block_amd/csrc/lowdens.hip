// Stage 2 forward at low selection density: a block-stationary schedule.
//
// The attention of Stage 2 ("Core Mechanism" of the alanhou.org page: fine
// logits plus log p of the block, one softmax over the selected blocks,
// weights on V) is a sum over (query row, selected block) pairs.  The dense
// walk (attn_fwd.hip) visits, for each 128-row query tile, the union of its
// rows' blocks with all 128 rows as MFMA columns; when the rows of a tile
// select few and different blocks (the pages' sparsity-aware implementation
// "skips zero blocks": AdaSplash-2 abstract on the thelatestinai.com page),
// that union is close to every candidate and most of the walked products
// belong to rows that did not select the block.
//
// This schedule turns the walk around.  For each key block b it lists the
// rows that selected it (a column of the Stage-1 masks, plus the block's
// own 64 rows under the causal mask) and runs those rows, 32 per wave, as
// the MFMA columns of S^T = K_b Q^T and O^T = V_b^T P^T, with K_b and V_b
// copied into LDS once per 128 listed rows.  Each (row, block) pair leaves
// a partial softmax: m = the block's max logit in log2 units with the
// prior log2 p_b added, l = the sum of the block's weights 2^(s - m_blk),
// and o = the unnormalised weighted sum of V (bf16).  A per-row merge then
// combines a row's partials in block order:
//   M = max_s m_s, L = sum_s 2^(m_s - M) l_s, O = sum_s 2^(m_s - M) o_s / L,
//   lse = (M + log2 L) ln 2.
// Every partial is computed the same way wherever its row sits among the
// MFMA columns, and the merge adds in a fixed order, so the results do not
// depend on scheduling.
//
// Which tiles take it: a tile whose dense walk would visit more than
// `ratio` times the pairs its rows need, as long as the pairs of all such
// tiles so far (in head-major tile order) fit in the caller's workspace;
// every other tile keeps the dense walk, which the same call runs over a
// device-side list of those tiles (fwd_mfma_list_kernel).  The lists are
// built from the masks without atomics (see the plan kernels), so they,
// too, are the same on every run.
#include "kernels.h"
#include "tiles.h"

#define LOG2E_F 1.4426950408889634f
#define LN2_F 0.6931471805599453f

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kItemRows = 128;  // listed rows per work item (4 waves x 32 columns)

// Candidate mask words of a row in block rb (causal: blocks 0 .. rb-1), and
// the bits of the last of them that are candidates.
__device__ __forceinline__ int cand_words(int rb) { return (rb + 31) >> 5; }
__device__ __forceinline__ uint32_t cand_bits(int rb, int w) {
  const int left = rb - 32 * w;
  return left >= 32 ? 0xFFFFFFFFu : ((1u << left) - 1u);
}

// ---------------------------------------------------------------------------- plan
// Work items are cut per (head, row range of DASH_LD_RANGE groups = 8192
// rows, column): a column's entries are in row order, so the entries of one
// range are a contiguous run of it, and consecutive items gather their
// query rows from one 2 MB slice of a head's queries rather than from the
// whole head (measured a little faster than items in plain column order;
// narrower ranges re-read each block's keys and values more often).
//
// The lists are built without atomics, from per-(row group, block) counts:
// row group g is the 64 rows of block g (the own block of all of them).
//   count:     grp[g][b] = rows of group g that selected candidate b (b < g),
//              grp[g][g] = 64 (the own block); gpairs[g] = the group's pairs;
//   tiles:     which tiles take the schedule, their first pair (one workgroup);
//   columns:   grp[g][b] becomes the exclusive prefix over the taken groups
//              g' < g of column b, col_cnt[b] the column's length;
//   bases:     column bases (exclusive scan of col_cnt);
//   items:     work items per head, then after the items of the heads before;
//   fill:      entry of (row, b) at base[b] + grp[g][b] + the row's rank
//              among the group's rows that selected b; each row's first pair
//              and count.
// The partials are laid out by (row group, block, rank): group g's pairs
// from the group's first pair on, block by block (the own block last),
// within a block its selecting rows in row order.  An item (one column)
// then writes runs of consecutive partials, one per group, and the merge
// reads each group's partials from one contiguous range; row_pos lists,
// row by row, where each of a row's pairs went.
// Every position is a function of the masks alone, so the lists (and
// everything after them) are the same on every run.

// One wave per row group (bh, g).
__global__ __launch_bounds__(256) void ld_count_kernel(LdArgs a) {
  const int nb = a.T / DASH_BLOCK, nbw = (nb + 31) / 32;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gw >= a.BH * nb) return;
  const int l = threadIdx.x & 63;
  const size_t bh = gw / nb;
  const int g = gw % nb;
  const uint32_t* mw = a.mask + (bh * a.T + (size_t)g * DASH_BLOCK + l) * nbw;
  int* grp = a.grp_cnt + ((size_t)bh * nb + g) * nb;
  int sel = 0;
  const int ncw = cand_words(g);
  for (int w0 = 0; w0 < ncw; w0 += 4) {
    uint32_t wd[4];  // four words loaded together: one memory wait per four
#pragma unroll
    for (int j = 0; j < 4; ++j) wd[j] = w0 + j < ncw ? mw[w0 + j] & cand_bits(g, w0 + j) : 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int w = w0 + j;
      if (w >= ncw) break;  // the same on every lane
      const uint32_t word = wd[j];
      sel += __popc(word);
      int cnt = 0;  // lane b < 32: rows that selected block 32 w + b
#pragma unroll
      for (int bit = 0; bit < 32; ++bit) {
        const int c = __popcll(__ballot((word >> bit) & 1u));
        if (l == bit) cnt = c;
      }
      if (l < 32 && 32 * w + l < g) grp[32 * w + l] = cnt;
    }
  }
  if (l == 0) grp[g] = DASH_BLOCK;
  const int pairs = (int)wave_sum((float)(sel + 1));  // <= 64 * 1537: exact in fp32
  if (l == 0) a.gpairs[bh * nb + g] = pairs;
}

// Exclusive scan of n ints in order by one 1024-thread workgroup: value i
// is load(i); calls emit(i, value, exclusive prefix (64-bit)) for every i.
// Each pass covers 4096 values, 4 consecutive ones per thread; the prefix
// of the passes so far is carried in LDS.
template <typename LD, typename F>
__device__ __forceinline__ void block_scan(int n, LD load, F emit) {
  constexpr int PER = 4;
  __shared__ long long wsum[16];
  __shared__ long long carry;
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < n; base += 1024 * PER) {
    const int i0 = base + PER * tid;
    int v[PER];
    int tsum = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      v[e] = i0 + e < n ? load(i0 + e) : 0;
      tsum += v[e];
    }
    int x = tsum;  // inclusive scan of the thread sums in the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (l >= o) x += y;
    }
    if (l == 63) wsum[w] = x;
    __syncthreads();
    long long before = carry;
    for (int k = 0; k < w; ++k) before += wsum[k];
    long long run = before + x - tsum;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      if (i0 + e < n) emit(i0 + e, v[e], run);
      run += v[e];
    }
    __syncthreads();
    if (tid == 1023) carry = before + x;
    __syncthreads();
  }
}

// Tiles: a tile qualifies when its dense walk (list length x rows) exceeds
// ratio x its pairs; a qualifying tile is taken while the inclusive prefix
// of the qualifying tiles' pairs fits in the workspace (so the taken tiles
// are a prefix of the qualifying ones in head-major tile order).
__global__ __launch_bounds__(1024) void ld_scan_tiles_kernel(LdArgs a) {
  const int nb = a.T / DASH_BLOCK;
  const int ntile = (a.T + DASH_QTILE - 1) / DASH_QTILE;
  const int n = a.BH * ntile;
  auto pairs_of = [&](int i) {
    const int bh = i / ntile, t = i % ntile;
    const int g0 = 2 * t;
    const int p = a.gpairs[bh * nb + g0] + (g0 + 1 < nb ? a.gpairs[bh * nb + g0 + 1] : 0);
    const int rows = min(DASH_QTILE, a.T - t * DASH_QTILE);
    const float walked = (float)a.tile_cnt[i] * (float)rows;
    return walked > a.ratio * (float)p ? p : 0;
  };
  block_scan(n, pairs_of, [&](int i, int v, long long excl) {
    a.tile_off[i] = (v > 0 && excl + v <= a.cap) ? (int)excl : -1;
  });
  __syncthreads();
  // the tiles left to the dense walk, as its row-group numbers (one KV head
  // per query head: row group L is tile ntile - 1 - L % ntile of head
  // L / ntile), in increasing order (each head's longest rows first)
  auto dense_at = [&](int L) { return a.tile_off[(L / ntile) * ntile + (ntile - 1 - L % ntile)] < 0 ? 1 : 0; };
  block_scan(n, dense_at, [&](int L, int v, long long excl) {
    if (v) a.dense_list[excl] = L;
    if (L == n - 1) a.dense_n[0] = (int)(excl + v);
  });
}

__device__ __forceinline__ bool group_taken(const LdArgs& a, size_t bh, int g) {
  const int ntile = (a.T + DASH_QTILE - 1) / DASH_QTILE;
  return a.tile_off[bh * ntile + g * DASH_BLOCK / DASH_QTILE] >= 0;
}

// Columns: one workgroup of 16 waves per (bh, 64 consecutive blocks); lane =
// column, wave k = a range of row groups.  Each wave sums its range, the 16
// range totals are scanned in LDS, then each wave rewrites its range as
// prefixes.  Groups of tiles left to the dense walk count 0.
__global__ __launch_bounds__(1024) void ld_colscan_kernel(LdArgs a) {
  const int nb = a.T / DASH_BLOCK;
  const int nchunk = (nb + 63) / 64;
  const size_t bh = blockIdx.x / nchunk;
  const int b = (blockIdx.x % nchunk) * 64 + (threadIdx.x & 63);
  const int k = threadIdx.x >> 6;
  const int per = (nb + 15) / 16;
  const int g0 = max(k * per, b), g1 = min(nb, (k + 1) * per);  // column b: groups b .. nb-1
  int* grp = a.grp_cnt + (size_t)bh * nb * nb;
  __shared__ int tot[16][64];
  int s = 0;
  if (b < nb)
    for (int g = g0; g < g1; ++g)
      if (group_taken(a, bh, g)) s += grp[(size_t)g * nb + b];
  tot[k][threadIdx.x & 63] = s;
  __syncthreads();
  int before = 0, all = 0;
  for (int x = 0; x < 16; ++x) {
    const int v = tot[x][threadIdx.x & 63];
    if (x < k) before += v;
    all += v;
  }
  if (b < nb) {
    const int nr = (nb + DASH_LD_RANGE - 1) / DASH_LD_RANGE;
    int* rp = a.rng_pref + (size_t)bh * (nr + 1) * nb + b;
    for (int g = g0; g < g1; ++g) {
      if (g % DASH_LD_RANGE == 0) rp[(size_t)(g / DASH_LD_RANGE) * nb] = before;  // rows before the range
      if (group_taken(a, bh, g)) {
        int* c = grp + (size_t)g * nb + b;
        const int v = *c;
        *c = before;
        before += v;
      }
    }
    if (k == 0) {
      // boundaries at or before the column's first group hold none of it
      for (int r = 0; r * DASH_LD_RANGE <= b; ++r) rp[(size_t)r * nb] = 0;
      a.col_cnt[bh * nb + b] = all;
      rp[(size_t)nr * nb] = all;
    }
  }
}

// Column bases: exclusive scan of the column counts (one workgroup).
__global__ __launch_bounds__(1024) void ld_scan_cols_kernel(LdArgs a) {
  block_scan(a.BH * (a.T / DASH_BLOCK), [&](int i) { return a.col_cnt[i]; },
             [&](int i, int v, long long excl) { a.col_base[i] = (int)excl; });
}

// Work items, one workgroup per head: the entries of column b from row
// range r (n of them) give ceil(n / 128) items {column, first entry,
// entries}, in (head, range, column) order.  With EMIT false the kernel
// only counts the head's items; with EMIT true it writes them after the
// items of the heads before it.
template <bool EMIT>
__global__ __launch_bounds__(1024) void ld_items_kernel(LdArgs a) {
  const int nb = a.T / DASH_BLOCK;
  const int nr = (nb + DASH_LD_RANGE - 1) / DASH_LD_RANGE;
  const size_t bh = blockIdx.x;
  // run i = (r, b) of this head: entries rng_pref[r + 1][b] - rng_pref[r][b]
  auto run = [&](int i, int& first) {
    const int b = i % nb, r = i / nb;
    const int* rp = a.rng_pref + (bh * (nr + 1) + r) * nb + b;
    first = a.col_base[bh * nb + b] + rp[0];
    return rp[nb] - rp[0];
  };
  const int nrun = nr * nb;
  auto items_of = [&](int i) { int f; return (run(i, f) + kItemRows - 1) / kItemRows; };
  if constexpr (!EMIT) {
    __shared__ int total;
    block_scan(nrun, items_of, [&](int i, int v, long long excl) {
      if (i == nrun - 1) total = (int)(excl + v);
    });
    __syncthreads();
    if (threadIdx.x == 0) a.head_items[bh] = total;
  } else {
    long long hb = 0;  // the items of the heads before this one
    for (size_t x = 0; x < bh; ++x) hb += a.head_items[x];
    block_scan(nrun, items_of, [&](int i, int v, long long excl) {
      int first;
      const int cnt = run(i, first);
      const int col = (int)(bh * nb) + i % nb;
      for (int k = 0; k < v; ++k)
        a.items[hb + excl + k] = make_int4(col, first + k * kItemRows, min(kItemRows, cnt - k * kItemRows), 0);
      if (bh == (size_t)a.BH - 1 && i == nrun - 1) a.n_items[0] = (int)(hb + excl + v);
    });
  }
}

// Fill: one wave (one 64-thread workgroup) per row group of a taken tile.
// Entry = (row, partial index); row_pos[first pair of the row + slot] =
// partial index, slot = the block's rank among the row's pairs (ascending
// blocks, the own block last); row_info = (first pair, pairs) per row.
// A row's partial indices are gathered in LDS, 64 at a time, and written
// out row by row as contiguous runs.
__global__ __launch_bounds__(64) void ld_fill_kernel(LdArgs a) {
  constexpr int kBuf = 64;  // buffered slots per row
  __shared__ int rbuf[64][kBuf];
  const int nb = a.T / DASH_BLOCK, nbw = (nb + 31) / 32;
  const int ntile = (a.T + DASH_QTILE - 1) / DASH_QTILE;
  const int gw = blockIdx.x;
  if (gw >= a.BH * nb) return;
  const int l = threadIdx.x & 63;
  const size_t bh = gw / nb;
  const int g = gw % nb;
  const int t = g * DASH_BLOCK / DASH_QTILE;
  const int toff = a.tile_off[bh * ntile + t];
  if (toff < 0) return;  // the tile takes the dense walk
  const int r = g * DASH_BLOCK + l;
  const uint32_t* mw = a.mask + (bh * a.T + r) * nbw;
  const int* grp = a.grp_cnt + ((size_t)bh * nb + g) * nb;
  const int* cbase = a.col_base + bh * nb;
  const unsigned long long below = (1ull << l) - 1ull;
  // the group's first pair, then each row's (the rows in order)
  const int gfirst = toff + ((g & 1) ? a.gpairs[bh * nb + g - 1] : 0);
  int cnt = 1;
  for (int w0 = 0; w0 < cand_words(g); w0 += 4) {  // four words loaded together
    uint32_t wd[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) wd[j] = w0 + j < cand_words(g) ? mw[w0 + j] & cand_bits(g, w0 + j) : 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) cnt += __popc(wd[j]);
  }
  int x = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (l >= o) x += y;
  }
  const int rfirst = gfirst + x - cnt;
  a.row_info[bh * a.T + r] = make_int2(rfirst, cnt);
  int slot = 0, flushed = 0;
  // write every row's buffered indices: row i's run by the whole wave
  auto flush = [&]() {
    __builtin_amdgcn_wave_barrier();
    for (int i = 0; i < 64; ++i) {
      const int n = __shfl(slot - flushed, i, 64);
      const int dst = __shfl(rfirst + flushed, i, 64);
      if (l < n) a.row_pos[dst + l] = rbuf[i][l];
    }
    __builtin_amdgcn_wave_barrier();
    flushed = slot;
  };
  int goff = gfirst;  // the group's first partial of the next word's blocks
  // per word: block 32 w + b's ballot over the group's rows, its first
  // column entry and its first partial, for lane b < 32 and, through LDS,
  // for the rows' own loops over their selected blocks
  __shared__ unsigned long long sbal[32];
  __shared__ int sbase[32], sgof[32];
  const int ncw = cand_words(g);
  // word w + 1's mask word and (lane b < 32) its block's column base are
  // loaded while word w is handled
  uint32_t word_nx = ncw > 0 ? mw[0] & cand_bits(g, 0) : 0u;
  int base_nx = l < 32 && l < g ? cbase[l] + grp[l] : 0;
  for (int w = 0; w < ncw; ++w) {
    const uint32_t word = word_nx;
    const int base = base_nx;
    if (w + 1 < ncw) {
      word_nx = mw[w + 1] & cand_bits(g, w + 1);
      const int bn = 32 * (w + 1) + l;
      base_nx = l < 32 && bn < g ? cbase[bn] + grp[bn] : 0;
    }
    unsigned long long mybal = 0ull;
#pragma unroll
    for (int bit = 0; bit < 32; ++bit) {
      const unsigned long long bal = __ballot((word >> bit) & 1u);
      if (l == bit) mybal = bal;
    }
    const int cntb = l < 32 ? __popcll(mybal) : 0;
    int xs = cntb;  // inclusive scan of the blocks' counts
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
      const int y = __shfl_up(xs, o, 64);
      if (l >= o) xs += y;
    }
    if (__ballot(slot - flushed + __popc(word) > kBuf) != 0ull) flush();
    __builtin_amdgcn_wave_barrier();
    if (l < 32) {
      sbal[l] = mybal;
      sbase[l] = base;
      sgof[l] = goff + xs - cntb;
    }
    __builtin_amdgcn_wave_barrier();
    // this row's selected blocks of the word, in order
    for (uint32_t rem = word; rem; rem &= rem - 1u) {
      const int bit = __builtin_ctz(rem);
      const int rank = __popcll(sbal[bit] & below);
      a.col_ent[sbase[bit] + rank] = make_int2(r, sgof[bit] + rank);
      rbuf[l][slot - flushed] = sgof[bit] + rank;
      ++slot;
    }
    goff += __shfl(xs, 31, 64);
    __builtin_amdgcn_wave_barrier();
  }
  a.col_ent[cbase[g] + grp[g] + l] = make_int2(r, goff + l);
  if (__ballot(slot - flushed == kBuf) != 0ull) flush();
  rbuf[l][slot - flushed] = goff + l;
  ++slot;
  flush();
}

// A barrier for LDS hand-overs: this wave's LDS reads and writes are
// complete (lgkmcnt 0), then s_barrier.  Unlike __syncthreads(), whose
// workgroup release also waits for every global load and store in flight,
// it leaves the vector-memory counter alone; the empty asm statements keep
// the compiler from moving memory accesses across it.  (The s_waitcnt
// immediate is the gfx9 encoding with lgkmcnt 0, vmcnt 63 and expcnt 7.)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------- partials
// Persistent: workgroup g takes items g, g + grid, ... (XCD-aware: each XCD
// a contiguous run of items per round).  Its partials go out with streaming
// (nontemporal) stores: they are read once, by the merge.  Wave w takes the item's entries
// 32w .. 32w+31 as MFMA columns.  Software-pipelined over items: while
// item i is computed from one LDS buffer pair, item i+1's K and V tiles are
// copied into the other (with the block's summary row, the prior's
// operand) and its query rows, prior inputs and destinations are loaded,
// item i+2's column entries and item i+3's descriptor arrive.
// The one wait for all of them comes after item i's output is staged in LDS
// and before its global stores are issued, so no wait ever covers the
// stores of the item just finished (the vector-memory counter counts
// stores too, in order).
template <int D>
__global__ __launch_bounds__(256, 2) void ld_part_kernel(LdArgs a) {
  constexpr int CH = D / 8, KS = D / 16, NDT = D / 32;
  __shared__ __attribute__((aligned(16))) bf16_t kt0[64 * D];
  __shared__ __attribute__((aligned(16))) bf16_t vt0[64 * D];
  __shared__ __attribute__((aligned(16))) bf16_t kt1[64 * D];
  __shared__ __attribute__((aligned(16))) bf16_t vt1[64 * D];
  // the block's summary row (the prior's MFMA operand), copied with the
  // tiles: 64 lanes x 16 bytes, the lanes past the row read as zero
  __shared__ __attribute__((aligned(16))) bf16_t kb0[64 * 8];
  __shared__ __attribute__((aligned(16))) bf16_t kb1[64 * 8];
  const int nb = a.T / DASH_BLOCK;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, j = l & 31, h = l >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  TileCopy<D, TileSwz<D>::k> kcp;
  TileCopy<D, TileSwz<D>::v> vcp;
  kcp.init(wu, l);
  vcp.init(wu, l);
  const CoarseArith ca = a.ca;
  const float sl2 = a.fine_scale * LOG2E_F;
  const int n_items = a.n_items[0];
  const int nwg = gridDim.x, wg = blockIdx.x;
  const int first = (nwg % 8 == 0) ? (wg % 8) * (nwg / 8) + wg / 8 : wg;
  if (first >= n_items) return;  // the whole workgroup
  const int x = 32 * w + j;  // this lane's column within an item

  // the current item's column state (registers), filled one item ahead
  int c_col = 0, c_nent = 0, c_row = 0, c_dest = 0;
  bool c_valid = false, c_own = false;
  float c_tau = 0.f, c_ln = 0.f;
  bf16x8 qb[KS];

  auto copy_tiles = [&](int col, bf16_t* kd, bf16_t* vd, bf16_t* kbd) {
    const size_t bh = col / nb;
    const int b = col % nb;
    const size_t o = (bh * a.T + (size_t)b * DASH_BLOCK) * D;
    kcp.copy(reinterpret_cast<const bf16_t*>(a.k) + o, kd, wu);
    vcp.copy(reinterpret_cast<const bf16_t*>(a.v) + o, vd, wu);
    if (wu == 0) {
      const bf16_t* src = reinterpret_cast<const bf16_t*>(a.kbar) + (bh * nb + b) * D;
      const uint64_t ad = reinterpret_cast<uint64_t>(src);
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)ad);
      const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(ad >> 32));
      copy16_to_lds(tile_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo), D * 2), 16u * l, kbd);
    }
  };
  // the column data of an item whose entry is known
  auto load_cols = [&](int col, int nent, int2 ent) {
    const size_t bh = col / nb;
    const int b = col % nb;
    c_col = col;
    c_nent = nent;
    c_valid = x < nent;
    c_row = ent.x;
    c_dest = ent.y;
    c_own = c_valid && c_row / DASH_BLOCK == b;
    const bf16_t* Q = reinterpret_cast<const bf16_t*>(a.q) + (bh * a.T + c_row) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) qb[s] = c_valid ? load8(Q + 16 * s + 8 * h) : bf16x8{};
    c_tau = c_valid ? a.tau[bh * a.T + c_row] : 0.f;
    c_ln = c_valid ? a.lognorm[bh * a.T + c_row] : 0.f;
  };

  // work-item descriptors through the scalar cache (read-only here): their
  // waits go on the LDS/scalar counter, not behind the vector stores
  auto item_at = [&](int i) -> int4 {
    const __attribute__((address_space(4))) int* p =
        (const __attribute__((address_space(4))) int*)(uintptr_t)(a.items + i);
    return make_int4(p[0], p[1], p[2], p[3]);
  };
  // prologue: item `first` into buffers 0 and registers, entries of the
  // next item, descriptors of the two after it
  int it = first;
  int4 cur = item_at(it);
  int4 nx1 = it + nwg < n_items ? item_at(it + nwg) : make_int4(0, 0, 0, 0);
  int4 nx2 = it + 2 * nwg < n_items ? item_at(it + 2 * nwg) : make_int4(0, 0, 0, 0);
  copy_tiles(cur.x, kt0, vt0, kb0);
  load_cols(cur.x, cur.z, x < cur.z ? a.col_ent[cur.y + x] : make_int2(0, 0));
  int2 ent1 = (it + nwg < n_items && x < nx1.z) ? a.col_ent[nx1.y + x] : make_int2(0, 0);
  tile_copies_done();

  // one item from buffers (kt, vt), the next one's copy into (ko, vo);
  // called with fixed buffers (the loop is unrolled by two), so that the
  // compiler sees that the operand reads of one pair are not ordered
  // behind the copy into the other.  Returns whether more items follow.
  auto step = [&](bf16_t* kt, bf16_t* vt, bf16_t* kbt, bf16_t* ko, bf16_t* vo, bf16_t* kbo) -> bool {
    // item it's tiles are in (kt, vt, kbt) (every wave waited for its copies
    // before the last barrier of the previous step); everyone is done with
    // the other set (its staging reads fed the stores already issued)
    lds_barrier();
    const bool more = it + nwg < n_items;
    const bool more2 = it + 2 * nwg < n_items;
    const bool more3 = it + 3 * nwg < n_items;
    // oldest first: item it+3's descriptor and item it+2's entries, so that
    // a wait for them (the descriptor goes to scalar registers) leaves the
    // later copies and gathers in flight
    const int4 nx3 = more3 ? item_at(it + 3 * nwg) : make_int4(0, 0, 0, 0);
    const int2 ent2 = (more2 && x < nx2.z) ? a.col_ent[nx2.y + x] : make_int2(0, 0);
    if (more) copy_tiles(nx1.x, ko, vo, kbo);

    const int b = c_col % nb;
    const int nent = c_nent;
    const bool wave_has = 32 * w < nent;
    const bool valid = c_valid, own = c_own;
    const int row = c_row, dest = c_dest;
    // the prior: the Stage-1 score of (row, b) from the same MFMA chain
    // (every A row is kbar_b, so every accumulator of the column is it)
    float p2 = 0.f;
    f32x16 s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
    if (wave_has) {
      bf16x8 ka[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) ka[s] = load8(kbt + 16 * s + 8 * h);
      const f32x16 z = coarse_acc_q<D>(ka, qb);
      if (valid && !own) p2 = ca.logp(ca.u_of(z[0]), c_tau, c_ln) * LOG2E_F;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int c = 2 * s + h;
        const bf16x8 a0 = load8(kt + j * D + 8 * (c ^ TileSwz<D>::k(j)));
        const bf16x8 a1 = load8(kt + (32 + j) * D + 8 * (c ^ TileSwz<D>::k(32 + j)));
        s0 = mfma32(a0, qb[s], s0);
        s1 = mfma32(a1, qb[s], s1);
      }
    }
    // the next items' data, while this item's products run
    if (more) load_cols(nx1.x, nx1.z, ent1);

    f32x16 oacc[NDT];
    float mcol = -INFINITY, ltot = 0.f;
    if (wave_has) {
      if (__ballot(own) != 0ull && own) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = b * DASH_BLOCK + acc_row32(r, l);
          if (key > row) s0[r] = -INFINITY;
          if (key + 32 > row) s1[r] = -INFINITY;
        }
      }
      float mb = fmaxf(s0[0], s0[1]);
#pragma unroll
      for (int r = 2; r < 16; ++r) mb = fmaxf(mb, s0[r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mb = fmaxf(mb, s1[r]);
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mb), __float_as_uint(mb), false, false);
        mb = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      // every column has a finite score (a listed row attends the whole
      // block before its own, and key = row in its own block)
      const float m2 = mb * sl2;
      mcol = m2 + p2;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
      const int tg = l & 15, grp = l >> 4;
      const int dof = 16 * (grp & 1) + 4 * (tg & 3);
      float ps0 = 0.f, ps1 = 0.f;
      bf16x2 one2;
      one2[0] = (__bf16)1.f;
      one2[1] = (__bf16)1.f;
      auto vread = [&](int s, int dt) -> bf16x8 {
        const int r1 = 16 * s + 4 * h + (tg >> 2), r2 = r1 + 8;
        const int cc = 32 * dt + dof;
        const int c = cc >> 3, half = (cc >> 2) & 1;
        const bf16x4 lo = ds_read_tr4(vt + r1 * D + 8 * (c ^ TileSwz<D>::v(r1)) + 4 * half);
        const bf16x4 hi = ds_read_tr4(vt + r2 * D + 8 * (c ^ TileSwz<D>::v(r2)) + 4 * half);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      bf16x8 vnext[NDT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) vnext[dt] = vread(0, dt);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 pb;
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) {
          const float sv = (s < 2) ? s0[8 * (s & 1) + e8] : s1[8 * (s & 1) + e8];
          pb[e8] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sv, sl2, -m2));
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
      const float lh = ps0 + ps1;
      ltot = lh + __shfl_xor(lh, 32, 64);
    }
    lds_barrier();  // every wave is done with this item's K and V tiles
    // staging of a wave's 32 partial rows for 16-byte stores, in this item's
    // buffers: chunk c of row x at slot c ^ (x % CH) of the wave's quarter
    bf16_t* ost = (w < 2 ? kt : vt) + (w & 1) * 32 * D;
    if (wave_has) {
      // lane (j, h) holds d = 32 dt + 8 r4 + 4 h + 0..3 of column j
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int c = 4 * dt + r4;
          bf16x4 o4;
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = (__bf16)oacc[dt][4 * r4 + e];
          *reinterpret_cast<bf16x4*>(ost + j * D + 8 * (c ^ (j & (CH - 1))) + 4 * h) = o4;
        }
      if (valid && h == 0) {
        f32x2 ml;
        ml[0] = mcol;
        ml[1] = ltot;
        __builtin_nontemporal_store(ml, reinterpret_cast<f32x2*>(a.part_ml + dest));
      }
    }
    // item i+1's tiles and column data, item i+2's entries, item i+3's
    // descriptor (and the staging above) are complete past this point;
    // this item's stores below are not waited for until the next item's
    // staging is done
    tile_copies_done();
    __syncthreads();
    if (wave_has) {
      // rolled: unrolled, the staging addresses of every store would be kept
      // (and spilled) across the loop over items
#pragma unroll 1
      for (int q = 0; q < 32 * CH / 64; ++q) {
        const int idx = q * 64 + l;
        const int cx = idx / CH, ch = idx % CH;
        const int dcx = __shfl(dest, cx, 64);
        // streaming (nontemporal) stores: the partials are read once, by the
        // merge, and should not evict the queries and tiles the next items
        // read from L2
        if (32 * w + cx < nent)
          __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(ost + cx * D + 8 * (ch ^ (cx & (CH - 1)))),
                                      reinterpret_cast<u32x4*>(a.part_o + (size_t)dcx * D + 8 * ch));
      }
    }
    // the staging of this item is read before the barrier at the top of the
    // next step, after which the copy of item it + 2 overwrites it
    ent1 = ent2;
    nx1 = nx2;
    nx2 = nx3;
    it += nwg;
    return more;
  };
  while (step(kt0, vt0, kb0, kt1, vt1, kb1) && step(kt1, vt1, kb1, kt0, vt0, kb0)) {
  }
}

// ---------------------------------------------------------------------------- merge
// 16 lanes per row, 4 rows per wave, 16 rows per workgroup (all in one
// tile).  Lane t of a row holds D/16 consecutive output values.  The
// workgroups are numbered XCD-aware (consecutive ids go round-robin over
// the 8 XCDs; each XCD takes a contiguous range of row blocks), so the
// four workgroups of a 64-row group, whose rows read the group's partials
// and (max, sum) records in interleaved order, share one L2.
template <int D>
__global__ __launch_bounds__(256) void ld_merge_kernel(LdArgs a) {
  constexpr int VPL = D / 16;
  const int ntile = (a.T + DASH_QTILE - 1) / DASH_QTILE;
  const int rows_per_head = a.T;
  const int nwg = gridDim.x, wg = blockIdx.x;
  const int logical = (nwg % 8 == 0) ? (wg % 8) * (nwg / 8) + wg / 8 : wg;
  const size_t grow = (size_t)logical * 16 + (threadIdx.x >> 4);
  const size_t bh = grow / rows_per_head;
  const int r = (int)(grow % rows_per_head);
  if (bh >= (size_t)a.BH) return;
  if (a.tile_off[bh * ntile + r / DASH_QTILE] < 0) return;  // a dense-walk tile (the whole workgroup)
  const int l = threadIdx.x & 63, t = l & 15, gbase = l & ~15;
  const int2 info = a.row_info[bh * a.T + r];
  const int off = info.x, n = info.y;
  const int* pos = a.row_pos + off;
  typedef uint16_t u16v __attribute__((ext_vector_type(VPL)));
  // one pass with a running maximum: a chunk of 16 slots issues its (max,
  // sum) record and its 16 partial rows together, and the next chunk's
  // positions are in flight meanwhile, so a row waits on about one load
  // round trip per chunk; when the maximum rises the sums so far are
  // rescaled by 2^(old - new)
  float M = -INFINITY, L = 0.f;
  float acc[VPL];
#pragma unroll
  for (int e = 0; e < VPL; ++e) acc[e] = 0.f;
  int ps = t < n ? pos[t] : -1;  // lane t: the chunk's slot t (-1 past the row's end)
  for (int s0 = 0; s0 < n; s0 += 16) {
    const int s = s0 + t;
    const int ps_nx = s + 16 < n ? pos[s + 16] : -1;
    const float2 ml = ps >= 0 ? a.part_ml[ps] : make_float2(-INFINITY, 0.f);
    u16v ov[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int pk = __shfl(ps, gbase + k, 64);
      if (pk >= 0) ov[k] = *reinterpret_cast<const u16v*>(a.part_o + (size_t)pk * D + VPL * t);
      else ov[k] = u16v{};
    }
    float cm = ml.x;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) cm = fmaxf(cm, __shfl_xor(cm, o, 64));
    const float Mn = fmaxf(M, cm);  // finite: every chunk holds at least one slot
    const float c = __builtin_amdgcn_exp2f(M - Mn);
    M = Mn;
    const float wgt = ps >= 0 ? __builtin_amdgcn_exp2f(ml.x - M) : 0.f;
    L = fmaf(L, c, wgt * ml.y);
#pragma unroll
    for (int e = 0; e < VPL; ++e) acc[e] *= c;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float wk = __shfl(wgt, gbase + k, 64);
#pragma unroll
      for (int e = 0; e < VPL; ++e) acc[e] = fmaf(wk, bf2f(ov[k][e]), acc[e]);
    }
    ps = ps_nx;
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) L += __shfl_xor(L, o, 64);
  const float inv = 1.f / L;
  bf16_t* O = reinterpret_cast<bf16_t*>(a.o) + (bh * a.T + r) * D + VPL * t;
  u16v ov;
#pragma unroll
  for (int e = 0; e < VPL; ++e) ov[e] = f2bf(acc[e] * inv);
  *reinterpret_cast<u16v*>(O) = ov;
  if (t == 0) a.lse[bh * a.T + r] = (M + __builtin_amdgcn_logf(L)) * LN2_F;
}

}  // namespace

hipError_t launch_lowdens_plan(const LdArgs& a, hipStream_t st) {
  const int nb = a.T / DASH_BLOCK;
  const unsigned groups = (unsigned)((a.BH * nb + 3) / 4);
  ld_count_kernel<<<groups, 256, 0, st>>>(a);
  ld_scan_tiles_kernel<<<1, 1024, 0, st>>>(a);
  ld_colscan_kernel<<<(unsigned)(a.BH * ((nb + 63) / 64)), 1024, 0, st>>>(a);
  ld_scan_cols_kernel<<<1, 1024, 0, st>>>(a);
  ld_items_kernel<false><<<a.BH, 1024, 0, st>>>(a);
  ld_items_kernel<true><<<a.BH, 1024, 0, st>>>(a);
  ld_fill_kernel<<<(unsigned)(a.BH * nb), 64, 0, st>>>(a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_part(const LdArgs& a, hipStream_t st) {
  // persistent: as many workgroups as are resident at once, so that every
  // workgroup starts at once and the static item order balances
  int dev = 0, ncu = 256, occ = 2;
  hipError_t e;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, ld_part_kernel<D>, 256, 0)) != hipSuccess) return e;
  ld_part_kernel<D><<<ncu * (occ < 1 ? 1 : occ), 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_lowdens_attend(const LdArgs& a, hipStream_t st) {
  hipError_t e = a.D == 128 ? launch_part<128>(a, st) : launch_part<64>(a, st);
  if (e != hipSuccess) return e;
  const size_t rows = (size_t)a.BH * a.T;
  const dim3 mg((unsigned)((rows + 15) / 16));
  if (a.D == 128) ld_merge_kernel<128><<<mg, 256, 0, st>>>(a);
  else ld_merge_kernel<64><<<mg, 256, 0, st>>>(a);
  return hipGetLastError();
}
