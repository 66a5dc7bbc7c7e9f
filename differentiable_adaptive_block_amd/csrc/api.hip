// C ABI of the DashAttention hot path: host-side validation and launches.
// The declarations, argument meaning, layouts and error behaviour are in
// include/dash.h.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "dash.h"
#include "kernels.h"
#include "attn_bwd.h"
#include "summariser.h"
#include "decode.h"
#include "ragged.h"

namespace {

thread_local std::string g_err;

dash_status fail(dash_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
dash_status fail(dash_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

dash_status hip_fail(hipError_t e, const char* where) {
  return fail(DASH_EHIP, "%s: %s", where, hipGetErrorString(e));
}

bool ok_ptr(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool ok_opt(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool finite_pos(float x) { return std::isfinite(x) && x > 0.f; }

CoarseArith make_ca(float alpha, float coarse_scale) {
  CoarseArith ca;
  ca.coarse_scale = coarse_scale;
  ca.softmax = alpha == 1.0f;
  ca.am1 = alpha - 1.0f;
  ca.m = ca.softmax ? 1.0f : 1.0f / (alpha - 1.0f);
  return ca;
}

dash_status check_common(int D, int block, float alpha, float fs, float cs, int dtype) {
  if (!(alpha >= 1.0f && alpha <= 2.0f)) return fail(DASH_EINVAL, "alpha must lie in [1, 2] (got %g)", alpha);
  if (!finite_pos(fs) || !finite_pos(cs)) return fail(DASH_EINVAL, "scales must be finite and positive");
  if (dtype != DASH_F32 && dtype != DASH_BF16) return fail(DASH_EINVAL, "unknown dtype %d", dtype);
  if (block != DASH_BLOCK) return fail(DASH_EUNSUPPORTED, "block must be 64 (got %d)", block);
  if (D != 64 && D != 128) return fail(DASH_EUNSUPPORTED, "head dim must be 64 or 128 (got %d)", D);
  return DASH_OK;
}

// ragged: a T that is not a multiple of 64 is accepted (causal only); the
// entries that take it (dash_fwd, dash_bwd and their sizes) run on copies
// padded to whole blocks.
dash_status check_params(const dash_params* p, bool limit_T = true, bool ragged = false) {
  if (!p) return fail(DASH_EINVAL, "null params");
  if (p->B < 1 || p->H < 1) return fail(DASH_EINVAL, "B and H must be >= 1");
  if (p->T < 1) return fail(DASH_EINVAL, "T must be positive (got %d)", p->T);
  if (p->T % DASH_BLOCK) {
    if (!ragged)
      return fail(DASH_EINVAL, "T must be a multiple of 64 here (got %d); dash_fwd and dash_bwd accept others", p->T);
    if (p->causal != 1) return fail(DASH_EINVAL, "a partial last block (T = %d) needs causal attention", p->T);
  }
  if (p->causal != 0 && p->causal != 1) return fail(DASH_EINVAL, "causal must be 0 or 1");
  dash_status s = check_common(p->D, p->block, p->alpha, p->fine_scale, p->coarse_scale, p->dtype);
  if (s != DASH_OK) return s;
  if (limit_T && (p->T + DASH_BLOCK - 1) / DASH_BLOCK > DASH_MAX_NB)
    return fail(DASH_EUNSUPPORTED, "T above %d is not built", DASH_MAX_NB * DASH_BLOCK);
  return DASH_OK;
}

bool is_ragged(const dash_params* p) { return p->T % DASH_BLOCK != 0; }

// The same problem padded to whole blocks.
dash_params padded(const dash_params* p) {
  dash_params q = *p;
  q.T = (p->T + DASH_BLOCK - 1) / DASH_BLOCK * DASH_BLOCK;
  return q;
}

size_t elem_bytes(const dash_params* p) { return p->dtype == DASH_BF16 ? 2 : 4; }

int ntile_of(int T) { return (T + DASH_QTILE - 1) / DASH_QTILE; }
int nbw_of(int nb) { return (nb + 31) / 32; }

dash_status check_sel(const dash_sel* sel, bool need_bits) {
  if (!sel) return fail(DASH_EINVAL, "null selection struct");
  if (!ok_ptr(sel->tau) || !ok_ptr(sel->lognorm) || !ok_ptr(sel->tile_cnt) || !ok_ptr(sel->tile_blk) ||
      !ok_ptr(sel->tile_bits))
    return fail(DASH_EINVAL, "selection buffers tau/lognorm/tile_cnt/tile_blk/tile_bits must be non-null and 16-byte aligned");
  if (!ok_opt(sel->nsel) || !ok_opt(sel->mask) || !ok_opt(sel->passes))
    return fail(DASH_EINVAL, "nsel/mask/passes must be 16-byte aligned");
  (void)need_bits;
  return DASH_OK;
}

size_t bwd_ws_layout(const dash_params* p, size_t off[4]) {
  const size_t BH = (size_t)p->B * p->H, T = p->T, D = p->D, nb = T / DASH_BLOCK, nt = ntile_of(p->T);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o += (bytes + 255) & ~size_t(255); return r; };
  off[0] = take(BH * T * sizeof(float));               // delta
  off[1] = take(BH * T * D * sizeof(float));           // dq accumulator
  // listed-entry room per head; the fp32 path keeps one value per (row, block) instead
  const size_t per_head = p->dtype == DASH_F32 ? T * nb : bwd_entries_per_head(p->causal, (int)nb, (int)nt) * DASH_QTILE;
  off[2] = take(BH * per_head * sizeof(float));  // G (fp32 path: coarse-scaled dz)
  off[3] = take(BH * per_head * sizeof(float));  // prior
  return o;
}

size_t decode_ws_layout(const dash_decode_params* p, size_t off[5], int* nsplit, int* chunk) {
  const size_t SH = (size_t)p->S * p->H, nb = p->N / DASH_BLOCK, D = p->D;
  const int ch = 4;  // waves per split-KV workgroup
  const int ns = DASH_DEC_SPLIT;
  if (nsplit) *nsplit = ns;
  if (chunk) *chunk = ch;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o += (bytes + 255) & ~size_t(255); return r; };
  off[0] = take(SH * 2 * sizeof(float));           // tau, lognorm
  off[1] = take(SH * sizeof(int));                 // list length
  off[2] = take(SH * nb * sizeof(int));            // list
  off[3] = take(SH * nb * sizeof(float));          // log2 priors
  off[4] = take(SH * DASH_DEC_SPLIT_GQA * (D + 2) * sizeof(float));  // partials (the larger split count)
  return o;
}

// Scratch of dash_decode_static: the decode workspace (row statistics,
// block lists, split partials) of callers that cannot allocate.
// Each GPU the library runs on holds its own copy until the process ends.
// In host code `scratch` is the host-side stand-in of the array, not a
// device address: the device address comes from hipGetSymbolAddress, once
// per device, with that device current.
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on its first use on
// that device); nullptr with an error message on failure.
void* static_scratch(hipError_t* err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *err = hipSuccess;
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int32_t dash_query_tile(void) { return DASH_QTILE; }

const char* dash_last_error(void) { return g_err.c_str(); }

dash_status dash_sel_sizes(const dash_params* p, size_t out[8]) {
  dash_status s = check_params(p, true, true);
  if (s != DASH_OK) return s;
  if (!out) return fail(DASH_EINVAL, "null output array");
  const dash_params pp = padded(p);  // a partial last block is laid out as a whole one
  const size_t BH = (size_t)p->B * p->H, T = pp.T, nb = T / DASH_BLOCK, nbw = nbw_of((int)nb), nt = ntile_of(p->T);
  out[0] = BH * T;
  out[1] = BH * T;
  out[2] = BH * T;
  out[3] = BH * T * nbw;
  out[4] = BH * nt;
  out[5] = BH * nt * nb;
  out[6] = BH * nt * nbw;
  out[7] = BH * T;
  return DASH_OK;
}

// Padded copies for the backward of a ragged T (rows of Tp = whole blocks
// per head): q, k, v, o, dout, dq, dk, dv and lse, after the whole-block
// backward's own workspace.
size_t ragged_bwd_layout(const dash_params* p, size_t off[14]) {
  const dash_params pp = padded(p);
  size_t o = bwd_ws_layout(&pp, off);  // off[0..3]
  const size_t BH = (size_t)p->B * p->H, rows = BH * pp.T, mat = rows * p->D * elem_bytes(p);
  auto take = [&](size_t bytes) { size_t r = o; o += (bytes + 255) & ~size_t(255); return r; };
  for (int i = 4; i < 12; ++i) off[i] = take(mat);  // q k v o dout dq dk dv
  off[12] = take(rows * sizeof(float));            // lse
  return o;
}

size_t dash_fwd_workspace_bytes(const dash_params* p) {
  (void)p;
  return 0;  // a partial last block is handled inside the kernels
}

size_t dash_bwd_workspace_bytes(const dash_params* p) {
  if (check_params(p, true, true) != DASH_OK) return 0;
  size_t off[14];
  if (is_ragged(p)) return ragged_bwd_layout(p, off);
  return bwd_ws_layout(p, off);
}

size_t dash_decode_workspace_bytes(const dash_decode_params* p) {
  if (!p || p->S < 1 || p->H < 1 || p->N < DASH_BLOCK || p->N % DASH_BLOCK) return 0;
  size_t off[5];
  return decode_ws_layout(p, off, nullptr, nullptr);
}

dash_status dash_pool(const dash_params* p, const void* k, void* kbar, void* stream) {
  dash_status s = check_params(p, false);
  if (s != DASH_OK) return s;
  if (!ok_ptr(k) || !ok_ptr(kbar)) return fail(DASH_EINVAL, "k and kbar must be non-null and 16-byte aligned");
  hipError_t e = launch_pool(k, kbar, p->B * p->H, p->T, p->D, p->dtype, (hipStream_t)stream);
  return e == hipSuccess ? DASH_OK : hip_fail(e, "pool");
}

// Stage 1 (scores, entmax, masks, tile lists) from summaries already in kbar;
// grp query heads per key/value head (their tile lists are the group's union).
static dash_status select_from_kbar(const dash_params* p, const void* q, const void* kbar, const dash_sel* sel,
                                    hipStream_t st, int grp = 1, int Tr = -1) {
  const int BH = p->B * p->H;
  const int nb = p->T / DASH_BLOCK;
  hipError_t e;
  if ((e = launch_fill_u32(sel->tile_bits, (size_t)BH * ntile_of(p->T) * nbw_of(nb), 0u, st)) != hipSuccess)
    return hip_fail(e, "clear tile bits");
  SelectArgs sa;
  sa.q = q;
  sa.kbar = kbar;
  sa.T = p->T;
  sa.Tr = Tr < 0 ? p->T : Tr;
  sa.D = p->D;
  sa.causal = p->causal;
  sa.grp = grp;
  sa.ca = make_ca(p->alpha, p->coarse_scale);
  sa.tau = sel->tau;
  sa.lognorm = sel->lognorm;
  sa.nsel = sel->nsel;
  sa.mask = sel->mask;
  sa.passes = sel->passes;
  sa.tile_bits = sel->tile_bits;
  if ((e = launch_select(sa, BH, p->dtype, st)) != hipSuccess) return hip_fail(e, "select");
  if ((e = launch_group_union(sel->tile_bits, BH, grp, (size_t)ntile_of(p->T) * nbw_of(nb), st)) != hipSuccess)
    return hip_fail(e, "group union");
  if ((e = launch_tile_lists(sel->tile_bits, sel->tile_cnt, sel->tile_blk, BH, p->T, p->causal, st)) != hipSuccess)
    return hip_fail(e, "tile lists");
  return DASH_OK;
}

dash_status dash_fwd_select(const dash_params* p, const void* q, const void* k, void* kbar, const dash_sel* sel,
                            void* stream) {
  dash_status s = check_params(p);
  if (s != DASH_OK) return s;
  if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(kbar)) return fail(DASH_EINVAL, "q, k and kbar must be non-null and 16-byte aligned");
  if ((s = check_sel(sel, true)) != DASH_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if ((e = launch_pool(k, kbar, p->B * p->H, p->T, p->D, p->dtype, st)) != hipSuccess) return hip_fail(e, "pool");
  return select_from_kbar(p, q, kbar, sel, st);
}

dash_status dash_select(const dash_params* p, const void* q, const void* kbar, const dash_sel* sel, void* stream) {
  dash_status s = check_params(p);
  if (s != DASH_OK) return s;
  if (!ok_ptr(q) || !ok_ptr(kbar)) return fail(DASH_EINVAL, "q and kbar must be non-null and 16-byte aligned");
  if ((s = check_sel(sel, true)) != DASH_OK) return s;
  return select_from_kbar(p, q, kbar, sel, (hipStream_t)stream);
}

dash_status dash_pool_attn(const dash_params* p, const void* k, const float* w, void* kbar, void* stream) {
  dash_status s = check_params(p, false);
  if (s != DASH_OK) return s;
  if (!ok_ptr(k) || !ok_ptr(kbar) || !ok_ptr(w)) return fail(DASH_EINVAL, "k, w and kbar must be non-null and 16-byte aligned");
  hipError_t e = launch_pool_attn(k, w, kbar, p->B * p->H, p->H, p->T, p->D, p->dtype, (hipStream_t)stream);
  return e == hipSuccess ? DASH_OK : hip_fail(e, "attention pooling");
}

size_t dash_pool_attn_bwd_workspace_bytes(const dash_params* p) {
  if (check_params(p, false) != DASH_OK) return 0;
  return (size_t)p->B * p->H * (p->T / DASH_BLOCK) * p->D * sizeof(float);
}

dash_status dash_pool_attn_bwd(const dash_params* p, const void* k, const float* w, const float* dkbar, void* dk,
                               float* dw, void* workspace, size_t workspace_bytes, void* stream) {
  dash_status s = check_params(p, false);
  if (s != DASH_OK) return s;
  if (!ok_ptr(k) || !ok_ptr(w) || !ok_ptr(dkbar) || !ok_ptr(dk) || !ok_ptr(dw))
    return fail(DASH_EINVAL, "k, w, dkbar, dk and dw must be non-null and 16-byte aligned");
  const size_t need = dash_pool_attn_bwd_workspace_bytes(p);
  if (workspace_bytes < need) return fail(DASH_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (!ok_ptr(workspace)) return fail(DASH_EINVAL, "workspace must be non-null and 16-byte aligned");
  hipError_t e = launch_pool_attn_bwd(k, w, dkbar, dk, dw, static_cast<float*>(workspace), p->B, p->H, p->T, p->D,
                                      p->dtype, (hipStream_t)stream);
  return e == hipSuccess ? DASH_OK : hip_fail(e, "attention pooling backward");
}

static dash_status attend_common(const dash_params* p, const void* q, const void* k, const void* v,
                                 const void* kbar, const dash_sel* sel, void* o, float* lse, void* stream, int grp,
                                 int Tr = -1, const int* dense_list = nullptr, const int* dense_n = nullptr) {
  FwdArgs fa;
  fa.dense_list = dense_list;
  fa.dense_n = dense_n;
  fa.Tr = Tr < 0 ? p->T : Tr;
  fa.q = q;
  fa.k = k;
  fa.v = v;
  fa.kbar = kbar;
  fa.o = o;
  fa.lse = lse;
  fa.tau = sel->tau;
  fa.lognorm = sel->lognorm;
  fa.tile_cnt = sel->tile_cnt;
  fa.tile_blk = sel->tile_blk;
  fa.BH = p->B * p->H;
  fa.T = p->T;
  fa.D = p->D;
  fa.causal = p->causal;
  fa.grp = grp;
  fa.fine_scale = p->fine_scale;
  fa.ca = make_ca(p->alpha, p->coarse_scale);
  hipError_t e = launch_fwd(fa, p->dtype, (hipStream_t)stream);
  return e == hipSuccess ? DASH_OK : hip_fail(e, "stage 2 forward");
}

dash_status dash_fwd_attend(const dash_params* p, const void* q, const void* k, const void* v, const void* kbar,
                            const dash_sel* sel, void* o, float* lse, void* stream) {
  dash_status s = check_params(p);
  if (s != DASH_OK) return s;
  if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(o) || !ok_ptr(lse) || !ok_ptr(kbar))
    return fail(DASH_EINVAL, "q, k, v, o, lse and kbar must be non-null and 16-byte aligned");
  if ((s = check_sel(sel, true)) != DASH_OK) return s;
  return attend_common(p, q, k, v, kbar, sel, o, lse, stream, 1);
}

static dash_status check_groups(const dash_params* p, int32_t kv_heads) {
  if (kv_heads < 1 || p->H % kv_heads) return fail(DASH_EINVAL, "kv_heads (%d) must divide H (%d)", kv_heads, p->H);
  if (kv_heads != p->H && p->dtype != DASH_BF16)
    return fail(DASH_EUNSUPPORTED, "grouped-query heads are built for bf16 only");
  return DASH_OK;
}

dash_status dash_fwd_gqa(const dash_params* p, int32_t kv_heads, const void* q, const void* k, const void* v,
                         void* o, float* lse, void* kbar, const dash_sel* sel, void* stream) {
  dash_status s = check_params(p);
  if (s != DASH_OK) return s;
  if ((s = check_groups(p, kv_heads)) != DASH_OK) return s;
  if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(o) || !ok_ptr(lse) || !ok_ptr(kbar))
    return fail(DASH_EINVAL, "q, k, v, o, lse and kbar must be non-null and 16-byte aligned");
  if ((s = check_sel(sel, true)) != DASH_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  const int grp = p->H / kv_heads;
  hipError_t e;
  if ((e = launch_pool(k, kbar, p->B * kv_heads, p->T, p->D, p->dtype, st)) != hipSuccess) return hip_fail(e, "pool");
  if ((s = select_from_kbar(p, q, kbar, sel, st, grp)) != DASH_OK) return s;
  return attend_common(p, q, k, v, kbar, sel, o, lse, stream, grp);
}

// Workspace of the low-density Stage-2 schedule for `cap` (row, block)
// pairs: offsets of grp_cnt, gpairs, tile_off, row_info, col_cnt,
// col_base, n_items, items, col_ent, part_ml, part_o, row_pos, rng_pref,
// dense_list, dense_n, head_items; returns the total.
static size_t ld_layout(const dash_params* p, long long cap, size_t off[16]) {
  const size_t BH = (size_t)p->B * p->H, nb = p->T / DASH_BLOCK, ntile = ntile_of(p->T);
  const size_t nr = (nb + DASH_LD_RANGE - 1) / DASH_LD_RANGE;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o += (bytes + 255) & ~size_t(255); return r; };
  off[0] = take(BH * nb * nb * 4);
  off[1] = take(BH * nb * 4);
  off[2] = take(BH * ntile * 4);
  off[3] = take(BH * p->T * 8);
  off[4] = take(BH * nb * 4);
  off[5] = take(BH * nb * 4);
  off[6] = take(16);
  off[7] = take(((size_t)cap / 128 + BH * nr * nb + 1) * 16);
  off[8] = take((size_t)cap * 8);
  off[9] = take((size_t)cap * 8);
  off[10] = take((size_t)cap * 2 * p->D);
  off[11] = take((size_t)cap * 4);
  off[12] = take(BH * (nr + 1) * nb * 4);
  off[13] = take(BH * ntile * 4);
  off[14] = take(16);
  off[15] = take(BH * 4);
  return o;
}

static constexpr long long kLdMaxPairs = 0x7FFFFFFFll;  // pair indices are int32

// Pairs a workspace of `bytes` holds (0 when it does not hold the fixed part).
static long long ld_cap_of(const dash_params* p, size_t bytes) {
  size_t off[16];
  const size_t base = ld_layout(p, 0, off);
  if (bytes < base) return 0;
  // the largest cap whose layout fits (the layout grows with cap)
  long long lo = 0, hi = kLdMaxPairs;
  if (ld_layout(p, hi, off) <= bytes) return hi;
  while (hi - lo > 1) {
    const long long mid = lo + (hi - lo) / 2;
    if (ld_layout(p, mid, off) <= bytes) lo = mid;
    else hi = mid;
  }
  return lo;
}

static bool ld_supported(const dash_params* p, const dash_sel* sel) {
  return p->dtype == DASH_BF16 && p->causal && p->T % DASH_BLOCK == 0 && sel->mask != nullptr;
}

size_t dash_fwd_lowdens_workspace_bytes(const dash_params* p, int64_t max_pairs) {
  if (check_params(p) != DASH_OK || max_pairs < 0 || max_pairs > kLdMaxPairs) return 0;
  size_t off[16];
  return ld_layout(p, max_pairs, off);
}

static dash_status attend_lowdens(const dash_params* p, const void* q, const void* k, const void* v,
                                  const void* kbar, const dash_sel* sel, float ratio, void* o, float* lse,
                                  void* workspace, size_t workspace_bytes, hipStream_t st) {
  LdArgs la;
  la.q = q;
  la.k = k;
  la.v = v;
  la.kbar = kbar;
  la.o = o;
  la.lse = lse;
  la.tau = sel->tau;
  la.lognorm = sel->lognorm;
  la.mask = sel->mask;
  la.tile_cnt = sel->tile_cnt;
  la.BH = p->B * p->H;
  la.T = p->T;
  la.D = p->D;
  la.fine_scale = p->fine_scale;
  la.ca = make_ca(p->alpha, p->coarse_scale);
  la.ratio = ratio;
  la.cap = ld_cap_of(p, workspace_bytes);
  size_t off[16];
  ld_layout(p, la.cap, off);
  char* ws = static_cast<char*>(workspace);
  la.grp_cnt = reinterpret_cast<int*>(ws + off[0]);
  la.gpairs = reinterpret_cast<int*>(ws + off[1]);
  la.tile_off = reinterpret_cast<int*>(ws + off[2]);
  la.row_info = reinterpret_cast<int2*>(ws + off[3]);
  la.col_cnt = reinterpret_cast<int*>(ws + off[4]);
  la.col_base = reinterpret_cast<int*>(ws + off[5]);
  la.n_items = reinterpret_cast<int*>(ws + off[6]);
  la.items = reinterpret_cast<int4*>(ws + off[7]);
  la.col_ent = reinterpret_cast<int2*>(ws + off[8]);
  la.part_ml = reinterpret_cast<float2*>(ws + off[9]);
  la.part_o = reinterpret_cast<bf16_t*>(ws + off[10]);
  la.row_pos = reinterpret_cast<int*>(ws + off[11]);
  la.rng_pref = reinterpret_cast<int*>(ws + off[12]);
  la.dense_list = reinterpret_cast<int*>(ws + off[13]);
  la.dense_n = reinterpret_cast<int*>(ws + off[14]);
  la.head_items = reinterpret_cast<int*>(ws + off[15]);
  hipError_t e;
  if ((e = launch_lowdens_plan(la, st)) != hipSuccess) return hip_fail(e, "low-density plan");
  dash_status s = attend_common(p, q, k, v, kbar, sel, o, lse, st, 1, -1, la.dense_list, la.dense_n);
  if (s != DASH_OK) return s;
  if ((e = launch_lowdens_attend(la, st)) != hipSuccess) return hip_fail(e, "low-density attention");
  return DASH_OK;
}

dash_status dash_fwd_attend_lowdens(const dash_params* p, const void* q, const void* k, const void* v,
                                    const void* kbar, const dash_sel* sel, float ratio, void* o, float* lse,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  dash_status s = check_params(p);
  if (s != DASH_OK) return s;
  if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(o) || !ok_ptr(lse) || !ok_ptr(kbar))
    return fail(DASH_EINVAL, "q, k, v, o, lse and kbar must be non-null and 16-byte aligned");
  if ((s = check_sel(sel, true)) != DASH_OK) return s;
  if (!(ratio >= 0.f) || !std::isfinite(ratio)) return fail(DASH_EINVAL, "ratio must be finite and >= 0 (got %g)", ratio);
  if (!ld_supported(p, sel))
    return fail(DASH_EUNSUPPORTED, "the low-density schedule is built for causal bf16 attention and needs sel->mask");
  size_t off[16];
  const size_t need = ld_layout(p, 0, off);
  if (workspace_bytes < need) return fail(DASH_EWORKSPACE, "workspace of at least %zu bytes needed, %zu given", need, workspace_bytes);
  if (!ok_ptr(workspace)) return fail(DASH_EINVAL, "workspace must be non-null and 16-byte aligned");
  return attend_lowdens(p, q, k, v, kbar, sel, ratio, o, lse, workspace, workspace_bytes, (hipStream_t)stream);
}

dash_status dash_fwd(const dash_params* p, const void* q, const void* k, const void* v, void* o, float* lse,
                     void* kbar, const dash_sel* sel, void* workspace, size_t workspace_bytes, void* stream) {
  dash_status s = check_params(p, true, true);
  if (s != DASH_OK) return s;
  if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(o) || !ok_ptr(lse) || !ok_ptr(kbar))
    return fail(DASH_EINVAL, "q, k, v, o, lse and kbar must be non-null and 16-byte aligned");
  if ((s = check_sel(sel, true)) != DASH_OK) return s;
  if (!is_ragged(p)) {
    if ((s = dash_fwd_select(p, q, k, kbar, sel, stream)) != DASH_OK) return s;
    // a workspace with room for pairs switches on the low-density schedule
    if (ld_supported(p, sel) && ok_ptr(workspace) && ld_cap_of(p, workspace_bytes) > 0)
      return attend_lowdens(p, q, k, v, kbar, sel, DASH_LOWDENS_RATIO, o, lse, workspace, workspace_bytes,
                            (hipStream_t)stream);
    return dash_fwd_attend(p, q, k, v, kbar, sel, o, lse, stream);
  }
  // a partial last block: the kernels take the tensors as they are (T rows
  // per head) and treat the block as whole, its missing rows as zeros
  const dash_params pp = padded(p);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if ((e = launch_pool(k, kbar, p->B * p->H, pp.T, p->D, p->dtype, st, p->T)) != hipSuccess) return hip_fail(e, "pool");
  if ((s = select_from_kbar(&pp, q, kbar, sel, st, 1, p->T)) != DASH_OK) return s;
  return attend_common(&pp, q, k, v, kbar, sel, o, lse, stream, 1, p->T);
}

static dash_status bwd_common(const dash_params* p, const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, const void* kbar, const dash_sel* sel, void* dq,
                              void* dk, void* dv, float* dkbar, void* workspace, size_t workspace_bytes, void* stream,
                              float pool_scale, int dk_f32 = 0) {
  dash_status s = check_params(p);
  if (s != DASH_OK) return s;
  if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(o) || !ok_ptr(lse) || !ok_ptr(dout) || !ok_ptr(kbar) ||
      !ok_ptr(dq) || !ok_ptr(dk) || !ok_ptr(dv) || !ok_ptr(dkbar))
    return fail(DASH_EINVAL, "tensor pointers must be non-null and 16-byte aligned");
  if ((s = check_sel(sel, true)) != DASH_OK) return s;
  size_t off[4];
  const size_t need = bwd_ws_layout(p, off);
  if (workspace_bytes < need) return fail(DASH_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (!ok_ptr(workspace)) return fail(DASH_EINVAL, "workspace must be non-null and 16-byte aligned");
  char* ws = static_cast<char*>(workspace);
  BwdArgs ba;
  ba.q = q;
  ba.k = k;
  ba.v = v;
  ba.o = o;
  ba.lse = lse;
  ba.dout = dout;
  ba.kbar = kbar;
  ba.tau = sel->tau;
  ba.lognorm = sel->lognorm;
  ba.tile_cnt = sel->tile_cnt;
  ba.tile_blk = sel->tile_blk;
  ba.tile_bits = sel->tile_bits;
  ba.dq = dq;
  ba.dk = dk;
  ba.dv = dv;
  ba.dkbar = dkbar;
  ba.delta = reinterpret_cast<float*>(ws + off[0]);
  ba.dq_acc = reinterpret_cast<float*>(ws + off[1]);
  ba.gbuf = reinterpret_cast<float*>(ws + off[2]);
  ba.pbuf = reinterpret_cast<float*>(ws + off[3]);
  ba.BH = p->B * p->H;
  ba.T = p->T;
  ba.D = p->D;
  ba.causal = p->causal;
  ba.fine_scale = p->fine_scale;
  ba.pool_scale = pool_scale;
  ba.dk_f32 = dk_f32;
  ba.grp = 1;
  ba.gsum = nullptr;
  ba.phbuf = nullptr;
  ba.ca = make_ca(p->alpha, p->coarse_scale);
  hipError_t e = launch_bwd(ba, p->dtype, (hipStream_t)stream);
  return e == hipSuccess ? DASH_OK : hip_fail(e, "backward");
}

static size_t bwd_gqa_ws_layout(const dash_params* p, int32_t kv_heads, size_t off[9]) {
  size_t base = bwd_ws_layout(p, off);
  const size_t BH = (size_t)p->B * p->H, T = p->T, D = p->D, nb = T / DASH_BLOCK, nt = ntile_of(p->T);
  const size_t grp = (size_t)p->H / kv_heads;
  size_t o = base;
  auto take = [&](size_t bytes) { size_t r = o; o += (bytes + 255) & ~size_t(255); return r; };
  const size_t ent = bwd_entries_per_head(p->causal, (int)nb, (int)nt);
  off[4] = take(BH / grp * ent * DASH_QTILE * sizeof(float));  // G summed over each group
  off[5] = take(BH * T * D * 2);                                   // dK per query head
  off[6] = take(BH * T * D * 2);                                   // dV per query head
  off[7] = take(BH * nb * D * sizeof(float));                      // dkbar per query head
  off[8] = take(BH * ent * DASH_QTILE * sizeof(float));             // each row's own log2 p
  return o;
}

size_t dash_bwd_gqa_workspace_bytes(const dash_params* p, int32_t kv_heads) {
  if (check_params(p) != DASH_OK || kv_heads < 1 || p->H % kv_heads) return 0;
  size_t off[9];
  if (kv_heads == p->H) return bwd_ws_layout(p, off);
  return bwd_gqa_ws_layout(p, kv_heads, off);
}

dash_status dash_bwd_gqa(const dash_params* p, int32_t kv_heads, const void* q, const void* k, const void* v,
                         const void* o, const float* lse, const void* dout, const void* kbar, const dash_sel* sel,
                         void* dq, void* dk, void* dv, float* dkbar, void* workspace, size_t workspace_bytes,
                         void* stream) {
  dash_status s = check_params(p);
  if (s != DASH_OK) return s;
  if ((s = check_groups(p, kv_heads)) != DASH_OK) return s;
  if (kv_heads == p->H)
    return bwd_common(p, q, k, v, o, lse, dout, kbar, sel, dq, dk, dv, dkbar, workspace, workspace_bytes, stream,
                      1.f / DASH_BLOCK);
  if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(o) || !ok_ptr(lse) || !ok_ptr(dout) || !ok_ptr(kbar) ||
      !ok_ptr(dq) || !ok_ptr(dk) || !ok_ptr(dv) || !ok_ptr(dkbar))
    return fail(DASH_EINVAL, "tensor pointers must be non-null and 16-byte aligned");
  if ((s = check_sel(sel, true)) != DASH_OK) return s;
  size_t off[9];
  const size_t need = bwd_gqa_ws_layout(p, kv_heads, off);
  if (workspace_bytes < need) return fail(DASH_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (!ok_ptr(workspace)) return fail(DASH_EINVAL, "workspace must be non-null and 16-byte aligned");
  char* ws = static_cast<char*>(workspace);
  BwdArgs ba;
  ba.q = q;
  ba.k = k;
  ba.v = v;
  ba.o = o;
  ba.lse = lse;
  ba.dout = dout;
  ba.kbar = kbar;
  ba.tau = sel->tau;
  ba.lognorm = sel->lognorm;
  ba.tile_cnt = sel->tile_cnt;
  ba.tile_blk = sel->tile_blk;
  ba.tile_bits = sel->tile_bits;
  ba.dq = dq;
  ba.dk = ws + off[5];
  ba.dv = ws + off[6];
  ba.dkbar = reinterpret_cast<float*>(ws + off[7]);
  ba.delta = reinterpret_cast<float*>(ws + off[0]);
  ba.dq_acc = reinterpret_cast<float*>(ws + off[1]);
  ba.gbuf = reinterpret_cast<float*>(ws + off[2]);
  ba.pbuf = reinterpret_cast<float*>(ws + off[3]);
  ba.gsum = reinterpret_cast<float*>(ws + off[4]);
  ba.phbuf = reinterpret_cast<float*>(ws + off[8]);
  ba.BH = p->B * p->H;
  ba.T = p->T;
  ba.D = p->D;
  ba.causal = p->causal;
  ba.grp = p->H / kv_heads;
  ba.fine_scale = p->fine_scale;
  ba.pool_scale = 1.f / DASH_BLOCK;
  ba.dk_f32 = 0;
  ba.ca = make_ca(p->alpha, p->coarse_scale);
  hipError_t e = launch_bwd_gqa(ba, dk, dv, dkbar, (hipStream_t)stream);
  return e == hipSuccess ? DASH_OK : hip_fail(e, "grouped-query backward");
}

dash_status dash_bwd(const dash_params* p, const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dout, const void* kbar, const dash_sel* sel, void* dq, void* dk,
                     void* dv, float* dkbar, void* workspace, size_t workspace_bytes, void* stream) {
  dash_status s = check_params(p, true, true);
  if (s != DASH_OK) return s;
  if (!is_ragged(p))
    return bwd_common(p, q, k, v, o, lse, dout, kbar, sel, dq, dk, dv, dkbar, workspace, workspace_bytes, stream,
                      1.f / DASH_BLOCK);
  // a partial last block: the whole-block backward on padded copies; padded
  // rows get dout = 0 and lse = +inf (weight 0), so they add nothing
  if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(o) || !ok_ptr(lse) || !ok_ptr(dout) || !ok_ptr(kbar) ||
      !ok_ptr(dq) || !ok_ptr(dk) || !ok_ptr(dv) || !ok_ptr(dkbar))
    return fail(DASH_EINVAL, "tensor pointers must be non-null and 16-byte aligned");
  if ((s = check_sel(sel, true)) != DASH_OK) return s;
  size_t off[14];
  const size_t need = ragged_bwd_layout(p, off);
  if (workspace_bytes < need) return fail(DASH_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (!ok_ptr(workspace)) return fail(DASH_EINVAL, "workspace must be non-null and 16-byte aligned");
  char* ws = static_cast<char*>(workspace);
  const dash_params pp = padded(p);
  const int BH = p->B * p->H, rb = p->D * (int)elem_bytes(p);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  const void* src[5] = {q, k, v, o, dout};
  for (int i = 0; i < 5; ++i)
    if ((e = launch_pad_rows(src[i], ws + off[4 + i], BH, p->T, pp.T, rb, st)) != hipSuccess) return hip_fail(e, "pad");
  float* lsep = reinterpret_cast<float*>(ws + off[12]);
  if ((e = launch_pad_f32(lse, lsep, BH, p->T, pp.T, INFINITY, st)) != hipSuccess) return hip_fail(e, "pad");
  size_t boff[4];
  const size_t bneed = bwd_ws_layout(&pp, boff);
  if ((s = bwd_common(&pp, ws + off[4], ws + off[5], ws + off[6], ws + off[7], lsep, ws + off[8], kbar, sel,
                      ws + off[9], ws + off[10], ws + off[11], dkbar, ws, bneed, stream, 1.f / DASH_BLOCK)) != DASH_OK)
    return s;
  void* dst[3] = {dq, dk, dv};
  for (int i = 0; i < 3; ++i)
    if ((e = launch_unpad_rows(ws + off[9 + i], dst[i], BH, p->T, pp.T, rb, st)) != hipSuccess) return hip_fail(e, "unpad");
  return DASH_OK;
}

dash_status dash_bwd_no_pool(const dash_params* p, const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, const void* kbar, const dash_sel* sel, void* dq,
                             void* dk, void* dv, float* dkbar, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_common(p, q, k, v, o, lse, dout, kbar, sel, dq, dk, dv, dkbar, workspace, workspace_bytes, stream, 0.f);
}

size_t dash_bwd_learned_workspace_bytes(const dash_params* p) {
  if (check_params(p) != DASH_OK) return 0;
  size_t off[4];
  const size_t bw = (bwd_ws_layout(p, off) + 255) & ~size_t(255);
  const size_t dkf = ((size_t)p->B * p->H * p->T * p->D * sizeof(float) + 255) & ~size_t(255);
  return bw + dkf + dash_pool_attn_bwd_workspace_bytes(p);
}

dash_status dash_bwd_learned(const dash_params* p, const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, const void* kbar, const dash_sel* sel, const float* w,
                             void* dq, void* dk, void* dv, float* dkbar, float* dw, void* workspace,
                             size_t workspace_bytes, void* stream) {
  dash_status s = check_params(p);
  if (s != DASH_OK) return s;
  if (!ok_ptr(w) || !ok_ptr(dw)) return fail(DASH_EINVAL, "w and dw must be non-null and 16-byte aligned");
  const size_t need = dash_bwd_learned_workspace_bytes(p);
  if (workspace_bytes < need) return fail(DASH_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (!ok_ptr(workspace)) return fail(DASH_EINVAL, "workspace must be non-null and 16-byte aligned");
  size_t off[4];
  const size_t bw = (bwd_ws_layout(p, off) + 255) & ~size_t(255);
  const size_t dkf = ((size_t)p->B * p->H * p->T * p->D * sizeof(float) + 255) & ~size_t(255);
  char* ws = static_cast<char*>(workspace);
  // bf16: the Stage-2 and Stage-1 terms of dK stay unrounded in the workspace
  // and the summariser's term is added before the one rounding; fp32: dK
  // itself holds them
  const bool f32tmp = p->dtype == DASH_BF16;
  void* dk_stage = f32tmp ? static_cast<void*>(ws + bw) : dk;
  if ((s = bwd_common(p, q, k, v, o, lse, dout, kbar, sel, dq, dk_stage, dv, dkbar, ws, bw, stream, 0.f,
                      f32tmp ? 1 : 0)) != DASH_OK)
    return s;
  hipError_t e = launch_pool_attn_bwd(k, w, dkbar, dk, dw, reinterpret_cast<float*>(ws + bw + dkf), p->B, p->H, p->T,
                                      p->D, p->dtype, (hipStream_t)stream,
                                      f32tmp ? reinterpret_cast<const float*>(ws + bw) : nullptr);
  return e == hipSuccess ? DASH_OK : hip_fail(e, "attention pooling backward");
}

static dash_status check_decode_params(const dash_decode_params* p) {
  if (!p) return fail(DASH_EINVAL, "null params");
  if (p->S < 1 || p->H < 1) return fail(DASH_EINVAL, "S and H must be >= 1");
  if (p->N < DASH_BLOCK || p->N % DASH_BLOCK) return fail(DASH_EINVAL, "N must be a positive multiple of 64 (got %d)", p->N);
  dash_status s = check_common(p->D, p->block, p->alpha, p->fine_scale, p->coarse_scale, p->dtype);
  if (s != DASH_OK) return s;
  if (p->N / DASH_BLOCK > 2048) return fail(DASH_EUNSUPPORTED, "cache above 131072 tokens is not built");
  if (p->dtype != DASH_BF16 || p->D != 128) return fail(DASH_EUNSUPPORTED, "decode is built for bf16, D = 128");
  return DASH_OK;
}

// Validation and launch shared by dash_decode, dash_decode_varlen and
// dash_decode_step: rows hold len[s] + len_add tokens, or N when len is null.
static dash_status decode_common(const dash_decode_params* p, const void* q, const void* kc, const void* vc,
                                 const void* kbar, const int32_t* len, int len_add, void* o, float* lse,
                                 int32_t* nsel, float* tau, uint32_t* mask, void* workspace,
                                 size_t workspace_bytes, void* stream, int grp = 1) {
  if (!ok_ptr(q) || !ok_ptr(kc) || !ok_ptr(vc) || !ok_ptr(kbar) || !ok_ptr(o))
    return fail(DASH_EINVAL, "q, kc, vc, kbar and o must be non-null and 16-byte aligned");
  if (!ok_opt(lse) || !ok_opt(nsel) || !ok_opt(tau) || !ok_opt(mask))
    return fail(DASH_EINVAL, "lse/nsel/tau/mask must be 16-byte aligned");
  size_t off[5];
  int nsplit = 0, chunk = 0;
  const size_t need = decode_ws_layout(p, off, &nsplit, &chunk);
  if (workspace_bytes < need) return fail(DASH_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (!ok_ptr(workspace)) return fail(DASH_EINVAL, "workspace must be non-null and 16-byte aligned");
  char* ws = static_cast<char*>(workspace);
  DecodeArgs da;
  da.q = q;
  da.kc = kc;
  da.vc = vc;
  da.kbar = kbar;
  da.o = o;
  da.lse = lse;
  da.nsel = nsel;
  da.tau_out = tau;
  da.mask = mask;
  da.rowstat = reinterpret_cast<float*>(ws + off[0]);
  da.sel_cnt = reinterpret_cast<int*>(ws + off[1]);
  da.sel_blk = reinterpret_cast<int*>(ws + off[2]);
  da.sel_lp = reinterpret_cast<float*>(ws + off[3]);
  da.part = reinterpret_cast<float*>(ws + off[4]);
  da.len = len;
  da.len_add = len_add;
  da.grp = grp;
  da.SH = p->S * p->H;
  da.H = p->H;
  da.N = p->N;
  da.D = p->D;
  da.nsplit = nsplit;
  da.chunk = chunk;
  da.fine_scale = p->fine_scale;
  da.ca = make_ca(p->alpha, p->coarse_scale);
  hipError_t e = launch_decode(da, p->dtype, (hipStream_t)stream);
  return e == hipSuccess ? DASH_OK : hip_fail(e, "decode");
}

static dash_status append_common(const dash_decode_params* p, const void* k_new, const void* v_new,
                                 const int32_t* len, void* kc, void* vc, void* kbar, void* stream) {
  if (!ok_ptr(k_new) || !ok_ptr(v_new) || !ok_ptr(kc) || !ok_ptr(vc) || !ok_ptr(kbar))
    return fail(DASH_EINVAL, "k_new, v_new, kc, vc and kbar must be non-null and 16-byte aligned");
  if (!len || reinterpret_cast<uintptr_t>(len) % 4) return fail(DASH_EINVAL, "len must be non-null and 4-byte aligned");
  AppendArgs aa;
  aa.k_new = k_new;
  aa.v_new = v_new;
  aa.len = len;
  aa.kc = kc;
  aa.vc = vc;
  aa.kbar = kbar;
  aa.SH = p->S * p->H;
  aa.H = p->H;
  aa.N = p->N;
  aa.D = p->D;
  hipError_t e = launch_append(aa, p->dtype, (hipStream_t)stream);
  return e == hipSuccess ? DASH_OK : hip_fail(e, "cache append");
}

dash_status dash_decode(const dash_decode_params* p, const void* q, const void* kc, const void* vc,
                        const void* kbar, void* o, float* lse, int32_t* nsel, float* tau, uint32_t* mask,
                        void* workspace, size_t workspace_bytes, void* stream) {
  dash_status s = check_decode_params(p);
  if (s != DASH_OK) return s;
  return decode_common(p, q, kc, vc, kbar, nullptr, 0, o, lse, nsel, tau, mask, workspace, workspace_bytes, stream);
}

size_t dash_decode_static_max_bytes(void) { return kStaticScratchBytes; }

dash_status dash_decode_static(const dash_decode_params* p, const void* q, const void* kc, const void* vc,
                               const void* kbar, void* o, float* lse, int32_t* nsel, float* tau, uint32_t* mask,
                               void* stream) {
  dash_status s = check_decode_params(p);
  if (s != DASH_OK) return s;
  size_t off[5];
  const size_t need = decode_ws_layout(p, off, nullptr, nullptr);
  if (need > kStaticScratchBytes)
    return fail(DASH_EWORKSPACE, "this decode needs %zu bytes of scratch; the static scratch holds %zu "
                "(use dash_decode with a workspace)", need, kStaticScratchBytes);
  if (!ok_ptr(q) || !ok_ptr(kc) || !ok_ptr(vc) || !ok_ptr(kbar) || !ok_ptr(o))
    return fail(DASH_EINVAL, "q, kc, vc, kbar and o must be non-null and 16-byte aligned");
  if (!ok_opt(lse) || !ok_opt(nsel) || !ok_opt(tau) || !ok_opt(mask))
    return fail(DASH_EINVAL, "lse/nsel/tau/mask must be 16-byte aligned");
  hipError_t e;
  void* ws = static_scratch(&e);
  if (!ws) return hip_fail(e, "static scratch address");
  return decode_common(p, q, kc, vc, kbar, nullptr, 0, o, lse, nsel, tau, mask, ws, need, stream);
}

dash_status dash_decode_gqa(const dash_decode_params* p, int32_t kv_heads, const void* q, const void* kc,
                            const void* vc, const void* kbar, const int32_t* len, void* o, float* lse,
                            int32_t* nsel, float* tau, uint32_t* mask, void* workspace, size_t workspace_bytes,
                            void* stream) {
  dash_status s = check_decode_params(p);
  if (s != DASH_OK) return s;
  if (kv_heads < 1 || p->H % kv_heads) return fail(DASH_EINVAL, "kv_heads (%d) must divide H (%d)", kv_heads, p->H);
  const int grp = p->H / kv_heads;
  if (grp != 1 && grp != 2 && grp != 4 && grp != 8)
    return fail(DASH_EUNSUPPORTED, "1, 2, 4 or 8 query heads per KV head are built (got %d)", grp);
  if (len && reinterpret_cast<uintptr_t>(len) % 4) return fail(DASH_EINVAL, "len must be 4-byte aligned");
  return decode_common(p, q, kc, vc, kbar, len, 0, o, lse, nsel, tau, mask, workspace, workspace_bytes, stream, grp);
}

dash_status dash_cache_append(const dash_decode_params* p, const void* k_new, const void* v_new,
                              const int32_t* len, void* kc, void* vc, void* kbar, void* stream) {
  dash_status s = check_decode_params(p);
  if (s != DASH_OK) return s;
  return append_common(p, k_new, v_new, len, kc, vc, kbar, stream);
}

dash_status dash_decode_varlen(const dash_decode_params* p, const void* q, const void* kc, const void* vc,
                               const void* kbar, const int32_t* len, void* o, float* lse, int32_t* nsel,
                               float* tau, uint32_t* mask, void* workspace, size_t workspace_bytes, void* stream) {
  dash_status s = check_decode_params(p);
  if (s != DASH_OK) return s;
  if (!len || reinterpret_cast<uintptr_t>(len) % 4) return fail(DASH_EINVAL, "len must be non-null and 4-byte aligned");
  return decode_common(p, q, kc, vc, kbar, len, 0, o, lse, nsel, tau, mask, workspace, workspace_bytes, stream);
}

dash_status dash_decode_step(const dash_decode_params* p, const void* q, const void* k_new, const void* v_new,
                             const int32_t* len, void* kc, void* vc, void* kbar, void* o, float* lse,
                             int32_t* nsel, float* tau, uint32_t* mask, void* workspace, size_t workspace_bytes,
                             void* stream) {
  dash_status s = check_decode_params(p);
  if (s != DASH_OK) return s;
  // validate both halves before launching either
  if (!ok_ptr(q) || !ok_ptr(o)) return fail(DASH_EINVAL, "q and o must be non-null and 16-byte aligned");
  if (!ok_opt(lse) || !ok_opt(nsel) || !ok_opt(tau) || !ok_opt(mask))
    return fail(DASH_EINVAL, "lse/nsel/tau/mask must be 16-byte aligned");
  size_t off[5];
  if (workspace_bytes < decode_ws_layout(p, off, nullptr, nullptr))
    return fail(DASH_EWORKSPACE, "workspace of %zu bytes needed, %zu given", decode_ws_layout(p, off, nullptr, nullptr),
                workspace_bytes);
  if (!ok_ptr(workspace)) return fail(DASH_EINVAL, "workspace must be non-null and 16-byte aligned");
  if ((s = append_common(p, k_new, v_new, len, kc, vc, kbar, stream)) != DASH_OK) return s;
  // rows whose length was out of range for the append (len < 0 or >= N)
  // are out of range here too (len + 1 < 1 or > N): NaN outputs
  return decode_common(p, q, kc, vc, kbar, len, 1, o, lse, nsel, tau, mask, workspace, workspace_bytes, stream);
}

}  // extern "C"
