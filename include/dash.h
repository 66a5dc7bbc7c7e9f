/*
 * dash.h -- C ABI of the DashAttention hot path for AMD Instinct MI355X (gfx950).
 *
 * The method (DashAttention pages: "DashAttention: Making Sparse Attention Fully
 * Differentiable with Adaptive Block Selection", sections "Core Mechanism" and
 * "Key Concepts"; "DashAttention and the year sparse attention became a field",
 * section "What alpha-entmax changes"):
 *
 *   Stage 0  kbar_b = mean of the 64 keys of block b (the zero-initialised
 *            summariser starts from mean pooling);
 *   Stage 1  z_ib = coarse_scale * q_i . kbar_b for the candidate blocks of
 *            query i, p_i = alpha-entmax(z_i): u = (alpha-1) z,
 *            p_b = [u_b - tau_i]_+^(1/(alpha-1)), sum_b p_b = 1 (alpha = 1:
 *            softmax); blocks with p_ib = 0 are dropped;
 *   Stage 2  one softmax over the tokens j of the selected blocks of
 *            l_ij = fine_scale * q_i . k_j + log p_{i,blk(j)}, O_i = sum a_ij v_j.
 *
 * Conventions taken where the pages are silent:
 *   - causal: the candidates of query i are the blocks strictly before its own
 *     block; its own block is always attended with the causal mask (j <= i)
 *     and log-prior 0; non-causal: every block is a candidate;
 *   - kbar is the exact mean rounded once (to nearest even) to the tensor dtype;
 *   - decode: the new token is the last cached token (position N-1), so decode
 *     equals the last row of a causal prefill over the cache.
 *
 * Memory: every pointer is a DEVICE pointer owned by the caller.  The library
 * never allocates, frees or synchronises; all work is enqueued on `stream`
 * (a hipStream_t passed as void*, NULL = the default stream).  Tensors are
 * dense and contiguous, layout [B, H, T, D] (row-major, D fastest) for
 * q/k/v/o/dout/dq/dk/dv, [B, H, T/64, D] for kbar/dkbar.  Element type is
 * dash_params.dtype (bf16 or fp32); lse, tau, lognorm and dkbar are fp32.
 * Pointers must be 16-byte aligned.
 *
 * Errors: arguments are validated on the host before anything is launched, so
 * a call that returns an error has enqueued no work.  DASH_EHIP reports a
 * launch failure.  dash_last_error() returns a thread-local message for the
 * last failing call on the calling thread.
 *
 * Determinism: forward, decode and backward results do not depend on
 * scheduling (no floating-point atomics; the integer atomics that build the
 * low-density schedule's lists order work, not sums).
 */
#ifndef DASH_H
#define DASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DASH_OK = 0,
  DASH_EINVAL = 1,        /* null/misaligned pointer, bad shape, alpha or scale */
  DASH_EUNSUPPORTED = 2,  /* valid but not built: D not in {64,128}, block != 64, T too long */
  DASH_EWORKSPACE = 3,    /* workspace smaller than the *_workspace_bytes() result */
  DASH_EHIP = 4           /* a HIP launch failed; see dash_last_error() */
} dash_status;

typedef enum { DASH_F32 = 0, DASH_BF16 = 1 } dash_dtype;

/* Prefill / training shapes and hyper-parameters. */
typedef struct {
  int32_t B, H, T, D;   /* batch, heads, sequence length (<= 98304; a multiple of 64 except as
                           below), head dim (64|128) */
  int32_t block;        /* keys per block; must be 64 */
  float alpha;          /* entmax alpha in [1, 2] */
  int32_t causal;       /* 0 or 1 */
  float fine_scale;     /* scale of q.k in Stage 2 (usually 1/sqrt(D)); finite, > 0 */
  float coarse_scale;   /* scale of q.kbar in Stage 1; finite, > 0 */
  int32_t dtype;        /* dash_dtype of q, k, v, o, kbar, dout, dq, dk, dv */
} dash_params;

/*
 * Stage-1 selection, written by dash_fwd and read by dash_bwd.  All buffers are
 * caller-owned device memory; sizes (in elements) come from dash_sel_sizes().
 * nb = T/64, nbw = ceil(nb/32), ntile = ceil(T/dash_query_tile()).  With a
 * partial last block (see dash_fwd) T here means 64 ceil(T/64): rows past
 * the sequence are padding.
 *   tau      [B,H,T]        f32  entmax threshold (u-units for alpha>1, z-units
 *                                (log-sum-exp) for alpha=1; NaN when the row has
 *                                no candidate block)
 *   lognorm  [B,H,T]        f32  log of sum_b [u_b - tau]_+^(1/(alpha-1)) (about 0)
 *   nsel     [B,H,T]        i32  number of selected candidate blocks (may be NULL)
 *   mask     [B,H,T,nbw]    u32  bit b set iff block b is a selected candidate (may be NULL)
 *   tile_cnt [B,H,ntile]    i32  length of each query tile's block list
 *   tile_blk [B,H,ntile,nb] i32  ascending blocks the tile must visit: the union of its
 *                                rows' selected blocks plus, when causal, the tile's own
 *                                blocks
 *   tile_bits[B,H,ntile,nbw]u32  the same set as a bit mask
 *   passes   [B,H,T]        i32  passes over the row's scores the threshold solve took
 *                                (may be NULL; 0 for rows without candidates)
 */
typedef struct {
  float* tau;
  float* lognorm;
  int32_t* nsel;
  uint32_t* mask;
  int32_t* tile_cnt;
  int32_t* tile_blk;
  uint32_t* tile_bits;
  int32_t* passes;
} dash_sel;

/* Query rows per Stage-2 tile (the granularity of tile_cnt / tile_blk). */
int32_t dash_query_tile(void);

/* Element counts of the eight dash_sel buffers, in struct order. */
dash_status dash_sel_sizes(const dash_params* p, size_t out_elems[8]);

/*
 * Bytes of device workspace dash_fwd / dash_bwd need (dash_fwd: always 0;
 * a larger one lets it take the low-density schedule, see
 * dash_fwd_attend_lowdens).
 * dash_bwd's grows with T^2: besides O(B H T D) fp32 buffers it keeps, per
 * (query tile, list slot, row), G and the log2 prior as fp32, with room for
 * every slot a tile's list can hold: min(T/64, 2t + 2) for causal tile t
 * (the lower triangle), T/64 when not causal.  Causal, that is about
 * B H T^2 / 64 floats for each of the two: 541 MB in all at B2 H16 T16384,
 * 8.6 GB at B1 H32 T65536.
 */
size_t dash_fwd_workspace_bytes(const dash_params* p);
size_t dash_bwd_workspace_bytes(const dash_params* p);

/*
 * Stage 0 alone: kbar[B,H,T/64,D] = mean of each 64-key block of k[B,H,T,D],
 * accumulated in fp64 and rounded once to dtype.  (Stage 0 of the pages,
 * "What alpha-entmax changes"; used to build the summaries of a decode cache.)
 * Any T that is a multiple of 64 is accepted here (no 65536 limit).
 * For bf16 keys the fp64 sum of a block is exact, so it does not depend on
 * the summation order (this kernel, dash_cache_append and a sequential sum
 * agree bit for bit), as long as the block's non-zero magnitudes lie within
 * 2^39 of each other (8 significant bits per value, 6 bits of carry for 64
 * terms, 53 in a double) and the mean is a normal bf16; for keys outside
 * that range the rounding of the mean may depend on the order.
 */
dash_status dash_pool(const dash_params* p, const void* k, void* kbar, void* stream);

/*
 * Forward (Stages 0, 1, 2).  Inputs q, k, v.  Outputs: o [B,H,T,D] (dtype),
 * lse [B,H,T] (f32, log-sum-exp of the Stage-2 logits, for the backward),
 * kbar [B,H,T/64,D] (dtype) and the selection `sel`.
 *
 * dash_fwd and dash_bwd also take a causal T that is not a multiple of 64
 * (the other prefill entry points do not): the last block is partial; it is
 * the own block of its queries and no query's candidate, so only the
 * complete blocks have summaries (kbar and dkbar have ceil(T/64) rows; the
 * last one is not a summary, and dkbar's is 0).  dash_fwd's kernels take
 * the T-row tensors as they are and treat the missing rows of the last
 * block as zeros, never reading or writing past the tensors (its workspace
 * is 0 bytes; workspace may be NULL); dash_bwd runs the whole-block kernels
 * on copies padded with zeros in its workspace (dash_bwd_workspace_bytes)
 * and copies the T rows back.  The results are those of the unpadded
 * problem.  Non-causal attention needs whole blocks.
 */
dash_status dash_fwd(const dash_params* p, const void* q, const void* k, const void* v,
                     void* o, float* lse, void* kbar, const dash_sel* sel,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Stage 2 at low selection density (the AdaSplash-2 abstract on the
 * thelatestinai.com page: a sparsity-aware implementation that skips the
 * zero blocks at low cost).  The dense walk runs each 128-row query tile over
 * the union of its rows' blocks with all 128 rows; when the rows of a tile
 * select few, different blocks that union holds nearly every candidate and
 * most of the products are thrown away.  This schedule instead lists, for
 * every key block, the rows that selected it (plus, causal, its own 64 rows),
 * computes each (row, block) pair's partial softmax with those rows as the
 * MFMA columns over one LDS copy of the block's keys and values, and merges
 * each row's partials in block order.  The result is the same attention
 * (outputs within bf16 rounding of dash_fwd_attend's; the partials' weighted
 * values are kept in bf16), and deterministic: integer atomics only order
 * the lists, not the arithmetic.
 *
 * Per call, on the device: a query tile takes this schedule when the dense
 * walk would visit more than `ratio` times the (row, block) pairs its rows
 * need (list length x rows > ratio x sum over rows of (selected + 1)), as
 * long as the pairs of the qualifying tiles up to it, in head-major tile
 * order, fit in the workspace; every other tile takes the dense walk in the
 * same call.  ratio 0 sends every tile that fits here.
 *
 * Causal, bf16, whole blocks (T a multiple of 64), one KV head per query head;
 * sel must hold the masks (sel->mask written by dash_fwd_select with the same
 * params) besides what dash_fwd_attend reads.  Other cases return
 * DASH_EUNSUPPORTED.  Workspace: dash_fwd_lowdens_workspace_bytes(p, pairs)
 * for room for `pairs` pairs (B H T of them are the own blocks; the rest is
 * the sum of the rows' selected counts, sel->nsel); at least the value for
 * 0 pairs (then every tile takes the dense walk), else DASH_EWORKSPACE.  Per
 * pair it holds 20 + 2 D bytes; the fixed part is about
 * B H (8 T + 4 (T/64)^2) bytes (about 10 MB per head at T = 98304).
 *
 * dash_fwd takes the same schedule, with ratio DASH_LOWDENS_RATIO, when its
 * workspace holds at least one pair beyond that fixed part and the case is
 * supported (mask non-null); with no workspace it takes the dense walk.
 */
#define DASH_LOWDENS_RATIO 4.0f
size_t dash_fwd_lowdens_workspace_bytes(const dash_params* p, int64_t max_pairs);
dash_status dash_fwd_attend_lowdens(const dash_params* p, const void* q, const void* k, const void* v,
                                    const void* kbar, const dash_sel* sel, float ratio, void* o,
                                    float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two halves of dash_fwd, for callers that reuse a selection or time the
 * stages apart.  dash_fwd_select runs Stages 0 and 1 (kbar and `sel`);
 * dash_fwd_attend runs Stage 2 from q, k, v, kbar and a selection written by
 * dash_fwd_select with the same params (o and lse).  Same validation and
 * error behaviour as dash_fwd.
 */
dash_status dash_fwd_select(const dash_params* p, const void* q, const void* k, void* kbar,
                            const dash_sel* sel, void* stream);
dash_status dash_fwd_attend(const dash_params* p, const void* q, const void* k, const void* v,
                            const void* kbar, const dash_sel* sel, void* o, float* lse, void* stream);

/*
 * Backward of the scalar <dout, O>: gradients through Stage 2, log p, the
 * alpha-entmax Jacobian (s = p^(2-alpha), dz = s*(g - <s,g>/sum s), g = dL/dp),
 * the block scores and mean pooling.  Inputs are the forward's q, k, v, o, lse,
 * kbar and sel plus dout.  Outputs dq, dk, dv (dtype; dk includes the pooling
 * path dkbar/64) and dkbar [B,H,T/64,D] (f32, gradient w.r.t. the summaries).
 * The rounding of kbar to dtype is treated as the identity.
 */
dash_status dash_bwd(const dash_params* p, const void* q, const void* k, const void* v,
                     const void* o, const float* lse, const void* dout, const void* kbar,
                     const dash_sel* sel, void* dq, void* dk, void* dv, float* dkbar,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * The learned Stage-0 summariser (the montana-research page, "What
 * alpha-entmax changes": each chunk is summarised by a small learned
 * attention head initialised at zero, so training starts from mean pooling).
 * The head is one vector per attention head, w [H, D] (f32).  For block b:
 * e_j = w[h] . k_j over the block's 64 keys, a = softmax(e), kbar_b =
 * sum_j a_j k_j, in fp64, rounded once to dtype.  At w = 0 this equals
 * dash_pool bit for bit.  Any T that is a multiple of 64; D <= 128.
 */
dash_status dash_pool_attn(const dash_params* p, const void* k, const float* w, void* kbar, void* stream);

/*
 * Stage 1 alone, from summaries the caller already holds in kbar (for
 * example dash_pool_attn's): writes the selection `sel` exactly as
 * dash_fwd_select does after its pooling.  Same validation.
 */
dash_status dash_select(const dash_params* p, const void* q, const void* kbar, const dash_sel* sel,
                        void* stream);

/*
 * dash_bwd without the Stage-0 term: dk holds the gradient through Stage 2
 * only (the mean-pooling share dkbar/64 is not added); every other output
 * is as dash_bwd.  For summaries that did not come from mean pooling: add
 * their own Stage-0 gradient afterwards (dash_pool_attn_bwd).
 */
dash_status dash_bwd_no_pool(const dash_params* p, const void* q, const void* k, const void* v,
                             const void* o, const float* lse, const void* dout, const void* kbar,
                             const dash_sel* sel, void* dq, void* dk, void* dv, float* dkbar,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of dash_pool_attn (its rounding taken as the identity): with
 * g = dkbar[b,h,blk,:] (f32, as dash_bwd writes it) and c_j = k_j.g - kbar.g
 * (kbar before rounding), adds a_j g + a_j c_j w[h] to dk (dtype, in place:
 * dk already holds the other gradient terms, e.g. from dash_bwd_no_pool) and
 * writes dw [H, D] (f32) = the sum over batch and blocks of a_j c_j k_j.
 * Workspace: dash_pool_attn_bwd_workspace_bytes (per-block partials of dw,
 * reduced in a fixed order, so the result is deterministic).
 */
size_t dash_pool_attn_bwd_workspace_bytes(const dash_params* p);
dash_status dash_pool_attn_bwd(const dash_params* p, const void* k, const float* w, const float* dkbar,
                               void* dk, float* dw, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * The whole backward with the learned summariser: dash_bwd_no_pool, then
 * dash_pool_attn_bwd, except that for bf16 the other dK terms stay
 * unrounded (fp32, in the workspace) until the summariser's term is added,
 * so dk is rounded once (at w = 0 it equals dash_bwd's dk bit for bit).
 * Outputs as dash_bwd plus dw [H, D] (f32).  Workspace:
 * dash_bwd_learned_workspace_bytes (the backward's, B*H*T*D floats, and
 * dash_pool_attn_bwd's).  Whole blocks only.
 */
size_t dash_bwd_learned_workspace_bytes(const dash_params* p);
dash_status dash_bwd_learned(const dash_params* p, const void* q, const void* k, const void* v,
                             const void* o, const float* lse, const void* dout, const void* kbar,
                             const dash_sel* sel, const float* w, void* dq, void* dk, void* dv,
                             float* dkbar, float* dw, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * Grouped-query heads with entmax head aggregation.  p->H query heads share
 * kv_heads key/value heads (kv_heads divides H; query head h uses KV head
 * h / (H / kv_heads), the expansion of a repeat_kv step, which the
 * codewithpapers.app entry for the DashAttention paper lists in its prefill
 * block selection).  The montana-research page ("Non-dispersive attention at
 * long context") calls entmax head aggregation non-dispersive; here it is:
 * every query head gets its own alpha-entmax p_h over its KV head's
 * summaries, the G = H / kv_heads heads of a group share pbar = (1/G) sum_h
 * p_h, and each attends the blocks of pbar's support (the union of the
 * heads' supports) with prior log pbar.
 *
 * k, v: [B, kv_heads, T, D]; kbar: [B, kv_heads, T/64, D] (written); q, o:
 * [B, H, T, D]; lse [B, H, T]; `sel` as for H heads: tau, lognorm, nsel and
 * mask are each head's own entmax, the tile lists the group's union.
 * kv_heads == H is the per-head method (dash_fwd).  bf16 only when
 * kv_heads < H.
 */
dash_status dash_fwd_gqa(const dash_params* p, int32_t kv_heads, const void* q, const void* k,
                         const void* v, void* o, float* lse, void* kbar, const dash_sel* sel,
                         void* stream);

/*
 * Backward of dash_fwd_gqa: dq [B, H, T, D]; dk, dv [B, kv_heads, T, D] (the
 * sums over each group's query heads, dk with the mean-pooling path);
 * dkbar [B, kv_heads, T/64, D] f32.  G_b, the gradient of log pbar_b, sums
 * the group's heads; each head's p_h then takes its own entmax Jacobian with
 * dL/dp_h = G / (G_heads pbar).  Workspace: dash_bwd_gqa_workspace_bytes.
 */
size_t dash_bwd_gqa_workspace_bytes(const dash_params* p, int32_t kv_heads);
dash_status dash_bwd_gqa(const dash_params* p, int32_t kv_heads, const void* q, const void* k,
                         const void* v, const void* o, const float* lse, const void* dout,
                         const void* kbar, const dash_sel* sel, void* dq, void* dk, void* dv,
                         float* dkbar, void* workspace, size_t workspace_bytes, void* stream);

/* Decode shapes: S sequences x H heads, one new query each, cache length N. */
typedef struct {
  int32_t S, H, N, D;   /* N multiple of 64, 64 <= N <= 131072; D = 128 (bf16 only) */
  int32_t block;        /* must be 64 */
  float alpha;
  float fine_scale;
  float coarse_scale;
  int32_t dtype;
} dash_decode_params;

size_t dash_decode_workspace_bytes(const dash_decode_params* p);

/*
 * Decode (the pages' decoding path; speed claim at 96K context in "The
 * numbers").  q [S,H,D]; caches kc, vc [S,H,N,D] with the new token at N-1;
 * kbar [S,H,N/64,D] the summaries of the cache (dash_pool).  Candidates are
 * blocks 0..N/64-2; block N/64-1 is attended whole with prior 0.
 * Outputs o [S,H,D] (dtype), lse [S,H] (f32, may be NULL), nsel [S,H] (i32,
 * may be NULL), tau [S,H] (f32, may be NULL) and mask [S,H,nbw] (u32, may be
 * NULL; nbw = ceil(N/64/32)): the Stage-1 output of the row, its sparse
 * block weights' support ("Core Mechanism" of the alanhou.org page), bit
 * b % 32 of word b / 32 set iff candidate block b has p > 0; bits of the
 * query's own block and of later blocks are 0.
 */
dash_status dash_decode(const dash_decode_params* p, const void* q, const void* kc,
                        const void* vc, const void* kbar, void* o, float* lse,
                        int32_t* nsel, float* tau, uint32_t* mask, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * dash_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same decode, its workspace taken from a scratch array of
 * dash_decode_static_max_bytes() bytes (32 MiB) that the library holds in
 * device memory, one per GPU, until the process ends.  The call allocates
 * and frees nothing.  Arguments and outputs as dash_decode, without the
 * workspace.  Sizes whose dash_decode_workspace_bytes() exceeds the scratch
 * (more than 736 rows at a 98304-token cache, 675 at 131072) return DASH_EWORKSPACE
 * with nothing launched.  Every call on one GPU uses that GPU's one scratch:
 * calls that overlap on a GPU (other streams, other host threads) race and
 * must be serialised by the caller.  Nothing in the scratch needs to start
 * at zero: each call writes every entry it reads.  The first call on a
 * device looks up the scratch's address there (with that device current).
 */
size_t dash_decode_static_max_bytes(void);
dash_status dash_decode_static(const dash_decode_params* p, const void* q, const void* kc,
                               const void* vc, const void* kbar, void* o, float* lse,
                               int32_t* nsel, float* tau, uint32_t* mask, void* stream);

/*
 * Decode cache maintenance and caches of any length (the decoding path keeps
 * one summary per 64-token chunk of the cache: the chunk-summarise stage
 * among the code samples that the codewithpapers.app entry "DashAttention:
 * Differentiable and Adaptive Sparse Hierarchical Attention" lists).
 *
 * In the three calls below p->N is the cache CAPACITY C (a multiple of 64,
 * 64 <= C <= 131072): kc, vc are [S,H,C,D], kbar [S,H,C/64,D], all dtype.
 * len is a DEVICE array of S int32: the number of tokens sequence s holds.
 * The library only reads len; the caller advances it.  Values are checked
 * on the device, not the host: a sequence whose length is out of range gets
 * the behaviour stated for each call, and no memory outside the caches is
 * touched.
 */

/*
 * Append one token per (sequence, head): kc[s,h,len[s],:] = k_new[s,h,:] and
 * vc likewise (k_new, v_new [S,H,D]).  When position len[s] is the last of
 * its block (len[s] % 64 == 63), that block is complete and
 * kbar[s,h,len[s]/64,:] becomes the mean of its 64 keys, summed in fp64 and
 * rounded once, bit-identical to dash_pool.  Summaries of incomplete blocks
 * are not written; for a cache filled by a prefill, dash_pool over the
 * whole capacity (T = C) gives the complete blocks' summaries, and the
 * entries of incomplete ones are ignored until an append completes them.
 * A sequence with len[s] < 0 or len[s] >= C is left unchanged.
 */
dash_status dash_cache_append(const dash_decode_params* p, const void* k_new, const void* v_new,
                              const int32_t* len, void* kc, void* vc, void* kbar, void* stream);

/*
 * Decode with a length per sequence: sequence s holds n = len[s] tokens, the
 * new one (whose query is q[s,h]) at position n-1, already appended.  The
 * result is row n-1 of a causal prefill over the first n tokens: candidates
 * are the complete blocks 0..(n-1)/64-1, and the query's own block is
 * attended over its n - 64*((n-1)/64) cached tokens with prior 0.  Cache
 * entries at positions >= n and summaries of blocks >= (n-1)/64 are never
 * read.  Outputs as dash_decode (mask words over the capacity's C/64
 * blocks); a sequence with len[s] < 1 or len[s] > C gets o = NaN,
 * lse = NaN, nsel = -1, tau = NaN and an all-zero mask.  Workspace: as
 * dash_decode for the same params.
 */
dash_status dash_decode_varlen(const dash_decode_params* p, const void* q, const void* kc,
                               const void* vc, const void* kbar, const int32_t* len, void* o,
                               float* lse, int32_t* nsel, float* tau, uint32_t* mask,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * One serving step: dash_cache_append of (k_new, v_new) at len[s], then
 * dash_decode_varlen over len[s] + 1 tokens, in stream order.  len is not
 * advanced.  Same outputs and workspace as dash_decode_varlen; a sequence
 * with len[s] < 0 or len[s] >= C is neither appended nor decoded (NaN
 * outputs, nsel = -1).
 */
dash_status dash_decode_step(const dash_decode_params* p, const void* q, const void* k_new,
                             const void* v_new, const int32_t* len, void* kc, void* vc, void* kbar,
                             void* o, float* lse, int32_t* nsel, float* tau, uint32_t* mask,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode for grouped-query heads (entmax head aggregation, as dash_fwd_gqa):
 * p->H query heads share kv_heads key/value heads (H / kv_heads is 1, 2, 4
 * or 8).  q [S,H,D]; kc, vc [S,kv_heads,N,D] and
 * kbar [S,kv_heads,N/64,D] (N the capacity); len: NULL (every cache full,
 * the new token at N-1) or device lengths as dash_decode_varlen.  Each query
 * head gets its own alpha-entmax over its KV head's summaries; the group
 * attends the blocks of pbar = the mean of the heads' p, with prior
 * log pbar, and its own block (prior 0).  The heads of a group walk the same
 * blocks together, so a block is read from HBM once per group.  Outputs
 * o, lse [S,H], nsel, tau and mask (each head's own entmax support; the
 * group walks the OR of its heads' masks plus the own block) as
 * dash_decode; workspace as dash_decode with the same params.
 */
dash_status dash_decode_gqa(const dash_decode_params* p, int32_t kv_heads, const void* q,
                            const void* kc, const void* vc, const void* kbar, const int32_t* len,
                            void* o, float* lse, int32_t* nsel, float* tau, uint32_t* mask,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Message of the last failing call on this thread ("" if none). */
const char* dash_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DASH_H */
