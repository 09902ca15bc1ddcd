/*
 * speed3r.h - C ABI of the MI355X (gfx950) sparse global attention library (libspeed3r.so).
 *
 * The library computes the forward pass of Speed3R's dual-branch global sparse attention
 * (Speed3R technical summary on gist.science, "Methodologie" section 1, dual-branch attention,
 * and section 2, gated aggregation; Speed3R README, "Overview"):
 *
 *   compression branch   Kc_j, Vc_j = means of the keys / values of contiguous block j
 *                        (B tokens; the last block may be shorter);
 *                        P_tj = softmax_j(scale * q_t . Kc_j), O_cmp_t = sum_j P_tj Vc_j;
 *                        Score[h][i][j] = sum over the queries t of query block i of P_tj.
 *   selection branch     Sel[h][i] = the k blocks with the largest Score[h][i][.] (ties: the
 *                        smaller block index wins; stored in ascending order);
 *                        O_sel_t = softmax attention of q_t over the tokens of those blocks.
 *   gated aggregation    out_t = g[h][0] * O_cmp_t + g[h][1] * O_sel_t.
 *
 * Conventions shared by every entry point
 *   - Token tensors q, k, v are bf16 or fp16 (params.dtype) [T][H][D] with D = 64
 *     contiguous, and out has their type; token and head strides
 *     are given in elements and must be multiples of 8 (16-byte rows); base pointers must be
 *     16-byte aligned. Query blocks and key blocks both have size B = params.block.
 *   - Numerics: logits are products of the input type accumulated in f32 (the pooled keys as a
 *     hi + lo pair of the input type); softmax runs in f32 with base-2 exponentials; the P.V
 *     products take fp16 operands with f32 accumulation. bf16 values of v are held as fp16
 *     after multiplying by 2^-8 (the outputs are multiplied back), which represents every
 *     bf16 value below 65504 * 2^8 (about 1.68e7) in magnitude, exactly from 2^-6 up and
 *     within 2^-17 below; fp16 values are held as they are. A bf16 value of v at or beyond
 *     that limit becomes an infinity in its fp16 record, and every output that attends to it
 *     is non-finite (never a wrong finite number).
 *   - Every pointer is device memory owned by the caller; the library never allocates, frees
 *     or synchronises. All work is enqueued on `stream` (NULL = the default stream) and the
 *     call returns before it completes. Asynchronous faults surface at the caller's next
 *     synchronisation.
 *   - Arguments are validated before anything is launched; on any error nothing is launched
 *     and no output is touched.
 *   - The library keeps no state between calls and may be called from several threads.
 *     Calls that share a workspace must be ordered by the caller (same stream).
 */
#ifndef SPEED3R_H
#define SPEED3R_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  S3R_OK = 0,
  S3R_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, negative forced_blocks, bad
                              stride or alignment */
  S3R_ERR_UNSUPPORTED = 2, /* well-formed but not built: D != 64, B not 16/32/64/128,
                              H > 65535, T >= 2^31, or more than 24576 blocks where the
                              separate top-k kernel is needed (speed3r_topk, and B = 128 or
                              more than 64 chosen blocks) */
  S3R_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the size query returns */
  S3R_ERR_HIP = 4,         /* a kernel launch failed (hipGetLastError) */
  S3R_ERR_SCRATCH = 5      /* speed3r_sparse_attn_fwd_noalloc: the problem needs more than
                              speed3r_noalloc_scratch_bytes() of workspace */
} s3r_status;

/* Element type of q, k, v and out. The model runs in bf16 or fp16 (README "Notice" 3). */
typedef enum { S3R_BF16 = 0, S3R_FP16 = 1 } s3r_dtype;

/* How the compression branch's softmax is normalised (params.cmp_mode); every mode gives the
 * same results up to rounding, and the same selection except between blocks whose scores
 * agree to rounding.
 *   S3R_CMP_TWO_PASS  pass 1 computes each query's log-sum-exp, pass 2 the probabilities,
 *                     O_cmp and the scores (speed3r_cmp_lse, then speed3r_cmp_fused[_topk]).
 *   S3R_CMP_SINGLE    one pass from a cheap lower bound of the log-sum-exp
 *                     (speed3r_cmp_lse_bound, then speed3r_cmp_single_topk), with the two
 *                     exact passes rerun where its check fails. Needs the folded selection
 *                     (B <= 64, n_sel - F' <= 64) and Nb >= 8; S3R_ERR_UNSUPPORTED otherwise.
 *   S3R_CMP_AUTO      (0) the single pass where it applies and k <= 48 (or every candidate
 *                     block fits its list of 64), the two passes otherwise. */
typedef enum { S3R_CMP_AUTO = 0, S3R_CMP_TWO_PASS = 1, S3R_CMP_SINGLE = 2 } s3r_cmp_mode;

typedef struct {
  int64_t T;            /* number of tokens (all views concatenated), >= 1 */
  int32_t H;            /* number of heads, >= 1 */
  int32_t D;            /* head width; must be 64 */
  int32_t block;        /* B: query and key block size, one of 16, 32, 64, 128 */
  int32_t topk;         /* k >= 1: key blocks kept per query block; clamped to Nb */
  float scale;          /* softmax scale; 0 selects 1/sqrt(D) */
  int32_t forced_blocks; /* F >= 0: key blocks 0..F-1 are selected for every query block in
                            addition to the top-k of the remaining blocks (the VGGT variant
                            keeps the reference frame's tokens dense, summary "Methodologie"
                            3). 0 = plain top-k */
  int64_t q_stride_t, q_stride_h; /* element strides of q between tokens / heads */
  int64_t k_stride_t, k_stride_h;
  int64_t v_stride_t, v_stride_h;
  int64_t gate_stride_t; /* 0: gates are [H][2]; otherwise per-token gates with
                            gate(t, h, b) = gates[t * gate_stride_t + h * 2 + b] */
  int32_t dtype;        /* s3r_dtype of q, k, v and out; 0 (zero-initialised) is bf16 */
  int32_t force_own;    /* nonzero: every query block also keeps its own key block (after the
                           forced prefix; top-k then runs over the remaining blocks) */
  int32_t cmp_mode;     /* s3r_cmp_mode; 0 (zero-initialised) is automatic */
} s3r_params;

/* Human-readable name of a status code (static storage); any other int gives
 * "S3R_ERR_UNKNOWN". The code is taken as an int so that a value outside the enumeration is
 * well defined. */
const char* speed3r_status_string(int status);

/* Nb = ceil(T / B), the number of key blocks (= query blocks). -1 if p is invalid. */
int64_t speed3r_num_blocks(const s3r_params* p);

/* Entries per selection row: n_sel = F' + o + min(k, Nb - F' - o) with F' = min(forced_blocks,
 * Nb) and o = 1 when force_own is set and F' < Nb. Rows hold the forced blocks 0..F'-1 and the
 * chosen ones (with the query block's own block when force_own), ascending; a row whose own
 * block is already forced holds one block fewer and ends with -1. -1 if p is invalid. */
int64_t speed3r_num_selected(const s3r_params* p);

/* Row stride (in floats) of the score matrix [H][Nb][ld]: Nb rounded up to 32. -1 if invalid. */
int64_t speed3r_score_row_stride(const s3r_params* p);

/* Bytes of workspace the per-stage entry points need (packed tiles of the pooled keys and
 * values, of the group keys of the bound pass, and of the raw keys and values, plus the
 * blocks' f32 column sums [H][Nb][128] that pooling reads). 0 if p is invalid. */
size_t speed3r_tiles_workspace_size(const s3r_params* p);

/* Bytes of workspace speed3r_sparse_attn_fwd needs: the tiles plus LSE [H][T] f32, O_cmp
 * [T][H][64] f32, the selected indices, the redo flags when the forward pass runs the single
 * compression pass and, only when the selection cannot be folded into the compression pass
 * (B = 128 or more than 64 chosen blocks), the score matrix [H][Nb][ld] f32. About 11.7 GB
 * at T = 1,374,000, H = 16, B = 64, k = 16. 0 if p is invalid. */
size_t speed3r_workspace_size(const s3r_params* p);

/* Bytes of workspace speed3r_dense_attn_fwd needs (packed raw keys and values). */
size_t speed3r_dense_workspace_size(const s3r_params* p);

/* The whole sparse forward pass (the method of the summary's "Methodologie" sections 1-2):
 * pool -> compressed LSE -> compressed output + block scores -> top-k -> selection attention
 * with the gate-combine epilogue. When B <= 64 and k_eff <= 64 the scores never leave the chip
 * (speed3r_cmp_fused_topk, or the single pass speed3r_cmp_single_topk per params.cmp_mode);
 * otherwise they go through the score matrix and speed3r_topk.
 *   gates    f32, [H][2] or per token (see gate_stride_t); column 0 multiplies the
 *            compression branch, column 1 the selection branch.
 *   out      [T][H][64] of the input type, contiguous.
 *   sel_idx  optional int32 [H][Nb][n_sel] (speed3r_num_selected); NULL keeps it in the
 *            workspace.
 *   workspace / workspace_bytes: at least speed3r_workspace_size(p) bytes, 256-byte aligned.
 */
s3r_status speed3r_sparse_attn_fwd(const s3r_params* p, const void* q, const void* k,
                                   const void* v, const float* gates, void* out,
                                   int32_t* sel_idx, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* Per-stage entry points (the same kernels the fused entry point runs), for per-kernel
 * timing and for feeding one stage with another implementation's intermediate results.
 * `workspace` must hold at least speed3r_tiles_workspace_size(p) bytes and is the one that
 * speed3r_pool filled. */

/* Compression branch, pooling (summary "Methodologie" 1, average pooling of blocks): fills the
 * workspace tiles from k and v (k and v are read once: the raw tiles and each block's column
 * sums come from one pass). k_mean / v_mean (optional, f32 [H][Nb][64]) receive the block means
 * themselves: a sum in f32 (rows added in order within each 32-row tile, then the tiles of the
 * block in order) then an IEEE division by the block's token count. Also writes the group keys
 * that speed3r_cmp_lse_bound reads. */
s3r_status speed3r_pool(const s3r_params* p, const void* k, const void* v, void* workspace,
                        size_t workspace_bytes, float* k_mean, float* v_mean,
                        hipStream_t stream);

/* Compression branch, first pass: lse[h][t] = log sum_j exp(scale * q_t . Kc_j) (natural log,
 * f32 [H][T]). The pooled keys enter as the sum of two terms of the input type (hi + lo) of
 * Kc * scale * log2(e), accumulated in f32. */
s3r_status speed3r_cmp_lse(const s3r_params* p, const void* q, const void* workspace,
                           size_t workspace_bytes, float* lse, hipStream_t stream);

/* Compression branch, second pass (summary "Methodologie" 1: coarse attention and the score
 * matrix that guides selection): P_tj = exp(scale * q_t . Kc_j - lse[h][t]);
 * o_cmp[t][h][:] = sum_j P_tj Vc_j (f32 [T][H][64]); score[(h*Nb + i)*ld + j] = sum over the
 * queries of block i of P_tj (f32, ld = speed3r_score_row_stride; columns >= Nb are
 * written with 0). */
s3r_status speed3r_cmp_fused(const s3r_params* p, const void* q, const void* workspace,
                             size_t workspace_bytes, const float* lse, float* o_cmp,
                             float* score, hipStream_t stream);

/* Compression branch, second pass with the selection folded in (the page's kernel keeps top-k
 * and softmax on chip without materialising the score matrix, summary "Methodologie" 4):
 * computes o_cmp exactly as speed3r_cmp_fused and, instead of the score matrix, keeps the
 * running top-k of each query block while the key blocks stream by, writing sel_idx [H][Nb]
 * [n_sel] in ascending order. The choice equals speed3r_topk applied to the score matrix
 * speed3r_cmp_fused writes, bit for bit. Requires B <= 64 and n_sel - F' <= 64
 * (S3R_ERR_UNSUPPORTED otherwise). */
s3r_status speed3r_cmp_fused_topk(const s3r_params* p, const void* q, const void* workspace,
                                  size_t workspace_bytes, const float* lse, float* o_cmp,
                                  int32_t* sel_idx, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * Single compression pass (an implementation choice of this library, not the page's: the
 * page's method needs each query's log-sum-exp before any probability is final, hence the
 * two passes above; this computes the same O_cmp and selection with one pass over the
 * pooled keys plus one over 1/8 of them).
 * ------------------------------------------------------------------------------------- */

/* Number of int32 flags speed3r_cmp_single_topk writes to `redo`: 4 per 256 queries per head,
 * H * ceil(T / 256) * 4. -1 if p is invalid. */
int64_t speed3r_redo_flag_count(const s3r_params* p);

/* Lower bound of the compression branch's log-sum-exp: with group keys G_g = the mean of
 * pooled keys 8g..8g+7 (g < floor(Nb / 8); the pooling stores them scaled like the pooled
 * keys, as hi + lo pairs of the input type), lse_bound[h][t] = log sum_g 8 exp(scale * q_t .
 * G_g) (f32 [H][T], natural log). Convexity of exp (Jensen) makes each group's term at most
 * the sum of exp over its 8 keys, so the exact value is <= the log-sum-exp of speed3r_cmp_lse.
 * The kernel multiplies the queries by the hi parts of the group keys alone (the scaled keys
 * rounded to the input type), so each logit may move by up to 2^-8 (bf16; fp16: 2^-11) of
 * scale * sum_d |q_d G_gd|; the single pass only needs a value low enough, which its Z check
 * verifies (a bound above the log-sum-exp makes it rerun the exact passes there).
 * S3R_ERR_UNSUPPORTED if Nb < 8. */
s3r_status speed3r_cmp_lse_bound(const s3r_params* p, const void* q, const void* workspace,
                                 size_t workspace_bytes, float* lse_bound, hipStream_t stream);

/* The compression branch in one pass from a lower bound lse_bound of each query's log-sum-exp
 * (any bound works; a loose one only makes the checks below fail more often). Writes what
 * speed3r_cmp_lse and speed3r_cmp_fused_topk write: lse [H][T] (natural log), o_cmp
 * [T][H][64] f32 and sel_idx [H][Nb][n_sel]. lse may be the same buffer as lse_bound.
 *   With weights u_tj = exp(c_tj - lse_bound_t) >= P_tj (c_tj = scale * q_t . Kc_j), one
 *   sweep over the pooled keys accumulates Z_t = sum_j u_tj, O_cmp_t * Z_t and, per key
 *   block, the upper bound U_ij = sum_{t in block i} u_tj of the score Score_ij. Each query
 *   block keeps the 64 candidate blocks of largest bound (all of them if fewer); at the end
 *   lse_t = lse_bound_t + log Z_t, O_cmp_t = (O_cmp_t * Z_t) / Z_t, and the listed blocks are
 *   rescored exactly with that lse (the same logits, on the same matrix instructions) and
 *   ranked by (score desc, index asc).
 *   Checks, per wave of 64 queries: 1 <= Z_t <= 2^15 for each of its queries (the offset was
 *   below lse_t, so every U bounds its Score, and no weight, each at most Z_t, overflowed the
 *   fp16 operands of P.V); and, per query block, the smallest bound in the list times
 *   (1 + 2^-8), plus 2^-17 (the rounding of the fp16 bound sums), over the smallest Z_t of the
 *   block's queries, is below the k-th exact score. Score_ij = sum_t u_tj / Z_t, so no
 *   unlisted block can belong to the top k. redo (int32 [H * ceil(T/256)][4],
 *   speed3r_redo_flag_count entries, 16-byte aligned; one per wave) receives bit 1 where the
 *   first check failed and bit 0 where the second did. Then, in the same call, speed3r_cmp_lse
 *   and speed3r_cmp_fused_topk rerun on the 256 queries around each wave with bit 1, and the
 *   selection part of speed3r_cmp_fused_topk (not O_cmp, which stands) on the waves with bit 0
 *   only, so every output ends as the two exact passes would give it. Requires B <= 64,
 *   n_sel - F' <= 64 and Nb >= 8 (S3R_ERR_UNSUPPORTED otherwise). */
s3r_status speed3r_cmp_single_topk(const s3r_params* p, const void* q, const void* workspace,
                                   size_t workspace_bytes, const float* lse_bound, float* lse,
                                   float* o_cmp, int32_t* sel_idx, int32_t* redo,
                                   hipStream_t stream);

/* Top-k selection (summary "Methodologie" 1, selection guided by the compression scores):
 * sel_idx[(h*Nb + i)*n_sel + a]: the forced blocks 0..F'-1, then the n_sel - F' largest
 * entries of score row (h, i) among blocks F'..Nb-1 by (value descending, index ascending),
 * in ascending order. Bit-exact, deterministic. Scores are compared as f32 (-0 equals +0). */
s3r_status speed3r_topk(const s3r_params* p, const float* score, int32_t* sel_idx,
                        hipStream_t stream);

/* Selection branch plus gated aggregation (summary "Methodologie" 1 selection branch and 2
 * gated aggregation): for every query of block i, softmax attention over the tokens of the
 * blocks sel_idx[h][i][0..k_eff), then out = g0 * o_cmp + g1 * O_sel rounded to the input type
 * [T][H][64]. Rows are read in order; an index outside [0, Nb) or equal to the previous index
 * of its row is skipped, so an ascending row (as speed3r_topk writes) attends to the union of
 * its blocks. o_sel (optional, f32 [T][H][64]) receives O_sel itself. */
s3r_status speed3r_sel_combine(const s3r_params* p, const void* q, const void* workspace,
                               size_t workspace_bytes, const int32_t* sel_idx,
                               const float* o_cmp, const float* gates, void* out,
                               float* o_sel, hipStream_t stream);

/* Dense global attention, the quadratic baseline the method replaces (summary
 * "Probleemstelling"): out = softmax(scale * q k^T) v over all T tokens per head, input type
 * [T][H][64]. Workspace: speed3r_dense_workspace_size(p) bytes. */
s3r_status speed3r_dense_attn_fwd(const s3r_params* p, const void* q, const void* k,
                                  const void* v, void* out, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * Training: forward pass that keeps what the backward pass needs, and the backward pass.
 * The model is trained end to end (arXiv abstract; README "Overview"). Gradients flow
 * through both branches and the gates with the forward pass's selection held fixed: top-k is
 * piecewise constant, so the block scores receive no gradient.
 * ------------------------------------------------------------------------------------- */

/* Bytes of the training workspace: speed3r_workspace_size plus the block means, O_sel
 * [T][H][64] f32 and the selection log-sum-exp [H][T] f32. 0 if p is invalid. */
size_t speed3r_train_workspace_size(const s3r_params* p);

/* speed3r_sparse_attn_fwd that leaves, in `workspace` (speed3r_train_workspace_size bytes),
 * everything speed3r_sparse_attn_bwd reads: the packed tiles, both log-sum-exps, O_cmp, O_sel,
 * the block means and the selection (also copied to sel_idx when it is not NULL). */
s3r_status speed3r_sparse_attn_fwd_train(const s3r_params* p, const void* q, const void* k,
                                         const void* v, const float* gates, void* out,
                                         int32_t* sel_idx, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream);

/* Bytes of scratch speed3r_sparse_attn_bwd needs: operand tiles of q, dout, k, v and the
 * block means, per-token scalars, the pooled gradients, a [H][Nb][ceil(Nb/32)] selection
 * bitmap, per-token gate gradients and four partial sums of the pooled gradients (about
 * 14.0 GB at T = 1,374,000, H = 16, B = 64). */
size_t speed3r_bwd_workspace_size(const s3r_params* p);

/* Gradients of the sparse forward pass. q, k, v, gates and p must be those of the
 * speed3r_sparse_attn_fwd_train call whose workspace is `train_workspace` (read only).
 *   dout     [T][H][64] of the input type (bf16 or fp16), the gradient of out; element
 *            strides multiples of 8.
 *   dq, dk, dv   f32 [T][H][64], contiguous; overwritten.
 *   dgates   f32 with the layout of gates ([H][2], or gate(t, h, b) at t * gate_stride_t +
 *            h * 2 + b for per-token gates); overwritten.
 * Every output element is written by one thread in a fixed order: results are bitwise
 * repeatable. Numerics: the recomputed logits use the same operands as the forward pass
 * (the input type; pooled keys as hi + lo), probabilities use the saved log-sum-exps, dP takes
 * dout and the values in the input type, and the products feeding dq, dk, dv take bf16
 * operands (P, dS and transposed images of q, k, dout, the pooled keys), all with f32
 * accumulation. */
s3r_status speed3r_sparse_attn_bwd(const s3r_params* p, const void* q, const void* k,
                                   const void* v, const float* gates, const void* dout,
                                   int64_t dout_stride_t, int64_t dout_stride_h,
                                   const void* train_workspace, size_t train_workspace_bytes,
                                   float* dq, float* dk, float* dv, float* dgates,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * 2-D pooling windows. The compression branch pools by spatial downsampling of the patch grid
 * (summary "Methodologie" 1) and the model takes image sides in multiples of 56 pixels, i.e.
 * patch grids in multiples of 4 patches (README "Notice" 1). With contiguous blocks that is
 * obtained by reordering the tokens: each view is `special` tokens followed by its row-major
 * grid_h x grid_w patch grid; in window order every view's grid is listed window by window
 * (windows row-major, patches row-major inside a window) and all views' special tokens follow
 * at the end, in view order. A block of B = win_h * win_w positions is then one spatial
 * window (B a multiple of win_h * win_w: a row of B / (win_h * win_w) windows).
 * ------------------------------------------------------------------------------------- */
typedef struct {
  int64_t views;     /* V >= 1 */
  int32_t special;   /* S >= 0 tokens at the start of every view */
  int32_t grid_h;    /* patch grid of every view, >= 1 */
  int32_t grid_w;
  int32_t win_h;     /* window shape: win_h divides grid_h, win_w divides grid_w */
  int32_t win_w;
} s3r_windows;

/* Caller token held at position `pos` of the window order, for T = V * (S + grid_h*grid_w)
 * tokens (host function). -1 if w is invalid or pos is outside [0, T). */
int64_t speed3r_window_source(const s3r_windows* w, int64_t pos);

/* Reorders a [T][H][64] tensor of 2-byte elements (bf16 or fp16) into window order (inverse = 0: dst[pos] =
 * src[source(pos)]) or back (inverse = 1: dst[source(pos)] = src[pos]), T = V * (S + grid).
 * Strides are in elements, multiples of 8; src and dst must not overlap. Byte-exact copy. */
s3r_status speed3r_window_permute(const s3r_windows* w, int32_t H, const void* src,
                                  int64_t src_stride_t, int64_t src_stride_h, void* dst,
                                  int64_t dst_stride_t, int64_t dst_stride_h, int32_t inverse,
                                  hipStream_t stream);

/* Bytes of workspace speed3r_sparse_attn_fwd_windows needs: window-ordered copies of q, k, v
 * (and of per-token gates), the window-ordered output, then speed3r_workspace_size of the
 * reordered problem. 0 if p or w is invalid or p->T != V * (S + grid_h*grid_w). */
size_t speed3r_windows_workspace_size(const s3r_params* p, const s3r_windows* w);

/* The sparse forward pass with 2-D windows as blocks: reorders q, k, v (and per-token gates)
 * into window order inside the workspace, runs speed3r_sparse_attn_fwd on them, and writes
 * out ([T][H][64] of the input type, contiguous) back in the caller's token order. sel_idx (optional,
 * [H][Nb][n_sel]) and forced_blocks refer to blocks of the window order: forced blocks
 * 0..F-1 are the first view's first windows. Arguments are checked as for
 * speed3r_sparse_attn_fwd; on any error nothing is launched. */
s3r_status speed3r_sparse_attn_fwd_windows(const s3r_params* p, const s3r_windows* w,
                                           const void* q, const void* k, const void* v,
                                           const float* gates, void* out, int32_t* sel_idx,
                                           void* workspace, size_t workspace_bytes,
                                           hipStream_t stream);

/* ---- Forward pass without allocation -------------------------------------------------------
 * For callers that cannot allocate device memory at call time (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same forward pass as
 * speed3r_sparse_attn_fwd, with its workspace taken from a fixed array the library holds in
 * device memory (one per GPU it runs on, kept until the process ends). */

/* Size of that array: the largest speed3r_workspace_size the no-allocation entry point takes
 * (512 MiB, e.g. 32 views x 1374 tokens x 16 heads at B = 64, k = 16). */
size_t speed3r_noalloc_scratch_bytes(void);

/* speed3r_sparse_attn_fwd without a workspace argument: arguments, results and errors as
 * there, plus S3R_ERR_SCRATCH (nothing launched) when speed3r_workspace_size(p) exceeds
 * speed3r_noalloc_scratch_bytes(). Calls nothing that allocates. The first call on a device
 * looks up that device's array (S3R_ERR_HIP if the lookup fails). Every call on one GPU uses
 * the same array: calls that overlap on one GPU (several streams, or several host threads
 * without ordering) race and give wrong results; calls ordered on one stream are safe. Every
 * part of the array a call reads is first written by that call, so nothing carries over. */
s3r_status speed3r_sparse_attn_fwd_noalloc(const s3r_params* p, const void* q, const void* k,
                                           const void* v, const float* gates, void* out,
                                           int32_t* sel_idx, hipStream_t stream);

/* ---- Measured ceilings (not part of the method) -------------------------------------------
 * The pages print no kernel figures; the kernels' roofline fractions are quoted against the
 * vendor's peaks and against what these two plain kernels reach on the same chip. */

/* Streaming copy of `bytes` (a multiple of 16; src and dst 16-byte aligned, not overlapping)
 * from src to dst: one 16-byte load and store per element, 4 in flight per thread. It moves
 * 2 * bytes through HBM. S3R_ERR_INVALID_ARG on a null or misaligned pointer or a bad size. */
s3r_status speed3r_calib_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

/* Floating-point operations one speed3r_calib_mfma call performs (-1 for a bad argument):
 * work_groups * 4 waves * iters * 8 chains * 16384 (one 16x16x32 bf16 matrix product). */
int64_t speed3r_calib_mfma_flops(int32_t work_groups, int32_t iters);

/* A loop of independent v_mfma_f32_16x16x32_bf16 products (8 accumulators per wave, 4 waves
 * per work-group, `iters` rounds); one f32 per thread is written to sink [work_groups * 256]
 * so the work is kept. S3R_ERR_INVALID_ARG on a null or misaligned sink or a size below 1. */
s3r_status speed3r_calib_mfma(float* sink, int32_t work_groups, int32_t iters,
                              hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEED3R_H */
