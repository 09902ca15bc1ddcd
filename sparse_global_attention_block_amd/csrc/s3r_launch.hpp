// Kernel argument blocks and host launchers shared between the kernel files and the C ABI
// layer. Private to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace s3r {

struct PoolArgs {
  const uint16_t* k; const uint16_t* v;
  int64_t k_st, k_sh, v_st, v_sh;
  int64_t T, Nb, n_tiles;
  int32_t H, B;
  int32_t half;            // inputs are fp16 (else bf16)
  float key_mult;          // scale * log2(e), folded into the packed pooled keys
  float v_mult;            // power of two the pooled values are multiplied by before their
                           // fp16 records are written (kept in fp16 range; see v_unscale)
  const float* bsum;       // [H][Nb][128] f32 column sums of each block's k (64) and v (64)
                           // rows, written by the packing kernel
  float* k_mean; float* v_mean;  // optional f32 [H][Nb][64]
  unsigned char* tiles;    // [H][n_tiles][12 KB]
  unsigned char* group_tiles;  // optional [H][n_gtiles][12 KB] (K records only): key g is the
  int64_t n_gtiles;            // mean of pooled keys 8g..8g+7, for g < 32 * n_gtiles
};

struct PackArgs {
  const uint16_t* k; const uint16_t* v;
  int64_t k_st, k_sh, v_st, v_sh;
  int64_t T, n_tiles;
  int32_t H;
  int32_t half;            // inputs are fp16 (else bf16)
  float v_mult;            // power of two applied to v before its fp16 V^T records
  unsigned char* tiles;    // [H][n_tiles][8 KB]
  float* bsum;             // optional [H][Nb][128]: per block of B tokens, the f32 column sums
  int64_t Nb;              // of its k rows (dims 0..63) and v rows (64..127), for pooling
  int32_t B;
};

struct CmpArgs {
  const uint16_t* q;
  int64_t q_st, q_sh;
  int64_t T, Nb, n_tiles;  // n_tiles = ceil(Nb / 32)
  int32_t H, B;
  int32_t half;            // q and the pooled key records are fp16 (else bf16)
  const unsigned char* tiles;  // pooled tiles
  float* lse;              // [H][T] natural log (written by the LSE pass, read by the fused pass)
  const float* lse_in;
  float* o_cmp;            // [T][H][64]
  float v_unscale;         // 1 / v_mult of the pooled value records, applied to O_cmp
  float* score;            // [H][Nb][ld]
  int64_t ld;
  int32_t* sel;            // running top-k output [H][Nb][n_sel] (fused selection only)
  int32_t n_sel;           // row length: forced prefix (+ own block) + chosen blocks
  int32_t forced;          // F': blocks 0..F'-1 always selected, top-k over the rest
  int32_t topk;            // k (chosen per row, clamped to the candidates)
  int32_t own;             // each query block also keeps its own block
  float lse_bias;          // added to every log-sum-exp the LSE pass writes (natural log)
  const int32_t* redo_in;  // if set: only work-groups whose 4 flags, or-ed, meet redo_mask and
  int32_t redo_mask;       // miss redo_skip run
  int32_t redo_skip;
  int32_t* redo_out;       // single pass: [work-group][4 waves], bit 0 = selection not proven,
                           // bit 1 = Z check failed (the log-sum-exp must be recomputed)
};

// The single compression pass starts from lse_in - kBoundMargin (base 2): a lower bound of
// the log-sum-exp must stay one after rounding.
constexpr float kBoundMargin = 0x1p-10f;
constexpr int kGroupBlocks = 8;  // pooled keys averaged into one key of the bound pass

struct TopkArgs {
  const float* score;
  int64_t ld;
  int64_t Nb;
  int64_t n_rows;          // H * Nb
  int32_t n_sel;           // row length of sel
  int32_t forced;          // F': blocks 0..F'-1 always selected
  int32_t topk;            // k chosen among the remaining blocks (clamped)
  int32_t own;             // row i also keeps block i (when i >= F')
  int32_t* sel;            // [n_rows][n_sel], rows padded with -1
};

struct AttnArgs {
  const uint16_t* q;
  int64_t q_st, q_sh;
  int64_t T, Nb, n_tiles;  // raw tiles: n_tiles = ceil(T / 32)
  int32_t H, B;
  int32_t half;            // q, k and out are fp16 (else bf16)
  float logit_mult;        // scale * log2(e)
  float v_unscale;         // 1 / v_mult of the raw value records, applied to the output
  const unsigned char* tiles;  // raw packed k/v tiles
  // selection only
  const int32_t* sel; int32_t k_eff;  // k_eff = entries per selection row (n_sel)
  const float* o_cmp;
  const float* gates; int64_t gate_st;
  float* o_sel;            // optional
  float* lse_sel;          // optional [H][T]: base-2 log-sum-exp of the selection softmax
                           // in units of the scaled logit (scale*log2(e)*q.k); +inf if empty
  uint16_t* out;           // [T][H][64], the input type
};

// Token layout of the window order (see s3r_window.hip): views x (special + grid_h*grid_w).
struct WindowLayout {
  int64_t views;
  int32_t special, grid_h, grid_w, win_h, win_w;
};

// Caller token of position pos of the window-ordered sequence (pos < views*(special+grid)).
__host__ __device__ inline int64_t window_source(const WindowLayout& w, int64_t pos) {
  const int64_t grid = (int64_t)w.grid_h * w.grid_w;
  const int64_t per_view = w.special + grid;
  const int64_t grid_total = w.views * grid;
  if (pos < grid_total) {
    const int64_t v = pos / grid;
    const int64_t r = pos - v * grid;
    const int64_t win = (int64_t)w.win_h * w.win_w;
    const int64_t wi = r / win, e = r - wi * win;
    const int64_t nwx = w.grid_w / w.win_w;
    const int64_t wy = wi / nwx, wx = wi - wy * nwx;
    const int64_t i = e / w.win_w, j = e - i * w.win_w;
    return v * per_view + w.special + (wy * w.win_h + i) * w.grid_w + wx * w.win_w + j;
  }
  const int64_t u = pos - grid_total;
  const int64_t v = u / w.special;
  return v * per_view + (u - v * w.special);
}

struct WindowCopyArgs {
  WindowLayout w;
  int64_t T;
  int32_t H;
  int32_t inverse;         // 0: dst[pos] = src[source(pos)]; 1: dst[source(pos)] = src[pos]
  const unsigned char* src;
  int64_t src_st, src_sh;  // byte strides between tokens / heads
  unsigned char* dst;
  int64_t dst_st, dst_sh;
};

// ---- backward pass ----------------------------------------------------------------------
// Operand-image record groups of 32 rows x 64 dims (4 KB each, bf16):
//   R  (rows as lanes):  record (s, c), lane l -> row 16s + l%16, dims 32c + 8(l/16) + 0..7;
//   TR (dims as lanes):  record mt, lane l -> dim 16mt + l%16, slot e -> row vkey(l/16, e).
// R images are in the input type (bf16 or fp16: they meet q, k in the logits and dP
// products), TR images always bf16 (they meet P and dS in the dq, dk, dv products).
// Query image (8 KB per 32 queries): [R(q)][R(dout)]; the kernels that need the transposed
// images build them on chip (cmp_dkv: a 16 KB LDS tile [R(q)][TR(q)][R(dout)][TR(dout)];
// sel_dkv: transposing LDS reads).
// Raw backward tile (8 KB per 32 keys): [R(v)][TR(k)].
// Pooled backward tile (8 KB per 32 pooled keys): [R(Vc)][TR(Kc)], from the f32 means.
constexpr int kQImgBytes = 8 * 1024;
constexpr int kQTileBytes = 16 * 1024;
constexpr int kBwdTileBytes = 8 * 1024;

struct RecPackArgs {
  const void* src;         // bf16 (kind 0) or f32 (kind 1) rows
  int64_t st, sh;          // element strides between rows / heads
  int64_t rows, n_tiles;   // valid rows; tiles of 32 rows
  int32_t H;
  unsigned char* dst;      // tile base of head 0
  int64_t tile_bytes;      // distance between consecutive tiles of one head
  int32_t r_off, tr_off;   // byte offsets of the R and TR groups inside a tile (-1: skip)
  int32_t half;            // 2-byte sources and R records are fp16 (else bf16); TR is bf16
};

struct BwdScalarArgs {
  int64_t T; int32_t H;
  int32_t half;            // dout is fp16 (else bf16)
  const float* lse_cmp;    // [H][T], natural log
  const float* lse_sel;    // [H][T], base 2 (selection kernel units)
  const float* gates; int64_t gate_st;
  const uint16_t* dout; int64_t d_st, d_sh;
  const float* o_cmp; const float* o_sel;  // [T][H][64]
  float* qs;               // [H][T][8]: L2c, g0, Dc, L2s, g1, Ds, 0, 0
  float* dg_tok; int64_t dg_st, dg_sh;  // per-token gate gradients: dg_tok[t*dg_st + h*dg_sh + b]
};

struct BwdArgs {
  int64_t T, Nb, n_ctiles, n_ktiles;
  int32_t H, B;
  int32_t half;            // q, k, v, dout and the R images are fp16 (else bf16)
  float scale;             // softmax scale
  float logit_mult;        // scale * log2(e)
  const unsigned char* pooled;      // forward pooled tiles (12 KB: K hi, K lo, V^T)
  const unsigned char* pooled_bwd;  // [R(Vc)][TR(Kc)]
  const unsigned char* raw;         // forward raw tiles (8 KB: K, V^T)
  const unsigned char* raw_bwd;     // [R(v)][TR(k)]
  const unsigned char* qtiles;      // query tiles
  const float* qs;                  // per-query scalars
  const uint16_t* q; int64_t q_st, q_sh;     // queries (resident operands of the dq kernels)
  const uint16_t* dout; int64_t d_st, d_sh;
  const int32_t* sel; int32_t n_sel;
  const uint32_t* bitmap; int64_t bm_words;  // [H][Nb][bm_words]: bit i of row u = i selected u
  float* dkc; float* dvc;           // [H][Nb][64]
  float* dkc_part; float* dvc_part; // [kDkvParts][H][Nb][64]: cmp_dkv's sums over each part
                                    // of the query tiles, added in order into dkc, dvc
  float* dq; float* dk; float* dv;  // [T][H][64]
};

hipError_t launch_rec_pack(const RecPackArgs& a, int kind, hipStream_t s);
hipError_t launch_bwd_scalars(const BwdScalarArgs& a, hipStream_t s);
hipError_t launch_gate_reduce(const float* dg_tok, int64_t T, int32_t H, float* dgates,
                              hipStream_t s);
hipError_t launch_sel_bitmap(const BwdArgs& a, uint32_t* bitmap, hipStream_t s);
hipError_t launch_cmp_dq(const BwdArgs& a, hipStream_t s);
hipError_t launch_cmp_dkv(const BwdArgs& a, hipStream_t s);  // also adds its parts
constexpr int kDkvParts = 4;  // cmp_dkv work-groups per (head, group of pooled tiles)
hipError_t launch_sel_dq(const BwdArgs& a, hipStream_t s);
hipError_t launch_sel_dkv(const BwdArgs& a, hipStream_t s);

hipError_t launch_pool(const PoolArgs& a, hipStream_t s);
hipError_t launch_pack(const PackArgs& a, hipStream_t s);
hipError_t launch_cmp_lse(const CmpArgs& a, hipStream_t s);
hipError_t launch_cmp_lse_bound(const CmpArgs& a, hipStream_t s);
hipError_t launch_cmp_fused(const CmpArgs& a, hipStream_t s);
hipError_t launch_cmp_fused_topk(const CmpArgs& a, hipStream_t s);
hipError_t launch_cmp_single_topk(const CmpArgs& a, hipStream_t s);
// the exact passes on the work-groups redo_in flags (fused: pass 2 with the running top-k;
// scores_only: without P.V and O_cmp)
hipError_t launch_cmp_rerun(const CmpArgs& a, hipStream_t s, bool fused, bool scores_only);
constexpr int kFusedTopkMaxK = 64;  // the running top-k keeps one entry per lane
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
hipError_t launch_sel(const AttnArgs& a, hipStream_t s);
hipError_t launch_dense(const AttnArgs& a, hipStream_t s);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);
hipError_t launch_window_copy(const WindowCopyArgs& a, int row_bytes, hipStream_t s);

}  // namespace s3r
