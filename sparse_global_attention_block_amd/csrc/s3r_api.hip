// C ABI of libspeed3r.so: argument validation, workspace layout and kernel launches.
// The functions are declared (and their contracts stated) in include/speed3r.h.
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/speed3r.h"
#include "s3r_common.hpp"
#include "s3r_launch.hpp"

using namespace s3r;

namespace {

// Longest score row the separate top-k path takes: the score matrix is H * Nb^2 floats
// (38.7 GB at H = 16, Nb = 24576), and the exact tie search of the top-k kernel indexes up to 2^16.
constexpr int64_t kMaxBlocks = 96 * 256;

// The P.V products take fp16 value records. bf16 values are stored times 2^-8 (exact for
// magnitudes 2^-6..2^24, within 2^-17 absolute below) and the outputs multiplied back by 2^8,
// so bf16 values up to 65504 * 2^8 (about 1.68e7) in magnitude are represented; fp16 values
// are stored as they are.
constexpr float kVMultBf16 = 0x1p-8f;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Dims {
  int64_t T, Nb, n_ctiles, n_ktiles, ld;
  int64_t k_eff;   // entries per selection row: forced prefix + chosen blocks (n_sel)
  int64_t forced;  // F' = min(forced_blocks, Nb)
  int64_t topk;    // k as given
  int32_t own;     // each query block also keeps its own block (and F' < Nb)
  int32_t H, B;
  int32_t half;    // q, k, v (and out) are fp16; else bf16
  float scale;
  bool fold_topk;  // selection folded into the compression pass (no score matrix)
  int64_t Nb_g;     // keys of the bound pass: full groups of kGroupBlocks pooled keys
  int64_t n_gtiles; // tiles of those keys, ceil(Nb_g / 32)
  int64_t n_redo;   // redo flags of the single pass: 4 per 256 queries per head
  bool single_ok;   // the single pass applies: folded selection and at least one group
  bool single;      // the forward pass runs the single pass (cmp_mode)
};

// Workspace regions, in this order, each 256-byte aligned.
struct Layout {
  size_t pooled, groups, raw, bsum, lse, o_cmp, score, sel, redo, tiles_end, end;
};

bool valid_stride(int64_t s) { return s >= 0 && (s % 8) == 0; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

s3r_status check_params(const s3r_params* p, Dims* d) {
  if (!p) return S3R_ERR_INVALID_ARG;
  if (p->T < 1 || p->H < 1 || p->topk < 1 || p->forced_blocks < 0) return S3R_ERR_INVALID_ARG;
  if (p->block < 1 || p->D < 1) return S3R_ERR_INVALID_ARG;
  if (p->dtype != S3R_BF16 && p->dtype != S3R_FP16) return S3R_ERR_INVALID_ARG;
  if (p->cmp_mode != S3R_CMP_AUTO && p->cmp_mode != S3R_CMP_TWO_PASS &&
      p->cmp_mode != S3R_CMP_SINGLE)
    return S3R_ERR_INVALID_ARG;
  if (!(p->scale >= 0.f) || isinf(p->scale)) return S3R_ERR_INVALID_ARG;
  if (!valid_stride(p->q_stride_t) || !valid_stride(p->q_stride_h) ||
      !valid_stride(p->k_stride_t) || !valid_stride(p->k_stride_h) ||
      !valid_stride(p->v_stride_t) || !valid_stride(p->v_stride_h) || p->gate_stride_t < 0)
    return S3R_ERR_INVALID_ARG;
  if (p->D != kD) return S3R_ERR_UNSUPPORTED;
  if (p->block != 16 && p->block != 32 && p->block != 64 && p->block != 128)
    return S3R_ERR_UNSUPPORTED;
  if (p->H > 65535 || p->T > ((int64_t)1 << 31) - 1) return S3R_ERR_UNSUPPORTED;
  d->T = p->T;
  d->H = p->H;
  d->half = p->dtype == S3R_FP16;
  d->B = p->block;
  d->Nb = (p->T + p->block - 1) / p->block;
  d->n_ctiles = (d->Nb + kTileKeys - 1) / kTileKeys;
  d->n_ktiles = (d->T + kTileKeys - 1) / kTileKeys;
  d->ld = d->n_ctiles * kTileKeys;
  d->forced = p->forced_blocks < d->Nb ? p->forced_blocks : d->Nb;
  d->topk = p->topk;
  d->own = (p->force_own != 0 && d->forced < d->Nb) ? 1 : 0;
  const int64_t rest = d->Nb - d->forced - d->own;
  d->k_eff = d->forced + d->own + (p->topk < rest ? p->topk : rest);
  d->scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)kD);
  // the running top-k holds one entry per lane; a row whose own block is forced chooses from
  // one more candidate
  const int64_t most = (p->topk < d->Nb - d->forced) ? p->topk : d->Nb - d->forced;
  d->fold_topk = d->B <= 64 && most <= kFusedTopkMaxK;
  d->Nb_g = d->Nb / kGroupBlocks;
  d->n_gtiles = (d->Nb_g + kTileKeys - 1) / kTileKeys;
  d->n_redo = (int64_t)d->H * ((d->T + 255) / 256) * 4;
  d->single_ok = d->fold_topk && d->Nb_g >= 1;
  // automatic: the single pass where its list of 64 bound-ranked candidates holds every
  // candidate or at least 4k/3 of them (k <= 48). At 1000 views (21,469 blocks) its check
  // fails on no wave for k = 16, 0.2 % for k = 32, 3 % for k = 40 (62 ms faster than two
  // passes), 23 % for k = 48 (32 ms faster) and 74 % for k = 56 (20 ms slower).
  d->single = d->single_ok && (p->cmp_mode == S3R_CMP_SINGLE ||
                               (p->cmp_mode == S3R_CMP_AUTO &&
                                (4 * most <= 3 * kFusedTopkMaxK || d->Nb - d->forced <= 64)));
  // the separate top-k kernel's exact tie search indexes a row with 16 bits and the score
  // matrix grows as Nb^2; the folded selection has no limit
  if (!d->fold_topk && d->Nb > kMaxBlocks) return S3R_ERR_UNSUPPORTED;
  return S3R_OK;
}

Layout layout(const Dims& d) {
  Layout L;
  size_t off = 0;
  L.pooled = off;
  off += align256((size_t)d.H * d.n_ctiles * kPooledTileBytes);
  L.groups = off;
  off += align256((size_t)d.H * d.n_gtiles * kPooledTileBytes);
  L.raw = off;
  off += align256((size_t)d.H * d.n_ktiles * kRawTileBytes);
  L.bsum = off;  // the blocks' column sums, from packing to pooling
  off += align256((size_t)d.H * d.Nb * 128 * sizeof(float));
  L.tiles_end = off;
  L.lse = off;
  off += align256((size_t)d.H * d.T * sizeof(float));
  L.o_cmp = off;
  off += align256((size_t)d.T * d.H * kD * sizeof(float));
  L.score = off;
  if (!d.fold_topk) off += align256((size_t)d.H * d.Nb * d.ld * sizeof(float));
  L.sel = off;
  off += align256((size_t)d.H * d.Nb * d.k_eff * sizeof(int32_t));
  L.redo = off;
  if (d.single) off += align256((size_t)d.n_redo * sizeof(int32_t));
  L.end = off;
  return L;
}

s3r_status check_ws(const void* ws, size_t bytes, size_t need) {
  if (!ws || !aligned(ws, 256) || bytes < need) return S3R_ERR_WORKSPACE;
  return S3R_OK;
}

bool tok_ok(const void* x) { return x && aligned(x, 16); }

s3r_status hip_status(hipError_t e) { return e == hipSuccess ? S3R_OK : S3R_ERR_HIP; }

PoolArgs pool_args(const s3r_params* p, const Dims& d, const void* k, const void* v, void* ws,
                   const Layout& L, float* k_mean, float* v_mean) {
  PoolArgs a;
  a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.k_st = p->k_stride_t; a.k_sh = p->k_stride_h; a.v_st = p->v_stride_t; a.v_sh = p->v_stride_h;
  a.T = d.T; a.Nb = d.Nb; a.n_tiles = d.n_ctiles; a.H = d.H; a.B = d.B; a.half = d.half;
  a.key_mult = d.scale * kLog2e;
  a.v_mult = d.half ? 1.0f : kVMultBf16;
  a.bsum = (const float*)((unsigned char*)ws + L.bsum);
  a.k_mean = k_mean; a.v_mean = v_mean;
  a.tiles = (unsigned char*)ws + L.pooled;
  a.group_tiles = d.n_gtiles > 0 ? (unsigned char*)ws + L.groups : nullptr;
  a.n_gtiles = d.n_gtiles;
  return a;
}

// bsum: where the blocks' column sums for pooling go (null: raw tiles only)
PackArgs pack_args(const s3r_params* p, const Dims& d, const void* k, const void* v,
                   unsigned char* tiles, float* bsum) {
  PackArgs a;
  a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.k_st = p->k_stride_t; a.k_sh = p->k_stride_h; a.v_st = p->v_stride_t; a.v_sh = p->v_stride_h;
  a.T = d.T; a.n_tiles = d.n_ktiles; a.H = d.H; a.half = d.half;
  a.v_mult = d.half ? 1.0f : kVMultBf16;
  a.tiles = tiles;
  a.bsum = bsum; a.Nb = d.Nb; a.B = d.B;
  return a;
}

CmpArgs cmp_args(const s3r_params* p, const Dims& d, const void* q, const void* ws,
                 const Layout& L) {
  CmpArgs a;
  memset(&a, 0, sizeof(a));
  a.q = (const uint16_t*)q; a.q_st = p->q_stride_t; a.q_sh = p->q_stride_h;
  a.T = d.T; a.Nb = d.Nb; a.n_tiles = d.n_ctiles; a.H = d.H; a.B = d.B; a.half = d.half;
  a.tiles = (const unsigned char*)ws + L.pooled;
  a.ld = d.ld;
  a.v_unscale = d.half ? 1.0f : 1.0f / kVMultBf16;
  return a;
}

AttnArgs attn_args(const s3r_params* p, const Dims& d, const void* q,
                   const unsigned char* raw_tiles) {
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.q = (const uint16_t*)q; a.q_st = p->q_stride_t; a.q_sh = p->q_stride_h;
  a.T = d.T; a.Nb = d.Nb; a.n_tiles = d.n_ktiles; a.H = d.H; a.B = d.B; a.half = d.half;
  a.logit_mult = d.scale * kLog2e;
  a.v_unscale = d.half ? 1.0f : 1.0f / kVMultBf16;
  a.tiles = raw_tiles;
  a.k_eff = (int32_t)d.k_eff;
  a.gate_st = p->gate_stride_t;
  return a;
}

s3r_status run_cmp_fused(const Dims& d, CmpArgs a, hipStream_t stream) {
  if (d.B > 64) {
    s3r_status st = hip_status(launch_fill_zero(a.score, (int64_t)d.H * d.Nb * d.ld, stream));
    if (st != S3R_OK) return st;
  }
  return hip_status(launch_cmp_fused(a, stream));
}

// The bound pass: the LSE pass over the group keys (mean of 8 pooled keys each), plus ln 8.
// By Jensen's inequality sum_{j in G} exp(c_j) >= 8 exp(mean_G c), and c is linear in the
// key, so log sum_G 8 exp(q . mean_G Kc) is at most the log-sum-exp over all pooled keys.
s3r_status run_lse_bound(const Dims& d, CmpArgs a, const unsigned char* ws, const Layout& L,
                         float* lse_bound, hipStream_t stream) {
  a.tiles = ws + L.groups;
  a.n_tiles = d.n_gtiles;
  a.Nb = d.Nb_g;
  a.lse = lse_bound;
  a.lse_bias = logf((float)kGroupBlocks);
  return hip_status(launch_cmp_lse_bound(a, stream));
}

// The single pass from the bound, then the two exact passes on the work-groups it flagged.
// `a` carries the selection fields; lse_bound may equal lse.
s3r_status run_single(CmpArgs a, const float* lse_bound, float* lse, int32_t* redo,
                      hipStream_t stream) {
  s3r_status st;
  a.lse_in = lse_bound;
  a.lse = lse;
  a.redo_out = redo;
  if ((st = hip_status(launch_cmp_single_topk(a, stream))) != S3R_OK) return st;
  a.redo_out = nullptr;
  a.redo_in = redo;
  a.redo_mask = 2;  // where a Z check failed: the log-sum-exp, then everything of pass 2
  a.redo_skip = 0;
  a.lse_bias = 0.f;
  if ((st = hip_status(launch_cmp_rerun(a, stream, false, false))) != S3R_OK) return st;
  a.lse_in = lse;
  if ((st = hip_status(launch_cmp_rerun(a, stream, true, false))) != S3R_OK) return st;
  a.redo_mask = 1;  // where only a selection was not proven: the scores and the top-k
  a.redo_skip = 2;
  return hip_status(launch_cmp_rerun(a, stream, true, true));
}

// Regions the training forward pass adds after the forward workspace: what the backward
// pass needs beyond it (block means, O_sel and the selection log-sum-exp).
struct TrainLayout {
  size_t k_mean, v_mean, o_sel, lse_sel, end;
};

TrainLayout train_layout(const Dims& d) {
  TrainLayout T;
  size_t off = layout(d).end;
  const size_t pooled = align256((size_t)d.H * d.Nb * kD * sizeof(float));
  T.k_mean = off; off += pooled;
  T.v_mean = off; off += pooled;
  T.o_sel = off; off += align256((size_t)d.T * d.H * kD * sizeof(float));
  T.lse_sel = off; off += align256((size_t)d.H * d.T * sizeof(float));
  T.end = off;
  return T;
}

// Backward workspace: operand tiles, per-token scalars, pooled gradients, selection bitmap
// and the per-token gate gradients (reduced per head when the gates are per head).
struct BwdLayout {
  size_t qtiles, raw_bwd, pooled_bwd, qs, dkc, dvc, dkv_part, bitmap, dg_tok, end;
  int64_t bm_words;
};

BwdLayout bwd_layout(const Dims& d) {
  BwdLayout B;
  size_t off = 0;
  B.bm_words = (d.Nb + 31) / 32;
  B.qtiles = off; off += align256((size_t)d.H * d.n_ktiles * kQImgBytes);
  B.raw_bwd = off; off += align256((size_t)d.H * d.n_ktiles * kBwdTileBytes);
  B.pooled_bwd = off; off += align256((size_t)d.H * d.n_ctiles * kBwdTileBytes);
  B.qs = off; off += align256((size_t)d.H * d.T * 8 * sizeof(float));
  B.dkc = off; off += align256((size_t)d.H * d.Nb * kD * sizeof(float));
  B.dvc = off; off += align256((size_t)d.H * d.Nb * kD * sizeof(float));
  B.dkv_part = off; off += 2 * align256((size_t)kDkvParts * d.H * d.Nb * kD * sizeof(float));
  B.bitmap = off; off += align256((size_t)d.H * d.Nb * B.bm_words * sizeof(uint32_t));
  B.dg_tok = off; off += align256((size_t)d.T * d.H * 2 * sizeof(float));
  B.end = off;
  return B;
}

// The forward pass on a validated problem. With `train`, the pooling also writes the block
// means, the selection kernel writes O_sel and its log-sum-exp, and the selection stays in
// the workspace.
s3r_status run_forward(const s3r_params* p, const Dims& d, const Layout& L, const void* q,
                       const void* k, const void* v, const float* gates, void* out,
                       int32_t* sel_idx, unsigned char* ws, const TrainLayout* train,
                       hipStream_t stream) {
  s3r_status st;
  float* lse = (float*)(ws + L.lse);
  float* o_cmp = (float*)(ws + L.o_cmp);
  float* score = (float*)(ws + L.score);
  int32_t* sel = sel_idx ? sel_idx : (int32_t*)(ws + L.sel);
  float* k_mean = train ? (float*)(ws + train->k_mean) : nullptr;
  float* v_mean = train ? (float*)(ws + train->v_mean) : nullptr;
  if ((st = hip_status(launch_pack(pack_args(p, d, k, v, ws + L.raw, (float*)(ws + L.bsum)),
                                     stream))) != S3R_OK ||
      (st = hip_status(launch_pool(pool_args(p, d, k, v, ws, L, k_mean, v_mean), stream))) !=
          S3R_OK)
    return st;
  CmpArgs c = cmp_args(p, d, q, ws, L);
  c.o_cmp = o_cmp;
  if (d.single) {
    c.sel = sel;
    c.n_sel = (int32_t)d.k_eff;
    c.forced = (int32_t)d.forced;
    c.topk = (int32_t)d.topk;
    c.own = d.own;
    if ((st = run_lse_bound(d, c, ws, L, lse, stream)) != S3R_OK) return st;
    if ((st = run_single(c, lse, lse, (int32_t*)(ws + L.redo), stream)) != S3R_OK) return st;
  } else if (d.fold_topk) {
    c.lse = lse;
    if ((st = hip_status(launch_cmp_lse(c, stream))) != S3R_OK) return st;
    c.lse_in = lse;
    c.sel = sel;
    c.n_sel = (int32_t)d.k_eff;
    c.forced = (int32_t)d.forced;
    c.topk = (int32_t)d.topk;
    c.own = d.own;
    if ((st = hip_status(launch_cmp_fused_topk(c, stream))) != S3R_OK) return st;
  } else {
    c.lse = lse;
    if ((st = hip_status(launch_cmp_lse(c, stream))) != S3R_OK) return st;
    c.lse_in = lse;
    c.score = score;
    if ((st = run_cmp_fused(d, c, stream)) != S3R_OK) return st;
    TopkArgs t;
    t.score = score; t.ld = d.ld; t.Nb = d.Nb; t.n_rows = (int64_t)d.H * d.Nb;
    t.n_sel = (int32_t)d.k_eff; t.forced = (int32_t)d.forced; t.sel = sel;
    t.topk = (int32_t)d.topk; t.own = d.own;
    if ((st = hip_status(launch_topk(t, stream))) != S3R_OK) return st;
  }
  AttnArgs a = attn_args(p, d, q, ws + L.raw);
  a.sel = sel; a.o_cmp = o_cmp; a.gates = gates; a.out = (uint16_t*)out;
  a.o_sel = train ? (float*)(ws + train->o_sel) : nullptr;
  a.lse_sel = train ? (float*)(ws + train->lse_sel) : nullptr;
  return hip_status(launch_sel(a, stream));
}

// ---------------------------------------------------------------------------------------
// 2-D windows: layout checks and the workspace of the windowed forward pass
// ---------------------------------------------------------------------------------------
bool window_layout(const s3r_windows* w, WindowLayout* L, int64_t* T) {
  if (!w || w->views < 1 || w->special < 0 || w->grid_h < 1 || w->grid_w < 1 ||
      w->win_h < 1 || w->win_w < 1 || w->grid_h % w->win_h || w->grid_w % w->win_w)
    return false;
  const int64_t per_view = (int64_t)w->special + (int64_t)w->grid_h * w->grid_w;
  if (w->views > (((int64_t)1 << 31) - 1) / per_view) return false;
  L->views = w->views; L->special = w->special; L->grid_h = w->grid_h; L->grid_w = w->grid_w;
  L->win_h = w->win_h; L->win_w = w->win_w;
  *T = w->views * per_view;
  return true;
}

// window-ordered copies of q, k, v, gates and out, then the inner workspace
struct WindowWs {
  size_t q, k, v, gates, out, inner, end;
};

WindowWs window_ws(const Dims& d, bool token_gates, size_t inner_bytes) {
  WindowWs L;
  const size_t tok = align256((size_t)d.T * d.H * kD * 2);
  size_t off = 0;
  L.q = off; off += tok;
  L.k = off; off += tok;
  L.v = off; off += tok;
  L.gates = off; off += token_gates ? align256((size_t)d.T * d.H * 2 * sizeof(float)) : 0;
  L.out = off; off += tok;
  L.inner = off; off += inner_bytes;
  L.end = off;
  return L;
}

s3r_params windowed_params(const s3r_params* p) {
  s3r_params r = *p;
  r.q_stride_t = r.k_stride_t = r.v_stride_t = (int64_t)p->H * kD;
  r.q_stride_h = r.k_stride_h = r.v_stride_h = kD;
  r.gate_stride_t = p->gate_stride_t ? 2 * (int64_t)p->H : 0;
  return r;
}

WindowCopyArgs copy_args(const WindowLayout& w, int64_t T, int32_t H, int32_t inverse,
                         const void* src, int64_t src_st, int64_t src_sh, void* dst,
                         int64_t dst_st, int64_t dst_sh) {
  WindowCopyArgs a;
  a.w = w; a.T = T; a.H = H; a.inverse = inverse;
  a.src = (const unsigned char*)src; a.src_st = src_st; a.src_sh = src_sh;
  a.dst = (unsigned char*)dst; a.dst_st = dst_st; a.dst_sh = dst_sh;
  return a;
}

// ---------------------------------------------------------------------------------------
// Workspace without allocation: a fixed device array (one copy per GPU, held until the
// process ends) that speed3r_sparse_attn_fwd_noalloc uses in place of a caller workspace.
// Host code must not pass `scratch` itself to a kernel (on the host it names a stand-in, not
// the device copy): its device address is looked up once per device and kept.
// ---------------------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(512) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (the current device), looked up on first use.
s3r_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return S3R_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return S3R_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return S3R_OK;
}

}  // namespace

extern "C" {

const char* speed3r_status_string(int status) {
  switch (status) {
    case S3R_OK: return "S3R_OK";
    case S3R_ERR_INVALID_ARG: return "S3R_ERR_INVALID_ARG";
    case S3R_ERR_UNSUPPORTED: return "S3R_ERR_UNSUPPORTED";
    case S3R_ERR_WORKSPACE: return "S3R_ERR_WORKSPACE";
    case S3R_ERR_HIP: return "S3R_ERR_HIP";
    case S3R_ERR_SCRATCH: return "S3R_ERR_SCRATCH";
  }
  return "S3R_ERR_UNKNOWN";
}

int64_t speed3r_num_blocks(const s3r_params* p) {
  Dims d;
  return check_params(p, &d) == S3R_OK ? d.Nb : -1;
}

int64_t speed3r_num_selected(const s3r_params* p) {
  Dims d;
  return check_params(p, &d) == S3R_OK ? d.k_eff : -1;
}

int64_t speed3r_score_row_stride(const s3r_params* p) {
  Dims d;
  return check_params(p, &d) == S3R_OK ? d.ld : -1;
}

size_t speed3r_tiles_workspace_size(const s3r_params* p) {
  Dims d;
  return check_params(p, &d) == S3R_OK ? layout(d).tiles_end : 0;
}

size_t speed3r_workspace_size(const s3r_params* p) {
  Dims d;
  return check_params(p, &d) == S3R_OK ? layout(d).end : 0;
}

size_t speed3r_dense_workspace_size(const s3r_params* p) {
  Dims d;
  return check_params(p, &d) == S3R_OK ? align256((size_t)d.H * d.n_ktiles * kRawTileBytes) : 0;
}

s3r_status speed3r_pool(const s3r_params* p, const void* k, const void* v, void* workspace,
                        size_t workspace_bytes, float* k_mean, float* v_mean,
                        hipStream_t stream) {
  Dims d;
  s3r_status st = check_params(p, &d);
  if (st != S3R_OK) return st;
  if (!tok_ok(k) || !tok_ok(v) || (k_mean && !aligned(k_mean, 16)) ||
      (v_mean && !aligned(v_mean, 16)))
    return S3R_ERR_INVALID_ARG;
  const Layout L = layout(d);
  if ((st = check_ws(workspace, workspace_bytes, L.tiles_end)) != S3R_OK) return st;
  unsigned char* ws = (unsigned char*)workspace;
  st = hip_status(launch_pack(pack_args(p, d, k, v, ws + L.raw, (float*)(ws + L.bsum)), stream));
  if (st != S3R_OK) return st;
  return hip_status(launch_pool(pool_args(p, d, k, v, workspace, L, k_mean, v_mean), stream));
}

s3r_status speed3r_cmp_lse(const s3r_params* p, const void* q, const void* workspace,
                           size_t workspace_bytes, float* lse, hipStream_t stream) {
  Dims d;
  s3r_status st = check_params(p, &d);
  if (st != S3R_OK) return st;
  if (!tok_ok(q) || !lse || !aligned(lse, 4)) return S3R_ERR_INVALID_ARG;
  const Layout L = layout(d);
  if ((st = check_ws(workspace, workspace_bytes, L.tiles_end)) != S3R_OK) return st;
  CmpArgs a = cmp_args(p, d, q, workspace, L);
  a.lse = lse;
  return hip_status(launch_cmp_lse(a, stream));
}

s3r_status speed3r_cmp_fused(const s3r_params* p, const void* q, const void* workspace,
                             size_t workspace_bytes, const float* lse, float* o_cmp,
                             float* score, hipStream_t stream) {
  Dims d;
  s3r_status st = check_params(p, &d);
  if (st != S3R_OK) return st;
  if (!tok_ok(q) || !lse || !aligned(lse, 4) || !o_cmp || !aligned(o_cmp, 16) || !score ||
      !aligned(score, 4))
    return S3R_ERR_INVALID_ARG;
  const Layout L = layout(d);
  if ((st = check_ws(workspace, workspace_bytes, L.tiles_end)) != S3R_OK) return st;
  CmpArgs a = cmp_args(p, d, q, workspace, L);
  a.lse_in = lse;
  a.o_cmp = o_cmp;
  a.score = score;
  return run_cmp_fused(d, a, stream);
}

s3r_status speed3r_cmp_fused_topk(const s3r_params* p, const void* q, const void* workspace,
                                  size_t workspace_bytes, const float* lse, float* o_cmp,
                                  int32_t* sel_idx, hipStream_t stream) {
  Dims d;
  s3r_status st = check_params(p, &d);
  if (st != S3R_OK) return st;
  if (!tok_ok(q) || !lse || !aligned(lse, 4) || !o_cmp || !aligned(o_cmp, 16) || !sel_idx ||
      !aligned(sel_idx, 4))
    return S3R_ERR_INVALID_ARG;
  if (!d.fold_topk) return S3R_ERR_UNSUPPORTED;
  const Layout L = layout(d);
  if ((st = check_ws(workspace, workspace_bytes, L.tiles_end)) != S3R_OK) return st;
  CmpArgs a = cmp_args(p, d, q, workspace, L);
  a.lse_in = lse;
  a.o_cmp = o_cmp;
  a.sel = sel_idx;
  a.n_sel = (int32_t)d.k_eff;
  a.forced = (int32_t)d.forced;
  a.topk = (int32_t)d.topk;
  a.own = d.own;
  return hip_status(launch_cmp_fused_topk(a, stream));
}

int64_t speed3r_redo_flag_count(const s3r_params* p) {
  Dims d;
  return check_params(p, &d) == S3R_OK ? d.n_redo : -1;
}

s3r_status speed3r_cmp_lse_bound(const s3r_params* p, const void* q, const void* workspace,
                                 size_t workspace_bytes, float* lse_bound, hipStream_t stream) {
  Dims d;
  s3r_status st = check_params(p, &d);
  if (st != S3R_OK) return st;
  if (!tok_ok(q) || !lse_bound || !aligned(lse_bound, 4)) return S3R_ERR_INVALID_ARG;
  if (d.Nb_g < 1) return S3R_ERR_UNSUPPORTED;
  const Layout L = layout(d);
  if ((st = check_ws(workspace, workspace_bytes, L.tiles_end)) != S3R_OK) return st;
  return run_lse_bound(d, cmp_args(p, d, q, workspace, L), (const unsigned char*)workspace, L,
                       lse_bound, stream);
}

s3r_status speed3r_cmp_single_topk(const s3r_params* p, const void* q, const void* workspace,
                                   size_t workspace_bytes, const float* lse_bound, float* lse,
                                   float* o_cmp, int32_t* sel_idx, int32_t* redo,
                                   hipStream_t stream) {
  Dims d;
  s3r_status st = check_params(p, &d);
  if (st != S3R_OK) return st;
  if (!tok_ok(q) || !lse_bound || !aligned(lse_bound, 4) || !lse || !aligned(lse, 4) ||
      !o_cmp || !aligned(o_cmp, 16) || !sel_idx || !aligned(sel_idx, 4) || !redo ||
      !aligned(redo, 16))
    return S3R_ERR_INVALID_ARG;
  if (!d.single_ok) return S3R_ERR_UNSUPPORTED;
  const Layout L = layout(d);
  if ((st = check_ws(workspace, workspace_bytes, L.tiles_end)) != S3R_OK) return st;
  CmpArgs a = cmp_args(p, d, q, workspace, L);
  a.o_cmp = o_cmp;
  a.sel = sel_idx;
  a.n_sel = (int32_t)d.k_eff;
  a.forced = (int32_t)d.forced;
  a.topk = (int32_t)d.topk;
  a.own = d.own;
  return run_single(a, lse_bound, lse, redo, stream);
}

s3r_status speed3r_topk(const s3r_params* p, const float* score, int32_t* sel_idx,
                        hipStream_t stream) {
  Dims d;
  s3r_status st = check_params(p, &d);
  if (st != S3R_OK) return st;
  if (!score || !aligned(score, 4) || !sel_idx || !aligned(sel_idx, 4))
    return S3R_ERR_INVALID_ARG;
  if (d.Nb > kMaxBlocks) return S3R_ERR_UNSUPPORTED;
  TopkArgs a;
  a.score = score; a.ld = d.ld; a.Nb = d.Nb; a.n_rows = (int64_t)d.H * d.Nb;
  a.n_sel = (int32_t)d.k_eff; a.forced = (int32_t)d.forced; a.sel = sel_idx;
  a.topk = (int32_t)d.topk; a.own = d.own;
  return hip_status(launch_topk(a, stream));
}

s3r_status speed3r_sel_combine(const s3r_params* p, const void* q, const void* workspace,
                               size_t workspace_bytes, const int32_t* sel_idx,
                               const float* o_cmp, const float* gates, void* out,
                               float* o_sel, hipStream_t stream) {
  Dims d;
  s3r_status st = check_params(p, &d);
  if (st != S3R_OK) return st;
  if (!tok_ok(q) || !sel_idx || !aligned(sel_idx, 4) || !o_cmp || !aligned(o_cmp, 16) ||
      !gates || !aligned(gates, 4) || !out || !aligned(out, 8) || (o_sel && !aligned(o_sel, 16)))
    return S3R_ERR_INVALID_ARG;
  const Layout L = layout(d);
  if ((st = check_ws(workspace, workspace_bytes, L.tiles_end)) != S3R_OK) return st;
  AttnArgs a = attn_args(p, d, q, (const unsigned char*)workspace + L.raw);
  a.sel = sel_idx; a.o_cmp = o_cmp; a.gates = gates; a.o_sel = o_sel; a.out = (uint16_t*)out;
  return hip_status(launch_sel(a, stream));
}

s3r_status speed3r_sparse_attn_fwd(const s3r_params* p, const void* q, const void* k,
                                   const void* v, const float* gates, void* out,
                                   int32_t* sel_idx, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  Dims d;
  s3r_status st = check_params(p, &d);
  if (st != S3R_OK) return st;
  if (p->cmp_mode == S3R_CMP_SINGLE && !d.single_ok) return S3R_ERR_UNSUPPORTED;
  if (!tok_ok(q) || !tok_ok(k) || !tok_ok(v) || !gates || !aligned(gates, 4) || !out ||
      !aligned(out, 8) || (sel_idx && !aligned(sel_idx, 4)))
    return S3R_ERR_INVALID_ARG;
  const Layout L = layout(d);
  if ((st = check_ws(workspace, workspace_bytes, L.end)) != S3R_OK) return st;
  return run_forward(p, d, L, q, k, v, gates, out, sel_idx, (unsigned char*)workspace, nullptr,
                     stream);
}

size_t speed3r_noalloc_scratch_bytes(void) { return kScratchBytes; }

s3r_status speed3r_sparse_attn_fwd_noalloc(const s3r_params* p, const void* q, const void* k,
                                           const void* v, const float* gates, void* out,
                                           int32_t* sel_idx, hipStream_t stream) {
  Dims d;
  s3r_status st = check_params(p, &d);
  if (st != S3R_OK) return st;
  if (p->cmp_mode == S3R_CMP_SINGLE && !d.single_ok) return S3R_ERR_UNSUPPORTED;
  if (!tok_ok(q) || !tok_ok(k) || !tok_ok(v) || !gates || !aligned(gates, 4) || !out ||
      !aligned(out, 8) || (sel_idx && !aligned(sel_idx, 4)))
    return S3R_ERR_INVALID_ARG;
  const Layout L = layout(d);
  if (L.end > kScratchBytes) return S3R_ERR_SCRATCH;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != S3R_OK) return st;
  return run_forward(p, d, L, q, k, v, gates, out, sel_idx, (unsigned char*)ws, nullptr,
                     stream);
}

size_t speed3r_train_workspace_size(const s3r_params* p) {
  Dims d;
  return check_params(p, &d) == S3R_OK ? train_layout(d).end : 0;
}

s3r_status speed3r_sparse_attn_fwd_train(const s3r_params* p, const void* q, const void* k,
                                         const void* v, const float* gates, void* out,
                                         int32_t* sel_idx, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
  Dims d;
  s3r_status st = check_params(p, &d);
  if (st != S3R_OK) return st;
  if (p->cmp_mode == S3R_CMP_SINGLE && !d.single_ok) return S3R_ERR_UNSUPPORTED;
  if (!tok_ok(q) || !tok_ok(k) || !tok_ok(v) || !gates || !aligned(gates, 4) || !out ||
      !aligned(out, 8) || (sel_idx && !aligned(sel_idx, 4)))
    return S3R_ERR_INVALID_ARG;
  const Layout L = layout(d);
  const TrainLayout TL = train_layout(d);
  if ((st = check_ws(workspace, workspace_bytes, TL.end)) != S3R_OK) return st;
  unsigned char* ws = (unsigned char*)workspace;
  if ((st = run_forward(p, d, L, q, k, v, gates, out, nullptr, ws, &TL, stream)) != S3R_OK)
    return st;
  if (sel_idx)
    return hip_status(hipMemcpyAsync(sel_idx, ws + L.sel,
                                     (size_t)d.H * d.Nb * d.k_eff * sizeof(int32_t),
                                     hipMemcpyDeviceToDevice, stream));
  return S3R_OK;
}

size_t speed3r_bwd_workspace_size(const s3r_params* p) {
  Dims d;
  return check_params(p, &d) == S3R_OK ? bwd_layout(d).end : 0;
}

s3r_status speed3r_sparse_attn_bwd(const s3r_params* p, const void* q, const void* k,
                                   const void* v, const float* gates, const void* dout,
                                   int64_t dout_stride_t, int64_t dout_stride_h,
                                   const void* train_workspace, size_t train_workspace_bytes,
                                   float* dq, float* dk, float* dv, float* dgates,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Dims d;
  s3r_status st = check_params(p, &d);
  if (st != S3R_OK) return st;
  if (!tok_ok(q) || !tok_ok(k) || !tok_ok(v) || !gates || !aligned(gates, 4) || !tok_ok(dout) ||
      !valid_stride(dout_stride_t) || !valid_stride(dout_stride_h) || !dq || !aligned(dq, 16) ||
      !dk || !aligned(dk, 16) || !dv || !aligned(dv, 16) || !dgates || !aligned(dgates, 4))
    return S3R_ERR_INVALID_ARG;
  const Layout L = layout(d);
  const TrainLayout TL = train_layout(d);
  const BwdLayout BL = bwd_layout(d);
  if ((st = check_ws(train_workspace, train_workspace_bytes, TL.end)) != S3R_OK) return st;
  if ((st = check_ws(workspace, workspace_bytes, BL.end)) != S3R_OK) return st;
  const unsigned char* tw = (const unsigned char*)train_workspace;
  unsigned char* ws = (unsigned char*)workspace;

  // operand images of q, dout (query tiles), v, k (raw) and the block means (pooled)
  RecPackArgs r;
  r.H = d.H;
  r.half = d.half;
  auto pack = [&](const void* src, int64_t st_, int64_t sh_, int64_t rows, int64_t n_tiles,
                  unsigned char* dst, int64_t tile_bytes, int r_off, int tr_off, int kind) {
    r.src = src; r.st = st_; r.sh = sh_; r.rows = rows; r.n_tiles = n_tiles; r.dst = dst;
    r.tile_bytes = tile_bytes; r.r_off = r_off; r.tr_off = tr_off;
    return hip_status(launch_rec_pack(r, kind, stream));
  };
  const int64_t nk = d.n_ktiles, nc = d.n_ctiles, Nb64 = d.Nb * kD;
  if ((st = pack(q, p->q_stride_t, p->q_stride_h, d.T, nk, ws + BL.qtiles, kQImgBytes, 0, -1,
                 0)) != S3R_OK ||
      (st = pack(dout, dout_stride_t, dout_stride_h, d.T, nk, ws + BL.qtiles, kQImgBytes, 4096,
                 -1, 0)) != S3R_OK ||
      (st = pack(v, p->v_stride_t, p->v_stride_h, d.T, nk, ws + BL.raw_bwd, kBwdTileBytes, 0, -1,
                 0)) != S3R_OK ||
      (st = pack(k, p->k_stride_t, p->k_stride_h, d.T, nk, ws + BL.raw_bwd, kBwdTileBytes, -1,
                 4096, 0)) != S3R_OK ||
      (st = pack(tw + TL.v_mean, kD, Nb64, d.Nb, nc, ws + BL.pooled_bwd, kBwdTileBytes, 0, -1,
                 1)) != S3R_OK ||
      (st = pack(tw + TL.k_mean, kD, Nb64, d.Nb, nc, ws + BL.pooled_bwd, kBwdTileBytes, -1, 4096,
                 1)) != S3R_OK)
    return st;

  // per-token scalars and gate gradients
  BwdScalarArgs sa;
  sa.T = d.T; sa.H = d.H; sa.half = d.half;
  sa.lse_cmp = (const float*)(tw + L.lse);
  sa.lse_sel = (const float*)(tw + TL.lse_sel);
  sa.gates = gates; sa.gate_st = p->gate_stride_t;
  sa.dout = (const uint16_t*)dout; sa.d_st = dout_stride_t; sa.d_sh = dout_stride_h;
  sa.o_cmp = (const float*)(tw + L.o_cmp);
  sa.o_sel = (const float*)(tw + TL.o_sel);
  sa.qs = (float*)(ws + BL.qs);
  const bool token_gates = p->gate_stride_t != 0;
  sa.dg_tok = token_gates ? dgates : (float*)(ws + BL.dg_tok);
  sa.dg_st = token_gates ? p->gate_stride_t : 2;          // scratch: [H][T][2]
  sa.dg_sh = token_gates ? 2 : 2 * d.T;
  if ((st = hip_status(launch_bwd_scalars(sa, stream))) != S3R_OK) return st;
  if (!token_gates &&
      (st = hip_status(launch_gate_reduce(sa.dg_tok, d.T, d.H, dgates, stream))) != S3R_OK)
    return st;

  BwdArgs b;
  memset(&b, 0, sizeof(b));
  b.T = d.T; b.Nb = d.Nb; b.n_ctiles = nc; b.n_ktiles = nk; b.H = d.H; b.B = d.B;
  b.half = d.half;
  b.scale = d.scale; b.logit_mult = d.scale * kLog2e;
  b.pooled = tw + L.pooled; b.pooled_bwd = ws + BL.pooled_bwd;
  b.raw = tw + L.raw; b.raw_bwd = ws + BL.raw_bwd;
  b.qtiles = ws + BL.qtiles; b.qs = (const float*)(ws + BL.qs);
  b.q = (const uint16_t*)q; b.q_st = p->q_stride_t; b.q_sh = p->q_stride_h;
  b.dout = (const uint16_t*)dout; b.d_st = dout_stride_t; b.d_sh = dout_stride_h;
  b.sel = (const int32_t*)(tw + L.sel); b.n_sel = (int32_t)d.k_eff;
  b.bitmap = (const uint32_t*)(ws + BL.bitmap); b.bm_words = BL.bm_words;
  b.dkc = (float*)(ws + BL.dkc); b.dvc = (float*)(ws + BL.dvc);
  b.dkc_part = (float*)(ws + BL.dkv_part);
  b.dvc_part = (float*)(ws + BL.dkv_part +
                        align256((size_t)kDkvParts * d.H * d.Nb * kD * sizeof(float)));
  b.dq = dq; b.dk = dk; b.dv = dv;

  // selection bitmap (cleared with a kernel, not a memset)
  if ((st = hip_status(launch_fill_zero((float*)(ws + BL.bitmap),
                                        (int64_t)d.H * d.Nb * BL.bm_words, stream))) != S3R_OK ||
      (st = hip_status(launch_sel_bitmap(b, (uint32_t*)(ws + BL.bitmap), stream))) != S3R_OK)
    return st;
  if ((st = hip_status(launch_cmp_dq(b, stream))) != S3R_OK) return st;
  if ((st = hip_status(launch_cmp_dkv(b, stream))) != S3R_OK) return st;
  if ((st = hip_status(launch_sel_dq(b, stream))) != S3R_OK) return st;
  return hip_status(launch_sel_dkv(b, stream));
}

s3r_status speed3r_dense_attn_fwd(const s3r_params* p, const void* q, const void* k,
                                  const void* v, void* out, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  Dims d;
  s3r_status st = check_params(p, &d);
  if (st != S3R_OK) return st;
  if (!tok_ok(q) || !tok_ok(k) || !tok_ok(v) || !out || !aligned(out, 8))
    return S3R_ERR_INVALID_ARG;
  const size_t need = align256((size_t)d.H * d.n_ktiles * kRawTileBytes);
  if ((st = check_ws(workspace, workspace_bytes, need)) != S3R_OK) return st;
  unsigned char* raw = (unsigned char*)workspace;
  if ((st = hip_status(launch_pack(pack_args(p, d, k, v, raw, nullptr), stream))) != S3R_OK)
    return st;
  AttnArgs a = attn_args(p, d, q, raw);
  a.out = (uint16_t*)out;
  return hip_status(launch_dense(a, stream));
}

int64_t speed3r_window_source(const s3r_windows* w, int64_t pos) {
  WindowLayout L;
  int64_t T;
  if (!window_layout(w, &L, &T) || pos < 0 || pos >= T) return -1;
  return window_source(L, pos);
}

s3r_status speed3r_window_permute(const s3r_windows* w, int32_t H, const void* src,
                                  int64_t src_stride_t, int64_t src_stride_h, void* dst,
                                  int64_t dst_stride_t, int64_t dst_stride_h, int32_t inverse,
                                  hipStream_t stream) {
  WindowLayout L;
  int64_t T;
  if (!window_layout(w, &L, &T) || H < 1 || H > 65535 || !tok_ok(src) || !tok_ok(dst) ||
      !valid_stride(src_stride_t) || !valid_stride(src_stride_h) ||
      !valid_stride(dst_stride_t) || !valid_stride(dst_stride_h) ||
      (inverse != 0 && inverse != 1))
    return S3R_ERR_INVALID_ARG;
  return hip_status(launch_window_copy(
      copy_args(L, T, H, inverse, src, src_stride_t * 2, src_stride_h * 2, dst,
                dst_stride_t * 2, dst_stride_h * 2), 128, stream));
}

size_t speed3r_windows_workspace_size(const s3r_params* p, const s3r_windows* w) {
  Dims d;
  WindowLayout L;
  int64_t T;
  if (check_params(p, &d) != S3R_OK || !window_layout(w, &L, &T) || T != p->T) return 0;
  return window_ws(d, p->gate_stride_t != 0, layout(d).end).end;
}

s3r_status speed3r_sparse_attn_fwd_windows(const s3r_params* p, const s3r_windows* w,
                                           const void* q, const void* k, const void* v,
                                           const float* gates, void* out, int32_t* sel_idx,
                                           void* workspace, size_t workspace_bytes,
                                           hipStream_t stream) {
  Dims d;
  s3r_status st = check_params(p, &d);
  if (st != S3R_OK) return st;
  if (p->cmp_mode == S3R_CMP_SINGLE && !d.single_ok) return S3R_ERR_UNSUPPORTED;
  WindowLayout L;
  int64_t T;
  if (!window_layout(w, &L, &T) || T != p->T) return S3R_ERR_INVALID_ARG;
  if (!tok_ok(q) || !tok_ok(k) || !tok_ok(v) || !gates || !aligned(gates, 4) || !out ||
      !aligned(out, 16) || (sel_idx && !aligned(sel_idx, 4)))
    return S3R_ERR_INVALID_ARG;
  // per-token gates move as 8-byte (token, head) pairs
  if (p->gate_stride_t && (!aligned(gates, 8) || p->gate_stride_t % 2)) return S3R_ERR_INVALID_ARG;
  const bool token_gates = p->gate_stride_t != 0;
  const WindowWs W = window_ws(d, token_gates, layout(d).end);
  if ((st = check_ws(workspace, workspace_bytes, W.end)) != S3R_OK) return st;
  unsigned char* ws = (unsigned char*)workspace;
  const s3r_params pw = windowed_params(p);
  const int64_t row = (int64_t)d.H * kD * 2;
  const void* srcs[3] = {q, k, v};
  const int64_t st_t[3] = {p->q_stride_t, p->k_stride_t, p->v_stride_t};
  const int64_t st_h[3] = {p->q_stride_h, p->k_stride_h, p->v_stride_h};
  const size_t offs[3] = {W.q, W.k, W.v};
  for (int x = 0; x < 3; ++x) {
    st = hip_status(launch_window_copy(copy_args(L, T, d.H, 0, srcs[x], st_t[x] * 2,
                                                 st_h[x] * 2, ws + offs[x], row, kD * 2),
                                       128, stream));
    if (st != S3R_OK) return st;
  }
  const float* g = gates;
  if (token_gates) {
    st = hip_status(launch_window_copy(copy_args(L, T, d.H, 0, gates, p->gate_stride_t * 4, 8,
                                                 ws + W.gates, (int64_t)d.H * 8, 8),
                                       8, stream));
    if (st != S3R_OK) return st;
    g = (const float*)(ws + W.gates);
  }
  st = speed3r_sparse_attn_fwd(&pw, ws + W.q, ws + W.k, ws + W.v, g, ws + W.out, sel_idx,
                               ws + W.inner, workspace_bytes - W.inner, stream);
  if (st != S3R_OK) return st;
  return hip_status(launch_window_copy(copy_args(L, T, d.H, 1, ws + W.out, row, kD * 2, out,
                                                 row, kD * 2), 128, stream));
}

}  // extern "C"
