// C ABI of libspeed3r.so: argument validation, workspace layout and kernel launches.
// The functions are declared (and their contracts stated) in include/speed3r.h.
#include <math.h>
#include <string.h>

#include "../../include/speed3r.h"
#include "s3r_common.hpp"
#include "s3r_launch.hpp"

using namespace s3r;

namespace {

constexpr int64_t kMaxBlocks = 96 * 256;  // top-k holds a row of up to 96 keys per thread

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Dims {
  int64_t T, Nb, n_ctiles, n_ktiles, ld;
  int64_t k_eff;   // entries per selection row: forced prefix + chosen blocks (n_sel)
  int64_t forced;  // F' = min(forced_blocks, Nb)
  int32_t H, B;
  float scale;
  bool fold_topk;  // selection folded into the compression pass (no score matrix)
};

// Workspace regions, in this order, each 256-byte aligned.
struct Layout {
  size_t pooled, raw, lse, o_cmp, score, sel, tiles_end, end;
};

bool valid_stride(int64_t s) { return s >= 0 && (s % 8) == 0; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

s3r_status check_params(const s3r_params* p, Dims* d) {
  if (!p) return S3R_ERR_INVALID_ARG;
  if (p->T < 1 || p->H < 1 || p->topk < 1 || p->forced_blocks < 0) return S3R_ERR_INVALID_ARG;
  if (p->block < 1 || p->D < 1) return S3R_ERR_INVALID_ARG;
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
  d->B = p->block;
  d->Nb = (p->T + p->block - 1) / p->block;
  if (d->Nb > kMaxBlocks) return S3R_ERR_UNSUPPORTED;
  d->n_ctiles = (d->Nb + kTileKeys - 1) / kTileKeys;
  d->n_ktiles = (d->T + kTileKeys - 1) / kTileKeys;
  d->ld = d->n_ctiles * kTileKeys;
  d->forced = p->forced_blocks < d->Nb ? p->forced_blocks : d->Nb;
  const int64_t rest = d->Nb - d->forced;
  d->k_eff = d->forced + (p->topk < rest ? p->topk : rest);
  d->scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)kD);
  d->fold_topk = d->B <= 64 && d->k_eff - d->forced <= kFusedTopkMaxK;
  return S3R_OK;
}

Layout layout(const Dims& d) {
  Layout L;
  size_t off = 0;
  L.pooled = off;
  off += align256((size_t)d.H * d.n_ctiles * kPooledTileBytes);
  L.raw = off;
  off += align256((size_t)d.H * d.n_ktiles * kRawTileBytes);
  L.tiles_end = off;
  L.lse = off;
  off += align256((size_t)d.H * d.T * sizeof(float));
  L.o_cmp = off;
  off += align256((size_t)d.T * d.H * kD * sizeof(float));
  L.score = off;
  if (!d.fold_topk) off += align256((size_t)d.H * d.Nb * d.ld * sizeof(float));
  L.sel = off;
  off += align256((size_t)d.H * d.Nb * d.k_eff * sizeof(int32_t));
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
  a.T = d.T; a.Nb = d.Nb; a.n_tiles = d.n_ctiles; a.H = d.H; a.B = d.B;
  a.key_mult = d.scale * kLog2e;
  a.k_mean = k_mean; a.v_mean = v_mean;
  a.tiles = (unsigned char*)ws + L.pooled;
  return a;
}

PackArgs pack_args(const s3r_params* p, const Dims& d, const void* k, const void* v,
                   unsigned char* tiles) {
  PackArgs a;
  a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.k_st = p->k_stride_t; a.k_sh = p->k_stride_h; a.v_st = p->v_stride_t; a.v_sh = p->v_stride_h;
  a.T = d.T; a.n_tiles = d.n_ktiles; a.H = d.H;
  a.tiles = tiles;
  return a;
}

CmpArgs cmp_args(const s3r_params* p, const Dims& d, const void* q, const void* ws,
                 const Layout& L) {
  CmpArgs a;
  memset(&a, 0, sizeof(a));
  a.q = (const uint16_t*)q; a.q_st = p->q_stride_t; a.q_sh = p->q_stride_h;
  a.T = d.T; a.Nb = d.Nb; a.n_tiles = d.n_ctiles; a.H = d.H; a.B = d.B;
  a.tiles = (const unsigned char*)ws + L.pooled;
  a.ld = d.ld;
  return a;
}

AttnArgs attn_args(const s3r_params* p, const Dims& d, const void* q,
                   const unsigned char* raw_tiles) {
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.q = (const uint16_t*)q; a.q_st = p->q_stride_t; a.q_sh = p->q_stride_h;
  a.T = d.T; a.Nb = d.Nb; a.n_tiles = d.n_ktiles; a.H = d.H; a.B = d.B;
  a.logit_mult = d.scale * kLog2e;
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

}  // namespace

extern "C" {

const char* speed3r_status_string(s3r_status s) {
  switch (s) {
    case S3R_OK: return "S3R_OK";
    case S3R_ERR_INVALID_ARG: return "S3R_ERR_INVALID_ARG";
    case S3R_ERR_UNSUPPORTED: return "S3R_ERR_UNSUPPORTED";
    case S3R_ERR_WORKSPACE: return "S3R_ERR_WORKSPACE";
    case S3R_ERR_HIP: return "S3R_ERR_HIP";
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
  st = hip_status(launch_pool(pool_args(p, d, k, v, workspace, L, k_mean, v_mean), stream));
  if (st != S3R_OK) return st;
  return hip_status(
      launch_pack(pack_args(p, d, k, v, (unsigned char*)workspace + L.raw), stream));
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
  return hip_status(launch_cmp_fused_topk(a, stream));
}

s3r_status speed3r_topk(const s3r_params* p, const float* score, int32_t* sel_idx,
                        hipStream_t stream) {
  Dims d;
  s3r_status st = check_params(p, &d);
  if (st != S3R_OK) return st;
  if (!score || !aligned(score, 4) || !sel_idx || !aligned(sel_idx, 4))
    return S3R_ERR_INVALID_ARG;
  TopkArgs a;
  a.score = score; a.ld = d.ld; a.Nb = d.Nb; a.n_rows = (int64_t)d.H * d.Nb;
  a.n_sel = (int32_t)d.k_eff; a.forced = (int32_t)d.forced; a.sel = sel_idx;
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
  if (!tok_ok(q) || !tok_ok(k) || !tok_ok(v) || !gates || !aligned(gates, 4) || !out ||
      !aligned(out, 8) || (sel_idx && !aligned(sel_idx, 4)))
    return S3R_ERR_INVALID_ARG;
  const Layout L = layout(d);
  if ((st = check_ws(workspace, workspace_bytes, L.end)) != S3R_OK) return st;
  unsigned char* ws = (unsigned char*)workspace;
  float* lse = (float*)(ws + L.lse);
  float* o_cmp = (float*)(ws + L.o_cmp);
  float* score = (float*)(ws + L.score);
  int32_t* sel = sel_idx ? sel_idx : (int32_t*)(ws + L.sel);

  if ((st = hip_status(launch_pool(pool_args(p, d, k, v, ws, L, nullptr, nullptr), stream))) !=
      S3R_OK)
    return st;
  if ((st = hip_status(launch_pack(pack_args(p, d, k, v, ws + L.raw), stream))) != S3R_OK)
    return st;
  CmpArgs c = cmp_args(p, d, q, ws, L);
  c.lse = lse;
  if ((st = hip_status(launch_cmp_lse(c, stream))) != S3R_OK) return st;
  c.lse_in = lse;
  c.o_cmp = o_cmp;
  if (d.fold_topk) {
    c.sel = sel;
    c.n_sel = (int32_t)d.k_eff;
    c.forced = (int32_t)d.forced;
    if ((st = hip_status(launch_cmp_fused_topk(c, stream))) != S3R_OK) return st;
  } else {
    c.score = score;
    if ((st = run_cmp_fused(d, c, stream)) != S3R_OK) return st;
    TopkArgs t;
    t.score = score; t.ld = d.ld; t.Nb = d.Nb; t.n_rows = (int64_t)d.H * d.Nb;
    t.n_sel = (int32_t)d.k_eff; t.forced = (int32_t)d.forced; t.sel = sel;
    if ((st = hip_status(launch_topk(t, stream))) != S3R_OK) return st;
  }
  AttnArgs a = attn_args(p, d, q, ws + L.raw);
  a.sel = sel; a.o_cmp = o_cmp; a.gates = gates; a.o_sel = nullptr; a.out = (uint16_t*)out;
  return hip_status(launch_sel(a, stream));
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
  if ((st = hip_status(launch_pack(pack_args(p, d, k, v, raw), stream))) != S3R_OK) return st;
  AttnArgs a = attn_args(p, d, q, raw);
  a.out = (uint16_t*)out;
  return hip_status(launch_dense(a, stream));
}

}  // extern "C"
