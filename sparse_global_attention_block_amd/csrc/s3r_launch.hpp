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
  float key_mult;          // scale * log2(e), folded into the packed pooled keys
  float* k_mean; float* v_mean;  // optional f32 [H][Nb][64]
  unsigned char* tiles;    // [H][n_tiles][12 KB]
};

struct PackArgs {
  const uint16_t* k; const uint16_t* v;
  int64_t k_st, k_sh, v_st, v_sh;
  int64_t T, n_tiles;
  int32_t H;
  unsigned char* tiles;    // [H][n_tiles][8 KB]
};

struct CmpArgs {
  const uint16_t* q;
  int64_t q_st, q_sh;
  int64_t T, Nb, n_tiles;  // n_tiles = ceil(Nb / 32)
  int32_t H, B;
  const unsigned char* tiles;  // pooled tiles
  float* lse;              // [H][T] natural log (written by the LSE pass, read by the fused pass)
  const float* lse_in;
  float* o_cmp;            // [T][H][64]
  float* score;            // [H][Nb][ld]
  int64_t ld;
  int32_t* sel;            // running top-k output [H][Nb][n_sel] (fused selection only)
  int32_t n_sel;           // row length: forced prefix + chosen blocks
  int32_t forced;          // F': blocks 0..F'-1 always selected, top-k over the rest
};

struct TopkArgs {
  const float* score;
  int64_t ld;
  int64_t Nb;
  int64_t n_rows;          // H * Nb
  int32_t n_sel;           // row length of sel
  int32_t forced;          // F': blocks 0..F'-1 always selected, top-(n_sel - F') of the rest
  int32_t* sel;            // [n_rows][n_sel]
};

struct AttnArgs {
  const uint16_t* q;
  int64_t q_st, q_sh;
  int64_t T, Nb, n_tiles;  // raw tiles: n_tiles = ceil(T / 32)
  int32_t H, B;
  float logit_mult;        // scale * log2(e)
  const unsigned char* tiles;  // raw packed k/v tiles
  // selection only
  const int32_t* sel; int32_t k_eff;  // k_eff = entries per selection row (n_sel)
  const float* o_cmp;
  const float* gates; int64_t gate_st;
  float* o_sel;            // optional
  uint16_t* out;           // bf16 [T][H][64]
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

hipError_t launch_pool(const PoolArgs& a, hipStream_t s);
hipError_t launch_pack(const PackArgs& a, hipStream_t s);
hipError_t launch_cmp_lse(const CmpArgs& a, hipStream_t s);
hipError_t launch_cmp_fused(const CmpArgs& a, hipStream_t s);
hipError_t launch_cmp_fused_topk(const CmpArgs& a, hipStream_t s);
constexpr int kFusedTopkMaxK = 64;  // the running top-k keeps one entry per lane
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
hipError_t launch_sel(const AttnArgs& a, hipStream_t s);
hipError_t launch_dense(const AttnArgs& a, hipStream_t s);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);
hipError_t launch_window_copy(const WindowCopyArgs& a, int row_bytes, hipStream_t s);

}  // namespace s3r
