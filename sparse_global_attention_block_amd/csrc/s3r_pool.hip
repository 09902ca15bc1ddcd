// Block pooling (compression branch input) and raw key/value packing.
//
// Pooling follows the compression branch of the Speed3R technical summary (gist.science,
// "Methodologie" section 1): each contiguous block of B tokens of the keys and values is
// replaced by its mean. The packing kernel streams k and v once (raw tiles plus the blocks'
// column sums) and is bound by HBM bandwidth; pooling then reads only the sums.
#include "s3r_common.hpp"
#include "s3r_launch.hpp"

namespace s3r {

// One work-group per (head, tile of 32 consecutive blocks). Thread (slot m = tid/8, dim group
// d8 = tid%8) takes block 32*tile + m: the f32 column sums of its k and v rows (written by the
// packing kernel, which reads k and v once for both), divided by the block's token count
// (IEEE division). Writes the f32 means (optional) and one pooled tile: the mean keys scaled
// by key_mult = scale*log2(e) as a hi + lo pair in the input type (hi = round(x), lo =
// round(x - hi); bf16 or fp16), and the mean values times v_mult (a power of two) as fp16 V^T
// records. Optionally also the group keys (means of 8 consecutive scaled pooled keys) of the
// bound pass, in the K records of group tiles.
template <bool kHalf>
__global__ __launch_bounds__(256) void pool_kernel(PoolArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char stage[kPooledTileBytes];
  const int tid = threadIdx.x;
  const int m = tid >> 3, d8 = tid & 7;
  const int64_t tile = blockIdx.x;
  const int h = blockIdx.y;
  const int64_t j = tile * kTileKeys + m;
  float ks[8], vs[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { ks[e] = 0.f; vs[e] = 0.f; }
  if (j < a.Nb) {
    const int64_t t0 = j * a.B;
    const int64_t n = ((t0 + a.B < a.T) ? t0 + a.B : a.T) - t0;
    const float4* bs = reinterpret_cast<const float4*>(a.bsum + ((int64_t)h * a.Nb + j) * 128);
    const float4 k0 = bs[2 * d8], k1 = bs[2 * d8 + 1], v0 = bs[16 + 2 * d8], v1 = bs[17 + 2 * d8];
    const float kx[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
    const float vx[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    const float fn = (float)n;
#pragma unroll
    for (int e = 0; e < 8; ++e) { ks[e] = kx[e] / fn; vs[e] = vx[e] / fn; }
    if (a.k_mean) {
      float4* km = reinterpret_cast<float4*>(a.k_mean + ((int64_t)h * a.Nb + j) * kD + d8 * 8);
      km[0] = make_float4(ks[0], ks[1], ks[2], ks[3]);
      km[1] = make_float4(ks[4], ks[5], ks[6], ks[7]);
    }
    if (a.v_mean) {
      float4* vm = reinterpret_cast<float4*>(a.v_mean + ((int64_t)h * a.Nb + j) * kD + d8 * 8);
      vm[0] = make_float4(vs[0], vs[1], vs[2], vs[3]);
      vm[1] = make_float4(vs[4], vs[5], vs[6], vs[7]);
    }
  }
  // K hi / lo chunks (16 bytes each, already in record order)
  u16 hi[8], lo[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = ks[e] * a.key_mult;
    hi[e] = float_to_in<kHalf>(x);
    lo[e] = float_to_in<kHalf>(x - in_to_float<kHalf>(hi[e]));
  }
  const int koff = k_chunk_offset(m, d8);
  uint4 hv, lv;
  hv.x = hi[0] | ((uint32_t)hi[1] << 16); hv.y = hi[2] | ((uint32_t)hi[3] << 16);
  hv.z = hi[4] | ((uint32_t)hi[5] << 16); hv.w = hi[6] | ((uint32_t)hi[7] << 16);
  lv.x = lo[0] | ((uint32_t)lo[1] << 16); lv.y = lo[2] | ((uint32_t)lo[3] << 16);
  lv.z = lo[4] | ((uint32_t)lo[5] << 16); lv.w = lo[6] | ((uint32_t)lo[7] << 16);
  *reinterpret_cast<uint4*>(stage + koff) = hv;
  *reinterpret_cast<uint4*>(stage + 4 * kRecBytes + koff) = lv;
  // V^T: 8 scattered bf16 per thread
  u16* vt = reinterpret_cast<u16*>(stage + 8 * kRecBytes);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    int rec, lane, slot;
    vt_position(m, d8 * 8 + e, rec, lane, slot);
    vt[(rec * 64 + lane) * 8 + slot] = f16_bits(vs[e] * a.v_mult);
  }
  if (a.group_tiles) {
    // group key 4*tile + wave: the mean of the scaled pooled keys 8*(4*tile + wave)..+7, held
    // by lanes 8*m' + d8 of this wave (m' = 0..7), written as a hi + lo pair like them
    const int64_t gk = tile * 4 + (tid >> 6);
    float gx[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = ks[e] * a.key_mult;
      x += __shfl_xor(x, 8);
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      gx[e] = x * 0.125f;
    }
    if ((tid & 63) < 8 && gk < kTileKeys * a.n_gtiles) {
      u16 ghi[8], glo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ghi[e] = float_to_in<kHalf>(gx[e]);
        glo[e] = float_to_in<kHalf>(gx[e] - in_to_float<kHalf>(ghi[e]));
      }
      unsigned char* gt =
          a.group_tiles + ((int64_t)h * a.n_gtiles + gk / kTileKeys) * kPooledTileBytes;
      const int goff = k_chunk_offset((int)(gk % kTileKeys), d8);
      uint4 gh, gl;
      gh.x = ghi[0] | ((uint32_t)ghi[1] << 16); gh.y = ghi[2] | ((uint32_t)ghi[3] << 16);
      gh.z = ghi[4] | ((uint32_t)ghi[5] << 16); gh.w = ghi[6] | ((uint32_t)ghi[7] << 16);
      gl.x = glo[0] | ((uint32_t)glo[1] << 16); gl.y = glo[2] | ((uint32_t)glo[3] << 16);
      gl.z = glo[4] | ((uint32_t)glo[5] << 16); gl.w = glo[6] | ((uint32_t)glo[7] << 16);
      *reinterpret_cast<uint4*>(gt + goff) = gh;
      *reinterpret_cast<uint4*>(gt + 4 * kRecBytes + goff) = gl;
    }
  }
  __syncthreads();
  uint4* dst = reinterpret_cast<uint4*>(a.tiles + ((int64_t)h * a.n_tiles + tile) * kPooledTileBytes);
  const uint4* src = reinterpret_cast<const uint4*>(stage);
#pragma unroll
  for (int r = 0; r < kPooledTileBytes / (16 * 256); ++r) dst[r * 256 + tid] = src[r * 256 + tid];
}

// One work-group per (head, group of kPackTiles tiles of 32 tokens). Thread (key m, dims d8)
// copies 16 bytes of k into its K record slot and scatters 8 values of v, times v_mult and
// converted to fp16, into the V^T records through LDS. Tokens beyond T are zero. In LDS, lane l's 16 bytes of a
// V^T record sit at slot l ^ ((l >> 3) & 7): every lane of one 2-byte store writes the same
// dim modulo 8, which the plain layout puts in 2 of the 32 banks; the copy out reads through
// the same swizzle (a permutation inside aligned groups of 8 slots, free of conflicts).
// With bsum set, the same read of k and v also yields the pooling sums: each thread puts its
// 8 + 8 values in an LDS row of the tile (rows padded to 129 floats: conflict-free both ways),
// and thread c of the first 128 (of 256 for B = 16, one per half tile) adds column c over the
// tile's rows of its block in row order, and over the tiles of a block in tile order
// (kPackTiles * 32 = 128 tokens is a whole number of blocks).
constexpr int kPackTiles = 4;
template <bool kHalf>
__global__ __launch_bounds__(256) void pack_kernel(PackArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char stage[4 * kRecBytes];
  __shared__ float red[kTileKeys][129];
  const int tid = threadIdx.x;
  const int m = tid >> 3, d8 = tid & 7;
  const int h = blockIdx.y;
  float run = 0.f;  // (bsum, B >= 32, tid < 128) running sum of column tid over the block
  for (int it = 0; it < kPackTiles; ++it) {
    const int64_t tile = (int64_t)blockIdx.x * kPackTiles + it;
    if (tile >= a.n_tiles) break;
    const int64_t t = tile * kTileKeys + m;
    uint4 kk = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
    if (t < a.T) {
      kk = *reinterpret_cast<const uint4*>(a.k + t * a.k_st + (int64_t)h * a.k_sh + d8 * 8);
      vv = *reinterpret_cast<const uint4*>(a.v + t * a.v_st + (int64_t)h * a.v_sh + d8 * 8);
    }
    unsigned char* out = a.tiles + ((int64_t)h * a.n_tiles + tile) * kRawTileBytes;
    *reinterpret_cast<uint4*>(out + k_chunk_offset(m, d8)) = kk;
    u16* vt = reinterpret_cast<u16*>(stage);
    float vx[8];
    unpack8<kHalf>(vv, vx);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int rec, lane, slot;
      vt_position(m, d8 * 8 + e, rec, lane, slot);
      // exact for fp16 inputs (v_mult = 1) and for bf16 values of magnitude 2^-6..2^24
      vt[(rec * 64 + (lane ^ ((lane >> 3) & 7))) * 8 + slot] = f16_bits(vx[e] * a.v_mult);
    }
    if (a.bsum) {
      float kx[8];
      unpack8<kHalf>(kk, kx);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        red[m][d8 * 8 + e] = kx[e];
        red[m][64 + d8 * 8 + e] = vx[e];
      }
    }
    __syncthreads();
    uint4* dst = reinterpret_cast<uint4*>(out + 4 * kRecBytes);
    const int l = tid & 63;
    dst[tid] = reinterpret_cast<const uint4*>(stage)[(tid & ~63) | (l ^ ((l >> 3) & 7))];
    if (a.bsum) {
      if (a.B >= kTileKeys) {
        if (tid < 128) {
          float s = 0.f;
#pragma unroll 8
          for (int r = 0; r < kTileKeys; ++r) s += red[r][tid];
          run += s;
          // the block ends with this tile
          if ((tile + 1) * kTileKeys % a.B == 0 || tile + 1 == a.n_tiles) {
            const int64_t blk = tile * kTileKeys / a.B;
            a.bsum[((int64_t)h * a.Nb + blk) * 128 + tid] = run;
            run = 0.f;
          }
        }
      } else {  // B = 16: two blocks per tile
        const int half = tid >> 7, c = tid & 127;
        float s = 0.f;
#pragma unroll 8
        for (int r = 0; r < 16; ++r) s += red[16 * half + r][c];
        const int64_t blk = 2 * tile + half;
        if (blk < a.Nb) a.bsum[((int64_t)h * a.Nb + blk) * 128 + c] = s;
      }
    }
    __syncthreads();
  }
}

hipError_t launch_pool(const PoolArgs& a, hipStream_t s) {
  dim3 grid((unsigned)a.n_tiles, (unsigned)a.H);
  if (a.half) hipLaunchKernelGGL((pool_kernel<true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((pool_kernel<false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pack(const PackArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.n_tiles + kPackTiles - 1) / kPackTiles), (unsigned)a.H);
  if (a.half) hipLaunchKernelGGL((pack_kernel<true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((pack_kernel<false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace s3r
