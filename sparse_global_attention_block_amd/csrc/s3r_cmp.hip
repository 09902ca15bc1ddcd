// Compression branch: attention of every query to all pooled (coarse) tokens, in two passes.
//
// Speed3R technical summary (gist.science), "Methodologie" section 1: the compression branch
// attends at coarse resolution to pooled tokens and produces the score matrix that steers the
// selection. The score of (query block i, key block j) is read here as the sum over the
// block's queries of the normalised coarse attention probabilities, which needs each query's
// log-sum-exp before any probability is final; hence two passes over the coarse tokens:
//   pass 1 (cmp_lse):   L_t = log sum_j exp(c_tj)
//   pass 2 (cmp_fused): P_tj = exp(c_tj - L_t), O_cmp_t = sum_j P_tj Vc_j,
//                       Score[i][j] = sum_{t in block i} P_tj
// with c_tj = scale * q_t . Kc_j. Both passes are MFMA-bound (bf16 16x16x32, f32 accumulate).
//
// Work decomposition: a work-group of 4 waves owns 256 consecutive queries of one head; each
// wave holds 64 queries (4 column tiles of 16) as resident B operands and streams the pooled
// tiles (32 coarse tokens each) through a double-buffered LDS ring. The accumulator tile is
// S^T (keys x queries): lane l holds query l%16 and keys 4*(l/16)+r, so P feeds the P.V MFMA
// directly as its B operand (in fp16, against fp16 pooled values). The pooled keys arrive
// pre-multiplied by scale*log2(e) as bf16 hi + lo, so logits come out in base-2 units; the query's offset (-running max in pass 1,
// -L_t*log2(e) in pass 2) is the MFMA's C input, leaving one exp2 per logit on the VALU.
#include "s3r_common.hpp"
#include "s3r_launch.hpp"

namespace s3r {

constexpr int kCmpWaves = 4;
constexpr int kCmpQueries = 64 * kCmpWaves;

// kQB: query blocks per wave (64 / B for B <= 64, else 1; B = 128 blocks span two waves and
// their scores are completed with a second atomic add onto a zeroed matrix).
template <bool kFused, int kQB>
__global__ __launch_bounds__(256) void cmp_kernel(CmpArgs a) {
  constexpr int kTileU4 = (kFused ? 12 : 8) * kRecBytes / 16;  // bytes of a tile this pass reads
  constexpr int kLoads = kTileU4 / 256;
  __shared__ uint4 lds[2][kTileU4];

  const int64_t n_qtiles = (a.T + kCmpQueries - 1) / kCmpQueries;
  const int64_t total = (int64_t)a.H * n_qtiles;
  const int64_t logical = xcd_logical_id(blockIdx.x, total);
  if (logical >= total) return;
  const int h = (int)(logical / n_qtiles);
  const int64_t qt = logical % n_qtiles;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, li = lane & 15;
  const int64_t q0 = qt * kCmpQueries + wave * 64;

  // Resident query operands: column tile nt, dim chunk c.
  bf16x8 qb[4][2];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int64_t t = q0 + 16 * nt + li;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      if (t < a.T) {
        qb[nt][c] = *reinterpret_cast<const bf16x8*>(a.q + t * a.q_st + (int64_t)h * a.q_sh +
                                                      32 * c + 8 * g);
      } else {
        qb[nt][c] = bf16x8{};
      }
    }
  }

  const uint4* tiles = reinterpret_cast<const uint4*>(a.tiles) +
                       (int64_t)h * a.n_tiles * (kPooledTileBytes / 16);
  constexpr int kTileStrideU4 = kPooledTileBytes / 16;

  // Per-lane softmax state. Pass 1: running offset m (base 2) and partial sum l of this lane's
  // keys; pass 2: the fixed offset L_t*log2(e).
  float off[4], lsum[4];
  floatx4 cneg[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int64_t t = q0 + 16 * nt + li;
    if constexpr (kFused) {
      off[nt] = (t < a.T) ? a.lse_in[(int64_t)h * a.T + t] * kLog2e : INFINITY;
    } else {
      off[nt] = 0.f;
    }
    lsum[nt] = 0.f;
    cneg[nt] = floatx4{-off[nt], -off[nt], -off[nt], -off[nt]};
  }
  floatx4 o[4][4];
  if constexpr (kFused) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) o[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  uint4 stg[kLoads];
#pragma unroll
  for (int r = 0; r < kLoads; ++r) stg[r] = tiles[r * 256 + tid];
#pragma unroll
  for (int r = 0; r < kLoads; ++r) lds[0][r * 256 + tid] = stg[r];
  __syncthreads();

  constexpr int kNtPerQB = 4 / kQB;

  for (int64_t tau = 0; tau < a.n_tiles; ++tau) {
    const int buf = (int)(tau & 1);
    const bool has_next = tau + 1 < a.n_tiles;
    if (has_next) {
      const uint4* src = tiles + (tau + 1) * kTileStrideU4;
#pragma unroll
      for (int r = 0; r < kLoads; ++r) stg[r] = src[r * 256 + tid];
    }
    const uint4* L = lds[buf];

    floatx4 acc[2][4];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const bf16x8 h0 = *reinterpret_cast<const bf16x8*>(&L[(2 * s2 + 0) * 64 + lane]);
      const bf16x8 h1 = *reinterpret_cast<const bf16x8*>(&L[(2 * s2 + 1) * 64 + lane]);
      const bf16x8 l0 = *reinterpret_cast<const bf16x8*>(&L[256 + (2 * s2 + 0) * 64 + lane]);
      const bf16x8 l1 = *reinterpret_cast<const bf16x8*>(&L[256 + (2 * s2 + 1) * 64 + lane]);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        floatx4 x = mfma16(h0, qb[nt][0], cneg[nt]);
        x = mfma16(h1, qb[nt][1], x);
        x = mfma16(l0, qb[nt][0], x);
        acc[s2][nt] = mfma16(l1, qb[nt][1], x);
      }
    }
    if (tau == a.n_tiles - 1) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t key = tau * kTileKeys + 16 * s2 + 4 * g + r;
          if (key >= a.Nb) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) acc[s2][nt][r] = -INFINITY;
          }
        }
    }

    if constexpr (!kFused) {
      // ---- pass 1: partial sums with a lazily moved offset -------------------------------
      bool bad = false;
      float prev[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        float s = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int r = 0; r < 4; ++r) s += fast_exp2(acc[s2][nt][r]);
        prev[nt] = lsum[nt];
        lsum[nt] += s;
        // the sum must stay inside [2^-64, 2^64]: otherwise move the offset to this tile's max
        bad |= !(lsum[nt] >= 0x1p-64f && lsum[nt] <= 0x1p64f);
      }
      if (__builtin_expect(__any(bad), 0)) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          if (!(lsum[nt] >= 0x1p-64f && lsum[nt] <= 0x1p64f)) {
            float mx = -INFINITY;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
              for (int r = 0; r < 4; ++r) mx = fmaxf(mx, acc[s2][nt][r]);
            if (mx == -INFINITY) {
              lsum[nt] = prev[nt];
            } else {
              float s = 0.f;
#pragma unroll
              for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int r = 0; r < 4; ++r) s += fast_exp2(acc[s2][nt][r] - mx);
              lsum[nt] = prev[nt] * fast_exp2(-mx) + s;
              off[nt] += mx;
              cneg[nt] = floatx4{-off[nt], -off[nt], -off[nt], -off[nt]};
            }
          }
        }
      }
    } else {
      // ---- pass 2: probabilities, P.V and block scores -----------------------------------
      float p[2][4][4];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r) p[s2][nt][r] = fast_exp2(acc[s2][nt][r]);
      halfx8 pb[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        pb[nt] = pack8h(p[0][nt][0], p[0][nt][1], p[0][nt][2], p[0][nt][3], p[1][nt][0],
                        p[1][nt][1], p[1][nt][2], p[1][nt][3]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const halfx8 vt = *reinterpret_cast<const halfx8*>(&L[512 + mt * 64 + lane]);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) o[mt][nt] = mfma16h(vt, pb[nt], o[mt][nt]);
      }
      // column sums over the queries of each query block
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        float v[2][4];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float s = 0.f;
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
              if (nt >= qb * kNtPerQB && nt < (qb + 1) * kNtPerQB) s += p[s2][nt][r];
            v[s2][r] = s;
          }
        const float tot = row_reduce_scatter8(v, lane);
        const int64_t qblk = (q0 + 16 * qb * kNtPerQB) / a.B;
        if (((lane & 2) == 0) && qblk < a.Nb) {
          float* dst = a.score + ((int64_t)h * a.Nb + qblk) * a.ld + tau * kTileKeys +
                       reduced_key(lane);
          if (a.B > 64) {
            atomicAdd(dst, tot);
          } else {
            *dst = tot;
          }
        }
      }
    }

    if (has_next) {
#pragma unroll
      for (int r = 0; r < kLoads; ++r) lds[buf ^ 1][r * 256 + tid] = stg[r];
    }
    __syncthreads();
  }

  if constexpr (!kFused) {
    // combine the four lane groups of each query: offsets and partial sums
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      float m = (lsum[nt] > 0.f) ? off[nt] : -INFINITY;
      float l = lsum[nt];
#pragma unroll
      for (int sh = 16; sh <= 32; sh *= 2) {
        const float m2 = __shfl_xor(m, sh);
        const float l2 = __shfl_xor(l, sh);
        const float M = fmaxf(m, m2);
        l = ((m == -INFINITY) ? 0.f : l * fast_exp2(m - M)) +
            ((m2 == -INFINITY) ? 0.f : l2 * fast_exp2(m2 - M));
        m = M;
      }
      const int64_t t = q0 + 16 * nt + li;
      if (g == 0 && t < a.T) a.lse[(int64_t)h * a.T + t] = (m + __log2f(l)) * kLn2;
    }
  } else {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t t = q0 + 16 * nt + li;
      if (t < a.T) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          *reinterpret_cast<float4*>(a.o_cmp + (t * a.H + h) * kD + 16 * mt + 4 * g) =
              make_float4(o[mt][nt][0], o[mt][nt][1], o[mt][nt][2], o[mt][nt][3]);
        }
      }
    }
  }
}

static hipError_t launch_cmp(const CmpArgs& a, hipStream_t s, bool fused) {
  const int64_t n_qtiles = (a.T + kCmpQueries - 1) / kCmpQueries;
  const int64_t total = (int64_t)a.H * n_qtiles;
  const int64_t grid = ((total + 7) / 8) * 8;
  const dim3 g3((unsigned)grid), b3(256);
  if (fused) {
    switch (a.B) {
      case 16: hipLaunchKernelGGL((cmp_kernel<true, 4>), g3, b3, 0, s, a); break;
      case 32: hipLaunchKernelGGL((cmp_kernel<true, 2>), g3, b3, 0, s, a); break;
      default: hipLaunchKernelGGL((cmp_kernel<true, 1>), g3, b3, 0, s, a); break;
    }
  } else {
    hipLaunchKernelGGL((cmp_kernel<false, 1>), g3, b3, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_cmp_lse(const CmpArgs& a, hipStream_t s) { return launch_cmp(a, s, false); }
hipError_t launch_cmp_fused(const CmpArgs& a, hipStream_t s) { return launch_cmp(a, s, true); }

}  // namespace s3r
