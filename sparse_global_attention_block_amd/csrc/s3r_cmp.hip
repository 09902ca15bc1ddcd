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
// with c_tj = scale * q_t . Kc_j, on 16x16x32 MFMAs with f32 accumulation.
//
// Work decomposition: a work-group of 4 waves owns 256 consecutive queries of one head; each
// wave holds 64 queries (4 column tiles of 16) as resident B operands and streams the pooled
// tiles (32 coarse tokens each) through a 2-slot LDS ring. The accumulator tile is S^T (keys x
// queries): lane l holds query l%16 and keys 4*(l/16)+r, so P feeds the P.V MFMA directly as
// its B operand (in fp16, against fp16 pooled values). The pooled keys arrive pre-multiplied
// by scale*log2(e) as bf16 hi + lo, so logits come out in base-2 units. The query's offset is
// the first MFMA's C input in pass 1 (the running offset) and one VALU subtraction per logit in
// pass 2 (-L_t*log2(e)): pass 2 is register-bound, and the 16 registers of that operand decide
// between two and three resident waves per SIMD.
//
// Tiles reach LDS by direct global->LDS copies (each wave copies its share of the records),
// kAhead tiles ahead of the one being computed, so no registers are held for tiles in flight.
// A software pipeline inside one wave (logits of tile t+1 on the matrix cores while the VALU
// works on tile t) was measured slower on MI355X: its second accumulator set costs occupancy.
#include "s3r_common.hpp"
#include "s3r_launch.hpp"

namespace s3r {

constexpr int kLseWaves = 4;
constexpr int kFusedWaves = 4;
constexpr int kLseAhead = 1;    // tiles in flight, pass 1
constexpr int kFusedAhead = 1;  // tiles in flight, pass 2

// kQB: query blocks per wave (64 / B for B <= 64, else 1; B = 128 blocks span two waves and
// their scores are completed with a second atomic add onto a zeroed matrix).
// kTopk (pass 2, B <= 64, k <= 64): instead of writing the score matrix, each wave keeps the
// running top-k of its query block(s) in registers, one entry per lane, and writes the chosen
// indices at the end. The entries are ordered by (score desc, block index asc), a total order,
// so the final set does not depend on the order in which blocks arrive, and the decision is
// made on exactly the f32 column sums the score matrix would have held.
template <bool kFused, int kQB, int kWaves, bool kTopk = false, bool kHalf = false>
// (second bound: resident waves per SIMD the register allocation must allow)
__global__ __launch_bounds__(64 * kWaves, kFused ? 3 : 4) void cmp_kernel(CmpArgs a) {
  constexpr int kAhead = kFused ? kFusedAhead : kLseAhead;  // tiles in flight
  constexpr int kRing = kAhead + 1;
  constexpr int kQueries = 64 * kWaves;
  constexpr int kRecs = kFused ? 12 : 8;  // records of a tile this pass reads
  constexpr int kRecsPerWave = kRecs / kWaves;
  static_assert(kRecsPerWave * kWaves == kRecs, "each wave copies whole records");
  constexpr int kNtPerQB = 4 / kQB;
  __shared__ uint4 lds[kRing][kRecs * 64];

  const int64_t n_qtiles = (a.T + kQueries - 1) / kQueries;
  const int64_t total = (int64_t)a.H * n_qtiles;
  const int64_t logical = xcd_logical_id(blockIdx.x, total);
  if (logical >= total) return;
  const int h = (int)(logical / n_qtiles);
  const int64_t qt = logical % n_qtiles;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 4, li = lane & 15;
  const int64_t q0 = qt * kQueries + wave * 64;
  const int64_t n = a.n_tiles;

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

  // Per-lane softmax state. Pass 1: running offset m (base 2) and partial sum l of this lane's
  // keys; pass 2: the fixed offset L_t*log2(e) (+inf for a query past the end: P = 0).
  // Pass 1 holds -offset as the first MFMA's C operand; pass 2 subtracts it on the VALU, which
  // saves the 16 registers of that operand (pass 2 is register-bound).
  float off[4], lsum[4];
  floatx4 cneg[kFused ? 1 : 4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int64_t t = q0 + 16 * nt + li;
    if constexpr (kFused) {
      off[nt] = (t < a.T) ? a.lse_in[(int64_t)h * a.T + t] * kLog2e : INFINITY;
    } else {
      off[nt] = 0.f;
      cneg[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    lsum[nt] = 0.f;
  }
  // running top-k: lane e holds entry e (score, block index) of each query block's list;
  // th_v / th_j mirror entry K-1 (the current k-th best) in scalar registers
  float tk_v[kQB], th_v[kQB];
  int tk_j[kQB], th_j[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    tk_v[qb] = -1.0f;  // below every score (scores are sums of probabilities, >= 0)
    tk_j[qb] = 0x7FFFFFFF;
    th_v[qb] = -1.0f;
    th_j[qb] = 0x7FFFFFFF;
  }
  // blocks chosen per query block: top-k among those neither forced nor (with own blocks) the
  // query block's own
  auto chosen = [&](int64_t qblk, bool& own) {
    own = a.own && qblk >= a.forced;
    const int64_t nc = a.Nb - a.forced - (own ? 1 : 0);
    return (int)(a.topk < nc ? a.topk : nc);
  };
  auto better = [](float v1, int j1, float v2, int j2) {
    return v1 > v2 || (v1 == v2 && j1 < j2);
  };

  floatx4 o[4][4];
  if constexpr (kFused) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) o[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  const unsigned char* tiles = a.tiles + (int64_t)h * n * kPooledTileBytes;
  // this wave's share of tile t into ring slot `slot` (kRecsPerWave vector-memory operations)
  auto copy = [&](int64_t t, int slot) {
#pragma unroll
    for (int r = 0; r < kRecsPerWave; ++r) {
      const int rec = wave * kRecsPerWave + r;
      copy16_to_lds(tiles + t * kPooledTileBytes + rec * kRecBytes + 16 * lane,
                    &lds[slot][rec * 64]);
    }
  };

  // S^T of one tile: keys (16 per half s2) x queries (16 per column tile nt), offset applied.
  auto qk = [&](const uint4* L, floatx4 (&acc)[2][4]) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const bf16x8 h0 = *reinterpret_cast<const bf16x8*>(&L[(2 * s2 + 0) * 64 + lane]);
      const bf16x8 h1 = *reinterpret_cast<const bf16x8*>(&L[(2 * s2 + 1) * 64 + lane]);
      const bf16x8 l0 = *reinterpret_cast<const bf16x8*>(&L[256 + (2 * s2 + 0) * 64 + lane]);
      const bf16x8 l1 = *reinterpret_cast<const bf16x8*>(&L[256 + (2 * s2 + 1) * 64 + lane]);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        // pass 2 subtracts its fixed offset on the VALU instead (registers)
        floatx4 x = mfma_in<kHalf>(h0, qb[nt][0],
                                   kFused ? floatx4{0.f, 0.f, 0.f, 0.f} : cneg[kFused ? 0 : nt]);
        x = mfma_in<kHalf>(h1, qb[nt][1], x);
        x = mfma_in<kHalf>(l0, qb[nt][0], x);
        acc[s2][nt] = mfma_in<kHalf>(l1, qb[nt][1], x);
      }
    }
  };

  auto process = [&](int64_t tau, const uint4* L, floatx4 (&acc)[2][4], bool last) {
    if (last) {
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
      // ---- pass 1: partial sums with a lazily moved offset -----------------------------
      bool bad = false;
      float prev[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        float s = fast_exp2(acc[0][nt][0]);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int r = (s2 == 0 ? 1 : 0); r < 4; ++r) s += fast_exp2(acc[s2][nt][r]);
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
              cneg[kFused ? 0 : nt] = floatx4{-off[nt], -off[nt], -off[nt], -off[nt]};
            }
          }
        }
      }
    } else {
      // ---- pass 2: probabilities, P.V and block scores ---------------------------------
      float p[2][4][4];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            p[s2][nt][r] = fast_exp2(acc[s2][nt][r] - off[nt]);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const halfx8 pb = pack8h(p[0][nt][0], p[0][nt][1], p[0][nt][2], p[0][nt][3],
                                 p[1][nt][0], p[1][nt][1], p[1][nt][2], p[1][nt][3]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const halfx8 vt = *reinterpret_cast<const halfx8*>(&L[512 + mt * 64 + lane]);
          o[mt][nt] = mfma16h(vt, pb, o[mt][nt]);
        }
      }
      // column sums over the queries of each query block
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        float v[2][4];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float s = p[s2][qb * kNtPerQB][r];
#pragma unroll
            for (int nt = qb * kNtPerQB + 1; nt < (qb + 1) * kNtPerQB; ++nt) s += p[s2][nt][r];
            v[s2][r] = s;
          }
        const float tot = row_reduce_scatter8(v, lane);
        const int64_t qblk = (q0 + 16 * qb * kNtPerQB) / a.B;
        if constexpr (kTopk) {
          if (qblk < a.Nb) {
            // lanes with bit 1 clear hold the 32 distinct keys of this tile; a block can only
            // enter the list if its score is >= the current k-th score (one compare per tile)
            const int j = (int)(tau * kTileKeys) + reduced_key(lane);
            bool own;
            const int K = chosen(qblk, own);
            const bool mine = ((lane & 2) == 0) && K > 0 && j >= a.forced && j < a.Nb &&
                              !(own && j == qblk);
            uint64_t cand = __ballot(mine && tot >= th_v[qb]);
            while (cand) {  // rare after the first tiles
              const int c = __builtin_ctzll(cand);
              cand &= cand - 1;
              const float cv = __builtin_bit_cast(
                  float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tot), c));
              const int cj = __builtin_amdgcn_readlane(j, c);
              if (!better(cv, cj, th_v[qb], th_j[qb])) continue;
              const bool ahead = lane < K && better(tk_v[qb], tk_j[qb], cv, cj);
              const int pos = __popcll(__ballot(ahead));
              // shift entries pos.. one lane up (DPP wave_shr:1), then place the new one
              const float up_v = __builtin_bit_cast(
                  float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, tk_v[qb]),
                                                     kDppWaveShr1, 0xF, 0xF, false));
              const int up_j = __builtin_amdgcn_update_dpp(0, tk_j[qb], kDppWaveShr1, 0xF, 0xF,
                                                           false);
              tk_v[qb] = lane == pos ? cv : (lane > pos ? up_v : tk_v[qb]);
              tk_j[qb] = lane == pos ? cj : (lane > pos ? up_j : tk_j[qb]);
              th_v[qb] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                       __builtin_bit_cast(int, tk_v[qb]), K - 1));
              th_j[qb] = __builtin_amdgcn_readlane(tk_j[qb], K - 1);
            }
          }
        } else if (((lane & 2) == 0) && qblk < a.Nb) {
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
  };

  // Ring of kRing slots, kAhead tiles in flight. Every step requests one tile (the last one
  // again once the sequence is exhausted) so that "tile t+1 has landed" is always "at most
  // (kAhead - 1) * kRecsPerWave copies of this wave pending"; the barrier then publishes
  // every wave's share. Slot (t + kAhead) % kRing was last read in step t - 1, before the
  // barrier that ended it.
#pragma unroll
  for (int s = 0; s < kAhead; ++s) copy(s < n ? s : n - 1, s);
  wait_vmem<(kAhead - 1) * kRecsPerWave>();
  lds_barrier();
  floatx4 acc[2][4];
  for (int64_t tau = 0; tau + 1 < n; ++tau) {
    copy(tau + kAhead < n ? tau + kAhead : n - 1, (int)((tau + kAhead) % kRing));
    const uint4* L = lds[(int)(tau % kRing)];
    qk(L, acc);
    process(tau, L, acc, false);
    wait_vmem<(kAhead - 1) * kRecsPerWave>();
    lds_barrier();
  }
  {
    const uint4* L = lds[(int)((n - 1) % kRing)];
    qk(L, acc);
    process(n - 1, L, acc, true);
  }
  wait_vmem<0>();  // no copy outlives the work-group

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
    if constexpr (kTopk) {
      // the chosen blocks of each query block, in ascending index order
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        const int64_t qblk = (q0 + 16 * qb * kNtPerQB) / a.B;
        if (qblk < a.Nb) {
          int32_t* row = a.sel + ((int64_t)h * a.Nb + qblk) * a.n_sel;
          bool own;
          const int K = chosen(qblk, own);
          for (int m = lane; m < a.forced; m += 64) row[m] = m;
          for (int m = a.forced + (own ? 1 : 0) + K + lane; m < a.n_sel; m += 64) row[m] = -1;
          int rank = (own && qblk < tk_j[qb]) ? 1 : 0, own_pos = 0;
          for (int m = 0; m < K; ++m) {
            const int o = __builtin_amdgcn_readlane(tk_j[qb], m);
            rank += o < tk_j[qb];
            own_pos += o < qblk;
          }
          if (lane < K) row[a.forced + rank] = tk_j[qb];
          if (own && lane == 0) row[a.forced + own_pos] = (int32_t)qblk;
        }
      }
    }
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

static dim3 cmp_grid(const CmpArgs& a, int waves) {
  const int64_t q = 64 * waves;
  const int64_t total = (int64_t)a.H * ((a.T + q - 1) / q);
  return dim3((unsigned)(((total + 7) / 8) * 8));
}

template <bool kHalf>
static hipError_t launch_cmp_t(const CmpArgs& a, hipStream_t s, bool fused, bool topk) {
  if (fused) {
    const dim3 g3 = cmp_grid(a, kFusedWaves), b3(64 * kFusedWaves);
    if (topk) {
      switch (a.B) {
        case 16: hipLaunchKernelGGL((cmp_kernel<true, 4, kFusedWaves, true, kHalf>), g3, b3, 0, s, a); break;
        case 32: hipLaunchKernelGGL((cmp_kernel<true, 2, kFusedWaves, true, kHalf>), g3, b3, 0, s, a); break;
        default: hipLaunchKernelGGL((cmp_kernel<true, 1, kFusedWaves, true, kHalf>), g3, b3, 0, s, a); break;
      }
    } else {
      switch (a.B) {
        case 16: hipLaunchKernelGGL((cmp_kernel<true, 4, kFusedWaves, false, kHalf>), g3, b3, 0, s, a); break;
        case 32: hipLaunchKernelGGL((cmp_kernel<true, 2, kFusedWaves, false, kHalf>), g3, b3, 0, s, a); break;
        default: hipLaunchKernelGGL((cmp_kernel<true, 1, kFusedWaves, false, kHalf>), g3, b3, 0, s, a); break;
      }
    }
  } else {
    hipLaunchKernelGGL((cmp_kernel<false, 1, kLseWaves, false, kHalf>), cmp_grid(a, kLseWaves),
                       dim3(64 * kLseWaves), 0, s, a);
  }
  return hipGetLastError();
}

static hipError_t launch_cmp(const CmpArgs& a, hipStream_t s, bool fused, bool topk) {
  return a.half ? launch_cmp_t<true>(a, s, fused, topk) : launch_cmp_t<false>(a, s, fused, topk);
}

hipError_t launch_cmp_lse(const CmpArgs& a, hipStream_t s) { return launch_cmp(a, s, false, false); }
hipError_t launch_cmp_fused(const CmpArgs& a, hipStream_t s) { return launch_cmp(a, s, true, false); }
hipError_t launch_cmp_fused_topk(const CmpArgs& a, hipStream_t s) {
  return launch_cmp(a, s, true, true);
}

}  // namespace s3r
