// Compression branch: attention of every query to all pooled (coarse) tokens, in two passes
// or (the default where it applies) in a single pass from a lower bound of the log-sum-exp.
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
//
// Single pass (kBound). Its offset is a lower bound L'_t <= L_t (from the LSE pass over the
// means of groups of 8 pooled keys: Jensen), so every weight u_tj = 2^(c_tj - L'_t) >= P_tj.
// One sweep accumulates O_cmp * Z_t and Z_t = sum_j u_tj, and per key block the upper bound
// sum_t u_tj of its score; a running list keeps the 64 blocks of largest bound. At the end
// L_t = L'_t + log2 Z_t, O_cmp = O / Z, and the listed blocks are rescored exactly (their
// logits recomputed on the same MFMA sequence) and ranked. Since P_tj = u_tj / Z_t, an unlisted
// block's score is at most its bound over the query block's smallest Z_t. A wave whose Z_t
// leave [1, 2^15] or whose list cannot prove the top k (its last bound, over that Z_t, not
// below the k-th score) sets a redo flag;
// the exact passes rerun only on the flagged work-groups (kDeep, kScoresOnly), so the outputs
// are those of the two passes up to rounding.
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
// kBound with kFused (and kTopk): the single pass (above). kBound without kFused: the bound
// pass, pass 1 over the group keys on their hi parts alone (half the MFMAs and half the
// records): its result need not be exact, only low enough, which the single pass checks.
// kDeep: tiles in flight for the exact reruns after the single pass, where few work-groups
// (at 1000 views, 16 heads: none of 343,500 waves flagged at k = 16, 0.2 % at k = 32) sweep
// all tiles and the latency of each copy, not the chip's throughput, decides.
// kScoresOnly (rerun of pass 2 with the running top-k where only the single pass's selection
// was not proven: its O_cmp stands): no V^T records, no P.V, no O_cmp write.
template <bool kFused, int kQB, int kWaves, bool kTopk = false, bool kHalf = false,
          bool kBound = false, int kDeep = 0, bool kScoresOnly = false>
// (second bound: resident waves per SIMD the register allocation must allow)
__global__ __launch_bounds__(64 * kWaves, kFused ? 3 : 4) void cmp_kernel(CmpArgs a) {
  static_assert(!kBound || !kFused || kTopk, "the single pass keeps the running top-k");
  static_assert(!kBound || kFused || kDeep == 0, "the bound pass has no rerun");
  constexpr bool kSingle = kBound && kFused;   // the single pass
  constexpr bool kHiOnly = kBound && !kFused;  // the bound pass: hi parts of the keys only
  constexpr int kAhead = kDeep ? kDeep : (kFused ? kFusedAhead : kLseAhead);  // tiles in flight
  constexpr int kRing = kAhead + 1;
  constexpr int kQueries = 64 * kWaves;
  static_assert(!kScoresOnly || (kFused && kTopk && !kBound), "a rerun of the top-k pass");
  // records of a tile this pass reads
  constexpr int kRecs = (kFused && !kScoresOnly) ? 12 : (kHiOnly ? 4 : 8);
  constexpr int kRecsPerWave = kRecs / kWaves;
  static_assert(kRecsPerWave * kWaves == kRecs, "each wave copies whole records");
  constexpr int kNtPerQB = 4 / kQB;
  __shared__ uint4 lds[kRing][kRecs * 64];
  // (single pass) each lane's parts of Z_t for its 4 column tiles: read, added to and written
  // back once per tile, so that no register holds them through the logits
  __shared__ floatx4 zpart[kSingle ? kWaves : 1][64];

  const int64_t n_qtiles = (a.T + kQueries - 1) / kQueries;
  const int64_t total = (int64_t)a.H * n_qtiles;
  // (reruns: logical id = block id, so that the dispatcher deals the flagged work-groups,
  // which cluster where block scores are close, round-robin over the XCDs, not onto a few)
  const int64_t logical = kDeep ? (int64_t)blockIdx.x : xcd_logical_id(blockIdx.x, total);
  if (logical >= total) return;
  // (scores-only rerun) a wave whose own selection the single pass proved only copies its
  // share of each tile: no logits, no list, no write (its rows stand)
  bool idle = false;
  if (a.redo_in) {  // exact rerun of the work-groups the single pass flagged
    const int4 f = *reinterpret_cast<const int4*>(a.redo_in + 4 * logical);
    const int any = f.x | f.y | f.z | f.w;
    if ((any & a.redo_mask) == 0 || (any & a.redo_skip) != 0) return;
    if constexpr (kScoresOnly) {
      const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
      const int mine = w == 0 ? f.x : (w == 1 ? f.y : (w == 2 ? f.z : f.w));
      idle = (mine & a.redo_mask) == 0;
    }
  }
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
    if constexpr (kSingle) {
      // a lower bound of L_t (base 2), lowered by kBoundMargin so that rounding cannot lift
      // it above L_t
      off[nt] = (t < a.T) ? a.lse_in[(int64_t)h * a.T + t] * kLog2e - kBoundMargin : INFINITY;
    } else if constexpr (kFused) {
      off[nt] = (t < a.T) ? a.lse_in[(int64_t)h * a.T + t] * kLog2e : INFINITY;
    } else {
      off[nt] = 0.f;
      cneg[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    lsum[nt] = 0.f;
  }
  if constexpr (kSingle) zpart[wave][lane] = floatx4{0.f, 0.f, 0.f, 0.f};  // this lane's own
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
  // length of the running list: k for the exact pass; the single pass ranks upper bounds and
  // keeps every candidate up to one per lane
  auto list_len = [&](int64_t qblk, bool& own) {
    if constexpr (kSingle) {
      own = a.own && qblk >= a.forced;
      const int64_t nc = a.Nb - a.forced - (own ? 1 : 0);
      return (int)(nc < 64 ? nc : 64);
    } else {
      return chosen(qblk, own);
    }
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
      bf16x8 l0, l1;
      if constexpr (!kHiOnly) {
        l0 = *reinterpret_cast<const bf16x8*>(&L[256 + (2 * s2 + 0) * 64 + lane]);
        l1 = *reinterpret_cast<const bf16x8*>(&L[256 + (2 * s2 + 1) * 64 + lane]);
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        // pass 2 subtracts its fixed offset on the VALU instead (registers)
        floatx4 x = mfma_in<kHalf>(h0, qb[nt][0],
                                   kFused ? floatx4{0.f, 0.f, 0.f, 0.f} : cneg[kFused ? 0 : nt]);
        x = mfma_in<kHalf>(h1, qb[nt][1], x);
        if constexpr (kHiOnly) {
          acc[s2][nt] = x;
        } else {
          x = mfma_in<kHalf>(l0, qb[nt][0], x);
          acc[s2][nt] = mfma_in<kHalf>(l1, qb[nt][1], x);
        }
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
      if constexpr (kSingle) {
        // this lane's part of Z_t; the empty asm ties the LDS read to the weights, so that
        // the compiler cannot hoist it (and the 4 registers) above the logits
        int zl = lane;
        asm volatile("" : "+v"(zl) : "v"(p[1][3][3]));
        floatx4 zz = zpart[wave][zl];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          float z = p[0][nt][0];
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int r = (s2 == 0 ? 1 : 0); r < 4; ++r) z += p[s2][nt][r];
          zz[nt] += z;
        }
        zpart[wave][zl] = zz;
      }
      // column sums over the queries of each query block (the single pass's are only upper
      // bounds: it adds the packed fp16 weights, and its check allows for their rounding)
      float tots[kQB];
      halfx8 hs[kQB];
      auto column_sums = [&]() {
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
          tots[qb] = row_reduce_scatter8(v, lane);
        }
      };
#pragma unroll
      for (int nt = 0; nt < (kScoresOnly ? 0 : 4); ++nt) {
        const halfx8 pb = pack8h(p[0][nt][0], p[0][nt][1], p[0][nt][2], p[0][nt][3],
                                 p[1][nt][0], p[1][nt][1], p[1][nt][2], p[1][nt][3]);
        if constexpr (kSingle) hs[nt / kNtPerQB] = (nt % kNtPerQB == 0) ? pb : hs[nt / kNtPerQB] + pb;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const halfx8 vt = *reinterpret_cast<const halfx8*>(&L[512 + mt * 64 + lane]);
          o[mt][nt] = mfma16h(vt, pb, o[mt][nt]);
        }
      }
      if constexpr (kSingle) {
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) tots[qb] = row_reduce_scatter8_h(hs[qb], lane);
      } else {
        column_sums();
      }
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        const float tot = tots[qb];
        // single pass: B = 64 / kQB (a shift; the division stays in the exact kernels, whose
        // register allocation it happens to suit)
        const int64_t qblk = kSingle ? (q0 + 16 * qb * kNtPerQB) / (64 / kQB)
                                    : (q0 + 16 * qb * kNtPerQB) / a.B;
        if constexpr (kTopk) {
          if (qblk < a.Nb) {
            // lanes with bit 1 clear hold the 32 distinct keys of this tile; a block can only
            // enter the list if its score is >= the current k-th score (one compare per tile)
            const int j = (int)(tau * kTileKeys) + reduced_key(lane);
            bool own;
            const int K = list_len(qblk, own);
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

  // (single pass) Exact scores of the listed blocks of query block qi, from the exact L_t:
  // the blocks' pooled keys are gathered 16 at a time into this wave's LDS records R and meet
  // the resident queries in the same MFMA sequence as in the pass, so every logit is the
  // pass's own. The k best by (score desc, index asc) are kept if the largest upper bound of
  // a block outside the list, over the query block's smallest Z_t, stays below the k-th
  // score; otherwise `fail` is set. zq: Z_t of this lane's queries (+inf past the end).
  auto rescore = [&](int qi, const float (&L2)[4], const float (&zq)[4], uint4* R, bool& fail) {
    // (a list short of entries, from non-finite bounds, has also failed the Z check)
    const int64_t qblk = (q0 + 16 * qi * kNtPerQB) / a.B;
    if (qblk >= a.Nb) return;
    bool own;
    const int Kc = list_len(qblk, own);
    const int K = chosen(qblk, own);
    if (Kc <= 0) return;
    const int j = tk_j[qi];
    float S = -1.0f;
    fail |= lane < Kc && !(j >= 0 && j < a.Nb);
    for (int gq = 0; gq < (Kc + 15) / 16; ++gq) {
      const int e = 16 * gq + li;
      int je = __shfl(j, e);
      je = (e < Kc && je >= 0 && je < a.Nb) ? je : 0;
      const int kk = je & 31, s = kk >> 4;
      const unsigned char* src =
          tiles + (int64_t)(je >> 5) * kPooledTileBytes + 16 * ((kk & 15) + 16 * g);
      wait_lds();  // the previous group's operands have been read
      copy16_to_lds(src + (2 * s) * kRecBytes, R);            // hi, dims 0..31
      copy16_to_lds(src + (2 * s + 1) * kRecBytes, R + 64);   // hi, dims 32..63
      copy16_to_lds(src + (4 + 2 * s) * kRecBytes, R + 128);  // lo, dims 0..31
      copy16_to_lds(src + (5 + 2 * s) * kRecBytes, R + 192);  // lo, dims 32..63
      wait_vmem<0>();
      const bf16x8 h0 = *reinterpret_cast<const bf16x8*>(&R[lane]);
      const bf16x8 h1 = *reinterpret_cast<const bf16x8*>(&R[64 + lane]);
      const bf16x8 l0 = *reinterpret_cast<const bf16x8*>(&R[128 + lane]);
      const bf16x8 l1 = *reinterpret_cast<const bf16x8*>(&R[192 + lane]);
      float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nt = qi * kNtPerQB; nt < (qi + 1) * kNtPerQB; ++nt) {
        floatx4 x = mfma_in<kHalf>(h0, qb[nt][0], floatx4{0.f, 0.f, 0.f, 0.f});
        x = mfma_in<kHalf>(h1, qb[nt][1], x);
        x = mfma_in<kHalf>(l0, qb[nt][0], x);
        x = mfma_in<kHalf>(l1, qb[nt][1], x);
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] += fast_exp2(x[r] - L2[nt]);
      }
      // sum over the 16 queries of each column tile: lane group g then holds the scores of
      // listed entries 16 gq + 4 g + r
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int sh = 1; sh < 16; sh *= 2) v[r] += __shfl_xor(v[r], sh);
      const int from = 16 * (li >> 2);
      const float t0 = __shfl(v[0], from), t1 = __shfl(v[1], from);
      const float t2 = __shfl(v[2], from), t3 = __shfl(v[3], from);
      const int rr = lane & 3;
      const float pick = rr == 0 ? t0 : (rr == 1 ? t1 : (rr == 2 ? t2 : t3));
      if (g == gq) S = pick;
    }
    // exact rank of each entry among the Kc listed ones
    int rank = 0;
    for (int m = 0; m < Kc; ++m) {
      const float sm =
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, S), m));
      const int jm = __builtin_amdgcn_readlane(j, m);
      rank += better(sm, jm, S, j) ? 1 : 0;
    }
    if (lane >= Kc) rank = lane;
    const uint64_t at = __ballot(rank == K - 1);
    const int kth = at ? __builtin_ctzll(at) : 0;
    const float sk =
        __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, S), kth));
    // Every block outside the list has a bound <= the list's last entry th_v (it fell below
    // the threshold of its tile, was pushed out from the last place, or tied with it), and
    // the threshold only rises. With at most 64 candidates every one is listed. A bound is a
    // sum of fp16-rounded weights taken in fp16: each of its 64 terms passes at most 6
    // roundings of 2^-11 relative (packing, 3 sums over column tiles, 2 halvings of the lane
    // reduction), 6 * 2^-11 < 2^-8 in all, and the at most 136 roundings of values below 2^-14
    // add at most 2^-25 each, < 2^-17 in all (fp16 subnormals are kept: the kernels run with
    // f16 denormals on, the compiler's default; flushing them would cost up to 2^-14 each).
    // So a block's sum of weights sum_t w_tj is at most its bound * (1 + 2^-8) + 2^-17, and
    // its exact score sum_t 2^(c_tj - L_t) = sum_t w_tj / Z_t is at most that sum over the
    // smallest Z_t of the query block's queries.
    // The f32 roundings of the scores, of log2 Z_t and of this division add far less than
    // 2^-10 relative (for exponents below 2^10 in magnitude), the room 2^-8 leaves over
    // 6 * 2^-11.
    float zmin = zq[qi * kNtPerQB];
#pragma unroll
    for (int nt = qi * kNtPerQB + 1; nt < (qi + 1) * kNtPerQB; ++nt) zmin = fminf(zmin, zq[nt]);
#pragma unroll
    for (int sh = 1; sh < 16; sh *= 2) zmin = fminf(zmin, __shfl_xor(zmin, sh));
    // (a Z_t outside [1, 2^15] fails the Z check, whose full rerun replaces this wave's results)
    zmin = fminf(fmaxf(zmin, 1.0f), 0x1p15f);
    const int64_t nc = a.Nb - a.forced - (own ? 1 : 0);
    const float rmax = nc <= Kc ? -1.0f : th_v[qi];
    fail |= !(at != 0 && (rmax < 0.f || (rmax * (1.0f + 0x1p-8f) + 0x1p-17f) / zmin < sk));
    tk_j[qi] = __builtin_amdgcn_ds_permute(4 * rank, j);  // entry of exact rank e to lane e
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
    if (!(kScoresOnly && idle)) {
      qk(L, acc);
      process(tau, L, acc, false);
    }
    wait_vmem<(kAhead - 1) * kRecsPerWave>();
    lds_barrier();
  }
  if (!(kScoresOnly && idle)) {
    const uint4* L = lds[(int)((n - 1) % kRing)];
    qk(L, acc);
    process(n - 1, L, acc, true);
  }
  wait_vmem<0>();  // no copy outlives the work-group
  if (kScoresOnly && idle) return;

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
      if (g == 0 && t < a.T) a.lse[(int64_t)h * a.T + t] = (m + __log2f(l)) * kLn2 + a.lse_bias;
    }
  } else {
    // 1 / Z_t (single pass) times the undoing of the value records' power of two
    float zinv[4] = {a.v_unscale, a.v_unscale, a.v_unscale, a.v_unscale};
    if constexpr (kSingle) {
      // Z_t and the exact L_t = offset + log2 Z_t. Z_t >= 1 proves offset <= L_t, i.e. every
      // weight was at least its probability, so each block's accumulated sum bounds its score
      // from above; Z_t <= 2^15 proves that no weight (each is at most Z_t) overflowed fp16 in
      // P.V. A wave that holds a query outside [1, 2^15] fails (flag bit 1: both exact passes
      // rerun); one whose selection is not proven fails with bit 0 (only the second reruns:
      // its L_t are exact).
      bool zfail = false, fail = false;
      float L2[4], zq[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        float z = zpart[wave][lane][nt];
        z += __shfl_xor(z, 16);
        z += __shfl_xor(z, 32);
        const int64_t t = q0 + 16 * nt + li;
        zq[nt] = t < a.T ? z : INFINITY;
        zfail |= t < a.T && !(z >= 1.0f && z <= 0x1p15f);
        L2[nt] = (t < a.T && z > 0.f) ? off[nt] + __log2f(z) : INFINITY;
        zinv[nt] = z > 0.f ? a.v_unscale / z : 0.f;
        if (g == 0 && t < a.T) a.lse[(int64_t)h * a.T + t] = L2[nt] * kLn2;
      }
      lds_barrier();  // every wave is done with the ring: each takes a quarter of it
      static_assert(kRing * kRecs * 64 / kWaves >= 4 * 64, "four records per wave");
      uint4* R = &lds[0][0] + wave * (kRing * kRecs * 64 / kWaves);
#pragma unroll
      for (int qi = 0; qi < kQB; ++qi) rescore(qi, L2, zq, R, fail);
      const int flag = (__any(zfail) ? 2 : 0) | (__any(fail) ? 1 : 0);
      if (lane == 0) a.redo_out[4 * logical + wave] = flag;
    }
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
    for (int nt = 0; nt < (kScoresOnly ? 0 : 4); ++nt) {
      const int64_t t = q0 + 16 * nt + li;
      if (t < a.T) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          *reinterpret_cast<float4*>(a.o_cmp + (t * a.H + h) * kD + 16 * mt + 4 * g) =
              make_float4(o[mt][nt][0] * zinv[nt], o[mt][nt][1] * zinv[nt],
                          o[mt][nt][2] * zinv[nt], o[mt][nt][3] * zinv[nt]);
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

template <bool kHalf>
static hipError_t launch_bound_t(const CmpArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((cmp_kernel<false, 1, kLseWaves, false, kHalf, true>), cmp_grid(a, kLseWaves),
                     dim3(64 * kLseWaves), 0, s, a);
  return hipGetLastError();
}

template <bool kHalf>
static hipError_t launch_single_t(const CmpArgs& a, hipStream_t s) {
  const dim3 g3 = cmp_grid(a, kFusedWaves), b3(64 * kFusedWaves);
  switch (a.B) {
    case 16: hipLaunchKernelGGL((cmp_kernel<true, 4, kFusedWaves, true, kHalf, true>), g3, b3, 0, s, a); break;
    case 32: hipLaunchKernelGGL((cmp_kernel<true, 2, kFusedWaves, true, kHalf, true>), g3, b3, 0, s, a); break;
    default: hipLaunchKernelGGL((cmp_kernel<true, 1, kFusedWaves, true, kHalf, true>), g3, b3, 0, s, a); break;
  }
  return hipGetLastError();
}

constexpr int kRerunAhead = 3;

template <bool kHalf, bool kScoresOnly>
static void launch_rerun_fused(const CmpArgs& a, hipStream_t s) {
  const dim3 g3 = cmp_grid(a, kFusedWaves), b4(64 * 4);
  switch (a.B) {
    case 16: hipLaunchKernelGGL((cmp_kernel<true, 4, kFusedWaves, true, kHalf, false, kRerunAhead, kScoresOnly>), g3, b4, 0, s, a); break;
    case 32: hipLaunchKernelGGL((cmp_kernel<true, 2, kFusedWaves, true, kHalf, false, kRerunAhead, kScoresOnly>), g3, b4, 0, s, a); break;
    default: hipLaunchKernelGGL((cmp_kernel<true, 1, kFusedWaves, true, kHalf, false, kRerunAhead, kScoresOnly>), g3, b4, 0, s, a); break;
  }
}

template <bool kHalf>
static hipError_t launch_rerun_t(const CmpArgs& a, hipStream_t s, bool fused, bool scores_only) {
  const dim3 b4(64 * 4);
  if (fused) {
    if (scores_only) launch_rerun_fused<kHalf, true>(a, s);
    else launch_rerun_fused<kHalf, false>(a, s);
  } else {
    hipLaunchKernelGGL((cmp_kernel<false, 1, kLseWaves, false, kHalf, false, kRerunAhead>),
                       cmp_grid(a, kLseWaves), b4, 0, s, a);
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
hipError_t launch_cmp_lse_bound(const CmpArgs& a, hipStream_t s) {
  return a.half ? launch_bound_t<true>(a, s) : launch_bound_t<false>(a, s);
}
hipError_t launch_cmp_single_topk(const CmpArgs& a, hipStream_t s) {
  return a.half ? launch_single_t<true>(a, s) : launch_single_t<false>(a, s);
}
hipError_t launch_cmp_rerun(const CmpArgs& a, hipStream_t s, bool fused, bool scores_only) {
  return a.half ? launch_rerun_t<true>(a, s, fused, scores_only)
                : launch_rerun_t<false>(a, s, fused, scores_only);
}

}  // namespace s3r
