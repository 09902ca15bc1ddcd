// Backward pass of the dual-branch sparse attention (gradients of q, k, v and the gates).
//
// The model is trained end to end (arXiv abstract; README "Overview"). The selection is held
// fixed: top-k is piecewise constant, so no gradient flows through the block scores. With
// out_t = g0 O_cmp_t + g1 O_sel_t (summary "Methodologie" 2), each branch is a softmax
// attention and the chain rule gives, per branch,
//   P = softmax(logits), dP_tu = (g dout_t) . v_u, D_t = sum_u P_tu dP_tu = g dout_t . O_t,
//   dS_tu = P_tu (dP_tu - D_t),  dq_t += scale sum_u dS_tu k_u,
//   dk_u += scale sum_t dS_tu q_t,  dv_u += sum_t P_tu g dout_t,
// with, for the compression branch, keys and values the block means Kc_j, Vc_j (whose
// gradients are spread back as 1/n_j over the tokens of block j), and for the selection
// branch the tokens of the selected blocks. The probabilities are recomputed from the
// log-sum-exps the forward pass saved.
//
// Kernels (all deterministic: every output element is written by one wave, in a fixed order):
//   rec_pack      operand images of q, dout (query tiles), v, k (raw) and the means (pooled)
//   bwd_scalars   per (token, head): D_cmp, D_sel and the per-token gate gradients
//   cmp_dq        compression dq, query-centric over all pooled tiles (S^T layout)
//   cmp_dkv       compression dKc, dVc, key-centric over all query tiles (S layout)
//   sel_dq        selection dq, query-centric over the selected blocks
//   sel_dkv       selection dk, dv plus the spread-back pooled gradients, key-centric over the
//                 query blocks that selected the key block (from a selection bitmap)
#include <type_traits>

#include "s3r_common.hpp"
#include "s3r_launch.hpp"

namespace s3r {

// ---------------------------------------------------------------------------------------
// Operand images. Thread (row m, dims 8*d8..+7) of a 256-thread work-group; the TR group is
// assembled in LDS (swizzled like cmp_dkv's: each 2-byte store has every lane on the same dim
// modulo 8) and written linearly.
// ---------------------------------------------------------------------------------------
// Slot of lane l's 16 bytes in a transposed record staged in LDS: a permutation inside each
// aligned group of 8 slots, so 16-byte lane reads through it stay free of bank conflicts.
__device__ __forceinline__ int tr_swizzle(int l) { return l ^ ((l >> 3) & 7); }

// kKind 0: 2-byte source of type kHalf; 1: f32 source. R records are written in the input
// type (kHalf), TR records in bf16.
template <int kKind, bool kHalf>
__global__ __launch_bounds__(256) void rec_pack_kernel(RecPackArgs a) {
  __shared__ __attribute__((aligned(16))) u16 stage[4 * kRecBytes / 2];
  const int tid = threadIdx.x;
  const int m = tid >> 3, d8 = tid & 7;
  const int h = blockIdx.y;
  for (int64_t tile = blockIdx.x; tile < a.n_tiles; tile += gridDim.x) {
    const int64_t row = tile * kTileKeys + m;
    float x[8];
    if (row < a.rows) {
      if constexpr (kKind == 0) {
        const uint4 w = *reinterpret_cast<const uint4*>(
            reinterpret_cast<const u16*>(a.src) + row * a.st + (int64_t)h * a.sh + d8 * 8);
        unpack8<kHalf>(w, x);
      } else {
        const float4* f = reinterpret_cast<const float4*>(
            reinterpret_cast<const float*>(a.src) + row * a.st + (int64_t)h * a.sh + d8 * 8);
        const float4 lo = f[0], hi = f[1];
        x[0] = lo.x; x[1] = lo.y; x[2] = lo.z; x[3] = lo.w;
        x[4] = hi.x; x[5] = hi.y; x[6] = hi.z; x[7] = hi.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
    unsigned char* out = a.dst + ((int64_t)h * a.n_tiles + tile) * a.tile_bytes;
    if (a.r_off >= 0) {
      uint4 w;
      w.x = float_to_in<kHalf>(x[0]) | ((uint32_t)float_to_in<kHalf>(x[1]) << 16);
      w.y = float_to_in<kHalf>(x[2]) | ((uint32_t)float_to_in<kHalf>(x[3]) << 16);
      w.z = float_to_in<kHalf>(x[4]) | ((uint32_t)float_to_in<kHalf>(x[5]) << 16);
      w.w = float_to_in<kHalf>(x[6]) | ((uint32_t)float_to_in<kHalf>(x[7]) << 16);
      *reinterpret_cast<uint4*>(out + a.r_off + k_chunk_offset(m, d8)) = w;
    }
    if (a.tr_off >= 0) {  // uniform over the work-group
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        int rec, lane, slot;
        vt_position(m, d8 * 8 + e, rec, lane, slot);
        stage[(rec * 64 + tr_swizzle(lane)) * 8 + slot] = bf16_bits(x[e]);
      }
      __syncthreads();
      reinterpret_cast<uint4*>(out + a.tr_off)[tid] =
          reinterpret_cast<const uint4*>(stage)[(tid & ~63) | tr_swizzle(tid & 63)];
      __syncthreads();
    }
  }
}

hipError_t launch_rec_pack(const RecPackArgs& a, int kind, hipStream_t s) {
  const dim3 grid((unsigned)(a.n_tiles < 2048 ? a.n_tiles : 2048), (unsigned)a.H);
  if (kind == 0) {
    if (a.half) hipLaunchKernelGGL((rec_pack_kernel<0, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((rec_pack_kernel<0, false>), grid, dim3(256), 0, s, a);
  } else {
    if (a.half) hipLaunchKernelGGL((rec_pack_kernel<1, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((rec_pack_kernel<1, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Per (token, head) scalars: 8 lanes per pair, 8 dims each.
//   qs = {L_cmp*log2(e), g0, g0 dout.O_cmp, L_sel (base 2), g1, g1 dout.O_sel, 0, 0}
//   dg_tok[t][h] = {dout.O_cmp, dout.O_sel} (the gate gradients of token t)
// ---------------------------------------------------------------------------------------
template <bool kHalf>
__global__ __launch_bounds__(256) void bwd_scalars_kernel(BwdScalarArgs a) {
  const int sub = threadIdx.x & 7;
  const int64_t n = a.T * a.H;
  const int64_t stride = ((int64_t)gridDim.x * 256) >> 3;
  for (int64_t idx = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 3; idx < n; idx += stride) {
    const int64_t t = idx / a.H;
    const int h = (int)(idx - t * a.H);
    const uint4 w = *reinterpret_cast<const uint4*>(a.dout + t * a.d_st + (int64_t)h * a.d_sh +
                                                    sub * 8);
    float dv8[8];
    unpack8<kHalf>(w, dv8);
    const float4* oc = reinterpret_cast<const float4*>(a.o_cmp + idx * kD + sub * 8);
    const float4* os = reinterpret_cast<const float4*>(a.o_sel + idx * kD + sub * 8);
    const float4 c0 = oc[0], c1 = oc[1], s0 = os[0], s1 = os[1];
    const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    float dc = 0.f, ds = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      dc = fmaf(dv8[e], cv[e], dc);
      ds = fmaf(dv8[e], sv[e], ds);
    }
#pragma unroll
    for (int x = 1; x < 8; x <<= 1) {
      dc += __shfl_xor(dc, x);
      ds += __shfl_xor(ds, x);
    }
    if (sub == 0) {
      const float g0 = a.gates[t * a.gate_st + (int64_t)h * 2];
      const float g1 = a.gates[t * a.gate_st + (int64_t)h * 2 + 1];
      float4* q = reinterpret_cast<float4*>(a.qs + ((int64_t)h * a.T + t) * 8);
      q[0] = make_float4(a.lse_cmp[(int64_t)h * a.T + t] * kLog2e, g0, g0 * dc,
                         a.lse_sel[(int64_t)h * a.T + t]);
      q[1] = make_float4(g1, g1 * ds, 0.f, 0.f);
      a.dg_tok[t * a.dg_st + (int64_t)h * a.dg_sh] = dc;
      a.dg_tok[t * a.dg_st + (int64_t)h * a.dg_sh + 1] = ds;
    }
  }
}

hipError_t launch_bwd_scalars(const BwdScalarArgs& a, hipStream_t s) {
  const int64_t want = (a.T * a.H + 31) / 32;
  const dim3 g3((unsigned)(want < 16384 ? want : 16384)), b3(256);
  if (a.half) hipLaunchKernelGGL((bwd_scalars_kernel<true>), g3, b3, 0, s, a);
  else hipLaunchKernelGGL((bwd_scalars_kernel<false>), g3, b3, 0, s, a);
  return hipGetLastError();
}

// Per-head gate gradients from [H][T][2] per-token values: sum over tokens in a fixed order
// (float64 partial sums).
__global__ __launch_bounds__(256) void gate_reduce_kernel(const float* dg_tok, int64_t T,
                                                          int32_t H, float* dgates) {
  __shared__ double part[2][256];
  const int h = blockIdx.x, tid = threadIdx.x;
  const float2* src = reinterpret_cast<const float2*>(dg_tok) + (int64_t)h * T;
  double s0 = 0.0, s1 = 0.0;
  for (int64_t t = tid; t < T; t += 256) {
    const float2 v = src[t];
    s0 += v.x;
    s1 += v.y;
  }
  part[0][tid] = s0;
  part[1][tid] = s1;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) {
      part[0][tid] += part[0][tid + w];
      part[1][tid] += part[1][tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) {
    dgates[h * 2] = (float)part[0][0];
    dgates[h * 2 + 1] = (float)part[1][0];
  }
}

hipError_t launch_gate_reduce(const float* dg_tok, int64_t T, int32_t H, float* dgates,
                              hipStream_t s) {
  hipLaunchKernelGGL(gate_reduce_kernel, dim3((unsigned)H), dim3(256), 0, s, dg_tok, T, H,
                     dgates);
  return hipGetLastError();
}

// Bit i of bitmap row (h, u) <- query block i selected key block u (bitmap zeroed before).
__global__ __launch_bounds__(256) void sel_bitmap_kernel(const int32_t* sel, int64_t Nb,
                                                         int32_t n_sel, int64_t n, int64_t words,
                                                         uint32_t* bm) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < n; idx += stride) {
    const int64_t row = idx / n_sel;  // h * Nb + i
    const int64_t h = row / Nb, i = row - h * Nb;
    const int64_t u = sel[idx];
    if (u >= 0 && u < Nb) atomicOr(&bm[(h * Nb + u) * words + (i >> 5)], 1u << (i & 31));
  }
}

hipError_t launch_sel_bitmap(const BwdArgs& a, uint32_t* bitmap, hipStream_t s) {
  const int64_t n = (int64_t)a.H * a.Nb * a.n_sel;
  const int64_t want = (n + 255) / 256;
  hipLaunchKernelGGL(sel_bitmap_kernel, dim3((unsigned)(want < 65536 ? want : 65536)),
                     dim3(256), 0, s, a.sel, a.Nb, a.n_sel, n, a.bm_words, bitmap);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Compression dq. A work-group of 4 waves owns 256 queries of one head (64 per wave, held as
// B operands with their dout rows); the pooled tiles stream through a 2-slot LDS ring, 16 KB
// per tile: [K hi][K lo] of the forward tile and [R(Vc)][TR(Kc)] of the backward tile.
// Per tile: S^T (hi + lo, minus the saved log-sum-exp in the C operand), dP^T = Vc . dout^T,
// dS = P (g0 dP - D) in registers, dq^T += Kc^T . dS^T.
// ---------------------------------------------------------------------------------------
template <bool kHalf>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void cmp_dq_kernel(
    BwdArgs a) {
  constexpr int kStepU4 = 16 * kRecBytes / 16;  // 1024 uint4 per tile step
  __shared__ uint4 lds[2][kStepU4];
  const int64_t n_qtiles = (a.T + 255) / 256;
  const int64_t total = (int64_t)a.H * n_qtiles;
  const int64_t logical = xcd_logical_id(blockIdx.x, total);
  if (logical >= total) return;
  const int h = (int)(logical / n_qtiles);
  const int64_t qt = logical % n_qtiles;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, li = lane & 15;
  const int64_t q0 = qt * 256 + wave * 64;

  bf16x8 qb[4][2], ob[4][2];
  float g0[4], dl[4];
  floatx4 cneg[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int64_t t = q0 + 16 * nt + li;
    const bool ok = t < a.T;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      qb[nt][c] = ok ? *reinterpret_cast<const bf16x8*>(a.q + t * a.q_st + (int64_t)h * a.q_sh +
                                                        32 * c + 8 * g)
                     : bf16x8{};
      ob[nt][c] = ok ? *reinterpret_cast<const bf16x8*>(a.dout + t * a.d_st +
                                                        (int64_t)h * a.d_sh + 32 * c + 8 * g)
                     : bf16x8{};
    }
    float L = INFINITY;
    g0[nt] = 0.f;
    dl[nt] = 0.f;
    if (ok) {
      const float4 s = *reinterpret_cast<const float4*>(a.qs + ((int64_t)h * a.T + t) * 8);
      L = s.x;
      g0[nt] = s.y;
      dl[nt] = s.z;
    }
    cneg[nt] = floatx4{-L, -L, -L, -L};
  }
  floatx4 dqa[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) dqa[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int64_t n = a.n_ctiles;
  const uint4* fwd = reinterpret_cast<const uint4*>(a.pooled) +
                     (int64_t)h * n * (kPooledTileBytes / 16);
  const uint4* bwd = reinterpret_cast<const uint4*>(a.pooled_bwd) +
                     (int64_t)h * n * (kBwdTileBytes / 16);
  uint4 s0, s1, s2, s3;
  auto fetch = [&](int64_t t) {
    const uint4* f = fwd + t * (kPooledTileBytes / 16);
    const uint4* b = bwd + t * (kBwdTileBytes / 16);
    s0 = f[tid];
    s1 = f[256 + tid];
    s2 = b[tid];
    s3 = b[256 + tid];
  };
  auto stash = [&](int slot) {
    lds[slot][tid] = s0;
    lds[slot][256 + tid] = s1;
    lds[slot][512 + tid] = s2;
    lds[slot][768 + tid] = s3;
  };
  fetch(0);
  stash(0);
  __syncthreads();
  // kLast: only the last tile can hold keys past the last pooled token (masked per element)
  auto step = [&](int64_t tau, auto last_tile) {
    constexpr bool kLast = decltype(last_tile)::value;
    fetch(tau + 1 < n ? tau + 1 : tau);
    const uint4* L = lds[(int)(tau & 1)];
    // one 16-key half at a time: its dS values wait in d0 until the second half completes the
    // 32-key B operand of the dq product
    float d0[4][4];
#pragma unroll
    for (int s2_ = 0; s2_ < 2; ++s2_) {
      const bf16x8 h0 = *reinterpret_cast<const bf16x8*>(&L[(2 * s2_) * 64 + lane]);
      const bf16x8 h1 = *reinterpret_cast<const bf16x8*>(&L[(2 * s2_ + 1) * 64 + lane]);
      const bf16x8 l0 = *reinterpret_cast<const bf16x8*>(&L[256 + (2 * s2_) * 64 + lane]);
      const bf16x8 l1 = *reinterpret_cast<const bf16x8*>(&L[256 + (2 * s2_ + 1) * 64 + lane]);
      const bf16x8 v0 = *reinterpret_cast<const bf16x8*>(&L[512 + (2 * s2_) * 64 + lane]);
      const bf16x8 v1 = *reinterpret_cast<const bf16x8*>(&L[512 + (2 * s2_ + 1) * 64 + lane]);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        floatx4 x = mfma_in<kHalf>(h0, qb[nt][0], cneg[nt]);
        x = mfma_in<kHalf>(h1, qb[nt][1], x);
        x = mfma_in<kHalf>(l0, qb[nt][0], x);
        x = mfma_in<kHalf>(l1, qb[nt][1], x);
        floatx4 y = mfma_in<kHalf>(v0, ob[nt][0], floatx4{0.f, 0.f, 0.f, 0.f});
        y = mfma_in<kHalf>(v1, ob[nt][1], y);
        float d[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // keys past the last pooled token carry no probability
          const bool live = !kLast || tau * kTileKeys + 16 * s2_ + 4 * g + r < a.Nb;
          d[r] = live ? fast_exp2(x[r]) * fmaf(g0[nt], y[r], -dl[nt]) : 0.f;
        }
        if (s2_ == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) d0[nt][r] = d[r];
        } else {
          const bf16x8 pb = pack8(d0[nt][0], d0[nt][1], d0[nt][2], d0[nt][3], d[0], d[1], d[2],
                                  d[3]);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            const bf16x8 kt = *reinterpret_cast<const bf16x8*>(&L[768 + mt * 64 + lane]);
            dqa[mt][nt] = mfma16(kt, pb, dqa[mt][nt]);
          }
        }
      }
    }
    stash((int)((tau + 1) & 1));
    __syncthreads();
  };
  for (int64_t tau = 0; tau + 1 < n; ++tau) step(tau, std::false_type{});
  step(n - 1, std::true_type{});
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int64_t t = q0 + 16 * nt + li;
    if (t >= a.T) continue;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int64_t base = (t * a.H + h) * kD + 16 * mt + 4 * g;
      *reinterpret_cast<float4*>(a.dq + base) =
          make_float4(a.scale * dqa[mt][nt][0], a.scale * dqa[mt][nt][1],
                      a.scale * dqa[mt][nt][2], a.scale * dqa[mt][nt][3]);
    }
  }
}

hipError_t launch_cmp_dq(const BwdArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.H * ((a.T + 255) / 256);
  const dim3 g3((unsigned)(((total + 7) / 8) * 8)), b3(256);
  if (a.half) hipLaunchKernelGGL((cmp_dq_kernel<true>), g3, b3, 0, s, a);
  else hipLaunchKernelGGL((cmp_dq_kernel<false>), g3, b3, 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Compression dKc, dVc. A work-group of kWaves waves owns kWaves pooled tiles (32 pooled keys
// per wave, held as B operands: K hi, K lo, Vc rows) and streams one of kDkvParts equal parts
// of the head's query tiles (its 8 KB of row images + the 32 queries' scalars) through a
// 2-slot LDS ring, writing its partial sums; dkv_combine adds the parts in order. (One work-
// group fills a CU: with the query tiles split, 16 heads x 84 groups make 21 full rounds of
// 256 CUs instead of 5.25.) Per query tile: S (queries x
// keys, so that P^T and dS^T come out with queries in the k-slots), dP = dout . Vc^T,
// dVc += (g0 P)^T . dout, dKc += dS^T . q.
// ---------------------------------------------------------------------------------------
constexpr int kDkvWaves = 8;
constexpr int kDkvAhead = 1;  // query tiles in flight beyond the one being computed on (2 is
                              // built and measured 5 % slower)

template <int kWaves, bool kHalf>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2))) void
cmp_dkv_kernel(BwdArgs a) {
  constexpr int kThreads = 64 * kWaves;
  constexpr int kQU4 = kQTileBytes / 16;  // 1024
  constexpr int kSU4 = kTileKeys * 8 / 4;  // 64: 8 floats per query
  constexpr int kChunks = 512 / kThreads;  // 16-byte row chunks staged per thread
  static_assert(kDkvAhead == 1 || kDkvAhead == 2, "one or two tiles in flight");
  __shared__ uint4 lds[2][kQU4 + kSU4];
  const int64_t n_groups = (a.n_ctiles + kWaves - 1) / kWaves;
  const int64_t total = (int64_t)a.H * kDkvParts * n_groups;
  const int64_t logical = xcd_logical_id(blockIdx.x, total);
  if (logical >= total) return;
  // consecutive work-groups (one XCD) share a head and a part: they stream the same tiles
  const int h = (int)(logical / (kDkvParts * n_groups));
  const int part = (int)(logical / n_groups % kDkvParts);
  const int64_t grp = logical % n_groups;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, li = lane & 15;
  const int64_t ct = grp * kWaves + wave;
  const bool active = ct < a.n_ctiles;

  bf16x8 kh[2][2], kl[2][2], vc[2][2];
  {
    const int64_t c = active ? ct : 0;
    const bf16x8* P = reinterpret_cast<const bf16x8*>(
        a.pooled + ((int64_t)h * a.n_ctiles + c) * kPooledTileBytes);
    const bf16x8* PB = reinterpret_cast<const bf16x8*>(
        a.pooled_bwd + ((int64_t)h * a.n_ctiles + c) * kBwdTileBytes);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        kh[s][c2] = P[(2 * s + c2) * 64 + lane];
        kl[s][c2] = P[256 + (2 * s + c2) * 64 + lane];
        vc[s][c2] = PB[(2 * s + c2) * 64 + lane];
      }
  }
  floatx4 dV[2][4], dK[2][4];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      dV[s][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
      dK[s][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

  const int64_t n = a.n_ktiles;  // query tiles
  const int64_t t_begin = part * n / kDkvParts, t_end = (part + 1) * n / kDkvParts;
  constexpr int kImgU4 = kQImgBytes / 16;  // 512: R(q) then R(dout)
  const uint4* qtl = reinterpret_cast<const uint4*>(a.qtiles) + (int64_t)h * n * kImgU4;
  const float* qs = a.qs + (int64_t)h * a.T * 8;
  // The query images hold only the row images R(q), R(dout) (8 KB); each thread scatters its
  // 16-byte chunks into the transposed images TR(q), TR(dout) while staging, which halves the
  // bytes streamed. In LDS the TR records are swizzled (lane l's 16 bytes at slot tr_swizzle(l)):
  // each 2-byte store instruction has every lane write the same dim modulo 8, which in the
  // plain layout puts all 64 lanes in 2 of the 32 banks; the swizzle spreads them over 16,
  // and it only permutes slots inside aligned groups of 8, so the operand reads stay free of
  // conflicts.
  const int tr_lane = tr_swizzle(lane);
  int rsrc[kChunks], tr_pos[kChunks][8];
#pragma unroll
  for (int x = 0; x < kChunks; ++x) {
    const int c = tid + x * kThreads;                      // chunk 0..511
    rsrc[x] = (c < 256) ? c : 512 + (c - 256);             // uint4 index in the LDS tile
    const int trbase = (c < 256) ? 256 : 768;              // its TR group
    const int rec = (c & 255) >> 6, lp = c & 63;
    const int m = 16 * (rec >> 1) + (lp & 15), d0 = 32 * (rec & 1) + 8 * (lp >> 4);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int trec, tlane, tslot;
      vt_position(m, d0 + j, trec, tlane, tslot);
      tr_pos[x][j] = trbase * 8 + (trec * 64 + tr_swizzle(tlane)) * 8 + tslot;  // u16 units
    }
  }
  // staging registers; with kDkvAhead = 2 two tiles are in flight and the loop is unrolled
  // by two so that the buffers stay in named registers
  uint4 r0[2][kChunks], r2[2];
  auto fetch = [&](int b, int64_t t) {
    t = t < n ? t : n - 1;  // past the end the last tile is re-read (and never used)
#pragma unroll
    for (int x = 0; x < kChunks; ++x) r0[b][x] = qtl[t * kImgU4 + tid + x * kThreads];
    if (tid < kSU4) {
      const int64_t qi = t * kTileKeys + (tid >> 1);
      r2[b] = (qi < a.T) ? reinterpret_cast<const uint4*>(qs + qi * 8)[tid & 1]
              : ((tid & 1) ? make_uint4(0, 0, 0, 0)
                           : make_uint4(__builtin_bit_cast(uint32_t, INFINITY), 0, 0,
                                        __builtin_bit_cast(uint32_t, INFINITY)));
    }
  };
  auto stash = [&](int b, int slot) {
    u16* tr = reinterpret_cast<u16*>(lds[slot]);
#pragma unroll
    for (int x = 0; x < kChunks; ++x) {
      lds[slot][rsrc[x]] = r0[b][x];
      const uint32_t w[4] = {r0[b][x].x, r0[b][x].y, r0[b][x].z, r0[b][x].w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t e = (j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xFFFFu);
        // TR images are bf16 (they meet bf16 P and dS in the dKc, dVc products)
        tr[tr_pos[x][j]] = kHalf ? bf16_bits(in_to_float<true>(e)) : (u16)e;
      }
    }
    if (tid < kSU4) lds[slot][kQU4 + tid] = r2[b];
  };
  auto body = [&](int64_t tau, int ld, int st) {
    // load tile tau + kDkvAhead into buffer ld; compute on tile tau; stage tile tau + 1 from
    // buffer st
    fetch(ld, tau + kDkvAhead);
    if (active) {
      const uint4* L = lds[(int)(tau & 1)];
      const float* S = reinterpret_cast<const float*>(L + kQU4);
      float l2[2][4], g0[2][4], dl[2][4];
#pragma unroll
      for (int qh = 0; qh < 2; ++qh)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float4 v = *reinterpret_cast<const float4*>(S + (16 * qh + 4 * g + r) * 8);
          l2[qh][r] = v.x;
          g0[qh][r] = v.y;
          dl[qh][r] = v.z;
        }
      float pg[2][2][4], dc[2][2][4];
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) {
        const bf16x8 qa0 = *reinterpret_cast<const bf16x8*>(&L[(2 * qh) * 64 + lane]);
        const bf16x8 qa1 = *reinterpret_cast<const bf16x8*>(&L[(2 * qh + 1) * 64 + lane]);
        const bf16x8 oa0 = *reinterpret_cast<const bf16x8*>(&L[512 + (2 * qh) * 64 + lane]);
        const bf16x8 oa1 = *reinterpret_cast<const bf16x8*>(&L[512 + (2 * qh + 1) * 64 + lane]);
        const floatx4 cq = {-l2[qh][0], -l2[qh][1], -l2[qh][2], -l2[qh][3]};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          floatx4 x = mfma_in<kHalf>(qa0, kh[s][0], cq);
          x = mfma_in<kHalf>(qa1, kh[s][1], x);
          x = mfma_in<kHalf>(qa0, kl[s][0], x);
          x = mfma_in<kHalf>(qa1, kl[s][1], x);
          floatx4 y = mfma_in<kHalf>(oa0, vc[s][0], floatx4{0.f, 0.f, 0.f, 0.f});
          y = mfma_in<kHalf>(oa1, vc[s][1], y);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = fast_exp2(x[r]);
            pg[qh][s][r] = g0[qh][r] * p;
            dc[qh][s][r] = p * fmaf(g0[qh][r], y[r], -dl[qh][r]);
          }
        }
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 ap = pack8(pg[0][s][0], pg[0][s][1], pg[0][s][2], pg[0][s][3], pg[1][s][0],
                                pg[1][s][1], pg[1][s][2], pg[1][s][3]);
        const bf16x8 ac = pack8(dc[0][s][0], dc[0][s][1], dc[0][s][2], dc[0][s][3], dc[1][s][0],
                                dc[1][s][1], dc[1][s][2], dc[1][s][3]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const bf16x8 tro = *reinterpret_cast<const bf16x8*>(&L[768 + mt * 64 + tr_lane]);
          const bf16x8 trq = *reinterpret_cast<const bf16x8*>(&L[256 + mt * 64 + tr_lane]);
          dV[s][mt] = mfma16(ap, tro, dV[s][mt]);
          dK[s][mt] = mfma16(ac, trq, dK[s][mt]);
        }
      }
    }
    stash(st, (int)((tau + 1) & 1));
    lds_barrier();
  };
  fetch(0, t_begin);
  stash(0, (int)(t_begin & 1));
  if constexpr (kDkvAhead == 2) fetch(0, t_begin + 1);
  lds_barrier();
  if constexpr (kDkvAhead == 1) {
    for (int64_t tau = t_begin; tau < t_end; ++tau) body(tau, 0, 0);
  } else {
    for (int64_t tau = t_begin; tau < t_end; tau += 2) {
      body(tau, 1, 0);
      if (tau + 1 < t_end) body(tau + 1, 0, 1);
    }
  }
  if (!active) return;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t j = ct * kTileKeys + 16 * s + 4 * g + r;
      if (j >= a.Nb) continue;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int64_t o = ((int64_t)part * a.H * a.Nb + (int64_t)h * a.Nb + j) * kD + 16 * mt + li;
        a.dkc_part[o] = dK[s][mt][r];
        a.dvc_part[o] = dV[s][mt][r];
      }
    }
}

// dKc = scale * (part 0 + part 1 + ...), dVc likewise, in that order (repeatable bits)
__global__ __launch_bounds__(256) void dkv_combine_kernel(BwdArgs a, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const float4* pk = reinterpret_cast<const float4*>(a.dkc_part) + i;
  const float4* pv = reinterpret_cast<const float4*>(a.dvc_part) + i;
  float4 k = pk[0], v = pv[0];
#pragma unroll
  for (int p = 1; p < kDkvParts; ++p) {
    const float4 k2 = pk[p * n4], v2 = pv[p * n4];
    k.x += k2.x; k.y += k2.y; k.z += k2.z; k.w += k2.w;
    v.x += v2.x; v.y += v2.y; v.z += v2.z; v.w += v2.w;
  }
  reinterpret_cast<float4*>(a.dkc)[i] =
      make_float4(a.scale * k.x, a.scale * k.y, a.scale * k.z, a.scale * k.w);
  reinterpret_cast<float4*>(a.dvc)[i] = v;
}

hipError_t launch_cmp_dkv(const BwdArgs& a, hipStream_t s) {
  const int64_t total =
      (int64_t)a.H * kDkvParts * ((a.n_ctiles + kDkvWaves - 1) / kDkvWaves);
  const dim3 g3((unsigned)(((total + 7) / 8) * 8)), b3(64 * kDkvWaves);
  if (a.half) hipLaunchKernelGGL((cmp_dkv_kernel<kDkvWaves, true>), g3, b3, 0, s, a);
  else hipLaunchKernelGGL((cmp_dkv_kernel<kDkvWaves, false>), g3, b3, 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n4 = (int64_t)a.H * a.Nb * kD / 4;
  hipLaunchKernelGGL(dkv_combine_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, a,
                     n4);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Selection dq: one wave per 32 queries of a query block (16 for B = 16), walking the block's
// selection as the forward selection kernel does. For each selected tile: S^T = K . q^T, dP^T = V . dout^T (rows of v from
// the backward raw tile), dS = P (g1 dP - D), dq^T += K^T . dS^T; added onto the compression
// dq already in dq.
// ---------------------------------------------------------------------------------------
struct BwdSelIter {
  int idx;
  int64_t prev, tile, tile_end, blk_lo, blk_hi;
};

__device__ __forceinline__ bool bwd_next_block(const BwdArgs& a, const int32_t* row,
                                               BwdSelIter& it) {
  while (it.idx < a.n_sel) {
    const int64_t j = row[it.idx++];
    if (j < 0 || j >= a.Nb || j == it.prev) continue;
    it.prev = j;
    it.blk_lo = j * a.B;
    it.blk_hi = (it.blk_lo + a.B < a.T) ? it.blk_lo + a.B : a.T;
    it.tile = it.blk_lo / kTileKeys;
    it.tile_end = (it.blk_hi - 1) / kTileKeys + 1;
    return true;
  }
  return false;
}

template <int NT, bool kHalf>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void sel_dq_kernel(
    BwdArgs a) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, li = lane & 15;
  const int parts = (a.B > 32) ? a.B / 32 : 1;  // 32 queries per wave
  const int64_t n_items = (int64_t)a.H * a.Nb * parts;
  const int64_t n_wg = (n_items + 3) / 4;
  const int64_t wg = xcd_logical_id(blockIdx.x, n_wg);
  const int64_t item = wg * 4 + wave;
  if (wg >= n_wg || item >= n_items) return;
  const int part = (int)(item % parts);
  const int64_t hi_ = item / parts;
  const int h = (int)(hi_ / a.Nb);
  const int64_t i = hi_ % a.Nb;
  const int64_t q0 = i * a.B + 32 * part;

  bf16x8 qb[NT][2], ob[NT][2];
  float l2[NT], g1[NT], dl[NT];
  bool ok[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int64_t t = q0 + 16 * nt + li;
    ok[nt] = t < a.T && 16 * nt + li + 32 * part < a.B;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      qb[nt][c] = ok[nt] ? *reinterpret_cast<const bf16x8*>(a.q + t * a.q_st +
                                                            (int64_t)h * a.q_sh + 32 * c + 8 * g)
                         : bf16x8{};
      ob[nt][c] = ok[nt] ? *reinterpret_cast<const bf16x8*>(a.dout + t * a.d_st +
                                                            (int64_t)h * a.d_sh + 32 * c + 8 * g)
                         : bf16x8{};
    }
    l2[nt] = INFINITY;
    g1[nt] = 0.f;
    dl[nt] = 0.f;
    if (ok[nt]) {
      const float4 s = *reinterpret_cast<const float4*>(a.qs + ((int64_t)h * a.T + t) * 8);
      const float4 s2 = *reinterpret_cast<const float4*>(a.qs + ((int64_t)h * a.T + t) * 8 + 4);
      l2[nt] = s.w;
      g1[nt] = s2.x;
      dl[nt] = s2.y;
    }
  }
  floatx4 dqa[4][NT];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) dqa[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int32_t* row = a.sel + ((int64_t)h * a.Nb + i) * a.n_sel;
  const unsigned char* raw = a.raw + (int64_t)h * a.n_ktiles * kRawTileBytes;
  const unsigned char* rawb = a.raw_bwd + (int64_t)h * a.n_ktiles * kBwdTileBytes;
  BwdSelIter it{0, -1, 0, 0, 0, 0};
  bool valid = bwd_next_block(a, row, it);
  while (valid) {
    const bf16x8* K = reinterpret_cast<const bf16x8*>(raw + it.tile * kRawTileBytes);
    const bf16x8* RB = reinterpret_cast<const bf16x8*>(rawb + it.tile * kBwdTileBytes);
    bf16x8 kr[4], vr[4], tk[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      kr[x] = K[x * 64 + lane];
      vr[x] = RB[x * 64 + lane];
      tk[x] = RB[256 + x * 64 + lane];
    }
    const int64_t t0 = it.tile * kTileKeys;
    const int lo = (int)((it.blk_lo > t0) ? it.blk_lo - t0 : 0);
    const int hi = (int)((it.blk_hi < t0 + kTileKeys) ? it.blk_hi - t0 : kTileKeys);
    floatx4 acc[2][NT], dp[2][NT];
#pragma unroll
    for (int s2_ = 0; s2_ < 2; ++s2_)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const floatx4 x = mfma_in<kHalf>(kr[2 * s2_], qb[nt][0], floatx4{0.f, 0.f, 0.f, 0.f});
        acc[s2_][nt] = mfma_in<kHalf>(kr[2 * s2_ + 1], qb[nt][1], x);
        const floatx4 y = mfma_in<kHalf>(vr[2 * s2_], ob[nt][0], floatx4{0.f, 0.f, 0.f, 0.f});
        dp[s2_][nt] = mfma_in<kHalf>(vr[2 * s2_ + 1], ob[nt][1], y);
      }
#pragma unroll
    for (int s2_ = 0; s2_ < 2; ++s2_)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = 16 * s2_ + 4 * g + r;
        if (key < lo || key >= hi) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[s2_][nt][r] = -INFINITY;
        }
      }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float d[2][4];
#pragma unroll
      for (int s2_ = 0; s2_ < 2; ++s2_)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          d[s2_][r] = fast_exp2(fmaf(acc[s2_][nt][r], a.logit_mult, -l2[nt])) *
                      fmaf(g1[nt], dp[s2_][nt][r], -dl[nt]);
      const bf16x8 pb = pack8(d[0][0], d[0][1], d[0][2], d[0][3], d[1][0], d[1][1], d[1][2],
                              d[1][3]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) dqa[mt][nt] = mfma16(tk[mt], pb, dqa[mt][nt]);
    }
    if (it.tile + 1 < it.tile_end) {
      ++it.tile;
    } else {
      valid = bwd_next_block(a, row, it);
    }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (!ok[nt]) continue;
    const int64_t t = q0 + 16 * nt + li;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      float4* p = reinterpret_cast<float4*>(a.dq + (t * a.H + h) * kD + 16 * mt + 4 * g);
      const float4 o = *p;
      *p = make_float4(o.x + a.scale * dqa[mt][nt][0], o.y + a.scale * dqa[mt][nt][1],
                       o.z + a.scale * dqa[mt][nt][2], o.w + a.scale * dqa[mt][nt][3]);
    }
  }
}

hipError_t launch_sel_dq(const BwdArgs& a, hipStream_t s) {
  const int parts = (a.B > 32) ? a.B / 32 : 1;
  const int64_t n_wg = ((int64_t)a.H * a.Nb * parts + 3) / 4;
  const dim3 g3((unsigned)(((n_wg + 7) / 8) * 8)), b3(256);
  if (a.B == 16) {
    if (a.half) hipLaunchKernelGGL((sel_dq_kernel<1, true>), g3, b3, 0, s, a);
    else hipLaunchKernelGGL((sel_dq_kernel<1, false>), g3, b3, 0, s, a);
  } else {
    if (a.half) hipLaunchKernelGGL((sel_dq_kernel<2, true>), g3, b3, 0, s, a);
    else hipLaunchKernelGGL((sel_dq_kernel<2, false>), g3, b3, 0, s, a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Selection dk, dv. One work-group of 4 waves per (head, key block u); wave w owns key tile
// kt = w % KT of the block (KT = B/32 tiles of 32 keys, at least 1) and split w / KT of the
// query tiles. Per selecting query tile: S = q . K^T, dP = dout . V^T, dv += (g1 P)^T . dout,
// dk += dS^T . q. The epilogue adds the split sums in fixed order, then the compression
// branch's pooled gradients spread over the block, dKc_u / n_u and dVc_u / n_u, and writes dk,
// dv for every token of the block.
//
// The query blocks that chose u are listed in LDS first (bitmap row, ascending; up to
// kSdListCap at a time), then their tiles stream through an LDS ring: a stage is the NSPLIT
// tiles that the splits consume together, copied with global_load_lds by all four waves, up
// to DEPTH - 1 stages ahead of the one computed on. Only the row images R(q), R(dout) and the
// tile's 32 rows of per-query scalars are copied (9 KB a tile); the transposed operands
// (queries in the k-slots, for dv and dk) are read from the row images with
// ds_read_b64_tr_b16, which hands lane i of each 16-lane group column i of the four 16-element
// rows that the group's lanes address. The ring is read with inline-asm LDS reads, each block
// waiting for its own reads: an ordinary LDS read would make the compiler wait for every copy
// in flight, since it cannot tell the ring's slots apart.
// ---------------------------------------------------------------------------------------
constexpr int kSdTileLds = 9 * 1024;  // R(q) 4 KB, R(dout) 4 KB, scalars (512 B used)
constexpr int kSdRingTiles = 8;       // 72 KB of query tiles
constexpr int kSdListCap = 1024;      // selecting query blocks listed at a time

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Two fp16 values -> the same two values rounded to bf16 (nearest even).
__device__ __forceinline__ uint32_t f16x2_to_bf16x2(uint32_t w) {
  return bf16_bits(in_to_float<true>(w & 0xFFFFu)) |
         ((uint32_t)bf16_bits(in_to_float<true>(w >> 16)) << 16);
}

// Row images in LDS. 16-byte chunk c of a 1 KB record sits in slot tau(c), tau(16 g' + i) =
// 16 g' + (i ^ 12 (g' & 1)) (an involution): measured with the LDS bank-conflict counter on
// gfx950, both the transposed reads below and the 16-byte row-operand reads (lane l takes slot
// tau(l)) are then free of conflicts (the plain layout conflicts on the transposed reads, and
// XOR 4 or 8 alone on one of the two).
__device__ __forceinline__ int chunk_slot(int c) { return c ^ (12 * ((c >> 4) & 1)); }

// ds_read_b64_tr_b16 (gfx950): lane i of each 16-lane group receives column i of the four
// 16-element rows that the group's lanes address (lanes 4j..4j+3 give row j, four elements
// each). On a row image it yields a transposed operand: lane (n, g) gets, for query rows
// 4g + j of a 16-row half, the element of dim n of a 16-dim group. Byte offset of this lane
// in a record pair (mt, half): tr_lane_offset(lane) + 1024 (2 half + mt / 2) + 512 (mt % 2).
// (It delivers about half the LDS bandwidth of a 16-byte read, 110 against 200 bytes per
// clock per CU, measured; cmp_dkv, whose LDS pipe is busy, keeps building its transposed
// images with 2-byte stores while staging: with these reads it was 20 % slower.)
__device__ __forceinline__ uint32_t tr_lane_offset(int lane) {
  const int g = lane >> 4, j = (lane >> 2) & 3, hi = (lane & 3) >> 1;
  return (uint32_t)((16 * hi + ((4 * g + j) ^ (12 * hi))) * 16 + 8 * (lane & 1));
}

// 4-byte global->LDS copy per lane: lane l's 4 bytes at src land at dst + 4 l (dst the same
// for every lane). Out of line of the kernel template for the same reason as copy16_to_lds.
__device__ __forceinline__ void copy4_to_lds(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
}

// Waits until at most p stages of L copies each are still in flight (p <= P).
template <int L, int P>
__device__ __forceinline__ void wait_stages(int64_t p) {
  if constexpr (P <= 0) {
    wait_vmem<0>();
  } else {
    if (p >= P) wait_vmem<P * L>();
    else wait_stages<L, P - 1>(p);
  }
}

template <int KT, bool kHalf>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void sel_dkv_kernel(
    BwdArgs a) {
  constexpr int NSPLIT = 4 / KT;                // waves sharing a key tile
  constexpr int STAGE = NSPLIT * kSdTileLds;    // bytes per stage
  constexpr int DEPTH = kSdRingTiles / NSPLIT;  // stages in the ring
  constexpr int LOADS = 3 * NSPLIT;             // copies per wave per stage
  static_assert(DEPTH >= 2, "at least one stage ahead");
  static_assert((NSPLIT - 1) * KT * 16 * 64 * 16 <= kSdRingTiles * kSdTileLds,
                "the split sums fit in the ring");
  __shared__ __attribute__((aligned(16))) unsigned char ring[kSdRingTiles * kSdTileLds];
  __shared__ int list[kSdListCap];
  __shared__ int wsum[16];
  const int64_t total = (int64_t)a.H * a.Nb;
  const int64_t logical = xcd_logical_id(blockIdx.x, total);
  if (logical >= total) return;
  const int h = (int)(logical / a.Nb);
  const int64_t u = logical % a.Nb;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, li = lane & 15;
  const int kt = wave % KT, split = wave / KT;
  const int64_t k_lo = u * a.B;
  const int64_t k_hi = (k_lo + a.B < a.T) ? k_lo + a.B : a.T;
  const int64_t tile = k_lo / kTileKeys + kt;
  const bool active = tile * kTileKeys < k_hi;

  bf16x8 kr[2][2], vr[2][2];
  {
    const int64_t tt = active ? tile : k_lo / kTileKeys;
    const bf16x8* K = reinterpret_cast<const bf16x8*>(
        a.raw + ((int64_t)h * a.n_ktiles + tt) * kRawTileBytes);
    const bf16x8* RB = reinterpret_cast<const bf16x8*>(
        a.raw_bwd + ((int64_t)h * a.n_ktiles + tt) * kBwdTileBytes);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        kr[s][c] = K[(2 * s + c) * 64 + lane];
        vr[s][c] = RB[(2 * s + c) * 64 + lane];
      }
  }
  floatx4 dK[2][4], dV[2][4];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      dK[s][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
      dV[s][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

  const uint32_t* bm = a.bitmap + ((int64_t)h * a.Nb + u) * a.bm_words;
  // Lists the set bits of the bitmap row whose rank (ascending order) lies in
  // [lo, lo + kSdListCap) and returns the row's count. 256 words per round, one per thread,
  // four rounds loaded together; ranks from a scan over the threads.
  auto build_list = [&](int64_t lo) -> int64_t {
    int64_t base = 0;
    for (int64_t w0 = 0; w0 < a.bm_words; w0 += 1024) {
      uint32_t wd[4];
      int cnt[4], inc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t w = w0 + 256 * r + tid;
        wd[r] = (w < a.bm_words) ? bm[w] : 0u;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        cnt[r] = __builtin_popcount(wd[r]);
        inc[r] = wave_inclusive_sum(cnt[r], lane);
        if (lane == 63) wsum[4 * r + wave] = inc[r];
      }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int before = 0, all = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int x = wsum[4 * r + w];
          before += (w < wave) ? x : 0;
          all += x;
        }
        int64_t rank = base + before + inc[r] - cnt[r] - lo;
        const int64_t word = w0 + 256 * r + tid;
        uint32_t bits = wd[r];
        while (bits) {
          const int b = __builtin_ctz(bits);
          bits &= bits - 1;
          if (rank >= 0 && rank < kSdListCap) list[rank] = (int)(word * 32 + b);
          ++rank;
        }
        base += all;
      }
      __syncthreads();
    }
    return base;
  };

  const unsigned char* qtl = a.qtiles + (int64_t)h * a.n_ktiles * kQImgBytes;
  const float* qs = a.qs + (int64_t)h * a.T * 8;
  const uint32_t ring_lds = lds_address(ring);
  // LDS layout of a tile: the row images with their chunks permuted (chunk_slot; the copying
  // lane l fetches chunk chunk_slot(l)), then the scalars field-major, [L_sel, g1,
  // g1 dout . O_sel, unused][32 rows]; transposed reads at tr_lane_offset.
  const int tau_lane = chunk_slot(lane);
  const uint32_t tr_lane = tr_lane_offset(lane);
  const uint32_t qs_lane = 8192 + 16 * g;  // rows 4g..4g+3 of a field

  // item i of the list: query tile i % KT of block list[i / KT] (for B = 16 the 32-row tile
  // holding the block); tile indices fit 32 bits (T < 2^31)
  auto item_tile = [&](int blk, int i) -> int {
    return (int)((int64_t)blk * a.B / kTileKeys) + i % KT;
  };
  const int n_qtiles = (int)a.n_ktiles;
  const int T32 = (int)a.T;
  // copies of stage n: per tile, wave w copies R(q) record w, R(dout) record w and scalar
  // field w (qs[t][3 + w] of the tile's 32 rows, by lanes 0..31); items past the list re-read
  // a valid tile that is never used
  auto issue = [&](int n, int n_items) {
    unsigned char* st = ring + (n % DEPTH) * STAGE;
#pragma unroll
    for (int j = 0; j < NSPLIT; ++j) {
      const int i = n * NSPLIT + j;
      int qt = (i < n_items) ? item_tile(__builtin_amdgcn_readfirstlane(list[i / KT]), i) : 0;
      qt = (qt < n_qtiles) ? qt : n_qtiles - 1;
      const unsigned char* src = qtl + (int64_t)qt * kQImgBytes;
      unsigned char* dst = st + j * kSdTileLds;
      copy16_to_lds(src + wave * kRecBytes + 16 * tau_lane, dst + wave * kRecBytes);
      copy16_to_lds(src + 4096 + wave * kRecBytes + 16 * tau_lane, dst + 4096 + wave * kRecBytes);
      int t = qt * kTileKeys + (lane & 31);
      t = (t < T32) ? t : T32 - 1;
      if (lane < 32) copy4_to_lds(qs + (int64_t)t * 8 + 3 + wave, dst + 8192 + 128 * wave);
    }
  };

  auto compute = [&](int n, int n_items) {
    const int i = n * NSPLIT + split;
    if (i >= n_items) return;
    const int blk = __builtin_amdgcn_readfirstlane(list[i / KT]);
    const int qt = item_tile(blk, i);
    // rows of the tile inside the block: [lo_rel, hi_rel)
    const int64_t b_lo = (int64_t)blk * a.B;
    const int64_t b_hi = (b_lo + a.B < a.T) ? b_lo + a.B : a.T;
    const int64_t t0 = (int64_t)qt * kTileKeys;
    if (t0 >= b_hi) return;
    const int lo_rel = (b_lo > t0) ? (int)(b_lo - t0) : 0;
    const int hi_rel = (b_hi - t0 < kTileKeys) ? (int)(b_hi - t0) : kTileKeys;
    const uint32_t sb = ring_lds + (uint32_t)((n % DEPTH) * STAGE + split * kSdTileLds);

    // row images and per-row scalars in one block (one wait)
    u32x4 rq[4], ro[4], l2v[2], g1v[2], dlv[2];
    asm volatile(
        "ds_read_b128 %0, %14\n\t"
        "ds_read_b128 %1, %14 offset:1024\n\t"
        "ds_read_b128 %2, %14 offset:2048\n\t"
        "ds_read_b128 %3, %14 offset:3072\n\t"
        "ds_read_b128 %4, %14 offset:4096\n\t"
        "ds_read_b128 %5, %14 offset:5120\n\t"
        "ds_read_b128 %6, %14 offset:6144\n\t"
        "ds_read_b128 %7, %14 offset:7168\n\t"
        "ds_read_b128 %8, %15\n\t"
        "ds_read_b128 %9, %15 offset:64\n\t"
        "ds_read_b128 %10, %15 offset:128\n\t"
        "ds_read_b128 %11, %15 offset:192\n\t"
        "ds_read_b128 %12, %15 offset:256\n\t"
        "ds_read_b128 %13, %15 offset:320\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(rq[0]), "=&v"(rq[1]), "=&v"(rq[2]), "=&v"(rq[3]), "=&v"(ro[0]), "=&v"(ro[1]),
          "=&v"(ro[2]), "=&v"(ro[3]), "=&v"(l2v[0]), "=&v"(l2v[1]), "=&v"(g1v[0]),
          "=&v"(g1v[1]), "=&v"(dlv[0]), "=&v"(dlv[1])
        : "v"(sb + 16 * tau_lane), "v"(sb + qs_lane)
        : "memory");

    float pg[2][2][4], ds[2][2][4];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      float l2[4], g1[4], dl[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rel = 16 * qh + 4 * g + r;
        const bool in = rel >= lo_rel && rel < hi_rel;
        // (element copies first: a bit cast of a vector element reads element 0)
        const uint32_t wl = l2v[qh][r], wg = g1v[qh][r], wd = dlv[qh][r];
        l2[r] = in ? __builtin_bit_cast(float, wl) : INFINITY;
        g1[r] = in ? __builtin_bit_cast(float, wg) : 0.f;
        dl[r] = in ? __builtin_bit_cast(float, wd) : 0.f;
      }
      const bf16x8 qa0 = __builtin_bit_cast(bf16x8, rq[2 * qh]);
      const bf16x8 qa1 = __builtin_bit_cast(bf16x8, rq[2 * qh + 1]);
      const bf16x8 oa0 = __builtin_bit_cast(bf16x8, ro[2 * qh]);
      const bf16x8 oa1 = __builtin_bit_cast(bf16x8, ro[2 * qh + 1]);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        floatx4 x = mfma_in<kHalf>(qa0, kr[s][0], floatx4{0.f, 0.f, 0.f, 0.f});
        x = mfma_in<kHalf>(qa1, kr[s][1], x);
        floatx4 y = mfma_in<kHalf>(oa0, vr[s][0], floatx4{0.f, 0.f, 0.f, 0.f});
        y = mfma_in<kHalf>(oa1, vr[s][1], y);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = fast_exp2(fmaf(x[r], a.logit_mult, -l2[r]));
          pg[qh][s][r] = g1[r] * p;
          ds[qh][s][r] = p * fmaf(g1[r], y[r], -dl[r]);
        }
      }
    }

    // P^T and dS^T operands (keys 16s.., queries in the k-slots)
    u32x4 apw[2], asw[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      apw[s] = __builtin_bit_cast(u32x4, pack8(pg[0][s][0], pg[0][s][1], pg[0][s][2], pg[0][s][3],
                                               pg[1][s][0], pg[1][s][1], pg[1][s][2], pg[1][s][3]));
      asw[s] = __builtin_bit_cast(u32x4, pack8(ds[0][s][0], ds[0][s][1], ds[0][s][2], ds[0][s][3],
                                               ds[1][s][0], ds[1][s][1], ds[1][s][2], ds[1][s][3]));
    }
    // Transposed operands: [mt][query half], record (2 half + mt / 2), dims 16 (mt % 2)...
    // The P^T, dS^T operands pass through the block: they are formed from every S and dP
    // product, so no matrix product still reads a register when the block's reads land in
    // registers the compiler has freed (it does not see the LDS writes inside the asm).
    u32x2 tq[4][2], to[4][2];
    asm volatile(
        "ds_read_b64_tr_b16 %0, %20\n\t"
        "ds_read_b64_tr_b16 %1, %20 offset:2048\n\t"
        "ds_read_b64_tr_b16 %2, %20 offset:512\n\t"
        "ds_read_b64_tr_b16 %3, %20 offset:2560\n\t"
        "ds_read_b64_tr_b16 %4, %20 offset:1024\n\t"
        "ds_read_b64_tr_b16 %5, %20 offset:3072\n\t"
        "ds_read_b64_tr_b16 %6, %20 offset:1536\n\t"
        "ds_read_b64_tr_b16 %7, %20 offset:3584\n\t"
        "ds_read_b64_tr_b16 %8, %20 offset:4096\n\t"
        "ds_read_b64_tr_b16 %9, %20 offset:6144\n\t"
        "ds_read_b64_tr_b16 %10, %20 offset:4608\n\t"
        "ds_read_b64_tr_b16 %11, %20 offset:6656\n\t"
        "ds_read_b64_tr_b16 %12, %20 offset:5120\n\t"
        "ds_read_b64_tr_b16 %13, %20 offset:7168\n\t"
        "ds_read_b64_tr_b16 %14, %20 offset:5632\n\t"
        "ds_read_b64_tr_b16 %15, %20 offset:7680\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(tq[0][0]), "=&v"(tq[0][1]), "=&v"(tq[1][0]), "=&v"(tq[1][1]), "=&v"(tq[2][0]),
          "=&v"(tq[2][1]), "=&v"(tq[3][0]), "=&v"(tq[3][1]), "=&v"(to[0][0]), "=&v"(to[0][1]),
          "=&v"(to[1][0]), "=&v"(to[1][1]), "=&v"(to[2][0]), "=&v"(to[2][1]), "=&v"(to[3][0]),
          "=&v"(to[3][1]), "+v"(apw[0]), "+v"(apw[1]), "+v"(asw[0]), "+v"(asw[1])
        : "v"(sb + tr_lane)
        : "memory");
    bf16x8 trq[4], tro[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      u32x4 wq = {tq[mt][0].x, tq[mt][0].y, tq[mt][1].x, tq[mt][1].y};
      u32x4 wo = {to[mt][0].x, to[mt][0].y, to[mt][1].x, to[mt][1].y};
      if constexpr (kHalf) {  // the products with P and dS take both operands in bf16
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wq[e] = f16x2_to_bf16x2(wq[e]);
          wo[e] = f16x2_to_bf16x2(wo[e]);
        }
      }
      trq[mt] = __builtin_bit_cast(bf16x8, wq);
      tro[mt] = __builtin_bit_cast(bf16x8, wo);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8 ap = __builtin_bit_cast(bf16x8, apw[s]);
      const bf16x8 as = __builtin_bit_cast(bf16x8, asw[s]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        dV[s][mt] = mfma16(ap, tro[mt], dV[s][mt]);
        dK[s][mt] = mfma16(as, trq[mt], dK[s][mt]);
      }
    }
  };

  // every wave takes part in listing, copying and the barriers; waves whose key tile lies past
  // the end of the sequence skip the products
  const int64_t n_sel = build_list(0);
  for (int64_t lo = 0; lo < n_sel; lo += kSdListCap) {
    if (lo > 0) {
      __syncthreads();  // the ring and the list are no longer read
      build_list(lo);
    }
    const int n_items = (int)((n_sel - lo < kSdListCap) ? n_sel - lo : kSdListCap) * KT;
    const int n_stages = (n_items + NSPLIT - 1) / NSPLIT;
    int issued = 0;
    for (; issued < DEPTH - 1 && issued < n_stages; ++issued) issue(issued, n_items);
    for (int n = 0; n < n_stages; ++n) {
      wait_stages<LOADS, DEPTH - 2>(issued - n - 1);  // this wave's copies of stage n landed
      lds_barrier();  // everyone's copies of stage n landed; stage n - 1 has been read
      if (issued < n_stages) {
        issue(issued, n_items);
        ++issued;
      }
      if (active) compute(n, n_items);
    }
  }
  if (NSPLIT > 1 && n_sel > 0) {  // add the split sums of the waves sharing a tile, in order
    floatx4(*red)[16][64] = reinterpret_cast<floatx4(*)[16][64]>(ring);
    __syncthreads();  // the ring is free
    if (split > 0) {
      const int slot = (split - 1) * KT + kt;
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          red[slot][s * 4 + mt][lane] = dK[s][mt];
          red[slot][8 + s * 4 + mt][lane] = dV[s][mt];
        }
    }
    __syncthreads();
    if (split == 0) {
      for (int sp = 1; sp < NSPLIT; ++sp) {
        const int slot = (sp - 1) * KT + kt;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            dK[s][mt] += red[slot][s * 4 + mt][lane];
            dV[s][mt] += red[slot][8 + s * 4 + mt][lane];
          }
      }
    }
  }
  if (split != 0 || !active) return;
  const float inv_n = 1.0f / (float)(k_hi - k_lo);
  const float* dkc = a.dkc + ((int64_t)h * a.Nb + u) * kD;
  const float* dvc = a.dvc + ((int64_t)h * a.Nb + u) * kD;
  float ck[4], cv[4];  // the pooled gradients spread over the block, read before any store
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    ck[mt] = dkc[16 * mt + li] * inv_n;
    cv[mt] = dvc[16 * mt + li] * inv_n;
  }
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t t = tile * kTileKeys + 16 * s + 4 * g + r;
      if (t < k_lo || t >= k_hi) continue;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int64_t o = (t * a.H + h) * kD + 16 * mt + li;
        a.dk[o] = a.scale * dK[s][mt][r] + ck[mt];
        a.dv[o] = dV[s][mt][r] + cv[mt];
      }
    }
}

hipError_t launch_sel_dkv(const BwdArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.H * a.Nb;
  const dim3 g3((unsigned)(((total + 7) / 8) * 8)), b3(256);
  switch (a.B) {
    case 16:
    case 32:
      if (a.half) hipLaunchKernelGGL((sel_dkv_kernel<1, true>), g3, b3, 0, s, a);
      else hipLaunchKernelGGL((sel_dkv_kernel<1, false>), g3, b3, 0, s, a);
      break;
    case 64:
      if (a.half) hipLaunchKernelGGL((sel_dkv_kernel<2, true>), g3, b3, 0, s, a);
      else hipLaunchKernelGGL((sel_dkv_kernel<2, false>), g3, b3, 0, s, a);
      break;
    case 128:
      if (a.half) hipLaunchKernelGGL((sel_dkv_kernel<4, true>), g3, b3, 0, s, a);
      else hipLaunchKernelGGL((sel_dkv_kernel<4, false>), g3, b3, 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace s3r
