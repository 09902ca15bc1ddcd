// Top-k block selection per (head, query block), after an optional forced prefix of blocks and
// the query block's own block.
//
// Speed3R technical summary (gist.science), "Methodologie" section 1: the selection branch
// keeps, per query block, the k key blocks with the highest compression score. This kernel
// makes that choice exactly and deterministically: order by (score descending, block index
// ascending), output the k indices in ascending order.
//
// One work-group (4 waves) per score row. The row is streamed once with 16-byte loads and no
// part of it is held in registers (so many rows are in flight per CU); in step 2 only the few
// threads whose maximum reaches theta read entries again, and most of them one chunk.
//  1. Each thread's maximum key over its entries (order-preserving 32-bit keys), the chunk
//     that holds it, and the largest key among its other chunks; theta = the k-th largest of
//     the 256 thread maxima (bitwise search in one wave). The k largest thread maxima are k
//     distinct entries >= theta, so every entry of the true top-k is >= theta.
//  2. Entries >= theta (usually a few dozen) are compacted into LDS: a thread whose other
//     chunks all lie below theta re-reads only the chunk of its maximum, the others (ties, or
//     several large entries in one thread) re-read all their chunks. Each candidate's rank is
//     its number of better candidates; rank < k selects it, and its output slot is the number
//     of selected candidates with a smaller index.
//  3. If more than kCap candidates survive (heavy ties), an exact fallback finds the k-th key
//     and the cut inside the tied keys by bitwise search over all entries (re-reading the
//     row), then writes the selected indices in ascending order with block-wide prefix counts.
#include "s3r_common.hpp"
#include "s3r_launch.hpp"

namespace s3r {

constexpr int kCap = 256;

// Unsigned key whose order equals the float order; -0 is folded onto +0 first. Negative
// numbers have every bit flipped, the others only the sign bit.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int sh = 1; sh < 64; sh *= 2) x += __shfl_xor(x, sh);
  return x;
}

__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
  __shared__ uint32_t tmax_s[256];
  __shared__ uint32_t cand_key[kCap];
  __shared__ int32_t cand_idx[kCap];
  __shared__ int32_t cand_rank[kCap];
  __shared__ int part[4];
  __shared__ uint32_t s_theta;
  __shared__ int s_count;

  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int Nb = (int)a.Nb;
  const int F = a.forced;       // blocks 0..F-1 are selected outright
  const int qi = (int)(row % a.Nb);
  const bool own = a.own && qi >= F;  // the row's own block, selected outright too
  const int ncand = Nb - F - (own ? 1 : 0);
  const int k = a.topk < ncand ? a.topk : ncand;  // chosen among the other blocks
  int32_t* row_out = a.sel + row * a.n_sel;
  for (int j = tid; j < F; j += 256) row_out[j] = j;
  for (int j = F + (own ? 1 : 0) + k + tid; j < a.n_sel; j += 256) row_out[j] = -1;
  if (k >= ncand) {  // every block: F..Nb-1 in order (the own block among them)
    for (int j = F + tid; j < Nb; j += 256) row_out[j] = j;
    return;
  }
  int32_t* out = row_out + F;
  const float* src = a.score + row * a.ld;
  auto candidate = [&](int j) { return j >= F && j < Nb && !(own && j == qi); };
  auto key_of = [&](float f, int j) { return candidate(j) ? order_key(f) : 0u; };
  // Thread tid owns entries 1024c + 4tid .. +3 of chunk c. The row stride is a multiple of 32
  // floats, so a 16-byte load starting below Nb stays inside the row; chunks past the end
  // re-read the row's first entries (their keys are masked).
  const int nchunks = (Nb + 1023) / 1024;
  auto load4 = [&](int c, int& j0) {
    j0 = c * 1024 + 4 * tid;
    return *reinterpret_cast<const float4*>(src + (j0 < Nb ? j0 : 0));
  };

  // 1. thread maxima (and where they are), theta
  uint32_t tmax = 0;  // largest key of this thread's entries
  uint32_t t2 = 0;    // largest key among its chunks other than cbest
  int cbest = 0;      // first chunk holding tmax
#pragma unroll 4
  for (int c = 0; c < nchunks; ++c) {
    int j0;
    const float4 v = load4(c, j0);
    const uint32_t m01 = max(key_of(v.x, j0), key_of(v.y, j0 + 1));
    const uint32_t m23 = max(key_of(v.z, j0 + 2), key_of(v.w, j0 + 3));
    const uint32_t m = max(m01, m23);
    t2 = max(t2, min(tmax, m));  // the smaller of the old best and this chunk is "other"
    cbest = m > tmax ? c : cbest;
    tmax = max(tmax, m);
  }
  tmax_s[tid] = tmax;
  if (tid == 0) s_count = 0;
  __syncthreads();

  if (wave == 0) {
    uint32_t t4[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) t4[x] = tmax_s[lane * 4 + x];
    uint32_t theta = 0;
    for (int b = 31; b >= 0; --b) {
      const uint32_t cand = theta | (1u << b);
      int cnt = 0;
#pragma unroll
      for (int x = 0; x < 4; ++x) cnt += __popcll(__ballot(t4[x] >= cand));
      if (cnt >= k) theta = cand;
    }
    if (lane == 0) s_theta = theta;
  }
  __syncthreads();
  const uint32_t theta = s_theta;

  // 2. candidates >= theta: only a thread whose maximum reaches theta can hold one, so only
  //    those threads (typically k or a few more of the 256) read entries again: the chunk of
  //    their maximum, or every chunk if another one also reaches theta
  auto take = [&](int c) {
    int j0;
    const float4 v = load4(c, j0);
    const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t key = order_key(f[i]);
      if (candidate(j0 + i) && key >= theta) {
        const int pos = atomicAdd(&s_count, 1);
        if (pos < kCap) {
          cand_key[pos] = key;
          cand_idx[pos] = j0 + i;
        }
      }
    }
  };
  if (t2 >= theta) {
#pragma unroll 4
    for (int c = 0; c < nchunks; ++c) take(c);
  } else if (tmax >= theta) {
    take(cbest);
  }
  __syncthreads();
  const int C = s_count;

  if (C <= kCap) {
    if (tid < C) {
      const uint32_t mk = cand_key[tid];
      const int mi = cand_idx[tid];
      int rank = 0;
      for (int c = 0; c < C; ++c) {
        const uint32_t ok = cand_key[c];
        rank += (ok > mk) || (ok == mk && cand_idx[c] < mi);
      }
      cand_rank[tid] = rank;
    }
    __syncthreads();
    if (tid < C && cand_rank[tid] < k) {
      const int mi = cand_idx[tid];
      int pos = (own && qi < mi) ? 1 : 0;
      for (int c = 0; c < C; ++c) pos += (cand_rank[c] < k) && (cand_idx[c] < mi);
      out[pos] = mi;
    }
    if (own && tid == 0) {
      int pos = 0;
      for (int c = 0; c < C; ++c) pos += (cand_rank[c] < k) && (cand_idx[c] < qi);
      out[pos] = qi;
    }
    return;
  }

  // ---- 3. exact fallback: k-th key by bitwise search over all entries ---------------------
  // (one entry per thread per step of 256: j = 256e + tid, the row re-read each time)
  auto block_count = [&](int local) -> int {
    const int w = wave_sum(local);
    __syncthreads();
    if (lane == 0) part[wave] = w;
    __syncthreads();
    return part[0] + part[1] + part[2] + part[3];
  };
  const int E = (Nb + 255) / 256;
  auto key_e = [&](int e) {  // 0 for entries that are not candidates
    const int j = e * 256 + tid;
    return j < Nb ? key_of(src[j], j) : 0u;
  };
  uint32_t kth = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = kth | (1u << b);
    int local = 0;
    for (int e = 0; e < E; ++e) local += key_e(e) >= cand;
    if (block_count(local) >= k) kth = cand;
  }
  int greater = 0;
  for (int e = 0; e < E; ++e) greater += key_e(e) > kth;
  const int need = k - block_count(greater);  // tied entries to keep, >= 1
  // largest J with #{ties with index < J} < need: J is the index of the last tie kept
  int J = 0;
  for (int b = 15; b >= 0; --b) {
    const int cand = J | (1 << b);
    int local = 0;
    for (int e = 0; e < E; ++e) {
      const int j = e * 256 + tid;
      local += candidate(j) && key_e(e) == kth && j < cand;
    }
    if (block_count(local) < need) J = cand;
  }
  int base = 0;
  for (int e = 0; e < E; ++e) {
    const int j = e * 256 + tid;
    const uint32_t key = key_e(e);
    const bool take = (candidate(j) && (key > kth || (key == kth && j <= J))) || (own && j == qi);
    const uint64_t m = __ballot(take);
    const int before = __popcll(m & ((1ull << lane) - 1ull));
    __syncthreads();
    if (lane == 0) part[wave] = __popcll(m);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wave; ++w) off += part[w];
    if (take) out[off + before] = j;
    base += part[0] + part[1] + part[2] + part[3];
  }
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)a.n_rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace s3r
