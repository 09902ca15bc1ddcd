// Shared device-side definitions of the gfx950 kernels: MFMA operand types, the packed tile
// layouts, DPP helpers and launch geometry. Private to the library (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace s3r {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

constexpr int kD = 64;           // head width
constexpr int kTileKeys = 32;    // keys per packed tile
constexpr int kRecBytes = 1024;  // one MFMA A-operand record: 64 lanes x 16 bytes
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------------------
// Packed tile layouts. Every tile covers 32 consecutive keys of one head and is stored as a
// sequence of 1 KB records, each the exact register image of one A operand of
// v_mfma_f32_16x16x32_bf16 (lane l holds row l%16, k-slots 8*(l/16)..+7), so a wave loads
// an operand with one linear 16-byte read per lane.
//
//  K record (s, c), s = key half (0/1), c = dim chunk (0/1):
//      lane l -> key 16*s + l%16, dims 32*c + 8*(l/16) + 0..7.           record index 2*s + c
//  V^T record mt = 0..3 (16 output dims each):
//      lane l -> dim 16*mt + l%16, slot e -> key vkey(l/16, e)           record index mt
//      vkey(g, e) = e < 4 ? 4g + e : 16 + 4g + (e - 4).
//  The S^T accumulator of keys 16*s..+15 x 16 queries puts key 16*s + 4g + r in lane group
//  g = l/16, register r; the P operand of P.V therefore takes slot e < 4 from half 0 and
//  slot e >= 4 from half 1, which is exactly vkey.
//
//  Pooled tiles (compression branch): [K hi: 4 records][K lo: 4 records][V^T: 4 records].
//  Raw tiles (selection and dense):   [K: 4 records][V^T: 4 records].
//  K records hold bf16 (the logits Q.K are exact products of bf16 inputs); V^T records hold
//  fp16, because the P.V product takes both operands in fp16: the attention weights P lie in
//  [0, 2^8] and fp16 rounds them 8x finer than bf16 at the same MFMA rate, and bf16 values of
//  magnitude below 65504 convert to fp16 exactly (subnormal-range values to within 2^-25).
// ---------------------------------------------------------------------------------------
constexpr int kPooledTileBytes = 12 * kRecBytes;
constexpr int kRawTileBytes = 8 * kRecBytes;

__device__ __forceinline__ int vkey(int g, int e) { return e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4); }

// (key m within the tile, dim d) -> (record, lane, slot) of the V^T records
__device__ __forceinline__ void vt_position(int m, int d, int& rec, int& lane, int& slot) {
  const int half = m >> 4, w = m & 15;
  const int g = w >> 2, e = (w & 3) + 4 * half;
  rec = d >> 4;
  lane = (d & 15) + 16 * g;
  slot = e;
}

// (key m, dim group d8 of 8 dims) -> byte offset of the 16-byte chunk in the K records
__device__ __forceinline__ int k_chunk_offset(int m, int d8) {
  const int s = m >> 4, c = d8 >> 2;
  const int lane = (m & 15) + 16 * (d8 & 3);
  return ((2 * s + c) * 64 + lane) * 16;
}

__device__ __forceinline__ floatx4 mfma16(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mfma16h(const halfx8& a, const halfx8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Element type of the caller's q, k, v (and of the output): bf16 (kHalf = false) or fp16.
// Operands stay 16-byte bit patterns; the matrix product picks the instruction.
template <bool kHalf>
__device__ __forceinline__ floatx4 mfma_in(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  if constexpr (kHalf) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8, a),
                                                  __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
}

template <bool kHalf>
__device__ __forceinline__ float in_to_float(uint32_t bits16) {
  if constexpr (kHalf) {
    return (float)__builtin_bit_cast(_Float16, (u16)bits16);
  } else {
    return __builtin_bit_cast(float, bits16 << 16);
  }
}

// round to nearest even
template <bool kHalf>
__device__ __forceinline__ u16 float_to_in(float x) {
  if constexpr (kHalf) {
    return __builtin_bit_cast(u16, (_Float16)x);
  } else {
    return __builtin_bit_cast(u16, (__bf16)x);
  }
}

// the 8 elements of a 16-byte chunk
template <bool kHalf>
__device__ __forceinline__ void unpack8(const uint4& w, float (&x)[8]) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = in_to_float<kHalf>(ws[e] & 0xFFFFu);
    x[2 * e + 1] = in_to_float<kHalf>(ws[e] >> 16);
  }
}

__device__ __forceinline__ u16 bf16_bits(float x) {
  __bf16 b = (__bf16)x;  // round to nearest even
  return __builtin_bit_cast(u16, b);
}
__device__ __forceinline__ float bf16_to_float(u16 b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

__device__ __forceinline__ u16 f16_bits(float x) {
  _Float16 b = (_Float16)x;  // round to nearest even
  return __builtin_bit_cast(u16, b);
}

__device__ __forceinline__ halfx8 pack8h(float a0, float a1, float a2, float a3, float a4,
                                         float a5, float a6, float a7) {
  halfx8 r;
  r[0] = (_Float16)a0; r[1] = (_Float16)a1; r[2] = (_Float16)a2; r[3] = (_Float16)a3;
  r[4] = (_Float16)a4; r[5] = (_Float16)a5; r[6] = (_Float16)a6; r[7] = (_Float16)a7;
  return r;
}

__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4, float a5,
                                        float a6, float a7) {
  bf16x8 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
  return r;
}

// ---------------------------------------------------------------------------------------
// DPP lane exchanges (gfx9 encodings). All but the wave shift stay inside a row of 16 lanes.
// ---------------------------------------------------------------------------------------
enum : int {
  kDppXor1 = 0xB1,        // quad_perm [1,0,3,2]
  kDppXor2 = 0x4E,        // quad_perm [2,3,0,1]
  kDppRor8 = 0x128,       // row_ror:8  (lane i <- i^8 inside a 16-lane row)
  kDppHalfMirror = 0x141, // row_half_mirror (lane i <- 7-i inside each 8-lane half)
  kDppWaveShr1 = 0x138,   // wave_shr:1 (lane i <- lane i-1 across the whole wave)
};

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, false));
}

// Sum over the 16 lanes of each DPP row of 8 values per lane, v[s][r] (key 16s + 4g + r of
// lane group g). Returns the total for key 16*bit3 + 4g + 2*bit2 + bit0 of the lane index
// inside the row; lanes i and i^2 hold the same key.
__device__ __forceinline__ float row_reduce_scatter8(const float (&v)[2][4], int lane) {
  const bool b3 = lane & 8, b2 = lane & 4, b0 = lane & 1;
  float a[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float keep = b3 ? v[1][r] : v[0][r];
    const float send = b3 ? v[0][r] : v[1][r];
    a[r] = keep + dpp<kDppRor8>(send);
  }
  float b[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const float keep = b2 ? a[2 + x] : a[x];
    const float send = b2 ? a[x] : a[2 + x];
    b[x] = keep + dpp<kDppHalfMirror>(send);
  }
  const float keep = b0 ? b[1] : b[0];
  const float send = b0 ? b[0] : b[1];
  const float c = keep + dpp<kDppXor1>(send);
  return c + dpp<kDppXor2>(c);
}

// row_reduce_scatter8 on fp16 values packed as pack8h packs them (element e: v[e/4][e%4]):
// the first two halvings add packed pairs, the last two run in f32. Each fp16 addition rounds
// to 2^-11 relative (2^-25 absolute below 2^-14).
__device__ __forceinline__ float row_reduce_scatter8_h(const halfx8& v, int lane) {
  typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));
  const bool b3 = lane & 8, b2 = lane & 4, b0 = lane & 1;
  auto word = [&](int i) { return __builtin_bit_cast(uint32_t, halfx2{v[2 * i], v[2 * i + 1]}); };
  auto dpp_u = [](uint32_t x, auto ctrl) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, decltype(ctrl)::value, 0xF, 0xF, false);
  };
  auto add = [](uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(halfx2, a) + __builtin_bit_cast(halfx2, b));
  };
  uint32_t a[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const uint32_t keep = b3 ? word(2 + x) : word(x);
    const uint32_t send = b3 ? word(x) : word(2 + x);
    a[x] = add(keep, dpp_u(send, std::integral_constant<int, kDppRor8>{}));
  }
  const uint32_t keep = b2 ? a[1] : a[0];
  const uint32_t send = b2 ? a[0] : a[1];
  const halfx2 b = __builtin_bit_cast(halfx2, add(keep, dpp_u(send, std::integral_constant<int, kDppHalfMirror>{})));
  const float lo = (float)b[0], hi = (float)b[1];
  const float k0 = b0 ? hi : lo;
  const float s0 = b0 ? lo : hi;
  const float c = k0 + dpp<kDppXor1>(s0);
  return c + dpp<kDppXor2>(c);
}

__device__ __forceinline__ int reduced_key(int lane) {
  const int i = lane & 15, g = lane >> 4;
  return 16 * ((i >> 3) & 1) + 4 * g + 2 * ((i >> 2) & 1) + (i & 1);
}

// Work-group barrier that orders LDS only: waits for this wave's LDS operations, not for its
// global loads, so a prefetch for a later step stays in flight across it (__syncthreads
// waits for every outstanding memory operation).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Waits on one counter of this wave (s_waitcnt, gfx9 field layout: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4, lgkmcnt 11:8; a field at its maximum does not wait). The empty asm keeps
// the compiler from moving memory accesses across the wait.
template <int N>
__device__ __forceinline__ void wait_vmem() {  // at most N vector-memory operations pending
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_lds() {  // every LDS (and scalar-memory) operation done
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
  asm volatile("" ::: "memory");
}

// inclusive prefix sum over the lanes of a wave
__device__ __forceinline__ int wave_inclusive_sum(int x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

// LDS byte address of a __shared__ object (for inline asm)
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct global->LDS copy of 16 bytes per lane: lane l's 16 bytes at src land at dst + 16 l
// (dst the same for every lane of the wave). Counts on vmcnt like a load. (Kept out of line of
// kernel templates: there the host pass of hipcc rejects the builtin and silently drops the
// kernel's launch stub.)
__device__ __forceinline__ void copy16_to_lds(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// One packed tile (8 records of 1 KB) copied from global memory straight into LDS, without
// passing through registers: record x of lane l (16 bytes) lands at dst[64 x + l]. dst must
// be the same for every lane of the wave. Completion counts on vmcnt, 8 operations per tile;
// the data may be read only after wait_vmem() has covered them.
__device__ __forceinline__ void tile_to_lds(const unsigned char* src, uint4* dst, int lane) {
#pragma unroll
  for (int x = 0; x < kRawTileBytes / kRecBytes; ++x)
    copy16_to_lds(src + x * kRecBytes + 16 * lane, dst + 64 * x);
}

// Work-group id remapped so that consecutive logical ids share an XCD: the dispatcher hands
// work-groups to the 8 XCDs round-robin, so logical id x*per + s runs on XCD x.
__device__ __forceinline__ int64_t xcd_logical_id(int64_t b, int64_t total) {
  const int64_t per = (total + 7) / 8;
  return (b % 8) * per + b / 8;
}

}  // namespace s3r
