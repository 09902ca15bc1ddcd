// Exact softmax attention over packed key/value tiles: the selection branch (over the tokens
// of each query block's chosen key blocks, with the gated-aggregation epilogue) and the dense
// global attention it replaces.
//
// Speed3R technical summary (gist.science): "Methodologie" section 1 (the selection branch
// attends finely to the selected tokens only) and section 2 (a learned gate mixes the two
// branch outputs); "Probleemstelling" (dense global attention over all tokens is the
// quadratic cost being removed).
//
// Both kernels share one tile step: S^T = K . Q^T on v_mfma_f32_16x16x32_bf16 (lane l holds
// query l%16, keys 4*(l/16)+r), base-2 online softmax with a per-query offset shared by the
// four lanes that hold a query, and O^T += V^T . P^T in fp16 with P taken straight from the
// S^T registers. The offset only moves when a logit exceeds it by more than 15 (base 2), i.e.
// a weight exceeds 2^15, which happens on the first tile and rarely afterwards.
#include "s3r_common.hpp"
#include "s3r_launch.hpp"

namespace s3r {

// The offset of a query only moves once one of its weights exceeds 2^15 (15 in base 2 of
// headroom above the offset), so the fp16 weights of a tile stay at most 2^15 (fp16 holds up
// to 65504; the P.V and denominator products accumulate in f32). A selection row walks only
// a few dozen tiles, so every offset move (the weights of the tile computed again) is a
// sizeable share of the row; a generous headroom keeps them rare.
constexpr uint32_t kWeightLimitF32 = 0x47000000u;  // f32 bits of 2^15

template <int NT, bool kHalf = false>
struct Flash {
  float m[NT];          // per-query offset (base 2), identical in the 4 lanes of a query
  float nm[NT];         // -m, or 0 while m = -inf (weights then come out 0 or get rescaled)
  floatx4 l[NT];        // sum over keys of the fp16-rounded weights (all 4 entries equal)
  floatx4 o[4][NT];     // O^T accumulators: dims 16*mt + 4g + r, query 16*nt + l%16
  bool fresh;           // some query has no offset yet (before the first tile)

  __device__ void init() {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      m[nt] = -INFINITY;
      nm[nt] = 0.f;
      l[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) o[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    fresh = true;
  }

  // S^T = K . Q^T of one tile of 32 keys (unscaled logits); k = the tile's four K records
  // (this lane's 16 bytes of each).
  __device__ static void logits(const bf16x8* k, const bf16x8 (&qb)[NT][2], floatx4 (&acc)[2][NT]) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        floatx4 x = mfma_in<kHalf>(k[2 * s2], qb[nt][0], floatx4{0.f, 0.f, 0.f, 0.f});
        acc[s2][nt] = mfma_in<kHalf>(k[2 * s2 + 1], qb[nt][1], x);
      }
  }

  // fp16 weights exp2(logit * mult - m) of column tile nt, packed as its P.V operand; big is
  // set if one of them exceeds the headroom (weights are >= 0, so their f32 bit patterns order
  // like the numbers: an integer max, which needs no NaN handling)
  __device__ halfx8 weights(const floatx4 (&acc)[2][NT], int nt, float mult, bool& big) const {
    float p[2][4];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int r = 0; r < 4; ++r) p[s2][r] = fast_exp2(fmaf(acc[s2][nt][r], mult, nm[nt]));
    uint32_t b = __float_as_uint(p[0][0]);
#pragma unroll
    for (int e = 1; e < 8; ++e) b = max(b, __float_as_uint(p[e >> 2][e & 3]));
    big = b > kWeightLimitF32;
    return pack8h(p[0][0], p[0][1], p[0][2], p[0][3], p[1][0], p[1][1], p[1][2], p[1][3]);
  }

  // Moves the offset of the queries of column tile nt to their running maximum (rare: the
  // first tile, and when a logit exceeds the offset by more than the headroom) and rescales
  // their sums.
  __device__ void rescale(const floatx4 (&acc)[2][NT], int nt, float mult) {
    float M = acc[0][nt][0];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int r = 0; r < 4; ++r) M = fmaxf(M, acc[s2][nt][r]);
    M *= mult;
    M = fmaxf(M, __shfl_xor(M, 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    if (M > m[nt]) {
      const float f = (m[nt] == -INFINITY) ? 0.f : fast_exp2(m[nt] - M);
      l[nt] *= f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) o[mt][nt] *= f;
      m[nt] = M;
      nm[nt] = -M;
    }
  }

  // Online-softmax update with one tile: acc = its logits (masked here to keys [lo, hi) of the
  // tile), v = its four V^T records (fp16). The softmax denominator is a ones-row MFMA over the
  // same fp16 weights that multiply V, so numerator and denominator see identical rounding.
  __device__ void update(floatx4 (&acc)[2][NT], const bf16x8* v, int lo, int hi, float mult,
                         int g) {
    if (lo > 0 || hi < kTileKeys) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = 16 * s2 + 4 * g + r;
          if (key < lo || key >= hi) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[s2][nt][r] = -INFINITY;
          }
        }
    }
    const halfx8 ones = pack8h(1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f);
    // the weights of all column tiles first and one (rarely taken) branch for the tile, so
    // that the exps and the matrix products share one scheduling region; the column tiles
    // that need it are rescaled before their products, as if taken one at a time
    halfx8 pb[NT];
    bool big_any = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      bool big;
      pb[nt] = weights(acc, nt, mult, big);
      big_any |= big;
    }
    if (__builtin_expect(__any(big_any) || fresh, 0)) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        bool big;
        (void)weights(acc, nt, mult, big);
        if (__any(big) || fresh) {
          rescale(acc, nt, mult);
          pb[nt] = weights(acc, nt, mult, big);
        }
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        o[mt][nt] = mfma16h(__builtin_bit_cast(halfx8, v[mt]), pb[nt], o[mt][nt]);
      l[nt] = mfma16h(ones, pb[nt], l[nt]);
    }
    if (__builtin_expect(fresh, 0)) {
      bool unset = false;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) unset |= m[nt] == -INFINITY;
      fresh = __any(unset);
    }
  }

  // One tile: rec[0..3] = K records (bf16), rec[4..7] = V^T records (fp16).
  __device__ void step(const bf16x8 (&rec)[8], const bf16x8 (&qb)[NT][2], int lo, int hi,
                       float mult, int g) {
    floatx4 acc[2][NT];
    logits(rec, qb, acc);
    update(acc, rec + 4, lo, hi, mult, g);
  }

  // unscale / softmax denominator per query (unscale undoes the power of two the value
  // records were stored with), 0 for an empty softmax
  __device__ void finish(float (&inv)[NT], float unscale) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) inv[nt] = (l[nt][0] > 0.f) ? unscale / l[nt][0] : 0.f;
  }
};

template <int NT>
__device__ __forceinline__ void load_q(const AttnArgs& a, int h, int64_t q0, int g, int li,
                                       bf16x8 (&qb)[NT][2]) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int64_t t = q0 + 16 * nt + li;
#pragma unroll
    for (int c = 0; c < 2; ++c)
      qb[nt][c] = (t < a.T) ? *reinterpret_cast<const bf16x8*>(a.q + t * a.q_st +
                                                               (int64_t)h * a.q_sh + 32 * c + 8 * g)
                            : bf16x8{};
  }
}

// ---------------------------------------------------------------------------------------
// Selection branch. One wave per (head, query block) (two waves for B = 128, 64 queries
// each). The wave walks the tiles of its selected blocks in list order. The tiles are
// gathered from all over the key sequence, so each costs a full memory latency: the wave
// keeps two tiles in flight, copied from global memory straight into two LDS slots of its own
// (no registers held while in flight), and computes on a third, read from its slot into
// registers just before the slot is refilled. Rows of at most 64 entries and 128 tile steps
// (kPre) get their step schedule built once at the start, one step per lane, and each step
// reads its tile with readlane; longer rows are walked block by block (SelIter).
// ---------------------------------------------------------------------------------------
// Walks a selection row block by block and tile by tile. The row is held 64 entries at a time
// in one register (lane l: entry base + l) and read with readlane, so that walking it issues
// no memory access (a vector load inside the tile loop would make the compiler wait for every
// tile copy in flight); only rows longer than 64 entries reload it, once per 64 entries.
struct SelIter {
  int idx;          // position in the selection row
  int base;         // first entry held in chunk
  int32_t chunk;    // lane l: row[base + l] (-1 past the end)
  int64_t prev;     // last block taken
  int64_t tile, tile_end;
  int64_t blk_lo, blk_hi;  // token range of the current block
};

__device__ __forceinline__ int32_t sel_chunk(const AttnArgs& a, const int32_t* row, int base,
                                             int lane) {
  return (base + lane < a.k_eff) ? row[base + lane] : -1;
}

__device__ __forceinline__ bool sel_next_block(const AttnArgs& a, const int32_t* row, int lane,
                                               SelIter& it) {
  while (it.idx < a.k_eff) {
    if (it.idx >= it.base + 64) {
      it.base += 64;
      it.chunk = sel_chunk(a, row, it.base, lane);
      wait_vmem<0>();  // here, so that the common path below carries no pending load
    }
    const int64_t j = __builtin_amdgcn_readlane(it.chunk, it.idx - it.base);
    ++it.idx;
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

__device__ __forceinline__ bool sel_advance(const AttnArgs& a, const int32_t* row, int lane,
                                            SelIter& it) {
  if (it.tile + 1 < it.tile_end) {
    ++it.tile;
    return true;
  }
  return sel_next_block(a, row, lane, it);
}

constexpr int kSelSlots = 2;  // tiles in flight per wave (the vmcnt waits below assume 2)

template <int NT, bool kHalf, bool kPre = false>
__global__ __launch_bounds__(256) void sel_kernel(AttnArgs a) {
  __shared__ uint4 ring[4][kSelSlots][kRawTileBytes / 16];  // 16 KB per wave
  // wave-uniform as far as the compiler can see: the LDS copy destinations (M0), the item and
  // the row walk then live in scalar registers
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 4, li = lane & 15;
  const int parts = (a.B > 64) ? a.B / 64 : 1;
  const int64_t n_items = (int64_t)a.H * a.Nb * parts;
  const int64_t n_wg = (n_items + 3) / 4;
  const int64_t wg = xcd_logical_id(blockIdx.x, n_wg);
  const int64_t item = wg * 4 + wave;
  if (wg >= n_wg || item >= n_items) return;
  const int part = (int)(item % parts);
  const int64_t hi_ = item / parts;
  const int h = (int)(hi_ / a.Nb);
  const int64_t i = hi_ % a.Nb;
  const int64_t q0 = i * a.B + 64 * part;

  bf16x8 qb[NT][2];
  load_q<NT>(a, h, q0, g, li, qb);
  const int32_t* row = a.sel + ((int64_t)h * a.Nb + i) * a.k_eff;
  const unsigned char* tiles = a.tiles + (int64_t)h * a.n_tiles * kRawTileBytes;

  // O_cmp of this wave's queries for the gated epilogue, copied into the wave's (then idle)
  // LDS slots while the last tile is computed: copy x = nt*4 + mt, lane li + 16g fetches query
  // 16nt + li, dims 16mt + 4g..+3, so the epilogue's read of (nt, mt) is one contiguous,
  // conflict-free 1 KB record. Rows past the end read the last row (not used).
  uint4* const cmp_lds = ring[wave][0];
  auto fetch_ocmp = [&](int64_t first) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      int64_t t = first + 16 * nt + li;
      t = t < a.T ? t : a.T - 1;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        copy16_to_lds(a.o_cmp + (t * a.H + h) * kD + 16 * mt + 4 * g, cmp_lds + 64 * (nt * 4 + mt));
    }
  };
  static_assert(NT * 4 * 1024 <= kSelSlots * kRawTileBytes, "O_cmp fits the wave's slots");

  Flash<NT, kHalf> f;
  f.init();
  if constexpr (kPre) {
    // The row's step schedule, built once (rows of at most 64 entries and 128 tile steps):
    // lane e holds entry e, which counts if its block is valid and differs from the last
    // valid entry before it (the walk's rule: a block repeated right away counts once); its
    // tiles become steps incl - c .. incl - 1, scattered through this wave's second slot
    // (no copy has been issued yet) and read back two steps per lane, s and s + 64.
    const int nb = (int)a.Nb, tt = (int)a.T;
    const int j = (lane < a.k_eff) ? row[lane] : -1;
    const bool valid = (unsigned)j < (unsigned)nb;
    const uint64_t below = __ballot(valid) & ((1ull << lane) - 1);
    const int pl = below ? 63 - __builtin_clzll(below) : lane;
    const int jp = __shfl(j, pl);
    const bool taken = valid && (pl == lane || jp != j);
    const int lo = valid ? j * a.B : 0;
    const int hi = (lo + a.B < tt) ? lo + a.B : tt;
    const int ts = lo / kTileKeys;
    const int c = taken ? (hi - 1) / kTileKeys + 1 - ts : 0;
    const int incl = wave_inclusive_sum(c, lane);
    const int n = __builtin_amdgcn_readlane(incl, 63);
    uint2* sc = reinterpret_cast<uint2*>(ring[wave][1]);
#pragma unroll
    for (int x = 0; x < 128 / kTileKeys; ++x) {  // (B <= 128: at most 4 tiles per block)
      if (x < c) {
        const int t0 = (ts + x) * kTileKeys;
        const int rl = (lo > t0) ? lo - t0 : 0;
        const int rh = (hi < t0 + kTileKeys) ? hi - t0 : kTileKeys;
        sc[incl - c + x] = make_uint2((uint32_t)(ts + x), (uint32_t)(rl | (rh << 8)));
      }
    }
    const uint2 m0 = sc[lane], m1 = sc[64 + lane];
    const int s_tile0 = (int)m0.x, s_range0 = (int)m0.y;
    const int s_tile1 = (int)m1.x, s_range1 = (int)m1.y;
    wait_lds();  // both reads are done before tile 1 is copied over the scratch
    auto tile_of = [&](int t) {
      return t < 64 ? __builtin_amdgcn_readlane(s_tile0, t)
                    : __builtin_amdgcn_readlane(s_tile1, t - 64);
    };
    if (n > 0) tile_to_lds(tiles + (int64_t)tile_of(0) * kRawTileBytes, ring[wave][0], lane);
    if (n > 1) tile_to_lds(tiles + (int64_t)tile_of(1) * kRawTileBytes, ring[wave][1], lane);
    if (n == 0) fetch_ocmp(q0);
    for (int t = 0; t < n; ++t) {
      const int slot = t & 1;
      // tile t has landed once at most tile t + 1's copies are pending
      if (t + 1 < n) wait_vmem<8>();
      else wait_vmem<0>();
      // (after the explicit wait above the compiler orders these reads behind nothing else)
      bf16x8 cur[8];
      const bf16x8* L = reinterpret_cast<const bf16x8*>(ring[wave][slot]);
#pragma unroll
      for (int x = 0; x < 8; ++x) cur[x] = L[x * 64 + lane];
      if (t + 2 < n) {
        wait_lds();  // the slot is read before the next tile overwrites it
        tile_to_lds(tiles + (int64_t)tile_of(t + 2) * kRawTileBytes, ring[wave][slot], lane);
      } else if (t + 1 == n) {
        int64_t qq = q0;
        asm volatile("" : "+s"(qq));
        fetch_ocmp(qq);  // last tile: both slots are free once it is read
      }
      const int range = t < 64 ? __builtin_amdgcn_readlane(s_range0, t)
                               : __builtin_amdgcn_readlane(s_range1, t - 64);
      f.step(cur, qb, range & 0xFF, range >> 8, a.logit_mult, g);
    }
  } else {
  // cons: the tile being computed; prod: the next tile to request (kSelSlots ahead)
  SelIter cons{0, 0, sel_chunk(a, row, 0, lane), -1, 0, 0, 0, 0};
  bool cvalid = sel_next_block(a, row, lane, cons);
  SelIter prod = cons;
  bool pvalid = cvalid;
  int issued = 0;
#pragma unroll
  for (int s = 0; s < kSelSlots; ++s) {
    if (pvalid) {
      tile_to_lds(tiles + prod.tile * kRawTileBytes, ring[wave][s], lane);
      ++issued;
      pvalid = sel_advance(a, row, lane, prod);
    }
  }
  if (!cvalid) fetch_ocmp(q0);
  for (int t = 0; cvalid; ++t) {
    const int slot = t % kSelSlots;
    // tile t has landed once at most the copies issued after it are pending
    if (issued > t + 1) wait_vmem<8>();
    else wait_vmem<0>();
    bf16x8 cur[8];
    const bf16x8* L = reinterpret_cast<const bf16x8*>(ring[wave][slot]);
#pragma unroll
    for (int x = 0; x < 8; ++x) cur[x] = L[x * 64 + lane];
    SelIter nx = cons;
    const bool nvalid = sel_advance(a, row, lane, nx);
    if (pvalid) {
      wait_lds();  // the slot is read before the next tile overwrites it
      tile_to_lds(tiles + prod.tile * kRawTileBytes, ring[wave][slot], lane);
      ++issued;
      pvalid = sel_advance(a, row, lane, prod);
    } else if (!nvalid) {
      wait_lds();  // last tile: both slots are free once it is read
      // (the opaque copy of q0 keeps the compiler from hoisting the copy's 16 addresses out
      // of the loop, where they would hold registers for the whole loop)
      int64_t qq = q0;
      asm volatile("" : "+s"(qq));
      fetch_ocmp(qq);
    }
    const int64_t t0 = cons.tile * kTileKeys;
    const int lo = (int)((cons.blk_lo > t0) ? cons.blk_lo - t0 : 0);
    const int hi = (int)((cons.blk_hi < t0 + kTileKeys) ? cons.blk_hi - t0 : kTileKeys);
    f.step(cur, qb, lo, hi, a.logit_mult, g);
    cons = nx;
    cvalid = nvalid;
  }
  }
  wait_vmem<0>();  // O_cmp has landed

  float inv[NT];
  f.finish(inv, a.v_unscale);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int64_t t = q0 + 16 * nt + li;
    if (t >= a.T || 16 * nt + li + 64 * part >= a.B) continue;
    if (a.lse_sel && g == 0)  // saved for the backward pass
      a.lse_sel[(int64_t)h * a.T + t] =
          (f.l[nt][0] > 0.f) ? f.m[nt] + __log2f(f.l[nt][0]) : INFINITY;
    const float* gp = a.gates + t * a.gate_st + (int64_t)h * 2;
    const float g_cmp = gp[0], g_sel = gp[1];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int64_t base = (t * a.H + h) * kD + 16 * mt + 4 * g;
      const float4 oc = __builtin_bit_cast(float4, cmp_lds[64 * (nt * 4 + mt) + lane]);
      const float s0 = f.o[mt][nt][0] * inv[nt], s1 = f.o[mt][nt][1] * inv[nt];
      const float s2 = f.o[mt][nt][2] * inv[nt], s3 = f.o[mt][nt][3] * inv[nt];
      if (a.o_sel) *reinterpret_cast<float4*>(a.o_sel + base) = make_float4(s0, s1, s2, s3);
      uint2 w;
      w.x = float_to_in<kHalf>(g_cmp * oc.x + g_sel * s0) |
            ((uint32_t)float_to_in<kHalf>(g_cmp * oc.y + g_sel * s1) << 16);
      w.y = float_to_in<kHalf>(g_cmp * oc.z + g_sel * s2) |
            ((uint32_t)float_to_in<kHalf>(g_cmp * oc.w + g_sel * s3) << 16);
      *reinterpret_cast<uint2*>(a.out + base) = w;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Dense attention. A work-group of 4 waves owns 256 queries of one head and streams every
// raw tile of that head through a double-buffered LDS ring (8 KB per tile).
// ---------------------------------------------------------------------------------------
template <bool kHalf>
__global__ __launch_bounds__(256) void dense_kernel(AttnArgs a) {
  constexpr int kTileU4 = kRawTileBytes / 16;  // 512
  __shared__ uint4 lds[2][kTileU4];
  const int64_t n_qtiles = (a.T + 255) / 256;
  const int64_t total = (int64_t)a.H * n_qtiles;
  const int64_t logical = xcd_logical_id(blockIdx.x, total);
  if (logical >= total) return;
  const int h = (int)(logical / n_qtiles);
  const int64_t qt = logical % n_qtiles;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, li = lane & 15;
  const int64_t q0 = qt * 256 + wave * 64;

  bf16x8 qb[4][2];
  load_q<4>(a, h, q0, g, li, qb);
  const uint4* tiles = reinterpret_cast<const uint4*>(a.tiles) + (int64_t)h * a.n_tiles * kTileU4;

  Flash<4, kHalf> f;
  f.init();
  uint4 s0 = tiles[tid], s1 = tiles[256 + tid];
  lds[0][tid] = s0;
  lds[0][256 + tid] = s1;
  __syncthreads();
  for (int64_t tau = 0; tau < a.n_tiles; ++tau) {
    const int buf = (int)(tau & 1);
    {
      // prefetch the next tile (the last iteration re-reads its own tile; nobody consumes it)
      const int64_t nxt = (tau + 1 < a.n_tiles) ? tau + 1 : tau;
      s0 = tiles[nxt * kTileU4 + tid];
      s1 = tiles[nxt * kTileU4 + 256 + tid];
    }
    bf16x8 rec[8];
    const bf16x8* L = reinterpret_cast<const bf16x8*>(lds[buf]);
#pragma unroll
    for (int x = 0; x < 8; ++x) rec[x] = L[x * 64 + lane];
    const int64_t t0 = tau * kTileKeys;
    const int hi = (int)((a.T - t0 < kTileKeys) ? a.T - t0 : kTileKeys);
    f.step(rec, qb, 0, hi, a.logit_mult, g);
    lds[buf ^ 1][tid] = s0;
    lds[buf ^ 1][256 + tid] = s1;
    __syncthreads();
  }
  float inv[4];
  f.finish(inv, a.v_unscale);
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int64_t t = q0 + 16 * nt + li;
    if (t >= a.T) continue;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int64_t base = (t * a.H + h) * kD + 16 * mt + 4 * g;
      uint2 w;
      w.x = float_to_in<kHalf>(f.o[mt][nt][0] * inv[nt]) |
            ((uint32_t)float_to_in<kHalf>(f.o[mt][nt][1] * inv[nt]) << 16);
      w.y = float_to_in<kHalf>(f.o[mt][nt][2] * inv[nt]) |
            ((uint32_t)float_to_in<kHalf>(f.o[mt][nt][3] * inv[nt]) << 16);
      *reinterpret_cast<uint2*>(a.out + base) = w;
    }
  }
}

hipError_t launch_sel(const AttnArgs& a, hipStream_t s) {
  const int parts = (a.B > 64) ? a.B / 64 : 1;
  const int64_t n_items = (int64_t)a.H * a.Nb * parts;
  const int64_t n_wg = (n_items + 3) / 4;
  const dim3 g3((unsigned)(((n_wg + 7) / 8) * 8)), b3(256);
  // the step schedule in registers: rows of at most 64 entries and 128 tile steps, token
  // indices below 2^31
  const int tiles_per_block = a.B > kTileKeys ? a.B / kTileKeys : 1;
  const bool pre = a.k_eff <= 64 && (int64_t)a.k_eff * tiles_per_block <= 128 &&
                   a.T + a.B < ((int64_t)1 << 31);
#define S3R_SEL(NT)                                                                        \
  do {                                                                                      \
    if (pre) {                                                                              \
      if (a.half) hipLaunchKernelGGL((sel_kernel<NT, true, true>), g3, b3, 0, s, a);        \
      else hipLaunchKernelGGL((sel_kernel<NT, false, true>), g3, b3, 0, s, a);              \
    } else {                                                                                \
      if (a.half) hipLaunchKernelGGL((sel_kernel<NT, true, false>), g3, b3, 0, s, a);       \
      else hipLaunchKernelGGL((sel_kernel<NT, false, false>), g3, b3, 0, s, a);             \
    }                                                                                       \
  } while (0)
  switch (a.B) {
    case 16: S3R_SEL(1); break;
    case 32: S3R_SEL(2); break;
    default: S3R_SEL(4); break;
  }
#undef S3R_SEL
  return hipGetLastError();
}

hipError_t launch_dense(const AttnArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.H * ((a.T + 255) / 256);
  const dim3 g3((unsigned)(((total + 7) / 8) * 8)), b3(256);
  if (a.half) hipLaunchKernelGGL((dense_kernel<true>), g3, b3, 0, s, a);
  else hipLaunchKernelGGL((dense_kernel<false>), g3, b3, 0, s, a);
  return hipGetLastError();
}

__global__ void fill_zero_kernel(float* p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0.f;
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace s3r
