// Window token order: moves whole (token, head) rows between the caller's token order and the
// order in which contiguous blocks are spatial windows of each view's patch grid.
//
// Speed3R technical summary (gist.science), "Methodologie" section 1: the compression branch
// downsamples spatially by average pooling; README "Notice" 1: image sides are multiples of
// 56 pixels, i.e. patch grids in multiples of 4. Each view is `special` tokens followed by its
// row-major patch grid. In window order, every view's grid is listed window by window
// (windows row-major, patches row-major inside a window), and all views' special tokens
// follow at the end, so a run of win_h * win_w positions is one window.
//
// The copy is bound by HBM: one wave per token position, the position's source token
// computed once per wave (wave-uniform, so on the scalar unit), and the position's H rows of
// 128 bytes moved with 16-byte lane accesses.
#include "s3r_common.hpp"
#include "s3r_launch.hpp"

namespace s3r {

template <int kVecBytes>
struct Vec;
template <>
struct Vec<16> { typedef uint4 type; };
template <>
struct Vec<8> { typedef uint2 type; };

// kVecBytes: bytes one lane moves; kPerRow: lanes per (token, head) row.
template <int kVecBytes, int kPerRow>
__global__ __launch_bounds__(256) void window_permute_kernel(WindowCopyArgs a) {
  typedef typename Vec<kVecBytes>::type V;
  constexpr int kRowsPerPass = 64 / kPerRow;
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * 4;
  const int64_t first = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int part = lane % kPerRow;
  for (int64_t pos = first; pos < a.T; pos += waves) {
    const int64_t p = __builtin_amdgcn_readfirstlane((int)pos);  // T < 2^31
    const int64_t tok = window_source(a.w, p);
    const int64_t s_t = a.inverse ? p : tok;
    const int64_t d_t = a.inverse ? tok : p;
    const unsigned char* src = a.src + s_t * a.src_st;
    unsigned char* dst = a.dst + d_t * a.dst_st;
    for (int h = lane / kPerRow; h < a.H; h += kRowsPerPass) {
      const V x = reinterpret_cast<const V*>(src + h * a.src_sh)[part];
      reinterpret_cast<V*>(dst + h * a.dst_sh)[part] = x;
    }
  }
}

hipError_t launch_window_copy(const WindowCopyArgs& a, int row_bytes, hipStream_t s) {
  // enough waves to keep every CU streaming; each wave walks positions with a fixed stride
  const int64_t want = (a.T + 3) / 4;
  const unsigned grid = (unsigned)(want < 8192 ? want : 8192);
  if (row_bytes == 128) {
    hipLaunchKernelGGL((window_permute_kernel<16, 8>), dim3(grid), dim3(256), 0, s, a);
  } else if (row_bytes == 8) {
    hipLaunchKernelGGL((window_permute_kernel<8, 1>), dim3(grid), dim3(256), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace s3r
