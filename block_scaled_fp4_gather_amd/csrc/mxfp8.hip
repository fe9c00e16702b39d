// MXFP8 quantisation of bf16 activation rows (the W4A8-MX variant's input
// step).  Each thread takes 8 consecutive values (one 16-byte load); the 4
// threads of a 32-value block are consecutive lanes and share their maximum
// magnitude through two lane exchanges.
#include <hip/hip_runtime.h>

#include "mxfp8.h"

namespace moe {

__global__ void __launch_bounds__(256)
    mxfp8_quantize_rows(const uint16_t* __restrict__ x, int64_t items, int cols8, uint8_t* __restrict__ codes,
                        uint8_t* __restrict__ scales, int sstride) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // the loop bound is uniform per block of 4 lanes (items is a multiple of 4)
  for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < items; it += stride) {
    const int64_t row = it / cols8;
    const int c8 = (int)(it - row * cols8);
    const uint4 raw = *(const uint4*)(x + it * 8);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    float v[8];
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      amax = max(amax, (w[i] << 16) & 0x7FFFFFFFu);
      amax = max(amax, w[i] & 0x7FFF0000u);
    }
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
    const uint32_t sb = mx_scale_byte(amax);
    uint32_t lo = 0x7F7F7F7Fu, hi = 0x7F7F7F7Fu;
    if (sb != 255u) {
      const float inv = mx_inv_scale(sb);
      lo = hi = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo |= e4m3_code(v[i] * inv) << (8 * i);
        hi |= e4m3_code(v[4 + i] * inv) << (8 * i);
      }
    }
    *(uint2*)(codes + it * 8) = make_uint2(lo, hi);
    if ((c8 & 3) == 0) scales[row * sstride + c8 / 4] = (uint8_t)sb;
  }
}

}  // namespace moe

hipError_t launch_mxfp8_quantize(const uint16_t* x, int64_t rows, int cols, uint8_t* codes,
                                 uint8_t* scales, int sstride, hipStream_t st) {
  const int64_t items = rows * (cols / 8);
  if (items == 0) return hipSuccess;
  const int64_t blocks = (items + 255) / 256;
  const unsigned grid = (unsigned)(blocks < 4096 ? blocks : 4096);
  hipLaunchKernelGGL(moe::mxfp8_quantize_rows, dim3(grid), dim3(256), 0, st, x, items, cols / 8, codes,
                     scales, sstride);
  return hipGetLastError();
}
