// Weight preparation for the gfx950 kernels: a pure byte permutation of the
// logical FP4 tensors into the tiled resident layout (layout.h), its inverse,
// and a test-only dequantising export that reads the resident layout with the
// forward kernels' decode instructions.
#include <hip/hip_runtime.h>

#include "decode.h"
#include "decode_path.h"
#include "layout.h"

namespace moe {

// Items per expert: one per 16-byte code unit or 4-byte scale word of every
// lane of every tile.
struct PrepShape {
  int64_t per1;   // items of one FC1 tile: 64 * (nC1 + nQ1)
  int64_t per2;   // items of one FC2 tile: 64 * (nC2 + nQ2)
  int64_t fc1;    // items of all FC1 tiles of one expert
  int64_t expert; // items of one expert
};

static PrepShape prep_shape(const Layout& L) {
  PrepShape p;
  p.per1 = 64 * (int64_t)(L.nC1 + L.nQ1);
  p.per2 = 64 * (int64_t)(L.nC2 + L.nQ2);
  p.fc1 = p.per1 * L.nB1;
  p.expert = p.fc1 + p.per2 * L.nB2;
  return p;
}

// dir = 0: logical -> prepared.  dir = 1: prepared -> logical.
__global__ void __launch_bounds__(256) repack_kernel(Layout L, PrepShape P, int dir,
                                                     uint8_t* w13c, uint8_t* w13s, uint8_t* w2c,
                                                     uint8_t* w2s, uint8_t* prep) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= P.expert * L.E) return;
  const int e = (int)(idx / P.expert);
  int64_t rem = idx % P.expert;
  const bool fc1 = rem < P.fc1;
  if (!fc1) rem -= P.fc1;
  const int64_t per = fc1 ? P.per1 : P.per2;
  const int tile = (int)(rem / per);
  const int r2 = (int)(rem % per);
  const int nC = fc1 ? L.nC1 : L.nC2;
  const int lane = r2 % 64;
  const int slot = r2 / 64;  // chunk (< nC) or scale word (>= nC)
  const int cols = fc1 ? L.H : L.I;
  const int rows = fc1 ? 2 * L.Ip : L.H;
  const int row = fc1 ? fc1_row(L, tile, lane) : tile * 64 + lane;
  const int64_t toff = fc1 ? fc1_tile_offset(L, e, tile) : fc2_tile_offset(L, e, tile);
  const bool real = row < rows;
  if (slot < nC) {
    uint4* dst = (uint4*)(prep + toff + (int64_t)slot * 1024 + lane * 16);
    uint8_t* codes = fc1 ? w13c : w2c;
    uint4* src = (uint4*)(codes + ((int64_t)e * rows + row) * (cols / 2) + (int64_t)slot * 16);
    if (dir == 0)
      *dst = real ? *src : make_uint4(0, 0, 0, 0);
    else if (real)
      *src = *dst;
  } else {
    const int q = slot - nC;
    const int nsc = cols / L.G;  // scale bytes per logical row
    uint8_t* dst = prep + toff + (int64_t)nC * 1024 + (int64_t)q * 256 + lane * 4;
    uint8_t* scales = fc1 ? w13s : w2s;
    uint8_t* src = scales + ((int64_t)e * rows + row) * nsc;
    for (int j = 0; j < 4; ++j) {
      const int col = 4 * q + j;
      const bool ok = real && col < nsc;
      if (dir == 0)
        dst[j] = ok ? src[col] : (uint8_t)0;
      else if (ok)
        src[col] = dst[j];
    }
  }
}

// CSF blocks (layout.h): one thread per (expert, tile, lane) of every FC1 and
// FC2 tile.  The lane's logical row of scale bytes gives its base byte (the
// smallest byte, or 255 for an exception row: bytes spanning more than the
// offsets reach (1 MXFP4, 15 NVFP4), or a smallest byte of 255) and its
// offsets (0 for exception and padding rows), written as one word per group
// of chunks.
__global__ void __launch_bounds__(256) csf_kernel(Layout L, const uint8_t* __restrict__ w13s,
                                                  const uint8_t* __restrict__ w2s, uint8_t* __restrict__ prep) {
  const int64_t per_e = 64 * (int64_t)(L.nB1 + L.nB2);
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= per_e * L.E) return;
  const int e = (int)(idx / per_e);
  const int r = (int)(idx % per_e);
  const int tile = r / 64, lane = r % 64;
  const bool fc1 = tile < L.nB1;
  const int t = fc1 ? tile : tile - L.nB1;
  const int rows = fc1 ? 2 * L.Ip : L.H;
  const int row = fc1 ? fc1_row(L, t, lane) : t * 64 + lane;
  const int nC = fc1 ? L.nC1 : L.nC2;
  const int nsc = (fc1 ? L.H : L.I) / L.G;  // scale bytes per row
  uint8_t* blk = prep + (fc1 ? fc1_tile_offset(L, e, t) + csf_offset1(L) : fc2_tile_offset(L, e, t) + csf_offset2(L));
  const uint8_t* src = (fc1 ? w13s : w2s) + ((int64_t)e * rows + row) * nsc;
  const uint32_t reach = L.fmt == kMXFP4 ? 1u : 15u;
  uint32_t base = 0u;
  if (row < rows) {
    uint32_t lo = 255u, hi = 0u;
    for (int j = 0; j < nsc; ++j) {
      lo = src[j] < lo ? src[j] : lo;
      hi = src[j] > hi ? src[j] : hi;
    }
    base = (lo == 255u || hi - lo > reach) ? 255u : lo;
  }
  const bool packed = row < rows && base != 255u;
  const int cw = csf_chunks_per_word(L.fmt);
  for (int g = 0; g < (nC + cw - 1) / cw; ++g) {
    uint32_t w = base;
    for (int j = 0; j < cw && packed && cw * g + j < nC; ++j) {
      const int c = cw * g + j;
      if (L.fmt == kMXFP4)
        w |= ((uint32_t)src[c] - base) << (8 + j);
      else
        w |= (((uint32_t)src[2 * c] - base) | (((uint32_t)src[2 * c + 1] - base) << 4)) << (8 + 8 * j);
    }
    *(uint32_t*)(blk + 256 * g + 4 * lane) = w;
  }
}

// Globals header: words [0, E) = g13, [E, 2E) = g2, the rest zero padding.
__global__ void globals_kernel(int E, int words, int dir, float* g13, float* g2,
                               float* prep_globals) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= words) return;
  if (dir == 0) {
    prep_globals[i] = i < E ? g13[i] : (i < 2 * E ? g2[i - E] : 0.0f);
  } else if (i < E) {
    g13[i] = prep_globals[i];
  } else if (i < 2 * E) {
    g2[i - E] = prep_globals[i];
  }
}

// One thread per (row, 32-element chunk) of the requested logical matrix.
__global__ void __launch_bounds__(256) export_kernel(Layout L, int e, int which,
                                                     const uint8_t* __restrict__ prep,
                                                     float* __restrict__ out) {
  const bool fc1 = which == 0;
  const int rows = fc1 ? 2 * L.Ip : L.H;
  const int nC = fc1 ? L.nC1 : L.nC2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)rows * nC) return;
  const int row = (int)(idx / nC), c = (int)(idx % nC);
  int tile, lane;
  int64_t toff;
  if (fc1) {
    const bool up = row >= L.Ip;
    const int n = up ? row - L.Ip : row;
    tile = n / 32;
    lane = (up ? 32 : 0) + n % 32;
    toff = fc1_tile_offset(L, e, tile);
  } else {
    tile = row / 64;
    lane = row % 64;
    toff = fc2_tile_offset(L, e, tile);
  }
  const uint4 u = *(const uint4*)(prep + toff + (int64_t)c * 1024 + lane * 16);
  const uint32_t* sw = (const uint32_t*)(prep + toff + (int64_t)nC * 1024) + lane;
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  float v[32];
  if (fc1) {
    bf16x2_t p[16];
    for (int d = 0; d < 4; ++d) fp4x8_to_bf16(w[d], p + 4 * d);
    for (int i = 0; i < 16; ++i) {
      v[2 * i] = (float)p[i].x;
      v[2 * i + 1] = (float)p[i].y;
    }
  } else {
    f32x2_t p[16];
    for (int d = 0; d < 4; ++d) fp4x8_to_f32(w[d], p + 4 * d);
    for (int i = 0; i < 16; ++i) {
      v[2 * i] = p[i].x;
      v[2 * i + 1] = p[i].y;
    }
  }
  float s0, s1;
  const uint8_t* csf = L.csf ? prep + toff + (fc1 ? csf_offset1(L) : csf_offset2(L)) : nullptr;
  if (L.fmt == kMXFP4) {
    const uint32_t word = csf ? csf_scale_word<kMXFP4>(csf, lane, c, sw[64 * (c / 4)]) : sw[64 * (c / 4)];
    s0 = s1 = mx_scale(word, c);
  } else {
    const uint32_t word = csf ? csf_scale_word<kNVFP4>(csf, lane, c, sw[64 * (c / 2)]) : sw[64 * (c / 2)];
    const f32x2_t s = e4m3x2_to_f32(word, c & 1);
    s0 = s.x;
    s1 = s.y;
  }
  float g = 1.f;
  if (L.fmt == kNVFP4) g = ((const float*)prep)[(fc1 ? 0 : L.E) + e];
  float* o = out + (int64_t)row * (nC * 32) + c * 32;
  for (int i = 0; i < 32; ++i) {
    float d = v[i] * (i < 16 ? s0 : s1);
    if (L.fmt == kNVFP4) d = d * g;
    o[i] = d;
  }
}

hipError_t launch_repack(const Layout& L, int dir, uint8_t* w13c, uint8_t* w13s, uint8_t* w2c,
                         uint8_t* w2s, float* g13, float* g2, uint8_t* prep, hipStream_t st) {
  const PrepShape P = prep_shape(L);
  const int64_t n = P.expert * L.E;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(repack_kernel, dim3((unsigned)blocks), dim3(256), 0, st, L, P, dir, w13c, w13s,
                     w2c, w2s, prep);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (L.csf && dir == 0) {
    const int64_t m = 64 * (int64_t)(L.nB1 + L.nB2) * L.E;
    hipLaunchKernelGGL(csf_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st, L, w13s, w2s, prep);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (L.fmt == kNVFP4) {
    const int words = (int)(L.globals / 4);
    hipLaunchKernelGGL(globals_kernel, dim3((words + 255) / 256), dim3(256), 0, st, L.E, words, dir,
                       g13, g2, (float*)prep);
    err = hipGetLastError();
  }
  return err;
}

hipError_t launch_export(const Layout& L, int e, int which, const uint8_t* prep, float* out,
                         hipStream_t st) {
  const int rows = which == 0 ? 2 * L.Ip : L.H;
  const int nC = which == 0 ? L.nC1 : L.nC2;
  const int64_t n = (int64_t)rows * nC;
  hipLaunchKernelGGL(export_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, L, e, which,
                     prep, out);
  return hipGetLastError();
}

}  // namespace moe
