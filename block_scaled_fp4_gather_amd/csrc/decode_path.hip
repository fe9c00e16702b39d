// Decode-band forward (few tokens): two launches, FC1 then FC2.
//
// Prior art is the two-launch tiny-decode kernel of b12x PR #22 ("rp-native
// tiny-decode kernel for w4a8_mx (M=1)", What section): gate+up dot products
// into an fp32 intermediate, then FC2 with inline SiLU and a router-weighted
// epilogue into the bf16 output, and no grid barrier (its Notes section records
// the grid-barrier variant deadlocking).
//
// On gfx950 the lanes of a wave own rows instead of K-slices: every lane reads
// the same 32-element K chunk of its own row, so the activation chunk is
// wave-uniform and arrives through scalar loads into SGPRs, each wave load of
// codes is one contiguous KiB of the resident layout, and no cross-lane
// reduction is needed.  All cross-wave sums stay inside a workgroup, in LDS
// and in a fixed order: no workgroup ever waits for or signals another one,
// and results are bit-reproducible.
//   FC1: one workgroup per (route slot, 64-row tile); its waves split K into
//        slabs; the slab sums meet in LDS, then SiLU(gate)*up is written to
//        the workspace activation.
//   FC2: one workgroup per 64-row tile of H; its waves split the route slots
//        (experts); the weighted expert sums meet in LDS and are written to the
//        output as bf16, overwriting it.
// Experts are streamed once per call however many tokens route to them: a
// slot works only if its id is valid and no earlier slot holds the same id
// (b12x PR #22, Notes: re-reading weights per routed row is what limited the
// prior kernel to M=1).  Invalid ids read nothing and add nothing (b12x PR
// #311: commit message on invalid routes and the tiny_decode.py review).
#include <hip/hip_runtime.h>

#include "decode.h"
#include "decode_path.h"
#include "layout.h"

namespace moe {

// The route table as one wave sees it: lane l holds slot l (token l / k,
// route l % k).  rid is the expert id, or -1 for an invalid id or a lane past
// the last slot.
struct Routes {
  int rid;
  float w;
};

template <typename IdT>
__device__ __forceinline__ Routes load_routes(const IdT* __restrict__ ids,
                                              const float* __restrict__ tw, int slots, int E) {
  const int l = threadIdx.x & 63;
  Routes r{-1, 0.0f};
  if (l < slots) {
    const int64_t v = (int64_t)ids[l];
    r.rid = (v >= 0 && v < E) ? (int)v : -1;
    if (tw) r.w = tw[l];
  }
  return r;
}

// Expert of slot s when s is the first slot that holds it (else -1), and the
// mask of all slots that hold it.
__device__ __forceinline__ int slot_expert(const Routes& R, int s, uint64_t* mask) {
  const int e = __builtin_amdgcn_readlane(R.rid, s);
  if (e < 0) return -1;
  const uint64_t m = __ballot(R.rid == e);
  if (m & ((1ull << s) - 1ull)) return -1;
  *mask = m;
  return e;
}

__device__ __forceinline__ uint64_t token_routes(uint64_t mask, int t, int k) {
  const uint64_t kmask = k >= 64 ? ~0ull : ((1ull << k) - 1ull);
  return (mask >> (t * k)) & kmask;
}

// SiLU(gate)*up across the lane pair (l, l+32) of an FC1 tile.  The fp32
// activation a is stored as two bf16 planes, a = hi + lo (hi = bf16(a),
// lo = bf16(a - hi)), which keeps 16 significant bits for FC2's bf16 dot
// products.
__device__ __forceinline__ void fc1_finish(float v, float g13, int lane, int b, int r,
                                           const Layout& L, uint16_t* __restrict__ act_hi,
                                           uint16_t* __restrict__ act_lo) {
  v *= g13;
  const float up = __shfl(v, (lane + 32) & 63);
  if (lane < 32) {
    const float a = v / (1.0f + __expf(-v)) * up;
    const uint16_t hi = f32_to_bf16_rne(a);
    const float rest = a - __uint_as_float((uint32_t)hi << 16);
    const int64_t at = (int64_t)r * L.I + 32 * b + lane;
    act_hi[at] = hi;
    act_lo[at] = f32_to_bf16_rne(rest);
  }
}

template <int FMT, int CS, typename IdT>
__global__ void __launch_bounds__(1024)
    fc1_kernel(const uint8_t* __restrict__ prep, const Layout L, const uint16_t* __restrict__ x,
               const IdT* __restrict__ ids, const int M, const int k,
               uint16_t* __restrict__ act_hi, uint16_t* __restrict__ act_lo) {
  constexpr int SPD = FMT == kMXFP4 ? 4 : 2;  // chunks per scale dword
  constexpr int ND = CS / SPD;
  extern __shared__ float part[];  // [token index][wave][lane]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int W = blockDim.x >> 6;
  const int b = blockIdx.x % L.nB1;
  const int s = blockIdx.x / L.nB1;
  const Routes R = load_routes(ids, (const float*)nullptr, M * k, L.E);
  uint64_t mask = 0;
  const int e = slot_expert(R, s, &mask);
  if (e < 0) return;  // same decision in every wave of the workgroup
  const uint8_t* tile = prep + fc1_tile_offset(L, e, b);
  const uint32_t* sw = (const uint32_t*)(tile + (int64_t)L.nC1 * 1024) + lane;
  const int S = (L.nC1 + CS - 1) / CS;
  int m = 0;
  for (int t = 0; t < M; ++t) m += token_routes(mask, t, k) != 0;
  for (int i = 0; i < m; ++i) part[(i * W + wave) * 64 + lane] = 0.0f;

  for (int slab = wave; slab < S; slab += W) {
    const int c0 = slab * CS;
    const int n = min(CS, L.nC1 - c0);
    // Unconditional loads (a tail slab re-reads its last chunk, a cache hit):
    // guarded loads become branches, and the compiler then waits for each
    // load to land before issuing the next one.
    u32x4 q[CS];
#pragma unroll
    for (int i = 0; i < CS; ++i)
      q[i] = __builtin_nontemporal_load((const u32x4*)(tile + (int64_t)min(c0 + i, L.nC1 - 1) * 1024) + lane);
    uint32_t sd[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) sd[i] = __builtin_nontemporal_load(sw + 64 * min(c0 / SPD + i, L.nQ1 - 1));
    int ti = 0;
    for (int t = 0; t < M; ++t) {
      if (!token_routes(mask, t, k)) continue;
      const uint32_t* xr = (const uint32_t*)(x + (int64_t)t * L.H) + c0 * 16;
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < CS; ++i) {
        if (i < n) {
          bf16x2_t wv[16];
          fp4x8_to_bf16(q[i].x, wv);
          fp4x8_to_bf16(q[i].y, wv + 4);
          fp4x8_to_bf16(q[i].z, wv + 8);
          fp4x8_to_bf16(q[i].w, wv + 12);
          const uint32_t* xc = xr + i * 16;
          if (FMT == kMXFP4) {
            float p = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) p = __builtin_amdgcn_fdot2_f32_bf16(wv[j], as_bf16x2(xc[j]), p, false);
            acc = fmaf(p, mx_scale(sd[i / 4], i), acc);
          } else {
            float pa = 0.0f, pb = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) pa = __builtin_amdgcn_fdot2_f32_bf16(wv[j], as_bf16x2(xc[j]), pa, false);
#pragma unroll
            for (int j = 8; j < 16; ++j) pb = __builtin_amdgcn_fdot2_f32_bf16(wv[j], as_bf16x2(xc[j]), pb, false);
            const f32x2_t sc = e4m3x2_to_f32(sd[i / 2], (i & 1) != 0);
            acc = fmaf(pa, sc.x, acc);
            acc = fmaf(pb, sc.y, acc);
          }
        }
      }
      part[(ti * W + wave) * 64 + lane] += acc;
      ++ti;
    }
  }
  __syncthreads();
  const float g13 = FMT == kNVFP4 ? ((const float*)prep)[e] : 1.0f;
  int ti = 0;
  for (int t = 0; t < M; ++t) {
    const uint64_t tm = token_routes(mask, t, k);
    if (!tm) continue;
    if (ti % W == wave) {
      float v = 0.0f;
      for (int w = 0; w < W; ++w) v += part[(ti * W + w) * 64 + lane];
      fc1_finish(v, g13, lane, b, t * k + __builtin_ctzll(tm), L, act_hi, act_lo);
    }
    ++ti;
  }
}

template <int FMT, int NB, typename IdT>
__global__ void __launch_bounds__(64 * kMaxWaves2)
    fc2_kernel(const uint8_t* __restrict__ prep, const Layout L, const IdT* __restrict__ ids,
               const float* __restrict__ tw, const int M, const int k,
               const uint16_t* __restrict__ act_hi, const uint16_t* __restrict__ act_lo,
               uint16_t* __restrict__ out) {
  constexpr int SPD = FMT == kMXFP4 ? 4 : 2;
  constexpr int ND = NB / SPD;
  extern __shared__ float part[];  // [token][wave][lane]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int W = blockDim.x >> 6;
  const int hb = blockIdx.x;
  const int h = hb * 64 + lane;
  const int slots = M * k;
  const Routes R = load_routes(ids, tw, slots, L.E);
  for (int t = 0; t < M; ++t) part[(t * W + wave) * 64 + lane] = 0.0f;

  for (int s = wave; s < slots; s += W) {
    uint64_t mask = 0;
    const int e = slot_expert(R, s, &mask);
    if (e < 0) continue;
    const uint8_t* tile = prep + fc2_tile_offset(L, e, hb);
    const uint32_t* sw = (const uint32_t*)(tile + (int64_t)L.nC2 * 1024) + lane;
    const float g2 = FMT == kNVFP4 ? ((const float*)prep)[L.E + e] : 1.0f;
    for (int c0 = 0; c0 < L.nC2; c0 += NB) {
      const int n = min(NB, L.nC2 - c0);
      u32x4 q[NB];  // unconditional loads, as in fc1_kernel
#pragma unroll
      for (int i = 0; i < NB; ++i)
        q[i] = __builtin_nontemporal_load((const u32x4*)(tile + (int64_t)min(c0 + i, L.nC2 - 1) * 1024) + lane);
      uint32_t sd[ND];
#pragma unroll
      for (int i = 0; i < ND; ++i) sd[i] = __builtin_nontemporal_load(sw + 64 * min(c0 / SPD + i, L.nQ2 - 1));
      for (int t = 0; t < M; ++t) {
        uint64_t tm = token_routes(mask, t, k);
        if (!tm) continue;
        const int r = t * k + __builtin_ctzll(tm);
        float wsum = 0.0f;  // duplicate routes of a token share one FC2 result
        while (tm) {
          const int j = __builtin_ctzll(tm);
          tm &= tm - 1;
          wsum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(R.w), t * k + j));
        }
        const uint32_t* ah = (const uint32_t*)(act_hi + (int64_t)r * L.I) + 16 * c0;
        const uint32_t* al = (const uint32_t*)(act_lo + (int64_t)r * L.I) + 16 * c0;
        float y = 0.0f;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          if (i < n) {
            bf16x2_t wv[16];
            fp4x8_to_bf16(q[i].x, wv);
            fp4x8_to_bf16(q[i].y, wv + 4);
            fp4x8_to_bf16(q[i].z, wv + 8);
            fp4x8_to_bf16(q[i].w, wv + 12);
            const uint32_t* hc = ah + 16 * i;
            const uint32_t* lc = al + 16 * i;
            if (FMT == kMXFP4) {
              float p = 0.0f;
#pragma unroll
              for (int j = 0; j < 16; ++j) {
                p = __builtin_amdgcn_fdot2_f32_bf16(wv[j], as_bf16x2(hc[j]), p, false);
                p = __builtin_amdgcn_fdot2_f32_bf16(wv[j], as_bf16x2(lc[j]), p, false);
              }
              y = fmaf(p, mx_scale(sd[i / 4], i), y);
            } else {
              float pa = 0.0f, pb = 0.0f;
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                pa = __builtin_amdgcn_fdot2_f32_bf16(wv[j], as_bf16x2(hc[j]), pa, false);
                pa = __builtin_amdgcn_fdot2_f32_bf16(wv[j], as_bf16x2(lc[j]), pa, false);
              }
#pragma unroll
              for (int j = 8; j < 16; ++j) {
                pb = __builtin_amdgcn_fdot2_f32_bf16(wv[j], as_bf16x2(hc[j]), pb, false);
                pb = __builtin_amdgcn_fdot2_f32_bf16(wv[j], as_bf16x2(lc[j]), pb, false);
              }
              const f32x2_t sc = e4m3x2_to_f32(sd[i / 2], (i & 1) != 0);
              y = fmaf(pa, sc.x, y);
              y = fmaf(pb, sc.y, y);
            }
          }
        }
        part[(t * W + wave) * 64 + lane] += (y * g2) * wsum;
      }
    }
  }
  __syncthreads();
  if (h >= L.H) return;
  for (int t = wave; t < M; t += W) {
    float v = 0.0f;
    for (int w = 0; w < W; ++w) v += part[(t * W + w) * 64 + lane];
    out[(int64_t)t * L.H + h] = f32_to_bf16_rne(v);
  }
}

template <int FMT, typename IdT>
hipError_t launch_decode_fmt(const Layout& L, const uint8_t* prep, const uint16_t* x, int M, int k,
                             const IdT* ids, const float* tw, uint16_t* out, uint8_t* ws,
                             const DecodeWs& W, int cs, int phases, hipStream_t st) {
  const int slots = M * k;
  uint16_t* act_hi = (uint16_t*)(ws + W.act_hi);
  uint16_t* act_lo = (uint16_t*)(ws + W.act_lo);
  if (phases & 1) {
    const int S = (L.nC1 + cs - 1) / cs;
    const int waves = S < kMaxWaves ? S : kMaxWaves;
    const size_t lds = (size_t)M * waves * 64 * sizeof(float);
    const dim3 grid((unsigned)((int64_t)slots * L.nB1)), block(64 * waves);
    if (cs == 4)
      hipLaunchKernelGGL((fc1_kernel<FMT, 4, IdT>), grid, block, lds, st, prep, L, x, ids, M, k, act_hi, act_lo);
    else if (cs == 8)
      hipLaunchKernelGGL((fc1_kernel<FMT, 8, IdT>), grid, block, lds, st, prep, L, x, ids, M, k, act_hi, act_lo);
    else
      hipLaunchKernelGGL((fc1_kernel<FMT, 16, IdT>), grid, block, lds, st, prep, L, x, ids, M, k, act_hi, act_lo);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (phases & 2) {
    const int waves = slots < kMaxWaves2 ? slots : kMaxWaves2;
    const size_t lds = (size_t)M * waves * 64 * sizeof(float);
    const dim3 grid(L.nB2), block(64 * waves);
    const uint16_t* ah = act_hi;
    const uint16_t* al = act_lo;
    // chunk batch: the smallest of 4, 8, 12, 16 that covers I (or 16)
    if (L.nC2 <= 4)
      hipLaunchKernelGGL((fc2_kernel<FMT, 4, IdT>), grid, block, lds, st, prep, L, ids, tw, M, k, ah, al, out);
    else if (L.nC2 <= 8)
      hipLaunchKernelGGL((fc2_kernel<FMT, 8, IdT>), grid, block, lds, st, prep, L, ids, tw, M, k, ah, al, out);
    else if (L.nC2 <= 12)
      hipLaunchKernelGGL((fc2_kernel<FMT, 12, IdT>), grid, block, lds, st, prep, L, ids, tw, M, k, ah, al, out);
    else
      hipLaunchKernelGGL((fc2_kernel<FMT, 16, IdT>), grid, block, lds, st, prep, L, ids, tw, M, k, ah, al, out);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename IdT>
hipError_t launch_decode(const Layout& L, const uint8_t* prep, const uint16_t* x, int M, int k,
                         const IdT* ids, const float* tw, uint16_t* out, uint8_t* ws,
                         const DecodeWs& W, int cs, int phases, hipStream_t st) {
  if (L.fmt == kMXFP4)
    return launch_decode_fmt<kMXFP4, IdT>(L, prep, x, M, k, ids, tw, out, ws, W, cs, phases, st);
  return launch_decode_fmt<kNVFP4, IdT>(L, prep, x, M, k, ids, tw, out, ws, W, cs, phases, st);
}

template hipError_t launch_decode<int32_t>(const Layout&, const uint8_t*, const uint16_t*, int, int,
                                           const int32_t*, const float*, uint16_t*, uint8_t*,
                                           const DecodeWs&, int, int, hipStream_t);
template hipError_t launch_decode<int64_t>(const Layout&, const uint8_t*, const uint16_t*, int, int,
                                           const int64_t*, const float*, uint16_t*, uint8_t*,
                                           const DecodeWs&, int, int, hipStream_t);

}  // namespace moe
