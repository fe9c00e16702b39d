// Grouped (prefill) forward: many tokens, each routed expert's rows batched
// into grouped GEMMs on the CDNA4 matrix cores.
//
// The pages' prefill kernel distributes per-expert tiles whose row count
// follows the routed rows, so sparse routing does not pad every expert to a
// large tile (flashinfer #4285, description: MoEDynamicKernel with tiles
// smaller than 128 rows), and reduces the routed outputs into fp32 before one
// cast (b12x #311, commit on the prefill fused-sum epilogue).  Here:
//   route_count / route_scatter  group the valid routes by expert in route
//                                order (deterministic), and number the
//                                128-row m-tiles of every expert;
//   fc1_gemm   x rows gathered into LDS, FP4 weight tiles dequantised to
//              bf16 into LDS (exact: E2M1 times a UE8M0 or E4M3 block scale
//              has at most 6 significant bits), v_mfma_f32_32x32x16_bf16 with
//              fp32 accumulation, SiLU(gate)*up epilogue -> activation rows as
//              two bf16 planes, hi = bf16(a) and lo = bf16(a - hi);
//   fc2_gemm   the same over the activation rows and W2, one MFMA per plane
//              (so the activation keeps 16 significant bits, as in the decode
//              path), times the NVFP4 global and the route's router weight ->
//              fp32 rows;
//   combine    per token, the fp32 sum of its valid routes' rows in route
//              order, rounded once to bf16.
// Invalid ids (negative or >= E) join no group and are skipped by combine.
#include <hip/hip_runtime.h>

#include "decode.h"
#include "layout.h"
#include "prefill.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;            // K elements per main-loop step (2 units)
constexpr int kLdsRow = kBK + 8;   // bf16 per LDS row: 144 B, rotates banks by 4 per row

template <typename IdT>
__device__ __forceinline__ int route_expert(const IdT* __restrict__ ids, int r, int R, int E) {
  if (r >= R) return -1;
  const int64_t v = (int64_t)ids[r];
  return (v >= 0 && v < E) ? (int)v : -1;
}

// One wave per expert: number of valid routes holding it.
template <typename IdT>
__global__ void __launch_bounds__(256)
    route_count(const IdT* __restrict__ ids, int R, int E, int* __restrict__ counts) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  int cnt = 0;
  for (int base = 0; base < R; base += 64) cnt += __popcll(__ballot(route_expert(ids, base + lane, R, E) == e));
  if (lane == 0) counts[e] = cnt;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// One wave per expert: its group's start, its m-tiles' start, and the
// grouped position of each of its routes (route order within the group).
template <typename IdT>
__global__ void __launch_bounds__(256)
    route_scatter(const IdT* __restrict__ ids, int R, int E, const int* __restrict__ counts,
                  int* __restrict__ grp_start, int* __restrict__ tile_start, int* __restrict__ perm,
                  int* __restrict__ rpos) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  int off = 0, toff = 0;
  for (int q = lane; q < e; q += 64) {
    const int c = counts[q];
    off += c;
    toff += (c + kGemmBM - 1) / kGemmBM;
  }
  off = wave_sum(off);
  toff = wave_sum(toff);
  const int ce = counts[e];
  if (lane == 0) {
    grp_start[e] = off;
    tile_start[e] = toff;
    if (e == E - 1) tile_start[E] = toff + (ce + kGemmBM - 1) / kGemmBM;
  }
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  int pos = off;
  for (int base = 0; base < R; base += 64) {
    const int r = base + lane;
    const bool mine = route_expert(ids, r, R, E) == e;
    const uint64_t m = __ballot(mine);
    if (mine) {
      const int p = pos + __popcll(m & below);
      perm[p] = r;
      rpos[r] = p;
    }
    pos += __popcll(m);
  }
}

// Expert of grouped m-tile gm (tile_start is non-decreasing; the expert is
// the last e with tile_start[e] <= gm).
__device__ __forceinline__ int tile_expert(const int* __restrict__ tile_start, int E, int gm) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (tile_start[mid] <= gm)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// 32 E2M1 values of one unit as bf16 with the block scale(s) applied
// (exact), written as 4 x 16 B to LDS.
template <int FMT>
__device__ __forceinline__ void dequant_unit_to_lds(u32x4 q, uint32_t sword, int c, __bf16* dst) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  u32x4* d = (u32x4*)dst;
  if (FMT == kMXFP4) {
    // v_cvt_scalef32_pk_bf16_fp4 scales by the exponent of its fp32 operand,
    // which is the UE8M0 byte placed in the exponent field.
    const float s = __uint_as_float(((sword >> (8 * (c & 3))) & 0xFFu) << 23);
#pragma unroll
    for (int dd = 0; dd < 4; ++dd) {
      bf16x2_t p[4];
      p[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[dd], s, 0);
      p[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[dd], s, 1);
      p[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[dd], s, 2);
      p[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[dd], s, 3);
      d[dd] = u32x4{__builtin_bit_cast(uint32_t, p[0]), __builtin_bit_cast(uint32_t, p[1]),
                    __builtin_bit_cast(uint32_t, p[2]), __builtin_bit_cast(uint32_t, p[3])};
    }
  } else {
    const f32x2_t sc = e4m3x2_to_f32(sword, (c & 1) != 0);
#pragma unroll
    for (int dd = 0; dd < 4; ++dd) {
      const float s = dd < 2 ? sc.x : sc.y;
      f32x2_t f[4];
      fp4x8_to_f32(w[dd], f);
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x2_t b;
        b.x = (__bf16)(f[i].x * s);  // exact: at most 6 significant bits
        b.y = (__bf16)(f[i].y * s);
        o[i] = __builtin_bit_cast(uint32_t, b);
      }
      d[dd] = u32x4{o[0], o[1], o[2], o[3]};
    }
  }
}

__device__ __forceinline__ bf16x8_t lds_frag(const __bf16* p) {
  return __builtin_bit_cast(bf16x8_t, *(const u32x4*)p);
}

// Grouped GEMM main loop for one 128 x 128 output tile, K in steps of 64.
// Each thread's A row comes from `arow` (bf16, K contiguous) and, when
// SPLIT, a second plane `arow_lo` whose products are added to the same
// accumulators.  B rows are two 64-row prepared tiles (tile1 reads as zero
// when !tile1_ok).  Waves form a 2 x 2 grid of 64 x 64 sub-tiles, each 2 x 2
// MFMA 32x32x16 blocks; this wave's B rows start at bcol0.
template <int FMT, bool SPLIT>
__device__ __forceinline__ void gemm_main(const uint16_t* __restrict__ arow,
                                          const uint16_t* __restrict__ arow_lo, int kmax,
                                          const uint8_t* tile0, const uint8_t* tile1, bool tile1_ok,
                                          int nC, __bf16 (*As)[kGemmBM][kLdsRow],
                                          __bf16 (*Bs)[kLdsRow], f32x16_t (&acc)[2][2], int bcol0) {
  constexpr int SPD = FMT == kMXFP4 ? 4 : 2;
  constexpr int NP = SPLIT ? 2 : 1;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wr = wave >> 1;
  // loader roles
  const int ia = t >> 1, ha = t & 1;   // A: tile row, 32-element half of the step
  const int ib = t & 127, hb = t >> 7; // B: tile row, unit of the step
  const uint8_t* btile = ib < 64 ? tile0 : tile1;
  const bool bok = ib < 64 || tile1_ok;
  const int brow = ib & 63;
  const int nsteps = (nC + 1) / 2;

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

  u32x4 ra[NP][4];
  u32x4 rb;
  uint32_t rs;
  auto load = [&](int ks) {
    const int ka = ks * kBK + 32 * ha;
    const bool aok = ka < kmax;
#pragma unroll
    for (int pl = 0; pl < NP; ++pl) {
      const u32x4* ap = (const u32x4*)((pl ? arow_lo : arow) + (aok ? ka : 0));
#pragma unroll
      for (int i = 0; i < 4; ++i) ra[pl][i] = aok ? ap[i] : u32x4{0u, 0u, 0u, 0u};
    }
    const int c = ks * 2 + hb;
    const bool cok = bok && c < nC;
    const int cc = cok ? c : 0;
    rb = cok ? __builtin_nontemporal_load((const u32x4*)(btile + (int64_t)cc * 1024 + brow * 16))
             : u32x4{0u, 0u, 0u, 0u};
    rs = cok ? __builtin_nontemporal_load((const uint32_t*)(btile + (int64_t)nC * 1024 + (cc / SPD) * 256 + brow * 4))
             : 0u;
  };
  load(0);
  for (int ks = 0; ks < nsteps; ++ks) {
    // stage the loaded step in LDS
#pragma unroll
    for (int pl = 0; pl < NP; ++pl) {
      u32x4* ad = (u32x4*)&As[pl][ia][32 * ha];
#pragma unroll
      for (int i = 0; i < 4; ++i) ad[i] = ra[pl][i];
    }
    dequant_unit_to_lds<FMT>(rb, rs, ks * 2 + hb, &Bs[ib][32 * hb]);
    __syncthreads();
    if (ks + 1 < nsteps) load(ks + 1);  // next step's loads overlap this step's MFMAs
#pragma unroll
    for (int k16 = 0; k16 < kBK / 16; ++k16) {
      const int kk = k16 * 16 + 8 * (lane >> 5);
      bf16x8_t bf[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) bf[j] = lds_frag(&Bs[bcol0 + j * 32 + (lane & 31)][kk]);
#pragma unroll
      for (int pl = 0; pl < NP; ++pl) {
        bf16x8_t af[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) af[i] = lds_frag(&As[pl][wr * 64 + i * 32 + (lane & 31)][kk]);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();
  }
}

// Row (within the 32x32 block) of accumulator register r of this lane.
__device__ __forceinline__ int acc_row(int r, int lane) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }

template <int FMT>
__global__ void __launch_bounds__(256)
    fc1_gemm(const uint8_t* __restrict__ prep, const Layout L, const uint16_t* __restrict__ x, int k,
             const int* __restrict__ counts, const int* __restrict__ grp_start,
             const int* __restrict__ tile_start, const int* __restrict__ perm,
             uint16_t* __restrict__ act, int64_t plane) {
  __shared__ __bf16 As[1][kGemmBM][kLdsRow];
  __shared__ __bf16 Bs[128][kLdsRow];
  const int gm = blockIdx.x;
  if (gm >= tile_start[L.E]) return;
  const int e = tile_expert(tile_start, L.E, gm);
  const int m0 = (gm - tile_start[e]) * kGemmBM;
  const int rows = min(kGemmBM, counts[e] - m0);
  const int gs = grp_start[e] + m0;
  const int n0 = blockIdx.y * 64;  // gate columns n0..n0+63 (prepared tiles n0/32, n0/32 + 1)
  const int b0 = n0 / 32;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  // A row of this thread's loader role: the token of grouped row gs + ia
  const int ia = t >> 1;
  const int token = perm[gs + min(ia, rows - 1)] / k;
  f32x16_t acc[2][2];
  // wave column wc uses prepared tile b0 + wc: its rows 0..31 are gate, 32..63 up
  gemm_main<FMT, false>(x + (int64_t)token * L.H, nullptr, L.H, prep + fc1_tile_offset(L, e, b0),
                 prep + fc1_tile_offset(L, e, min(b0 + 1, L.nB1 - 1)), b0 + 1 < L.nB1, L.nC1, As, Bs,
                 acc, wc * 64);
  const float g13 = FMT == kNVFP4 ? ((const float*)prep)[e] : 1.0f;
  const int n = n0 + wc * 32 + (lane & 31);
  if (n >= L.I) return;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wr * 64 + i * 32 + acc_row(r, lane);
      if (row >= rows) continue;
      const float gate = acc[i][0][r] * g13;
      const float up = acc[i][1][r] * g13;
      const float a = gate / (1.0f + __expf(-gate)) * up;
      const uint16_t hi = f32_to_bf16_rne(a);
      const int64_t o = (int64_t)(gs + row) * L.I + n;
      act[o] = hi;
      act[plane + o] = f32_to_bf16_rne(a - __uint_as_float((uint32_t)hi << 16));
    }
  }
}

template <int FMT>
__global__ void __launch_bounds__(256)
    fc2_gemm(const uint8_t* __restrict__ prep, const Layout L, const float* __restrict__ tw,
             const int* __restrict__ counts, const int* __restrict__ grp_start,
             const int* __restrict__ tile_start, const int* __restrict__ perm,
             const uint16_t* __restrict__ act, int64_t plane, float* __restrict__ y) {
  __shared__ __bf16 As[2][kGemmBM][kLdsRow];
  __shared__ __bf16 Bs[128][kLdsRow];
  __shared__ float wrow[kGemmBM];
  const int gm = blockIdx.x;
  if (gm >= tile_start[L.E]) return;
  const int e = tile_expert(tile_start, L.E, gm);
  const int m0 = (gm - tile_start[e]) * kGemmBM;
  const int rows = min(kGemmBM, counts[e] - m0);
  const int gs = grp_start[e] + m0;
  const int n0 = blockIdx.y * 128;  // output columns (rows of W2) n0..n0+127
  const int hb0 = n0 / 64;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  if (t < kGemmBM) wrow[t] = t < rows ? tw[perm[gs + t]] : 0.0f;
  const int ia = t >> 1;
  f32x16_t acc[2][2];
  const uint16_t* arow = act + (int64_t)(gs + min(ia, rows - 1)) * L.I;
  gemm_main<FMT, true>(arow, arow + plane, L.I, prep + fc2_tile_offset(L, e, hb0),
                 prep + fc2_tile_offset(L, e, min(hb0 + 1, L.nB2 - 1)), hb0 + 1 < L.nB2, L.nC2, As, Bs,
                 acc, wc * 64);
  const float g2 = FMT == kNVFP4 ? ((const float*)prep)[L.E + e] : 1.0f;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wc * 64 + j * 32 + (lane & 31);
    if (n >= L.H) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wr * 64 + i * 32 + acc_row(r, lane);
        if (row >= rows) continue;
        y[(int64_t)(gs + row) * L.H + n] = (acc[i][j][r] * g2) * wrow[row];
      }
    }
  }
}

// out[t][h] = bf16(sum over valid routes j of token t, in route order, of
// y[grouped row of (t, j)][h]); a token with no valid route gives +0.
template <typename IdT>
__global__ void __launch_bounds__(256)
    combine(const IdT* __restrict__ ids, int k, int E, int H, const int* __restrict__ rpos,
            const float* __restrict__ y, uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  const int h = (blockIdx.y * 256 + threadIdx.x) * 2;
  if (h >= H) return;
  float a0 = 0.0f, a1 = 0.0f;
  for (int j = 0; j < k; ++j) {
    const int64_t id = (int64_t)ids[t * k + j];
    if (id < 0 || id >= E) continue;
    const f32x2_t v = *(const f32x2_t*)(y + (int64_t)rpos[t * k + j] * H + h);
    a0 += v.x;
    a1 += v.y;
  }
  *(uint32_t*)(out + (int64_t)t * H + h) = (uint32_t)f32_to_bf16_rne(a0) | ((uint32_t)f32_to_bf16_rne(a1) << 16);
}

template <int FMT, typename IdT>
hipError_t launch_prefill_fmt(const Layout& L, const uint8_t* prep, const uint16_t* x, int M, int k,
                              const IdT* ids, const float* tw, uint16_t* out, uint8_t* ws,
                              const PrefillWs& W, int phases, hipStream_t st) {
  const int R = M * k;
  int* counts = (int*)(ws + W.counts);
  int* grp_start = (int*)(ws + W.grp_start);
  int* tile_start = (int*)(ws + W.tile_start);
  int* perm = (int*)(ws + W.perm);
  int* rpos = (int*)(ws + W.rpos);
  uint16_t* act = (uint16_t*)(ws + W.act);
  const int64_t plane = (W.y - W.act) / 4;  // elements from the hi plane to the lo plane
  float* y = (float*)(ws + W.y);
  const dim3 gE((L.E + 3) / 4);
  // m-tiles: at most one partial tile per expert beyond R / 128 full ones
  const unsigned mt = (unsigned)((R + kGemmBM - 1) / kGemmBM + L.E);
  if (phases & 1) {
    hipLaunchKernelGGL((route_count<IdT>), gE, dim3(256), 0, st, ids, R, L.E, counts);
    hipLaunchKernelGGL((route_scatter<IdT>), gE, dim3(256), 0, st, ids, R, L.E, (const int*)counts,
                       grp_start, tile_start, perm, rpos);
    hipLaunchKernelGGL((fc1_gemm<FMT>), dim3(mt, (L.I + 63) / 64), dim3(256), 0, st, prep, L, x, k,
                       (const int*)counts, (const int*)grp_start, (const int*)tile_start,
                       (const int*)perm, act, plane);
  }
  if (phases & 2) {
    hipLaunchKernelGGL((fc2_gemm<FMT>), dim3(mt, (L.H + 127) / 128), dim3(256), 0, st, prep, L, tw,
                       (const int*)counts, (const int*)grp_start, (const int*)tile_start,
                       (const int*)perm, (const uint16_t*)act, plane, y);
    hipLaunchKernelGGL((combine<IdT>), dim3(M, (L.H + 511) / 512), dim3(256), 0, st, ids, k, L.E, L.H,
                       (const int*)rpos, (const float*)y, out);
  }
  return hipGetLastError();
}

template <typename IdT>
hipError_t launch_prefill(const Layout& L, const uint8_t* prep, const uint16_t* x, int M, int k,
                          const IdT* ids, const float* tw, uint16_t* out, uint8_t* ws,
                          const PrefillWs& W, int phases, hipStream_t st) {
  if (L.fmt == kMXFP4)
    return launch_prefill_fmt<kMXFP4, IdT>(L, prep, x, M, k, ids, tw, out, ws, W, phases, st);
  return launch_prefill_fmt<kNVFP4, IdT>(L, prep, x, M, k, ids, tw, out, ws, W, phases, st);
}

template hipError_t launch_prefill<int32_t>(const Layout&, const uint8_t*, const uint16_t*, int, int,
                                            const int32_t*, const float*, uint16_t*, uint8_t*,
                                            const PrefillWs&, int, hipStream_t);
template hipError_t launch_prefill<int64_t>(const Layout&, const uint8_t*, const uint16_t*, int, int,
                                            const int64_t*, const float*, uint16_t*, uint8_t*,
                                            const PrefillWs&, int, hipStream_t);

}  // namespace moe
